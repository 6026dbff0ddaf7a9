"""Device-resident compact cache (one layer): allocation and bookkeeping.

Holds the tensors the C ABI works on: v_cache, kr_cache, seq_lens and, for a
paged cache, the block table. Writes go through gva_append; reads through
gva_decode. No arithmetic happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (GvaShape, gva_append, gva_decode, gva_decode_step, gva_decode_step_workspace_bytes,
               gva_decode_workspace_bytes, make_shape)

_TD = {"bf16": torch.bfloat16, "f32": torch.float32}


class GvaCache:
    """Compact GVA cache of one layer for B sequences.

    Contiguous:  v_cache [B, G, capacity, d_v], kr_cache [B, capacity, d_r]
    Paged:       v_cache [num_blocks, G, 64, d_v], kr_cache [num_blocks, 64, d_r],
                 block_table [B, max_blocks_per_seq] (int32, caller-chosen ids)
    """

    def __init__(self, B: int, H: int, G: int, d_n: int, d_v: int, d_r: int, *, dtype="bf16",
                 capacity: int = 0, block_table: Optional[torch.Tensor] = None,
                 num_blocks: int = 0, device="cuda"):
        self.B, self.H, self.G, self.d_n, self.d_v, self.d_r = B, H, G, d_n, d_v, d_r
        self.dtype = dtype
        td = _TD[dtype]
        self.paged = block_table is not None
        if self.paged:
            self.block_table = block_table.to(device=device, dtype=torch.int32).contiguous()
            self.num_blocks = int(num_blocks)
            self.max_blocks = int(self.block_table.shape[1])
            self.capacity = self.max_blocks * 64
            self.v_cache = torch.zeros(self.num_blocks, G, 64, d_v, dtype=td, device=device)
            self.kr_cache = torch.zeros(self.num_blocks, 64, max(d_r, 1), dtype=td, device=device)
        else:
            self.block_table = None
            self.num_blocks = 0
            self.max_blocks = 0
            self.capacity = int(capacity)
            self.v_cache = torch.zeros(B, G, self.capacity, d_v, dtype=td, device=device)
            self.kr_cache = torch.zeros(B, self.capacity, max(d_r, 1), dtype=td, device=device)
        if d_r == 0:
            self.kr_cache = None
        self.seq_lens = torch.zeros(B, dtype=torch.int32, device=device)

    def shape(self, max_seq_len: int, split_tokens: int = 0, B: Optional[int] = None) -> GvaShape:
        return make_shape(self.B if B is None else B, self.H, self.G, self.d_n, self.d_v, self.d_r,
                          capacity=0 if self.paged else self.capacity,
                          max_seq_len=min(int(max_seq_len), self.capacity),
                          block_size=64 if self.paged else 0, num_blocks=self.num_blocks,
                          max_blocks_per_seq=self.max_blocks, split_tokens=split_tokens,
                          dtype=self.dtype)

    def append(self, v_new: torch.Tensor, kr_new: Optional[torch.Tensor],
               rope_base: float = 10000.0, stream=None) -> None:
        """Append v_new [B, G, n, d_v] and pre-RoPE kr_new [B, n, d_r] to every sequence."""
        n = int(v_new.shape[2])
        gva_append(self.shape(self.capacity), v_new, kr_new, n, self.seq_lens, self.v_cache,
                   self.kr_cache, self.block_table, rope_base, stream)

    def append_one(self, b: int, v_new: torch.Tensor, kr_new: Optional[torch.Tensor],
                   rope_base: float = 10000.0, stream=None) -> None:
        """Append v_new [G, n, d_v] / kr_new [n, d_r] to sequence b only."""
        n = int(v_new.shape[1])
        if self.paged:
            v, k, table = self.v_cache, self.kr_cache, self.block_table[b:b + 1]
        else:
            v = self.v_cache[b:b + 1]
            k = None if self.kr_cache is None else self.kr_cache[b:b + 1]
            table = None
        gva_append(self.shape(self.capacity, B=1), v_new.unsqueeze(0).contiguous(),
                   None if kr_new is None else kr_new.unsqueeze(0).contiguous(), n,
                   self.seq_lens[b:b + 1], v, k, table, rope_base, stream)

    def workspace(self, max_seq_len: int, split_tokens: int = 0) -> Optional[torch.Tensor]:
        n = gva_decode_workspace_bytes(self.shape(max_seq_len, split_tokens))
        if n == 0:
            return None
        return torch.zeros((n + 3) // 4, dtype=torch.float32, device=self.v_cache.device)

    def decode(self, q_nope, q_rope, M, scale: float, out, max_seq_len: int,
               split_tokens: int = 0, workspace=None, stream=None) -> None:
        shape = self.shape(max_seq_len, split_tokens)
        if workspace is None:
            workspace = self.workspace(max_seq_len, split_tokens)
        gva_decode(shape, q_nope, q_rope, M, self.v_cache, self.kr_cache, self.seq_lens,
                   self.block_table, scale, out, workspace, stream)

    def step_workspace(self, max_seq_len: int, split_tokens: int = 0) -> torch.Tensor:
        n = gva_decode_step_workspace_bytes(self.shape(max_seq_len, split_tokens))
        return torch.zeros((n + 3) // 4, dtype=torch.float32, device=self.v_cache.device)

    def step(self, v_new, kr_new, q_nope, q_rope, M, scale: float, out, max_seq_len: int,
             split_tokens: int = 0, workspace=None, rope_base: float = 10000.0, stream=None) -> None:
        """One fused decode step: append v_new [B, G, d_v] / pre-RoPE kr_new [B, d_r],
        rotate pre-RoPE q_rope, decode into out. max_seq_len bounds the lengths
        after the append."""
        shape = self.shape(max_seq_len, split_tokens)
        if workspace is None:
            workspace = self.step_workspace(max_seq_len, split_tokens)
        gva_decode_step(shape, v_new, kr_new, q_nope, q_rope, M, self.v_cache, self.kr_cache,
                        self.seq_lens, self.block_table, scale, rope_base, out, workspace, stream)

    def snapshot(self) -> dict:
        """Host copy of the cache state (checkpoint): both caches, the lengths
        and, for a paged cache, the block table. Synchronous device-to-host
        copies; the state of the device tensors is unchanged."""
        state = {"v_cache": self.v_cache.cpu(), "seq_lens": self.seq_lens.cpu()}
        if self.kr_cache is not None:
            state["kr_cache"] = self.kr_cache.cpu()
        if self.block_table is not None:
            state["block_table"] = self.block_table.cpu()
        return state

    def restore(self, state: dict) -> None:
        """Put a snapshot() back into this cache's device tensors (resume). The
        snapshot must come from a cache of the same sizes and layout."""
        pairs = [("v_cache", self.v_cache), ("seq_lens", self.seq_lens),
                 ("kr_cache", self.kr_cache), ("block_table", self.block_table)]
        for name, dst in pairs:
            if (dst is None) != (name not in state):
                raise ValueError(f"snapshot and cache disagree on {name}")
            if dst is None:
                continue
            src = state[name]
            if tuple(src.shape) != tuple(dst.shape) or src.dtype != dst.dtype:
                raise ValueError(f"{name}: snapshot {tuple(src.shape)} {src.dtype} does not fit "
                                 f"{tuple(dst.shape)} {dst.dtype}")
        for name, dst in pairs:
            if dst is not None:
                dst.copy_(state[name])
