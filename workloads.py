"""Seeded synthetic workloads for GVA decode (shared by tests, bench and smoke).

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no RoPE, no attention, no reconstruction map products.
Every array it returns is float64 holding values that are exactly
representable in the workload's storage dtype (bf16 or fp32), so the CPU
oracle and the HIP path see identical numbers.

Recipe (the pages measure trained models on datasets that are not available
here, so seeded synthetic caches of the same shapes stand in for them):
  * generator numpy PCG64(seed), seed = 20260 + workload index (1..5);
  * draw order: sequence lengths (ragged workload only), V, pre-RoPE k_r,
    q_nope, pre-RoPE q_rope, M; every draw is float64 standard normal,
    M is scaled by 1/sqrt(d_v) (variance 1/64);
  * each draw is rounded once to the storage dtype (torch's fp32 then bf16
    conversion, round-to-nearest-even each);
  * the ragged workload draws lengths uniformly in [1024, 32768] and its page
    pool is a seeded random permutation (block_table).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """Sizes of one GVA decode workload (names follow the pages' notation)."""

    name: str
    index: int            # workload number 1..5, selects the seed
    B: int                # sequences in the batch
    H: int                # query heads
    G: int                # value groups (head h reads group h // (H // G))
    d_n: int              # content (unrotated) query width
    d_v: int              # value width
    d_r: int              # shared positional-key width
    S: int                # cached tokens per sequence (uniform workloads)
    dtype: str            # 'bf16' or 'f32' storage / call dtype
    len_lo: int = 0       # ragged workload: min sequence length
    len_hi: int = 0       # ragged workload: max sequence length
    block_size: int = 0   # 0 = contiguous cache, else paged block size
    split_tokens: int = 0 # 0 = automatic split-K partition size
    steps: int = 1        # decode steps (one appended token each)
    rope_base: float = 10000.0

    @property
    def seed(self) -> int:
        return 20260 + self.index

    @property
    def ragged(self) -> bool:
        return self.len_hi > 0

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d_n + d_r) as the fp32 value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.d_n + self.d_r)))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, B=1, H=16, G=4, d_n=64, d_v=64, d_r=16,
                         S=256, dtype="f32"),
    "mid_bf16": Workload("mid_bf16", 2, B=16, H=16, G=4, d_n=64, d_v=64, d_r=16,
                         S=4096, dtype="bf16", steps=100),
    "wide_dr24": Workload("wide_dr24", 3, B=32, H=16, G=4, d_n=64, d_v=64, d_r=24,
                          S=8192, dtype="bf16"),
    "long_split": Workload("long_split", 4, B=4, H=16, G=4, d_n=64, d_v=64, d_r=16,
                           S=131072, dtype="bf16", split_tokens=4096),
    "ragged_paged": Workload("ragged_paged", 5, B=64, H=16, G=4, d_n=64, d_v=64,
                             d_r=16, S=0, dtype="bf16", len_lo=1024,
                             len_hi=32768, block_size=64),
}


def round_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws once to the storage dtype; return them as float64."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).float()
    if dtype == "bf16":
        t = t.bfloat16()
    elif dtype != "f32":
        raise ValueError(dtype)
    return t.double().numpy()


def torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def to_torch(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Exact conversion of storage-representable float64 values to a CPU tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    return t.to(torch_dtype(dtype))


@dataclasses.dataclass
class GvaInputs:
    """One decode problem. Arrays are float64 with storage-exact values.

    lens[b]         tokens already cached for sequence b (before `extra` appends)
    V[b]            [G, lens[b] + extra, d_v]   values (the last `extra` rows are
                    appended during decode steps)
    kr[b]           [lens[b] + extra, d_r]      positional keys BEFORE RoPE
    q_nope          [B, H, d_n]
    q_rope          [B, H, d_r]                 BEFORE RoPE
    M               [H, d_v, d_n]               reconstruction maps, K_h = V_g M_h
    """

    wl: Workload
    lens: np.ndarray
    extra: int
    V: List[np.ndarray]
    kr: List[np.ndarray]
    q_nope: np.ndarray
    q_rope: np.ndarray
    M: np.ndarray


def ragged_lens(wl: Workload, seed: Optional[int] = None) -> np.ndarray:
    """The ragged workload's sequence lengths: the first draw of the
    workload's generator, exactly as make_gva_inputs draws them."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    return rng.integers(wl.len_lo, wl.len_hi, size=wl.B, endpoint=True)


def make_gva_inputs(wl: Workload, extra: int = 0, seed: Optional[int] = None,
                    lens: Optional[np.ndarray] = None) -> GvaInputs:
    """Draw one seeded problem. `extra` = tokens reserved for later appends."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    if lens is None:
        if wl.ragged:
            lens = rng.integers(wl.len_lo, wl.len_hi, size=wl.B, endpoint=True)
        else:
            lens = np.full(wl.B, wl.S, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    V = [round_storage(rng.standard_normal((wl.G, int(n) + extra, wl.d_v)), wl.dtype)
         for n in lens]
    kr = [round_storage(rng.standard_normal((int(n) + extra, wl.d_r)), wl.dtype)
          for n in lens]
    q_nope = round_storage(rng.standard_normal((wl.B, wl.H, wl.d_n)), wl.dtype)
    q_rope = round_storage(rng.standard_normal((wl.B, wl.H, wl.d_r)), wl.dtype)
    M = round_storage(rng.standard_normal((wl.H, wl.d_v, wl.d_n)) / math.sqrt(wl.d_v),
                      wl.dtype)
    return GvaInputs(wl, lens, extra, V, kr, q_nope, q_rope, M)


def make_gqa_inputs(wl: Workload, seed: Optional[int] = None):
    """Matched GQA problem: K, V [B, G, S, d_h] (K drawn as post-RoPE values),
    q [B, H, d_h] (already rotated). d_h = d_v."""
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 1000))
    shape = (wl.B, wl.G, wl.S, wl.d_v)
    K = round_storage(rng.standard_normal(shape), wl.dtype)
    V = round_storage(rng.standard_normal(shape), wl.dtype)
    q = round_storage(rng.standard_normal((wl.B, wl.H, wl.d_v)), wl.dtype)
    return q, K, V


def make_projection_inputs(wl: Workload, d_model: int, seed: Optional[int] = None):
    """Hidden states and query-projection weights of one layer: x [B, d_model]
    ~ N(0, 1); W_q,nope [H, d_n, d_model] and W_q,rope [H, d_r, d_model] ~
    N(0, 1/d_model), so the projected queries are ~ N(0, 1) like the directly
    drawn ones. Each rounded once to the workload dtype."""
    rng = np.random.Generator(np.random.PCG64((wl.seed if seed is None else seed) + 2000))
    x = round_storage(rng.standard_normal((wl.B, d_model)), wl.dtype)
    wq_nope = round_storage(rng.standard_normal((wl.H, wl.d_n, d_model)) / math.sqrt(d_model), wl.dtype)
    wq_rope = round_storage(rng.standard_normal((wl.H, wl.d_r, d_model)) / math.sqrt(d_model), wl.dtype)
    return x, wq_nope, wq_rope


def draw_post_rope(wl: Workload, lens: np.ndarray, rows_extra: int = 0,
                   seed: int = 0):
    """Draw k_r and q_rope directly as post-RoPE values (for decode-only
    problems where the rotation is not under test)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed * 7919 + seed))
    kr = [round_storage(rng.standard_normal((int(n) + rows_extra, wl.d_r)), wl.dtype)
          for n in lens]
    q_rope = round_storage(rng.standard_normal((wl.B, wl.H, wl.d_r)), wl.dtype)
    return kr, q_rope


# --------------------------------------------------------------------------
# Cache layouts (plain data movement, used to hand the same values to the
# device in the layout the library expects).
# --------------------------------------------------------------------------

def contiguous_cache(rows: List[np.ndarray], capacity: int, token_axis: int) -> np.ndarray:
    """Stack per-sequence arrays into [B, ..., capacity, ...] zero padded."""
    B = len(rows)
    shp = list(rows[0].shape)
    shp[token_axis] = capacity
    out = np.zeros([B] + shp, dtype=np.float64)
    for b, r in enumerate(rows):
        n = r.shape[token_axis]
        idx = [slice(None)] * r.ndim
        idx[token_axis] = slice(0, n)
        out[(b,) + tuple(idx)] = r
    return out


def paged_pool(lens_cap: np.ndarray, block_size: int, seed: int,
               max_blocks_per_seq: Optional[int] = None):
    """Seeded shuffled block table: block_table[b, j] = pool block holding
    tokens [j*block_size, (j+1)*block_size) of sequence b. Unused entries -1."""
    need = [int(math.ceil(int(n) / block_size)) for n in lens_cap]
    total = int(sum(need))
    mb = max(need) if max_blocks_per_seq is None else max_blocks_per_seq
    rng = np.random.Generator(np.random.PCG64(seed + 5000))
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(need), mb), -1, dtype=np.int32)
    pos = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return table, total


def scatter_paged(rows_v: List[np.ndarray], rows_kr: List[np.ndarray],
                  table: np.ndarray, n_blocks: int, block_size: int):
    """Place per-sequence V [G, n, d_v] / k_r [n, d_r] into a page pool
    V_pool [n_blocks, G, block_size, d_v], kr_pool [n_blocks, block_size, d_r]."""
    G, _, d_v = rows_v[0].shape
    d_r = rows_kr[0].shape[1]
    vp = np.zeros((n_blocks, G, block_size, d_v))
    kp = np.zeros((n_blocks, block_size, d_r))
    for b, (v, k) in enumerate(zip(rows_v, rows_kr)):
        n = v.shape[1]
        for j in range(int(math.ceil(n / block_size))):
            blk = table[b, j]
            lo, hi = j * block_size, min(n, (j + 1) * block_size)
            vp[blk, :, :hi - lo, :] = v[:, lo:hi, :]
            kp[blk, :hi - lo, :] = k[lo:hi, :]
    return vp, kp
