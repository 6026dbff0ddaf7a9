"""Grouped Value Attention (GVA) decode over a compact KV cache, for MI355X.

Thin torch binding of the C ABI in include/gva.h: each function here checks
and marshals its tensor arguments (device pointers, the current HIP stream)
and calls the function of the same name in libgva.so. All arithmetic runs in
the library's HIP kernels; torch only provides device memory and streams.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib
from ._lib import GVA_BF16, GVA_F32, GvaShape

__all__ = [
    "GvaShape", "GVA_F32", "GVA_BF16", "GvaError", "make_shape", "lib",
    "gva_append", "gva_rope_query", "gva_decode", "gva_decode_step", "gva_decode_step_noalloc",
    "gva_gqa_ref_decode",
    "gva_fold_query_projection", "gva_query_projection", "gva_rope_query_multi", "gva_decode_multi",
    "gva_decode_multi_workspace_bytes", "gva_prefill", "gva_copy_blocks", "gva_fork", "gva_rollback",
    "gva_decode_workspace_bytes", "gva_decode_step_workspace_bytes", "gva_decode_split_tokens", "gva_cache_bytes_per_token",
    "gva_status_string", "gva_abi_version", "workspace_for",
]

lib = _lib.load()

_DTYPES = {"bf16": GVA_BF16, "f32": GVA_F32, torch.bfloat16: GVA_BF16, torch.float32: GVA_F32}
_TORCH = {GVA_BF16: torch.bfloat16, GVA_F32: torch.float32}


class GvaError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        name = lib.gva_status_string(status).decode()
        detail = lib.gva_last_error().decode()
        super().__init__(f"{fn}: {name}: {detail}")


def make_shape(B: int, H: int, G: int, d_n: int, d_v: int, d_r: int, *, capacity: int = 0,
               max_seq_len: int = 0, block_size: int = 0, num_blocks: int = 0,
               max_blocks_per_seq: int = 0, split_tokens: int = 0, dtype="bf16") -> GvaShape:
    return GvaShape(B, H, G, d_n, d_v, d_r, capacity, max_seq_len, block_size, num_blocks,
                    max_blocks_per_seq, split_tokens, _DTYPES[dtype])


def _ptr(t: Optional[torch.Tensor], dtype: Optional[torch.dtype], what: str, numel: int = 0):
    """Device pointer of `t` after checking it: a contiguous device tensor of
    `dtype` holding at least `numel` elements (the extent the C call will
    touch for the given shape; a shorter tensor would be read or written out
    of bounds by the kernels)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.numel() < numel:
        raise ValueError(f"{what} holds {t.numel()} elements; the shape needs at least {numel}")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _n_cache(shape: GvaShape, width: int) -> int:
    """Elements of a value-like cache ([.., G, .., width]) for `shape`."""
    if shape.block_size:
        return shape.num_blocks * shape.G * 64 * width
    return shape.B * shape.G * shape.capacity * width


def _n_kr(shape: GvaShape) -> int:
    """Elements of the positional-key cache for `shape`."""
    if shape.block_size:
        return shape.num_blocks * 64 * shape.d_r
    return shape.B * shape.capacity * shape.d_r


def _n_table(shape: GvaShape) -> int:
    return shape.B * shape.max_blocks_per_seq if shape.block_size else 0


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, fn: str):
    if status != _lib.GVA_OK:
        raise GvaError(status, fn)


def gva_append(shape: GvaShape, v_new, kr_new, n_new: int, seq_lens, v_cache, kr_cache,
               block_table=None, rope_base: float = 10000.0, stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    B, G, nn = shape.B, shape.G, max(int(n_new), 0)
    _check(lib.gva_append(shape, _ptr(v_new, dt, "v_new", B * G * nn * shape.d_v),
                          _ptr(kr_new, dt, "kr_new", B * nn * shape.d_r), int(n_new),
                          _ptr(seq_lens, torch.int32, "seq_lens", B),
                          _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                          _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                          _ptr(block_table, torch.int32, "block_table", _n_table(shape)), float(rope_base),
                          _stream(stream)), "gva_append")


def gva_rope_query(shape: GvaShape, q_rope_in, q_rope_out, seq_lens, rope_base: float = 10000.0,
                   stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    nr = shape.B * shape.H * shape.d_r
    _check(lib.gva_rope_query(shape, _ptr(q_rope_in, dt, "q_rope_in", nr),
                              _ptr(q_rope_out, dt, "q_rope_out", nr),
                              _ptr(seq_lens, torch.int32, "seq_lens", shape.B), float(rope_base),
                              _stream(stream)), "gva_rope_query")


def gva_decode(shape: GvaShape, q_nope, q_rope, M, v_cache, kr_cache, seq_lens, block_table,
               scale: float, out, workspace=None, stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    B, H = shape.B, shape.H
    _check(lib.gva_decode(shape, _ptr(q_nope, dt, "q_nope", B * H * shape.d_n),
                          _ptr(q_rope, dt, "q_rope", B * H * shape.d_r),
                          _ptr(M, dt, "M", H * shape.d_v * shape.d_n),
                          _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                          _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                          _ptr(seq_lens, torch.int32, "seq_lens", B),
                          _ptr(block_table, torch.int32, "block_table", _n_table(shape)), float(scale),
                          _ptr(out, dt, "out", B * H * shape.d_v), _ptr(workspace, None, "workspace"), ws_bytes,
                          _stream(stream)), "gva_decode")


def gva_decode_step(shape: GvaShape, v_new, kr_new, q_nope, q_rope, M, v_cache, kr_cache, seq_lens,
                    block_table, scale: float, rope_base: float, out, workspace, stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    B, H, G = shape.B, shape.H, shape.G
    _check(lib.gva_decode_step(shape, _ptr(v_new, dt, "v_new", B * G * shape.d_v),
                               _ptr(kr_new, dt, "kr_new", B * shape.d_r),
                               _ptr(q_nope, dt, "q_nope", B * H * shape.d_n),
                               _ptr(q_rope, dt, "q_rope", B * H * shape.d_r),
                               _ptr(M, dt, "M", H * shape.d_v * shape.d_n),
                               _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                               _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                               _ptr(seq_lens, torch.int32, "seq_lens", B),
                               _ptr(block_table, torch.int32, "block_table", _n_table(shape)), float(scale),
                               float(rope_base), _ptr(out, dt, "out", B * H * shape.d_v),
                               _ptr(workspace, None, "workspace"), ws_bytes, _stream(stream)),
           "gva_decode_step")


def gva_decode_step_noalloc(shape: GvaShape, v_new, kr_new, q_nope, q_rope, M, v_cache, kr_cache, seq_lens,
                            block_table, scale: float, rope_base: float, out, stream=None) -> None:
    """gva_decode_step without a workspace: the library's fixed per-device
    scratch (4 MiB) serves the split-K partials. Calls that overlap in time on
    one device race."""
    dt = _TORCH.get(shape.dtype)
    B, H, G = shape.B, shape.H, shape.G
    _check(lib.gva_decode_step_noalloc(shape, _ptr(v_new, dt, "v_new", B * G * shape.d_v),
                                       _ptr(kr_new, dt, "kr_new", B * shape.d_r),
                                       _ptr(q_nope, dt, "q_nope", B * H * shape.d_n),
                                       _ptr(q_rope, dt, "q_rope", B * H * shape.d_r),
                                       _ptr(M, dt, "M", H * shape.d_v * shape.d_n),
                                       _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                                       _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                                       _ptr(seq_lens, torch.int32, "seq_lens", B),
                                       _ptr(block_table, torch.int32, "block_table", _n_table(shape)),
                                       float(scale), float(rope_base), _ptr(out, dt, "out", B * H * shape.d_v),
                                       _stream(stream)), "gva_decode_step_noalloc")


def gva_rope_query_multi(shape: GvaShape, n_q: int, q_rope_in, q_rope_out, seq_lens,
                         rope_base: float = 10000.0, stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    nr = shape.B * max(int(n_q), 0) * shape.H * shape.d_r
    _check(lib.gva_rope_query_multi(shape, int(n_q), _ptr(q_rope_in, dt, "q_rope_in", nr),
                                    _ptr(q_rope_out, dt, "q_rope_out", nr),
                                    _ptr(seq_lens, torch.int32, "seq_lens", shape.B), float(rope_base),
                                    _stream(stream)), "gva_rope_query_multi")


def gva_decode_multi(shape: GvaShape, n_q: int, q_nope, q_rope, M, v_cache, kr_cache, seq_lens,
                     block_table, scale: float, out, workspace=None, stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    BQH = shape.B * max(int(n_q), 0) * shape.H
    _check(lib.gva_decode_multi(shape, int(n_q), _ptr(q_nope, dt, "q_nope", BQH * shape.d_n),
                                _ptr(q_rope, dt, "q_rope", BQH * shape.d_r),
                                _ptr(M, dt, "M", shape.H * shape.d_v * shape.d_n),
                                _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                                _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                                _ptr(seq_lens, torch.int32, "seq_lens", shape.B),
                                _ptr(block_table, torch.int32, "block_table", _n_table(shape)), float(scale),
                                _ptr(out, dt, "out", BQH * shape.d_v), _ptr(workspace, None, "workspace"), ws_bytes,
                                _stream(stream)), "gva_decode_multi")


def gva_decode_multi_workspace_bytes(shape: GvaShape, n_q: int) -> int:
    return int(lib.gva_decode_multi_workspace_bytes(shape, int(n_q)))


def gva_prefill(shape: GvaShape, n_q: int, q_nope, q_rope, M, v_cache, kr_cache, seq_lens, block_table,
                scale: float, out, stream=None) -> None:
    """Causal attention of the last n_q cached tokens of every sequence (any n_q;
    bf16): q_nope [B, n_q, H, d_n], q_rope [B, n_q, H, d_r] rotated, out
    [B, n_q, H, d_v]."""
    dt = _TORCH.get(shape.dtype)
    BQH = shape.B * max(int(n_q), 0) * shape.H
    _check(lib.gva_prefill(shape, int(n_q), _ptr(q_nope, dt, "q_nope", BQH * shape.d_n),
                           _ptr(q_rope, dt, "q_rope", BQH * shape.d_r),
                           _ptr(M, dt, "M", shape.H * shape.d_v * shape.d_n),
                           _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                           _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                           _ptr(seq_lens, torch.int32, "seq_lens", shape.B),
                           _ptr(block_table, torch.int32, "block_table", _n_table(shape)),
                           float(scale), _ptr(out, dt, "out", BQH * shape.d_v), _stream(stream)), "gva_prefill")


def gva_copy_blocks(shape: GvaShape, src_blocks, dst_blocks, v_cache, kr_cache, block_table=None,
                    remap_seqs=None, remap_slots=None, stream=None) -> None:
    """Copy whole 64-token blocks (int32 device index tensors); with remap_seqs
    and remap_slots also point those block-table slots at the copies."""
    dt = _TORCH.get(shape.dtype)
    n = int(src_blocks.numel())
    if int(dst_blocks.numel()) != n or (remap_seqs is not None and int(remap_seqs.numel()) != n):
        raise ValueError("index tensors must have the same length")
    _check(lib.gva_copy_blocks(shape, _ptr(src_blocks, torch.int32, "src_blocks"),
                               _ptr(dst_blocks, torch.int32, "dst_blocks"), n,
                               _ptr(remap_seqs, torch.int32, "remap_seqs"),
                               _ptr(remap_slots, torch.int32, "remap_slots", n if remap_seqs is not None else 0),
                               _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                               _ptr(kr_cache, dt, "kr_cache", _n_kr(shape)),
                               _ptr(block_table, torch.int32, "block_table", _n_table(shape)),
                               _stream(stream)), "gva_copy_blocks")


def gva_fork(shape: GvaShape, src_seqs, dst_seqs, seq_lens, block_table, stream=None) -> None:
    n = int(src_seqs.numel())
    if int(dst_seqs.numel()) != n:
        raise ValueError("src_seqs and dst_seqs must have the same length")
    _check(lib.gva_fork(shape, _ptr(src_seqs, torch.int32, "src_seqs"), _ptr(dst_seqs, torch.int32, "dst_seqs"),
                        n, _ptr(seq_lens, torch.int32, "seq_lens", shape.B),
                        _ptr(block_table, torch.int32, "block_table", _n_table(shape)), _stream(stream)), "gva_fork")


def gva_rollback(shape: GvaShape, seq_lens, n_drop, stream=None) -> None:
    _check(lib.gva_rollback(shape, _ptr(seq_lens, torch.int32, "seq_lens", shape.B),
                            _ptr(n_drop, torch.int32, "n_drop", shape.B),
                            _stream(stream)), "gva_rollback")


def gva_fold_query_projection(M, wq_nope, w_fold, stream=None) -> None:
    """w_fold[h] = M[h] @ wq_nope[h]: M [H, d_v, d_n], wq_nope [H, d_n, d_model],
    w_fold [H, d_v, d_model], all of one dtype (bf16 or fp32)."""
    if M.dim() != 3 or wq_nope.dim() != 3 or w_fold.dim() != 3:
        raise ValueError("M, wq_nope and w_fold must be 3-D")
    H, d_v, d_n = M.shape
    d_model = wq_nope.shape[2]
    if tuple(wq_nope.shape) != (H, d_n, d_model) or tuple(w_fold.shape) != (H, d_v, d_model):
        raise ValueError(f"shapes M {tuple(M.shape)}, wq_nope {tuple(wq_nope.shape)}, "
                         f"w_fold {tuple(w_fold.shape)} do not match")
    code = {torch.bfloat16: 1, torch.float32: 0}.get(M.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {M.dtype}")
    _check(lib.gva_fold_query_projection(H, d_v, d_n, d_model, code, _ptr(M, M.dtype, "M"),
                                         _ptr(wq_nope, M.dtype, "wq_nope"),
                                         _ptr(w_fold, M.dtype, "w_fold"), _stream(stream)),
           "gva_fold_query_projection")


def gva_query_projection(shape: GvaShape, x, w_fold, w_rope, q_abs, q_rope, stream=None) -> None:
    """q_abs = w_fold . x and q_rope = w_rope . x (pre-RoPE) for the B new tokens:
    x [B, d_model], w_fold [H, d_v, d_model], w_rope [H, d_r, d_model]."""
    dt = _TORCH.get(shape.dtype)
    d_model = x.shape[-1]
    B, H = shape.B, shape.H
    _check(lib.gva_query_projection(shape, int(d_model), _ptr(x, dt, "x", B * d_model),
                                    _ptr(w_fold, dt, "w_fold", H * shape.d_v * d_model),
                                    _ptr(w_rope, dt, "w_rope", H * shape.d_r * d_model),
                                    _ptr(q_abs, dt, "q_abs", B * H * shape.d_v),
                                    _ptr(q_rope, dt, "q_rope", B * H * shape.d_r), _stream(stream)),
           "gva_query_projection")


def gva_gqa_ref_decode(shape: GvaShape, q, k_cache, v_cache, seq_lens, block_table, scale: float,
                       out, workspace=None, stream=None) -> None:
    dt = _TORCH.get(shape.dtype)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    B, H = shape.B, shape.H
    _check(lib.gva_gqa_ref_decode(shape, _ptr(q, dt, "q", B * H * shape.d_n),
                                  _ptr(k_cache, dt, "k_cache", _n_cache(shape, shape.d_n)),
                                  _ptr(v_cache, dt, "v_cache", _n_cache(shape, shape.d_v)),
                                  _ptr(seq_lens, torch.int32, "seq_lens", B),
                                  _ptr(block_table, torch.int32, "block_table", _n_table(shape)), float(scale),
                                  _ptr(out, dt, "out", B * H * shape.d_v), _ptr(workspace, None, "workspace"),
                                  ws_bytes, _stream(stream)), "gva_gqa_ref_decode")


def gva_decode_workspace_bytes(shape: GvaShape) -> int:
    return int(lib.gva_decode_workspace_bytes(shape))


def gva_decode_step_workspace_bytes(shape: GvaShape) -> int:
    return int(lib.gva_decode_step_workspace_bytes(shape))


def gva_decode_split_tokens(shape: GvaShape) -> int:
    return int(lib.gva_decode_split_tokens(shape))


def gva_cache_bytes_per_token(G: int, d_v: int, d_r: int, dtype="bf16") -> int:
    return int(lib.gva_cache_bytes_per_token(G, d_v, d_r, _DTYPES[dtype]))


def gva_status_string(status: int) -> str:
    return lib.gva_status_string(status).decode()


def gva_abi_version() -> int:
    return int(lib.gva_abi_version())


def workspace_for(shape: GvaShape, device="cuda") -> Optional[torch.Tensor]:
    """Zero-filled device workspace of the size gva_decode needs (None if none)."""
    n = gva_decode_workspace_bytes(shape)
    if n == 0:
        return None
    return torch.zeros((n + 3) // 4, dtype=torch.float32, device=device)
