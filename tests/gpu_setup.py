"""Shared set-up for the GPU tests: move seeded workloads onto the device in
the layouts the library expects, and the tolerance checks. Uses only the
workload generator and the package's binding (no oracle arithmetic)."""
from __future__ import annotations

import math

import numpy as np
import torch

import workloads as W

BF16_MAX_ABS = 2e-2
BF16_REL = 1e-2
F32_REL = 1e-5


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    return W.to_torch(x, dtype).cuda()


def errors(out: np.ndarray, ref: np.ndarray):
    d = out - ref
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    rows_d = np.linalg.norm(d.reshape(-1, d.shape[-1]), axis=1)
    rows_r = np.linalg.norm(ref.reshape(-1, ref.shape[-1]), axis=1)
    live = rows_r > 0
    row_rel = float(np.max(rows_d[live] / rows_r[live])) if live.any() else 0.0
    return dict(max_abs=float(np.max(np.abs(d))) if d.size else 0.0, rel=rel, row_rel=row_rel,
                ref_max=float(np.max(np.abs(ref))) if ref.size else 0.0)


def assert_close(out: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    e = errors(out, ref)
    print(f"[parity] {what} dtype={dtype} max_abs={e['max_abs']:.3e} rel={e['rel']:.3e} "
          f"row_rel={e['row_rel']:.3e}", flush=True)
    if dtype == "f32":
        assert e["rel"] <= F32_REL, e
        assert e["max_abs"] <= F32_REL * e["ref_max"], e
    else:
        assert e["max_abs"] <= BF16_MAX_ABS, e
        assert e["rel"] <= BF16_REL, e
        assert e["row_rel"] <= BF16_REL, e
    return e


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def uniform_cache_from_host(wl: W.Workload, V_rows, kr_rows, capacity: int, lens):
    """Contiguous cache tensors holding the given (already final) rows."""
    v = W.contiguous_cache(V_rows, capacity, token_axis=1)          # [B, G, cap, d_v]
    k = W.contiguous_cache(kr_rows, capacity, token_axis=0)         # [B, cap, d_r]
    seq = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    return dev(v, wl.dtype), dev(k, wl.dtype), seq


def paged_cache_from_host(wl: W.Workload, V_rows, kr_rows, lens_cap, seed: int):
    table, n_blocks = W.paged_pool(np.asarray(lens_cap), 64, seed)
    vp, kp = W.scatter_paged(V_rows, kr_rows, table, n_blocks, 64)
    return dev(vp, wl.dtype), dev(kp, wl.dtype), torch.tensor(table, device="cuda"), n_blocks


def workspace(shape):
    import compact_kv_cache_amd as gva
    n = gva.gva_decode_workspace_bytes(shape)
    return None if n == 0 else torch.zeros((n + 3) // 4, dtype=torch.float32, device="cuda")


def scale_of(wl: W.Workload) -> float:
    return wl.scale


def gqa_scale(d_h: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d_h)))
