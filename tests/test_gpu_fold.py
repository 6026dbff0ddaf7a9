"""GPU tests of the maps folded into the query projection: gva_fold_query_projection,
gva_query_projection, and gva_decode / gva_decode_step with M = NULL (the
absorbed queries given directly), against the CPU oracle's plain layer step
(q_nope = W_q,nope x, materialized keys V M)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_setup as S

pytestmark = pytest.mark.gpu

gva = pytest.importorskip("compact_kv_cache_amd")
from compact_kv_cache_amd.cache import GvaCache  # noqa: E402

BASE = 10000.0
D_MODEL = 1024  # H * d_n: the hidden width of a standard layer with these heads


@pytest.fixture(autouse=True)
def _gpu():
    S.need_gpu()
    yield
    torch.cuda.synchronize()


def _rel(got, ref):
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fold_matches_oracle(dtype):
    wl = W.Workload("fold", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype=dtype)
    inp = W.make_gva_inputs(wl, lens=np.array([1, 1]))
    _, wq_nope, _ = W.make_projection_inputs(wl, D_MODEL)
    print(f"[case] fold dtype={dtype}", flush=True)
    w_fold = torch.empty(16, 64, D_MODEL, dtype=W.torch_dtype(dtype), device="cuda")
    gva.gva_fold_query_projection(S.dev(inp.M, dtype), S.dev(wq_nope, dtype), w_fold)
    ref = O.fold_query_projection(inp.M, wq_nope)
    got = S.host(w_fold)
    if dtype == "f32":
        assert _rel(got, ref) <= 1e-6
    else:  # fp32 sum of 64 products, rounded once to bf16
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6), np.abs(got - ref).max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B", [16, 5])
def test_projection_matches_oracle(dtype, B):
    wl = W.Workload("proj", 9, B=B, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype=dtype)
    x, wq_nope, wq_rope = W.make_projection_inputs(wl, D_MODEL)
    print(f"[case] projection dtype={dtype} B={B}", flush=True)
    shape = gva.make_shape(B, 16, 4, 64, 64, 16, capacity=64, max_seq_len=64, dtype=dtype)
    td = W.torch_dtype(dtype)
    q_abs = torch.empty(B, 16, 64, dtype=td, device="cuda")
    q_rope = torch.empty(B, 16, 16, dtype=td, device="cuda")
    gva.gva_query_projection(shape, S.dev(x, dtype), S.dev(wq_nope, dtype), S.dev(wq_rope, dtype),
                             q_abs, q_rope)
    for got, w in ((q_abs, wq_nope), (q_rope, wq_rope)):
        ref = O.query_projection(x, w)
        g = S.host(got)
        if dtype == "f32":
            assert _rel(g, ref) <= 1e-5
        else:  # fp32 accumulation of 1024 products, rounded once
            assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 2e-3), np.abs(g - ref).max()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("paged", [False, True])
def test_folded_layer_step_matches_oracle(dtype, paged):
    """Prefill, then fold once, project the new tokens' hidden states and run
    the fused step without M, twice; each against the oracle's plain layer
    step from the same hidden states."""
    wl = W.Workload("fold_step", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype=dtype)
    lens = np.array([900, 64, 2100])
    inp = W.make_gva_inputs(wl, lens=lens, extra=2, seed=21)
    cap = 2200
    if paged:
        table, nblk = W.paged_pool(np.full(wl.B, cap), 64, 5)
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, 16, dtype=dtype, block_table=torch.tensor(table),
                         num_blocks=nblk)
    else:
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, 16, dtype=dtype, capacity=cap)
    for b, n in enumerate(lens):
        cache.append_one(b, S.dev(inp.V[b][:, :n], dtype), S.dev(inp.kr[b][:n], dtype), BASE)
    td = W.torch_dtype(dtype)
    _, wq_nope, wq_rope = W.make_projection_inputs(wl, D_MODEL, seed=22)
    w_fold = torch.empty(16, 64, D_MODEL, dtype=td, device="cuda")
    gva.gva_fold_query_projection(S.dev(inp.M, dtype), S.dev(wq_nope, dtype), w_fold)
    wr = S.dev(wq_rope, dtype)
    q_abs = torch.empty(wl.B, 16, 64, dtype=td, device="cuda")
    q_rope = torch.empty(wl.B, 16, 16, dtype=td, device="cuda")
    out = torch.empty(wl.B, 16, 64, dtype=td, device="cuda")
    ws = cache.step_workspace(cap, 256)
    rng = np.random.default_rng(23)
    for i in range(2):
        print(f"[case] folded layer step dtype={dtype} paged={paged} i={i}", flush=True)
        x = W.round_storage(rng.standard_normal((wl.B, D_MODEL)), dtype)
        shape = cache.shape(cap, 256)
        gva.gva_query_projection(shape, S.dev(x, dtype), w_fold, wr, q_abs, q_rope)
        v_new = S.dev(np.stack([inp.V[b][:, n + i] for b, n in enumerate(lens)]), dtype)
        k_new = S.dev(np.stack([inp.kr[b][n + i] for b, n in enumerate(lens)]), dtype)
        cache.step(v_new, k_new, q_abs, q_rope, None, wl.scale, out, cap, 256, workspace=ws)
        torch.cuda.synchronize()
        ref = O.gva_layer_decode_step(inp.V, inp.kr, x, wq_nope, wq_rope, inp.M, lens + i + 1, wl.scale,
                                      BASE, dtype)
        S.assert_close(S.host(out), ref, dtype, f"folded layer step {dtype} paged={paged} {i}")
    assert cache.seq_lens.cpu().tolist() == (lens + 2).tolist()


def test_decode_without_maps_equals_decode_with_folded_queries():
    """gva_decode with M = NULL on q' = M q_nope (formed by the oracle and
    rounded to bf16) against gva_decode with M on q_nope: both within the
    tolerance of the oracle, and close to each other."""
    wl = W.WORKLOADS["mid_bf16"].replace(B=4, S=3000)
    inp = W.make_gva_inputs(wl, seed=31)
    cache = GvaCache(4, 16, 4, 64, 64, 16, dtype="bf16", capacity=3000)
    cache.append(S.dev(np.stack(inp.V), "bf16"), S.dev(np.stack(inp.kr), "bf16"), BASE)
    q_rot = torch.empty(4, 16, 16, dtype=torch.bfloat16, device="cuda")
    gva.gva_rope_query(cache.shape(3000), S.dev(inp.q_rope, "bf16"), q_rot, cache.seq_lens, BASE)
    q_abs = np.einsum("hvn,bhn->bhv", inp.M, inp.q_nope)
    out_m = torch.empty(4, 16, 64, dtype=torch.bfloat16, device="cuda")
    out_f = torch.empty_like(out_m)
    print("[case] decode with and without maps", flush=True)
    cache.decode(S.dev(inp.q_nope, "bf16"), q_rot, S.dev(inp.M, "bf16"), wl.scale, out_m, 3000)
    cache.decode(S.dev(q_abs, "bf16"), q_rot, None, wl.scale, out_f, 3000)
    torch.cuda.synchronize()
    ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, inp.lens, wl.scale, BASE, "bf16")
    S.assert_close(S.host(out_m), ref, "bf16", "decode with M")
    S.assert_close(S.host(out_f), ref, "bf16", "decode without M (folded queries)")


def test_projection_validation():
    shape = gva.make_shape(2, 16, 4, 64, 64, 16, capacity=64, max_seq_len=64, dtype="bf16")
    x = torch.zeros(2, 1000, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16, 64, 1000, dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros(16, 16, 1000, dtype=torch.bfloat16, device="cuda")
    qa = torch.zeros(2, 16, 64, dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros(2, 16, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gva.GvaError, match="128"):
        gva.gva_query_projection(shape, x, w, wr, qa, qr)
    with pytest.raises(gva.GvaError, match="non-NULL"):
        gva.gva_query_projection(shape, torch.zeros(2, 1024, dtype=torch.bfloat16, device="cuda"),
                                 torch.zeros(16, 64, 1024, dtype=torch.bfloat16, device="cuda"), None, qa, None)
