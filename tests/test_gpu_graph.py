"""HIP graph capture of the decode and of the fused step: every replay, with
eager work and synchronizations between replays, equals the eager calls bit
for bit. (No call of the library records a memset: the split-K counters are
zero-filled once with the workspace and reset by the kernels themselves.)"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import gpu_setup as S

pytestmark = pytest.mark.gpu

gva = pytest.importorskip("compact_kv_cache_amd")
from compact_kv_cache_amd.cache import GvaCache  # noqa: E402

BASE = 10000.0


@pytest.fixture(autouse=True)
def _gpu():
    S.need_gpu()
    yield
    torch.cuda.synchronize()


def _filled_cache(wl, inp, lens, cap):
    c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", capacity=cap)
    for b, n in enumerate(lens):
        c.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), S.dev(inp.kr[b][:n], "bf16"), BASE)
    torch.cuda.synchronize()
    return c


def test_decode_graph_replays_match_eager():
    wl = W.Workload("graph", 9, B=4, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([700, 1500, 64, 2049])
    inp = W.make_gva_inputs(wl, lens=lens, seed=11)
    cache = _filled_cache(wl, inp, lens, 2100)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    split = 256
    ws = cache.workspace(2100, split)
    out_e = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    cache.decode(qn, qr, Md, wl.scale, out_e, 2100, split, workspace=ws)
    torch.cuda.synchronize()

    out_g = torch.empty_like(out_e)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            cache.decode(qn, qr, Md, wl.scale, out_g, 2100, split, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        print(f"[case] decode graph replay {rep}", flush=True)
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), rep
        # eager work between replays, sharing the workspace
        other = torch.empty_like(out_e)
        cache.decode(qn, qr, Md, wl.scale, other, 2100, split, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(other, out_e)


def test_step_graph_replays_match_eager_steps():
    """Three captured fused steps, replayed three times, against nine eager
    steps with the same inputs on an identical cache: output, caches and
    lengths agree after every replay."""
    wl = W.Workload("graph_step", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([500, 1030, 77])
    inp = W.make_gva_inputs(wl, lens=lens, extra=3, seed=12)
    cap = 1100
    ca = _filled_cache(wl, inp, lens, cap)    # graph
    cb = _filled_cache(wl, inp, lens, cap)    # eager
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    news = [(S.dev(np.stack([inp.V[b][:, n + i] for b, n in enumerate(lens)]), "bf16"),
             S.dev(np.stack([inp.kr[b][n + i] for b, n in enumerate(lens)]), "bf16")) for i in range(3)]
    split = 128
    ws_a, ws_b = ca.step_workspace(cap, split), cb.step_workspace(cap, split)
    out_a = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for v1, k1 in news:
            ca.step(v1, k1, qn, qr, Md, wl.scale, out_a, cap, split, workspace=ws_a)
    torch.cuda.synchronize()
    # capture does not run the kernels
    assert ca.seq_lens.cpu().tolist() == lens.tolist()
    for rep in range(3):
        print(f"[case] step graph replay {rep}", flush=True)
        g.replay()
        for v1, k1 in news:
            cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, cap, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens), rep
        assert torch.equal(out_a, out_b), rep
        assert torch.equal(ca.v_cache, cb.v_cache) and torch.equal(ca.kr_cache, cb.kr_cache), rep
    assert ca.seq_lens.cpu().tolist() == (lens + 9).tolist()
