"""GPU test of gva_decode_step_noalloc, the fused decode step without a
workspace argument (for callers that cannot allocate device memory). Through
the C ABI its output, lengths and caches equal those of gva_decode_step with a
caller workspace bit for bit, on two calls in a row (the second with a smaller
batch, shorter sequences and an explicit partition), and a shape whose
scratch need exceeds the library's fixed array is refused."""
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


def _compare(B, lens, split, seed):
    wl = W.Workload("noalloc", 9, B=B, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.asarray(lens)
    inp = W.make_gva_inputs(wl, lens=lens, extra=1, seed=seed)
    cap = int(lens.max()) + 1
    ca, cb = (GvaCache(B, 16, 4, 64, 64, 16, dtype="bf16", capacity=cap) for _ in range(2))
    for c in (ca, cb):
        for b, n in enumerate(lens):
            c.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), S.dev(inp.kr[b][:n], "bf16"), BASE)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    v1 = S.dev(np.stack([inp.V[b][:, n] for b, n in enumerate(lens)]), "bf16")
    k1 = S.dev(np.stack([inp.kr[b][n] for b, n in enumerate(lens)]), "bf16")
    out_a = torch.full((B, 16, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_b = torch.full_like(out_a, float("nan"))
    print(f"[case] noalloc B={B} max_len={cap} split={split}", flush=True)
    ca.step(v1, k1, qn, qr, Md, wl.scale, out_a, cap, split, workspace=ca.step_workspace(cap, split))
    gva.gva_decode_step_noalloc(cb.shape(cap, split), v1, k1, qn, qr, Md, cb.v_cache, cb.kr_cache, cb.seq_lens,
                                None, wl.scale, BASE, out_b)
    torch.cuda.synchronize()
    assert not torch.isnan(out_b.float()).any()
    assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
    assert torch.equal(ca.seq_lens, cb.seq_lens)
    assert torch.equal(ca.v_cache, cb.v_cache) and torch.equal(ca.kr_cache, cb.kr_cache)


def test_noalloc_step_equals_step_on_two_calls():
    # the mid shape (16 sequences of 4096 tokens, automatic partitions), then a
    # smaller batch with mixed lengths and 256-token partitions
    _compare(16, [4096] * 16, 0, seed=101)
    _compare(3, [700, 65, 1200], 256, seed=102)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    # 64 sequences of up to 131072 tokens in 4096-token partitions need 8.6 MB
    # of partials, more than the fixed 4 MiB; refused before any launch
    B, mb = 64, 2048
    shape = gva.make_shape(B, 16, 4, 64, 64, 16, max_seq_len=mb * 64, block_size=64, num_blocks=1,
                           max_blocks_per_seq=mb, split_tokens=4096, dtype="bf16")
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    table = torch.zeros(B, mb, dtype=torch.int32, device="cuda")
    with pytest.raises(gva.GvaError, match="GVA_ERR_WORKSPACE"):
        gva.gva_decode_step_noalloc(shape, z(B, 4, 64), z(B, 16), z(B, 16, 64), z(B, 16, 16), z(16, 64, 64),
                                    z(1, 4, 64, 64), z(1, 64, 16), lens, table, 0.1, BASE, z(B, 16, 64))


def test_noalloc_step_under_graph_capture():
    """The callers this entry point is for capture it: three allocation-free
    fused steps captured in one graph, replayed three times with eager work
    between the replays, equal nine eager steps through gva_decode_step with a
    caller workspace on an identical cache, bit for bit after every replay."""
    wl = W.Workload("noalloc_graph", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([500, 1030, 77])
    inp = W.make_gva_inputs(wl, lens=lens, extra=10, seed=103)
    cap = 1100
    ca, cb = (GvaCache(3, 16, 4, 64, 64, 16, dtype="bf16", capacity=cap) for _ in range(2))
    for c in (ca, cb):
        for b, n in enumerate(lens):
            c.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), S.dev(inp.kr[b][:n], "bf16"), BASE)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    news = [(S.dev(np.stack([inp.V[b][:, n + i] for b, n in enumerate(lens)]), "bf16"),
             S.dev(np.stack([inp.kr[b][n + i] for b, n in enumerate(lens)]), "bf16")) for i in range(4)]
    split = 128
    shape = ca.shape(cap, split)
    out_a = torch.empty(3, 16, 64, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    ws_b = cb.step_workspace(cap, split)
    print("[case] noalloc graph capture", flush=True)
    # one eager call on each side first (the scratch is set up outside capture)
    v0, k0 = news[0]
    gva.gva_decode_step_noalloc(shape, v0, k0, qn, qr, Md, ca.v_cache, ca.kr_cache, ca.seq_lens, None, wl.scale,
                                BASE, out_a)
    cb.step(v0, k0, qn, qr, Md, wl.scale, out_b, cap, split, workspace=ws_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for v1, k1 in news[1:]:
            gva.gva_decode_step_noalloc(shape, v1, k1, qn, qr, Md, ca.v_cache, ca.kr_cache, ca.seq_lens, None,
                                        wl.scale, BASE, out_a)
    torch.cuda.synchronize()
    assert ca.seq_lens.cpu().tolist() == (lens + 1).tolist()  # capture runs nothing
    for rep in range(3):
        print(f"[case] noalloc graph replay {rep}", flush=True)
        g.replay()
        for v1, k1 in news[1:]:
            cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, cap, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens), rep
        assert torch.equal(out_a, out_b), rep
        assert torch.equal(ca.v_cache, cb.v_cache) and torch.equal(ca.kr_cache, cb.kr_cache), rep
    assert ca.seq_lens.cpu().tolist() == (lens + 10).tolist()
