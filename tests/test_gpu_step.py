"""GPU tests of the fused decode step (gva_decode_step): bit-for-bit equal to
gva_append + gva_rope_query + gva_decode on an identical cache, and equal to
the CPU oracle's step within the decode tolerance."""
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


@pytest.fixture(autouse=True)
def _gpu():
    S.need_gpu()
    yield
    torch.cuda.synchronize()


def _pair_of_caches(wl, lens, cap, paged, seed, kr_boost=()):
    """Two identical caches (one per path) prefilled with the same tokens.
    `kr_boost`: (first token, factor) pairs scaling the positional keys (before
    rotation) of every sequence from that token on; powers of two keep them
    exact."""
    inp = W.make_gva_inputs(wl, lens=lens, extra=8, seed=seed)
    for t0, factor in kr_boost:
        for rows in inp.kr:
            rows[t0:] *= factor
    caches = []
    table = nblk = None
    if paged:
        table, nblk = W.paged_pool(np.full(wl.B, cap), 64, seed)
    for _ in range(2):
        if paged:
            c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype=wl.dtype,
                         block_table=torch.tensor(table), num_blocks=nblk)
        else:
            c = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype=wl.dtype, capacity=cap)
        for b, n in enumerate(lens):
            if n > 0:
                kr = None if wl.d_r == 0 else S.dev(inp.kr[b][:n], wl.dtype)
                c.append_one(b, S.dev(inp.V[b][:, :n], wl.dtype), kr, BASE)
        caches.append(c)
    torch.cuda.synchronize()
    return inp, caches


def _new_token(inp, lens, i, dtype):
    v = np.stack([inp.V[b][:, n + i] for b, n in enumerate(lens)])   # [B, G, d_v]
    k = np.stack([inp.kr[b][n + i] for b, n in enumerate(lens)])     # [B, d_r]
    return S.dev(v, dtype), S.dev(k, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("split", [0, 64, 256])
def test_step_equals_three_calls(dtype, paged, split):
    wl = W.Workload("step", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype=dtype)
    lens = np.array([300, 77, 1000])
    cap = 1100
    inp, (ca, cb) = _pair_of_caches(wl, lens, cap, paged, seed=7)
    qn, qr, Md = (S.dev(x, dtype) for x in (inp.q_nope, inp.q_rope, inp.M))
    td = W.torch_dtype(dtype)
    out_a = torch.empty(wl.B, wl.H, 64, dtype=td, device="cuda")
    out_b = torch.empty_like(out_a)
    q_rot = torch.empty_like(qr)
    ws_b = cb.step_workspace(int(lens.max()) + 3, split)
    for i in range(3):
        max_len = int(lens.max()) + i + 1
        print(f"[case] step dtype={dtype} paged={paged} split={split} i={i}", flush=True)
        v1, k1 = _new_token(inp, lens, i, dtype)
        ca.append(v1.unsqueeze(2).contiguous(), k1.unsqueeze(1).contiguous(), BASE)
        gva.gva_rope_query(ca.shape(max_len, split), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, max_len, split)
        cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, max_len, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
    assert torch.equal(ca.v_cache, cb.v_cache)
    assert torch.equal(ca.kr_cache, cb.kr_cache)
    assert torch.equal(qr, S.dev(inp.q_rope, dtype)), "q_rope must not be modified"


@pytest.mark.parametrize("hpg,d_r", [(4, 8), (4, 24), (4, 32), (1, 16), (2, 16), (2, 24)])
def test_step_positional_widths_and_head_groups(hpg, d_r):
    """Fused step at the other positional widths (the rotation spans one or
    two waves of the workgroup) and heads per group: bit-for-bit equal to the
    three calls, and within tolerance of the oracle's step."""
    wl = W.Workload("step_shapes", 9, B=3, H=4 * hpg, G=4, d_n=64, d_v=64, d_r=d_r, S=0, dtype="bf16")
    lens = np.array([300, 77, 700])
    cap = 800
    inp, (ca, cb) = _pair_of_caches(wl, lens, cap, False, seed=11 + d_r + hpg)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    out_a = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    q_rot = torch.empty_like(qr)
    ws_b = cb.step_workspace(int(lens.max()) + 3, 256)
    for i in range(2):
        max_len = int(lens.max()) + i + 1
        print(f"[case] step hpg={hpg} d_r={d_r} i={i}", flush=True)
        v1, k1 = _new_token(inp, lens, i, "bf16")
        ca.append(v1.unsqueeze(2).contiguous(), k1.unsqueeze(1).contiguous(), BASE)
        gva.gva_rope_query(ca.shape(max_len, 256), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, max_len, 256)
        cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, max_len, 256, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
        ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, lens + i + 1, wl.scale, BASE, "bf16")
        S.assert_close(S.host(out_b), ref, "bf16", f"fused step hpg={hpg} d_r={d_r} i={i}")
    assert torch.equal(ca.v_cache, cb.v_cache)
    assert torch.equal(ca.kr_cache, cb.kr_cache)


def test_step_matches_oracle_mid():
    """Mid-workload shape (B=16, S=4096): prefill, then two fused steps, each
    against the oracle's step from pre-RoPE inputs."""
    wl = W.WORKLOADS["mid_bf16"]
    inp = W.make_gva_inputs(wl, extra=2)
    cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", capacity=wl.S + 2)
    Vd = S.dev(np.stack(inp.V), "bf16")
    Kd = S.dev(np.stack(inp.kr), "bf16")
    cache.append(Vd[:, :, :wl.S].contiguous(), Kd[:, :wl.S].contiguous(), BASE)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    out = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    ws = cache.step_workspace(wl.S + 2)
    for i in range(2):
        n = wl.S + i + 1
        print(f"[case] fused step mid i={i}", flush=True)
        cache.step(Vd[:, :, n - 1].contiguous(), Kd[:, n - 1].contiguous(), qn, qr, Md, wl.scale,
                   out, n, workspace=ws)
        ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, np.full(wl.B, n),
                                wl.scale, BASE, "bf16")
        S.assert_close(S.host(out), ref, "bf16", f"fused step mid {i}")
    assert cache.seq_lens.cpu().tolist() == [wl.S + 2] * wl.B


def test_step_from_empty_and_when_full():
    wl = W.Workload("step_edge", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([0, 62])
    cap = 64
    inp, (ca, cb) = _pair_of_caches(wl, lens, cap, False, seed=9)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    out_a = torch.empty(2, 16, 64, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    q_rot = torch.empty_like(qr)
    ws = cb.step_workspace(cap)
    for i in range(4):           # sequence 1 reaches the capacity and stays there
        print(f"[case] step edge i={i}", flush=True)
        v1, k1 = _new_token(inp, lens, i, "bf16")
        ca.append(v1.unsqueeze(2).contiguous(), k1.unsqueeze(1).contiguous(), BASE)
        gva.gva_rope_query(ca.shape(cap), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, cap)
        cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, cap, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(out_a, out_b)
        if i == 0:   # a single token: the output is that token's value row
            assert torch.equal(out_b[0], v1[0].repeat_interleave(4, dim=0))
    assert cb.seq_lens.cpu().tolist() == [4, 64]
    assert torch.equal(ca.v_cache, cb.v_cache) and torch.equal(ca.kr_cache, cb.kr_cache)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("split", [0, 256])
def test_step_equals_three_calls_moving_reference(paged, split):
    """Positional keys scaled by 8 from token 640 on and by 32 from token 1600
    on, so the softmax reference of every column moves in the middle of the
    sequence (the decode's rescale branch, checked against the oracle in the
    parity tests): the fused step stays bit-identical to the three calls."""
    wl = W.Workload("step_move", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([2100, 1700, 900])
    cap = 2200
    inp, (ca, cb) = _pair_of_caches(wl, lens, cap, paged, seed=17, kr_boost=((640, 8.0), (1600, 4.0)))
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    out_a = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    q_rot = torch.empty_like(qr)
    ws_b = cb.step_workspace(int(lens.max()) + 2, split)
    for i in range(2):
        max_len = int(lens.max()) + i + 1
        print(f"[case] step moving reference paged={paged} split={split} i={i}", flush=True)
        v1, k1 = _new_token(inp, lens, i, "bf16")
        ca.append(v1.unsqueeze(2).contiguous(), k1.unsqueeze(1).contiguous(), BASE)
        gva.gva_rope_query(ca.shape(max_len, split), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, max_len, split)
        cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, max_len, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
        assert torch.isfinite(out_a.float()).all()


@pytest.mark.parametrize("paged", [False, True])
def test_step_two_partitions_per_workgroup(paged):
    """64-token partitions over 33-34 partitions and 16 (sequence, group)
    pairs: two partitions per workgroup in the fused step and in the decode
    of the three calls, bit for bit equal, and the step against the oracle's
    step; the steps carry the longest sequence across a partition boundary."""
    wl = W.Workload("step_ppw", 9, B=4, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([2111, 2048, 1000, 0])
    cap = 2200
    split = 64
    inp, (ca, cb) = _pair_of_caches(wl, lens, cap, paged, seed=27)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    out_a = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    q_rot = torch.empty_like(qr)
    ws_b = cb.step_workspace(int(lens.max()) + 2, split)
    for i in range(2):
        max_len = int(lens.max()) + i + 1
        print(f"[case] step two partitions per workgroup paged={paged} i={i}", flush=True)
        v1, k1 = _new_token(inp, lens, i, "bf16")
        ca.append(v1.unsqueeze(2).contiguous(), k1.unsqueeze(1).contiguous(), BASE)
        gva.gva_rope_query(ca.shape(max_len, split), qr, q_rot, ca.seq_lens, BASE)
        ca.decode(qn, q_rot, Md, wl.scale, out_a, max_len, split)
        cb.step(v1, k1, qn, qr, Md, wl.scale, out_b, max_len, split, workspace=ws_b)
        torch.cuda.synchronize()
        assert torch.equal(ca.seq_lens, cb.seq_lens)
        assert torch.equal(out_a, out_b), (out_a.float() - out_b.float()).abs().max()
        ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, lens + i + 1, wl.scale, BASE,
                                "bf16")
        S.assert_close(S.host(out_b), ref, "bf16", f"step two partitions per workgroup i={i}")
    assert torch.equal(ca.v_cache, cb.v_cache)
    assert torch.equal(ca.kr_cache, cb.kr_cache)
