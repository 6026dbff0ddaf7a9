"""GPU tests of the decode of several new tokens' queries at once
(gva_decode_multi, gva_rope_query_multi): query j of a sequence with n cached
tokens sits at n - n_q + j and reads the cache up to its own token. Against
the CPU oracle from pre-RoPE inputs."""
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


def _run(wl, lens, nq, *, paged, split, seed):
    """Prefill lens - nq tokens, append the nq new ones in one gva_append,
    rotate the nq queries, decode them. Returns (gpu, oracle) [B, nq, H, d_v]."""
    inp = W.make_gva_inputs(wl, lens=lens, seed=seed)
    rng = np.random.default_rng(seed + 1)
    qn = W.round_storage(rng.standard_normal((wl.B, nq, wl.H, wl.d_n)), "bf16")
    qr = W.round_storage(rng.standard_normal((wl.B, nq, wl.H, wl.d_r)), "bf16")
    cap = int(max(lens)) + 70
    if paged:
        table, nblk = W.paged_pool(np.full(wl.B, cap), 64, seed + 2)
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16",
                         block_table=torch.tensor(table), num_blocks=nblk)
    else:
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", capacity=cap)
    pre = np.maximum(lens - nq, 0)
    for b, n in enumerate(pre):
        if n > 0:
            cache.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), S.dev(inp.kr[b][:n], "bf16"), BASE)
    # the nq new tokens of every sequence in one append (sequences shorter than
    # nq get all their tokens here)
    newv = np.zeros((wl.B, wl.G, nq, 64))
    newk = np.zeros((wl.B, nq, wl.d_r))
    counts = lens - pre
    assert np.all(counts == np.minimum(lens, nq))
    for b in range(wl.B):
        newv[b, :, :counts[b]] = inp.V[b][:, pre[b]:lens[b]]
        newk[b, :counts[b]] = inp.kr[b][pre[b]:lens[b]]
    if np.all(counts == nq):
        cache.append(S.dev(newv, "bf16"), S.dev(newk, "bf16"), BASE)
    else:
        for b in range(wl.B):
            if counts[b] > 0:
                cache.append_one(b, S.dev(newv[b][:, :counts[b]], "bf16"), S.dev(newk[b][:counts[b]], "bf16"),
                                 BASE)
    torch.cuda.synchronize()
    assert cache.seq_lens.cpu().tolist() == lens.tolist()
    shape = cache.shape(int(max(lens)), split)
    q_rot = torch.empty(wl.B, nq, wl.H, wl.d_r, dtype=torch.bfloat16, device="cuda")
    gva.gva_rope_query_multi(shape, nq, S.dev(qr, "bf16"), q_rot, cache.seq_lens, BASE)
    out = torch.empty(wl.B, nq, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    nb = gva.gva_decode_multi_workspace_bytes(shape, nq)
    ws = torch.zeros(max(nb, 4) // 4 + 1, dtype=torch.float32, device="cuda")
    gva.gva_decode_multi(shape, nq, S.dev(qn, "bf16"), q_rot, S.dev(inp.M, "bf16"), cache.v_cache,
                         cache.kr_cache, cache.seq_lens, cache.block_table, wl.scale, out, ws)
    torch.cuda.synchronize()
    ref = O.gva_decode_multi_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    return S.host(out), ref, (cache, shape, qn, q_rot, inp, ws)


@pytest.mark.parametrize("nq", [2, 4])
@pytest.mark.parametrize("hpg", [1, 2, 4])
@pytest.mark.parametrize("paged,split", [(False, 0), (False, 64), (True, 256)])
def test_multi_matches_oracle(nq, hpg, paged, split):
    wl = W.Workload("multi", 9, B=4, H=4 * hpg, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([3, 65, 700, 1029])
    print(f"[case] multi nq={nq} hpg={hpg} paged={paged} split={split}", flush=True)
    got, ref, _ = _run(wl, lens, nq, paged=paged, split=split, seed=60 + nq + hpg)
    for j in range(nq):
        S.assert_close(got[:, j], ref[:, j], "bf16", f"multi nq={nq} hpg={hpg} query {j}")


@pytest.mark.parametrize("nq", [2, 4])
@pytest.mark.parametrize("split", [0, 256])
def test_multi_reference_moves_on_later_tiles(nq, split):
    """Positional keys scaled by 8 from token 640 on and by 32 from token 1600
    on (exact powers of two), so the columns' softmax references move
    mid-sequence; keys and queries drawn as rotated values and handed to both
    sides as they are (a rotated key's last-place difference would otherwise
    be amplified by these logits)."""
    wl = W.Workload("multi_move", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([2100, 1700])
    inp = W.make_gva_inputs(wl, lens=lens, seed=90 + nq)
    kr_rot, _ = W.draw_post_rope(wl, lens, seed=90 + nq)
    for rows in kr_rot:
        rows[640:] *= 8.0
        rows[1600:] *= 4.0
    rng = np.random.default_rng(91 + nq)
    qn = W.round_storage(rng.standard_normal((wl.B, nq, wl.H, wl.d_n)), "bf16")
    q_rot = W.round_storage(rng.standard_normal((wl.B, nq, wl.H, wl.d_r)), "bf16")
    cap = int(max(lens))
    v, k, seq = S.uniform_cache_from_host(wl, inp.V, kr_rot, cap, lens)
    shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, wl.d_r, capacity=cap, max_seq_len=cap,
                           split_tokens=split, dtype="bf16")
    out = torch.empty(wl.B, nq, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    nb = gva.gva_decode_multi_workspace_bytes(shape, nq)
    ws = torch.zeros(max(nb, 4) // 4 + 1, dtype=torch.float32, device="cuda")
    print(f"[case] multi moving reference nq={nq} split={split}", flush=True)
    gva.gva_decode_multi(shape, nq, S.dev(qn, "bf16"), S.dev(q_rot, "bf16"), S.dev(inp.M, "bf16"), v, k, seq,
                         None, wl.scale, out, ws)
    torch.cuda.synchronize()
    ref = O.gva_decode_multi(inp.V, kr_rot, qn, q_rot, inp.M, lens, wl.scale)
    got = S.host(out)
    for j in range(nq):
        S.assert_close(got[:, j], ref[:, j], "bf16", f"multi moving reference nq={nq} split={split} query {j}")


def test_multi_shorter_sequences_than_queries():
    """A sequence with fewer tokens than queries: the early queries read
    nothing and give zero rows; an empty sequence gives zeros throughout."""
    wl = W.Workload("multi_short", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([1, 2, 4])
    print("[case] multi short sequences", flush=True)
    got, ref, _ = _run(wl, lens, 4, paged=False, split=0, seed=70)
    assert np.all(got[0, :3] == 0) and np.all(got[1, :2] == 0)
    # a single visible token: that token's value row, exactly
    S.assert_close(got[:, 3], ref[:, 3], "bf16", "multi short, last query")
    assert np.array_equal(got[0, 3], ref[0, 3])


def test_multi_single_query_is_decode_bitwise():
    wl = W.Workload("multi1", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([100, 1500, 64])
    print("[case] multi n_q=1 against gva_decode", flush=True)
    got, ref, (cache, shape, qn, q_rot, inp, ws) = _run(wl, lens, 1, paged=False, split=128, seed=80)
    out = torch.empty(3, 16, 64, dtype=torch.bfloat16, device="cuda")
    gva.gva_decode(shape, S.dev(qn[:, 0], "bf16"), q_rot[:, 0].contiguous(), S.dev(inp.M, "bf16"),
                   cache.v_cache, cache.kr_cache, cache.seq_lens, None, wl.scale, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(S.host(out), got[:, 0])


def test_rope_query_multi_positions():
    rng = np.random.default_rng(90)
    B, H, nq, d_r = 4, 16, 4, 16
    q = W.round_storage(rng.standard_normal((B, nq, H, d_r)), "bf16")
    lens = np.array([0, 2, 4097, 131072], dtype=np.int32)
    shape = gva.make_shape(B, H, 4, 64, 64, d_r, capacity=131072, max_seq_len=131072, dtype="bf16")
    out = torch.empty(B, nq, H, d_r, dtype=torch.bfloat16, device="cuda")
    print("[case] rope_query_multi", flush=True)
    gva.gva_rope_query_multi(shape, nq, S.dev(q, "bf16"), out, torch.tensor(lens, device="cuda"), BASE)
    pos = np.maximum(lens[:, None] - nq + np.arange(nq)[None, :], 0)
    ref = O.round_storage(O.rope(q, pos[:, :, None]), "bf16")
    got = S.host(out)
    ulps = np.abs(torch.tensor(got).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64)
                  - torch.tensor(ref).to(torch.bfloat16).view(torch.int16).numpy().astype(np.int64))
    assert ulps.max() <= 1 and (ulps > 0).mean() < 1e-2


def test_multi_mid_size_all_sequences():
    """Mid workload shape (B=16, n = 4100), four queries per sequence, against
    the oracle on every sequence."""
    wl = W.WORKLOADS["mid_bf16"]
    lens = np.full(16, 4100)
    print("[case] multi mid size", flush=True)
    inp = W.make_gva_inputs(wl, lens=lens, seed=95)
    rng = np.random.default_rng(96)
    qn = W.round_storage(rng.standard_normal((16, 4, 16, 64)), "bf16")
    qr = W.round_storage(rng.standard_normal((16, 4, 16, 16)), "bf16")
    cache = GvaCache(16, 16, 4, 64, 64, 16, dtype="bf16", capacity=4100)
    cache.append(S.dev(np.stack(inp.V), "bf16"), S.dev(np.stack(inp.kr), "bf16"), BASE)
    shape = cache.shape(4100)
    q_rot = torch.empty(16, 4, 16, 16, dtype=torch.bfloat16, device="cuda")
    gva.gva_rope_query_multi(shape, 4, S.dev(qr, "bf16"), q_rot, cache.seq_lens, BASE)
    out = torch.empty(16, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    nb = gva.gva_decode_multi_workspace_bytes(shape, 4)
    ws = torch.zeros(max(nb, 4) // 4 + 1, dtype=torch.float32, device="cuda")
    gva.gva_decode_multi(shape, 4, S.dev(qn, "bf16"), q_rot, S.dev(inp.M, "bf16"), cache.v_cache,
                         cache.kr_cache, cache.seq_lens, None, wl.scale, out, ws)
    torch.cuda.synchronize()
    got = S.host(out)
    for b in range(16):
        ref = O.gva_decode_multi_step([inp.V[b]], [inp.kr[b]], qn[b:b + 1], qr[b:b + 1], inp.M,
                                      lens[b:b + 1], wl.scale, BASE, "bf16")
        S.assert_close(got[b:b + 1].reshape(4, 16, 64), ref[0], "bf16", f"multi mid b={b}")


def test_multi_validation():
    shape = gva.make_shape(2, 16, 4, 64, 64, 16, capacity=64, max_seq_len=64, dtype="bf16")
    # tensors of the sizes the shape needs, so that the library's own check
    # (not the binding's size check) refuses the call
    t = torch.zeros(2, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros(2, 4, 64, 64, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(2, 64, 16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gva.GvaError, match="n_q = 3"):
        gva.gva_decode_multi(shape, 3, t, t, None, vc, kc, torch.zeros(2, dtype=torch.int32, device="cuda"),
                             None, 0.1, t)
    shape32 = gva.make_shape(2, 16, 4, 64, 64, 16, capacity=64, max_seq_len=64, dtype="f32")
    t32 = torch.zeros(2, 4, 16, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(gva.GvaError, match="bf16"):
        gva.gva_decode_multi(shape32, 2, t32, t32, None, vc.float(), kc.float(),
                             torch.zeros(2, dtype=torch.int32, device="cuda"), None, 0.1, t32)
