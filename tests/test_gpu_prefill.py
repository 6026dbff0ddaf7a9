"""GPU tests of the causal prefill (gva_prefill): the last n_q cached tokens
of every sequence attend to the cache up to and including themselves, the
whole prompt when n_q = n. Against the CPU oracle from pre-RoPE inputs."""
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


def _cache(wl, inp, lens, paged, seed, extra=8):
    cap = int(max(lens)) + extra
    if paged:
        table, nblk = W.paged_pool(np.full(wl.B, cap), 64, seed)
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", block_table=torch.tensor(table),
                         num_blocks=nblk)
    else:
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", capacity=cap)
    for b, n in enumerate(lens):
        if n > 0:
            kr = S.dev(inp.kr[b][:n], "bf16") if wl.d_r else None
            cache.append_one(b, S.dev(inp.V[b][:, :n], "bf16"), kr, BASE)
    torch.cuda.synchronize()
    assert cache.seq_lens.cpu().tolist() == list(map(int, lens))
    return cache


def _queries(wl, nq, seed):
    rng = np.random.default_rng(seed)
    qn = W.round_storage(rng.standard_normal((wl.B, nq, wl.H, wl.d_n)), "bf16")
    qr = W.round_storage(rng.standard_normal((wl.B, nq, wl.H, max(wl.d_r, 1))), "bf16")[..., :wl.d_r]
    return qn, qr


def _rotate(cache, shape, nq, qr):
    if qr.shape[-1] == 0:
        return None
    q_rot = torch.empty(qr.shape, dtype=torch.bfloat16, device="cuda")
    gva.gva_rope_query_multi(shape, nq, S.dev(qr, "bf16"), q_rot, cache.seq_lens, BASE)
    return q_rot


def _prefill(cache, shape, nq, qn_dev, q_rot, M_dev, scale):
    B, H = qn_dev.shape[0], qn_dev.shape[2]
    out = torch.full((B, nq, H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    gva.gva_prefill(shape, nq, qn_dev, q_rot, M_dev, cache.v_cache, cache.kr_cache, cache.seq_lens,
                    cache.block_table, scale, out)
    torch.cuda.synchronize()
    return S.host(out)


@pytest.mark.parametrize("hpg", [1, 2, 4])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("nq", ["full", 100])
def test_prefill_matches_oracle(hpg, paged, nq):
    wl = W.Workload("prefill", 9, B=4, H=4 * hpg, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([300, 77, 129, 1])
    nq = 300 if nq == "full" else nq
    inp = W.make_gva_inputs(wl, lens=lens, seed=70 + hpg)
    print(f"[case] prefill hpg={hpg} paged={paged} nq={nq}", flush=True)
    cache = _cache(wl, inp, lens, paged, seed=71)
    shape = cache.shape(int(max(lens)))
    qn, qr = _queries(wl, nq, seed=72 + hpg)
    got = _prefill(cache, shape, nq, S.dev(qn, "bf16"), _rotate(cache, shape, nq, qr), S.dev(inp.M, "bf16"),
                   wl.scale)
    ref = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    assert not np.isnan(got).any()
    S.assert_close(got, ref, "bf16", f"prefill hpg={hpg} paged={paged} nq={nq}")
    # rows whose position is negative read nothing
    for b, n in enumerate(lens):
        assert np.all(got[b, :max(nq - n, 0)] == 0)


@pytest.mark.parametrize("paged", [False, True])
def test_prefill_reference_moves_on_later_tiles(paged):
    """Positional keys scaled by 8 from token 200 on and by 32 from token 400
    on (powers of two: the stored values stay exact): for the later queries
    the scores of later tiles pass the first tile's max by far more than 2^8
    (log2 units), so the columns' references move mid-sweep, in the rescale
    branch of the online softmax. Keys and queries are drawn as rotated
    values and handed to both sides as they are: with scores this large, a
    one-unit difference in a rotated key's last place (which the rotation
    is allowed) would move a weight by several percent. The values are
    halved (exact) so that the outputs, which here follow single large-score
    tokens, stay below 2.5: their own bf16 rounding then stays well inside
    the absolute bound."""
    wl = W.Workload("prefill_move", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([700, 450])
    nq = 700
    inp = W.make_gva_inputs(wl, lens=lens, seed=110)
    for rows in inp.V:
        rows *= 0.5
    kr_rot, _ = W.draw_post_rope(wl, lens, seed=110)
    for rows in kr_rot:
        rows[200:] *= 8.0
        rows[400:] *= 4.0
    qn, q_rot = _queries(wl, nq, seed=112)  # q_rot: drawn directly as rotated values
    cap = int(max(lens))
    print(f"[case] prefill moving reference paged={paged}", flush=True)
    if paged:
        v, k, table, nblk = S.paged_cache_from_host(wl, inp.V, kr_rot, lens, 113)
        shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, wl.d_r, max_seq_len=cap, block_size=64,
                               num_blocks=nblk, max_blocks_per_seq=table.shape[1], dtype="bf16")
    else:
        v, k, _ = S.uniform_cache_from_host(wl, inp.V, kr_rot, cap, lens)
        table = None
        shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, wl.d_r, capacity=cap, max_seq_len=cap, dtype="bf16")
    seq = torch.tensor(lens.astype(np.int32), device="cuda")
    out = torch.full((wl.B, nq, wl.H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    gva.gva_prefill(shape, nq, S.dev(qn, "bf16"), S.dev(q_rot, "bf16"), S.dev(inp.M, "bf16"), v, k, seq,
                    table, wl.scale, out)
    torch.cuda.synchronize()
    got = S.host(out)
    ref = O.gva_prefill(inp.V, kr_rot, qn, q_rot, inp.M, lens, wl.scale)
    assert not np.isnan(got).any()
    S.assert_close(got, ref, "bf16", f"prefill moving reference paged={paged}")


@pytest.mark.parametrize("d_r", [0, 8, 24, 32])
def test_prefill_positional_widths(d_r):
    wl = W.Workload("prefill_dr", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=d_r, S=0, dtype="bf16")
    lens = np.array([200, 65, 64])
    inp = W.make_gva_inputs(wl, lens=lens, seed=80 + d_r)
    print(f"[case] prefill d_r={d_r}", flush=True)
    cache = _cache(wl, inp, lens, False, seed=81)
    shape = cache.shape(int(max(lens)))
    qn, qr = _queries(wl, 130, seed=82)
    got = _prefill(cache, shape, 130, S.dev(qn, "bf16"), _rotate(cache, shape, 130, qr), S.dev(inp.M, "bf16"),
                   wl.scale)
    ref = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    S.assert_close(got, ref, "bf16", f"prefill d_r={d_r}")


def test_prefill_folded_queries():
    """M = NULL with the absorbed queries q' = M q (formed by the oracle, rounded
    to bf16): within the tolerance of the oracle, as the path with M is."""
    wl = W.Workload("prefill_fold", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([257, 190])
    inp = W.make_gva_inputs(wl, lens=lens, seed=90)
    print("[case] prefill folded", flush=True)
    cache = _cache(wl, inp, lens, True, seed=91)
    shape = cache.shape(int(max(lens)))
    qn, qr = _queries(wl, 257, seed=92)
    q_rot = _rotate(cache, shape, 257, qr)
    q_abs = np.einsum("hvn,bjhn->bjhv", inp.M, qn)
    got_m = _prefill(cache, shape, 257, S.dev(qn, "bf16"), q_rot, S.dev(inp.M, "bf16"), wl.scale)
    got_f = _prefill(cache, shape, 257, S.dev(q_abs, "bf16"), q_rot, None, wl.scale)
    ref = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    S.assert_close(got_m, ref, "bf16", "prefill with M")
    S.assert_close(got_f, ref, "bf16", "prefill without M (folded queries)")


@pytest.mark.parametrize("nq", [1, 2, 4])
def test_prefill_agrees_with_multi_query_decode(nq):
    """For n_q of 1, 2 and 4 the split-K decode kernel computes the same
    thing; both within tolerance of each other and of the oracle."""
    wl = W.Workload("prefill_vs_multi", 9, B=3, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([1500, 3, 640])
    inp = W.make_gva_inputs(wl, lens=lens, seed=100 + nq)
    print(f"[case] prefill vs multi nq={nq}", flush=True)
    cache = _cache(wl, inp, lens, False, seed=101)
    shape = cache.shape(int(max(lens)), 256)
    qn, qr = _queries(wl, nq, seed=102)
    q_rot = _rotate(cache, shape, nq, qr)
    got = _prefill(cache, shape, nq, S.dev(qn, "bf16"), q_rot, S.dev(inp.M, "bf16"), wl.scale)
    out = torch.empty(3, nq, 16, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(gva.gva_decode_multi_workspace_bytes(shape, nq) // 4 + 1, device="cuda")
    gva.gva_decode_multi(shape, nq, S.dev(qn, "bf16"), q_rot, S.dev(inp.M, "bf16"), cache.v_cache, cache.kr_cache,
                         cache.seq_lens, None, wl.scale, out, ws)
    torch.cuda.synchronize()
    ref = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    S.assert_close(got, ref, "bf16", f"prefill nq={nq}")
    S.assert_close(got, S.host(out), "bf16", f"prefill vs multi-query decode nq={nq}")


def test_prefill_mid_size_sampled():
    """The prefill workload's shape (B=16, a 4096-token prompt, all 4096 tokens
    as queries), in the launch configuration of the benchmark, against the
    oracle: every query of two whole sequences (the oracle's causal prefill),
    and sampled (sequence, query) rows of the others computed one by one with
    the decode oracle."""
    wl = W.WORKLOADS["mid_bf16"]
    n = 4096
    lens = np.full(16, n)
    inp = W.make_gva_inputs(wl, lens=lens, seed=110)
    print("[case] prefill mid size", flush=True)
    cache = GvaCache(16, 16, 4, 64, 64, 16, dtype="bf16", capacity=n)
    cache.append(S.dev(np.stack(inp.V), "bf16"), S.dev(np.stack(inp.kr), "bf16"), BASE)
    shape = cache.shape(n)
    qn, qr = _queries(wl, n, seed=111)
    got = _prefill(cache, shape, n, S.dev(qn, "bf16"), _rotate(cache, shape, n, qr), S.dev(inp.M, "bf16"),
                   wl.scale)
    assert not np.isnan(got).any()
    rng = np.random.default_rng(112)
    samples = [(0, 0), (15, n - 1), (3, 63), (3, 64), (7, 1000), (11, 2047), (12, 4032)]
    samples += [(int(b), int(j)) for b, j in zip(rng.integers(0, 16, 9), rng.integers(0, n, 9))]
    for b, j in samples:
        kr_rot = O.append_positional_keys(inp.kr[b][:j + 1], 0, BASE, "bf16")
        q_rot = O.rope(qr[b, j], float(j), BASE)
        ref = O.gva_decode_seq(inp.V[b], kr_rot, qn[b, j], q_rot, inp.M, j + 1, wl.scale)
        S.assert_close(got[b, j], ref, "bf16", f"prefill mid b={b} j={j}")
    for b in (5, 14):
        ref = O.gva_prefill_step([inp.V[b]], [inp.kr[b]], qn[b:b + 1], qr[b:b + 1], inp.M, [n], wl.scale, BASE,
                                 "bf16")
        S.assert_close(got[b:b + 1], ref, "bf16", f"prefill mid, every query of b={b}")


def test_prefill_empty_and_validation():
    wl = W.Workload("prefill_edge", 9, B=2, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    lens = np.array([0, 5])
    inp = W.make_gva_inputs(wl, lens=np.array([1, 5]), seed=120)
    print("[case] prefill empty sequence", flush=True)
    cache = _cache(wl, inp, lens, False, seed=121)
    shape = cache.shape(8)
    qn, qr = _queries(wl, 5, seed=122)
    got = _prefill(cache, shape, 5, S.dev(qn, "bf16"), _rotate(cache, shape, 5, qr), S.dev(inp.M, "bf16"),
                   wl.scale)
    assert np.all(got[0] == 0)
    ref = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, wl.scale, BASE, "bf16")
    S.assert_close(got, ref, "bf16", "prefill with an empty sequence")
    t = torch.zeros(2, 5, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gva.GvaError, match="n_q"):
        gva.gva_prefill(shape, 0, t, t, None, cache.v_cache, cache.kr_cache, cache.seq_lens, None, 0.1, t)
    shape32 = gva.make_shape(2, 16, 4, 64, 64, 16, capacity=8, max_seq_len=8, dtype="f32")
    t32 = torch.zeros(2, 5, 16, 64, dtype=torch.float32, device="cuda")
    with pytest.raises(gva.GvaError, match="bf16"):
        gva.gva_prefill(shape32, 5, t32, t32, None, t32, t32, cache.seq_lens, None, 0.1, t32)
