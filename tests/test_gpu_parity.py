"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs. Tolerances: fp32 relative 1e-5 (global norm and max
abs relative to max |ref|); bf16 max abs 2e-2 and relative 1e-2 (global and
per (b, h) row). Cache writes: bit-exact values, positional keys within one
unit in the last place of the cache dtype."""
import math

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


def _ulp_diff(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """|a - b| in units of the dtype's spacing at the larger magnitude."""
    if dtype == "bf16":
        ia = torch.from_numpy(a).float().bfloat16().view(torch.int16).numpy().astype(np.int64)
        ib = torch.from_numpy(b).float().bfloat16().view(torch.int16).numpy().astype(np.int64)
    else:
        ia = a.astype(np.float32).view(np.int32).astype(np.int64)
        ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    # same-sign values: integer distance of the bit patterns
    same = np.sign(a) == np.sign(b)
    d = np.where(same, np.abs(ia - ib), np.where((a == 0) & (b == 0), 0, 1 << 20))
    return d


def _small_wl(dtype="bf16", d_r=16, B=3):
    return W.Workload("small", 9, B=B, H=16, G=4, d_n=64, d_v=64, d_r=d_r, S=0, dtype=dtype)


# ---------------------------------------------------------------------------
# Append and query rotation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d_r", [16, 24])
def test_append_matches_oracle(dtype, paged, d_r):
    wl = _small_wl(dtype, d_r)
    chunks = [150, 1, 5, 64]                      # bulk (2 launches), single, small, one block
    total = sum(chunks)
    inp = W.make_gva_inputs(wl, lens=np.zeros(wl.B, dtype=np.int64), extra=total)
    print(f"[case] append dtype={dtype} paged={paged} d_r={d_r} chunks={chunks}", flush=True)
    if paged:
        table, nblk = W.paged_pool(np.full(wl.B, total), 64, seed=3)
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, d_r, dtype=dtype,
                         block_table=torch.tensor(table), num_blocks=nblk)
    else:
        cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, d_r, dtype=dtype, capacity=total + 7)
    pos = 0
    for n in chunks:
        v = S.dev(np.stack([inp.V[b][:, pos:pos + n] for b in range(wl.B)]), dtype)
        k = S.dev(np.stack([inp.kr[b][pos:pos + n] for b in range(wl.B)]), dtype)
        cache.append(v, k, BASE)
        pos += n
    torch.cuda.synchronize()
    assert cache.seq_lens.cpu().tolist() == [total] * wl.B
    vc, kc = S.host(cache.v_cache), S.host(cache.kr_cache)
    for b in range(wl.B):
        if paged:
            blocks = table[b, :math.ceil(total / 64)]
            got_v = np.concatenate([vc[blk] for blk in blocks], axis=1)[:, :total]
            got_k = np.concatenate([kc[blk] for blk in blocks], axis=0)[:total]
        else:
            got_v, got_k = vc[b][:, :total], kc[b][:total]
        assert np.array_equal(got_v, inp.V[b]), "values must be copied unchanged"
        ref_k = O.append_positional_keys(inp.kr[b], 0, BASE, dtype)
        ulps = _ulp_diff(got_k, ref_k, dtype)
        assert ulps.max() <= 1, ulps.max()
        assert (ulps > 0).mean() < 1e-3


def test_append_far_positions_bf16():
    """Positional keys at positions up to 131071 (long-context workload)."""
    n = 131072
    wl = _small_wl("bf16", 16, B=1)
    inp = W.make_gva_inputs(wl, lens=np.array([n]))
    print(f"[case] append far positions n={n}", flush=True)
    cache = GvaCache(1, 16, 4, 64, 64, 16, dtype="bf16", capacity=n)
    cache.append(S.dev(inp.V[0][None], "bf16"), S.dev(inp.kr[0][None], "bf16"), BASE)
    got = S.host(cache.kr_cache)[0]
    ref = O.append_positional_keys(inp.kr[0], 0, BASE, "bf16")
    ulps = _ulp_diff(got, ref, "bf16")
    assert ulps.max() <= 1 and (ulps > 0).mean() < 1e-3, (ulps.max(), (ulps > 0).mean())


def test_append_past_capacity_is_clamped():
    wl = _small_wl("bf16", 16, B=2)
    inp = W.make_gva_inputs(wl, lens=np.zeros(2, dtype=np.int64), extra=70)
    cache = GvaCache(2, 16, 4, 64, 64, 16, dtype="bf16", capacity=64)
    print("[case] append past capacity", flush=True)
    cache.append(S.dev(np.stack([v for v in inp.V]), "bf16"),
                 S.dev(np.stack([k for k in inp.kr]), "bf16"), BASE)
    torch.cuda.synchronize()
    assert cache.seq_lens.cpu().tolist() == [64, 64]
    assert np.array_equal(S.host(cache.v_cache)[1], inp.V[1][:, :64])


@pytest.mark.parametrize("dtype,d_r", [("bf16", 16), ("bf16", 24), ("f32", 16)])
def test_rope_query_matches_oracle(dtype, d_r):
    rng = np.random.Generator(np.random.PCG64(5))
    B, H = 6, 16
    q = W.round_storage(rng.standard_normal((B, H, d_r)), dtype)
    lens = np.array([0, 1, 2, 4097, 65536, 131072], dtype=np.int32)
    shape = gva.make_shape(B, H, 4, 64, 64, d_r, capacity=131072, max_seq_len=131072, dtype=dtype)
    qd = S.dev(q, dtype)
    out = torch.empty_like(qd)
    print(f"[case] rope_query dtype={dtype} d_r={d_r}", flush=True)
    gva.gva_rope_query(shape, qd, out, torch.tensor(lens, device="cuda"), BASE)
    ref = O.round_storage(O.rope(q, np.maximum(lens - 1, 0)[:, None]), dtype)
    ulps = _ulp_diff(S.host(out), ref, dtype)
    assert ulps.max() <= 1
    # in place
    gva.gva_rope_query(shape, qd, qd, torch.tensor(lens, device="cuda"), BASE)
    assert torch.equal(qd, out)


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

def _decode_post_rope(wl, lens, *, paged=False, split=0, seed=0, kr_boost=(), m_factor=1.0, v_factor=1.0):
    """Decode-only problem: k_r and q_rope drawn directly as rotated values.
    `kr_boost`: (first token, factor) pairs; the positional keys of every
    sequence from that token on are multiplied by the factor. `m_factor`,
    `v_factor` multiply the maps and the values. All factors are powers of
    two, so the stored values stay exact. Returns (gpu_out, oracle_out)."""
    inp = W.make_gva_inputs(wl, lens=lens, seed=wl.seed + seed)
    kr_rot, q_rot = W.draw_post_rope(wl, inp.lens, seed=seed)
    for t0, factor in kr_boost:
        for rows in kr_rot:
            rows[t0:] *= factor
    if m_factor != 1.0:
        inp.M[...] *= m_factor
    if v_factor != 1.0:
        for rows in inp.V:
            rows *= v_factor
    cap = max(int(max(lens)), 1)
    if paged:
        v, k, table, nblk = S.paged_cache_from_host(wl, inp.V, kr_rot, np.maximum(lens, 1), seed)
        shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, wl.d_r, max_seq_len=cap, block_size=64,
                               num_blocks=nblk, max_blocks_per_seq=table.shape[1],
                               split_tokens=split, dtype=wl.dtype)
    else:
        v, k, seq = S.uniform_cache_from_host(wl, inp.V, kr_rot, cap, lens)
        table = None
        shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, wl.d_r, capacity=cap, max_seq_len=cap,
                               split_tokens=split, dtype=wl.dtype)
    seq = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    out = torch.empty(wl.B, wl.H, 64, dtype=W.torch_dtype(wl.dtype), device="cuda")
    print(f"[case] decode {wl.name} B={wl.B} max_len={cap} paged={paged} split={split} "
          f"d_r={wl.d_r} dtype={wl.dtype} split_used={gva.gva_decode_split_tokens(shape)}",
          flush=True)
    gva.gva_decode(shape, S.dev(inp.q_nope, wl.dtype), S.dev(q_rot, wl.dtype),
                   S.dev(inp.M, wl.dtype), v, k, seq, table, wl.scale, out, S.workspace(shape))
    torch.cuda.synchronize()
    ref = O.gva_decode(inp.V, kr_rot, inp.q_nope, q_rot, inp.M, lens, wl.scale)
    return S.host(out), ref


def test_decode_tiny_f32_end_to_end():
    """Tiny fp32 workload: prefill 256 tokens through gva_append, rotate the
    query, decode; the oracle starts from the same pre-RoPE inputs."""
    wl = W.WORKLOADS["tiny_f32"]
    inp = W.make_gva_inputs(wl)
    print("[case] tiny_f32 end to end", flush=True)
    cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="f32", capacity=wl.S)
    cache.append(S.dev(np.stack(inp.V), "f32"), S.dev(np.stack(inp.kr), "f32"), BASE)
    q_rot = torch.empty(wl.B, wl.H, wl.d_r, dtype=torch.float32, device="cuda")
    gva.gva_rope_query(cache.shape(wl.S), S.dev(inp.q_rope, "f32"), q_rot, cache.seq_lens, BASE)
    out = torch.empty(wl.B, wl.H, 64, dtype=torch.float32, device="cuda")
    cache.decode(S.dev(inp.q_nope, "f32"), q_rot, S.dev(inp.M, "f32"), wl.scale, out, wl.S)
    ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, inp.lens, wl.scale,
                            BASE, "f32")
    S.assert_close(S.host(out), ref, "f32", "tiny_f32 e2e")


@pytest.mark.parametrize("n", [1, 2, 3, 63, 64, 65, 129, 1000])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_small_edges_bf16(n, paged):
    wl = _small_wl("bf16", 16, B=3)
    lens = np.array([n, max(n - 1, 0), max(n // 2, 1)])
    out, ref = _decode_post_rope(wl, lens, paged=paged, split=64 if n > 64 else 0, seed=n)
    S.assert_close(out, ref, "bf16", f"edges n={n} paged={paged}")


@pytest.mark.parametrize("split", [0, 64, 128, 448])
def test_decode_split_f32(split):
    wl = _small_wl("f32", 16, B=2)
    lens = np.array([700, 513])
    out, ref = _decode_post_rope(wl, lens, split=split, seed=11)
    S.assert_close(out, ref, "f32", f"f32 split={split}")


def test_decode_empty_and_single_token():
    wl = _small_wl("bf16", 16, B=3)
    lens = np.array([0, 1, 0])
    out, ref = _decode_post_rope(wl, lens, seed=21)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.array_equal(out[2], np.zeros_like(out[2]))
    S.assert_close(out, ref, "bf16", "empty/single")


def test_decode_d_r_zero_and_head_groups():
    for hpg in (1, 2, 4):
        wl = W.Workload("hpg", 9, B=2, H=4 * hpg, G=4, d_n=64, d_v=64, d_r=0, S=0, dtype="bf16")
        out, ref = _decode_post_rope(wl, np.array([300, 77]), seed=hpg)
        S.assert_close(out, ref, "bf16", f"d_r=0 hpg={hpg}")


def test_split_and_paged_invariance():
    wl = _small_wl("bf16", 16, B=2)
    lens = np.array([3000, 1999])
    outs = [_decode_post_rope(wl, lens, paged=p, split=s, seed=31)[0]
            for p in (False, True) for s in (0, 64, 1024)]
    for o in outs[1:]:
        S.assert_close(o, outs[0], "bf16", "split/paged invariance")


@pytest.mark.parametrize("paged,split", [(False, 0), (False, 64), (True, 256)])
def test_decode_reference_moves_on_later_tiles(paged, split):
    """Positional keys scaled by 8 from token 640 on and by 32 from token 1600
    on: the later tiles' scores pass the first tiles' max by far more than 2^8
    (log2 units), so every column's reference moves in the middle of the
    sequence (the rescale branch of the online softmax), in some partitions
    more than once."""
    wl = _small_wl("bf16", 16, B=2)
    lens = np.array([2100, 1700])
    out, ref = _decode_post_rope(wl, lens, paged=paged, split=split, seed=41,
                                 kr_boost=((640, 8.0), (1600, 4.0)))
    S.assert_close(out, ref, "bf16", f"moving reference paged={paged} split={split}")


@pytest.mark.parametrize("paged,split", [(False, 0), (True, 256)])
def test_decode_peaked_content_scores(paged, split):
    """Maps scaled by 8 and values halved (exact): content logits with a
    standard deviation of about 3.6 and the top ones well apart, far more
    peaked than the N(0,1) workloads. The absorbed query q' = M q is the one
    operand the kernel forms itself and rounds to bf16; the error this adds
    grows with the logits and must stay inside the tolerance here."""
    wl = _small_wl("bf16", 16, B=2)
    lens = np.array([4097, 2500])
    out, ref = _decode_post_rope(wl, lens, paged=paged, split=split, seed=51, m_factor=8.0, v_factor=0.5)
    S.assert_close(out, ref, "bf16", f"peaked content scores paged={paged} split={split}")


@pytest.mark.parametrize("paged", [False, True])
def test_decode_two_partitions_per_workgroup(paged):
    """An explicit 64-token partition length over 33 partitions and 16
    (sequence, group) pairs (528 partitions, more than two rounds of
    workgroups) is served two partitions per workgroup. Lengths: an odd and
    an even partition count in the last workgroup, a sequence that ends
    halfway (workgroups past it exit early) and an empty one; against the
    oracle, and against a partition length that keeps one per workgroup."""
    wl = _small_wl("bf16", 16, B=4)
    lens = np.array([2100, 2112, 1000, 0])
    out, ref = _decode_post_rope(wl, lens, paged=paged, split=64, seed=61)
    S.assert_close(out, ref, "bf16", f"two partitions per workgroup paged={paged}")
    assert np.array_equal(out[3], np.zeros_like(out[3]))
    out1, _ = _decode_post_rope(wl, lens, paged=paged, split=128, seed=61)
    S.assert_close(out, out1, "bf16", "two partitions per workgroup against one")


@pytest.mark.parametrize("name", ["mid_bf16", "wide_dr24", "long_split", "ragged_paged"])
def test_decode_full_size(name):
    wl = W.WORKLOADS[name]
    if wl.ragged:
        rng = np.random.Generator(np.random.PCG64(wl.seed))
        lens = rng.integers(wl.len_lo, wl.len_hi, size=wl.B, endpoint=True)
    else:
        lens = np.full(wl.B, wl.S)
    out, ref = _decode_post_rope(wl, lens, paged=wl.block_size > 0, split=wl.split_tokens)
    S.assert_close(out, ref, wl.dtype, f"full {name}")


def test_decode_auto_thirds_equals_plain_split():
    """A batch that fills the compute units by itself (B*G = 256) with a few
    sequences long enough for the automatic split into thirds (ties in length
    included, one empty sequence): identical to the explicit split of the same
    length, and within tolerance of the oracle."""
    wl = W.Workload("ranked", 9, B=64, H=16, G=4, d_n=64, d_v=64, d_r=16, S=0, dtype="bf16")
    rng = np.random.default_rng(61)
    lens = rng.integers(1, 3000, size=wl.B)
    lens[[5, 17, 40, 63]] = [30800, 31000, 30721, 30800]   # ties in length too
    lens[3] = 0
    inp = W.make_gva_inputs(wl, lens=lens, seed=62)
    kr_rot, q_rot = W.draw_post_rope(wl, inp.lens, seed=62)
    cap = int(lens.max())
    v, k, table, nblk = S.paged_cache_from_host(wl, inp.V, kr_rot, np.maximum(lens, 1), 63)
    seq = torch.tensor(lens.astype(np.int32), device="cuda")
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, q_rot, inp.M))

    def shape(split):
        return gva.make_shape(wl.B, wl.H, wl.G, 64, 64, wl.d_r, max_seq_len=cap, block_size=64, num_blocks=nblk,
                              max_blocks_per_seq=table.shape[1], split_tokens=split, dtype="bf16")
    s_auto = shape(0)
    auto = gva.gva_decode_split_tokens(s_auto)
    assert 3 * auto >= cap > 2 * auto, "the automatic split cuts the longest sequences into thirds"
    s_plain = shape(auto)
    outs = []
    for label, sh in (("auto", s_auto), ("explicit", s_plain)):
        print(f"[case] decode thirds {label} split={auto}", flush=True)
        out = torch.full((wl.B, wl.H, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        gva.gva_decode(sh, qn, qr, Md, v, k, seq, table, wl.scale, out, S.workspace(sh))
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    ref = O.gva_decode(inp.V, kr_rot, inp.q_nope, q_rot, inp.M, lens, wl.scale)
    S.assert_close(S.host(outs[0]), ref, "bf16", "auto thirds")


def test_decode_mid_bf16_end_to_end_steps():
    """Mid workload through the whole path: prefill 4096 tokens with
    gva_append, then three steps of {append one token, rotate the query,
    decode}, each compared with the oracle step."""
    wl = W.WORKLOADS["mid_bf16"]
    steps = 3
    inp = W.make_gva_inputs(wl, extra=steps)
    cap = wl.S + steps
    print("[case] mid_bf16 end to end", flush=True)
    cache = GvaCache(wl.B, wl.H, wl.G, 64, 64, wl.d_r, dtype="bf16", capacity=cap)
    Vd = S.dev(np.stack(inp.V), "bf16")          # [B, G, S+steps, d_v]
    Kd = S.dev(np.stack(inp.kr), "bf16")         # [B, S+steps, d_r]
    cache.append(Vd[:, :, :wl.S].contiguous(), Kd[:, :wl.S].contiguous(), BASE)
    qn, qr, Md = (S.dev(x, "bf16") for x in (inp.q_nope, inp.q_rope, inp.M))
    q_rot = torch.empty_like(qr)
    out = torch.empty(wl.B, wl.H, 64, dtype=torch.bfloat16, device="cuda")
    for i in range(steps):
        n = wl.S + i + 1
        cache.append(Vd[:, :, n - 1:n].contiguous(), Kd[:, n - 1:n].contiguous(), BASE)
        gva.gva_rope_query(cache.shape(n), qr, q_rot, cache.seq_lens, BASE)
        cache.decode(qn, q_rot, Md, wl.scale, out, n)
        ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M,
                                np.full(wl.B, n), wl.scale, BASE, "bf16")
        S.assert_close(S.host(out), ref, "bf16", f"mid e2e step {i}")


# ---------------------------------------------------------------------------
# GQA comparison kernel
# ---------------------------------------------------------------------------

def _gqa_run(wl, lens, *, paged=False, split=0, seed=0):
    q, K, V = W.make_gqa_inputs(wl.replace(S=int(max(lens))), seed=wl.seed + seed)
    Kr = [K[b][:, :int(n)] for b, n in enumerate(lens)]
    Vr = [V[b][:, :int(n)] for b, n in enumerate(lens)]
    cap = int(max(lens))
    if paged:
        table, nblk = W.paged_pool(np.maximum(lens, 1), 64, seed)
        kp, _ = W.scatter_paged(Kr, [np.zeros((int(n), 0)) for n in lens], table, nblk, 64)
        vp, _ = W.scatter_paged(Vr, [np.zeros((int(n), 0)) for n in lens], table, nblk, 64)
        kd, vd, td = S.dev(kp, wl.dtype), S.dev(vp, wl.dtype), torch.tensor(table, device="cuda")
        shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, 0, max_seq_len=cap, block_size=64,
                               num_blocks=nblk, max_blocks_per_seq=table.shape[1],
                               split_tokens=split, dtype=wl.dtype)
    else:
        kd = S.dev(W.contiguous_cache(Kr, cap, 1), wl.dtype)
        vd = S.dev(W.contiguous_cache(Vr, cap, 1), wl.dtype)
        td = None
        shape = gva.make_shape(wl.B, wl.H, wl.G, 64, 64, 0, capacity=cap, max_seq_len=cap,
                               split_tokens=split, dtype=wl.dtype)
    seq = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    out = torch.empty(wl.B, wl.H, 64, dtype=W.torch_dtype(wl.dtype), device="cuda")
    sc = S.gqa_scale(64)
    print(f"[case] gqa B={wl.B} max_len={cap} paged={paged} split={split}", flush=True)
    gva.gva_gqa_ref_decode(shape, S.dev(q, wl.dtype), kd, vd, seq, td, sc, out, S.workspace(shape))
    torch.cuda.synchronize()
    ref = O.gqa_decode(q, Kr, Vr, lens, sc)
    return S.host(out), ref


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("lens", [[1, 65, 300], [0, 2, 1000], [4096, 4095]])
def test_gqa_reference_matches_oracle(paged, lens):
    wl = _small_wl("bf16", 0, B=len(lens))
    out, ref = _gqa_run(wl, np.array(lens), paged=paged, split=0 if max(lens) < 1000 else 256)
    S.assert_close(out, ref, "bf16", f"gqa lens={lens} paged={paged}")


def test_gqa_reference_full_wide():
    """Matched GQA cache of the wide workload (B=32, S=8192, G=4, d_h=64)."""
    wl = W.WORKLOADS["wide_dr24"].replace(d_r=0)
    out, ref = _gqa_run(wl, np.full(wl.B, wl.S))
    S.assert_close(out, ref, "bf16", "gqa full wide")
