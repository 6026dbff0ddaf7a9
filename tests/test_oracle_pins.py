"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test targets a mistake the oracle could plausibly make (a transposed
map, a wrong head->group map, a dropped positional term, a wrong query
position, a RoPE sign error, a wrong softmax or aggregation, wrong
rounding), using values the pages print, library routines, closed forms,
invariants or brute force on tiny inputs. CPU only.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def _problem(rng, B=2, H=8, G=2, d=16, d_r=4, n=12, m_scale=0.25):
    V = [rng.standard_normal((G, n, d)) for _ in range(B)]
    kr = [rng.standard_normal((n, d_r)) for _ in range(B)]
    q_nope = rng.standard_normal((B, H, d))
    q_rope = rng.standard_normal((B, H, d_r))
    M = rng.standard_normal((H, d, d)) * m_scale
    return V, kr, q_nope, q_rope, M


# ---------------------------------------------------------------------------
# Pages' printed numbers
# ---------------------------------------------------------------------------

def test_cache_savings_match_pages():
    """The shared positional key reading reproduces every printed saving."""
    g = _load("cache_savings.json")
    G, d_v, d_h = g["workload_dims"]["G"], g["workload_dims"]["d_v"], g["workload_dims"]["d_h"]
    for d_r, pct in g["saving_pct_by_dr"].items():
        ratio = O.gva_scalars_per_token(G, d_v, int(d_r)) / O.gqa_scalars_per_token(G, d_h)
        saving = 100.0 * (1.0 - ratio)
        assert round(saving) == pct
        lo, hi = g["saving_range_pct"]
        assert lo - 0.5 <= saving <= hi + 0.5
        u_lo, u_hi = g["units_per_100"]
        assert u_lo <= round(100 * ratio) <= u_hi
    ratio0 = O.gva_scalars_per_token(G, d_v, 0) / O.gqa_scalars_per_token(G, d_h)
    assert 100.0 * (1.0 - ratio0) == g["saving_pct_no_positional_key"]
    # exact values at the workload dims
    assert O.gva_scalars_per_token(4, 64, 16) == 272
    assert O.gva_scalars_per_token(4, 64, 24) == 280
    assert O.gqa_scalars_per_token(4, 64) == 512


def test_per_group_positional_key_contradicts_pages():
    """A positional key per group (instead of one shared by all heads) gives a
    saving far from both printed figures: the shared reading is forced."""
    g = _load("cache_savings.json")
    G, d_v, d_h = 4, 64, 64
    for d_r, pct in g["saving_pct_by_dr"].items():
        per_group = (G * d_v + G * int(d_r)) / O.gqa_scalars_per_token(G, d_h)
        assert abs(100 * (1 - per_group) - pct) > 5


def test_gqa_memory_example():
    g = _load("gqa_memory_example.json")
    GiB = 1024 ** 3
    mha = O.kv_cache_bytes(g["layers"], g["context_tokens"], g["mha_kv_heads"], g["head_dim"],
                           g["bytes_per_elem"], g["sequences"])
    gqa = O.kv_cache_bytes(g["layers"], g["context_tokens"], g["gqa_kv_heads"], g["head_dim"],
                           g["bytes_per_elem"], g["sequences"])
    assert mha / GiB == pytest.approx(g["mha_total_gib_approx"], rel=1e-12)
    assert gqa / GiB == pytest.approx(g["gqa_total_gib_approx"], rel=1e-12)


def test_head_group_map_matches_diagram():
    g = _load("head_group_diagram.json")
    assert [O.head_group(h, g["H"], g["G"]) for h in range(g["H"])] == g["group_of_head"]


# ---------------------------------------------------------------------------
# Rounding
# ---------------------------------------------------------------------------

def test_round_bf16_matches_library_and_ties():
    rng = _rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000) * 1e-39])
    x32 = x.astype(np.float32).astype(np.float64)       # torch rounds fp32 -> bf16 with RNE
    ref = torch.from_numpy(x32).float().bfloat16().double().numpy()
    assert np.array_equal(O.round_bf16(x32), ref)
    # hand-worked ties: spacing above 1.0 is 2^-7
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0                     # tie -> even (1.0)
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie -> even (1 + 2^-6)
    assert O.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert O.round_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    assert np.isinf(O.round_bf16(3.5e38))


def test_round_bf16_from_double_is_direct():
    """Float64 inputs round once (no detour through fp32): a value just above
    a bf16 tie must round up even when fp32 would have hit the tie."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40    # fp32 rounds this to the tie 1 + 2^-8
    assert O.round_bf16(x) == 1.0 + 2.0 ** -7


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_thetas_closed_form():
    th = O.rope_thetas(16, 10000.0)
    assert th[0] == 1.0
    assert th[4] == pytest.approx(1e-2, rel=1e-14)      # 10000^(-8/16)
    assert th[2] == pytest.approx(1e-1, rel=1e-14)      # 10000^(-4/16)
    assert O.rope_thetas(2, 10000.0).tolist() == [1.0]


def test_rope_is_complex_rotation():
    """Pair (x[2i], x[2i+1]) as a complex number is multiplied by e^{i pos theta_i}."""
    rng = _rng(2)
    x = rng.standard_normal(16)
    pos = 37
    y = O.rope(x, pos)
    for i in range(8):
        theta = 10000.0 ** (-2.0 * i / 16)
        z = complex(x[2 * i], x[2 * i + 1]) * cmath.exp(1j * pos * theta)
        assert y[2 * i] == pytest.approx(z.real, abs=1e-12)
        assert y[2 * i + 1] == pytest.approx(z.imag, abs=1e-12)


def test_rope_invariants():
    rng = _rng(3)
    x = rng.standard_normal((5, 24))
    assert np.array_equal(O.rope(x, 0), x)                               # position 0 = identity
    y = O.rope(x, np.arange(5) * 1000 + 7)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # relative property: <R_p a, R_t b> depends only on p - t
    a, b = x[0], x[1]
    d1 = O.rope(a, 130) @ O.rope(b, 100)
    d2 = O.rope(a, 131100) @ O.rope(b, 131070)
    assert d1 == pytest.approx(d2, rel=1e-9)
    # composition: R_p R_t = R_{p+t}
    assert np.allclose(O.rope(O.rope(x, 11), 5), O.rope(x, 16), atol=1e-13)


def test_append_rotates_at_own_position_then_rounds():
    rng = _rng(4)
    kr = O.round_bf16(rng.standard_normal((6, 16)))
    cached = O.append_positional_keys(kr, 0, 10000.0, "bf16")
    assert np.array_equal(cached[0], kr[0])                # token 0 is not turned
    for t in range(6):
        assert np.array_equal(cached[t], O.round_bf16(O.rope(kr[t], t)))
    later = O.append_positional_keys(kr[3:], 3, 10000.0, "bf16")
    assert np.array_equal(later, cached[3:])


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------

def test_absorption_identity_pages_form():
    """Materialized scores (K = V M) equal absorbed scores with Q' = Q M^T
    written in the pages' row-vector form. A transposed map fails."""
    rng = _rng(5)
    n, d = 40, 16
    Vg = rng.standard_normal((n, d))
    M_h = rng.standard_normal((d, d))
    q = rng.standard_normal(d)
    kr = np.zeros((n, 0))
    s_mat = O.gva_head_scores(Vg, kr, q, np.zeros(0), M_h, 1.0)
    q_abs = q[None, :] @ M_h.T                      # Q' = Q M^T
    s_abs = (Vg @ q_abs[0])
    assert np.allclose(s_mat, s_abs, rtol=1e-12, atol=1e-12)
    assert not np.allclose(s_mat, Vg @ (q[None, :] @ M_h)[0], rtol=1e-3)


def test_shared_kv_reduces_to_library_attention():
    """M_h = I and d_r = 0 is shared-KV (K = V) attention; it must equal torch's
    scaled_dot_product_attention in float64 with heads mapped to groups."""
    rng = _rng(6)
    B, H, G, d, n = 2, 8, 2, 16, 33
    V = [rng.standard_normal((G, n, d)) for _ in range(B)]
    q = rng.standard_normal((B, H, d))
    M = np.broadcast_to(np.eye(d), (H, d, d)).copy()
    kr = [np.zeros((n, 0)) for _ in range(B)]
    scale = 0.3
    out = O.gva_decode(V, kr, q, np.zeros((B, H, 0)), M, [n, n], scale)
    Vt = torch.from_numpy(np.stack(V))                            # [B, G, n, d]
    idx = torch.tensor([h // (H // G) for h in range(H)])
    Kx = Vt[:, idx]                                               # [B, H, n, d]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], Kx, Kx, scale=scale)[:, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)
    # and the GQA oracle with K := V agrees
    out_gqa = O.gqa_decode(q, V, V, [n, n], scale)
    assert np.allclose(out, out_gqa, rtol=1e-13, atol=1e-14)


def test_gqa_oracle_matches_library_attention():
    rng = _rng(7)
    B, H, G, d, n = 3, 8, 2, 16, 29
    K = rng.standard_normal((B, G, n, d))
    V = rng.standard_normal((B, G, n, d))
    q = rng.standard_normal((B, H, d))
    out = O.gqa_decode(q, K, V, [n] * B, 0.25)
    idx = torch.tensor([h // (H // G) for h in range(H)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(K)[:, idx],
        torch.from_numpy(V)[:, idx], scale=0.25)[:, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_full_gva_matches_library_attention_on_explicit_keys():
    """The decode output equals library attention given the per-head keys
    [V_g M_h || k_r] (pins scale, softmax and value aggregation)."""
    rng = _rng(8)
    B, H, G, d, d_r, n = 2, 8, 2, 16, 4, 21
    V, kr, q_nope, q_rope, M = _problem(rng, B, H, G, d, d_r, n)
    scale = 1 / math.sqrt(d + d_r)
    out = O.gva_decode(V, kr, q_nope, q_rope, M, [n, n], scale)
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            K = np.concatenate([V[b][g] @ M[h], kr[b]], axis=1)
            Q = np.concatenate([q_nope[b, h], q_rope[b, h]])
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None],
                torch.from_numpy(V[b][g])[None], scale=scale)[0, 0].numpy()
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-13)


def test_single_token_returns_its_value():
    rng = _rng(9)
    V, kr, q_nope, q_rope, M = _problem(rng, n=1)
    out = O.gva_decode(V, kr, q_nope, q_rope, M, [1, 1], 0.7)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(out[b, h], V[b][h // 4][0])


def test_two_tokens_closed_form():
    rng = _rng(10)
    V, kr, q_nope, q_rope, M = _problem(rng, B=1, n=2)
    scale = 0.4
    out = O.gva_decode(V, kr, q_nope, q_rope, M, [2], scale)
    for h in range(8):
        g = h // 4
        s = [scale * ((V[0][g][t] @ M[h]) @ q_nope[0, h] + kr[0][t] @ q_rope[0, h]) for t in (0, 1)]
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        ref = w0 * V[0][g][0] + (1 - w0) * V[0][g][1]
        assert np.allclose(out[0, h], ref, rtol=1e-12, atol=1e-14)


def test_group_constant_values_pin_head_map():
    """Group g holds constant rows c_g: head h must return exactly c_{h // (H/G)}."""
    rng = _rng(11)
    B, H, G, d, n = 1, 8, 4, 16, 9
    c = rng.standard_normal((G, d))
    V = [np.broadcast_to(c[:, None, :], (G, n, d)).copy()]
    _, kr, q_nope, q_rope, M = _problem(rng, B, H, G, d, 4, n)
    out = O.gva_decode(V, kr, q_nope, q_rope, M, [n], 0.5)
    for h in range(H):
        assert np.allclose(out[0, h], c[h // 2], rtol=0, atol=1e-14)
        if h // 2 != h % G:
            assert not np.allclose(out[0, h], c[h % G])


def test_zero_query_gives_mean_of_values():
    rng = _rng(12)
    V, kr, q_nope, q_rope, M = _problem(rng)
    out = O.gva_decode(V, kr, np.zeros_like(q_nope), np.zeros_like(q_rope), M, [12, 7], 0.9)
    for b, n in enumerate([12, 7]):
        for h in range(8):
            assert np.allclose(out[b, h], V[b][h // 4][:n].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_token_permutation_invariance():
    """Permuting cache rows (value row with its positional key) changes nothing;
    this is what lets paged blocks sit anywhere in the pool."""
    rng = _rng(13)
    V, kr, q_nope, q_rope, M = _problem(rng, B=1, n=30)
    perm = rng.permutation(30)
    out = O.gva_decode(V, kr, q_nope, q_rope, M, [30], 0.3)
    outp = O.gva_decode([V[0][:, perm]], [kr[0][perm]], q_nope, q_rope, M, [30], 0.3)
    assert np.allclose(out, outp, rtol=1e-12, atol=1e-14)


def test_empty_sequence_gives_zeros():
    rng = _rng(14)
    V, kr, q_nope, q_rope, M = _problem(rng)
    out = O.gva_decode(V, kr, q_nope, q_rope, M, [0, 5], 0.3)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    assert np.any(out[1] != 0)


def test_large_scores_are_stable():
    rng = _rng(15)
    V, kr, q_nope, q_rope, M = _problem(rng)
    out = O.gva_decode(V, kr, q_nope * 1e3, q_rope * 1e3, M, [12, 12], 1.0)
    assert np.all(np.isfinite(out))


def test_positional_term_and_query_position():
    """Content term off (M = 0). The query's positional slice equals token n-1's
    pre-RoPE key x (x lives in pair 0 only, large), and token n-2's pre-RoPE
    key is R_2 x. With the query at p = n-1 the rotated keys give scores |x|^2
    (token n-1) and |x|^2 cos(theta_0) (token n-2), so out ~ V[n-1]. With a
    wrong query position p = n the roles swap; with the positional term
    dropped the output is the mean of the values."""
    rng = _rng(16)
    G, H, d, d_r, n = 1, 2, 8, 4, 10
    V = [rng.standard_normal((G, n, d))]
    x = np.array([40.0, 0.0, 0.0, 0.0])
    kr_pre = rng.standard_normal((n, d_r)) * 0.1
    kr_pre[n - 1] = x
    kr_pre[n - 2] = O.rope(x, 2)
    q_rope_pre = np.tile(x, (1, H, 1))
    M = np.zeros((H, d, d))
    q_nope = rng.standard_normal((1, H, d))
    out = O.gva_decode_step(V, [kr_pre], q_nope, q_rope_pre, M, [n], 1.0 / math.sqrt(d + d_r),
                            10000.0, "f64")
    for h in range(H):
        assert np.allclose(out[0, h], V[0][0][n - 1], atol=1e-6)


def test_shift_invariance_of_positions():
    """Moving the whole sequence to later positions (query and keys together)
    leaves the output unchanged: RoPE enters only through relative offsets."""
    rng = _rng(17)
    G, H, d, d_r, n, c = 2, 4, 8, 8, 15, 100000
    V = [rng.standard_normal((G, n, d))]
    kr_pre = rng.standard_normal((n, d_r))
    q_nope = rng.standard_normal((1, H, d))
    q_rope_pre = rng.standard_normal((1, H, d_r))
    M = rng.standard_normal((H, d, d)) * 0.3
    scale = 0.35
    kr0 = O.rope(kr_pre, np.arange(n))
    q0 = O.rope(q_rope_pre, np.array([[n - 1]]))
    krc = O.rope(kr_pre, np.arange(n) + c)
    qc = O.rope(q_rope_pre, np.array([[n - 1 + c]]))
    o0 = O.gva_decode(V, [kr0], q_nope, q0, M, [n], scale)
    oc = O.gva_decode(V, [krc], q_nope, qc, M, [n], scale)
    assert np.allclose(o0, oc, rtol=1e-9, atol=1e-12)


def _brute_force(Vb, krb_pre, qn, qr_pre, M, n, scale, H, G, base=10000.0):
    """Scalar loops over Python floats; RoPE through complex multiplication."""
    d_v = len(Vb[0][0])
    d_n = len(M[0][0])
    d_r = len(qr_pre[0])
    hpg = H // G

    def rot(v, pos):
        r = []
        for i in range(d_r // 2):
            z = complex(v[2 * i], v[2 * i + 1]) * cmath.exp(1j * pos * base ** (-2.0 * i / d_r))
            r += [z.real, z.imag]
        return r

    out = []
    for h in range(H):
        g = h // hpg
        qrot = rot(qr_pre[h], n - 1)
        s = []
        for t in range(n):
            key = [sum(Vb[g][t][i] * M[h][i][j] for i in range(d_v)) for j in range(d_n)]
            key += rot(krb_pre[t], t)
            qv = list(qn[h]) + qrot
            s.append(scale * sum(a * b for a, b in zip(key, qv)))
        mx = max(s)
        w = [math.exp(v - mx) for v in s]
        tot = sum(w)
        out.append([sum(w[t] * Vb[g][t][k] for t in range(n)) / tot for k in range(d_v)])
    return out


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8])
def test_brute_force_tiny(n):
    rng = _rng(100 + n)
    H, G, d, d_r = 4, 2, 6, 4
    V = [rng.standard_normal((G, n, d))]
    kr_pre = rng.standard_normal((n, d_r))
    q_nope = rng.standard_normal((1, H, d))
    q_rope = rng.standard_normal((1, H, d_r))
    M = rng.standard_normal((H, d, d))
    scale = 1 / math.sqrt(d + d_r)
    ref = _brute_force(V[0].tolist(), kr_pre.tolist(), q_nope[0].tolist(), q_rope[0].tolist(),
                       M.tolist(), n, scale, H, G)
    out = O.gva_decode_step(V, [kr_pre], q_nope, q_rope, M, [n], scale, 10000.0, "f64")
    assert np.allclose(out[0], np.array(ref), rtol=1e-12, atol=1e-13)


def test_step_rounds_cached_keys_to_cache_dtype():
    """The end-to-end step sees positional keys as the bf16 cache holds them."""
    rng = _rng(18)
    G, H, d, d_r, n = 1, 2, 8, 4, 6
    V = [O.round_bf16(rng.standard_normal((G, n, d)))]
    kr_pre = O.round_bf16(rng.standard_normal((n, d_r)))
    q_nope = O.round_bf16(rng.standard_normal((1, H, d)))
    q_rope = O.round_bf16(rng.standard_normal((1, H, d_r)))
    M = O.round_bf16(rng.standard_normal((H, d, d)) / 8)
    out = O.gva_decode_step(V, [kr_pre], q_nope, q_rope, M, [n], 0.3, 10000.0, "bf16")
    kr_cache = O.round_bf16(O.rope(kr_pre, np.arange(n)))
    ref = O.gva_decode(V, [kr_cache], q_nope, O.rope(q_rope, np.array([[n - 1]])), M, [n], 0.3)
    assert np.array_equal(out, ref)


# ---------------------------------------------------------------------------
# Query projection and the fold of the maps into it ([digest] 与现有产品 /
# 工作流的接口: the reconstruction matrix can be folded into the query
# projection at inference)
# ---------------------------------------------------------------------------

def test_query_projection_matches_per_head_dot_products():
    """Against scalar loops over heads, channels and the hidden dimension."""
    rng = np.random.default_rng(40)
    H, d, d_model, B = 3, 5, 7, 2
    w = rng.standard_normal((H, d, d_model))
    x = rng.standard_normal((B, d_model))
    got = O.query_projection(x, w)
    for b in range(B):
        for h in range(H):
            for i in range(d):
                ref = sum(float(w[h, i, m]) * float(x[b, m]) for m in range(d_model))
                assert abs(got[b, h, i] - ref) < 1e-12


def test_fold_closed_forms():
    """Folding the identity map gives the projection back; folding into an
    identity projection (d_model = d_n) gives the maps back."""
    rng = np.random.default_rng(41)
    H, d, d_model = 2, 4, 6
    wq = rng.standard_normal((H, d, d_model))
    M = rng.standard_normal((H, d, d))
    eye = np.broadcast_to(np.eye(d), (H, d, d))
    assert np.allclose(O.fold_query_projection(eye, wq), wq, rtol=0, atol=0)
    assert np.allclose(O.fold_query_projection(M, eye), M, rtol=0, atol=0)


def test_layer_step_with_selection_projection_is_the_step():
    """With x holding every head's (q_nope, q_rope) and the projection rows
    selecting them, the layer step reduces to the step on those queries."""
    wl = W.Workload("pin_layer", 9, B=2, H=4, G=2, d_n=8, d_v=8, d_r=4, S=9, dtype="f32")
    inp = W.make_gva_inputs(wl, seed=42)
    dq = wl.d_n + wl.d_r
    d_model = wl.H * dq
    x = np.zeros((wl.B, d_model))
    wq_nope = np.zeros((wl.H, wl.d_n, d_model))
    wq_rope = np.zeros((wl.H, wl.d_r, d_model))
    for h in range(wl.H):
        x[:, h * dq:h * dq + wl.d_n] = inp.q_nope[:, h]
        x[:, h * dq + wl.d_n:(h + 1) * dq] = inp.q_rope[:, h]
        wq_nope[h, :, h * dq:h * dq + wl.d_n] = np.eye(wl.d_n)
        wq_rope[h, :, h * dq + wl.d_n:(h + 1) * dq] = np.eye(wl.d_r)
    got = O.gva_layer_decode_step(inp.V, inp.kr, x, wq_nope, wq_rope, inp.M, inp.lens, wl.scale,
                                  10000.0, "f32")
    ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, inp.lens, wl.scale,
                            10000.0, "f32")
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_folded_query_gives_the_materialized_scores():
    """Absorption through the fold: decoding with q' = (M W_q,nope) x against
    plain values (identity maps, K = V) equals the layer step with the
    materialized keys V M and q_nope = W_q,nope x ([digest] 方法, Q' = Q M^T)."""
    wl = W.Workload("pin_fold", 9, B=2, H=4, G=2, d_n=8, d_v=8, d_r=4, S=11, dtype="f32")
    inp = W.make_gva_inputs(wl, seed=43)
    x, wq_nope, wq_rope = W.make_projection_inputs(wl, d_model=16, seed=44)
    layer = O.gva_layer_decode_step(inp.V, inp.kr, x, wq_nope, wq_rope, inp.M, inp.lens, wl.scale,
                                    10000.0, "f32")
    q_abs = O.query_projection(x, O.fold_query_projection(inp.M, wq_nope))
    eye = np.broadcast_to(np.eye(wl.d_v), (wl.H, wl.d_v, wl.d_v))
    folded = O.gva_decode_step(inp.V, inp.kr, q_abs, O.query_projection(x, wq_rope), eye, inp.lens,
                               wl.scale, 10000.0, "f32")
    assert np.allclose(folded, layer, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# Several new tokens' queries at once (causal over the new tokens)
# ---------------------------------------------------------------------------

def test_multi_query_decode_brute_force_causal_mask():
    """Scalar loops with an explicit causal mask over the whole cache: query j
    at position n - n_q + j sees token t only when t <= n - n_q + j."""
    wl = W.Workload("pin_multi", 9, B=2, H=4, G=2, d_n=4, d_v=4, d_r=2, S=0, dtype="f32")
    lens = np.array([5, 3])
    inp = W.make_gva_inputs(wl, lens=lens, seed=50)
    nq = 4
    rng = np.random.default_rng(51)
    qn = rng.standard_normal((2, nq, 4, 4))
    qr = rng.standard_normal((2, nq, 4, 2))
    got = O.gva_decode_multi(inp.V, inp.kr, qn, qr, inp.M, lens, 0.4)
    for b in range(2):
        n = int(lens[b])
        for j in range(nq):
            p = n - nq + j
            for h in range(4):
                g = h // 2
                s = []
                for t in range(n):
                    if t > p:
                        s.append(-math.inf)
                        continue
                    k_c = [sum(inp.V[b][g, t, v] * inp.M[h][v, c] for v in range(4)) for c in range(4)]
                    dot = sum(k_c[c] * qn[b, j, h, c] for c in range(4))
                    dot += sum(inp.kr[b][t, c] * qr[b, j, h, c] for c in range(2))
                    s.append(0.4 * dot)
                mx = max(s)
                if mx == -math.inf:
                    assert np.all(got[b, j, h] == 0.0)
                    continue
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for c in range(4):
                    ref = sum(w[t] * inp.V[b][g, t, c] for t in range(n)) / tot
                    assert abs(got[b, j, h, c] - ref) < 1e-12


def test_multi_query_single_is_decode():
    wl = W.Workload("pin_multi1", 9, B=3, H=8, G=2, d_n=8, d_v=8, d_r=4, S=17, dtype="f32")
    inp = W.make_gva_inputs(wl, seed=52)
    got = O.gva_decode_multi_step(inp.V, inp.kr, inp.q_nope[:, None], inp.q_rope[:, None], inp.M,
                                  inp.lens, wl.scale, 10000.0, "f32")
    ref = O.gva_decode_step(inp.V, inp.kr, inp.q_nope, inp.q_rope, inp.M, inp.lens, wl.scale,
                            10000.0, "f32")
    assert np.array_equal(got[:, 0], ref)


def test_prefill_brute_force_causal():
    """The masked-matrix prefill against scalar loops over the explicit causal
    mask (including queries before the first cached token, which read nothing)."""
    wl = W.Workload("pin_prefill", 9, B=2, H=4, G=2, d_n=4, d_v=4, d_r=2, S=0, dtype="f32")
    lens = np.array([6, 3])
    inp = W.make_gva_inputs(wl, lens=lens, seed=60)
    nq = 5
    rng = np.random.default_rng(61)
    qn = rng.standard_normal((2, nq, 4, 4))
    qr = rng.standard_normal((2, nq, 4, 2))
    got = O.gva_prefill(inp.V, inp.kr, qn, qr, inp.M, lens, 0.3)
    for b in range(2):
        n = int(lens[b])
        for j in range(nq):
            p = n - nq + j
            for h in range(4):
                g = h // 2
                if p < 0:
                    assert np.all(got[b, j, h] == 0.0)
                    continue
                s = []
                for t in range(p + 1):
                    k_c = [sum(inp.V[b][g, t, v] * inp.M[h][v, c] for v in range(4)) for c in range(4)]
                    dot = sum(k_c[c] * qn[b, j, h, c] for c in range(4))
                    dot += sum(inp.kr[b][t, c] * qr[b, j, h, c] for c in range(2))
                    s.append(0.3 * dot)
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for c in range(4):
                    ref = sum(w[t] * inp.V[b][g, t, c] for t in range(p + 1)) / tot
                    assert abs(got[b, j, h, c] - ref) < 1e-12


def test_prefill_closed_forms_and_causality():
    """Query 0 of a whole-prompt prefill sees only token 0 (its value row,
    exactly); constant value rows give that constant; the last query is the
    plain decode; and changing tokens after position p leaves query p alone."""
    wl = W.Workload("pin_prefill2", 9, B=2, H=8, G=4, d_n=8, d_v=8, d_r=4, S=0, dtype="f32")
    lens = np.array([12, 7])
    inp = W.make_gva_inputs(wl, lens=lens, seed=62)
    rng = np.random.default_rng(63)
    nq = 12
    qn = rng.standard_normal((2, nq, 8, 8))
    qr = rng.standard_normal((2, nq, 8, 4))
    got = O.gva_prefill(inp.V, inp.kr, qn, qr, inp.M, lens, 0.25)
    for h in range(8):
        assert np.array_equal(got[0, 0, h], inp.V[0][h // 2, 0])
    last = O.gva_decode_seq(inp.V[0], inp.kr[0], qn[0, -1], qr[0, -1], inp.M, 12, 0.25)
    assert np.allclose(got[0, -1], last, rtol=0, atol=1e-13)
    # sequence 1 (7 tokens, 12 queries): the first five read nothing
    assert np.all(got[1, :5] == 0.0) and np.all(np.abs(got[1, 5:]).sum(axis=-1) > 0)
    const = [np.full_like(v, 0.75) for v in inp.V]
    got_c = O.gva_prefill(const, inp.kr, qn, qr, inp.M, lens, 0.25)
    assert np.allclose(got_c[0], 0.75, atol=1e-14) and np.allclose(got_c[1, 5:], 0.75, atol=1e-14)
    V2 = [v.copy() for v in inp.V]
    kr2 = [k.copy() for k in inp.kr]
    V2[0][:, 6:] = rng.standard_normal(V2[0][:, 6:].shape)
    kr2[0][6:] = rng.standard_normal(kr2[0][6:].shape)
    got2 = O.gva_prefill(V2, kr2, qn, qr, inp.M, lens, 0.25)
    assert np.array_equal(got2[0, :6], got[0, :6]) and not np.allclose(got2[0, 6:], got[0, 6:])


def test_prefill_equals_the_per_query_decode_loop():
    """The masked-matrix form against the per-query loop (gva_decode_multi),
    from pre-RoPE inputs, including a sequence shorter than the query count."""
    wl = W.Workload("pin_prefill3", 9, B=3, H=8, G=2, d_n=8, d_v=8, d_r=4, S=0, dtype="f32")
    lens = np.array([20, 9, 1])
    inp = W.make_gva_inputs(wl, lens=lens, seed=64)
    rng = np.random.default_rng(65)
    nq = 10
    qn = rng.standard_normal((3, nq, 8, 8))
    qr = rng.standard_normal((3, nq, 8, 4))
    a = O.gva_prefill_step(inp.V, inp.kr, qn, qr, inp.M, lens, 0.3, 10000.0, "f32")
    b = O.gva_decode_multi_step(inp.V, inp.kr, qn, qr, inp.M, lens, 0.3, 10000.0, "f32")
    assert np.allclose(a, b, rtol=0, atol=1e-12)
