"""CPU fp64 oracle for Grouped Value Attention (GVA) decode over a compact cache.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark use it. It shares no
code with the HIP library (no kernels, headers, tables or helpers), and it
is deliberately plain and slow: it builds every per-head content key
explicitly and runs ordinary softmax attention in float64.

Pages cited (title, where it lives):
  [digest]   "Grouped Value Attention:通过按需 key 重建实现高效 KV 缓存",
             ai-feeds.com paper digest of arXiv 2609.13285
  [explain]  popular explainer of the same paper, m.szthrk.cn/tech/5057398
  [abstract] "Grouped Value Attention: Efficient KV Caching via On-Demand Key
             Reconstruction", Hugging Face papers page (abstract)
  [review]   "[논문리뷰] Grouped Value Attention: Efficient KV Caching via
             On-Demand Key Reconstruction", blog.secrett2633.cloud
  [gqa]      "GQA 分组查询注意力：KV Cache 与模型质量的折中",
             charlestar.github.io (generic GQA tutorial)

What the method computes, per sequence b, query head h, cached tokens t<n:
  g(h)   = h // (H / G)                             head -> value group
  K_h[t] = [ V_g(h)[t] M_h  ||  RoPE_t(k~_r[t]) ]   content key rebuilt from
           the value through the per-head map M_h ([digest] 方法 / GVA 核心
           流程; [review] 3. Method & Key Results), plus the one positional
           key shared by all heads ([explain] 位置信息怎么办; [review]
           Decoupled RoPE)
  Q_h    = [ q_nope,h || RoPE_p(q~_rope,h) ],  p = n - 1 (the query reads the
           earlier tokens and its own, [gqa] KV Cache 为什么会不断变大)
  out_h  = softmax_t(scale * Q_h . K_h[t]) weighted sum of V_g(h)[t]
           ([digest] 方法: the output is the usual value-weighted sum)
The decode kernels never build K_h: they fold M_h into the query. The two
forms are equal exactly in real arithmetic ([digest] 方法; [explain] 正式方案),
so the oracle is the plain materialized definition.

Readings where the pages are silent (each also listed in the design notes):
  * M_h has shape [d_v, d_n] and keys are row vectors K = V M (the pages'
    K_h = V_g(h) M_h); stored [H, d_v, d_n].
  * head h uses group h // (H/G) (contiguous head blocks, as in the GQA
    tutorial's diagram of heads 0-3 -> group 0, [gqa] MHA、MQA 与 GQA 的结构关系).
  * RoPE pairs adjacent channels (2i, 2i+1) and turns them by pos * theta_i,
    theta_i = base^(-2i/d_r), base 10000; the pages fix no convention and
    only require the cached key and the query to use the same one
    ([gqa] 与位置编码和 KV Cache 的关系).
  * The cache stores the positional key after RoPE, rounded once
    (round-to-nearest-even) to the cache dtype; V is never rotated.
  * An empty sequence (n = 0) yields a zero output row.
Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math
from typing import List, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# Rounding to storage formats
# ---------------------------------------------------------------------------

_BF16_MANT_BITS = 7          # stored fraction bits of bfloat16
_BF16_EMIN = -126            # smallest normal exponent (same as binary32)
_BF16_MAX = float.fromhex("0x1.fep127")


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even.

    A bfloat16 normal number 2^e * 1.f has 7 fraction bits, so its spacing is
    2^(e-7); below the normal range the spacing stays 2^(-126-7). Dividing by
    the spacing gives an exactly representable float64, which np.rint rounds
    half-to-even; multiplying back is exact. Values that round beyond the
    largest finite bfloat16 become +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                 # x = m * 2^e, 0.5 <= |m| < 1
    exp = np.maximum(e.astype(np.int64) - 1, _BF16_EMIN)
    quantum = np.ldexp(1.0, (exp - _BF16_MANT_BITS).astype(np.int64))
    r = np.rint(x[nz] / quantum) * quantum
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def round_storage(x, dtype: str) -> np.ndarray:
    """Round to the cache dtype: 'bf16' (RNE), 'f32' (IEEE RNE) or 'f64'."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f64":
        return x.copy()
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Rotary position embedding on the positional slice
# ---------------------------------------------------------------------------

def rope_thetas(d_r: int, base: float = 10000.0) -> np.ndarray:
    """Per-pair frequencies theta_i = base^(-2i/d_r), i = 0 .. d_r/2-1."""
    i = np.arange(d_r // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d_r)


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis of x (width d_r, even) by position pos.

    Pair i = (x[2i], x[2i+1]) is turned counter-clockwise by pos * theta_i.
    `pos` broadcasts against x's leading axes.
    """
    x = np.asarray(x, dtype=np.float64)
    d_r = x.shape[-1]
    if d_r == 0:
        return x.copy()
    assert d_r % 2 == 0
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_thetas(d_r, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# ---------------------------------------------------------------------------
# Head -> group map and cache accounting
# ---------------------------------------------------------------------------

def head_group(h: int, H: int, G: int) -> int:
    """Value group read by query head h: contiguous blocks of H/G heads."""
    assert H % G == 0
    return h // (H // G)


def gva_scalars_per_token(G: int, d_v: int, d_r: int) -> int:
    """Persistent cache scalars per token per layer for GVA: G grouped value
    rows plus ONE positional key shared by all heads ([explain] 位置信息怎么办
    and 省下来的到底是多少; [review] Decoupled RoPE)."""
    return G * d_v + d_r


def gqa_scalars_per_token(G: int, d_h: int) -> int:
    """Matched GQA stores a key and a value row per KV head ([gqa] KV Cache
    为什么会不断变大: the factor 2 counts K and V)."""
    return 2 * G * d_h


def kv_cache_bytes(layers: int, seq_len: int, kv_heads: int, head_dim: int,
                   bytes_per_elem: int, n_seqs: int = 1) -> int:
    """Bytes of a K+V cache: 2 * L * S * H_kv * d_h * b per sequence
    ([gqa] KV Cache 为什么会不断变大 and 用一个具体模型估算缓存)."""
    return 2 * layers * seq_len * kv_heads * head_dim * bytes_per_elem * n_seqs


# ---------------------------------------------------------------------------
# Cache writes (what one append step stores)
# ---------------------------------------------------------------------------

def append_positional_keys(kr_pre, start: int, base: float, cache_dtype: str) -> np.ndarray:
    """Cache contents for positional keys at positions start, start+1, ...:
    RoPE at each token's own position, then one rounding to the cache dtype.
    kr_pre: [n_new, d_r] before RoPE."""
    kr_pre = np.asarray(kr_pre, dtype=np.float64)
    pos = np.arange(start, start + kr_pre.shape[0], dtype=np.float64)
    return round_storage(rope(kr_pre, pos, base), cache_dtype)


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------

def _softmax(s: np.ndarray) -> np.ndarray:
    s = s - np.max(s)
    w = np.exp(s)
    return w / np.sum(w)


def materialized_keys(Vg, M_h, kr_rot) -> np.ndarray:
    """K_h = [V_g M_h || k_r (already rotated)], shape [n, d_n + d_r]."""
    Kc = np.asarray(Vg, dtype=np.float64) @ np.asarray(M_h, dtype=np.float64)
    return np.concatenate([Kc, np.asarray(kr_rot, dtype=np.float64)], axis=1)


def gva_head_scores(Vg, kr_rot, q_nope_h, q_rope_rot_h, M_h, scale: float) -> np.ndarray:
    """Scaled scores of one head over n tokens with explicit keys."""
    K = materialized_keys(Vg, M_h, kr_rot)
    Q = np.concatenate([np.asarray(q_nope_h, np.float64), np.asarray(q_rope_rot_h, np.float64)])
    return float(scale) * (K @ Q)


def gva_decode_seq(Vb, krb, q_nope_b, q_rope_b, M, n: int, scale: float) -> np.ndarray:
    """One sequence. Vb [G, >=n, d_v]; krb [>=n, d_r] (rotated cache rows);
    q_nope_b [H, d_n]; q_rope_b [H, d_r] (rotated); M [H, d_v, d_n].
    Returns out [H, d_v]."""
    G, _, d_v = Vb.shape
    H = q_nope_b.shape[0]
    out = np.zeros((H, d_v))
    if n == 0:
        return out
    for h in range(H):
        g = head_group(h, H, G)
        Vg = np.asarray(Vb[g, :n, :], dtype=np.float64)
        s = gva_head_scores(Vg, krb[:n], q_nope_b[h], q_rope_b[h], M[h], scale)
        out[h] = _softmax(s) @ Vg
    return out


def gva_decode(V: Sequence[np.ndarray], kr: Sequence[np.ndarray], q_nope, q_rope, M,
               seq_lens, scale: float) -> np.ndarray:
    """Batched decode. V[b] [G, >=n_b, d_v]; kr[b] [>=n_b, d_r] rotated cache
    rows; q_rope already rotated. Returns out [B, H, d_v] float64."""
    B = len(seq_lens)
    out = np.zeros((B, q_nope.shape[1], V[0].shape[-1]))
    for b in range(B):
        out[b] = gva_decode_seq(V[b], kr[b], q_nope[b], q_rope[b], M, int(seq_lens[b]), scale)
    return out


def gva_decode_step(V, kr_pre, q_nope, q_rope_pre, M, seq_lens, scale: float,
                    base: float, cache_dtype: str) -> np.ndarray:
    """End-to-end step from pre-RoPE inputs: the cache holds RoPE_t(k~_r[t])
    rounded to the cache dtype; the query's positional slice is rotated at
    p = n-1 (kept in float64). Then plain decode attention."""
    kr_rot = [append_positional_keys(np.asarray(k)[:int(n)], 0, base, cache_dtype)
              for k, n in zip(kr_pre, seq_lens)]
    pos = np.maximum(np.asarray(seq_lens, dtype=np.float64) - 1.0, 0.0)
    q_rot = rope(q_rope_pre, pos[:, None], base)
    return gva_decode(V, kr_rot, q_nope, q_rot, M, seq_lens, scale)


def gva_decode_multi(V, kr, q_nope, q_rope, M, seq_lens, scale: float) -> np.ndarray:
    """Decode of the last n_q cached tokens' queries at once. q_nope
    [B, n_q, H, d_n], q_rope [B, n_q, H, d_r] (rotated). Query j of sequence b
    sits at position p = n - n_q + j (n = seq_lens[b]) and reads the tokens up
    to and including its own, t <= p ([gqa] KV Cache 为什么会不断变大); a
    negative p reads nothing (zero row). Returns [B, n_q, H, d_v] float64."""
    q_nope = np.asarray(q_nope)
    B, nq = q_nope.shape[:2]
    out = np.zeros((B, nq, q_nope.shape[2], V[0].shape[-1]))
    for b in range(B):
        n = int(seq_lens[b])
        for j in range(nq):
            p = n - nq + j
            if p >= 0:
                out[b, j] = gva_decode_seq(V[b], kr[b], q_nope[b, j], q_rope[b, j], M, p + 1, scale)
    return out


def gva_decode_multi_step(V, kr_pre, q_nope, q_rope_pre, M, seq_lens, scale: float,
                          base: float, cache_dtype: str) -> np.ndarray:
    """As gva_decode_multi from pre-RoPE inputs: the cache holds RoPE_t(k~_r[t])
    rounded to the cache dtype, query j is rotated at its own position
    n - n_q + j (float64)."""
    q_rope_pre = np.asarray(q_rope_pre, dtype=np.float64)
    nq = q_rope_pre.shape[1]
    kr_rot = [append_positional_keys(np.asarray(k)[:int(n)], 0, base, cache_dtype)
              for k, n in zip(kr_pre, seq_lens)]
    pos = np.maximum(np.asarray(seq_lens, dtype=np.float64)[:, None] - nq + np.arange(nq)[None, :], 0.0)
    q_rot = rope(q_rope_pre, pos[:, :, None], base)
    return gva_decode_multi(V, kr_rot, q_nope, q_rot, M, seq_lens, scale)


def gva_prefill(V, kr, q_nope, q_rope, M, seq_lens, scale: float) -> np.ndarray:
    """Causal attention of the last n_q cached tokens of every sequence, the
    whole prompt when n_q = n ([gqa] KV Cache 为什么会不断变大: each token's
    query reads the tokens before it and itself). Plain definition with
    materialized keys, per (b, h): K = [V_g M_h | k_r] over the n cached tokens
    (k_r rotated), Q = [q_nope | q_rope] of the n_q queries (q_rope rotated),
    query j at position p_j = n - n_q + j; scores scale * Q K^T with the
    entries t > p_j removed, softmax per row, times V_g. A row with p_j < 0
    reads nothing and is zero. q_nope [B, n_q, H, d_n], q_rope
    [B, n_q, H, d_r]; returns [B, n_q, H, d_v] float64."""
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    B, nq, H = q_nope.shape[:3]
    G, _, d_v = np.asarray(V[0]).shape
    out = np.zeros((B, nq, H, d_v))
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        pos = n - nq + np.arange(nq)
        rows = pos >= 0
        allowed = np.arange(n)[None, :] <= pos[:, None]  # [n_q, n]
        for h in range(H):
            g = head_group(h, H, G)
            Vg = np.asarray(V[b][g, :n, :], dtype=np.float64)
            K = materialized_keys(Vg, M[h], np.asarray(kr[b])[:n])
            Q = np.concatenate([q_nope[b, :, h], q_rope[b, :, h]], axis=1)
            S = np.where(allowed, float(scale) * (Q @ K.T), -np.inf)
            S = S[rows]
            E = np.exp(S - S.max(axis=1, keepdims=True))
            out[b, rows, h] = (E / E.sum(axis=1, keepdims=True)) @ Vg
    return out


def gva_prefill_step(V, kr_pre, q_nope, q_rope_pre, M, seq_lens, scale: float, base: float,
                     cache_dtype: str) -> np.ndarray:
    """As gva_prefill from pre-RoPE inputs: the cache holds RoPE_t(k~_r[t])
    rounded to the cache dtype, query j is rotated at its own position
    n - n_q + j (float64)."""
    q_rope_pre = np.asarray(q_rope_pre, dtype=np.float64)
    nq = q_rope_pre.shape[1]
    kr_rot = [append_positional_keys(np.asarray(k)[:int(n)], 0, base, cache_dtype)
              for k, n in zip(kr_pre, seq_lens)]
    pos = np.maximum(np.asarray(seq_lens, dtype=np.float64)[:, None] - nq + np.arange(nq)[None, :], 0.0)
    q_rot = rope(q_rope_pre, pos[:, :, None], base)
    return gva_prefill(V, kr_rot, q_nope, q_rot, M, seq_lens, scale)


# ---------------------------------------------------------------------------
# The query projection, and the maps folded into it ([digest] 与现有产品 /
# 工作流的接口: at inference the reconstruction matrix can be folded into the
# query projection, so content keys are never formed)
# ---------------------------------------------------------------------------

def query_projection(x, w) -> np.ndarray:
    """Per-head linear projection of hidden states: w [H, d, d_model] applied
    to x [B, d_model] gives [B, H, d] (q[b, h] = w[h] @ x[b]), float64."""
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    return np.transpose(np.matmul(w, x.T), (2, 0, 1))


def fold_query_projection(M, wq_nope) -> np.ndarray:
    """W'_h = M_h @ W_q,nope,h, [H, d_v, d_model] float64. Since q_nope,h =
    W_q,nope,h x, the absorbed query M_h q_nope,h equals W'_h x."""
    return np.matmul(np.asarray(M, dtype=np.float64), np.asarray(wq_nope, dtype=np.float64))


def gva_layer_decode_step(V, kr_pre, x, wq_nope, wq_rope, M, seq_lens, scale: float,
                          base: float, cache_dtype: str) -> np.ndarray:
    """One layer's decode step from the new tokens' hidden states x [B, d_model],
    by the plain definition: q_nope = W_q,nope x and the pre-RoPE positional
    slice q_rope = W_q,rope x (float64, never rounded), then gva_decode_step
    with the materialized keys V_g(h) M_h. A folded path (W' = M W_q,nope,
    q' = W' x, no M in the decode) must reach the same result."""
    q_nope = query_projection(x, wq_nope)
    q_rope = query_projection(x, wq_rope)
    return gva_decode_step(V, kr_pre, q_nope, q_rope, M, seq_lens, scale, base, cache_dtype)


def gqa_decode(q, K, V, seq_lens, scale: float) -> np.ndarray:
    """Plain GQA decode: head h attends to K/V of group h // (H/G).
    q [B, H, d_h]; K, V [B, G, >=n, d_h] (K already rotated)."""
    B, H, _ = q.shape
    G = K.shape[1] if not isinstance(K, list) else K[0].shape[0]
    out = np.zeros((B, H, V[0].shape[-1]))
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        for h in range(H):
            g = head_group(h, H, G)
            Kg = np.asarray(K[b][g, :n, :], dtype=np.float64)
            Vg = np.asarray(V[b][g, :n, :], dtype=np.float64)
            s = float(scale) * (Kg @ np.asarray(q[b, h], dtype=np.float64))
            out[b, h] = _softmax(s) @ Vg
    return out
