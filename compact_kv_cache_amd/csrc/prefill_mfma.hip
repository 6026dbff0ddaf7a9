// Causal GVA prefill on the gfx950 matrix cores: the last nq cached tokens of
// every sequence are queries, query j at position p_j = seq_lens[b] - nq + j
// attending to the tokens t <= p_j (the GQA tutorial page, section on the
// KV cache: every new token's query reads the cache up to and including
// itself). With nq = seq_lens[b] this is the attention of a whole prompt.
//
// The keys are never formed. As in the decode, head h's key is
// [V_g(h) M_h | k_r] and its query [q_nope,h | RoPE(q_rope,h)], so the scores
// are q'_h . V_g(h)[t] + q_rope,h . k_r[t] with q'_h = M_h q_nope,h (GVA
// digest, 方法: Q' = Q M^T; explainer, 正式方案), and the values are V_g(h).
// One staged tile of V_g and k_r feeds every head of the group and every
// query of the workgroup.
//
// Work split: one workgroup of 4 waves per (sequence, group, block of
// queries). The block's (query, head) pairs form blocks of 16 matrix-core
// columns (16 queries of one head each); every wave owns four column blocks
// (three where four would not fit 256 registers without spilling: H/G < 4 or
// d_r = 32) and keeps their absorbed queries, running softmax state and
// output accumulators in registers (two waves per SIMD, two workgroups per
// compute unit). The workgroup walks the key tiles 0 .. (last query's
// position) / 64 once: each tile is loaded by its 256 threads (two 16-byte
// buffer loads each for the V rows, the positional keys alongside), stored
// to one of two LDS buffers while the other is computed, and read by every
// wave. (Measured at the mid shape: 4 waves x 4 blocks ran 1.29x faster than
// 8 waves x 2 blocks.) Per wave and tile, on the matrix cores:
//   scores  S^T[tok][col] = V[tok] . q'[col] + k_r[tok] . q_rope[col] - m_ref
//           (A = V rows from LDS, B = the column block's queries), 12 MFMAs of
//           16x16x32 per block: two for the content part and one for the
//           positional slice, whose spare channel carries the reference shift
//           (d_r <= 24);
//   mask    tokens past a column's own position (tiles on the diagonal only);
//   softmax online per column, the max over the wave's four 16-lane rows with
//           the row-swap permutes;
//   P.V     O^T[ch][col] += V^T[ch][tok] . P^T[tok][col], A = V^T from the
//           LDS transpose load (shared by the wave's column blocks), B = the score
//           accumulator in bf16, 8 MFMAs per block.
// Workgroup ids put all query blocks of one (sequence, group) on one XCD, so
// the tiles that every block re-reads come from that XCD's L2, and the
// latest (longest) query blocks are dispatched first.
#include "gva_device.hpp"
#include "launch.hpp"
#include "prefill.hpp"
#include "mfma_common.hpp"

namespace gva {
namespace {

constexpr int kPWaves = 4;           // waves per workgroup
constexpr float kRescaleLog2P = 8.f; // move the reference max only beyond 2^8

// 16-column blocks per wave: 4 where the state fits the 256 registers of a
// wave at two waves per SIMD without spilling, else 3.
template <int HPG, int KR>
constexpr int prefill_column_blocks() {
  return (HPG == 4 && KR <= 3) || (HPG == 2 && KR == 3) || KR == 0 ? 4 : 3;
}
template <int HPG, int KR>
constexpr int prefill_queries_per_block() {
  return 16 * prefill_column_blocks<HPG, KR>() * kPWaves / HPG;
}

template <int HPG, bool PAGED, int KR>
__global__ __launch_bounds__(64 * kPWaves, 2) void prefill_mfma_kernel(PrefillLaunch a) {
  constexpr bool DR = KR > 0;  // positional slice present (d_r = 8 * KR)
  constexpr int kCB = prefill_column_blocks<HPG, KR>();
  constexpr int QW = prefill_queries_per_block<HPG, KR>();
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, r = lane >> 4;
  const int H = a.H, G = a.G, d_r = a.d_r, nq = a.nq;

  // ---- workgroup -> (sequence, group) pair and query block -----------------
  const int pairs = a.B * G;
  const int p8 = (pairs + 7) / 8;
  const int xcd = blockIdx.x & 7, jj = blockIdx.x >> 3;
  const int pair = 8 * (jj % p8) + xcd;
  if (pair >= pairs) return;  // whole workgroup
  const int qblk = a.n_qblk - 1 - jj / p8;
  const int b = pair / G, g = pair % G;
  const int q0 = qblk * QW;
  const int n = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int first = n - nq;  // position of query 0 (negative: the early queries read nothing)

  // The workgroup reads tokens 0 .. its last query's position.
  const int p_last = first + min(q0 + QW, nq) - 1;
  const int n_tiles = p_last >= 0 ? p_last / kTile + 1 : 0;
  const float sl2 = a.scale * kLog2e;
  const float thr = kRescaleLog2P / sl2;  // the reference moves past this (raw score units)
  const int kr_off = DR ? 8 * min(r, KR - 1) : 0;  // lanes past d_r re-read a valid slice

  // ---- the wave's column blocks: absorbed queries as B operands ---------------
  const __bf16* qn = reinterpret_cast<const __bf16*>(a.q_nope);
  const __bf16* qrp = reinterpret_cast<const __bf16*>(a.q_rope);
  // Positional slice: one K = 32 product. Where d_r <= 24 its spare channel
  // k = d_r carries the reference shift (SK): the key side holds 1 there and
  // the query side -m_ref, rounded to bf16 (the reference is kept
  // bf16-representable), so the scores leave the matrix cores already
  // shifted, with no accumulator start to broadcast per tile. (An earlier form
  // took d_r <= 16 as a separate K = 16 product added per score: hipcc issued
  // a K = 16 and a K = 32 product chained through one accumulator back to
  // back without wait states, which summed wrongly on the GPU.)
  constexpr bool SK = KR >= 1 && KR <= 3;
  Frag qb[kCB][2], qr[DR ? kCB : 1];
  int wave_pmin = INT32_MAX, wave_pmax = -1;  // over the wave's columns (uniform)
#pragma unroll
  for (int u = 0; u < kCB; ++u) {
    const int cb = kCB * w + u, jh = cb % HPG, qg = cb / HPG;
    const int h = g * HPG + jh;
    const int j = q0 + 16 * qg + col;
    const bool jv = j < nq && first + j >= 0;
    const int j_lo = q0 + 16 * qg, j_hi = min(q0 + 16 * qg + 15, nq - 1);
    if (j_lo <= j_hi) {
      wave_pmin = min(wave_pmin, first + j_lo);
      wave_pmax = max(wave_pmax, first + j_hi);
    }
    const int64_t qrow = ((int64_t)b * nq + min(j, nq - 1)) * H + h;  // a valid row for every lane
    Frag q_in[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) q_in[kc].u = ld16(qn + qrow * kD, 32 * kc + 8 * r);
    if (a.M != nullptr) {  // uniform
      // q'^T = M_h q^T: A = rows of M_h in the permuted order that lands the
      // product in the B layout (lane (col, r) gets q'[32*kc + 8r + e] in
      // D[2kc + e/4][e%4]); accumulated in fp32 and rounded to bf16 once.
      const __bf16* Mh = reinterpret_cast<const __bf16*>(a.M) + (int64_t)h * kD * kD;
      f32x4 D[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int chan = 32 * (mb >> 1) + 8 * (col >> 2) + 4 * (mb & 1) + (col & 3);
        Frag m0, m1;
        m0.u = ld16(Mh, chan * kD + 8 * r);
        m1.u = ld16(Mh, chan * kD + 32 + 8 * r);
        D[mb] = mma(m0, q_in[0], kZero4);
        D[mb] = mma(m1, q_in[1], D[mb]);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[u][kc].h[e] = (__bf16)D[2 * kc + (e >> 2)][e & 3];
    } else {  // q_nope already holds q' (the maps folded into the projection)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) qb[u][kc].u = q_in[kc].u;
    }
    if constexpr (DR) {
      Frag x;
      x.u = ld16(qrp + qrow * d_r, kr_off);
      qr[u].u = x.u;  // as given: a scaled copy would add a rounding the scores do not need
      if (8 * r >= d_r) qr[u].u = u32x4{0u, 0u, 0u, 0u};
    }
    if (!jv) {
      qb[u][0].u = qb[u][1].u = u32x4{0u, 0u, 0u, 0u};
      if constexpr (DR) qr[u].u = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- key tiles: cooperative loads into two LDS buffers ------------------------
  // Stage layout per buffer as in the decode: 64 V rows of 128 bytes with
  // their 16-byte chunks XOR-swizzled per row, then the positional-key rows.
  constexpr int kOnesOff = 8192 + 1024 * (KR > 0 ? KR : 0);  // SK: the key side's shift channel
  constexpr int kStage = kOnesOff + (SK ? 3 * 256 * KR + 16 : 0);
  __shared__ __attribute__((aligned(16))) char stage[2][kStage];
  if constexpr (SK) {
    // one 16-byte chunk [1, 0, ..., 0] per 16-token sub-tile, at the sub-tile
    // stride of the positional-key rows, in both buffers (never overwritten)
    if (tid < 8) {
      Frag one;
      one.u = u32x4{0u, 0u, 0u, 0u};
      one.h[0] = (__bf16)1.f;
      *reinterpret_cast<u32x4*>(&stage[tid >> 2][kOnesOff + (tid & 3) * 256 * KR]) = one.u;
    }
  }
  // V: 16-byte chunk c = t + 64*kPWaves*i of the tile (row c/8, chunk c%8)
  constexpr int kNV = 512 / (64 * kPWaves);  // V chunks per thread
  const int vch = tid & 7;
  int v_lds[kNV];
#pragma unroll
  for (int i = 0; i < kNV; ++i) {
    const int vrow = (tid >> 3) + 8 * kPWaves * i;
    v_lds[i] = vrow * (kD * 2) + 16 * (vch ^ stage_swizzle(vrow));
  }
  const __bf16* vc = reinterpret_cast<const __bf16*>(a.v_cache);
  const __bf16* krc = reinterpret_cast<const __bf16*>(a.kr_cache);
  // Tile k's rows [64k, min(64k + 64, n)) form the buffer range; rows past it,
  // a missing page and a tile past the last read as zeros without a memory
  // access. The positional keys take 64*KR threads (1 KB each per 64); the
  // other threads re-read the tile's first 16 bytes and store nothing.
  static_assert(64 * 4 <= 64 * kPWaves, "one positional-key chunk per thread at d_r <= 32");
  auto load_tile = [&](int k, u32x4 (&rv)[kNV], u32x4& rk) {
    const int t0 = k * kTile;
    int rows = k < n_tiles ? min(kTile, n - t0) : 0;
    int64_t vbase = 0, kbase = 0;
    if constexpr (PAGED) {
      const int blk = a.block_table[(int64_t)b * a.max_blocks + min(k, a.max_blocks - 1)];
      const bool ok = blk >= 0 && blk < a.num_blocks;
      vbase = ok ? ((int64_t)blk * G + g) * kBlock * kD : 0;
      kbase = ok ? (int64_t)blk * kBlock * d_r : 0;
      rows = ok ? rows : 0;
    } else {
      vbase = rows > 0 ? (((int64_t)b * G + g) * a.capacity + t0) * kD : 0;
      kbase = rows > 0 ? ((int64_t)b * a.capacity + t0) * d_r : 0;
    }
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(vc + vbase), 0, rows * kD * 2, kBufferWord3);
#pragma unroll
    for (int i = 0; i < kNV; ++i)
      rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + 64 * kPWaves * i) * 16, 0, 0);
    if constexpr (DR) {
      const auto rk_ = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(krc + kbase), 0, rows * 16 * KR, kBufferWord3);
      rk = __builtin_amdgcn_raw_buffer_load_b128(rk_, tid < 64 * KR ? 16 * tid : 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf, const u32x4 (&rv)[kNV], const u32x4& rk) {
#pragma unroll
    for (int i = 0; i < kNV; ++i) *reinterpret_cast<u32x4*>(&stage[buf][v_lds[i]]) = rv[i];
    if constexpr (DR) {
      if (tid < 64 * KR) *reinterpret_cast<u32x4*>(&stage[buf][8192 + 16 * tid]) = rk;
    }
  };

  // ---- per-lane operand offsets (as in the decode) ------------------------------
  // V^T through the LDS transpose load: lane j of a 16-lane group r addresses
  // staged token 4r + j/4 (+ 16h + 32pr) and channels 16db + 4(j%4) .. +3;
  // lane col receives channel 16db + col of four consecutive tokens.
  // Channel block db only flips bits 5-6 of the offset: chunk 2db + (col%4)/2
  // XOR the row swizzle is (2db) ^ ((col%4)/2 ^ swizzle), so offset(db) =
  // offset(0) ^ 32db.
  int tr_off0;
  {
    const int row = 4 * r + (col >> 2);
    tr_off0 = row * (kD * 2) + 16 * (((col & 3) >> 1) ^ stage_swizzle(row)) + 8 * (col & 1);
  }

  // Scores come out of the matrix cores in raw units (q . k, the queries as
  // rounded once: q' = M q to bf16, the positional slice as given) and
  // already shifted by the column's reference max m_ref (through the
  // positional product's shift channel, or the accumulator start where there
  // is none), so p = 2^(scale*log2(e)*s) takes one multiply before the
  // exponential. m_ref is set by the column's first tile and moves only when
  // a tile's shifted max exceeds thr = 8 / (scale*log2(e)) (p stays below
  // about 2^8). (Folding scale*log2(e) into the queries before their bf16
  // rounding would save the multiply, but it rounds the positional slice a
  // second time: a relative error of 2^-9 in scores that can reach tens of
  // log2 units.)
  f32x4 acc[kCB][4];
  float m_ref[kCB], l_run[kCB];
#pragma unroll
  for (int u = 0; u < kCB; ++u) {
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[u][db] = kZero4;
    m_ref[u] = -INFINITY;
    l_run[u] = 0.f;
  }

  auto compute = [&](const char* st_base, int t0) {
    if (t0 > wave_pmax) return;  // every query of the wave is before this tile (uniform)
    Frag sa[4][2], kr[DR ? 4 : 1];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int row = 16 * st + col;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        sa[st][hh].u = *reinterpret_cast<const u32x4*>(st_base + row * (kD * 2) + 16 * ((4 * hh + r) ^ stage_swizzle(row)));
      if constexpr (SK)
        kr[st].u = *reinterpret_cast<const u32x4*>(
            st_base + (r == KR ? kOnesOff + st * 256 * KR : 8192 + row * (16 * KR) + 2 * kr_off));
      else if constexpr (DR)
        kr[st].u = *reinterpret_cast<const u32x4*>(st_base + 8192 + row * (16 * KR) + 2 * kr_off);
    }
    Frag pb[kCB][2];
#pragma unroll
    for (int u = 0; u < kCB; ++u) {
      f32x4 s[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        f32x4 c;
        if constexpr (SK) {
          c = mma(sa[st][0], qb[u][0], kZero4);
        } else {
          const float c0 = m_ref[u] == -INFINITY ? 0.f : -m_ref[u];
          c = mma(sa[st][0], qb[u][0], f32x4{c0, c0, c0, c0});
        }
        c = mma(sa[st][1], qb[u][1], c);
        if constexpr (DR) c = mma(kr[st], qr[u], c);
        s[st] = c;
      }
      // causal mask on the diagonal tiles: token past the column's position
      if (t0 + kTile - 1 > wave_pmin) {
        // position of this lane's column query (-1: no query, nothing visible)
        const int jq = q0 + 16 * ((kCB * w + u) / HPG) + col;
        const int pcol = (jq < nq && first + jq >= 0) ? first + jq : -1;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + 16 * st + 4 * r + i > pcol) s[st][i] = -INFINITY;
      }
      float lmx = -INFINITY;  // over this lane's 16 scores of the column
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmx = fmaxf(lmx, s[st][i]);
      // shift of the reference: the whole max on a column's first tile,
      // else only beyond 2^8; none for a column whose scores are all masked.
      // A lane's own max decides whether any column of the wave may need it;
      // only then is the column max formed across the four lanes.
      const bool unset = m_ref[u] == -INFINITY;
      if (__any(lmx > thr || (unset && lmx != -INFINITY))) {
        const float mx = rows_max(lmx);
        if constexpr (SK) {
          // move the (bf16-representable) reference: the whole max on a
          // column's first tile, else only beyond 2^8; none for a column
          // whose scores are all masked
          const bool move = mx != -INFINITY && (unset || mx > thr);
          if (__any(move)) {
            const float m_new = move ? (float)(__bf16)(unset ? mx : m_ref[u] + mx) : m_ref[u];
            const float shift = move ? (unset ? m_new : m_new - m_ref[u]) : 0.f;
            const float alpha = unset ? 1.f : __builtin_amdgcn_exp2f(-shift * sl2);  // unset: nothing accumulated
            l_run[u] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) acc[u][db] *= alpha;
            m_ref[u] = m_new;
#pragma unroll
            for (int st = 0; st < 4; ++st) s[st] -= shift;
            if (r == KR) qr[u].h[0] = (__bf16)(m_ref[u] == -INFINITY ? 0.f : -m_ref[u]);
          }
        } else {  // d_r = 0 or 32: the shift rides in the accumulator start
          const float shift = (mx == -INFINITY) ? 0.f : (unset || mx > thr) ? mx : 0.f;
          if (__any(shift != 0.f)) {
            const float alpha = unset ? 1.f : __builtin_amdgcn_exp2f(-shift * sl2);  // unset: nothing accumulated
            l_run[u] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db) acc[u][db] *= alpha;
            m_ref[u] = unset ? (mx == -INFINITY ? m_ref[u] : mx) : m_ref[u] + shift;
#pragma unroll
            for (int st = 0; st < 4; ++st) s[st] -= shift;
          }
        }
      }
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[st][i] = __builtin_amdgcn_exp2f(s[st][i] * sl2);
      float psum = s[0][0];  // (not 0 + ...: the compiler keeps an add of +0)
#pragma unroll
      for (int e = 1; e < 16; ++e) psum += s[e >> 2][e & 3];
      l_run[u] += psum;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[u][pr].h[i] = (__bf16)s[2 * pr][i];
          pb[u][pr].h[4 + i] = (__bf16)s[2 * pr + 1][i];
        }
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        Frag vt;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const i16x4 xv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(st_base + (tr_off0 ^ (32 * db)) + (32 * pr + 16 * hh) * (kD * 2)));
          const uint2 xb = __builtin_bit_cast(uint2, xv);
          vt.u[2 * hh] = xb.x;
          vt.u[2 * hh + 1] = xb.y;
        }
#pragma unroll
        for (int u = 0; u < kCB; ++u) acc[u][db] = mma(vt, pb[u][pr], acc[u][db]);
      }
  };

  u32x4 rv[kNV], rk = u32x4{0u, 0u, 0u, 0u};
  load_tile(0, rv, rk);
  store_tile(0, rv, rk);
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int k = 0; k < n_tiles; ++k) {
    load_tile(k + 1, rv, rk);  // past the last tile: empty range
    compute(stage[k & 1], k * kTile);
    store_tile((k + 1) & 1, rv, rk);
    __syncthreads();
  }

  // ---- outputs ---------------------------------------------------------------------
  __bf16* out = reinterpret_cast<__bf16*>(a.out);
#pragma unroll
  for (int u = 0; u < kCB; ++u) {
    const float l = rows_sum(l_run[u]);
    const int cb = kCB * w + u, jh = cb % HPG, qg = cb / HPG;
    const int j = q0 + 16 * qg + col;
    if (j < nq) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      __bf16* orow = out + (((int64_t)b * nq + j) * H + g * HPG + jh) * kD;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        union {
          __bf16 h[4];
          uint2 u;
        } v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v.h[i] = (__bf16)(acc[u][db][i] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * db + 4 * r) = v.u;
      }
    }
  }
}

template <int HPG, int KR>
hipError_t prefill_launch(const PrefillLaunch& a, hipStream_t s) {
  const int pairs = a.B * a.G;
  const dim3 grid(((pairs + 7) / 8) * 8 * a.n_qblk);
  if (a.paged)
    prefill_mfma_kernel<HPG, true, KR><<<grid, 64 * kPWaves, 0, s>>>(a);
  else
    prefill_mfma_kernel<HPG, false, KR><<<grid, 64 * kPWaves, 0, s>>>(a);
  return hipGetLastError();
}

template <int HPG>
hipError_t prefill_dr(const PrefillLaunch& a, hipStream_t s) {
  switch (a.d_r / 8) {
    case 0: return prefill_launch<HPG, 0>(a, s);
    case 1: return prefill_launch<HPG, 1>(a, s);
    case 2: return prefill_launch<HPG, 2>(a, s);
    case 3: return prefill_launch<HPG, 3>(a, s);
    default: return prefill_launch<HPG, 4>(a, s);
  }
}

}  // namespace

template <int HPG>
int queries_per_block_dr(int d_r) {
  switch (d_r / 8) {
    case 0: return prefill_queries_per_block<HPG, 0>();
    case 1: return prefill_queries_per_block<HPG, 1>();
    case 2: return prefill_queries_per_block<HPG, 2>();
    case 3: return prefill_queries_per_block<HPG, 3>();
    default: return prefill_queries_per_block<HPG, 4>();
  }
}

int prefill_queries_per_block(int hpg, int d_r) {
  return hpg == 1 ? queries_per_block_dr<1>(d_r) : hpg == 2 ? queries_per_block_dr<2>(d_r)
                                                             : queries_per_block_dr<4>(d_r);
}

hipError_t launch_prefill_mfma(const PrefillLaunch& a, hipStream_t s) {
  switch (a.H / a.G) {
    case 1: return prefill_dr<1>(a, s);
    case 2: return prefill_dr<2>(a, s);
    default: return prefill_dr<4>(a, s);
  }
}

}  // namespace gva
