// GVA decode (bf16 cache) on the gfx950 matrix cores, and the same-shape GQA
// comparison kernel built from the same skeleton.
//
// Work split: one workgroup per (sequence b, split-K partition, chunk of four
// value groups); wave w of the workgroup owns group g = 4*chunk + w and its
// H/G query heads. Every cache row is read from HBM once per group, never
// once per head (the GQA tutorial page asks fast kernels to read K/V through
// the head map instead of copying it per head, section 一次 GQA 计算如何展开).
//
// Per wave and 16-token sub-tile, all on v_mfma_f32_16x16x32_bf16:
//   scores   S^T[tok][col] = V[tok][:] . q'[head(col)][:]   (+ k_r . q_rope)
//            A operand = V rows exactly as loaded (lane l: token l%16, 8
//            consecutive channels), B operand = the absorbed queries
//            q'_h = M_h q_nope,h (GVA digest, 方法; explainer, 正式方案), with
//            the group's heads repeated across the 16 columns. q' is split
//            into bf16 hi + lo parts so the score keeps ~16 significant bits.
//   transpose  C[tok][c] = V[tok][:] . E[:][c] with E a 0/1 selection of 16
//            channels: produces V^T in the A-operand layout of the next
//            product, exactly (one nonzero term per output).
//   P.V      O^T[ch][col] += V^T[ch][tok] . P^T[tok][col] over 32 tokens; the
//            B operand P^T is the score accumulator itself (same lane layout),
//            rounded to bf16 after the softmax.
// Softmax is online (running max / sum per head, exp2 with scale*log2(e)
// folded into the queries). Long sequences are split into partitions merged
// by the last workgroup to finish (log-sum-exp), inside this launch.
#include "gva_device.hpp"
#include "launch.hpp"

namespace gva {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

union Frag {
  bf16x8 v;
  uint4 u;
  __bf16 h[8];
};

__device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint4 ld16(const __bf16* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Per-wave registers for one 64-token tile: 4 sub-tiles of 16 tokens.
// GVA: score rows = V (sa), positional rows = k_r (kr). GQA: score rows = K
// (sa), value rows = V (vb). For GVA vb aliases sa.
template <bool GQA, bool DR>
struct Tile {
  Frag sa[4][2];  // [sub-tile][channel half]: rows feeding the score product
  Frag vb[GQA ? 4 : 1][GQA ? 2 : 1];
  Frag kr[DR ? 4 : 1];
};

template <int HPG, bool PAGED, bool DR, bool GQA>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeLaunch a) {
  static_assert(!(GQA && DR), "GQA reference has no positional slice");
  const int split = blockIdx.x, chunk = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, r = lane >> 4;  // MFMA column / lane group
  const int H = a.H, G = a.G, d_r = a.d_r;
  const int g = chunk * 4 + w;
  const bool active = g < G;
  const int n = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int n_parts = (n + a.split - 1) / a.split;
  if (split >= max(n_parts, 1)) return;  // uniform per workgroup
  const int t_begin = split * a.split;
  const int t_end = min(n, t_begin + a.split);
  const float sl2 = a.scale * kLog2e;
  const int jcol = col % HPG;               // head (within group) of this lane's column
  const int h_col = g * HPG + jcol;         // its global head index

  __shared__ float qsh[4][4][kD];  // [wave][head in group][channel]

  // ---- prologue: queries into B-operand fragments --------------------------
  Frag qhi[2], qlo[2], qr;
  if (active) {
    if (!GQA) {
      // Absorption: q'_h[d] = sum_j M_h[d][j] q_nope,h[j], lane = d.
      for (int j = 0; j < HPG; ++j) {
        const int h = g * HPG + j;
        const __bf16* Mrow = reinterpret_cast<const __bf16*>(a.M) + ((int64_t)h * kD + lane) * kD;
        const __bf16* qn = reinterpret_cast<const __bf16*>(a.q_nope) + ((int64_t)b * H + h) * kD;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < kD; k += 8) {
          Frag m8, q8;
          m8.u = ld16(Mrow + k);
          q8.u = ld16(qn + k);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf((float)m8.h[e], (float)q8.h[e], acc);
        }
        qsh[w][j][lane] = acc * sl2;
      }
    } else {
      for (int j = 0; j < HPG; ++j) {
        const int h = g * HPG + j;
        qsh[w][j][lane] =
            (float)reinterpret_cast<const __bf16*>(a.q_nope)[((int64_t)b * H + h) * kD + lane] * sl2;
      }
    }
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qsh[w][jcol][32 * kc + 8 * r + e];
        const __bf16 hi = (__bf16)v;
        qhi[kc].h[e] = hi;
        qlo[kc].h[e] = (__bf16)(v - (float)hi);
      }
    }
    if (DR) {
      const __bf16* q = reinterpret_cast<const __bf16*>(a.q_rope) + ((int64_t)b * H + h_col) * d_r;
      qr.u = (8 * r < d_r) ? ld16(q + 8 * r) : zero4();
    }
  }
  // Selection fragments: sel[par] picks channel 16*db + col out of the 32
  // channels of half db/2 (par = db % 2).
  Frag sel[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sel[par].h[e] = (__bf16)((r == 2 * par + col / 8 && e == col % 8) ? 1.f : 0.f);

  // ---- streaming loop -------------------------------------------------------
  const CacheGeom cg{G, d_r, a.capacity, a.num_blocks, a.max_blocks, a.block_table};
  const __bf16* vc = reinterpret_cast<const __bf16*>(a.v_cache);
  const __bf16* sc = reinterpret_cast<const __bf16*>(GQA ? a.kr_cache : a.v_cache);
  const __bf16* kc_ptr = reinterpret_cast<const __bf16*>(a.kr_cache);

  f32x4 acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  auto load_tile = [&](Tile<GQA, DR>& T, int t0) {
    int blk = 0;
    if (PAGED) blk = page_of(cg, b, t0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int tok = t0 + 16 * st + col;
      const bool ok = active && tok < t_end && (!PAGED || blk >= 0);
      int64_t vrow, krow = 0;
      if (PAGED) {
        vrow = (((int64_t)blk * G + g) * kBlock + (tok % kBlock)) * kD;
        if (DR) krow = ((int64_t)blk * kBlock + (tok % kBlock)) * d_r;
      } else {
        vrow = (((int64_t)b * G + g) * a.capacity + tok) * kD;
        if (DR) krow = ((int64_t)b * a.capacity + tok) * d_r;
      }
      T.sa[st][0].u = ok ? ld16(sc + vrow + 8 * r) : zero4();
      T.sa[st][1].u = ok ? ld16(sc + vrow + 32 + 8 * r) : zero4();
      if constexpr (GQA) {
        T.vb[st][0].u = ok ? ld16(vc + vrow + 8 * r) : zero4();
        T.vb[st][1].u = ok ? ld16(vc + vrow + 32 + 8 * r) : zero4();
      }
      if constexpr (DR) T.kr[st].u = (ok && 8 * r < d_r) ? ld16(kc_ptr + krow + 8 * r) : zero4();
    }
  };

  auto process_tile = [&](const Tile<GQA, DR>& T, int t0) {
    f32x4 s[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      c = mma(T.sa[st][0], qhi[0], c);
      c = mma(T.sa[st][1], qhi[1], c);
      if (!GQA) {
        c = mma(T.sa[st][0], qlo[0], c);
        c = mma(T.sa[st][1], qlo[1], c);
      }
      if constexpr (DR) {
        const f32x4 cr = mma(T.kr[st], qr, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = fmaf(cr[i], sl2, c[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (t0 + 16 * st + 4 * r + i >= t_end) c[i] = -INFINITY;
      s[st] = c;
    }
    // online softmax for this lane's head (column)
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[st][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[st][i] = exp2f(s[st][i] - m_new);
        psum += s[st][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < 4; ++db) acc_o[db] *= alpha;
    }
    // P.V over two 32-token pairs of sub-tiles
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      Frag pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb.h[i] = (__bf16)s[2 * pr][i];
        pb.h[4 + i] = (__bf16)s[2 * pr + 1][i];
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        f32x4 ca, cb;
        if constexpr (GQA) {
          ca = mma(T.vb[2 * pr][db >> 1], sel[db & 1], f32x4{0.f, 0.f, 0.f, 0.f});
          cb = mma(T.vb[2 * pr + 1][db >> 1], sel[db & 1], f32x4{0.f, 0.f, 0.f, 0.f});
        } else {
          ca = mma(T.sa[2 * pr][db >> 1], sel[db & 1], f32x4{0.f, 0.f, 0.f, 0.f});
          cb = mma(T.sa[2 * pr + 1][db >> 1], sel[db & 1], f32x4{0.f, 0.f, 0.f, 0.f});
        }
        Frag vt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vt.h[i] = (__bf16)ca[i];
          vt.h[4 + i] = (__bf16)cb[i];
        }
        acc_o[db] = mma(vt, pb, acc_o[db]);
      }
    }
  };

  if (active && t_begin < t_end) {
    Tile<GQA, DR> A, B;
    load_tile(A, t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += 2 * kTile) {
      const int t1 = t0 + kTile;
      if (t1 < t_end) load_tile(B, t1);
      process_tile(A, t0);
      if (t1 >= t_end) break;
      if (t1 + kTile < t_end) load_tile(A, t1 + kTile);
      process_tile(B, t1);
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __bf16* out = reinterpret_cast<__bf16*>(a.out);
  const bool writer = active && col < HPG;  // first copy of each head's column
  if (n_parts <= 1) {
    if (writer) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out[((int64_t)b * H + h_col) * kD + 16 * db + 4 * r + i] = (__bf16)(acc_o[db][i] * inv);
    }
    return;
  }
  if (writer) {
    const int64_t slot = ((int64_t)b * H + h_col) * a.n_split + split;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.ws_o[slot * kD + 16 * db + 4 * r + i] = acc_o[db][i];
    if (r == 0) {
      a.ws_ml[2 * slot] = m_run;
      a.ws_ml[2 * slot + 1] = l_run;
    }
  }
  int32_t* counter = a.counters + (int64_t)b * gridDim.y + chunk;
  if (!arrive_last(counter, n_parts)) return;
  const int heads_here = min(4, G - chunk * 4) * HPG;
  for (int idx = tid; idx < heads_here * kD; idx += 256) {
    const int h = chunk * 4 * HPG + idx / kD, d = idx % kD;
    const int64_t slot0 = ((int64_t)b * H + h) * a.n_split;
    out[((int64_t)b * H + h) * kD + d] = (__bf16)merge_partials(a.ws_o, a.ws_ml, slot0, n_parts, d);
  }
  if (tid == 0) reset_counter(counter);
}

template <int HPG, bool DR, bool GQA>
hipError_t mfma_paged(const DecodeLaunch& a, hipStream_t s) {
  const dim3 grid(a.n_split, (a.G + 3) / 4, a.B);
  if (a.paged)
    decode_mfma_kernel<HPG, true, DR, GQA><<<grid, 256, 0, s>>>(a);
  else
    decode_mfma_kernel<HPG, false, DR, GQA><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int HPG, bool GQA>
hipError_t mfma_dr(const DecodeLaunch& a, hipStream_t s) {
  if (!GQA && a.d_r > 0) return mfma_paged<HPG, true, false>(a, s);
  return mfma_paged<HPG, false, GQA>(a, s);
}

template <bool GQA>
hipError_t mfma_dispatch(const DecodeLaunch& a, hipStream_t s) {
  switch (a.H / a.G) {
    case 1: return mfma_dr<1, GQA>(a, s);
    case 2: return mfma_dr<2, GQA>(a, s);
    default: return mfma_dr<4, GQA>(a, s);
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t s) { return mfma_dispatch<false>(a, s); }
hipError_t launch_gqa_mfma(const DecodeLaunch& a, hipStream_t s) { return mfma_dispatch<true>(a, s); }

}  // namespace gva
