// GVA decode on the vector ALUs (fp32 arithmetic throughout), with the split-K
// log-sum-exp combine done by the last workgroup of each (sequence, group).
//
// This path serves fp32 caches, where every product must stay in binary32,
// and is the simple cross-check of the matrix-core path for bf16.
//
// Per workgroup: one sequence b, one value group g, one split-K partition.
// Prologue: absorb the reconstruction maps into the queries of the group's
// heads, q'_h = M_h q_nope,h (GVA digest, 方法: Q' = Q M^T; explainer, 正式
// 方案), pre-scaled by scale*log2(e) so the softmax runs on exp2.
// Loop over 64-token tiles: stage V_g and k_r rows in LDS, score every head
// (q'_h . V + q_rope,h . k_r), online softmax, accumulate p . V from the same
// staged tile. Content keys are never formed.
#include "gva_device.hpp"
#include "launch.hpp"

namespace gva {
namespace {

template <typename T, int HPG, bool PAGED>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeLaunch a) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int H = a.H, d_r = a.d_r;
  const int n = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int n_parts = (n + a.split - 1) / a.split;  // partitions holding tokens
  if (split >= max(n_parts, 1)) return;              // uniform per workgroup
  const int t_begin = split * a.split;
  const int t_end = min(n, t_begin + a.split);

  __shared__ float qs[4][kD];
  __shared__ float qrs[4][32];
  __shared__ float Vs[kTile][kD + 1];
  __shared__ float Ks[kTile][33];
  __shared__ float Ps[4][kTile];

  const CacheGeom c{a.G, d_r, a.capacity, a.num_blocks, a.max_blocks, a.block_table};
  const T* vc = reinterpret_cast<const T*>(a.v_cache);
  const T* kc = reinterpret_cast<const T*>(a.kr_cache);
  const float sl2 = a.scale * kLog2e;
  const int h = g * HPG + w;  // head of this wave (valid when w < HPG)

  // Absorption prologue: thread (w, lane) forms q'[w][d = lane]. With M ==
  // nullptr the maps are folded into the query projection and q_nope already
  // holds q'.
  if (w < HPG) {
    const T* qn = reinterpret_cast<const T*>(a.q_nope) + ((int64_t)b * H + h) * kD;
    float acc = 0.f;
    if (a.M) {
      const T* Mh = reinterpret_cast<const T*>(a.M) + ((int64_t)h * kD + lane) * kD;
      for (int j = 0; j < kD; ++j) acc = fmaf(to_f32(Mh[j]), to_f32(qn[j]), acc);
    } else {
      acc = to_f32(qn[lane]);
    }
    qs[w][lane] = acc * sl2;
    if (lane < d_r)
      qrs[w][lane] = to_f32(reinterpret_cast<const T*>(a.q_rope)[((int64_t)b * H + h) * d_r + lane]) * sl2;
  }

  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
    const int nt = min(kTile, t_end - t0);
    __syncthreads();  // previous tile fully consumed (and prologue visible)
    for (int i = tid; i < kTile * kD; i += 256) {
      const int tt = i / kD, d = i % kD;
      float v = 0.f;
      if (tt < nt) {
        const int64_t r = v_row<PAGED>(c, b, g, t0 + tt);
        if (r >= 0) v = to_f32(vc[r + d]);
      }
      Vs[tt][d] = v;
    }
    for (int i = tid; i < kTile * d_r; i += 256) {
      const int tt = i / d_r, d = i % d_r;
      float v = 0.f;
      if (tt < nt) {
        const int64_t r = kr_row<PAGED>(c, b, t0 + tt);
        if (r >= 0) v = to_f32(kc[r + d]);
      }
      Ks[tt][d] = v;
    }
    __syncthreads();

    // Scores: thread (w, lane) = (head, token).
    float s = -INFINITY;
    if (w < HPG && lane < nt) {
      float acc = 0.f;
      for (int d = 0; d < kD; ++d) acc = fmaf(qs[w][d], Vs[lane][d], acc);
      for (int d = 0; d < d_r; ++d) acc = fmaf(qrs[w][d], Ks[lane][d], acc);
      s = acc;
    }
    const float m_new = fmaxf(m, wave_max(s));
    const float alpha = exp2f(m - m_new);  // 0 on the first tile
    const float p = (lane < nt) ? exp2f(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    m = m_new;
    Ps[w][lane] = p;
    __syncthreads();

    // p . V: thread (w, lane) = (head, channel).
    if (w < HPG) {
      float acc = 0.f;
      for (int tt = 0; tt < nt; ++tt) acc = fmaf(Ps[w][tt], Vs[tt][lane], acc);
      o = o * alpha + acc;
    }
  }

  T* out = reinterpret_cast<T*>(a.out);
  if (n_parts <= 1) {
    if (w < HPG) out[((int64_t)b * H + h) * kD + lane] = from_f32<T>(l > 0.f ? o / l : 0.f);
    return;
  }
  const int64_t slot0 = ((int64_t)b * H + h) * a.n_split;
  if (w < HPG) {
    st_dev(a.ws_o + (slot0 + split) * kD + lane, o);
    if (lane == 0) {
      st_dev_ml(a.ws_ml + 2 * (slot0 + split), m, l);
    }
  }
  int32_t* counter = a.counters + ((int64_t)b * a.G + g) * kCounterStride;
  if (!arrive_last(counter, n_parts)) return;
  if (w < HPG)
    out[((int64_t)b * H + h) * kD + lane] =
        from_f32<T>(merge_partials(a.ws_o, a.ws_ml, slot0, n_parts, lane));
  if (tid == 0) reset_counter(counter);
}

template <typename T, int HPG>
hipError_t valu_impl(const DecodeLaunch& a, hipStream_t s) {
  const dim3 grid(a.n_split, a.G, a.B);
  if (a.paged)
    decode_valu_kernel<T, HPG, true><<<grid, 256, 0, s>>>(a);
  else
    decode_valu_kernel<T, HPG, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t valu_dispatch(const DecodeLaunch& a, hipStream_t s) {
  switch (a.H / a.G) {
    case 1: return valu_impl<T, 1>(a, s);
    case 2: return valu_impl<T, 2>(a, s);
    default: return valu_impl<T, 4>(a, s);
  }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeLaunch& a, hipStream_t s) {
  return a.bf16 ? valu_dispatch<__bf16>(a, s) : valu_dispatch<float>(a, s);
}

}  // namespace gva
