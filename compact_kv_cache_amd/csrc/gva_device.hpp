// Device-side helpers shared by the GVA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gva {

constexpr int kD = 64;          // d_n = d_v built here
constexpr int kTile = 64;       // tokens per tile == paged block size
constexpr int kBlock = 64;      // paged block size (tokens)
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Scalar loads / stores in the call dtype (float or __bf16), as float.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Correctly rounded (to nearest, ties to even) conversion of a double.
// For bf16: round to odd into binary32 first (truncate, then set the last bit
// when inexact), which has 16 more fraction bits than bf16, then round to
// nearest even; the composition equals a single correct rounding.
template <typename T> __device__ __forceinline__ T from_f64(double x);
template <> __device__ __forceinline__ float from_f64<float>(double x) { return (float)x; }
template <> __device__ __forceinline__ __bf16 from_f64<__bf16>(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x && !__builtin_isnan(x)) f = __uint_as_float(__float_as_uint(f) | 1u);
  return (__bf16)f;
}

// ---------------------------------------------------------------------------
// Sine and cosine of a >= 0 in double precision, for the RoPE angles
// (a = pos * theta_i <= 2^32). Cody-Waite reduction by pi/2 split into two
// doubles (k * hi is exact in the fused multiply-add, and the dropped third
// part times k stays below 1e-28), so r = a - k*pi/2 lies in [-pi/4, pi/4]
// up to rounding; then the Taylor series of sin to r^15 and cos to r^16,
// whose first omitted terms are below 5e-17 there; then the quadrant k mod 4.
// Straight-line code: no large-argument path, no table.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void sincos_angle(double a, double& s, double& c) {
  constexpr double kTwoOverPi = 0.6366197723675814;
  constexpr double kPiO2Hi = 1.5707963267948966;     // pi/2 rounded to double
  constexpr double kPiO2Mid = 6.123233995736766e-17;  // pi/2 - kPiO2Hi, rounded
  const double k = rint(a * kTwoOverPi);
  const double r = fma(-k, kPiO2Mid, fma(-k, kPiO2Hi, a));
  const double r2 = r * r;
  // coefficients 1/n!
  double ps = -7.647163731819816e-13;              // -1/15!
  ps = fma(ps, r2, 1.6059043836821613e-10);        //  1/13!
  ps = fma(ps, r2, -2.505210838544172e-08);        // -1/11!
  ps = fma(ps, r2, 2.7557319223985893e-06);        //  1/9!
  ps = fma(ps, r2, -0.0001984126984126984);        // -1/7!
  ps = fma(ps, r2, 0.008333333333333333);          //  1/5!
  ps = fma(ps, r2, -0.16666666666666666);          // -1/3!
  const double sr = fma(r * r2, ps, r);
  double pc = 4.779477332387385e-14;               //  1/16!
  pc = fma(pc, r2, -1.1470745597729725e-11);       // -1/14!
  pc = fma(pc, r2, 2.08767569878681e-09);          //  1/12!
  pc = fma(pc, r2, -2.755731922398589e-07);        // -1/10!
  pc = fma(pc, r2, 2.48015873015873e-05);          //  1/8!
  pc = fma(pc, r2, -0.001388888888888889);         // -1/6!
  pc = fma(pc, r2, 0.041666666666666664);          //  1/4!
  pc = fma(pc, r2, -0.5);                          // -1/2!
  const double cr = fma(r2, pc, 1.0);
  const int q = (int)((long long)k & 3);
  const double s0 = (q & 1) ? cr : sr;
  const double c0 = (q & 1) ? sr : cr;
  s = (q & 2) ? -s0 : s0;
  c = ((q + 1) & 2) ? -c0 : c0;
}

// RoPE on one channel pair (2i, 2i+1) at position pos: counter-clockwise turn
// by pos * theta_i (theta_i = base^(-2i/d_r), precomputed on the host), in
// double precision.
__device__ __forceinline__ void rope_pair(double x0, double x1, double pos, double theta,
                                          double& y0, double& y1) {
  double s, c;
  sincos_angle(pos * theta, s, c);
  y0 = x0 * c - x1 * s;
  y1 = x0 * s + x1 * c;
}
// Rotate a stored pair and round it to the storage type T.
template <typename T>
__device__ __forceinline__ void rope_store(float x0, float x1, double pos, double theta, T& y0, T& y1) {
  double a, b;
  rope_pair((double)x0, (double)x1, pos, theta, a, b);
  y0 = from_f64<T>(a);
  y1 = from_f64<T>(b);
}

// ---------------------------------------------------------------------------
// Wave-wide reductions (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Cache addressing. Offsets are element offsets (64-bit).
// ---------------------------------------------------------------------------
struct CacheGeom {
  int G, d_r, capacity, num_blocks, max_blocks;
  const int32_t* block_table;  // null = contiguous
};

// Wave-uniform read of memory that no kernel writes while it runs (block
// tables): the load goes through the scalar data cache. Through a plain
// pointer the compiler must assume that a store earlier in the kernel (the
// fused step's appended rows) may have changed the value, and issues a vector
// load whose result the wave then waits for in full; the constant address
// space states that nothing does.
__device__ __forceinline__ int32_t ld_table(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// Pool block of token t of sequence b, or -1 if the table entry is invalid.
__device__ __forceinline__ int page_of(const CacheGeom& c, int b, int t) {
  const int j = t / kBlock;
  if (j >= c.max_blocks) return -1;
  const int blk = c.block_table[(size_t)b * c.max_blocks + j];
  return (blk >= 0 && blk < c.num_blocks) ? blk : -1;
}

// Offset of row (b, g, t) in a [.., G, .., d] value-like cache (d = kD); -1 if
// the row is outside the cache.
template <bool PAGED>
__device__ __forceinline__ int64_t v_row(const CacheGeom& c, int b, int g, int t) {
  if (PAGED) {
    const int blk = page_of(c, b, t);
    if (blk < 0) return -1;
    return (((int64_t)blk * c.G + g) * kBlock + (t % kBlock)) * kD;
  } else {
    if (t >= c.capacity) return -1;
    return (((int64_t)b * c.G + g) * c.capacity + t) * kD;
  }
}

template <bool PAGED>
__device__ __forceinline__ int64_t kr_row(const CacheGeom& c, int b, int t) {
  if (PAGED) {
    const int blk = page_of(c, b, t);
    if (blk < 0) return -1;
    return ((int64_t)blk * kBlock + (t % kBlock)) * c.d_r;
  } else {
    if (t >= c.capacity) return -1;
    return ((int64_t)b * c.capacity + t) * c.d_r;
  }
}

// ---------------------------------------------------------------------------
// Split-K hand-off between workgroups of one (sequence, group chunk).
// Partials are written and read with device-coherent accesses (relaxed
// agent-scope atomics: the store writes through the compute unit's and the
// XCD's caches to the memory side, the load misses in them), so no cache-wide
// write-back or invalidate is needed. Each workgroup waits until its own
// partial stores are acknowledged (all wait counters at zero, then a barrier
// for every wave), then bumps the arrival counter; the workgroup that arrives
// last has therefore seen every other workgroup's stores reach the memory side
// before its own atomic, reads the partials after the atomic's result, merges
// them and resets the counter to zero for the next call. This rests on the
// hardware's acknowledgement rule rather than on C++ ordering (relaxed atomics
// order nothing); an acq_rel arrival would add an L2 write-back (about 0.3 us)
// to every workgroup's path.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A partial's (m, l) pair (adjacent floats, 8-byte aligned) as one 8-byte
// device-coherent store or load: one memory instruction instead of two.
__device__ __forceinline__ void st_dev_ml(float* p, float m, float l) {
  const uint64_t v = (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(l) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_ml(const float* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Must be reached by every thread of the workgroup; returns the same value in
// all of them. `arrivals`: partials this workgroup contributes (its count on
// the counter).
__device__ __forceinline__ bool arrive_last(int32_t* counter, int n_parts, int arrivals = 1) {
  __shared__ int s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();                // ... and so are every other wave's
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(counter, arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old + arrivals == n_parts);
  }
  __syncthreads();
  return s_last != 0;
}

__device__ __forceinline__ void reset_counter(int32_t* counter) {
  __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Log-sum-exp merge of n_parts partials of one head for channel d:
// out = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s, M = max_s m_s, with
// m_s in log2 units and o_s unnormalized. Partials are fetched K at a time
// with all loads in flight together, merged online across batches of K = 16
// (48 loads, within the 63 a wave can count), so a long split pays fewer
// round trips; up to 8 partials take one exact batch (merge_partials_n).
template <int K>
__device__ __forceinline__ float merge_partials_k(const float* o, const float* ml, int64_t slot0,
                                                  int n_parts, int d) {
  float M = -INFINITY, num = 0.f, den = 0.f;
  for (int base = 0; base < n_parts; base += K) {
    float mv[K], lv[K], ov[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int64_t s = slot0 + min(base + i, n_parts - 1);
      mv[i] = ld_dev(ml + 2 * s);
      lv[i] = ld_dev(ml + 2 * s + 1);
      ov[i] = ld_dev(o + s * kD + d);
    }
    float bm = M;
#pragma unroll
    for (int i = 0; i < K; ++i)
      if (base + i < n_parts) bm = fmaxf(bm, mv[i]);
    const float rescale = exp2f(M - bm);  // 0 before the first batch
    num *= rescale;
    den *= rescale;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      if (base + i < n_parts) {
        const float w = exp2f(mv[i] - bm);
        num = fmaf(w, ov[i], num);
        den = fmaf(w, lv[i], den);
      }
    }
    M = bm;
  }
  return den > 0.f ? num / den : 0.f;
}

// The same merge for exactly N partials, one batch: N loads of o and N of the
// (m, l) pairs. Every vector memory instruction occupies the compute unit's
// address unit for the same time whatever its width, so the merge that ends
// the split-K hand-off issues only the loads it needs. Same arithmetic and
// order as merge_partials_k, bit for bit.
template <int N>
__device__ __forceinline__ float merge_partials_n(const float* o, const float* ml, int64_t slot0, int d) {
  float mv[N], lv[N], ov[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint64_t e = ld_dev_ml(ml + 2 * (slot0 + i));
    mv[i] = __uint_as_float((uint32_t)e);
    lv[i] = __uint_as_float((uint32_t)(e >> 32));
    ov[i] = ld_dev(o + (slot0 + i) * kD + d);
  }
  float bm = -INFINITY;
#pragma unroll
  for (int i = 0; i < N; ++i) bm = fmaxf(bm, mv[i]);
  const float rescale = exp2f(-INFINITY - bm);  // 0, or NaN when every partial is empty
  float num = 0.f * rescale, den = 0.f * rescale;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float w = exp2f(mv[i] - bm);
    num = fmaf(w, ov[i], num);
    den = fmaf(w, lv[i], den);
  }
  return den > 0.f ? num / den : 0.f;
}

__device__ __forceinline__ float merge_partials(const float* o, const float* ml, int64_t slot0,
                                                int n_parts, int d) {
  switch (n_parts) {
    case 1: return merge_partials_n<1>(o, ml, slot0, d);
    case 2: return merge_partials_n<2>(o, ml, slot0, d);
    case 3: return merge_partials_n<3>(o, ml, slot0, d);
    case 4: return merge_partials_n<4>(o, ml, slot0, d);
    case 5: return merge_partials_n<5>(o, ml, slot0, d);
    case 6: return merge_partials_n<6>(o, ml, slot0, d);
    case 7: return merge_partials_n<7>(o, ml, slot0, d);
    case 8: return merge_partials_n<8>(o, ml, slot0, d);
    default: return merge_partials_k<16>(o, ml, slot0, n_parts, d);
  }
}

}  // namespace gva
