// Cache append and query rotation kernels.
//
// Appending follows the decode loop of the GQA tutorial page ("GQA 分组查询
// 注意力", sections on cache growth and on RoPE and the KV cache): each new
// token writes its state once at the next position. For GVA that state is the
// grouped value rows (never rotated) and the single positional key after RoPE
// (GVA digest, 方法 / GVA 核心流程; review blog, Decoupled RoPE).
#include "gva_device.hpp"
#include "launch.hpp"

namespace gva {
namespace {

constexpr int kAppendTok = 64;  // tokens per append workgroup

template <typename T, bool PAGED>
__global__ __launch_bounds__(256) void append_kernel(AppendLaunch a, CacheGeom c, int cap_tokens,
                                                     bool advance_here) {
  const int b = blockIdx.y;
  const int t_lo = blockIdx.x * kAppendTok;
  const int t_hi = min(a.n_new, t_lo + kAppendTok);
  const int pos0 = max(a.seq_lens[b], 0);

  // Values: copy 16-byte pieces of each row unchanged.
  constexpr int kVecPerRow = kD * (int)sizeof(T) / 16;
  const uint4* vsrc = reinterpret_cast<const uint4*>(a.v_new);
  uint4* vdst = reinterpret_cast<uint4*>(a.v_cache);
  const int n_rows = a.G * (t_hi - t_lo);
  for (int i = threadIdx.x; i < n_rows * kVecPerRow; i += blockDim.x) {
    const int row = i / kVecPerRow, piece = i % kVecPerRow;
    const int g = row / (t_hi - t_lo), t = t_lo + row % (t_hi - t_lo);
    const int pos = pos0 + t;
    if (pos >= cap_tokens) continue;
    const int64_t dst = v_row<PAGED>(c, b, g, pos);
    if (dst < 0) continue;
    const int64_t src = (((int64_t)b * a.G + g) * a.n_new + t) * kD;
    vdst[(dst * (int64_t)sizeof(T)) / 16 + piece] = vsrc[(src * (int64_t)sizeof(T)) / 16 + piece];
  }

  // Positional keys: rotate pair i of token t by its absolute position.
  if (a.d_r > 0) {
    const T* ksrc = reinterpret_cast<const T*>(a.kr_new);
    T* kdst = reinterpret_cast<T*>(a.kr_cache);
    const int half = a.d_r / 2;
    for (int i = threadIdx.x; i < (t_hi - t_lo) * half; i += blockDim.x) {
      const int t = t_lo + i / half, p = i % half;
      const int pos = pos0 + t;
      if (pos >= cap_tokens) continue;
      const int64_t dst = kr_row<PAGED>(c, b, pos);
      if (dst < 0) continue;
      const int64_t src = ((int64_t)b * a.n_new + t) * a.d_r + 2 * p;
      rope_store<T>(to_f32(ksrc[src]), to_f32(ksrc[src + 1]), (double)pos, a.rope.theta[p], kdst[dst + 2 * p],
                    kdst[dst + 2 * p + 1]);
    }
  }

  if (advance_here) {
    __syncthreads();  // every thread has read seq_lens[b]
    if (threadIdx.x == 0) a.seq_lens[b] = min(pos0 + a.n_new, cap_tokens);
  }
}

__global__ void advance_kernel(int32_t* seq_lens, int B, int n_new, int cap_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) seq_lens[b] = min(max(seq_lens[b], 0) + n_new, cap_tokens);
}

// q[b][j] (j < nq) is the query of the token at position seq_lens[b] - nq + j
// (the last nq cached tokens; nq = 1: the newest one).
template <typename T>
__global__ __launch_bounds__(256) void rope_query_kernel(RopeQueryLaunch a) {
  const int b = blockIdx.x;
  const int half = a.d_r / 2;
  const int len = a.seq_lens[b];
  const T* src = reinterpret_cast<const T*>(a.q_in);
  T* dst = reinterpret_cast<T*>(a.q_out);
  for (int i = threadIdx.x; i < a.nq * a.H * half; i += blockDim.x) {
    const int j = i / (a.H * half), h = (i / half) % a.H, p = i % half;
    const double pos = (double)max(len - a.nq + j, 0);
    const int64_t off = (((int64_t)b * a.nq + j) * a.H + h) * a.d_r + 2 * p;
    T y0, y1;  // (the rotation may be in place)
    rope_store<T>(to_f32(src[off]), to_f32(src[off + 1]), pos, a.rope.theta[p], y0, y1);
    dst[off] = y0;
    dst[off + 1] = y1;
  }
}

template <typename T, bool PAGED>
hipError_t append_impl(const AppendLaunch& a, hipStream_t s) {
  CacheGeom c{a.G, a.d_r, a.capacity, a.num_blocks, a.max_blocks, a.block_table};
  const int cap_tokens = PAGED ? a.max_blocks * kBlock : a.capacity;
  const int chunks = (a.n_new + kAppendTok - 1) / kAppendTok;
  const bool one = chunks == 1;
  append_kernel<T, PAGED><<<dim3(chunks, a.B), 256, 0, s>>>(a, c, cap_tokens, one);
  if (!one) advance_kernel<<<(a.B + 255) / 256, 256, 0, s>>>(a.seq_lens, a.B, a.n_new, cap_tokens);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendLaunch& a, hipStream_t s) {
  if (a.bf16) return a.paged ? append_impl<__bf16, true>(a, s) : append_impl<__bf16, false>(a, s);
  return a.paged ? append_impl<float, true>(a, s) : append_impl<float, false>(a, s);
}

hipError_t launch_rope_query(const RopeQueryLaunch& a, hipStream_t s) {
  if (a.d_r == 0) return hipSuccess;
  if (a.bf16)
    rope_query_kernel<__bf16><<<a.B, 256, 0, s>>>(a);
  else
    rope_query_kernel<float><<<a.B, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace gva
