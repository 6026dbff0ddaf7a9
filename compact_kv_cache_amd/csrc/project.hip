// Folding the reconstruction maps into the query projection, and the query
// projection itself (GVA digest, section 与现有产品 / 工作流的接口: at
// inference the reconstruction matrix can be folded into the query
// projection, so content keys are never formed). With the fold
// W'_h = M_h W_q,nope,h the absorbed query is one product, q'_h = W'_h x,
// and the decode needs neither M nor its prologue GEMV.
#include "gva_device.hpp"
#include "launch.hpp"

namespace gva {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One thread per output element (h, v, m), fp32 accumulation over d_n. Runs
// once per model; written for clarity.
template <typename T>
__global__ __launch_bounds__(256) void fold_kernel(FoldLaunch a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.H * a.d_v * a.d_model;
  if (idx >= total) return;
  const int m = (int)(idx % a.d_model);
  const int64_t hv = idx / a.d_model;
  const int h = (int)(hv / a.d_v);
  const T* Mr = reinterpret_cast<const T*>(a.M) + hv * a.d_n;
  const T* W = reinterpret_cast<const T*>(a.wq) + (int64_t)h * a.d_n * a.d_model + m;
  float acc = 0.f;
  for (int n = 0; n < a.d_n; ++n) acc = fmaf(to_f32(Mr[n]), to_f32(W[(int64_t)n * a.d_model]), acc);
  reinterpret_cast<T*>(a.w_fold)[idx] = from_f32<T>(acc);
}

// Row r of the stacked projection [w_fold; w_rope] and where its result goes.
__device__ __forceinline__ const __bf16* proj_row(const ProjectLaunch& a, int r) {
  const int r1 = a.H * a.d_v;
  return r < r1 ? reinterpret_cast<const __bf16*>(a.w_fold) + (int64_t)r * a.d_model
                : reinterpret_cast<const __bf16*>(a.w_rope) + (int64_t)(r - r1) * a.d_model;
}

// bf16: out^T[row][b] = sum_k W[row][k] x[b][k] on v_mfma_f32_16x16x32_bf16
// (A = 16 rows of W, B = x^T for 16 batch rows). Workgroup = 16 rows x 16
// batch rows; its 4 waves take a quarter of d_model each and add their
// accumulators in LDS. d_model is a multiple of 128.
__global__ __launch_bounds__(256) void project_mfma_kernel(ProjectLaunch a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, r = lane >> 4;
  const int rows = a.H * (a.d_v + a.d_r);
  const int r0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
  const int row = min(r0 + col, rows - 1);  // rows past the end re-read the last one
  const int bb = min(b0 + col, a.B - 1);
  const __bf16* wr = proj_row(a, row);
  const __bf16* xr = reinterpret_cast<const __bf16*>(a.x) + (int64_t)bb * a.d_model;
  const int kq = a.d_model / 4;  // this wave's share of the contraction
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = w * kq; k0 < (w + 1) * kq; k0 += 32) {
    union { bf16x8 v; u32x4 u; } fa, fb;
    fa.u = *reinterpret_cast<const u32x4*>(wr + k0 + 8 * r);
    fb.u = *reinterpret_cast<const u32x4*>(xr + k0 + 8 * r);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa.v, fb.v, acc, 0, 0, 0);
  }
  __shared__ float part[4][16][16];  // [wave][row][batch]
#pragma unroll
  for (int i = 0; i < 4; ++i) part[w][4 * r + i][col] = acc[i];
  __syncthreads();
  // thread t < 256 -> (row 4r'+i..., batch): one output each
  const int orow = threadIdx.x >> 4, ob = threadIdx.x & 15;
  const int gr = r0 + orow, gb = b0 + ob;
  if (gr < rows && gb < a.B) {
    const float v = part[0][orow][ob] + part[1][orow][ob] + part[2][orow][ob] + part[3][orow][ob];
    const int r1 = a.H * a.d_v;
    if (gr < r1)
      reinterpret_cast<__bf16*>(a.q_abs)[(int64_t)gb * r1 + gr] = (__bf16)v;
    else
      reinterpret_cast<__bf16*>(a.q_rope)[(int64_t)gb * a.H * a.d_r + (gr - r1)] = (__bf16)v;
  }
}

// fp32: one thread per (batch row, output row), fp32 dot product.
__global__ __launch_bounds__(256) void project_f32_kernel(ProjectLaunch a) {
  const int rows = a.H * (a.d_v + a.d_r);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * a.B) return;
  const int gr = (int)(idx % rows), gb = (int)(idx / rows);
  const int r1 = a.H * a.d_v;
  const float* wr = gr < r1 ? reinterpret_cast<const float*>(a.w_fold) + (int64_t)gr * a.d_model
                            : reinterpret_cast<const float*>(a.w_rope) + (int64_t)(gr - r1) * a.d_model;
  const float* xr = reinterpret_cast<const float*>(a.x) + (int64_t)gb * a.d_model;
  float acc = 0.f;
  for (int k = 0; k < a.d_model; ++k) acc = fmaf(wr[k], xr[k], acc);
  if (gr < r1)
    reinterpret_cast<float*>(a.q_abs)[(int64_t)gb * r1 + gr] = acc;
  else
    reinterpret_cast<float*>(a.q_rope)[(int64_t)gb * a.H * a.d_r + (gr - r1)] = acc;
}

}  // namespace

hipError_t launch_fold(const FoldLaunch& a, hipStream_t s) {
  const int64_t total = (int64_t)a.H * a.d_v * a.d_model;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (a.bf16)
    fold_kernel<__bf16><<<grid, 256, 0, s>>>(a);
  else
    fold_kernel<float><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_project(const ProjectLaunch& a, hipStream_t s) {
  const int rows = a.H * (a.d_v + a.d_r);
  if (a.bf16) {
    const dim3 grid((rows + 15) / 16, (a.B + 15) / 16);
    project_mfma_kernel<<<grid, 256, 0, s>>>(a);
  } else {
    const int64_t total = (int64_t)rows * a.B;
    project_f32_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace gva
