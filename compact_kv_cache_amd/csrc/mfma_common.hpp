// Matrix-core building blocks shared by the decode and prefill kernels
// (gfx950, wave64): operand fragments of v_mfma_f32_16x16x32_bf16, row
// reductions with the row-swap permutes, the staged-row swizzle and buffer
// resource constants.
#pragma once
#include <hip/hip_runtime.h>

namespace gva {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

union Frag {
  bf16x8 v;
  u32x4 u;
  __bf16 h[8];
};

__device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// Max / sum over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48) with the gfx950 row-swap permutes: v_permlane16_swap pairs rows 0-1
// and 2-3, v_permlane32_swap the two halves; no LDS round trip. Every lane
// combines the same two operands in the same order, so all four rows end
// with the same value.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// 16-byte load; `base` is wave-uniform, `off` a per-lane element offset.
__device__ __forceinline__ u32x4 ld16(const __bf16* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
// Same, for data read exactly once (does not displace resident lines).
__device__ __forceinline__ u32x4 ld16_stream(const __bf16* base, int off) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
}

constexpr f32x4 kZero4 = {0.f, 0.f, 0.f, 0.f};
// Buffer resource word 3 for raw (untyped, unswizzled) loads: 32-bit data
// format, the value the gfx9-family matrix-core libraries use.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;  // cache-policy bit: non-temporal (streamed once)
// 16-byte chunk permutation inside a 128-byte staged row. Reading one chunk
// position of 16 consecutive rows then touches 16 distinct bank groups.
__device__ __forceinline__ int stage_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

}  // namespace gva
