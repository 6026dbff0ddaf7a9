// Host-side launcher declarations shared between the kernel sources and the
// C ABI layer. Arguments have been validated before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gva {

struct AppendLaunch {
  int B, G, d_r, n_new, capacity, num_blocks, max_blocks;
  bool paged, bf16;
  const void* v_new;
  const void* kr_new;
  int32_t* seq_lens;
  void* v_cache;
  void* kr_cache;
  const int32_t* block_table;
  double rope_base;
};

struct RopeQueryLaunch {
  int B, H, d_r;
  bool bf16;
  const void* q_in;
  void* q_out;
  const int32_t* seq_lens;
  double rope_base;
};

// Decode problem, shared by the GVA kernels and the GQA comparison kernel.
struct DecodeLaunch {
  int B, H, G, d_r, capacity, max_seq_len, num_blocks, max_blocks;
  int split, n_split;  // split-K partition length and count
  bool paged, bf16;
  const void* q_nope;  // GQA: q
  const void* q_rope;
  const void* M;
  const void* v_cache;
  const void* kr_cache;  // GQA: k_cache
  const int32_t* seq_lens;
  const int32_t* block_table;
  float scale;
  void* out;
  // Workspace (split-K only): int32 arrival counters [B*G] (zero before the
  // first call, left zero by every call), then float partials
  // o [B*H*n_split*64] and (m, l) [B*H*n_split*2].
  int32_t* counters;
  float* ws_o;
  float* ws_ml;
};

// Workspace layout helpers (bytes).
inline size_t ws_counter_bytes(int B, int G) { return (((size_t)B * G * 4) + 255) / 256 * 256; }
inline size_t ws_total_bytes(int B, int H, int G, int n_split) {
  if (n_split <= 1) return 0;
  return ws_counter_bytes(B, G) + (size_t)B * H * n_split * (64 + 2) * sizeof(float);
}

hipError_t launch_append(const AppendLaunch& a, hipStream_t s);
hipError_t launch_rope_query(const RopeQueryLaunch& a, hipStream_t s);
hipError_t launch_decode_valu(const DecodeLaunch& a, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t s);  // bf16 only
hipError_t launch_gqa_mfma(const DecodeLaunch& a, hipStream_t s);     // bf16 only

}  // namespace gva
