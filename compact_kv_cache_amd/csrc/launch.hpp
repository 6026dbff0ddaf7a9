// Host-side launcher declarations shared between the kernel sources and the
// C ABI layer. Arguments have been validated before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "../../include/gva.h"

namespace gva {

// RoPE frequencies theta_i = base^(-2i/d_r) for the d_r/2 channel pairs,
// computed once on the host in double precision and passed by value.
struct RopeTable {
  double theta[16];
};
inline RopeTable make_rope_table(double base, int d_r) {
  RopeTable t{};
  for (int i = 0; i < d_r / 2 && i < 16; ++i) t.theta[i] = std::pow(base, -2.0 * i / d_r);
  return t;
}

// theta_i of pair i, selected per lane among the table's uniform values. The
// empty asm statement keeps each value in a scalar register: without it the
// compiler folds the selection into a lane-indexed read of the kernel
// argument, a vector memory load that waits behind every load issued before.
template <int N = 16>
__device__ __forceinline__ double rope_theta(const RopeTable& t, int i) {
  static_assert(N >= 1 && N <= 16, "table size");
  double th = 0.0;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    double v = t.theta[k];
    asm volatile("" : "+s"(v));
    th = (i == k) ? v : th;
  }
  return th;
}

struct AppendLaunch {
  int B, G, d_r, n_new, capacity, num_blocks, max_blocks;
  bool paged, bf16;
  const void* v_new;
  const void* kr_new;
  int32_t* seq_lens;
  void* v_cache;
  void* kr_cache;
  const int32_t* block_table;
  RopeTable rope;
};

struct RopeQueryLaunch {
  int B, H, d_r;
  int nq;  // queries per sequence: q[b][j] sits at position seq_lens[b] - nq + j
  bool bf16;
  const void* q_in;
  void* q_out;
  const int32_t* seq_lens;
  RopeTable rope;
};

// Decode problem, shared by the GVA kernels and the GQA comparison kernel.
struct DecodeLaunch {
  int B, H, G, d_r, capacity, max_seq_len, num_blocks, max_blocks;
  int split, n_split;  // split-K partition length and count
  int nq;              // queries per sequence (the last nq tokens; 1, 2 or 4)
  int ppw;             // split-K partitions per workgroup: 1 or 2 (one query, GVA kernels)
  bool paged, bf16;
  const void* q_nope;  // GQA: q
  const void* q_rope;  // rotated; fused step: before RoPE
  const void* M;
  const void* v_cache;
  const void* kr_cache;  // GQA: k_cache
  const int32_t* seq_lens;
  const int32_t* block_table;
  float scale;
  void* out;
  // Workspace: int32 arrival counters (zero before the first call, left zero
  // by every call) -- [B*G] split-K, then [B] fused-step -- then float
  // partials o [B*nq*H*n_split*64] and (m, l) [B*nq*H*n_split*2].
  int32_t* counters;
  int32_t* counters_seq;
  float* ws_o;
  float* ws_ml;
  // Fused step only (append one token + rotate the query + decode).
  bool step;
  int cap_tokens;          // token slots per sequence (capacity or pages * 64)
  int32_t* seq_lens_rw;    // advanced by one, by the last workgroup of the sequence
  void* v_cache_rw;        // receives the appended value rows
  void* kr_cache_rw;       // receives the appended positional key
  const void* v_new;       // [B][G][d_v]
  const void* kr_new;      // [B][d_r] before RoPE
  RopeTable rope;
};

// Workspace layout (bytes): counters, partials, rotated-query scratch.
// Arrival counters sit 128 bytes apart: device-scope atomics on one cache
// line are serialized (about 11 ns each), so counters of different groups
// sharing a line would queue each other's arrivals.
constexpr int kCounterStride = 32;  // int32 slots per counter
inline size_t ws_counter_bytes(int B, int G) {
  return (((size_t)B * G + B) * kCounterStride * 4 + 255) / 256 * 256;
}
inline size_t ws_partial_bytes(int B, int H, int n_split, int nq) {
  return n_split <= 1 ? 0 : (size_t)B * nq * H * n_split * (64 + 2) * sizeof(float);
}
inline size_t ws_qrot_bytes(int B, int H) { return (((size_t)B * H * 32 * 4) + 255) / 256 * 256; }
inline size_t ws_total_bytes(int B, int H, int G, int n_split, int nq = 1) {
  if (n_split <= 1) return 0;
  return ws_counter_bytes(B, G) + ws_partial_bytes(B, H, n_split, nq);
}
inline size_t ws_step_bytes(int B, int H, int G, int n_split) {
  return ws_counter_bytes(B, G) + ws_partial_bytes(B, H, n_split, 1) + ws_qrot_bytes(B, H);
}

// Offline fold of the reconstruction maps into the query projection:
// w_fold[h] = M[h] (d_v x d_n) . wq[h] (d_n x d_model).
struct FoldLaunch {
  int H, d_v, d_n, d_model;
  bool bf16;
  const void* M;
  const void* wq;
  void* w_fold;
};

// Query projection from hidden states: rows 0 .. H*d_v-1 of the output are
// w_fold . x (q' per head), rows H*d_v .. H*(d_v+d_r)-1 are w_rope . x.
struct ProjectLaunch {
  int B, H, d_v, d_r, d_model;
  bool bf16;
  const void* x;       // [B][d_model]
  const void* w_fold;  // [H][d_v][d_model]
  const void* w_rope;  // [H][d_r][d_model] (unused when d_r == 0)
  void* q_abs;         // [B][H][d_v]
  void* q_rope;        // [B][H][d_r]
};

// Paged-cache lifecycle.
struct CopyBlocksLaunch {
  int B, num_blocks, max_blocks, n_pairs;
  int64_t v_block_bytes, kr_block_bytes;  // bytes of one block in each cache
  const int32_t* src;
  const int32_t* dst;
  const int32_t* remap_seqs;   // optional (copy-on-write table update)
  const int32_t* remap_slots;
  void* v_cache;
  void* kr_cache;
  int32_t* block_table;
};
struct ForkLaunch {
  int B, max_blocks, n;
  const int32_t* src;
  const int32_t* dst;
  int32_t* seq_lens;
  int32_t* block_table;
};

// Status reporting of the C ABI layer (sets the thread's gva_last_error text).
gva_status refuse_scratch(size_t need, size_t have);
gva_status hip_failure(hipError_t e, const char* what);

hipError_t launch_copy_blocks(const CopyBlocksLaunch& a, hipStream_t s);
hipError_t launch_fork(const ForkLaunch& a, hipStream_t s);
hipError_t launch_rollback(int32_t* seq_lens, const int32_t* n_drop, int B, hipStream_t s);
hipError_t launch_fold(const FoldLaunch& a, hipStream_t s);
hipError_t launch_project(const ProjectLaunch& a, hipStream_t s);
hipError_t launch_append(const AppendLaunch& a, hipStream_t s);
hipError_t launch_rope_query(const RopeQueryLaunch& a, hipStream_t s);
hipError_t launch_decode_valu(const DecodeLaunch& a, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t s);  // bf16 only
hipError_t launch_gqa_mfma(const DecodeLaunch& a, hipStream_t s);     // bf16 only
hipError_t launch_step_mfma(const DecodeLaunch& a, hipStream_t s);    // bf16 only, a.step set

}  // namespace gva
