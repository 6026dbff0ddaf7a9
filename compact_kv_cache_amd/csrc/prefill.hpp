// Launch description of the causal prefill kernel (prefill_mfma.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace gva {

// Causal prefill over the cache: the last nq cached tokens of every sequence
// are the queries, query j at position seq_lens[b] - nq + j reading tokens up
// to its own. bf16 only, d_n = d_v = 64.
struct PrefillLaunch {
  int B, H, G, d_r, capacity, num_blocks, max_blocks;
  int max_seq_len;  // tokens past it are not read (as in the decode)
  int nq;       // queries per sequence
  int n_qblk;   // query blocks per sequence (of 16 * 16 / (H/G) queries)
  bool paged;
  const void* q_nope;  // [B][nq][H][d_n], or the absorbed queries [B][nq][H][d_v] when M is NULL
  const void* q_rope;  // [B][nq][H][d_r], rotated
  const void* M;       // [H][d_v][d_n] or NULL
  const void* v_cache;
  const void* kr_cache;
  const int32_t* seq_lens;
  const int32_t* block_table;
  float scale;
  void* out;  // [B][nq][H][d_v]
};

hipError_t launch_prefill_mfma(const PrefillLaunch& a, hipStream_t s);
int prefill_queries_per_block(int hpg, int d_r);  // queries per workgroup of the prefill kernel

}  // namespace gva
