// Cache lifecycle on the paged cache: copy blocks (copy-on-write), share a
// sequence's blocks with others (fork), drop the newest tokens (rollback).
// The GQA tutorial page (section on RoPE and the KV cache) lists these as the
// engine's work for beam search, speculative decoding and prefix sharing:
// copying, sharing, committing or rolling back cache blocks. The caller keeps
// the allocator (which block ids are free); these calls move the data and
// edit the tables and lengths on the device.
#include "gva_device.hpp"
#include "launch.hpp"

namespace gva {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (pair, piece of the block): 16-byte copies of the V rows
// of all groups, then the k_r rows. Invalid block ids skip the pair.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksLaunch a) {
  const int i = blockIdx.y;
  const int src = a.src[i], dst = a.dst[i];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
  const int64_t v_vecs = (int64_t)a.v_block_bytes / 16;   // per block
  const int64_t k_vecs = (int64_t)a.kr_block_bytes / 16;
  const u32x4* vs = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v_cache) + src * a.v_block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(static_cast<char*>(a.v_cache) + dst * a.v_block_bytes);
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < v_vecs; k += (int64_t)gridDim.x * blockDim.x)
    vd[k] = __builtin_nontemporal_load(vs + k);
  if (k_vecs > 0) {
    const u32x4* ks = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.kr_cache) + src * a.kr_block_bytes);
    u32x4* kd = reinterpret_cast<u32x4*>(static_cast<char*>(a.kr_cache) + dst * a.kr_block_bytes);
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < k_vecs; k += (int64_t)gridDim.x * blockDim.x)
      kd[k] = __builtin_nontemporal_load(ks + k);
  }
  // copy-on-write: point the sequence's table slot at the copy
  if (a.remap_seqs && blockIdx.x == 0 && threadIdx.x == 0) {
    const int s = a.remap_seqs[i], slot = a.remap_slots[i];
    if (s >= 0 && s < a.B && slot >= 0 && slot < a.max_blocks) a.block_table[(int64_t)s * a.max_blocks + slot] = dst;
  }
}

// One workgroup per pair: table row and length of src to dst.
__global__ __launch_bounds__(256) void fork_kernel(ForkLaunch a) {
  const int i = blockIdx.x;
  const int src = a.src[i], dst = a.dst[i];
  if (src < 0 || src >= a.B || dst < 0 || dst >= a.B || src == dst) return;
  for (int k = threadIdx.x; k < a.max_blocks; k += blockDim.x)
    a.block_table[(int64_t)dst * a.max_blocks + k] = a.block_table[(int64_t)src * a.max_blocks + k];
  if (threadIdx.x == 0) a.seq_lens[dst] = a.seq_lens[src];
}

__global__ void rollback_kernel(int32_t* seq_lens, const int32_t* n_drop, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) seq_lens[b] = max(max(seq_lens[b], 0) - max(n_drop[b], 0), 0);
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksLaunch& a, hipStream_t s) {
  if (a.n_pairs == 0) return hipSuccess;
  copy_blocks_kernel<<<dim3(8, a.n_pairs), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fork(const ForkLaunch& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  fork_kernel<<<a.n, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_rollback(int32_t* seq_lens, const int32_t* n_drop, int B, hipStream_t s) {
  rollback_kernel<<<(B + 255) / 256, 256, 0, s>>>(seq_lens, n_drop, B);
  return hipGetLastError();
}

}  // namespace gva
