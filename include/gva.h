/*
 * gva.h - C ABI of the Grouped Value Attention (GVA) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * GVA keeps a compact KV cache: per layer and sequence only the grouped
 * values V_g [G, S, d_v] and ONE positional key k_r [S, d_r] shared by all
 * query heads. Query head h rebuilds its content key as K_h = V_g(h) M_h and,
 * at decode, folds M_h into its query instead (q'_h = M_h q_nope,h), so the
 * kernels score q'_h . V_g(h)[t] + q_rope,h . k_r[t] without building keys.
 *
 * Pages cited (title, where it lives):
 *   [digest]   "Grouped Value Attention:通过按需 key 重建实现高效 KV 缓存",
 *              ai-feeds.com paper digest of arXiv 2609.13285
 *   [explain]  popular explainer of the same paper, m.szthrk.cn
 *   [abstract] "Grouped Value Attention: Efficient KV Caching via On-Demand
 *              Key Reconstruction", Hugging Face papers page
 *   [review]   "[논문리뷰] Grouped Value Attention: ...", blog.secrett2633.cloud
 *   [gqa]      "GQA 分组查询注意力：KV Cache 与模型质量的折中", charlestar.github.io
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors), row-major, densely packed, in the call dtype unless stated.
 *     `shape` itself is a host pointer read during the call only.
 *   - The caller owns every buffer. The library allocates no memory and keeps
 *     no pointer after returning.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no
 *     call synchronizes the device.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call returns a status other than GVA_OK and enqueues nothing.
 *     gva_last_error() then describes the problem (thread-local text).
 *   - Device data that the host cannot see (seq_lens, block_table) is
 *     clamped in the kernels so that a contract violation never touches
 *     memory outside the buffers described by `shape`; the results of such
 *     a call are unspecified.
 *   - Head h reads value group h / (H/G) (contiguous head blocks, as in the
 *     [gqa] tutorial's structure diagram).
 *   - RoPE turns channel pairs (2i, 2i+1) by pos * theta_i with
 *     theta_i = rope_base^(-2i/d_r); angles and the rotation are computed in
 *     double precision and rounded once (to nearest even) to the cache dtype.
 *     The pages fix no pairing; they require the cached key and the query to
 *     share one convention ([gqa] section on RoPE and the KV cache).
 */
#ifndef GVA_H
#define GVA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gva_status {
  GVA_OK = 0,
  GVA_ERR_INVALID_ARGUMENT = 1, /* null pointer, inconsistent sizes          */
  GVA_ERR_UNSUPPORTED = 2,      /* valid but not built (e.g. d_v != 64)      */
  GVA_ERR_WORKSPACE = 3,        /* workspace missing or smaller than needed  */
  GVA_ERR_HIP = 4               /* a HIP runtime call or launch failed       */
} gva_status;

typedef enum gva_dtype {
  GVA_F32 = 0,  /* IEEE binary32 everywhere                                   */
  GVA_BF16 = 1  /* bfloat16 storage; every accumulation is fp32               */
} gva_dtype;

/*
 * Problem description shared by all calls.
 *   B, H, G          sequences, query heads, value groups (H % G == 0,
 *                    H/G in {1, 2, 4})
 *   d_n, d_v         content-query and value widths (the kernels take 64, 64)
 *   d_r              shared positional-key width (0, 8, 16, 24 or 32)
 *   capacity         contiguous cache: token slots per sequence (a
 *                    multiple of 512 keeps each (sequence, group) slab on a
 *                    64 KiB boundary; strides just past a power of two can
 *                    cost a decode of many slabs up to a third of its time in
 *                    memory-channel conflicts); paged cache: ignored
 *   max_seq_len      host-side upper bound of seq_lens[b] during the call
 *                    (sizes the decode grid); tokens beyond it are ignored.
 *                    Must be <= capacity (contiguous) or
 *                    <= max_blocks_per_seq * block_size (paged).
 *   block_size       0 = contiguous cache; 64 = paged cache of 64-token blocks
 *   num_blocks       paged: blocks in the pool
 *   max_blocks_per_seq  paged: row stride of block_table
 *   split_tokens     split-K partition length in tokens for decode
 *                    (0 = automatic; otherwise a positive multiple of 64).
 *                    Automatic: partitions of whole 64-token tiles, at least
 *                    512 tokens, sized so that the B*G*partitions workgroups
 *                    fill the 256 compute units in one round; when B*G >= 256
 *                    and the longest sequence has >= 480 tiles, thirds of it.
 *                    An explicit length whose B*G*partitions reach 512 or more
 *                    is served two partitions per workgroup (the last one of
 *                    a sequence and group takes an odd leftover too); every
 *                    partition still leaves its own partial for the merge.
 *   dtype            storage dtype of q, M, caches and out
 *
 * Cache layouts (call dtype):
 *   contiguous  v_cache  [B][G][capacity][d_v]    kr_cache [B][capacity][d_r]
 *   paged       v_cache  [num_blocks][G][64][d_v] kr_cache [num_blocks][64][d_r]
 *               block_table int32 [B][max_blocks_per_seq]: entry j of row b is
 *               the pool block holding tokens [64j, 64j+64) of sequence b.
 */
typedef struct gva_shape {
  int32_t B, H, G;
  int32_t d_n, d_v, d_r;
  int32_t capacity;
  int32_t max_seq_len;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t split_tokens;
  int32_t dtype; /* a gva_dtype value */
} gva_shape;

/*
 * gva_append - write new tokens into the compact cache.
 * Follows the decode loop of [gqa] (section on why the KV cache keeps
 * growing, and the cache-lifecycle list of the RoPE section): each new token
 * stores its state once and advances the sequence position. What is stored
 * is GVA's persistent cache: the grouped values (never rotated) and the one
 * positional key after RoPE ([digest] 方法 / GVA 核心流程; [explain] 位置信息
 * 怎么办; [review] Decoupled RoPE).
 *   v_new     [B][G][n_new][d_v]   values of the new tokens
 *   kr_new    [B][n_new][d_r]      positional keys BEFORE RoPE (may be NULL
 *                                  when d_r == 0)
 *   n_new     tokens appended to every sequence (>= 1)
 *   seq_lens  int32 [B], in/out: token t of the new block lands at position
 *             seq_lens[b] + t and is rotated by that position; on completion
 *             seq_lens[b] += n_new.
 *   block_table  NULL for a contiguous cache (shape->block_size == 0).
 * Writes past the cache capacity (or into a block id outside the pool) are
 * skipped; seq_lens is then clamped to the capacity.
 */
gva_status gva_append(const gva_shape* shape, const void* v_new, const void* kr_new,
                      int32_t n_new, int32_t* seq_lens, void* v_cache, void* kr_cache,
                      const int32_t* block_table, float rope_base, hipStream_t stream);

/*
 * gva_rope_query - rotate the positional slice of the decode queries.
 * The query of the newest token sits at position seq_lens[b] - 1 (it reads the
 * earlier tokens and itself, [gqa] section on cache growth); only the d_r
 * positional channels are rotated ([review] Decoupled RoPE).
 *   q_rope_in, q_rope_out  [B][H][d_r]  (may alias)
 * A sequence with seq_lens[b] <= 0 is rotated by position 0.
 */
gva_status gva_rope_query(const gva_shape* shape, const void* q_rope_in, void* q_rope_out,
                          const int32_t* seq_lens, float rope_base, hipStream_t stream);

/*
 * gva_rope_query_multi - as gva_rope_query for the queries of the last n_q
 * cached tokens of every sequence (speculative verification, chunked decode):
 * q[b][j] (j < n_q) belongs to the token at position seq_lens[b] - n_q + j and
 * is rotated by that position (by 0 where it would be negative).
 *   q_rope_in, q_rope_out  [B][n_q][H][d_r]  (may alias)
 * gva_rope_query is the case n_q = 1.
 */
gva_status gva_rope_query_multi(const gva_shape* shape, int32_t n_q, const void* q_rope_in, void* q_rope_out,
                                const int32_t* seq_lens, float rope_base, hipStream_t stream);

/*
 * gva_decode - one decode step of GVA attention over the compact cache.
 * Computes, for every sequence b and head h with n = seq_lens[b] tokens,
 *   s_t   = scale * ( (M_h q_nope[b,h]) . V[b, g(h), t] + q_rope[b,h] . k_r[b, t] )
 *   out[b,h] = sum_t softmax(s)_t V[b, g(h), t]
 * which equals softmax attention with the materialized keys
 * K_h = [V_g(h) M_h || k_r] ([digest] 方法: Q' = Q M^T absorption and the
 * value-weighted output; [explain] 正式方案; [review] 3. Method & Key
 * Results; [abstract]). Content keys are never formed: M_h is folded into
 * the query in the kernel prologue.
 *   q_nope   [B][H][d_n]      content slice of the queries
 *   q_rope   [B][H][d_r]      positional slice, ALREADY rotated (see
 *                             gva_rope_query); NULL allowed when d_r == 0
 *   M        [H][d_v][d_n]    reconstruction maps (K_h = V_g(h) M_h), or NULL:
 *                             then q_nope holds the absorbed queries
 *                             q'[b,h] = M_h q_nope[b,h] themselves, [B][H][d_v]
 *                             (the maps folded into the query projection, see
 *                             gva_fold_query_projection), used as given
 *   v_cache, kr_cache, block_table   as described at gva_shape
 *   seq_lens int32 [B]        tokens to attend (the query's own included)
 *   scale    softmax scale, finite and > 0 (e.g. 1/sqrt(d_n + d_r))
 *   out      [B][H][d_v]      call dtype; rows with seq_lens[b] <= 0 are zero
 *   workspace, workspace_bytes   device scratch of at least
 *            gva_decode_workspace_bytes(shape) bytes (may be NULL/0 when that
 *            is 0), 16-byte aligned (GVA_ERR_WORKSPACE otherwise; device
 *            allocations are). It must be zero-filled before its first use; every call
 *            that completes leaves it ready for the next one (its arrival
 *            counters return to zero). Calls that overlap in time need
 *            distinct workspaces.
 * Long sequences are split into partitions of split_tokens tokens; each
 * partition's workgroups write a partial result (unnormalized output, running
 * max, running sum) and the last one to finish merges them with a
 * log-sum-exp combine inside the same kernel launch.
 */
gva_status gva_decode(const gva_shape* shape, const void* q_nope, const void* q_rope,
                      const void* M, const void* v_cache, const void* kr_cache,
                      const int32_t* seq_lens, const int32_t* block_table, float scale,
                      void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gva_decode_multi - decode the queries of the last n_q cached tokens of every
 * sequence at once, each reading the cache up to and including its own token
 * (a causal mask over the new tokens; [gqa] section on cache growth: a token's
 * query reads the earlier tokens and itself; the same page's list of cache
 * lifecycles names speculative decoding). With n = seq_lens[b], query j sits
 * at position n - n_q + j and attends to tokens t <= n - n_q + j (none, and a
 * zero output row, where that is negative). The n_q tokens must already be
 * in the cache (gva_append with n_new = n_q).
 *   n_q      1, 2 or 4 (2 and 4: bf16 only)
 *   q_nope   [B][n_q][H][d_n] (or absorbed [B][n_q][H][d_v] when M is NULL)
 *   q_rope   [B][n_q][H][d_r] rotated (gva_rope_query_multi)
 *   out      [B][n_q][H][d_v]
 *   workspace at least gva_decode_multi_workspace_bytes(shape, n_q) bytes,
 *            same rules as for gva_decode.
 * Other arguments as for gva_decode, which is the case n_q = 1. The group's
 * heads times the n_q queries fill the matrix-core columns, so every cache row
 * read serves n_q * H/G query rows.
 */
gva_status gva_decode_multi(const gva_shape* shape, int32_t n_q, const void* q_nope, const void* q_rope,
                            const void* M, const void* v_cache, const void* kr_cache, const int32_t* seq_lens,
                            const int32_t* block_table, float scale, void* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace gva_decode_multi needs for `shape` and n_q (0 when
 * no sequence is split). Returns 0 for an invalid shape. */
size_t gva_decode_multi_workspace_bytes(const gva_shape* shape, int32_t n_q);

/*
 * gva_prefill - causal attention of many new tokens at once over the cache
 * (prefill of a prompt, or of one chunk of it): the same computation as
 * gva_decode_multi for any n_q, on a kernel built for it ([gqa] section on
 * cache growth: every token's query reads the tokens before it and itself;
 * the same page's cache lifecycle starts with the prefill of the prompt).
 * With n = min(seq_lens[b], max_seq_len), query j of sequence b sits at
 * position n - n_q + j and attends to the tokens t <= n - n_q + j (none, and a
 * zero output row, where that is negative). The n_q tokens must already be in
 * the cache (gva_append with n_new = n_q); with n_q = seq_lens[b] the whole
 * prompt attends to itself.
 *   n_q      >= 1 queries per sequence; bf16 only
 *   q_nope   [B][n_q][H][d_n], or the absorbed queries [B][n_q][H][d_v] when
 *            M is NULL
 *   q_rope   [B][n_q][H][d_r] rotated at the queries' positions
 *            (gva_rope_query_multi with the same n_q); NULL when d_r == 0
 *   M        [H][d_v][d_n] or NULL (as for gva_decode)
 *   out      [B][n_q][H][d_v]
 * Other arguments as for gva_decode. No workspace: every workgroup owns whole
 * query rows and reads every key tile they need. Returns
 * GVA_ERR_UNSUPPORTED for an fp32 shape, GVA_ERR_INVALID_ARGUMENT for n_q < 1,
 * a missing pointer or a bad scale.
 */
gva_status gva_prefill(const gva_shape* shape, int32_t n_q, const void* q_nope, const void* q_rope,
                       const void* M, const void* v_cache, const void* kr_cache, const int32_t* seq_lens,
                       const int32_t* block_table, float scale, void* out, hipStream_t stream);

/*
 * gva_decode_step - one whole decode step in a single call: append one token
 * per sequence, rotate the query's positional slice, decode. Equivalent, bit
 * for bit, to
 *     gva_append(shape, v_new, kr_new, 1, seq_lens, v_cache, kr_cache, ...);
 *     gva_rope_query(shape, q_rope, <rotated>, seq_lens, rope_base, ...);
 *     gva_decode(shape, q_nope, <rotated>, M, v_cache, kr_cache, seq_lens, ...);
 * (the decode loop of the [gqa] page: store the new token's state, then its
 * query reads every cached token including itself). For bf16 this is one
 * kernel launch; for fp32 the library runs the three kernels in sequence.
 *   v_new    [B][G][d_v]     values of the new token
 *   kr_new   [B][d_r]        its positional key BEFORE RoPE
 *   q_nope   [B][H][d_n]     query content slice ([B][H][d_v] absorbed queries
 *                            when M is NULL, as for gva_decode)
 *   q_rope   [B][H][d_r]     query positional slice BEFORE RoPE (not modified)
 *   seq_lens int32 [B], in/out: the new token lands at seq_lens[b] and the
 *            value grows by one (clamped to the capacity as in gva_append)
 *   shape->max_seq_len must bound the lengths AFTER the append.
 *   workspace at least gva_decode_step_workspace_bytes(shape) bytes, 16-byte
 *            aligned, zero before its first use, left reusable by every
 *            completed call.
 * Other arguments as for gva_append / gva_decode.
 */
gva_status gva_decode_step(const gva_shape* shape, const void* v_new, const void* kr_new,
                           const void* q_nope, const void* q_rope, const void* M, void* v_cache,
                           void* kr_cache, int32_t* seq_lens, const int32_t* block_table, float scale,
                           float rope_base, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Bytes of device workspace gva_decode_step needs (never 0 for a valid
 * shape). Returns 0 for an invalid shape. */
size_t gva_decode_step_workspace_bytes(const gva_shape* shape);

/*
 * gva_decode_step_noalloc - gva_decode_step without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). It allocates
 * nothing: the split-K scratch is a fixed 4 MiB device array inside the
 * library, one per device, held until the process ends (its address is
 * looked up on the first call on each device, which also clears its arrival
 * counters with one small kernel launch on `stream`).
 *   Arguments and results as for gva_decode_step.
 *   Limit: gva_decode_step_workspace_bytes(shape) <= 4 MiB and
 *   B*G + B <= 512; a larger shape returns GVA_ERR_WORKSPACE before anything
 *   is launched.
 *   All calls on one device share the scratch array: calls that overlap in
 *   time on one device (concurrent streams) race and give wrong results;
 *   serialize them.
 */
gva_status gva_decode_step_noalloc(const gva_shape* shape, const void* v_new, const void* kr_new,
                                   const void* q_nope, const void* q_rope, const void* M, void* v_cache,
                                   void* kr_cache, int32_t* seq_lens, const int32_t* block_table, float scale,
                                   float rope_base, void* out, hipStream_t stream);

/*
 * Cache lifecycle on the paged cache (block_size == 64). The [gqa] page
 * (与位置编码和 KV Cache 的关系) lists what an engine does with cache blocks for
 * beam search, speculative decoding and prefix sharing: copy, share, commit
 * or roll back. The caller keeps the block allocator; these calls do the
 * device-side work. All index arrays are int32 device arrays.
 *
 * gva_copy_blocks - block dst_blocks[i] := block src_blocks[i] for
 * i < n_pairs: the V rows of all G groups and the 64 positional-key rows.
 * With remap_seqs / remap_slots (both or neither), block_table[remap_seqs[i]]
 * [remap_slots[i]] is then set to dst_blocks[i]: copy-on-write of a shared
 * block in one call. Destinations must be distinct and not among the
 * sources; pairs with a block id outside [0, num_blocks) are skipped.
 */
gva_status gva_copy_blocks(const gva_shape* shape, const int32_t* src_blocks, const int32_t* dst_blocks,
                           int32_t n_pairs, const int32_t* remap_seqs, const int32_t* remap_slots, void* v_cache,
                           void* kr_cache, int32_t* block_table, hipStream_t stream);

/*
 * gva_fork - sequence dst_seqs[i] takes the block-table row and the length of
 * sequence src_seqs[i] (i < n): its blocks become shared. Before a forked
 * sequence appends into a shared, partly filled block, the caller copies it
 * (gva_copy_blocks with remap). Destinations must be distinct and not among
 * the sources; out-of-range or equal indices are skipped.
 */
gva_status gva_fork(const gva_shape* shape, const int32_t* src_seqs, const int32_t* dst_seqs, int32_t n,
                    int32_t* seq_lens, int32_t* block_table, hipStream_t stream);

/*
 * gva_rollback - drop the newest tokens: seq_lens[b] -= n_drop[b] for every
 * sequence (n_drop int32 [B]; negative values count as 0; lengths stop at 0),
 * e.g. the rejected tokens of a speculative step. The dropped rows stay in the
 * cache and are overwritten by the next appends. Works for both layouts.
 */
gva_status gva_rollback(const gva_shape* shape, int32_t* seq_lens, const int32_t* n_drop, hipStream_t stream);

/*
 * gva_fold_query_projection - fold the reconstruction maps into the query
 * projection, once per model ([digest] section 与现有产品 / 工作流的接口: at
 * inference the reconstruction matrix can be folded into the query projection
 * and content keys are never formed; the absorption itself is Q' = Q M^T,
 * [digest] 方法). With q_nope[h] = wq_nope[h] . x,
 *   w_fold[h] = M[h] . wq_nope[h]       so that   M_h q_nope,h = w_fold[h] . x
 *   M        [H][d_v][d_n]
 *   wq_nope  [H][d_n][d_model]   content rows of the query projection
 *   w_fold   [H][d_v][d_model]   output, dtype; fp32 accumulation, rounded once
 * d_v = d_n = 64; d_model >= 1. All pointers are device pointers.
 */
gva_status gva_fold_query_projection(int32_t H, int32_t d_v, int32_t d_n, int32_t d_model, int32_t dtype,
                                     const void* M, const void* wq_nope, void* w_fold, hipStream_t stream);

/*
 * gva_query_projection - the decode queries of one layer from its hidden
 * states, with the maps already folded:
 *   q_abs[b][h]  = w_fold[h] . x[b]    absorbed content queries (pass as
 *                                      q_nope with M = NULL)
 *   q_rope[b][h] = w_rope[h] . x[b]    positional slices BEFORE RoPE
 *   x        [B][d_model]        hidden states of the new tokens
 *   w_fold   [H][d_v][d_model]   from gva_fold_query_projection
 *   w_rope   [H][d_r][d_model]   positional rows of the query projection
 *                                (NULL when d_r == 0, and then q_rope too)
 *   q_abs    [B][H][d_v], q_rope [B][H][d_r]   outputs in the call dtype
 * Uses B, H, G, d_v, d_r and dtype of `shape`. fp32 accumulation; bf16 runs on
 * the matrix cores and needs d_model % 128 == 0.
 */
gva_status gva_query_projection(const gva_shape* shape, int32_t d_model, const void* x, const void* w_fold,
                                const void* w_rope, void* q_abs, void* q_rope, hipStream_t stream);

/*
 * gva_gqa_ref_decode - plain grouped-query attention decode over a K+V cache
 * of the same layout, the comparison point for bytes and time. GQA stores a
 * key and a value row per group and token ([gqa] sections on the K/V cache
 * shapes and one GQA computation; heads read their group's K/V through the
 * head map without copying the cache, as that page asks of fast kernels).
 *   shape    d_r must be 0 and d_n == d_v (= d_h)
 *   q        [B][H][d_h]      queries, already rotated
 *   k_cache, v_cache          [B][G][capacity][d_h] or paged
 *                             [num_blocks][G][64][d_h]; K already rotated
 *   other arguments as for gva_decode (same workspace size rule).
 */
gva_status gva_gqa_ref_decode(const gva_shape* shape, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens,
                              const int32_t* block_table, float scale, void* out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace gva_decode / gva_gqa_ref_decode need for
 * `shape` (0 when no sequence is split). Returns 0 for an invalid shape. */
size_t gva_decode_workspace_bytes(const gva_shape* shape);

/* Split-K partition length (tokens) that gva_decode will use for `shape`
 * (resolves split_tokens == 0). Returns 0 for an invalid shape. */
int32_t gva_decode_split_tokens(const gva_shape* shape);

/* Persistent cache bytes per token per layer: (G * d_v + d_r) * sizeof(dtype),
 * G value rows plus the one shared positional key ([explain] section on the
 * savings; [review] Decoupled RoPE). Returns 0 for an invalid dtype. */
size_t gva_cache_bytes_per_token(int32_t G, int32_t d_v, int32_t d_r, int32_t dtype);

/* Static description of a status code. */
const char* gva_status_string(gva_status status);

/* Thread-local description of the most recent failed call on this thread
 * ("" if none). Valid until the next call on the same thread. */
const char* gva_last_error(void);

/* Library ABI version (incremented on incompatible changes). */
int32_t gva_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GVA_H */
