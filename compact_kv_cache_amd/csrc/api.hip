// C ABI of the GVA decode library: argument validation, split-K planning and
// dispatch to the kernels. Nothing here allocates device memory.
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstdlib>
#include <string>

#include "../../include/gva.h"
#include "launch.hpp"
#include "prefill.hpp"

namespace {

thread_local std::string g_last_error;

gva_status fail(gva_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gva_status ok() {
  g_last_error.clear();
  return GVA_OK;
}

gva_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GVA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape checks common to every call. `gqa` selects the GQA comparison rules.
gva_status check_shape(const gva_shape* s, bool gqa) {
  if (!s) return fail(GVA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->G < 1)
    return fail(GVA_ERR_INVALID_ARGUMENT, "B, H, G must be >= 1 (got %d, %d, %d)", s->B, s->H, s->G);
  if (s->H % s->G != 0)
    return fail(GVA_ERR_INVALID_ARGUMENT, "H (%d) must be a multiple of G (%d)", s->H, s->G);
  const int hpg = s->H / s->G;
  if (hpg != 1 && hpg != 2 && hpg != 4)
    return fail(GVA_ERR_UNSUPPORTED, "H/G = %d; built for 1, 2 or 4 heads per group", hpg);
  if (s->d_n != 64 || s->d_v != 64)
    return fail(GVA_ERR_UNSUPPORTED, "d_n = %d, d_v = %d; built for d_n = d_v = 64", s->d_n, s->d_v);
  if (s->d_r < 0 || s->d_r % 2 != 0)
    return fail(GVA_ERR_INVALID_ARGUMENT, "d_r = %d must be even and >= 0", s->d_r);
  if (s->d_r % 8 != 0 || s->d_r > 32)
    return fail(GVA_ERR_UNSUPPORTED, "d_r = %d; built for 0, 8, 16, 24, 32", s->d_r);
  if (gqa && s->d_r != 0)
    return fail(GVA_ERR_INVALID_ARGUMENT, "GQA reference needs d_r == 0 (got %d)", s->d_r);
  if (s->dtype != GVA_F32 && s->dtype != GVA_BF16)
    return fail(GVA_ERR_INVALID_ARGUMENT, "dtype %d is not a gva_dtype", s->dtype);
  if (s->max_seq_len < 0) return fail(GVA_ERR_INVALID_ARGUMENT, "max_seq_len < 0");
  if (s->split_tokens < 0 || s->split_tokens % 64 != 0)
    return fail(GVA_ERR_INVALID_ARGUMENT, "split_tokens = %d must be 0 or a positive multiple of 64",
                s->split_tokens);
  if (s->block_size == 0) {
    if (s->capacity < 1) return fail(GVA_ERR_INVALID_ARGUMENT, "contiguous cache needs capacity >= 1");
    if (s->max_seq_len > s->capacity)
      return fail(GVA_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds capacity %d", s->max_seq_len,
                  s->capacity);
  } else if (s->block_size == 64) {
    if (s->num_blocks < 1 || s->max_blocks_per_seq < 1)
      return fail(GVA_ERR_INVALID_ARGUMENT, "paged cache needs num_blocks >= 1 and max_blocks_per_seq >= 1");
    if ((int64_t)s->max_seq_len > (int64_t)s->max_blocks_per_seq * 64)
      return fail(GVA_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds max_blocks_per_seq * 64", s->max_seq_len);
    if ((int64_t)s->max_blocks_per_seq * 64 > INT32_MAX)
      return fail(GVA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq too large");
  } else {
    return fail(GVA_ERR_UNSUPPORTED, "block_size %d; built for 0 (contiguous) or 64", s->block_size);
  }
  return GVA_OK;
}

// The automatic split of a batch that fills the units by itself (B*G >= 256)
// when thirds of the longest sequence stay long (>= 160 tiles).
bool thirds_split(const gva_shape* s) {
  return s->split_tokens <= 0 && (int64_t)s->B * s->G >= 256 && (s->max_seq_len + 63) / 64 >= 3 * 160;
}

int resolve_split(const gva_shape* s) {
  if (s->split_tokens > 0) return s->split_tokens;
  // About one workgroup of (sequence, group, partition) per compute unit
  // (256 of them; the decode kernel's LDS use, about 92 KB per workgroup,
  // allows one 512-thread workgroup per unit), so that all of them run in one
  // round: a second round pays each workgroup's fixed prologue and split-K
  // hand-off again. Each partition is a whole number of 64-token tiles, at
  // least one per wave of the eight-wave workgroup.
  const int64_t base = (int64_t)s->B * s->G;
  int64_t want_parts = (256 + base - 1) / base;
  const int64_t tiles = (s->max_seq_len + 63) / 64;
  // A batch that fills the units by itself (B*G >= 256) gets one partition
  // per (sequence, group), and uneven lengths then leave the time to the
  // longest sequences. When thirds of the longest stay long (>= 160 tiles),
  // split into thirds instead: the dispatcher hands the extra pieces to the
  // units that finish early. Measured on paged batches of 64 sequences:
  // lengths uniform in [1024, 32768] 124 -> 116 us (decode), equal lengths
  // of 32000 unchanged (186 us); shorter pieces cost more than they balance.
  if (thirds_split(s)) want_parts = 3;
  int64_t tiles_per = (tiles + want_parts - 1) / want_parts;
  if (tiles_per < 8) tiles_per = 8;
  return (int)(tiles_per * 64);
}

int n_splits(const gva_shape* s, int split) {
  return s->max_seq_len <= 0 ? 1 : (s->max_seq_len + split - 1) / split;
}

size_t workspace_for(const gva_shape* s, int nq = 1) {
  const int split = resolve_split(s);
  return gva::ws_total_bytes(s->B, s->H, s->G, n_splits(s, split), nq);
}

// The partials' (m, l) pairs are read and written as 8-byte words.
bool misaligned(const void* workspace) { return (reinterpret_cast<uintptr_t>(workspace) & 15) != 0; }

void set_workspace(gva::DecodeLaunch& a, void* workspace) {
  if (!workspace) return;
  char* base = static_cast<char*>(workspace);
  a.counters = reinterpret_cast<int32_t*>(base);
  a.counters_seq = a.counters + (size_t)a.B * a.G * gva::kCounterStride;
  a.ws_o = reinterpret_cast<float*>(base + gva::ws_counter_bytes(a.B, a.G));
  a.ws_ml = a.ws_o + (size_t)a.B * a.nq * a.H * a.n_split * 64;
}

size_t step_workspace_for(const gva_shape* s) {
  const int split = resolve_split(s);
  return gva::ws_step_bytes(s->B, s->H, s->G, n_splits(s, split));
}

// GVA_FORCE_VALU=1 routes bf16 decodes to the vector-ALU kernel (used to
// cross-check the two kernels against each other).
bool force_valu() {
  static const bool v = [] {
    const char* e = getenv("GVA_FORCE_VALU");
    return e && e[0] == '1';
  }();
  return v;
}

gva::DecodeLaunch make_decode(const gva_shape* s) {
  gva::DecodeLaunch a{};
  a.B = s->B;
  a.H = s->H;
  a.G = s->G;
  a.d_r = s->d_r;
  a.capacity = s->capacity;
  a.max_seq_len = s->max_seq_len;
  a.num_blocks = s->num_blocks;
  a.max_blocks = s->max_blocks_per_seq;
  a.split = resolve_split(s);
  a.n_split = n_splits(s, a.split);
  // An explicit partition length whose partitions would fill two or more
  // rounds of workgroups (>= 512 of them; one per compute unit) is served two
  // partitions per workgroup: the same partials, in about half the rounds.
  a.ppw = (s->split_tokens > 0 && a.n_split >= 2 && (int64_t)a.B * a.G * a.n_split >= 512) ? 2 : 1;
  a.paged = s->block_size != 0;
  a.bf16 = s->dtype == GVA_BF16;
  a.nq = 1;
  return a;
}

}  // namespace

namespace gva {
gva_status refuse_scratch(size_t need, size_t have) {
  return fail(GVA_ERR_WORKSPACE,
              "the shape needs %zu bytes of split-K scratch; the allocation-free entry point holds %zu "
              "(and up to 512 arrival counters, B*G + B)",
              need, have);
}
gva_status hip_failure(hipError_t e, const char* what) { return hip_status(e, what); }
}  // namespace gva

extern "C" {

gva_status gva_append(const gva_shape* shape, const void* v_new, const void* kr_new, int32_t n_new,
                      int32_t* seq_lens, void* v_cache, void* kr_cache, const int32_t* block_table,
                      float rope_base, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (n_new < 1) return fail(GVA_ERR_INVALID_ARGUMENT, "n_new must be >= 1 (got %d)", n_new);
  if (!v_new || !seq_lens || !v_cache)
    return fail(GVA_ERR_INVALID_ARGUMENT, "v_new, seq_lens and v_cache must be non-NULL");
  if (shape->d_r > 0 && (!kr_new || !kr_cache))
    return fail(GVA_ERR_INVALID_ARGUMENT, "kr_new and kr_cache must be non-NULL when d_r > 0");
  if (shape->block_size != 0 && !block_table)
    return fail(GVA_ERR_INVALID_ARGUMENT, "paged cache needs a block_table");
  if (!(rope_base > 0.f)) return fail(GVA_ERR_INVALID_ARGUMENT, "rope_base must be > 0");
  gva::AppendLaunch a{};
  a.B = shape->B;
  a.G = shape->G;
  a.d_r = shape->d_r;
  a.n_new = n_new;
  a.capacity = shape->capacity;
  a.num_blocks = shape->num_blocks;
  a.max_blocks = shape->max_blocks_per_seq;
  a.paged = shape->block_size != 0;
  a.bf16 = shape->dtype == GVA_BF16;
  a.v_new = v_new;
  a.kr_new = kr_new;
  a.seq_lens = seq_lens;
  a.v_cache = v_cache;
  a.kr_cache = kr_cache;
  a.block_table = block_table;
  a.rope = gva::make_rope_table(rope_base, shape->d_r);
  return hip_status(gva::launch_append(a, stream), "gva_append launch");
}

gva_status gva_rope_query(const gva_shape* shape, const void* q_rope_in, void* q_rope_out,
                          const int32_t* seq_lens, float rope_base, hipStream_t stream) {
  return gva_rope_query_multi(shape, 1, q_rope_in, q_rope_out, seq_lens, rope_base, stream);
}

gva_status gva_rope_query_multi(const gva_shape* shape, int32_t n_q, const void* q_rope_in, void* q_rope_out,
                                const int32_t* seq_lens, float rope_base, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (n_q < 1 || (int64_t)n_q * shape->B * shape->H * shape->d_r > INT32_MAX)
    return fail(GVA_ERR_INVALID_ARGUMENT, "n_q = %d must be >= 1", n_q);
  if (shape->d_r == 0) return ok();
  if (!q_rope_in || !q_rope_out || !seq_lens)
    return fail(GVA_ERR_INVALID_ARGUMENT, "q_rope_in, q_rope_out and seq_lens must be non-NULL");
  if (!(rope_base > 0.f)) return fail(GVA_ERR_INVALID_ARGUMENT, "rope_base must be > 0");
  gva::RopeQueryLaunch a{};
  a.B = shape->B;
  a.H = shape->H;
  a.d_r = shape->d_r;
  a.nq = n_q;
  a.bf16 = shape->dtype == GVA_BF16;
  a.q_in = q_rope_in;
  a.q_out = q_rope_out;
  a.seq_lens = seq_lens;
  a.rope = gva::make_rope_table(rope_base, shape->d_r);
  return hip_status(gva::launch_rope_query(a, stream), "gva_rope_query launch");
}

gva_status gva_decode(const gva_shape* shape, const void* q_nope, const void* q_rope, const void* M,
                      const void* v_cache, const void* kr_cache, const int32_t* seq_lens,
                      const int32_t* block_table, float scale, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return gva_decode_multi(shape, 1, q_nope, q_rope, M, v_cache, kr_cache, seq_lens, block_table, scale, out,
                          workspace, workspace_bytes, stream);
}

gva_status gva_decode_multi(const gva_shape* shape, int32_t n_q, const void* q_nope, const void* q_rope,
                            const void* M, const void* v_cache, const void* kr_cache, const int32_t* seq_lens,
                            const int32_t* block_table, float scale, void* out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (n_q != 1 && n_q != 2 && n_q != 4)
    return fail(GVA_ERR_UNSUPPORTED, "n_q = %d; built for 1, 2 or 4 queries per sequence", n_q);
  if (n_q > 1 && (shape->dtype != GVA_BF16 || force_valu()))
    return fail(GVA_ERR_UNSUPPORTED, "several queries per sequence need the bf16 matrix-core kernel");
  if (!q_nope || !v_cache || !seq_lens || !out)
    return fail(GVA_ERR_INVALID_ARGUMENT, "q_nope, v_cache, seq_lens and out must be non-NULL");
  if (shape->d_r > 0 && (!q_rope || !kr_cache))
    return fail(GVA_ERR_INVALID_ARGUMENT, "q_rope and kr_cache must be non-NULL when d_r > 0");
  if (shape->block_size != 0 && !block_table)
    return fail(GVA_ERR_INVALID_ARGUMENT, "paged cache needs a block_table");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GVA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  const size_t need = workspace_for(shape, n_q);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && misaligned(workspace)) return fail(GVA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  gva::DecodeLaunch a = make_decode(shape);
  a.nq = n_q;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.M = M;
  a.v_cache = v_cache;
  a.kr_cache = kr_cache;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.scale = scale;
  a.out = out;
  set_workspace(a, workspace);
  const hipError_t e = (a.bf16 && !force_valu()) ? gva::launch_decode_mfma(a, stream)
                                                 : gva::launch_decode_valu(a, stream);
  return hip_status(e, "gva_decode launch");
}

gva_status gva_prefill(const gva_shape* shape, int32_t n_q, const void* q_nope, const void* q_rope,
                       const void* M, const void* v_cache, const void* kr_cache, const int32_t* seq_lens,
                       const int32_t* block_table, float scale, void* out, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (shape->dtype != GVA_BF16)
    return fail(GVA_ERR_UNSUPPORTED, "gva_prefill is built for bf16 caches only");
  if (n_q < 1) return fail(GVA_ERR_INVALID_ARGUMENT, "n_q = %d must be >= 1", n_q);
  if (!q_nope || !v_cache || !seq_lens || !out)
    return fail(GVA_ERR_INVALID_ARGUMENT, "q_nope, v_cache, seq_lens and out must be non-NULL");
  if (shape->d_r > 0 && (!q_rope || !kr_cache))
    return fail(GVA_ERR_INVALID_ARGUMENT, "q_rope and kr_cache must be non-NULL when d_r > 0");
  if (shape->block_size != 0 && !block_table)
    return fail(GVA_ERR_INVALID_ARGUMENT, "paged cache needs a block_table");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GVA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  gva::PrefillLaunch a{};
  a.B = shape->B;
  a.H = shape->H;
  a.G = shape->G;
  a.d_r = shape->d_r;
  a.paged = shape->block_size != 0;
  a.capacity = a.paged ? 0 : shape->capacity;
  a.num_blocks = shape->num_blocks;
  a.max_blocks = shape->max_blocks_per_seq;
  a.max_seq_len = shape->max_seq_len;
  a.nq = n_q;
  const int qw = gva::prefill_queries_per_block(shape->H / shape->G, shape->d_r);
  a.n_qblk = (n_q + qw - 1) / qw;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.M = M;
  a.v_cache = v_cache;
  a.kr_cache = kr_cache;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.scale = scale;
  a.out = out;
  if ((int64_t)((a.B * a.G + 7) / 8) * 8 * a.n_qblk > INT32_MAX)
    return fail(GVA_ERR_INVALID_ARGUMENT, "grid too large");
  return hip_status(gva::launch_prefill_mfma(a, stream), "gva_prefill launch");
}

gva_status gva_decode_step(const gva_shape* shape, const void* v_new, const void* kr_new,
                           const void* q_nope, const void* q_rope, const void* M, void* v_cache,
                           void* kr_cache, int32_t* seq_lens, const int32_t* block_table, float scale,
                           float rope_base, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (!v_new || !q_nope || !v_cache || !seq_lens || !out)
    return fail(GVA_ERR_INVALID_ARGUMENT, "v_new, q_nope, v_cache, seq_lens and out must be non-NULL");
  if (shape->d_r > 0 && (!kr_new || !q_rope || !kr_cache))
    return fail(GVA_ERR_INVALID_ARGUMENT, "kr_new, q_rope and kr_cache must be non-NULL when d_r > 0");
  if (shape->block_size != 0 && !block_table)
    return fail(GVA_ERR_INVALID_ARGUMENT, "paged cache needs a block_table");
  if (shape->max_seq_len < 1)
    return fail(GVA_ERR_INVALID_ARGUMENT, "max_seq_len must bound the length after the append (>= 1)");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GVA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  if (!(rope_base > 0.f)) return fail(GVA_ERR_INVALID_ARGUMENT, "rope_base must be > 0");
  const size_t need = step_workspace_for(shape);
  if (!workspace || workspace_bytes < need)
    return fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (misaligned(workspace)) return fail(GVA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const bool paged = shape->block_size != 0;
  const int cap_tokens = paged ? shape->max_blocks_per_seq * 64 : shape->capacity;
  if (shape->dtype == GVA_BF16 && !force_valu()) {
    gva::DecodeLaunch a = make_decode(shape);
    a.q_nope = q_nope;
    a.q_rope = q_rope;
    a.M = M;
    a.v_cache = v_cache;
    a.kr_cache = kr_cache;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.scale = scale;
    a.out = out;
    set_workspace(a, workspace);
    a.step = true;
    a.cap_tokens = cap_tokens;
    a.seq_lens_rw = seq_lens;
    a.v_cache_rw = v_cache;
    a.kr_cache_rw = kr_cache;
    a.v_new = v_new;
    a.kr_new = kr_new;
    a.rope = gva::make_rope_table(rope_base, shape->d_r);
    return hip_status(gva::launch_step_mfma(a, stream), "gva_decode_step launch");
  }
  // fp32 (or forced vector-ALU path): the three kernels in sequence; the
  // rotated query goes to the scratch area at the end of the workspace.
  void* q_rot = static_cast<char*>(workspace) + need - gva::ws_qrot_bytes(shape->B, shape->H);
  gva::AppendLaunch ap{};
  ap.B = shape->B;
  ap.G = shape->G;
  ap.d_r = shape->d_r;
  ap.n_new = 1;
  ap.capacity = shape->capacity;
  ap.num_blocks = shape->num_blocks;
  ap.max_blocks = shape->max_blocks_per_seq;
  ap.paged = paged;
  ap.bf16 = shape->dtype == GVA_BF16;
  ap.v_new = v_new;
  ap.kr_new = kr_new;
  ap.seq_lens = seq_lens;
  ap.v_cache = v_cache;
  ap.kr_cache = kr_cache;
  ap.block_table = block_table;
  ap.rope = gva::make_rope_table(rope_base, shape->d_r);
  hipError_t e = gva::launch_append(ap, stream);
  if (e == hipSuccess && shape->d_r > 0) {
    gva::RopeQueryLaunch rq{};
    rq.B = shape->B;
    rq.H = shape->H;
    rq.d_r = shape->d_r;
    rq.nq = 1;
    rq.bf16 = ap.bf16;
    rq.q_in = q_rope;
    rq.q_out = q_rot;
    rq.seq_lens = seq_lens;
    rq.rope = gva::make_rope_table(rope_base, shape->d_r);
    e = gva::launch_rope_query(rq, stream);
  }
  if (e == hipSuccess) {
    gva::DecodeLaunch a = make_decode(shape);
    a.q_nope = q_nope;
    a.q_rope = shape->d_r > 0 ? q_rot : nullptr;
    a.M = M;
    a.v_cache = v_cache;
    a.kr_cache = kr_cache;
    a.seq_lens = seq_lens;
    a.block_table = block_table;
    a.scale = scale;
    a.out = out;
    set_workspace(a, workspace);
    e = gva::launch_decode_valu(a, stream);
  }
  return hip_status(e, "gva_decode_step launch");
}

gva_status gva_fold_query_projection(int32_t H, int32_t d_v, int32_t d_n, int32_t d_model, int32_t dtype,
                                     const void* M, const void* wq_nope, void* w_fold, hipStream_t stream) {
  if (H < 1 || d_model < 1) return fail(GVA_ERR_INVALID_ARGUMENT, "H and d_model must be >= 1");
  if (d_v != 64 || d_n != 64)
    return fail(GVA_ERR_UNSUPPORTED, "d_n = %d, d_v = %d; built for d_n = d_v = 64", d_n, d_v);
  if (dtype != GVA_F32 && dtype != GVA_BF16)
    return fail(GVA_ERR_INVALID_ARGUMENT, "dtype %d is not a gva_dtype", dtype);
  if (!M || !wq_nope || !w_fold)
    return fail(GVA_ERR_INVALID_ARGUMENT, "M, wq_nope and w_fold must be non-NULL");
  if ((int64_t)H * d_v * d_model > INT32_MAX)
    return fail(GVA_ERR_INVALID_ARGUMENT, "H * d_v * d_model too large");
  gva::FoldLaunch a{H, d_v, d_n, d_model, dtype == GVA_BF16, M, wq_nope, w_fold};
  return hip_status(gva::launch_fold(a, stream), "gva_fold_query_projection launch");
}

gva_status gva_query_projection(const gva_shape* shape, int32_t d_model, const void* x, const void* w_fold,
                                const void* w_rope, void* q_abs, void* q_rope, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (d_model < 1) return fail(GVA_ERR_INVALID_ARGUMENT, "d_model must be >= 1");
  if (shape->dtype == GVA_BF16 && d_model % 128 != 0)
    return fail(GVA_ERR_UNSUPPORTED, "bf16 projection needs d_model %% 128 == 0 (got %d)", d_model);
  if (!x || !w_fold || !q_abs) return fail(GVA_ERR_INVALID_ARGUMENT, "x, w_fold and q_abs must be non-NULL");
  if (shape->d_r > 0 && (!w_rope || !q_rope))
    return fail(GVA_ERR_INVALID_ARGUMENT, "w_rope and q_rope must be non-NULL when d_r > 0");
  if ((int64_t)shape->H * (shape->d_v + shape->d_r) * d_model > INT32_MAX ||
      (int64_t)shape->B * d_model > INT32_MAX)
    return fail(GVA_ERR_INVALID_ARGUMENT, "projection too large");
  gva::ProjectLaunch a{shape->B, shape->H, shape->d_v, shape->d_r, d_model, shape->dtype == GVA_BF16,
                       x, w_fold, w_rope, q_abs, q_rope};
  return hip_status(gva::launch_project(a, stream), "gva_query_projection launch");
}

gva_status gva_copy_blocks(const gva_shape* shape, const int32_t* src_blocks, const int32_t* dst_blocks,
                           int32_t n_pairs, const int32_t* remap_seqs, const int32_t* remap_slots, void* v_cache,
                           void* kr_cache, int32_t* block_table, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (shape->block_size != 64) return fail(GVA_ERR_INVALID_ARGUMENT, "block copies need a paged cache");
  if (n_pairs < 0 || n_pairs > 65535) return fail(GVA_ERR_INVALID_ARGUMENT, "n_pairs = %d out of range", n_pairs);
  if (n_pairs == 0) return ok();
  if (!src_blocks || !dst_blocks || !v_cache)
    return fail(GVA_ERR_INVALID_ARGUMENT, "src_blocks, dst_blocks and v_cache must be non-NULL");
  if (shape->d_r > 0 && !kr_cache) return fail(GVA_ERR_INVALID_ARGUMENT, "kr_cache must be non-NULL when d_r > 0");
  if ((remap_seqs == nullptr) != (remap_slots == nullptr) || (remap_seqs && !block_table))
    return fail(GVA_ERR_INVALID_ARGUMENT, "remap_seqs, remap_slots and block_table go together");
  const int es = shape->dtype == GVA_BF16 ? 2 : 4;
  gva::CopyBlocksLaunch a{};
  a.B = shape->B;
  a.num_blocks = shape->num_blocks;
  a.max_blocks = shape->max_blocks_per_seq;
  a.n_pairs = n_pairs;
  a.v_block_bytes = (int64_t)shape->G * 64 * shape->d_v * es;
  a.kr_block_bytes = (int64_t)64 * shape->d_r * es;
  a.src = src_blocks;
  a.dst = dst_blocks;
  a.remap_seqs = remap_seqs;
  a.remap_slots = remap_slots;
  a.v_cache = v_cache;
  a.kr_cache = kr_cache;
  a.block_table = block_table;
  return hip_status(gva::launch_copy_blocks(a, stream), "gva_copy_blocks launch");
}

gva_status gva_fork(const gva_shape* shape, const int32_t* src_seqs, const int32_t* dst_seqs, int32_t n,
                    int32_t* seq_lens, int32_t* block_table, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (shape->block_size != 64) return fail(GVA_ERR_INVALID_ARGUMENT, "fork needs a paged cache");
  if (n < 0 || n > 65535) return fail(GVA_ERR_INVALID_ARGUMENT, "n = %d out of range", n);
  if (n == 0) return ok();
  if (!src_seqs || !dst_seqs || !seq_lens || !block_table)
    return fail(GVA_ERR_INVALID_ARGUMENT, "src_seqs, dst_seqs, seq_lens and block_table must be non-NULL");
  gva::ForkLaunch a{shape->B, shape->max_blocks_per_seq, n, src_seqs, dst_seqs, seq_lens, block_table};
  return hip_status(gva::launch_fork(a, stream), "gva_fork launch");
}

gva_status gva_rollback(const gva_shape* shape, int32_t* seq_lens, const int32_t* n_drop, hipStream_t stream) {
  gva_status st = check_shape(shape, false);
  if (st != GVA_OK) return st;
  if (!seq_lens || !n_drop) return fail(GVA_ERR_INVALID_ARGUMENT, "seq_lens and n_drop must be non-NULL");
  return hip_status(gva::launch_rollback(seq_lens, n_drop, shape->B, stream), "gva_rollback launch");
}

size_t gva_decode_multi_workspace_bytes(const gva_shape* shape, int32_t n_q) {
  if (check_shape(shape, false) != GVA_OK || n_q < 1) return 0;
  return workspace_for(shape, n_q);
}

size_t gva_decode_step_workspace_bytes(const gva_shape* shape) {
  if (check_shape(shape, false) != GVA_OK) return 0;
  return step_workspace_for(shape);
}

gva_status gva_gqa_ref_decode(const gva_shape* shape, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* seq_lens, const int32_t* block_table,
                              float scale, void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  gva_status st = check_shape(shape, true);
  if (st != GVA_OK) return st;
  if (!q || !k_cache || !v_cache || !seq_lens || !out)
    return fail(GVA_ERR_INVALID_ARGUMENT, "q, k_cache, v_cache, seq_lens and out must be non-NULL");
  if (shape->block_size != 0 && !block_table)
    return fail(GVA_ERR_INVALID_ARGUMENT, "paged cache needs a block_table");
  if (shape->dtype != GVA_BF16)
    return fail(GVA_ERR_UNSUPPORTED, "GQA reference is built for bf16 caches only");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GVA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  const size_t need = workspace_for(shape);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(GVA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace ? workspace_bytes : (size_t)0);
  if (need > 0 && misaligned(workspace)) return fail(GVA_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  gva::DecodeLaunch a = make_decode(shape);
  a.q_nope = q;
  a.v_cache = v_cache;
  a.kr_cache = k_cache;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.scale = scale;
  a.out = out;
  set_workspace(a, workspace);
  return hip_status(gva::launch_gqa_mfma(a, stream), "gva_gqa_ref_decode launch");
}

size_t gva_decode_workspace_bytes(const gva_shape* shape) {
  if (check_shape(shape, false) != GVA_OK && check_shape(shape, true) != GVA_OK) return 0;
  return workspace_for(shape);
}

int32_t gva_decode_split_tokens(const gva_shape* shape) {
  if (check_shape(shape, false) != GVA_OK && check_shape(shape, true) != GVA_OK) return 0;
  return resolve_split(shape);
}

size_t gva_cache_bytes_per_token(int32_t G, int32_t d_v, int32_t d_r, int32_t dtype) {
  size_t el = dtype == GVA_F32 ? 4 : dtype == GVA_BF16 ? 2 : 0;
  if (G < 0 || d_v < 0 || d_r < 0) return 0;
  return ((size_t)G * d_v + d_r) * el;
}

const char* gva_status_string(gva_status status) {
  switch (status) {
    case GVA_OK: return "GVA_OK";
    case GVA_ERR_INVALID_ARGUMENT: return "GVA_ERR_INVALID_ARGUMENT";
    case GVA_ERR_UNSUPPORTED: return "GVA_ERR_UNSUPPORTED";
    case GVA_ERR_WORKSPACE: return "GVA_ERR_WORKSPACE";
    case GVA_ERR_HIP: return "GVA_ERR_HIP";
  }
  return "GVA_ERR_UNKNOWN";
}

const char* gva_last_error(void) { return g_last_error.c_str(); }

int32_t gva_abi_version(void) { return 1; }

}  // extern "C"
