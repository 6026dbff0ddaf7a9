// GVA decode (bf16 cache) on the gfx950 matrix cores, the fused decode step
// (append one token + rotate the query + decode, one launch), and the
// same-shape GQA comparison kernel, all from one skeleton.
//
// Work split: one workgroup per (sequence b, value group g, token range of
// split-K partition); its eight waves take interleaved 64-token tiles of the
// range and merge their softmax states in LDS at the end. Every cache row is
// read from HBM once per group, never once per head (the GQA tutorial page
// asks fast kernels to read K/V through the head map instead of copying it per
// head, section 一次 GQA 计算如何展开). Workgroup ids are mapped so that the G
// workgroups of one (sequence, range) land on the same XCD and share the
// positional-key rows k_r through that XCD's L2.
//
// Absorption prologue (GVA digest, 方法: Q' = Q M^T; explainer, 正式方案):
// q'_h = M_h q_nope,h on MFMA (A = rows of M_h, B = q_nope,h in every
// column), split over all eight waves (half a head each); M's rows are
// visited in a permuted order so the product comes out directly in the score
// operand's lane layout.
//
// Tiles: every 16-byte load instruction of a wave covers 1 KB of contiguous
// cache memory (8 whole V rows, or 1 KB of positional keys); the wave stores
// the tile to its own LDS buffer (16-byte chunks XOR-swizzled per row) and
// reads the matrix-core operands back from there. The first tile of every
// wave is requested from the host bound max_seq_len, before the stored length
// has arrived; rows past the stored end are cleared when the tile is staged.
//
// Per wave and 16-token sub-tile, all on v_mfma_f32_16x16x32_bf16:
//   scores     S^T[tok][col] = V[tok][:] . q'[head(col)][:] + k_r[tok] . q_rope:
//              A = V rows (lane l: token l%16, 8 channels), B = queries with
//              the group's heads repeated across the 16 columns; q' is
//              accumulated in fp32 and rounded to bf16 once.
//   P.V        O^T[ch][col] += V^T[ch][tok] . P^T[tok][col] over 32 tokens; B =
//              the score accumulator itself after the softmax, in bf16; A =
//              V^T read from the staged tile with the LDS transpose load
//              (ds_read_b64_tr_b16), no data movement through the ALUs.
// Softmax: scores stay unscaled; p = 2^(scale*log2(e)*(s - m_ref)) with one FMA
// and the raw v_exp_f32. The reference max m_ref only moves when a tile's max
// exceeds it by more than 2^8 in probability units, so the output rescale is
// rare and p stays below 256.
// Loads are non-temporal buffer loads over a per-tile range: rows past the end
// and missing pages read as zeros without touching memory, so no load is ever
// predicated and the next tile's loads stay in flight while the current one
// is computed.
//
// Fused step (the decode loop of the GQA tutorial page, section on cache
// growth: store the new token's state, then let its query read the cache up to
// and including itself): the appended position is the old seq_lens[b]; the
// positional key and the query slice are rotated in the prologue with the same
// routine as gva_append / gva_rope_query, split-0 workgroups
// store the new rows, and the workgroup whose tile holds the new position
// substitutes that row. The new length is stored by the last arrival on a
// per-sequence counter that every workgroup reaches only after reading
// seq_lens[b], so no workgroup can observe it mid-call. Results equal the
// three separate calls bit for bit.
#include "gva_device.hpp"
#include "launch.hpp"
#include "mfma_common.hpp"

namespace gva {
namespace {

constexpr int kWaves = 8;            // waves per workgroup
constexpr float kRescaleLog2 = 8.f;  // move the reference max only beyond 2^8

// One 64-token tile as loaded by one wave. Every 16-byte load instruction
// covers 1 KB of contiguous cache memory: 8 whole 128-byte rows of the score
// operand, or 1 KB of the positional-key rows (64 rows of 16*KR bytes).
// GVA: sa = V rows, kr = positional keys. GQA: sa = K rows, vb = V rows.
template <bool GQA, int KR>
struct Tile {
  u32x4 sa[8];
  u32x4 vb[GQA ? 8 : 1];
  u32x4 kr[KR > 0 ? KR : 1];
  int t0;     // first token of the tile
  int bound;  // last row of the tile that was read (rows past it load as zeros)
  bool ok;    // tile exists and its page is valid (wave-uniform)
};

// The same tile as matrix-core operands (4 sub-tiles of 16 tokens), read back
// from the wave's LDS stage: lane (col, r) holds row 16*st + col, channels
// 32*h + 8*r .. +7 in sa[st][h]. (The GQA value rows are read from the stage
// where they are used, which keeps the kernel within its registers.)
template <bool DR>
struct Frags {
  Frag sa[4][2];
  Frag kr[DR ? 4 : 1];
  int t0, bound;
  bool ok, full;
};


// The arguments that the first loads depend on come first, as scalars: gfx950
// preloads leading kernel arguments (14 dwords here) into scalar registers at
// wave launch, so the map, query and first tile requests wait for no
// kernel-argument fetch (a by-value struct is never preloaded). The launch
// struct repeats them; the copies below take precedence. H and d_r follow
// from the template (H = HPG * G, d_r = 8 * KR).
template <int HPG, bool PAGED, int KR, bool GQA, bool STEP, int NQ, bool PP2>
__global__ __launch_bounds__(64 * kWaves, 2) void decode_mfma_kernel(const void* arg_v_cache, const void* arg_kr_cache,
                                                                      const void* arg_M, const void* arg_q_nope,
                                                                      int arg_B, int arg_G, int arg_split,
                                                                      int arg_n_split, int arg_max_seq_len,
                                                                      int arg_capacity, DecodeLaunch launch) {
  DecodeLaunch a = launch;
  a.v_cache = arg_v_cache;
  a.kr_cache = arg_kr_cache;
  a.M = arg_M;
  a.q_nope = arg_q_nope;
  a.B = arg_B;
  a.G = arg_G;
  a.split = arg_split;
  a.n_split = arg_n_split;
  a.max_seq_len = arg_max_seq_len;
  a.capacity = arg_capacity;
  a.H = HPG * arg_G;
  a.d_r = 8 * KR;
  constexpr bool DR = KR > 0;  // positional slice present (d_r = 8 * KR)
  // NQ queries per sequence (the last NQ cached tokens, each reading the cache
  // up to its own position); the matrix-core column col carries query
  // (col % NCOL) / HPG of head (col % NCOL) % HPG.
  constexpr int NCOL = NQ * HPG;
  static_assert(NCOL <= 16, "at most 16 (query, head) columns");
  static_assert(NQ == 1 || (!GQA && !STEP), "several queries: GVA decode only");
  static_assert(!(GQA && DR), "GQA reference has no positional slice");
  static_assert(!(GQA && STEP), "the fused step is GVA only");
  // PP2: each workgroup takes two consecutive split-K partitions of its
  // (sequence, group), the last one also an odd leftover (in practice the
  // short tail of tokens appended past a multiple of the partition length),
  // one after the other in one stream of tiles, and leaves a partial for
  // each. Used where the partitions would otherwise need more than one round
  // of workgroups: the second round's start-up and the first round's hand-off
  // then overlap the stream instead of following it.
  static_assert(!PP2 || (NQ == 1 && !GQA), "two partitions per workgroup: one query, GVA");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, scalar
  const int col = lane & 15, r = lane >> 4;                 // MFMA column / lane group
  const int H = a.H, G = a.G, d_r = a.d_r;

  // Fused step: the first waves rotate the group's query slices (pairs
  // 0 .. HPG*d_r/2-1) and the appended key (the next d_r/2 pairs), exactly as
  // gva_rope_query and gva_append do, lane i of the workgroup taking pair i.
  // (Waves 0..3 get their load instructions through first and reach the
  // query barrier about a microsecond before waves 4..7, so the rotation
  // there stays off the barrier's path.)
  constexpr int half = 4 * (KR > 0 ? KR : 1);  // rotation pairs per row (d_r / 2)
  const int rot_i = w * 64 + lane;  // pair handled by this lane
  const bool rot_q = STEP && DR && w < 4 && rot_i < HPG * half;
  const bool rot_k = STEP && DR && w < 4 && !rot_q && rot_i < HPG * half + half;
  const int rot_j = rot_q ? rot_i / half : 0;  // head within the group
  const int rot_p = rot_q ? rot_i % half : (rot_k ? rot_i - HPG * half : 0);  // pair index

  // Workgroup id -> (sequence, partition) pair p and group g; the G groups of a
  // pair share id % 8 (one XCD) and have consecutive slots there.
  const int n_wsplit = PP2 ? max(a.n_split >> 1, 1) : a.n_split;  // workgroups per (sequence, group)
  const int pairs = a.B * n_wsplit;
  const int q8 = blockIdx.x >> 3;
  const int g = q8 % G;
  const int p = (q8 / G) * 8 + (blockIdx.x & 7);
  if (p >= pairs) return;
  const int b = p / n_wsplit, ws = p % n_wsplit;
  const int split = PP2 ? 2 * ws : ws;  // the workgroup's first partition
  const int n_own = PP2 ? (ws == n_wsplit - 1 ? a.n_split - split : 2) : 1;  // its partitions: 1 to 3

  // Partition range from the host-side bound max_seq_len. It does not depend
  // on the stored lengths, so the first tiles are requested before seq_lens[b]
  // has arrived; rows past the stored length are cleared before any use.
  const int t_begin = split * a.split;
  const int t_end_max = min(a.max_seq_len, t_begin + n_own * a.split);
  const int tiles_max = max(t_end_max - t_begin + kTile - 1, 0) / kTile;
  const float sl2 = a.scale * kLog2e;
  const int ccol = col % NCOL;
  const int jcol = ccol % HPG;       // head (within the group) of this lane's column
  const int jq = ccol / HPG;         // query of this lane's column
  const int h_col = g * HPG + jcol;  // its global head index

  __shared__ float qsh[NQ][4][kD];           // [query][head][channel] absorbed queries
  __shared__ float red_o[kWaves][NCOL][kD];  // per-wave unnormalized outputs
  __shared__ float red_ml[kWaves][NCOL][2];  // per-wave (max in log2 units, sum)
  __shared__ __bf16 qrot_sh[4][32];       // fused step: rotated query slices
  __shared__ __attribute__((aligned(16))) __bf16 krot_sh[32];  // fused step: rotated appended key
  __shared__ __attribute__((aligned(16))) __bf16 vnew_sh[kD];  // fused step: appended value row

  const __bf16* vc = reinterpret_cast<const __bf16*>(a.v_cache);
  const __bf16* sc = reinterpret_cast<const __bf16*>(GQA ? a.kr_cache : a.v_cache);
  const __bf16* kc = reinterpret_cast<const __bf16*>(a.kr_cache);
  const __bf16* qn = reinterpret_cast<const __bf16*>(a.q_nope);
  const int kr_off = DR ? 8 * min(r, KR - 1) : 0;  // lanes past d_r re-read a valid slice

  // ---- prologue loads (independent of the stored lengths) ------------------------
  // Query preparation is split evenly: wave w forms half w / 4 (32 channels) of
  // head (w % 4) % HPG of the group (with fewer heads, waves repeat a half and
  // store the same values).
  const int gm_j = (w & 3) % HPG, gm_half = w >> 2;
  const int h_w = g * HPG + gm_j;
  Frag mA[2][2], qB[2];
  uint32_t qv_bits[NQ];  // folded or GQA query elements (bf16 bits), converted after the tile issue
  // M == nullptr: the query projection already carries the reconstruction
  // map (GVA digest, section 与现有产品 / 工作流的接口: the map can be folded
  // into the query projection), so q_nope holds q' = M_h q_nope,h itself and
  // is used as loaded, like a GQA query.
  const bool folded = GQA || a.M == nullptr;  // wave-uniform
  if (!folded) {
    const __bf16* Mh = reinterpret_cast<const __bf16*>(a.M) + (int64_t)h_w * kD * kD;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mb = 2 * gm_half + m;
      const int chan = 32 * (mb >> 1) + 8 * (col >> 2) + 4 * (mb & 1) + (col & 3);
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2) mA[m][kc2].u = ld16(Mh, chan * kD + 32 * kc2 + 8 * r);
    }
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2)
      qB[kc2].u = ld16(qn + (((int64_t)b * NQ + col % NQ) * H + h_w) * kD, 32 * kc2 + 8 * r);  // column = query
  }
  // (loaded in every mode, so that no wave waits for it inside a branch)
#pragma unroll
  for (int jj = 0; jj < NQ; ++jj)
    qv_bits[jj] = reinterpret_cast<const uint16_t*>(qn)[(((int64_t)b * NQ + jj) * H + h_w) * kD + lane];
  Frag qr;
  if constexpr (DR && !STEP)
    qr.u = ld16(reinterpret_cast<const __bf16*>(a.q_rope) + (((int64_t)b * NQ + jq) * H + h_col) * d_r, kr_off);
  // Fused step: the appended value row (lane l holds channels 8*(l%8) .. +7);
  // it is kept in LDS, not in registers, for the one tile that holds it.
  u32x4 vnew_l = u32x4{0u, 0u, 0u, 0u};
  if constexpr (STEP) vnew_l = ld16(reinterpret_cast<const __bf16*>(a.v_new) + ((int64_t)b * G + g) * kD, 8 * (lane & 7));
  // Fused step: every lane loads one bf16 pair of each rotation source (lanes
  // with no pair re-read a valid one) and selects afterwards: a per-lane
  // choice of pointer would be compiled into a vector load of the kernel
  // argument, queued behind the tile loads.
  uint32_t rx = 0;
  if constexpr (STEP && DR) {
    const __bf16* qsrc = reinterpret_cast<const __bf16*>(a.q_rope) + ((int64_t)b * H + g * HPG + rot_j) * d_r;
    const __bf16* ksrc = reinterpret_cast<const __bf16*>(a.kr_new) + (int64_t)b * d_r;
    const uint32_t rq = *reinterpret_cast<const uint32_t*>(qsrc + 2 * (rot_k ? 0 : rot_p));
    const uint32_t rk = *reinterpret_cast<const uint32_t*>(ksrc + 2 * (rot_k ? rot_p : 0));
    rx = rot_k ? rk : rq;
  }

  // ---- tile loads ---------------------------------------------------------------
  // Stage of this wave in LDS: score-operand rows (swizzled 16-byte chunks),
  // then the GQA value rows or the positional keys (row-major).
  constexpr int kStageBytes = 8192 + (GQA ? 8192 : 1024 * KR);
  __shared__ __attribute__((aligned(16))) char stage_lds[kWaves * kStageBytes];
  char* const stage_w = stage_lds + w * kStageBytes;

  // Tile loads are buffer loads: the tile's rows [t0, t_hi) form the range of
  // a buffer resource, rows past it (and a whole missing tile) load as zeros
  // without a memory access, and the per-lane offsets are the same for every
  // tile. Instruction i, lane l fills staged row 8i + l/8, chunk position l%8,
  // with chunk (l%8) ^ swizzle(row) of that row; swizzle(8i + l/8) =
  // (l/8) ^ (i&1), so two offsets per 4 KB half (i even, odd) serve all
  // eight instructions with immediate offsets 1024*(i%4).
  int voff[2][2];
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      voff[hi][par] = 4096 * hi + (lane >> 3) * (kD * 2) + 16 * ((lane & 7) ^ (lane >> 3) ^ par);

  // Tile k of this partition: rows [t0, min(t0 + 64, t_hi)) (t_hi is the
  // partition end from max_seq_len for the first round, the stored end after).
  auto issue = [&](Tile<GQA, KR>& T, int k, int t_hi, int tiles) {
    const int t0 = t_begin + k * kTile;
    bool ok = k < tiles;
    int64_t vbase = 0, kbase = 0;
    if constexpr (PAGED) {
      const int jb = min(t0 / kBlock, a.max_blocks - 1);
      const int blk = ld_table(a.block_table + (int64_t)b * a.max_blocks + jb);
      ok = ok && blk >= 0 && blk < a.num_blocks;
      vbase = ((int64_t)blk * G + g) * kBlock * kD;
      kbase = (int64_t)blk * kBlock * d_r;
    } else {
      vbase = (((int64_t)b * G + g) * a.capacity + t0) * kD;
      kbase = ((int64_t)b * a.capacity + t0) * d_r;
    }
    if (!ok) vbase = kbase = 0;
    const int rows = ok ? min(kTile, t_hi - t0) : 0;
    T.t0 = t0;
    T.ok = ok;
    T.bound = max(rows - 1, 0);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(sc + vbase), 0, rows * kD * 2, kBufferWord3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      T.sa[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff[i >> 2][i & 1] + 1024 * (i & 3), 0, kNonTemporal);
    if constexpr (GQA) {
      const auto rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(vc + vbase), 0, rows * kD * 2, kBufferWord3);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        T.vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i >> 2][i & 1] + 1024 * (i & 3), 0, kNonTemporal);
    }
    if constexpr (DR) {
      // 1 KB of positional-key rows (16*KR bytes each) per instruction
      const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(kc + kbase), 0, rows * 16 * KR, kBufferWord3);
#pragma unroll
      for (int i = 0; i < KR; ++i) T.kr[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * lane + 1024 * i, 0, kNonTemporal);
    }
  };
  Tile<GQA, KR> X;
  // The prologue loads stay ahead of the tile loads (a load's result is only
  // counted complete once every earlier load of the wave is).
  __builtin_amdgcn_sched_barrier(0);
  issue(X, w, t_end_max, tiles_max);
  __builtin_amdgcn_sched_barrier(0);

  // ---- stored length --------------------------------------------------------------
  // Fused step: the token appended by this call sits at position `pos` (the
  // stored length) unless the cache is full.
  const int stored = max(a.seq_lens[b], 0);
  int pos = 0, n_full = stored;
  bool has_new = false;
  if constexpr (STEP) {
    pos = stored;
    has_new = pos < a.cap_tokens;
    n_full = has_new ? pos + 1 : a.cap_tokens;
  }
  const int n = min(n_full, a.max_seq_len);
  const int n_parts = (n + a.split - 1) / a.split;

  // Fused step: the new length is stored only once every workgroup of the
  // sequence has read the old one. Arrivals on the sequence's counter come
  // from each group's finalizer (the workgroup that writes the group's
  // output: the only participant, or the last to arrive for the split-K
  // merge, which every other participant reaches first) and from every
  // workgroup whose partition lies past the stored length (after a barrier
  // that follows its waves' reads). The last of these G * (1 + workgroups per
  // group - those holding tokens) arrivals stores the new length and clears
  // the counter;
  // no workgroup of the call reads seq_lens[b] after it. The arrival is one
  // atomic per finalizer at the end, made by the first lane of the last wave,
  // which has no merge loads of its own (loads of a wave complete in order, so
  // an atomic ahead of them would delay them by its round trip).
  static_assert(!STEP || NCOL < kWaves, "the last wave is free during the merge");
  constexpr int kSeqThread = 64 * (kWaves - 1);
  const int n_wparts = PP2 ? min(n_wsplit, (max(n_parts, 1) + 1) >> 1) : max(n_parts, 1);  // holding tokens
  const int seq_arrivals = G * (1 + n_wsplit - n_wparts);
  auto arrive_seq = [&]() {  // thread kSeqThread
    if constexpr (STEP) {
      const int ticket =
          __hip_atomic_fetch_add(a.counters_seq + (int64_t)b * kCounterStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (ticket == seq_arrivals - 1) {
        a.seq_lens_rw[b] = n_full;
        __hip_atomic_store(a.counters_seq + (int64_t)b * kCounterStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  if (split >= max(n_parts, 1)) {  // uniform per workgroup; its tile loads are simply dropped
    if constexpr (STEP) {
      __syncthreads();
      if (tid == kSeqThread) arrive_seq();
    }
    return;
  }
  const int t_end = min(n, t_begin + n_own * a.split);
  const int n_tiles = (t_end - t_begin + kTile - 1) / kTile;  // 0 only when n == 0
  const int p_col = n - NQ + jq;       // last token this lane's query reads (several queries)
  const int causal_lo = n - NQ + 1;    // tokens before it are read by every query

  // Registers -> LDS stage (plain contiguous stores), then the operand
  // fragments back. LDS operations of one wave complete in order, so the
  // fragments see the stage and the next stage cannot overtake them.
  // Rows at or past the stored end (a first-round tile may hold stale or
  // unwritten cache rows there) are staged as zeros: their scores are masked,
  // and zero value rows keep the probability-weighted sum exact.
  auto stage = [&](Tile<GQA, KR>& T) {
    if (!(T.ok && T.t0 + kTile <= t_end)) {  // wave-uniform
      const u32x4 z = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool past = T.t0 + 8 * i + (lane >> 3) >= t_end;
        T.sa[i] = past ? z : T.sa[i];
        if constexpr (GQA) T.vb[i] = past ? z : T.vb[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(stage_w + 1024 * i + 16 * lane) = T.sa[i];
      if constexpr (GQA) *reinterpret_cast<u32x4*>(stage_w + 8192 + 1024 * i + 16 * lane) = T.vb[i];
    }
    if constexpr (DR) {
#pragma unroll
      for (int i = 0; i < KR; ++i) *reinterpret_cast<u32x4*>(stage_w + 8192 + 1024 * i + 16 * lane) = T.kr[i];
    }
  };
  auto fragments = [&](Frags<DR>& F, const Tile<GQA, KR>& T) {
    F.t0 = T.t0;
    F.bound = T.bound;
    F.ok = T.ok;
    F.full = T.ok && T.t0 + kTile <= t_end;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int row = 16 * st + col;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int at = row * (kD * 2) + 16 * ((4 * h + r) ^ stage_swizzle(row));
        F.sa[st][h].u = *reinterpret_cast<const u32x4*>(stage_w + at);
      }
      if constexpr (DR) F.kr[st].u = *reinterpret_cast<const u32x4*>(stage_w + 8192 + row * (16 * KR) + 2 * kr_off);
    }
  };


  // ---- queries --------------------------------------------------------------------
  // query slots past d_r contribute nothing (masked after the tile issue, so
  // the wait for qr counts only the loads issued before it)
  if constexpr (DR && !STEP) {
    if (8 * r >= d_r) qr.u = u32x4{0u, 0u, 0u, 0u};
  }
  if (!folded) {
    f32x4 D[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      D[m] = mma(mA[m][0], qB[0], kZero4);
      D[m] = mma(mA[m][1], qB[1], D[m]);
    }
    // lane (col = query < NQ, group r) holds q'[32 * half + 8r + e] in D[e / 4][e % 4]
    if (col < NQ) {
#pragma unroll
      for (int e = 0; e < 8; ++e) qsh[col][gm_j][32 * gm_half + 8 * r + e] = D[e >> 2][e & 3];
    }
  } else {
    if (gm_half == 0) {
#pragma unroll
      for (int jj = 0; jj < NQ; ++jj) qsh[jj][gm_j][lane] = __uint_as_float(qv_bits[jj] << 16);
    }
  }
  if constexpr (STEP) {
    if (w == 0 && lane < 8) *reinterpret_cast<u32x4*>(vnew_sh + 8 * lane) = vnew_l;
  }
  if constexpr (STEP && DR) {
    if (rot_q || rot_k) {
      const float x0 = __uint_as_float(rx << 16);
      const float x1 = __uint_as_float(rx & 0xffff0000u);
      const double at = rot_q ? (double)max(n_full - 1, 0) : (double)pos;
      __bf16* dst = rot_q ? &qrot_sh[rot_j][2 * rot_p] : &krot_sh[2 * rot_p];
      // (the frequency table is read here, after the tile requests: read
      // before them, its scalar-cache miss holds the first request back)
      rope_store<__bf16>(x0, x1, at, rope_theta<half>(a.rope, rot_p), dst[0], dst[1]);
    }
  }
  __syncthreads();
  // absorbed query as the bf16 B operand (accumulated in fp32, rounded once)
  Frag qb[2];
#pragma unroll
  for (int kc2 = 0; kc2 < 2; ++kc2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[kc2].h[e] = (__bf16)qsh[jq][jcol][32 * kc2 + 8 * r + e];
  }
  if constexpr (STEP && DR) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qr.h[e] = (8 * r < d_r) ? qrot_sh[jcol][kr_off + e] : (__bf16)0.f;
    }
  }
  // Fused step: split-0 workgroups store the appended token's rows.
  if constexpr (STEP) {
    if (split == 0 && has_new && w == 0) {
      int64_t vrow = -1, krow = -1;
      if constexpr (PAGED) {
        const int blk = ld_table(a.block_table + (int64_t)b * a.max_blocks + pos / kBlock);
        if (blk >= 0 && blk < a.num_blocks) {
          vrow = (((int64_t)blk * G + g) * kBlock + pos % kBlock) * kD;
          krow = ((int64_t)blk * kBlock + pos % kBlock) * d_r;
        }
      } else {
        vrow = (((int64_t)b * G + g) * a.capacity + pos) * kD;
        krow = ((int64_t)b * a.capacity + pos) * d_r;
      }
      if (vrow >= 0) {
        __bf16* vdst = reinterpret_cast<__bf16*>(a.v_cache_rw) + vrow;
        if (lane < kD / 8) *reinterpret_cast<u32x4*>(vdst + 8 * lane) = *reinterpret_cast<const u32x4*>(vnew_sh + 8 * lane);
        if constexpr (DR) {
          if (g == 0 && lane < d_r / 8) {
            Frag kk;
#pragma unroll
            for (int e = 0; e < 8; ++e) kk.h[e] = krot_sh[8 * lane + e];
            *reinterpret_cast<u32x4*>(reinterpret_cast<__bf16*>(a.kr_cache_rw) + krow + 8 * lane) = kk.u;
          }
        }
      }
    }
  }

  // V^T operand of P.V through the LDS transpose load. Within each 16-lane
  // group r, ds_read_b64_tr_b16 hands lane col element e of the 8-byte chunk
  // addressed by lane 4*e + col/4 (its element col % 4). So lane j addresses
  // staged token 4*r + j/4 (+ 16*h + 32*pr) and channels 16*db + 4*(j%4)
  // .. +3, and lane col receives channel 16*db + col of four consecutive
  // tokens: the rows of V^T in the A layout, in the token order of the score
  // accumulator used as B (tokens 4r..4r+3 of sub-tile 2pr, then of 2pr+1).
  // Adding a multiple of 16 to the row leaves its swizzle unchanged, so one
  // per-lane offset per db serves every (pr, h).
  int tr_off[4];
  {
    const int row = 4 * r + (col >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int chan = 16 * db + 4 * (col & 3);
      tr_off[db] = row * (kD * 2) + 16 * ((chan >> 3) ^ stage_swizzle(row)) + 2 * (chan & 7);
    }
  }
  const char* const vstage = stage_w + (GQA ? 8192 : 0);

  // ---- streaming ------------------------------------------------------------------
  f32x4 acc_o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc_o[db] = kZero4;
  float m_ref = -INFINITY, l_run = 0.f;  // m_ref in raw score units
  const float thr = kRescaleLog2 / sl2;

  auto process = [&](Frags<DR>& T) {
    if (!T.ok) return;  // wave-uniform
    if constexpr (STEP) {
      // the appended row comes from the call's inputs, not from the cache
      if (has_new && pos >= T.t0 && pos < T.t0 + kTile) {
        Frag v0, v1, kk;
        v0.u = *reinterpret_cast<const u32x4*>(vnew_sh + 8 * r);
        v1.u = *reinterpret_cast<const u32x4*>(vnew_sh + 32 + 8 * r);
        if constexpr (DR) kk.u = *reinterpret_cast<const u32x4*>(krot_sh + kr_off);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          if (min(16 * st + col, T.bound) == pos - T.t0) {
            T.sa[st][0] = v0;
            T.sa[st][1] = v1;
            if constexpr (DR) T.kr[st] = kk;
          }
        }
        // ... and in the staged row that the value operand is read from
        if (pos < t_end && lane < kD / 8) {
          const int prow = pos - T.t0;
          *reinterpret_cast<u32x4*>(stage_w + prow * (kD * 2) + 16 * (lane ^ stage_swizzle(prow))) =
              *reinterpret_cast<const u32x4*>(vnew_sh + 8 * lane);
        }
      }
    }
    // V^T operands of P.V, read before the scores: they depend only on the
    // staged tile, so their LDS latency overlaps the score products and the
    // softmax
    Frag vts[2][4];
#pragma unroll
    for (int pr = 0; pr < 2; ++pr)
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(vstage + tr_off[db] + (32 * pr + 16 * h) * (kD * 2)));
          const uint2 xb = __builtin_bit_cast(uint2, x);
          vts[pr][db].u[2 * h] = xb.x;
          vts[pr][db].u[2 * h + 1] = xb.y;
        }
    f32x4 s[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      f32x4 c = mma(T.sa[st][0], qb[0], kZero4);
      c = mma(T.sa[st][1], qb[1], c);
      if constexpr (DR) c = mma(T.kr[st], qr, c);
      s[st] = c;
    }
    // Masks: tokens past the partition end, and (several queries) tokens past
    // the column's own position; tokens below causal_lo are seen by all.
    if (!T.full || (NQ > 1 && T.t0 + kTile > causal_lo)) {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = T.t0 + 16 * st + 4 * r + i;
          if (tok >= t_end || (NQ > 1 && tok > p_col)) s[st][i] = -INFINITY;
        }
    }
    float lmx = -INFINITY;  // over this lane's 16 scores of the column
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) lmx = fmaxf(lmx, s[st][i]);
    // The reference moves only where the column max passes it by thr; a
    // lane's own max decides whether that can happen anywhere in the wave,
    // and only then is the column max formed across the four lanes.
    if (__any(lmx > m_ref + thr)) {
      const float mx = rows_max(lmx);
      const float m_new = (mx > m_ref + thr) ? mx : m_ref;
      // 0 on a column's first tile; 1 where the max does not move (also a
      // column that has seen only masked scores so far)
      const float alpha = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f((m_ref - m_new) * sl2);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc_o[db] *= alpha;
      m_ref = m_new;
    }
    const float bias = (m_ref == -INFINITY) ? 0.f : -m_ref * sl2;  // all-masked column: p = 0
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[st][i] = __builtin_amdgcn_exp2f(fmaf(s[st][i], sl2, bias));
    float psum = s[0][0];  // (not 0 + ...: the compiler keeps an add of +0)
#pragma unroll
    for (int e = 1; e < 16; ++e) psum += s[e >> 2][e & 3];
    l_run += psum;
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      Frag pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb.h[i] = (__bf16)s[2 * pr][i];
        pb.h[4 + i] = (__bf16)s[2 * pr + 1][i];
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) acc_o[db] = mma(vts[pr][db], pb, acc_o[db]);
    }
  };

  // Each tile is staged, its registers are reloaded at once with the wave's
  // next tile, and the math runs on the staged copy: one tile in flight per
  // wave while it computes. (Eight waves of one compute unit then keep about
  // 80 KB of reads in flight, more than the rate needs. A second tile in
  // flight made a wave stall at load issue while the unit's request queue was
  // full, with a staged tile waiting behind the stalled instruction.)
  // With one tile in flight the wait before staging covers every outstanding
  // load on any path, so the reload is simply skipped after the wave's last
  // tile (an empty-range load would still take a slot in the request queue).
  Frags<DR> F;
  // PP2: the softmax states of the workgroup's first and second partitions,
  // set aside when the wave's tiles move on to the next partition (tiles
  // kTPP and 2 kTPP onward of the range); `reached` counts them (uniform).
  f32x4 acc_a[PP2 ? 4 : 1], acc_b[PP2 ? 4 : 1];
  float m_a = -INFINITY, l_a = 0.f, m_b = -INFINITY, l_b = 0.f;
  int reached = 0;
  const int kTPP = a.split / kTile;
#pragma clang loop unroll(disable)
  for (int k = w; k < n_tiles; k += kWaves) {
    if constexpr (PP2) {
      const int pk = (k >= kTPP) + (k >= 2 * kTPP);  // partition of this tile in the range
      if (reached == 0 && pk >= 1) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          acc_a[db] = acc_o[db];
          acc_o[db] = kZero4;
        }
        m_a = m_ref;
        l_a = l_run;
        m_ref = -INFINITY;
        l_run = 0.f;
        reached = 1;
      }
      if (reached == 1 && pk >= 2) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          acc_b[db] = acc_o[db];
          acc_o[db] = kZero4;
        }
        m_b = m_ref;
        l_b = l_run;
        m_ref = -INFINITY;
        l_run = 0.f;
        reached = 2;
      }
    }
    stage(X);
    fragments(F, X);
    if (k + kWaves < n_tiles) issue(X, k + kWaves, t_end, n_tiles);  // wave-uniform
    process(F);
  }

  // ---- merge the waves ----------------------------------------------------------------
  // merge thread: column jj = wave + 8u (query jj / HPG, head jj % HPG), channel d
  constexpr int kPer = (NCOL + kWaves - 1) / kWaves;
  const int d = lane;
  float o[kPer], l[kPer], mfin[kPer];
  int64_t orow[kPer];  // (sequence, query, head) row of the output and of the partials
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int jj = (tid >> 6) + u * kWaves;
    orow[u] = ((int64_t)b * NQ + jj / HPG) * H + g * HPG + jj % HPG;
  }
  // One partition's state of the eight waves, merged in LDS into o, l, mfin.
  auto merge_waves = [&](const f32x4 (&acc)[4], float m_w, float l_w) {
    l_w = rows_sum(l_w);
    if (col < NCOL) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[w][col][16 * db + 4 * r + i] = acc[db][i];
      if (r == 0) {
        red_ml[w][col][0] = m_w * sl2;  // log2 units (-inf for a wave without tiles)
        red_ml[w][col][1] = l_w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int jj = (tid >> 6) + u * kWaves;
      o[u] = 0.f;
      l[u] = 0.f;
      mfin[u] = -INFINITY;
      if (jj < NCOL) {
        // every LDS read of the merge in flight at once, then the arithmetic
        float2 ml8[kWaves];
        float ov[kWaves];
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          ml8[ww] = *reinterpret_cast<const float2*>(&red_ml[ww][jj][0]);
          ov[ww] = red_o[ww][jj][d];
        }
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) mfin[u] = fmaxf(mfin[u], ml8[ww].x);
        const float mref = mfin[u] == -INFINITY ? 0.f : mfin[u];  // no wave holds tokens: weights 0
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
          const float f = __builtin_amdgcn_exp2f(ml8[ww].x - mref);
          o[u] = fmaf(f, ov[ww], o[u]);
          l[u] = fmaf(f, ml8[ww].y, l[u]);
        }
      }
    }
  };
  auto store_partial = [&](int part) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if ((tid >> 6) + u * kWaves < NCOL) {
        const int64_t slot = orow[u] * a.n_split + part;
        st_dev(a.ws_o + slot * kD + d, o[u]);
        if (d == 0) st_dev_ml(a.ws_ml + 2 * slot, mfin[u], l[u]);
      }
    }
  };
  // Partition j of the range: set aside if the wave went past it, live if it
  // is the wave's current one, empty if the wave has no tile there. (Selected
  // per wave, then merged by every wave together: the merge holds a
  // workgroup barrier.)
  auto merge_part = [&](int j) {
    if constexpr (PP2) {
      const bool aside = reached > j, live = reached == j;
      f32x4 acc_j[4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc_j[db] = aside ? (j == 0 ? acc_a[db] : acc_b[db]) : (live ? acc_o[db] : kZero4);
      const float m_j = aside ? (j == 0 ? m_a : m_b) : (live ? m_ref : -INFINITY);
      const float l_j = aside ? (j == 0 ? l_a : l_b) : (live ? l_run : 0.f);
      merge_waves(acc_j, m_j, l_j);
    } else {
      merge_waves(acc_o, m_ref, l_run);
    }
  };
  merge_part(0);
  __bf16* out = reinterpret_cast<__bf16*>(a.out);
  if (n_parts <= 1) {
    if (tid == kSeqThread) arrive_seq();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if ((tid >> 6) + u * kWaves < NCOL) out[orow[u] * kD + d] = (__bf16)(l[u] > 0.f ? o[u] / l[u] : 0.f);
    return;
  }
  if constexpr (!PP2 && !STEP) {
    // Decode: each wave that owns output rows (rows w + 8u) hands off on its
    // own, with no workgroup barrier: it waits for its own partial stores'
    // acknowledgement and arrives on its own counter (slot 4w of the group's
    // counter line, which stays zero between calls); the last arrival merges
    // those rows. (The fused step keeps the workgroup-wide arrival below:
    // there this form measured about 0.1 us slower at the mid shape, against
    // 0.1-0.2 us faster for the decode.)
    constexpr int kOwn = NCOL < kWaves ? NCOL : kWaves;
    static_assert(4 * kWaves <= kCounterStride, "one counter slot per wave on the group's line");
    if (w >= kOwn) return;
    store_partial(split);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are acknowledged
    int32_t* wcounter = a.counters + ((int64_t)b * G + g) * kCounterStride + 4 * w;
    int ticket = 0;
    if (lane == 0) ticket = __hip_atomic_fetch_add(wcounter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket != n_parts - 1) return;
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if (w + u * kWaves < NCOL)
        out[orow[u] * kD + d] = (__bf16)merge_partials(a.ws_o, a.ws_ml, orow[u] * a.n_split, n_parts, d);
    if (lane == 0) reset_counter(wcounter);
    return;
  }
  store_partial(split);
  // partitions of the range that hold tokens (uniform)
  const int arrivals = min(split + n_own, n_parts) - split;
  if constexpr (PP2) {
    for (int j = 1; j < arrivals; ++j) {
      __syncthreads();  // every thread is done reading the previous partition's state
      merge_part(j);
      store_partial(split + j);
    }
  }
  int32_t* counter = a.counters + ((int64_t)b * G + g) * kCounterStride;
  if (arrive_last(counter, n_parts, arrivals)) {
    if (tid == kSeqThread) arrive_seq();
#pragma unroll
    for (int u = 0; u < kPer; ++u)
      if ((tid >> 6) + u * kWaves < NCOL)
        out[orow[u] * kD + d] = (__bf16)merge_partials(a.ws_o, a.ws_ml, orow[u] * a.n_split, n_parts, d);
    if (tid == 0) reset_counter(counter);
  }
}

template <int HPG, int KR, bool GQA, bool STEP, int NQ, bool PP2>
hipError_t mfma_launch_ppw(const DecodeLaunch& a, hipStream_t s) {
  const int pairs = a.B * (PP2 ? max(a.n_split >> 1, 1) : a.n_split);
  const dim3 grid(((pairs + 7) / 8) * 8 * a.G);
  if (a.paged)
    decode_mfma_kernel<HPG, true, KR, GQA, STEP, NQ, PP2><<<grid, 64 * kWaves, 0, s>>>(
        a.v_cache, a.kr_cache, a.M, a.q_nope, a.B, a.G, a.split, a.n_split, a.max_seq_len, a.capacity, a);
  else
    decode_mfma_kernel<HPG, false, KR, GQA, STEP, NQ, PP2><<<grid, 64 * kWaves, 0, s>>>(
        a.v_cache, a.kr_cache, a.M, a.q_nope, a.B, a.G, a.split, a.n_split, a.max_seq_len, a.capacity, a);
  return hipGetLastError();
}

template <int HPG, int KR, bool GQA, bool STEP, int NQ>
hipError_t mfma_launch(const DecodeLaunch& a, hipStream_t s) {
  if constexpr (NQ == 1 && !GQA) {
    if (a.ppw == 2) return mfma_launch_ppw<HPG, KR, GQA, STEP, NQ, true>(a, s);
  }
  return mfma_launch_ppw<HPG, KR, GQA, STEP, NQ, false>(a, s);
}

// queries per sequence: 1 (every path), 2 or 4 (GVA decode of several new tokens)
template <int HPG, int KR, bool GQA, bool STEP>
hipError_t mfma_paged(const DecodeLaunch& a, hipStream_t s) {
  if constexpr (!GQA && !STEP) {
    if (a.nq == 2) return mfma_launch<HPG, KR, false, false, 2>(a, s);
    if (a.nq == 4) return mfma_launch<HPG, KR, false, false, 4>(a, s);
  }
  return mfma_launch<HPG, KR, GQA, STEP, 1>(a, s);
}


// d_r = 8 * KR (validated on the host: 0, 8, 16, 24 or 32)
template <int HPG, bool GQA, bool STEP>
hipError_t mfma_dr(const DecodeLaunch& a, hipStream_t s) {
  if constexpr (!GQA) {
    switch (a.d_r / 8) {
      case 1: return mfma_paged<HPG, 1, false, STEP>(a, s);
      case 2: return mfma_paged<HPG, 2, false, STEP>(a, s);
      case 3: return mfma_paged<HPG, 3, false, STEP>(a, s);
      case 4: return mfma_paged<HPG, 4, false, STEP>(a, s);
      default: break;
    }
  }
  return mfma_paged<HPG, 0, GQA, STEP>(a, s);
}

template <bool GQA, bool STEP>
hipError_t mfma_dispatch(const DecodeLaunch& a, hipStream_t s) {
  switch (a.H / a.G) {
    case 1: return mfma_dr<1, GQA, STEP>(a, s);
    case 2: return mfma_dr<2, GQA, STEP>(a, s);
    default: return mfma_dr<4, GQA, STEP>(a, s);
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeLaunch& a, hipStream_t s) { return mfma_dispatch<false, false>(a, s); }
hipError_t launch_gqa_mfma(const DecodeLaunch& a, hipStream_t s) { return mfma_dispatch<true, false>(a, s); }
hipError_t launch_step_mfma(const DecodeLaunch& a, hipStream_t s) { return mfma_dispatch<false, true>(a, s); }

}  // namespace gva
