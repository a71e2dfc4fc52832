// a3/a4: paged decode attention with split-K and a log-sum-exp merge (gfx950).
//
// What is computed follows "mini-vLLM v0.4" (shadowgraph.io) section 5: for each
// query head, walk the sequence's block table, keep the online-softmax state
// (running max m, exp-sum l, weighted V sum acc) and never materialise a
// contiguous K/V copy; KV head = q head / group size.  Partial states are merged
// with the rescaling of the nano-vLLM lab manual's Fig. B-5.
//
// MI355X design.  A wave owns one KV head and a G-wide tile of its query heads,
// so each K/V byte is read from HBM once for the whole GQA group.  LANES lanes
// hold one token row of that head (16 bytes each: a 128-dim bf16 row is 16
// lanes), so one load instruction fetches RG consecutive tokens; q.k uses
// v_dot2_f32_bf16 and is reduced over the LANES lanes with DPP row moves.  Each
// row group keeps its own online-softmax state, folded once per emitted piece.
// The next chunk's K/V loads are in flight while the current chunk is reduced.
//
// Two ways of splitting the keys (both merged by the same rescaling):
//  * balanced (the default): every sequence's keys, in chunks of CH tokens, are
//    laid end to end and each wave of a KV head gets an equal contiguous slice,
//    whatever the sequence boundaries.  A sequence that lies inside one slice is
//    finished by that wave; one cut by slice boundaries leaves at most one
//    partial state per side in each wave it touches.  Every wave does the same
//    amount of work, which removes the ragged tail that sequence-aligned
//    partitions of a mixed-length batch leave behind.
//  * fixed partitions of P tokens per sequence (the caller's choice), with the
//    workspace layout documented in pa.h.
#include <limits.h>

#include <mutex>

#include "pa_decode_plan.h"

namespace pa {

// ---------------------------------------------------------------------------
// Fixed partitions: grid = (partition, head group, sequence).  One wave = one
// (sequence, KV head, head tile, partition); the waves of a workgroup are
// consecutive KV heads of the same tokens.  split == 0: one partition per
// sequence, written straight to `out`.
template <int D, int ET, int G>
__global__ __launch_bounds__(max_head_waves(G) * 64) void decode_kernel(
    void* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l, const void* __restrict__ qptr, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ context_lens, int num_blocks, int bs_log2, int HQ, int HKV,
    int group, float scale_log2, int part_size, int NP, int split) {
  using W = DecodeWave<D, ET, G>;
  using E = Elem<ET>;
  constexpr int CH = W::CH;
  constexpr int U = W::U;

  const int p = blockIdx.x;
  const int b = blockIdx.z;
  const int tiles = group / G;
  const int hw = blockIdx.y * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (hw >= HKV * tiles) return;  // padding wave of the last head group
  const int g = hw / tiles;
  const int h0 = g * group + (hw % tiles) * G;
  const int L = context_lens[b];
  const int start = split ? p * part_size : 0;
  const int end = split ? min(start + part_size, L) : L;
  if (start >= end) {
    if (!split) {  // empty context: the output row is zero
      for (int i = threadIdx.x & 63; i < G * D; i += 64)
        E::store(out, ((int64_t)b * HQ + h0 + i / D) * D + i % D, 0.0f);
    }
    return;
  }

  W st;
  st.init(kcache, vcache, g, HKV, bs_log2, maxb, num_blocks, scale_log2);
  st.load_q(qptr, (int64_t)b * HQ + h0);
  st.reset();
  const int32_t* bt = block_table + (int64_t)b * maxb;

  // A and B alternate; the chunk count is known up front, so every compute()
  // has exactly one set of loads still pending behind it.
  const int nchunks = (end - start + CH - 1) / CH;
  KVRegs<U> A, B;
  int idsA[U], idsB[U];
  int c = start;
  st.fetch_ids(bt, c, end, idsA);
  st.issue(A, c, end, idsA);
  st.fetch_ids(bt, c + CH, end, idsB);
  for (int k = 0; k < (nchunks - 1) / 2; ++k) {
    st.issue(B, c + CH, end, idsB);
    st.fetch_ids(bt, c + 2 * CH, end, idsA);
    st.compute(A, c, end);
    st.issue(A, c + 2 * CH, end, idsA);
    st.fetch_ids(bt, c + 3 * CH, end, idsB);
    st.compute(B, c + CH, end);
    c += 2 * CH;
  }
  if ((nchunks - 1) & 1) {
    st.issue(B, c + CH, end, idsB);
    st.compute(A, c, end);
    st.compute(B, c + CH, end);
  } else {
    st.compute(A, c, end);
  }

  st.fold();
  if (split)
    st.store_state(ws_acc, ws_m, ws_l, ((int64_t)b * HQ + h0) * NP + p, NP);
  else
    st.store_final(out, (int64_t)b * HQ + h0);
}

// Standalone balanced kernel: wave item i of the grid runs slice i / head_waves of head
// wave i % head_waves (head_waves = KV heads x query-head tiles per KV head).  Workgroups
// hold max_head_waves(G) waves whatever the number of head waves, so that the grid is
// about one workgroup per compute unit and every unit runs the same number of waves
// (with one workgroup per slice, 4 head waves made 4-wave workgroups, 1.5 per unit).
// APPEND: the cache holds the first context_lens[b] - 1 keys of each sequence and the last
// comes from the step's new rows `ap`, which the launch also stores to their slots.
template <int D, int ET, int G, bool APPEND>
__global__ __launch_bounds__(max_head_waves(G) * 64) void decode_balanced_kernel(
    void* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l, int32_t* __restrict__ ws_cuc, const void* __restrict__ qptr,
    const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ block_table, int maxb, const int32_t* __restrict__ context_lens,
    int B, int num_blocks, int bs_log2, int HQ, int HKV, int group, float scale_log2, int Wt,
    AppendRows ap) {
  const int head_waves = HKV * (group / G);
  const int item = blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  decode_balanced_body<D, ET, G, false, APPEND>(
      item / head_waves, item % head_waves, blockIdx.x == 0, out, ws_acc, ws_m, ws_l, ws_cuc,
      qptr, kcache, vcache, block_table, maxb, context_lens, nullptr, nullptr, 0, B, num_blocks,
      bs_log2, HQ, HKV, group, scale_log2, Wt, ap);
}

// ---------------------------------------------------------------------------
// Merges: one workgroup per (query head, sequence), one thread per element.

template <int ET, int W>
__global__ __launch_bounds__(64 * W) void merge_kernel(
    void* __restrict__ out, const float* __restrict__ ws_acc, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const int32_t* __restrict__ context_lens, int HQ, int D,
    int NP, int part_size) {
  using E = Elem<ET>;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t bh = (int64_t)b * HQ + h;
  const int L = context_lens[b];
  int n = L > 0 ? (L + part_size - 1) / part_size : 0;
  n = min(n, NP);
  if (n == 0) {
    for (int d = threadIdx.x; d < D; d += blockDim.x) E::store(out, bh * D + d, 0.0f);
    return;
  }
  merge_states<ET, W>(out, bh * D, ws_acc, ws_m, ws_l, n, D, [&](int k) { return bh * NP + k; });
}

// ---------------------------------------------------------------------------
// Host side.

typedef void (*decode_fn)(void*, float*, float*, float*, const void*, const void*, const void*,
                          const int32_t*, int, const int32_t*, int, int, int, int, int, float, int,
                          int, int);
typedef void (*balanced_fn)(void*, float*, float*, float*, int32_t*, const void*, const void*,
                            const void*, const int32_t*, int, const int32_t*, int, int, int, int,
                            int, int, float, int, AppendRows);

// The appending first pass keeps two waves per SIMD without spills for every head tile in
// bf16 and fp32, and in fp16 for tiles of 1, 2, 3 and 5 query heads (4 and 6 spill, 7 and 8
// fit only one wave per SIMD); those fp16 tiles store the new rows with a launch of their own.
template <int D, int ET, int G>
static balanced_fn append_kernel() {
  if constexpr (ET != PA_F16 || G <= 3 || G == 5) return decode_balanced_kernel<D, ET, G, true>;
  else return nullptr;
}

template <int D, int ET>
static void pick_g(int G, decode_fn* f, balanced_fn* fb, balanced_fn* fa) {
  switch (G) {
#define PA_CASE(g)                                \
  case g:                                         \
    *f = decode_kernel<D, ET, g>;                 \
    *fb = decode_balanced_kernel<D, ET, g, false>; \
    *fa = append_kernel<D, ET, g>();               \
    return;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
  }
  *f = nullptr;
  *fb = nullptr;
  *fa = nullptr;
}

static void pick_decode(int D, pa_dtype dt, int G, decode_fn* f, balanced_fn* fb, balanced_fn* fa) {
  if (dt == PA_BF16) D == 64 ? pick_g<64, PA_BF16>(G, f, fb, fa) : pick_g<128, PA_BF16>(G, f, fb, fa);
  else if (dt == PA_F16) D == 64 ? pick_g<64, PA_F16>(G, f, fb, fa) : pick_g<128, PA_F16>(G, f, fb, fa);
  else D == 64 ? pick_g<64, PA_F32>(G, f, fb, fa) : pick_g<128, PA_F32>(G, f, fb, fa);
}

static int validate_common(const char* fn, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes (seqs %d, q_heads %d, kv_heads %d)", fn, num_seqs,
                num_q_heads, num_kv_heads);
  if (num_q_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "%s: q_heads %d not a multiple of kv_heads %d", fn, num_q_heads,
                num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  return PA_OK;
}

static int validate_partition(const char* fn, int32_t partition_size) {
  if (partition_size == 0 || partition_size == -1) return PA_OK;
  if (!is_pow2(partition_size) || partition_size < 16)
    return fail(PA_ERR_UNSUPPORTED, "%s: partition_size %d (0, -1 or a power of two >= 16)", fn,
                partition_size);
  return PA_OK;
}

static int32_t resolve_max_ctx(int32_t max_ctx, int32_t maxb, int32_t bs) {
  if (max_ctx > 0) return max_ctx;
  const int64_t t = (int64_t)maxb * bs;
  return (int32_t)(t < INT32_MAX ? t : INT32_MAX);
}

static int launch_merge(void* out, const DecodePlan& pl, const WsPtrs& w,
                        const int32_t* context_lens, int32_t B, int32_t HQ, int32_t D,
                        pa_dtype dtype, hipStream_t s) {
  // Pieces per output row: about one more than the mean slices per sequence (balanced), or
  // the partitions of the longest sequence (fixed).
  const int64_t pieces = pl.mode == DecodePlan::kBalanced ? (pl.Wt + B - 1) / B + 1 : pl.NP;
  const int W = merge_waves(pieces, (int64_t)HQ * B);
  const dim3 grid(HQ, B), block(64 * W);
#define PA_MERGE_W(ET, WV)                                                                       \
  if (pl.mode == DecodePlan::kBalanced)                                                          \
    hipLaunchKernelGGL((merge_balanced_kernel<ET, false, WV>), grid, block, 0, s, out, w.acc,    \
                       w.m, w.l, w.cuc, nullptr, 0, B, HQ, D, pl.Wt);                            \
  else                                                                                           \
    hipLaunchKernelGGL((merge_kernel<ET, WV>), grid, block, 0, s, out, w.acc, w.m, w.l,          \
                       context_lens, HQ, D, pl.NP, pl.P);
#define PA_MERGE(ET)                                                                          \
  if (W == 1 && pl.mode == DecodePlan::kBalanced) {                                           \
    hipLaunchKernelGGL((merge_balanced_kernel<ET, false, 1, kMergeHeadsPerWG>),               \
                       dim3((HQ + kMergeHeadsPerWG - 1) / kMergeHeadsPerWG, B),                \
                       dim3(64 * kMergeHeadsPerWG), 0, s, out, w.acc, w.m, w.l, w.cuc, nullptr, \
                       0, B, HQ, D, pl.Wt);                                                    \
  } else if (W == 1) {                                                                        \
    PA_MERGE_W(ET, 1)                                                                         \
  } else if (W == 2) {                                                                        \
    PA_MERGE_W(ET, 2)           \
  } else if (W == 4) {          \
    PA_MERGE_W(ET, 4)           \
  } else {                      \
    PA_MERGE_W(ET, kMergeWaves) \
  }
  if (dtype == PA_BF16) {
    PA_MERGE(PA_BF16)
  } else if (dtype == PA_F16) {
    PA_MERGE(PA_F16)
  } else {
    PA_MERGE(PA_F32)
  }
#undef PA_MERGE
#undef PA_MERGE_W
  return check_launch("decode merge");
}

// First pass for any plan; kSingle writes `out` directly.
static int launch_decode(const char* fn, const DecodePlan& pl, void* out, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         int32_t maxb, const int32_t* context_lens, int32_t B, int32_t NB,
                         int32_t bs, int32_t HQ, int32_t HKV, int32_t D, float scale,
                         pa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t s,
                         const AppendRows* ap = nullptr, bool fuse = true) {
  if (pl.mode != DecodePlan::kSingle && (!workspace || workspace_bytes < pl.ws_bytes))
    return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes,
                pl.ws_bytes);
  decode_fn kern;
  balanced_fn bkern, akern;
  pick_decode(D, dtype, pl.G, &kern, &bkern, &akern);
  // The appending first pass exists for the balanced split (and the tiles append_kernel
  // names) and is used when the caller asks for it (fuse); otherwise the new rows are stored
  // by a launch of their own first and the first pass reads them from the cache.
  if (ap && (pl.mode != DecodePlan::kBalanced || !akern || !fuse)) {
    if (int st = launch_store_decode_rows(ap->key, ap->value, ap->key_stride, ap->value_stride,
                                          ap->kc, ap->vc, block_table, maxb, context_lens, B, NB,
                                          bs, (int64_t)HKV * D * elt_bytes(dtype), s))
      return st;
    ap = nullptr;
  }
  if (!kern) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for head tile %d", fn, pl.G);
  const int group = HQ / HKV;
  const int head_waves = HKV * (group / pl.G);
  const int wpb = head_waves < max_head_waves(pl.G) ? head_waves : max_head_waves(pl.G);
  const int groups = (head_waves + wpb - 1) / wpb;
  const WsPtrs w = pl.mode == DecodePlan::kSingle ? WsPtrs{} : carve(workspace, pl, B, HQ, D);
  if (pl.mode == DecodePlan::kBalanced) {
    const size_t lds = (size_t)(2 * B + 1) * sizeof(int);
    const int wpg = max_head_waves(pl.G);
    const int64_t n_wg = ceil_div((int64_t)pl.Wt * head_waves, wpg);
    if (n_wg > INT32_MAX) return fail(PA_ERR_SHAPE, "%s: grid too large", fn);
    hipLaunchKernelGGL(ap ? akern : bkern, dim3((unsigned)n_wg), dim3(wpg * 64), lds, s, out,
                       w.acc, w.m, w.l, w.cuc, q, k_cache, v_cache, block_table, maxb,
                       context_lens, B, NB, __builtin_ctz(bs), HQ, HKV, group, scale * kLog2e,
                       pl.Wt, ap ? *ap : AppendRows{});
  } else {
    const bool split = pl.mode == DecodePlan::kFixed;
    hipLaunchKernelGGL(kern, dim3(split ? pl.NP : 1, groups, B), dim3(wpb * 64), 0, s, out, w.acc,
                       w.m, w.l, q, k_cache, v_cache, block_table, maxb, context_lens, NB,
                       __builtin_ctz(bs), HQ, HKV, group, scale * kLog2e, split ? pl.P : 0,
                       split ? pl.NP : 1, split ? 1 : 0);
  }
  return check_launch(fn);
}

static int validate_decode(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, int32_t maxb, const int32_t* context_lens,
                           int32_t B, int32_t NB, int32_t bs, int32_t HQ, int32_t HKV, int32_t D,
                           pa_dtype dtype, const void* workspace) {
  int st = validate_common(fn, B, HQ, HKV, D, dtype);
  if (st) return st;
  if (!is_pow2(bs) || bs < 8 || bs > 1024)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d not a power of two in [8,1024]", fn, bs);
  if (maxb <= 0 || NB < 0 || (B > 0 && NB == 0))
    return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq %d, num_blocks %d", fn, maxb, NB);
  if (B == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens)
    return fail(PA_ERR_NULL, "%s: null pointer", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (workspace && !aligned16(workspace)))
    return fail(PA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      head_dim <= 0 || max_context_len <= 0 || partition_size < -1)
    return 0;
  // The chunk length (and so the slice count) depends on the element type: size
  // for the larger of the bf16 and fp32 layouts.
  const DecodePlan a = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, PA_BF16,
                                   max_context_len, partition_size, true);
  const DecodePlan b = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, PA_F32,
                                   max_context_len, partition_size, true);
  return a.ws_bytes > b.ws_bytes ? a.ws_bytes : b.ws_bytes;
}

extern "C" int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                         int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, float scale, pa_dtype dtype,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         void* stream) {
  clear_error();
  int st = validate_decode("pa_decode", q, k_cache, v_cache, block_table, max_blocks_per_seq,
                           context_lens, num_seqs, num_blocks, block_size, num_q_heads,
                           num_kv_heads, head_dim, dtype, workspace);
  if (st || num_seqs == 0) return st;
  if (!out) return fail(PA_ERR_NULL, "pa_decode: null pointer");
  if (!aligned16(out)) return fail(PA_ERR_ALIGN, "pa_decode: pointers must be 16-byte aligned");
  if ((st = validate_partition("pa_decode", partition_size))) return st;
  max_context_len = resolve_max_ctx(max_context_len, max_blocks_per_seq, block_size);
  if (debug_checks() &&
      (st = pa_check_decode_inputs(block_table, max_blocks_per_seq, context_lens, num_seqs,
                                   max_context_len, num_blocks, block_size, stream)))
    return st;
  const DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                                    max_context_len, partition_size, workspace != nullptr);
  const hipStream_t s = (hipStream_t)stream;
  st = launch_decode("pa_decode", pl, out, q, k_cache, v_cache, block_table, max_blocks_per_seq,
                     context_lens, num_seqs, num_blocks, block_size, num_q_heads, num_kv_heads,
                     head_dim, scale, dtype, workspace, workspace_bytes, s);
  if (st || pl.mode == DecodePlan::kSingle) return st;
  return launch_merge(out, pl, carve(workspace, pl, num_seqs, num_q_heads, head_dim), context_lens,
                      num_seqs, num_q_heads, head_dim, dtype, s);
}

extern "C" int pa_decode_partitions(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_table,
                                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t max_context_len, int32_t num_blocks,
                                    int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, float scale, pa_dtype dtype,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  clear_error();
  int st = validate_decode("pa_decode_partitions", q, k_cache, v_cache, block_table,
                           max_blocks_per_seq, context_lens, num_seqs, num_blocks, block_size,
                           num_q_heads, num_kv_heads, head_dim, dtype, workspace);
  if (st || num_seqs == 0) return st;
  if ((st = validate_partition("pa_decode_partitions", partition_size))) return st;
  max_context_len = resolve_max_ctx(max_context_len, max_blocks_per_seq, block_size);
  if (partition_size == -1 || !workspace)
    return fail(PA_ERR_WORKSPACE, "pa_decode_partitions: a split needs a workspace");
  if (debug_checks() &&
      (st = pa_check_decode_inputs(block_table, max_blocks_per_seq, context_lens, num_seqs,
                                   max_context_len, num_blocks, block_size, stream)))
    return st;
  const DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                                    max_context_len, partition_size, true);
  if (pl.mode == DecodePlan::kSingle)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_partitions: partition_size %d does not split "
                "max_context_len %d", partition_size, max_context_len);
  if (pl.mode == DecodePlan::kBalanced && (!out || !aligned16(out)))
    return fail(out ? PA_ERR_ALIGN : PA_ERR_NULL, "pa_decode_partitions: the balanced split "
                "writes unsplit rows to out");
  return launch_decode("pa_decode_partitions", pl, out, q, k_cache, v_cache, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, num_blocks, block_size,
                       num_q_heads, num_kv_heads, head_dim, scale, dtype, workspace,
                       workspace_bytes, (hipStream_t)stream);
}

extern "C" int pa_decode_merge(void* out, const void* workspace, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                               pa_dtype dtype, void* stream) {
  clear_error();
  int st = validate_common("pa_decode_merge", num_seqs, num_q_heads, num_kv_heads, head_dim, dtype);
  if (st) return st;
  if ((st = validate_partition("pa_decode_merge", partition_size))) return st;
  if (max_context_len <= 0 || partition_size == -1)
    return fail(PA_ERR_SHAPE, "pa_decode_merge: max_context_len %d, partition_size %d",
                max_context_len, partition_size);
  if (num_seqs == 0) return PA_OK;
  if (!out || !workspace || !context_lens) return fail(PA_ERR_NULL, "pa_decode_merge: null pointer");
  if (!aligned16(out) || !aligned16(workspace))
    return fail(PA_ERR_ALIGN, "pa_decode_merge: pointers must be 16-byte aligned");
  DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                              max_context_len, partition_size, true);
  if (pl.mode == DecodePlan::kSingle) {  // one partition per sequence
    pl.mode = DecodePlan::kFixed;
    pl.P = max_context_len;
    pl.NP = 1;
  }
  return launch_merge(out, pl, carve(const_cast<void*>(workspace), pl, num_seqs, num_q_heads, head_dim),
                      context_lens, num_seqs, num_q_heads, head_dim, dtype, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// pa_decode_append(_partitions): the store of the step's new K/V rows and the decode in one
// first pass (balanced split), or the store's own launch before it (other plans).

namespace pa {

static int decode_append(const char* fn, bool merge, void* out, const void* q, const void* key,
                         const void* value, int64_t key_token_stride, int64_t value_token_stride,
                         void* k_cache, void* v_cache, const int32_t* block_table, int32_t maxb,
                         const int32_t* context_lens, int32_t B, int32_t max_ctx, int32_t NB,
                         int32_t bs, int32_t HQ, int32_t HKV, int32_t D, float scale,
                         pa_dtype dtype, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream) {
  clear_error();
  int st = validate_decode(fn, q, k_cache, v_cache, block_table, maxb, context_lens, B, NB, bs,
                           HQ, HKV, D, dtype, workspace);
  if (st || B == 0) return st;
  if ((st = validate_partition(fn, partition_size))) return st;
  if (!key || !value) return fail(PA_ERR_NULL, "%s: null new rows", fn);
  if (key_token_stride < (int64_t)HKV * D || value_token_stride < (int64_t)HKV * D)
    return fail(PA_ERR_SHAPE, "%s: token stride smaller than a row", fn);
  const int eb = elt_bytes(dtype);
  if (!aligned16(key) || !aligned16(value) || (key_token_stride * eb) % 16 ||
      (value_token_stride * eb) % 16)
    return fail(PA_ERR_ALIGN, "%s: new rows and their strides must be 16-byte aligned", fn);
  if ((int64_t)NB * bs > INT32_MAX)
    return fail(PA_ERR_SHAPE, "%s: num_blocks*block_size exceeds int32 slots", fn);
  max_ctx = resolve_max_ctx(max_ctx, maxb, bs);
  if (!merge && (partition_size == -1 || !workspace))
    return fail(PA_ERR_WORKSPACE, "%s: a split needs a workspace", fn);
  if (debug_checks() &&
      ((st = pa_check_decode_inputs(block_table, maxb, context_lens, B, max_ctx, NB, bs, stream)) ||
       (st = check_append_slots(block_table, maxb, context_lens, B, NB, bs, (hipStream_t)stream))))
    return st;
  const DecodePlan pl = plan_decode(B, HQ, HKV, D, dtype, max_ctx, partition_size,
                                    !merge || workspace != nullptr);
  if (!merge && pl.mode == DecodePlan::kSingle)
    return fail(PA_ERR_UNSUPPORTED, "%s: partition_size %d does not split max_context_len %d", fn,
                partition_size, max_ctx);
  if ((merge || pl.mode == DecodePlan::kBalanced) && (!out || !aligned16(out)))
    return fail(out ? PA_ERR_ALIGN : PA_ERR_NULL, "%s: out must be a 16-byte aligned pointer", fn);
  const AppendRows ap{static_cast<const char*>(key), static_cast<const char*>(value),
                      key_token_stride * eb, value_token_stride * eb,
                      static_cast<char*>(k_cache), static_cast<char*>(v_cache)};
  // The store goes into the first pass when slices are short: the appending pass costs
  // ~0.05 us more per chunk of a slice, so a batch whose slices are long (the 256-row
  // Qwen3-0.6B decode: 182 chunks, 8.5 us more) is faster with the store's own ~4.6 us
  // launch.  The slice length is bounded as if every sequence held max_ctx keys.
  constexpr int64_t kAppendChunks = 128;
  const int64_t ch = chunk_tokens(D, eb, pl.G);
  const bool fuse = pl.mode == DecodePlan::kBalanced &&
                    ceil_div((int64_t)B * ceil_div(max_ctx, ch), pl.Wt) <= kAppendChunks;
  const hipStream_t s = (hipStream_t)stream;
  st = launch_decode(fn, pl, out, q, k_cache, v_cache, block_table, maxb, context_lens, B, NB, bs,
                     HQ, HKV, D, scale, dtype, workspace, workspace_bytes, s, &ap, fuse);
  if (st || !merge || pl.mode == DecodePlan::kSingle) return st;
  return launch_merge(out, pl, carve(workspace, pl, B, HQ, D), context_lens, B, HQ, D, dtype, s);
}

}  // namespace pa

extern "C" int pa_decode_append(void* out, const void* q, const void* key, const void* value,
                                int64_t key_token_stride, int64_t value_token_stride,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_context_len, int32_t num_blocks,
                                int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, float scale, pa_dtype dtype,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_append("pa_decode_append", true, out, q, key, value, key_token_stride,
                       value_token_stride, k_cache, v_cache, block_table, max_blocks_per_seq,
                       context_lens, num_seqs, max_context_len, num_blocks, block_size,
                       num_q_heads, num_kv_heads, head_dim, scale, dtype, partition_size,
                       workspace, workspace_bytes, stream);
}

extern "C" int pa_decode_append_partitions(
    void* out, const void* q, const void* key, const void* value, int64_t key_token_stride,
    int64_t value_token_stride, void* k_cache, void* v_cache, const int32_t* block_table,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t max_context_len, int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, float scale, pa_dtype dtype, int32_t partition_size,
    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_append("pa_decode_append_partitions", false, out, q, key, value,
                       key_token_stride, value_token_stride, k_cache, v_cache, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_blocks,
                       block_size, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                       partition_size, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// pa_decode_noalloc: pa_decode with its split-K workspace in a fixed array inside the
// library, for callers that cannot allocate.  The array lives in device global memory (one
// copy per device the library runs on, held until the process ends); host code never uses
// its name as an address: each device's address is looked up once, with that device
// current, and kept.

namespace pa {

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];  // per device, filled on the first call there

// The device address of `scratch` on the current device (looked up once per device).
static int scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array: %s", fn,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace pa

extern "C" int pa_decode_noalloc(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* block_table,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_context_len, int32_t num_blocks,
                                 int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float scale, pa_dtype dtype,
                                 int32_t partition_size, void* stream) {
  const char* fn = "pa_decode_noalloc";
  clear_error();
  int st = validate_decode(fn, q, k_cache, v_cache, block_table, max_blocks_per_seq, context_lens,
                           num_seqs, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                           dtype, nullptr);
  if (st || num_seqs == 0) return st;
  if (!out) return fail(PA_ERR_NULL, "%s: null pointer", fn);
  if (!aligned16(out)) return fail(PA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  if ((st = validate_partition(fn, partition_size))) return st;
  max_context_len = resolve_max_ctx(max_context_len, max_blocks_per_seq, block_size);
  // The plan of pa_decode with a workspace; refused before any HIP call when its workspace
  // would not fit in the array.
  const DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                                    max_context_len, partition_size, true);
  if (pl.mode != DecodePlan::kSingle && pl.ws_bytes > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE, "%s: the split needs %zu bytes of scratch, the library's "
                "array holds %d (use pa_decode with a workspace, or partition_size -1)",
                fn, pl.ws_bytes, PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (pl.mode != DecodePlan::kSingle && (st = scratch_on_current_device(fn, &ws))) return st;
  if (debug_checks() &&
      (st = pa_check_decode_inputs(block_table, max_blocks_per_seq, context_lens, num_seqs,
                                   max_context_len, num_blocks, block_size, stream)))
    return st;
  const hipStream_t s = (hipStream_t)stream;
  st = launch_decode(fn, pl, out, q, k_cache, v_cache, block_table, max_blocks_per_seq,
                     context_lens, num_seqs, num_blocks, block_size, num_q_heads, num_kv_heads,
                     head_dim, scale, dtype, ws, PA_NOALLOC_SCRATCH_BYTES, s);
  if (st || pl.mode == DecodePlan::kSingle) return st;
  return launch_merge(out, pl, carve(ws, pl, num_seqs, num_q_heads, head_dim), context_lens,
                      num_seqs, num_q_heads, head_dim, dtype, s);
}
