// Mixed prefill + decode in one launch over a varlen batch (gfx950).
//
// What is computed is the chunked-prefill attention of pa_prefill.hip for every
// sequence of the batch: query i of a sequence with Lq new queries over Lk
// cached + new keys sits at position Lk - Lq + i and attends keys 0 .. Lk-Lq+i
// ("大模型推理引擎学习入门-2 ... nano-vllm 的 KV Cache 以及 Paged Attention", section
// 3.5; the nano-vLLM lab manual, appendix B.6).  A decode row is the case
// Lq = 1, where this is exactly decode over Lk keys ("mini-vLLM v0.4", section
// 5), so one batch can hold prompt chunks and decode rows with no per-batch
// prefill/decode switch.
//
// MI355X design.  One grid of 512-thread workgroups: the first ones run the
// balanced split-K decode body over the sequences with Lq = 1 (each wave one
// (slice, KV-head tile) of the flattened decode keys), the last n_pf (at most one
// per compute unit) walk the list of query tiles of the sequences with Lq > 1
// (MFMA prefill body).  Workgroups are handed out in launch order, so the
// latency-bound prefill tiles take the compute units that the bandwidth-bound
// decode slices free in the decode's tail, and no workgroup is launched for a
// decode row's would-be prefill tile (measured on 256 decode rows + 8 x 256-token
// chunks: 384 us, against 386 us as two launches, 395 us with half the compute
// units on prefill tiles first and 414 us with all of them).  Decode rows cut by
// slice boundaries leave partial states in the workspace; a second small launch
// merges them.
#include "pa_decode_plan.h"
#include "pa_prefill_dev.h"

namespace pa {

constexpr int kMaxMixedSeqs = 4096;  // LDS holds 3 ints per sequence beside the prefill tiles

template <int D, int G, bool WIDE, int ET>
__global__ __launch_bounds__(kPrefillThreads) void mixed_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int total_q, int B,
    int num_blocks, int bs_log2, int HQ, int HKV, float scale_log2, int n_pf,
    float* __restrict__ ws_acc, float* __restrict__ ws_m, float* __restrict__ ws_l,
    int32_t* __restrict__ ws_cuc, int head_waves, int Wt) {
  const int pf_id = (int)blockIdx.x - ((int)gridDim.x - n_pf);  // prefill workers come last
  if (pf_id >= 0) {
    // Prefill workgroups walk a list of the batch's query tiles, built here from cu_q: a
    // sequence with Lq >= 2 has ceil(Lq / BM) tiles per KV head.  Items are numbered
    // sequence, then KV head, then tile, and handed out so that consecutive items run on
    // one XCD (tiles of one sequence and KV head read the same K/V rows through its L2).
    constexpr int BM = kPrefillRows / G;
    // [B + 1] exclusive prefix sums of tiles per sequence.
    extern __shared__ int s_items[];
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int seg = (B + 63) / 64;
      const int lo = min(B, lane * seg), hi = min(B, lo + seg);
      int sum = 0;
      for (int i = lo; i < hi; ++i) {
        const int Lq = cu_q[i + 1] - cu_q[i];
        sum += Lq >= 2 ? (Lq + BM - 1) / BM : 0;
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      int run = incl - sum;
      for (int i = lo; i < hi; ++i) {
        s_items[i] = run;
        const int Lq = cu_q[i + 1] - cu_q[i];
        run += Lq >= 2 ? (Lq + BM - 1) / BM : 0;
      }
      if (lane == 63) s_items[B] = incl;
    }
    __syncthreads();
    const int items = HKV * lds_uniform(s_items + B);
    for (int j = xcd_local_id(pf_id, n_pf); j < items; j += n_pf) {
      int lo = 0, hi = B;  // the sequence: largest b with HKV * s_items[b] <= j
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (HKV * lds_uniform(s_items + mid) <= j) lo = mid;
        else hi = mid;
      }
      const int first = lds_uniform(s_items + lo);
      const int T = lds_uniform(s_items + lo + 1) - first;
      const int r = j - HKV * first;
      prefill_body<D, G, WIDE, true, ET>(r % T, r / T, lo, out, q, kc, vc, block_table, maxb, cu_q,
                                     cu_k, total_q, num_blocks, bs_log2, HQ, HKV, scale_log2, 1);
      __syncthreads();  // the next item reuses this item's LDS
    }
  } else {
    const int i = blockIdx.x;
    const int item = i * (kPrefillThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    decode_balanced_body<D, ET, head_tile(G), true>(
        item / head_waves, item % head_waves, i == 0, out, ws_acc, ws_m, ws_l, ws_cuc, q, kc, vc,
        block_table, maxb, nullptr, cu_q, cu_k, total_q, B, num_blocks, bs_log2, HQ, HKV, G,
        scale_log2, Wt);
  }
}

typedef void (*mixed_fn)(uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                         const int32_t*, int, const int32_t*, const int32_t*, int, int, int, int,
                         int, int, float, int, float*, float*, float*, int32_t*, int, int);

template <int D, bool WIDE, int ET>
static mixed_fn pick_mixed_g(int G) {
  switch (G) {
    case 1: return mixed_kernel<D, 1, WIDE, ET>;
    case 2: return mixed_kernel<D, 2, WIDE, ET>;
    case 3: return mixed_kernel<D, 3, WIDE, ET>;
    case 4: return mixed_kernel<D, 4, WIDE, ET>;
    case 5: return mixed_kernel<D, 5, WIDE, ET>;
    case 6: return mixed_kernel<D, 6, WIDE, ET>;
    case 7: return mixed_kernel<D, 7, WIDE, ET>;
    case 8: return mixed_kernel<D, 8, WIDE, ET>;
    case 16: return mixed_kernel<D, 16, WIDE, ET>;
  }
  return nullptr;
}

template <int ET>
static mixed_fn pick_mixed(int D, bool wide, int G) {
  if (D == 64) return wide ? pick_mixed_g<64, true, ET>(G) : pick_mixed_g<64, false, ET>(G);
  return wide ? pick_mixed_g<128, true, ET>(G) : pick_mixed_g<128, false, ET>(G);
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_seqlen_k) {
  if (num_seqs <= 0 || num_seqs > kMaxMixedSeqs || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0 || max_seqlen_k <= 0)
    return 0;
  return plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, PA_BF16, max_seqlen_k, 0, true)
      .ws_bytes;
}

extern "C" int pa_attention_mixed(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t num_blocks,
                                  int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, float scale, pa_dtype dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  clear_error();
  const char* fn = "pa_attention_mixed";
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "%s: q_heads %d not a multiple of kv_heads %d", fn, num_q_heads,
                num_kv_heads);
  if (dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype must be PA_BF16 or PA_F16", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
  if ((int64_t)block_size * num_kv_heads * head_dim >= (int64_t)1 << 31)
    return fail(PA_ERR_UNSUPPORTED, "%s: block of %d x %d x %d elements too large", fn, block_size,
                num_kv_heads, head_dim);
  if (num_seqs > kMaxMixedSeqs)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d sequences (at most %d)", fn, num_seqs, kMaxMixedSeqs);
  if ((int64_t)total_q > (int64_t)num_seqs * max_seqlen_q)
    return fail(PA_ERR_SHAPE, "%s: total_q %d > num_seqs * max_seqlen_q", fn, total_q);
  if (max_seqlen_q > max_seqlen_k)
    return fail(PA_ERR_SHAPE, "%s: max_seqlen_q %d > max_seqlen_k %d", fn, max_seqlen_q,
                max_seqlen_k);
  if (!(scale > 0.0f)) return fail(PA_ERR_SHAPE, "%s: scale must be > 0", fn);
  if (num_blocks == 0 && total_q > 0) return fail(PA_ERR_SHAPE, "%s: empty pool", fn);
  const int G = num_q_heads / num_kv_heads;
  if (G > 8 && G != 16) return fail(PA_ERR_UNSUPPORTED, "%s: GQA group %d (1-8 or 16)", fn, G);
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !cu_seqlens_k)
    return fail(PA_ERR_NULL, "%s: null pointer", fn);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (workspace && !aligned16(workspace)))
    return fail(PA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  const DecodePlan pl = plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, dtype,
                                    max_seqlen_k > 0 ? max_seqlen_k : 1, 0, true);
  if (!workspace || workspace_bytes < pl.ws_bytes)
    return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes,
                pl.ws_bytes);
  if (debug_checks())
    if (int cs = pa_check_prefill_inputs(block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k,
                                       num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_blocks,
                                       block_size, stream))
      return cs;

  const bool wide = block_size >= kPrefillKeys;
  mixed_fn kern = dtype == PA_F16 ? pick_mixed<PA_F16>(head_dim, wide, G)
                                  : pick_mixed<PA_BF16>(head_dim, wide, G);
  // Prefill workgroups: at most one per compute unit, each looping over the tile list;
  // fewer when the batch cannot hold that many tiles (sum over prefill sequences of
  // ceil(Lq / BM) <= total_q / BM + number of such sequences).
  const int BM = kPrefillRows / G;
  int64_t n_pf = 0;
  if (max_seqlen_q > 1) {
    const int64_t seqs = num_seqs < total_q / 2 ? num_seqs : total_q / 2;
    int64_t tiles = total_q / BM + seqs;
    const int64_t by_len = (int64_t)num_seqs * ((max_seqlen_q + BM - 1) / BM);
    tiles = tiles < by_len ? tiles : by_len;
    n_pf = tiles * num_kv_heads;
    n_pf = n_pf < kNumCUs ? n_pf : kNumCUs;
  }
  const int head_waves = num_kv_heads * (G / head_tile(G));
  const int64_t n_dec = ceil_div((int64_t)pl.Wt * head_waves, kPrefillThreads / 64);
  if (n_pf + n_dec > INT32_MAX) return fail(PA_ERR_SHAPE, "%s: grid too large", fn);
  const WsPtrs w = carve(workspace, pl, num_seqs, num_q_heads, head_dim);
  const hipStream_t s = (hipStream_t)stream;
  const size_t lds = (size_t)(3 * num_seqs + 1) * sizeof(int);
  hipLaunchKernelGGL(kern, dim3((unsigned)(n_pf + n_dec)), dim3(kPrefillThreads), lds, s,
                     (uint16_t*)out, (const uint16_t*)q, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, block_table, max_blocks_per_seq, cu_seqlens_q,
                     cu_seqlens_k, total_q, num_seqs, num_blocks, __builtin_ctz(block_size),
                     num_q_heads, num_kv_heads, scale * kLog2e, (int)n_pf, w.acc, w.m, w.l,
                     w.cuc, head_waves, pl.Wt);
  int st = check_launch(fn);
  if (st) return st;
  // Pieces per decode row: at most one more than the slices per sequence.
  const int W = merge_waves((pl.Wt + num_seqs - 1) / num_seqs + 1);
  const dim3 mgrid(num_q_heads, num_seqs);
#define PA_MIXED_MERGE(ET, WV)                                                              \
  hipLaunchKernelGGL((merge_balanced_kernel<ET, true, WV>), mgrid, dim3(64 * WV), 0, s, out, \
                     w.acc, w.m, w.l, w.cuc, cu_seqlens_q, total_q, num_seqs, num_q_heads,  \
                     head_dim, pl.Wt)
  if (dtype == PA_F16) {
    if (W == 1) PA_MIXED_MERGE(PA_F16, 1);
    else PA_MIXED_MERGE(PA_F16, kMergeWaves);
  } else {
    if (W == 1) PA_MIXED_MERGE(PA_BF16, 1);
    else PA_MIXED_MERGE(PA_BF16, kMergeWaves);
  }
#undef PA_MIXED_MERGE
  return check_launch("pa_attention_mixed merge");
}
