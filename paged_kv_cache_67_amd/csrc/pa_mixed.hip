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
// MI355X design.  One grid of at most one 512-thread workgroup per compute unit (the
// prefill tiles' LDS allows no more), all resident at once.  Every workgroup first scans
// the batch's lengths (the decode chunk table of the balanced split, and the totals of
// decode keys and prefill query-key pairs) and from those totals picks, with the same
// arithmetic in every workgroup, how many workgroups take each side: the first ones run
// the balanced split-K decode body over the sequences with Lq = 1 (each wave one (slice,
// KV-head tile) of the flattened decode keys), the last n_pf walk the list of query tiles
// of the sequences with Lq > 1 (MFMA prefill body).  The decode rows are bound by HBM and
// reach its bandwidth on about 160-192 compute units; the prefill tiles are bound by the
// matrix cores and LDS of their own compute unit and read little, so the two sides run
// side by side and the step takes about the longer of the two instead of their sum.  The
// split minimises the larger of the two modelled times (decode bytes over the measured
// bandwidth of that many workgroups, rounds of prefill tiles times the mean tile's flops
// over a workgroup's rate).  Decode rows cut by slice boundaries leave partial states in the
// workspace; a second small launch merges them.
#include <algorithm>
#include <mutex>
#include <unordered_set>

#include "pa_decode_plan.h"
#include "pa_prefill_dev.h"

namespace pa {

// Rates of the split's cost model, measured on MI355X with the 256-row Qwen3-0.6B decode
// batch beside 8 prompt chunks and a fixed number of decode workgroups: decode K/V bytes
// per ns reached by n decode workgroups (eight waves each; linear between the points,
// flat past the last), taken at 90% while prefill tiles run beside them (the heavier
// mixes measured so); and flops per ns of one prefill workgroup (the prefill kernel's
// 540 TFLOP/s over 256 workgroups).
constexpr int kDecCurveN = 7;
__device__ constexpr float kDecCurveWGs[kDecCurveN] = {0, 96, 128, 144, 160, 176, 192};
__device__ constexpr float kDecCurveBytesPerNs[kDecCurveN] = {0, 4530, 5540, 5900, 6210, 6360, 6450};
constexpr float kDecBesidePrefill = 0.9f;
constexpr float kPfFlopsPerNsWG = 2100.0f;

__device__ __forceinline__ float decode_bytes_per_ns(float n) {
  float r = kDecCurveBytesPerNs[kDecCurveN - 1];
#pragma unroll
  for (int k = kDecCurveN - 1; k >= 1; --k)
    if (n <= kDecCurveWGs[k])
      r = kDecCurveBytesPerNs[k - 1] + (n - kDecCurveWGs[k - 1]) *
                                           (kDecCurveBytesPerNs[k] - kDecCurveBytesPerNs[k - 1]) /
                                           (kDecCurveWGs[k] - kDecCurveWGs[k - 1]);
  return kDecBesidePrefill * r;
}

constexpr int kMaxLdsBytes = 160 * 1024;  // LDS one workgroup may hold (gfx950)
// Dynamic LDS of a mixed workgroup: the split (4 ints), then the decode tables
// (3 * num_seqs + 1 ints; the prefill side reuses their first num_seqs + 1 for its tile scan).
inline size_t mixed_dyn_lds(int B) { return (size_t)(3 * B + 5) * sizeof(int); }
// The most sequences a mixed launch takes at head size D: the dynamic LDS beside the
// prefill body's static LDS stays within one workgroup's LDS.
constexpr int mixed_max_seqs(int D) {
  const int by_lds = ((kMaxLdsBytes - prefill_lds_bytes(D)) / (int)sizeof(int) - 5) / 3;
  return by_lds < kMaxBalancedSeqs ? by_lds : kMaxBalancedSeqs;
}

// Query heads per decode wave in a mixed launch: as in pa_decode, except that groups of 8
// and 16 take tiles of 4 heads.  An 8-head tile wants more than the 256 VGPRs a wave of a
// 512-thread workgroup may hold (pa_decode runs it in 256-thread workgroups); two 4-head
// waves of one KV head read the same K/V rows at about the same time, so the second read
// is served by the L2.
__host__ __device__ constexpr int mixed_head_tile(int G) { return G >= 8 ? 4 : head_tile(G); }

template <int D, int G, bool WIDE, int ET>
__global__ __launch_bounds__(kPrefillThreads) void mixed_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int total_q, int B,
    int num_blocks, int bs_log2, int HQ, int HKV, float scale_log2,
    float* __restrict__ ws_acc, float* __restrict__ ws_m, float* __restrict__ ws_l,
    int32_t* __restrict__ ws_cuc, int head_waves, int Wt_max, int dec_wgs_max) {
  constexpr int GT = mixed_head_tile(G);
  constexpr int CH = DecodeWave<D, ET, GT>::CH;
  constexpr int BM = kPrefillRows / G;
  constexpr int WAVES = kPrefillThreads / 64;
  extern __shared__ int s_dyn[];
  int* s_split = s_dyn;    // [0]: prefill workgroups
  int* s_mem = s_dyn + 4;  // decode tables, later the prefill tile scan
  const int n_wg = gridDim.x;
  const int i = blockIdx.x;

  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int tiles = 0;
    float pairs = 0.0f, dec_keys = 0.0f;
    const int dec_chunks = balanced_scan<CH, true>(
        s_mem, nullptr, cu_q, cu_k, total_q, B, [&](int nq, int nk, int L) {
          dec_keys += (float)L;
          if (nq >= 2) {  // causal query-key pairs of a chunk of nq queries over nk keys
            const float fq = (float)nq;
            tiles += (nq + BM - 1) / BM;
            pairs += fq * (float)(nk - nq) + 0.5f * fq * (fq + 1.0f);
          }
        });
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      tiles += __shfl_xor(tiles, o);
      pairs += __shfl_xor(pairs, o);
      dec_keys += __shfl_xor(dec_keys, o);
    }
    const int items = tiles * HKV;
    int n_pf;
    if (items == 0) {
      n_pf = 0;
    } else if (dec_chunks == 0) {
      n_pf = n_wg;
    } else {
      // Candidates: n_pf in [lo, hi], multiples of 8 on a full chip (each XCD then holds
      // the same share of both sides); each lane prices some, the cheapest wins (ties to
      // more prefill workgroups: equal modelled rounds of tiles run shorter on more of them).
      const int min_dec = (head_waves + WAVES - 1) / WAVES;
      const int lo = max(1, n_wg - dec_wgs_max), hi = n_wg - min_dec;
      const int step = n_wg >= 64 ? 8 : 1;
      const float dec_bytes = dec_keys * (float)(HKV * D * 2 * elt_bytes((pa_dtype)ET));
      const float tile_ns = pairs * (float)(HQ * D * 4) / (float)items / kPfFlopsPerNsWG;
      float best_t = __builtin_huge_valf();
      int best_n = lo;
      for (int c = (lo + step - 1) / step * step + lane * step; c <= hi; c += 64 * step) {
        const int nd = min(n_wg - c, dec_wgs_max);
        const float t_dec = dec_bytes / decode_bytes_per_ns((float)nd);
        const float t_pf = (float)((items + c - 1) / c) * tile_ns;
        const float t = fmaxf(t_dec, t_pf);
        if (t <= best_t) {
          best_t = t;
          best_n = c;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ot = __shfl_xor(best_t, o);
        const int on = __shfl_xor(best_n, o);
        if (ot < best_t || (ot == best_t && on > best_n)) {
          best_t = ot;
          best_n = on;
        }
      }
      n_pf = best_n;
#ifdef PA_MIXED_PF_WGS  // calibration builds: a fixed prefill share
      n_pf = min(max(PA_MIXED_PF_WGS, lo), hi);
#endif
    }
    if (lane == 0) s_split[0] = n_pf;
  }
  __syncthreads();
  const int n_pf = lds_uniform(s_split);
  const int n_dec = min(n_wg - n_pf, dec_wgs_max);
  // Slices per head wave of the decode side (n_dec * WAVES >= head_waves whenever there
  // are decode keys, so every head wave has a slice).
  const int Wt = max(1, min(Wt_max, n_dec * WAVES / head_waves));
  if (i == 0) {  // the chunk scan and slice count for the merge
    for (int k = threadIdx.x; k <= B; k += blockDim.x) ws_cuc[k] = s_mem[k];
    if (threadIdx.x == 0) ws_cuc[B + 1] = Wt;
  }

  if (i >= n_wg - n_pf) {
    // Prefill workgroups walk a list of the batch's query tiles: a sequence with Lq >= 2
    // has ceil(Lq / BM) tiles per KV head.  Items are numbered sequence, then KV head, then
    // tile, and handed out so that consecutive items run on one XCD (tiles of one sequence
    // and KV head read the same K/V rows through its L2).
    const int pf_id = i - (n_wg - n_pf);
    int* s_items = s_mem;  // [B + 1] exclusive prefix sums of tiles per sequence
    __syncthreads();       // the decode tables are no longer read
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int seg = (B + 63) / 64;
      const int lo = min(B, lane * seg), hi = min(B, lo + seg);
      int sum = 0;
      for (int k = lo; k < hi; ++k) {
        const int Lq = cu_q[k + 1] - cu_q[k];
        sum += Lq >= 2 ? (Lq + BM - 1) / BM : 0;
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      int run = incl - sum;
      for (int k = lo; k < hi; ++k) {
        s_items[k] = run;
        const int Lq = cu_q[k + 1] - cu_q[k];
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
      // The thread index passes through an empty asm so that the body's lane-dependent
      // setup is redone per item instead of being hoisted out of the loop (it would then
      // stay live across every item and spill).
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      prefill_body<D, G, WIDE, true, ET>(tid, r % T, r / T, lo, out, q, kc, vc, block_table, maxb,
                                         cu_q, cu_k, total_q, num_blocks, bs_log2, HQ, HKV,
                                         scale_log2, 1);
      __syncthreads();  // the next item reuses this item's LDS
    }
  } else if (i < n_dec) {
    const int item = i * WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    decode_balanced_run<D, ET, GT, true>(s_mem, item / head_waves, item % head_waves, false, out,
                                         ws_acc, ws_m, ws_l, ws_cuc, q, kc, vc, block_table, maxb,
                                         B, num_blocks, bs_log2, HQ, HKV, G, scale_log2, Wt);
  }
}

typedef void (*mixed_fn)(uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                         const int32_t*, int, const int32_t*, const int32_t*, int, int, int, int,
                         int, int, float, float*, float*, float*, int32_t*, int, int, int);

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

// The launch's LDS (static + dynamic) stays within a workgroup's only if the kernel's
// static LDS is the prefill body's, as mixed_max_seqs assumes; checked once per kernel.
static int check_static_lds(const void* kern, int D, const char* fn) {
  static std::mutex mu;
  static std::unordered_set<const void*> ok;
  std::lock_guard<std::mutex> lock(mu);
  if (ok.count(kern)) return PA_OK;
  hipFuncAttributes a;
  if (hipFuncGetAttributes(&a, kern) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: hipFuncGetAttributes failed", fn);
  if (a.sharedSizeBytes != (size_t)prefill_lds_bytes(D))
    return fail(PA_ERR_HIP, "%s: kernel holds %zu bytes of static LDS, expected %d", fn,
                a.sharedSizeBytes, prefill_lds_bytes(D));
  ok.insert(kern);
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim,
                                          int32_t max_seqlen_k) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads ||
      (head_dim != 64 && head_dim != 128) || num_seqs > mixed_max_seqs(head_dim) ||
      max_seqlen_k <= 0)
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
  if (num_seqs > mixed_max_seqs(head_dim))
    return fail(PA_ERR_UNSUPPORTED, "%s: %d sequences (at most %d at head_dim %d)", fn, num_seqs,
                mixed_max_seqs(head_dim), head_dim);
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
  if (int st = check_static_lds(reinterpret_cast<const void*>(kern), head_dim, fn)) return st;
  // Workgroups: up to one per compute unit.  The decode side has at most the balanced
  // split's own count (its slices times head waves, 8 waves a workgroup); the prefill side
  // at most one per tile the batch can hold (sum over prefill sequences of ceil(Lq / BM)
  // <= total_q / BM + number of such sequences).  The kernel divides them.
  const int BM = kPrefillRows / G;
  int64_t pf_wgs = 0;
  if (max_seqlen_q > 1) {
    const int64_t seqs = num_seqs < total_q / 2 ? num_seqs : total_q / 2;
    int64_t tiles = total_q / BM + seqs;
    const int64_t by_len = (int64_t)num_seqs * ((max_seqlen_q + BM - 1) / BM);
    tiles = tiles < by_len ? tiles : by_len;
    pf_wgs = tiles * num_kv_heads;
    pf_wgs = pf_wgs < kNumCUs ? pf_wgs : kNumCUs;
  }
  constexpr int kWaves = kPrefillThreads / 64;
  const int head_waves = num_kv_heads * (G / mixed_head_tile(G));
  // The balanced split's wave count (as pa_decode plans it), and at least one slice.
  const int64_t dec_wgs = std::max(ceil_div((int64_t)pl.Wt * num_kv_heads * (G / pl.G), kWaves),
                                   ceil_div(head_waves, kWaves));
  const int64_t n_wg = dec_wgs + pf_wgs < kNumCUs ? dec_wgs + pf_wgs : kNumCUs;
  if (dec_wgs > INT32_MAX) return fail(PA_ERR_SHAPE, "%s: grid too large", fn);
  const WsPtrs w = carve(workspace, pl, num_seqs, num_q_heads, head_dim);
  const hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(kern, dim3((unsigned)n_wg), dim3(kPrefillThreads), mixed_dyn_lds(num_seqs), s,
                     (uint16_t*)out, (const uint16_t*)q, (const uint16_t*)k_cache,
                     (const uint16_t*)v_cache, block_table, max_blocks_per_seq, cu_seqlens_q,
                     cu_seqlens_k, total_q, num_seqs, num_blocks, __builtin_ctz(block_size),
                     num_q_heads, num_kv_heads, scale * kLog2e, w.acc, w.m, w.l, w.cuc,
                     head_waves, pl.Wt, (int)dec_wgs);
  int st = check_launch(fn);
  if (st) return st;
  // Pieces per decode row: about one more than the mean slices per sequence.
  const int W = merge_waves((pl.Wt + num_seqs - 1) / num_seqs + 1,
                            (int64_t)num_q_heads * num_seqs);
  const dim3 mgrid(num_q_heads, num_seqs);
#define PA_MIXED_MERGE(ET, WV)                                                              \
  hipLaunchKernelGGL((merge_balanced_kernel<ET, true, WV>), mgrid, dim3(64 * WV), 0, s, out, \
                     w.acc, w.m, w.l, w.cuc, cu_seqlens_q, total_q, num_seqs, num_q_heads,  \
                     head_dim, pl.Wt)
#define PA_MIXED_MERGE1(ET)                                                                  \
  hipLaunchKernelGGL((merge_balanced_kernel<ET, true, 1, kMergeHeadsPerWG>),                 \
                     dim3((num_q_heads + kMergeHeadsPerWG - 1) / kMergeHeadsPerWG, num_seqs), \
                     dim3(64 * kMergeHeadsPerWG), 0, s, out, w.acc, w.m, w.l, w.cuc,          \
                     cu_seqlens_q, total_q, num_seqs, num_q_heads, head_dim, pl.Wt)
  if (dtype == PA_F16) {
    if (W == 1) PA_MIXED_MERGE1(PA_F16);
    else if (W == 2) PA_MIXED_MERGE(PA_F16, 2);
    else if (W == 4) PA_MIXED_MERGE(PA_F16, 4);
    else PA_MIXED_MERGE(PA_F16, kMergeWaves);
  } else {
    if (W == 1) PA_MIXED_MERGE1(PA_BF16);
    else if (W == 2) PA_MIXED_MERGE(PA_BF16, 2);
    else if (W == 4) PA_MIXED_MERGE(PA_BF16, 4);
    else PA_MIXED_MERGE(PA_BF16, kMergeWaves);
  }
#undef PA_MIXED_MERGE
#undef PA_MIXED_MERGE1
  return check_launch("pa_attention_mixed merge");
}
