// a5: varlen chunked-prefill attention over a paged, prefix-cached KV pool (gfx950, bf16 MFMA).
//
// What is computed follows "大模型推理引擎学习入门-2 ... nano-vllm 的 KV Cache 以及 Paged
// Attention" (juejin.cn) section 3.5: a sequence brings seqlen_q = seqlen - num_cached new
// queries and attends seqlen_k = seqlen keys, the cached prefix read from the paged pool
// through block_tables; query i sits at position seqlen_k - seqlen_q + i (the nano-vLLM lab
// manual, appendix B.6) and, causally, sees keys up to that position.
//
// Design (MI355X-specific):
//   grid = (query tile, kv head, sequence), 8 waves (two per SIMD, so one wave's softmax
//   and LDS traffic overlap the other's matrix work).  A workgroup owns 128 query rows: the
//   128/G positions of its tile times the G query heads of one GQA group, so each K/V tile
//   gathered through the block table serves every head that reads it; each wave owns 32
//   rows and one half of every key tile.  Workgroups are renumbered so the query tiles of
//   one (sequence, kv head) run on one XCD and share its L2.
//   Keys go in tiles of 128, loaded global -> LDS directly (no register staging) into two
//   K and two V buffers: a step issues the next tiles' loads first and waits for them only
//   at its end, one barrier per step.  Block ids come from an LDS copy of the block table,
//   never from global memory inside the loop.
//   Both K and V sit in LDS in their natural [key][d] layout.  Each wave computes
//   S^T = K Q^T (16 keys x 16 queries per v_mfma_f32_16x16x32_bf16), so every lane holds
//   scores of a single query: the online softmax needs two cross-lane exchanges per tile
//   and the probabilities already form the B operand of O^T += V^T P^T.  The V^T operand
//   comes from gfx950's transposing LDS load (ds_read_b64_tr_b16): in each 16-lane group,
//   lanes a, a+4, a+8, a+12 address four consecutive keys at the same d offset and lane
//   4a+c receives column c of them.  The running max moves only when it grows by more than
//   kLazyRescale (log2 units), which skips most rescales of the accumulator; the result is
//   unchanged because numerator and denominator share the stale max.
#include "pa_prefill_dev.h"

namespace pa {

template <int D, int G, bool WIDE, int ET>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int total_q,
    int num_blocks, int bs_log2, int HQ, int HKV, float scale_log2, int causal) {
  // Consecutive logical ids (query tiles of one sequence and KV head) share an XCD, so the
  // tiles that read the same K/V rows hit the same L2.
  const int nx = gridDim.x, ny = gridDim.y;
  const int lid = xcd_local_id(blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z), nx * ny * gridDim.z);
  prefill_body<D, G, WIDE, false, ET>(threadIdx.x, lid % nx, (lid / nx) % ny, lid / (nx * ny), out,
                                      q, kc, vc, block_table, maxb, cu_q, cu_k, total_q,
                                      num_blocks, bs_log2, HQ, HKV, scale_log2, causal);
}

typedef void (*prefill_fn)(uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                           const int32_t*, int, const int32_t*, const int32_t*, int, int, int, int,
                           int, float, int);

template <int D, bool WIDE, int ET>
static prefill_fn pick_prefill_g(int G) {
  switch (G) {
    case 1: return prefill_kernel<D, 1, WIDE, ET>;
    case 2: return prefill_kernel<D, 2, WIDE, ET>;
    case 3: return prefill_kernel<D, 3, WIDE, ET>;
    case 4: return prefill_kernel<D, 4, WIDE, ET>;
    case 5: return prefill_kernel<D, 5, WIDE, ET>;
    case 6: return prefill_kernel<D, 6, WIDE, ET>;
    case 7: return prefill_kernel<D, 7, WIDE, ET>;
    case 8: return prefill_kernel<D, 8, WIDE, ET>;
    case 16: return prefill_kernel<D, 16, WIDE, ET>;
  }
  return nullptr;
}

template <int ET>
static prefill_fn pick_prefill(int D, bool wide, int G) {
  if (D == 64) return wide ? pick_prefill_g<64, true, ET>(G) : pick_prefill_g<64, false, ET>(G);
  return wide ? pick_prefill_g<128, true, ET>(G) : pick_prefill_g<128, false, ET>(G);
}

}  // namespace pa

using namespace pa;

extern "C" int pa_prefill_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                float scale, int32_t causal, pa_dtype dtype, void* stream) {
  clear_error();
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: bad sizes");
  if (num_q_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: q_heads %d not a multiple of kv_heads %d",
                num_q_heads, num_kv_heads);
  if (dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: dtype must be PA_BF16 or PA_F16");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: head_dim %d (64 or 128)", head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: block_size %d", block_size);
  if ((int64_t)total_q > (int64_t)num_seqs * max_seqlen_q)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: total_q %d > num_seqs * max_seqlen_q", total_q);
  if (!(scale > 0.0f)) return fail(PA_ERR_SHAPE, "pa_prefill_paged: scale must be > 0");
  if (num_blocks == 0 && total_q > 0)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: empty pool");
  if ((int64_t)block_size * num_kv_heads * head_dim >= (int64_t)1 << 31)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: block of %d x %d x %d elements too large",
                block_size, num_kv_heads, head_dim);
  if (max_seqlen_q > max_seqlen_k)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: max_seqlen_q %d > max_seqlen_k %d", max_seqlen_q,
                max_seqlen_k);
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !cu_seqlens_k)
    return fail(PA_ERR_NULL, "pa_prefill_paged: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_ALIGN, "pa_prefill_paged: pointers must be 16-byte aligned");
  if (debug_checks())
    if (int cs = pa_check_prefill_inputs(block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k,
                                       num_seqs, total_q, max_seqlen_q, max_seqlen_k, num_blocks,
                                       block_size, stream))
      return cs;
  const int G = num_q_heads / num_kv_heads;
  const bool wide = block_size >= kPrefillKeys;
  prefill_fn fn = dtype == PA_F16 ? pick_prefill<PA_F16>(head_dim, wide, G)
                                  : pick_prefill<PA_BF16>(head_dim, wide, G);
  if (!fn) return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: GQA group %d (1-8 or 16)", G);
  const int BM = kPrefillRows / G;
  dim3 grid((max_seqlen_q + BM - 1) / BM, num_kv_heads, num_seqs);
  hipLaunchKernelGGL(fn, grid, dim3(kPrefillThreads), 0, (hipStream_t)stream, (uint16_t*)out,
                     (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                     block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k, total_q, num_blocks,
                     __builtin_ctz(block_size), num_q_heads, num_kv_heads, scale * kLog2e,
                     causal ? 1 : 0);
  return check_launch("pa_prefill_paged");
}
