// a5: varlen chunked-prefill attention over a paged, prefix-cached KV pool (gfx950, bf16 MFMA).
//
// What is computed follows "大模型推理引擎学习入门-2 ... nano-vllm 的 KV Cache 以及 Paged
// Attention" (juejin.cn) section 3.5: a sequence brings seqlen_q = seqlen - num_cached new
// queries and attends seqlen_k = seqlen keys, the cached prefix read from the paged pool
// through block_tables; query i sits at position seqlen_k - seqlen_q + i (the nano-vLLM lab
// manual, appendix B.6) and, causally, sees keys up to that position.
//
// Design (MI355X-specific):
//   grid = (query tile, kv head, sequence), 4 waves.  A workgroup owns 128 query rows: the
//   128/G positions of its tile times the G query heads of one GQA group, so each K/V tile
//   gathered through the block table serves every head that reads it.
//   Per 64-key tile: K rows are copied into LDS as they are; V is written into LDS
//   transposed (d-major) so that keys are the contiguous operand dimension of the second
//   product.  Each wave computes S^T = K Q^T (32 keys x 32 queries per
//   v_mfma_f32_32x32x16_bf16), so every lane ends up holding scores of a single query;
//   the online softmax then needs one cross-lane exchange (lane ^ 32) per tile, and the
//   probabilities are already laid out as the B operand of O^T += V^T P^T.
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPrefillRows = 128;  // query rows (position x head) per workgroup
constexpr int kPrefillKeys = 64;   // keys per tile

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(256) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int total_q,
    int num_blocks, int bs_log2, int HQ, int HKV, float scale_log2, int causal) {
  constexpr int BM = kPrefillRows / G;  // positions per workgroup
  constexpr int BN = kPrefillKeys;
  constexpr int KP = D + 8;   // padded K row (bf16 elements)
  constexpr int VP = BN + 8;  // padded V^T row
  constexpr int DS = D / 16;  // 16-wide d steps of S^T
  constexpr int DB = D / 32;  // 32-wide d blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VP];
  __shared__ int s_bad;

  const int qt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int q0 = cu_q[b];
  const int Lq = cu_q[b + 1] - q0;
  const int Lk = cu_k[b + 1] - cu_k[b];
  const int pos0 = qt * BM;
  if (pos0 >= Lq) return;
  const int npos = min(BM, Lq - pos0);
  const int prefix = Lk - Lq;
  const int nk = causal ? min(Lk, prefix + pos0 + npos) : Lk;  // keys any row of this tile sees

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, hl = lane >> 5;
  const int row = 32 * w + col;
  const int rpos = row / G, rhead = row % G;
  const int64_t qtok = (int64_t)q0 + pos0 + rpos;
  const bool rvalid = row < BM * G && rpos < npos && qtok >= 0 && qtok < total_q;
  const int h = g * G + rhead;
  const int row_nk = (causal && rvalid) ? prefix + pos0 + rpos + 1 : nk;
  const int bs_mask = (1 << bs_log2) - 1;

  if (tid == 0) s_bad = 0;
  __syncthreads();

  // B operand of S^T: this lane's query, d = 16*ds + 8*hl + 0..7.
  bf16x8_t qreg[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rvalid) v = *reinterpret_cast<const uint4*>(q + (qtok * HQ + h) * D + 16 * ds + 8 * hl);
    qreg[ds] = __builtin_bit_cast(bf16x8_t, v);
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const int32_t* bt = block_table + (int64_t)b * maxb;

  for (int kt = 0; kt < nk; kt += BN) {
    // Gather the K/V tile through the block table (16 bytes per thread per step).
    for (int c = tid; c < BN * D / 8; c += 256) {
      const int kr = c / (D / 8), dc = (c % (D / 8)) * 8;
      const int j = kt + kr;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (j < nk) {
        const int jb = j >> bs_log2;
        const int blk = jb < maxb ? bt[jb] : -1;
        if (blk >= 0 && blk < num_blocks) {
          const int64_t off = ((((int64_t)blk << bs_log2) + (j & bs_mask)) * HKV + g) * D + dc;
          kv = *reinterpret_cast<const uint4*>(kc + off);
          vv = *reinterpret_cast<const uint4*>(vc + off);
        } else {
          s_bad = 1;
        }
      }
      *reinterpret_cast<uint4*>(&sK[kr * KP + dc]) = kv;
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[(dc + 2 * e) * VP + kr] = uint16_t(vw[e] & 0xffffu);
        sVt[(dc + 2 * e + 1) * VP + kr] = uint16_t(vw[e] >> 16);
      }
    }
    __syncthreads();

    // S^T = K Q^T for the two 32-key halves of the tile.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(&sK[(kb * 32 + col) * KP + 16 * ds + 8 * hl]);
        s[kb] = mfma32(a, qreg[ds], s[kb]);
      }
    }

    // Online softmax for this lane's query; key of s[kb][i] = kt + 32kb + 8(i/4) + 4hl + i%4.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kt + 32 * kb + 8 * (i >> 2) + 4 * hl + (i & 3);
        const float v = key < row_nk ? s[kb][i] * scale_log2 : -INFINITY;
        s[kb][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m, mx);
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = fast_exp2(m - msafe);
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(s[kb][i] - msafe);
        s[kb][i] = p;
        rs += p;
      }
    l = l * alpha + rs;
    m = mnew;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

    // O^T += V^T P^T, 16 keys per step: MFMA k index (hl, i) is key 16ks + 8(i/4) + 4hl + i%4.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (__bf16)s[ks >> 1][8 * (ks & 1) + i];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = &sVt[(32 * db + col) * VP + 16 * ks + 4 * hl];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[db] = mfma32(a, pb, o[db]);
      }
    }
    __syncthreads();
  }

  // Epilogue: the two lanes of a query each summed half of its keys.
  l += __shfl_xor(l, 32);
  const float inv = s_bad ? NAN : 1.0f / l;
  if (!rvalid) return;
  uint16_t* dst = out + (qtok * HQ + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * db + 8 * a4 + 4 * hl;
      uint2 pk;
      pk.x = uint32_t(f32_to_bf16(o[db][4 * a4 + 0] * inv)) |
             (uint32_t(f32_to_bf16(o[db][4 * a4 + 1] * inv)) << 16);
      pk.y = uint32_t(f32_to_bf16(o[db][4 * a4 + 2] * inv)) |
             (uint32_t(f32_to_bf16(o[db][4 * a4 + 3] * inv)) << 16);
      *reinterpret_cast<uint2*>(dst + d) = pk;
    }
}

typedef void (*prefill_fn)(uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                           const int32_t*, int, const int32_t*, const int32_t*, int, int, int, int,
                           int, float, int);

template <int D>
static prefill_fn pick_prefill_g(int G) {
  switch (G) {
    case 1: return prefill_kernel<D, 1>;
    case 2: return prefill_kernel<D, 2>;
    case 3: return prefill_kernel<D, 3>;
    case 4: return prefill_kernel<D, 4>;
    case 5: return prefill_kernel<D, 5>;
    case 6: return prefill_kernel<D, 6>;
    case 7: return prefill_kernel<D, 7>;
    case 8: return prefill_kernel<D, 8>;
    case 16: return prefill_kernel<D, 16>;
  }
  return nullptr;
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
  if (dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: dtype must be PA_BF16");
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: head_dim %d (64 or 128)", head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: block_size %d", block_size);
  if ((int64_t)total_q > (int64_t)num_seqs * max_seqlen_q)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: total_q %d > num_seqs * max_seqlen_q", total_q);
  if (max_seqlen_q > max_seqlen_k)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: max_seqlen_q %d > max_seqlen_k %d", max_seqlen_q,
                max_seqlen_k);
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !cu_seqlens_k)
    return fail(PA_ERR_NULL, "pa_prefill_paged: null pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_ALIGN, "pa_prefill_paged: pointers must be 16-byte aligned");
  const int G = num_q_heads / num_kv_heads;
  prefill_fn fn = head_dim == 64 ? pick_prefill_g<64>(G) : pick_prefill_g<128>(G);
  if (!fn) return fail(PA_ERR_UNSUPPORTED, "pa_prefill_paged: GQA group %d (1-8 or 16)", G);
  const int BM = kPrefillRows / G;
  dim3 grid((max_seqlen_q + BM - 1) / BM, num_kv_heads, num_seqs);
  hipLaunchKernelGGL(fn, grid, dim3(256), 0, (hipStream_t)stream, (uint16_t*)out,
                     (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                     block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k, total_q, num_blocks,
                     __builtin_ctz(block_size), num_q_heads, num_kv_heads, scale * kLog2e,
                     causal ? 1 : 0);
  return check_launch("pa_prefill_paged");
}
