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
//   gathered through the block table serves every head that reads it; each wave owns 16
//   rows.  Workgroups are renumbered so the query tiles of one (sequence, kv head) run on
//   one XCD and share its L2.
//   Keys go in tiles of 64 through two LDS buffers and two register sets: a tile's global
//   loads are issued two iterations before its LDS store, one barrier per tile.  Block ids
//   come from an LDS copy of the block table, never from global memory inside the loop.
//   Both K and V sit in LDS in their natural [key][d] layout.  Each wave computes
//   S^T = K Q^T (16 keys x 16 queries per v_mfma_f32_16x16x32_bf16), so every lane holds
//   scores of a single query: the online softmax needs two cross-lane exchanges per tile
//   and the probabilities already form the B operand of O^T += V^T P^T.  The V^T operand
//   comes from gfx950's transposing LDS load (ds_read_b64_tr_b16): in each 16-lane group,
//   lanes a, a+4, a+8, a+12 address four consecutive keys at the same d offset and lane
//   4a+c receives column c of them.  The running max moves only when it grows by more than
//   kLazyRescale (log2 units), which skips most rescales of the accumulator; the result is
//   unchanged because numerator and denominator share the stale max.
#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte register chunk

constexpr int kPrefillRows = 128;     // query rows (position x head) per workgroup
constexpr int kPrefillKeys = 64;      // keys per tile
constexpr int kPrefillThreads = 512;  // 8 waves of 16 rows
constexpr int kBtCache = 2048;        // block-table entries of one sequence kept in LDS
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is moved

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 layouts (k index written as (group, i), group = lane / 16):
//   A[m][k]: lane holds m = lane % 16, k = (group, i = 0..7); B[k][n]: n = lane % 16;
//   C/D[m][n]: lane holds m = 4 * group + i (i = 0..3), n = lane % 16.
// S^T = K Q^T per 16-key block kb: lane holds the scores of query lane%16 for keys
// 16kb + 4*group + i.  For O^T += V^T P^T over 32 keys (step ks), the MFMA k index
// (group, i) stands for key 32ks + 16*(i/4) + 4*group + i%4 on both operands: P comes
// straight from S^T blocks 2ks and 2ks+1, V^T from two transposing LDS reads.
template <int D, int G>
__global__ __launch_bounds__(kPrefillThreads) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int total_q,
    int num_blocks, int bs_log2, int HQ, int HKV, float scale_log2, int causal) {
  constexpr int BM = kPrefillRows / G;  // positions per workgroup
  constexpr int BN = kPrefillKeys;
  constexpr int NT = kPrefillThreads;
  constexpr int KP = D + 8;    // K row pitch (bf16): 68 words for D=128
  constexpr int VP = D + 16;   // V row pitch (bf16): 72 words for D=128
  constexpr int DS = D / 32;   // 32-wide d steps of S^T
  constexpr int DB = D / 16;   // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int LPT = BN * CPR / NT;  // 16-byte loads per thread per tile (K and V each)
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][BN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][BN * VP];
  __shared__ int s_bt[kBtCache];
  __shared__ int s_bad;

  // Consecutive logical ids (query tiles of one sequence and KV head) share an XCD, so the
  // tiles that read the same K/V rows hit the same L2.
  const int nx = gridDim.x, ny = gridDim.y;
  const int lid = xcd_local_id(blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z), nx * ny * gridDim.z);
  const int qt = lid % nx, g = (lid / nx) % ny, b = lid / (nx * ny);
  const int q0 = cu_q[b];
  const int Lq = cu_q[b + 1] - q0;
  const int Lk = cu_k[b + 1] - cu_k[b];
  const int pos0 = qt * BM;
  if (pos0 >= Lq) return;
  const int npos = min(BM, Lq - pos0);
  const int prefix = Lk - Lq;
  const int nk = causal ? min(Lk, prefix + pos0 + npos) : Lk;
  const int ntiles = nk > 0 ? (nk + BN - 1) / BN : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int qc = lane & 15, grp = lane >> 4;
  const int row = 16 * w + qc;
  const int rpos = row / G, rhead = row % G;
  const int64_t qtok = (int64_t)q0 + pos0 + rpos;
  const bool rvalid = row < BM * G && rpos < npos && qtok >= 0 && qtok < total_q;
  const int h = g * G + rhead;
  const int row_nk = (causal && rvalid) ? prefix + pos0 + rpos + 1 : nk;
  const int nk_min = causal ? min(nk, prefix + pos0 + 1) : nk;
  const int bs_mask = (1 << bs_log2) - 1;
  const int32_t* bt = block_table + (int64_t)b * maxb;

  // s_bt[i] caches block-table entry btb + i for i < min(nblk - btb, kBtCache).  Block ids
  // are read only from LDS inside the key loop: a global read there would make each tile's
  // address computation wait for every K/V load still in flight.
  const int nblk = min(nk > 0 ? ((nk - 1) >> bs_log2) + 1 : 0, maxb);
  int btb = 0;
  for (int i = tid; i < min(nblk, kBtCache); i += NT) s_bt[i] = bt[i];
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // Slides the window to start at the block of key kt when the keys [kt, kt + BN) run past
  // it.  Called with the same kt by every thread (it holds barriers); rare: once per
  // kBtCache blocks.
  auto cover = [&](int kt) __attribute__((always_inline)) {
    if (((min(kt + BN, nk) - 1) >> bs_log2) >= btb + kBtCache) {
      __syncthreads();
      btb = min(kt, nk - 1) >> bs_log2;
      for (int i = tid; i < min(nblk - btb, kBtCache); i += NT) s_bt[i] = bt[btb + i];
      __syncthreads();
    }
  };

  bf16x8_t qreg[DS];  // B operand of S^T: this lane's query, d = 32ds + 8*grp + 0..7
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (rvalid) v = *reinterpret_cast<const uint4*>(q + (qtok * HQ + h) * D + 32 * ds + 8 * grp);
    qreg[ds] = __builtin_bit_cast(bf16x8_t, v);
  }

  // K/V tiles travel global -> registers -> LDS.  Two register sets (A, B) alternate so a
  // tile's loads are issued two iterations before its LDS store needs them.
  int bad = 0;
  u32x4_t rkA[LPT], rvA[LPT], rkB[LPT], rvB[LPT];
  auto load_tile = [&](int kt, u32x4_t (&rk)[LPT], u32x4_t (&rv)[LPT])
                       __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + NT * i;
      const int j = min(kt + c / CPR, nk - 1);
      const int jb = j >> bs_log2;
      // jb - btb lies in [0, kBtCache) after cover(kt); an entry past the cached ones is read
      // only when jb >= maxb, which marks the tile bad whatever it holds.
      int blk = s_bt[min(max(jb - btb, 0), kBtCache - 1)];
      const bool ok = jb < maxb && blk >= 0 && blk < num_blocks;
      bad |= !ok;
      blk = ok ? blk : 0;
      const int64_t off = ((((int64_t)blk << bs_log2) + (j & bs_mask)) * HKV + g) * D + (c % CPR) * 8;
      rk[i] = *reinterpret_cast<const u32x4_t*>(kc + off);
      rv[i] = *reinterpret_cast<const u32x4_t*>(vc + off);
    }
  };
  auto store_tile = [&](int buf, const u32x4_t (&rk)[LPT], const u32x4_t (&rv)[LPT])
                        __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = tid + NT * i;
      *reinterpret_cast<u32x4_t*>(&sK[buf][(c / CPR) * KP + (c % CPR) * 8]) = rk[i];
      *reinterpret_cast<u32x4_t*>(&sV[buf][(c / CPR) * VP + (c % CPR) * 8]) = rv[i];
    }
  };

  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;

  // Transposing read: lane p = a + 4t of group grp addresses key 4*grp + t (+32ks, +16 for
  // the second half) at d column 4a (+16db); lane 4a + c then holds d = 16db + 4a + c.
  const int tr_row = 4 * grp + ((lane & 15) >> 2);
  const int tr_col = 4 * (lane & 3);

  // Every path through the prologue and the loop issues the same loads in the same order
  // (a tile start of nk, past the last tile, loads key nk - 1 and is never stored), so the
  // compiler's wait counts stay exact: storing one register set waits for that set only.
  if (ntiles > 0) {
    load_tile(0, rkA, rvA);
    const int kt1 = ntiles > 1 ? BN : nk;
    cover(kt1);
    load_tile(kt1, rkB, rvB);
    store_tile(0, rkA, rvA);
    const int kt2 = ntiles > 2 ? 2 * BN : nk;
    cover(kt2);
    load_tile(kt2, rkA, rvA);
  }
  // Settle the Q loads here, behind the tile loads issued after them: otherwise the wait
  // for them lands in the loop header as a full drain of every load in flight.
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) asm volatile("" : "+v"(qreg[ds]));
  __syncthreads();

  // Iteration t computes tile t from LDS buffer t&1, moves tile t+1 from registers R into
  // the other buffer and refills R with tile t+3; R alternates B, A, B, ...
  auto step = [&](int t, u32x4_t (&rk)[LPT], u32x4_t (&rv)[LPT]) __attribute__((always_inline)) {
    const int kt = t * BN;
    const uint16_t* K = sK[t & 1];
    const uint16_t* V = sV[t & 1];

    f32x4_t s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(&K[(16 * kb + qc) * KP + 32 * ds + 8 * grp]);
        s[kb] = mfma16(a, qreg[ds], s[kb]);
      }
    }

    if (kt + BN > nk_min) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt + 16 * kb + 4 * grp + i;
          s[kb][i] = key < row_nk ? s[kb][i] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
    const bool grow = mx > m + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m - mx) : 1.0f;
      m = grow ? mx : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(s[kb][i], scale_log2, -m));
        s[kb][i] = p;
        l += p;
      }

#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)s[2 * ks][i];
        pb[4 + i] = (__bf16)s[2 * ks + 1][i];
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* base = V + (32 * ks + tr_row) * VP + 16 * db + tr_col;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4i16_t __attribute__((address_space(3)))*)(base));
        const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4i16_t __attribute__((address_space(3)))*)(base + 16 * VP));
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = mfma16(a, pb, o[db]);
      }
    }

    if (t + 1 < ntiles) store_tile((t + 1) & 1, rk, rv);
    const int kn = t + 3 < ntiles ? kt + 3 * BN : nk;
    cover(kn);
    load_tile(kn, rk, rv);
    __syncthreads();
  };
  if (ntiles > 0) {
    for (int t = 0;; t += 2) {
      step(t, rkB, rvB);
      if (t + 1 >= ntiles) break;
      step(t + 1, rkA, rvA);
      if (t + 2 >= ntiles) break;
    }
  }

  if (bad) s_bad = 1;
  __syncthreads();
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = s_bad ? NAN : 1.0f / l;
  if (!rvalid) return;
  uint16_t* dst = out + (qtok * HQ + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    uint2 pk;
    pk.x = uint32_t(f32_to_bf16(o[db][0] * inv)) | (uint32_t(f32_to_bf16(o[db][1] * inv)) << 16);
    pk.y = uint32_t(f32_to_bf16(o[db][2] * inv)) | (uint32_t(f32_to_bf16(o[db][3] * inv)) << 16);
    *reinterpret_cast<uint2*>(dst + 16 * db + 4 * grp) = pk;
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
  if (!(scale > 0.0f)) return fail(PA_ERR_SHAPE, "pa_prefill_paged: scale must be > 0");
  if (num_blocks == 0 && total_q > 0)
    return fail(PA_ERR_SHAPE, "pa_prefill_paged: empty pool");
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
  hipLaunchKernelGGL(fn, grid, dim3(kPrefillThreads), 0, (hipStream_t)stream, (uint16_t*)out,
                     (const uint16_t*)q, (const uint16_t*)k_cache, (const uint16_t*)v_cache,
                     block_table, max_blocks_per_seq, cu_seqlens_q, cu_seqlens_k, total_q, num_blocks,
                     __builtin_ctz(block_size), num_q_heads, num_kv_heads, scale * kLog2e,
                     causal ? 1 : 0);
  return check_launch("pa_prefill_paged");
}
