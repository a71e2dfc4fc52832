// Device side of the chunked prefill: the workgroup body shared by the prefill
// kernel and the mixed prefill + decode launch.  Method and design notes are in
// pa_prefill.hip.
#pragma once

#include "pa_internal.h"

namespace pa {


typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte register chunk

constexpr int kPrefillRows = 128;     // query rows (position x head) per workgroup
constexpr int kPrefillKeys = 64;      // keys per tile
constexpr int kPrefillThreads = 512;  // 8 waves: 4 row groups x 2 key halves
constexpr int kBtCache = 2048;        // block-table entries of one sequence kept in LDS
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is moved
// Running max before any unmasked key: finite, so that a masked score (-inf) still gives
// exp2(-inf - m) = 0 rather than NaN, and a key half that never sees a key merges with weight 0.
constexpr float kNoMax = -1.0e30f;

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// The 16-bit element types of the matrix-core path (ET = pa_dtype): operand vector,
// v_mfma_f32_16x16x32_{bf16,f16}, fp32 -> element conversion (round to nearest even) and
// the element's bits.
template <int ET>
struct Mfma;
template <>
struct Mfma<PA_BF16> {
  typedef bf16x8_t v8;
  __device__ static f32x4_t mma(const v8& a, const v8& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __bf16 cvt(float x) { return (__bf16)x; }
  __device__ static uint16_t bits(float x) { return f32_to_bf16(x); }
};
template <>
struct Mfma<PA_F16> {
  typedef f16x8_t v8;
  __device__ static f32x4_t mma(const v8& a, const v8& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static _Float16 cvt(float x) { return (_Float16)x; }
  __device__ static uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};

// Max over the four lanes l, l^16, l^32, l^48 (the lanes that hold one query's scores), on
// gfx950's lane-swap instructions instead of an LDS round trip.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// v_mfma_f32_16x16x32_bf16 layouts (k index written as (group, i), group = lane / 16):
//   A[m][k]: lane holds m = lane % 16, k = (group, i = 0..7); B[k][n]: n = lane % 16;
//   C/D[m][n]: lane holds m = 4 * group + i (i = 0..3), n = lane % 16.
// Wave w owns 32 query rows, 32*(w%4) + 16*qg + lane%16 for query groups qg = 0, 1, and
// the 32 keys 32*(w/4) + 0..31 of every 64-key tile (its key half).  Both query groups
// share every K and V operand read.  S^T = K Q^T per 16-key block kb: lane holds the
// scores of its query for keys 16kb + 4*group + i of the half.  For O^T += V^T P^T over
// the half's 32 keys, the MFMA k index (group, i) stands for key 16*(i/4) + 4*group + i%4
// on both operands: P comes straight from blocks kb = 0, 1, V^T from two transposing LDS
// reads.  The row sums l come from one more MFMA with an all-ones A operand, so they are
// summed from the same bf16 probabilities as the numerator.  The two key halves of a row
// keep separate (m, l, O) and are merged through LDS at the end.
//
// Pipeline: iteration t holds S_t in registers, computes S_{t+1} from K tile t+1 while it
// exponentiates S_t, then accumulates V tile t.  K therefore runs one tile ahead of V in
// LDS and in the loads: at the end of iteration t the register set R (B for even t, A for
// odd) holds K_{t+2} and V_{t+1}, is written to LDS, and is refilled with K_{t+4} and
// V_{t+3}.  WIDE (block_size >= 64): every tile lies inside one block, so a tile's address
// is a scalar base plus a per-lane offset that does not change from tile to tile.
// The body of one workgroup item: query tile qt of sequence b for KV head g.  MIXED: the
// batch also holds decode rows (sequences with one query), which the decode side of the
// launch handles; such a sequence is skipped here.
template <int D, int G, bool WIDE, bool MIXED, int ET>
__device__ __forceinline__ void prefill_body(
    int qt, int g, int b, uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_table, int maxb, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int total_q, int num_blocks, int bs_log2, int HQ, int HKV,
    float scale_log2, int causal) {
  using M = Mfma<ET>;
  using v8 = typename M::v8;
  constexpr int BM = kPrefillRows / G;  // positions per workgroup
  constexpr int BN = kPrefillKeys;
  constexpr int NT = kPrefillThreads;
  constexpr int P = D + 16;   // K and V row pitch (bf16); conflict-free for both LDS reads
  constexpr int DS = D / 32;  // 32-wide d steps of S^T
  constexpr int DB = D / 16;  // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int LPT = BN * CPR / NT;  // 16-byte loads per thread per tile (K and V each)
  // K tiles in buffers 0, 1 and V tiles in 2, 3; after the loop the same memory carries
  // the key-half partial results (4 x 2 x 32 x 64 floats of O, then m and l).
  __shared__ __attribute__((aligned(16))) uint16_t sKV[4][BN * P];
  static_assert(sizeof(sKV) >= (4 * 2 * (4 * DB + 2) * 64) * sizeof(float), "merge area");
  __shared__ int s_bt[kBtCache];
  static_assert(kBtCache % NT == 0, "block-table window split over the threads");
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  const int32_t* bt = block_table + (int64_t)b * maxb;
  // The first kBtCache block-table entries are fetched before the sequence lengths arrive
  // (they depend only on the sequence index), so the two loads overlap; they are checked
  // and kept once the lengths say how many are used.
  constexpr int BTPT = kBtCache / NT;
  int braw[BTPT];
#pragma unroll
  for (int i = 0; i < BTPT; ++i) braw[i] = tid + NT * i < maxb ? bt[tid + NT * i] : 0;
  // Both offset pairs are read before any of them is used (one round trip, not two).
  int q0 = cu_q[b], q1 = cu_q[b + 1], k0 = cu_k[b], k1 = cu_k[b + 1];
  asm volatile("" : "+s"(q0), "+s"(q1), "+s"(k0), "+s"(k1));
  const int Lq = q1 - q0;
  const int Lk = k1 - k0;
  const int pos0 = qt * BM;
  if (pos0 >= Lq || (MIXED && Lq == 1)) return;
  const int npos = min(BM, Lq - pos0);
  const int prefix = Lk - Lq;
  const int nk = causal ? min(Lk, prefix + pos0 + npos) : Lk;
  const int ntiles = nk > 0 ? (nk + BN - 1) / BN : 0;

  const int lane = tid & 63, w = tid >> 6;
  const int qc = lane & 15, grp = lane >> 4;
  const int rg = w & 3;  // row group
  const int kh = w >> 2;  // key half
  int64_t qtok[2];
  bool rvalid[2];
  int hq[2], row_nk[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const int row = 32 * rg + 16 * qg + qc;
    const int rpos = row / G;
    qtok[qg] = (int64_t)q0 + pos0 + rpos;
    rvalid[qg] = row < BM * G && rpos < npos && qtok[qg] >= 0 && qtok[qg] < total_q;
    hq[qg] = g * G + row % G;
    row_nk[qg] = (causal && rvalid[qg]) ? prefix + pos0 + rpos + 1 : nk;
  }
  const int nk_min = causal ? min(nk, prefix + pos0 + 1) : nk;
  const int bs_mask = (1 << bs_log2) - 1;
  const int HKVD = HKV * D;  // elements between consecutive tokens of a block

  // B operand of S^T: this lane's queries, d = 32ds + 8*grp + 0..7.  A row past the
  // sequence reads a clamped (valid) token instead: rows never mix and such a row is not
  // stored, and unconditional loads keep the compiler from draining the queue after each.
  v8 qreg[2][DS];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const int64_t tok = min(max(qtok[qg], (int64_t)0), (int64_t)total_q - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qreg[qg][ds] = __builtin_bit_cast(
          v8, *reinterpret_cast<const uint4*>(q + (tok * HQ + hq[qg]) * D + 32 * ds + 8 * grp));
  }

  // s_bt[i] holds block-table entry btb + i for i < nv = min(nblk - btb, kBtCache), each
  // checked against the pool when loaded (a bad id marks the output and reads block 0).
  // Block ids are read only from LDS inside the key loop: a global read there would make
  // each tile's address computation wait for every K/V load still in flight.
  const int nblk_need = nk > 0 ? ((nk - 1) >> bs_log2) + 1 : 0;
  const int nblk = min(nblk_need, maxb);
  int bad = nblk_need > maxb;
  int btb = 0;
  auto fill = [&]() __attribute__((always_inline)) {
    for (int i = tid; i < min(nblk - btb, kBtCache); i += NT) {
      const int v = bt[btb + i];
      const bool ok = v >= 0 && v < num_blocks;
      bad |= !ok;
      s_bt[i] = ok ? v : 0;
    }
  };
#pragma unroll
  for (int i = 0; i < BTPT; ++i) {
    if (tid + NT * i < min(nblk, kBtCache)) {
      const bool ok = braw[i] >= 0 && braw[i] < num_blocks;
      bad |= !ok;
      s_bt[tid + NT * i] = ok ? braw[i] : 0;
    }
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // Slides the window to start at the block of key kt when the keys [kt, kt + BN) run past
  // it.  Called with the same kt by every thread (it holds barriers); rare: once per
  // kBtCache blocks.
  auto cover = [&](int kt) __attribute__((always_inline)) {
    if (((min(kt + BN, nk) - 1) >> bs_log2) >= btb + kBtCache) {
      __syncthreads();
      btb = min(kt, nk - 1) >> bs_log2;
      fill();
      __syncthreads();
    }
  };
  // Entry 0 always holds a checked id (nblk >= 1 whenever there is a tile), so the clamp
  // keeps every read on a loaded entry; a key past the table (jb >= maxb) is already bad.
  auto lookup = [&](int jb) __attribute__((always_inline)) {
    return s_bt[max(min(jb - btb, min(nblk - btb, kBtCache) - 1), 0)];
  };

  // Thread tid moves 16-byte chunks c = tid + NT*i of a tile: key row c / CPR, d chunk c % CPR.
  int trow[LPT], tcol[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    trow[i] = (tid + NT * i) / CPR;
    tcol[i] = g * D + ((tid + NT * i) % CPR) * 8;
  }
  // A tile start of nk or more (past the last tile) loads key nk - 1 and is never used.
  int64_t off[LPT];  // general path: element offsets of the K tile loaded last
  auto tile_offsets = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int j = min(kt + trow[i], nk - 1);
      off[i] = (int64_t)lookup(j >> bs_log2) * ((int64_t)HKVD << bs_log2) +
               (int)((j & bs_mask) * HKVD + tcol[i]);
    }
  };
  auto load_wide = [&](const uint16_t* src, int kt, u32x4_t (&r)[LPT]) __attribute__((always_inline)) {
    const int ktc = min(kt, (ntiles - 1) * BN);
    const int blk = __builtin_amdgcn_readfirstlane(lookup(ktc >> bs_log2));
    const uint16_t* base = src + (((int64_t)blk << bs_log2) + (ktc & bs_mask)) * HKVD;
    const int lim = nk - 1 - ktc;
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      r[i] = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(base) +
                                               (uint32_t)(2 * (min(trow[i], lim) * HKVD + tcol[i])));
  };
  auto load_k = [&](int kt, u32x4_t (&r)[LPT]) __attribute__((always_inline)) {
    cover(kt);
    if constexpr (WIDE) {
      load_wide(kc, kt, r);
    } else {
      tile_offsets(kt);
#pragma unroll
      for (int i = 0; i < LPT; ++i) r[i] = *reinterpret_cast<const u32x4_t*>(kc + off[i]);
    }
  };
  // V tile kt always follows the K load of the same tile (no window move in between); the
  // general path reuses that load's offsets.
  auto load_v = [&](int kt, u32x4_t (&r)[LPT]) __attribute__((always_inline)) {
    if constexpr (WIDE) {
      load_wide(vc, kt, r);
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) r[i] = *reinterpret_cast<const u32x4_t*>(vc + off[i]);
    }
  };
  auto store = [&](uint16_t* dst, const u32x4_t (&r)[LPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      *reinterpret_cast<u32x4_t*>(dst + trow[i] * P + (tcol[i] - g * D)) = r[i];
  };
  const int krow = 32 * kh + qc;  // K operand row of block kb = 0 in this wave's key half
  auto scores = [&](const uint16_t* K, f32x4_t (&s)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[0][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      s[1][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const v8 a = *reinterpret_cast<const v8*>(&K[(krow + 16 * kb) * P + 32 * ds + 8 * grp]);
        s[0][kb] = M::mma(a, qreg[0][ds], s[0][kb]);
        s[1][kb] = M::mma(a, qreg[1][ds], s[1][kb]);
      }
    }
  };

  f32x4_t o[2][DB];
  f32x4_t lsum[2];
  float m[2], thr[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qg][db] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    lsum[qg] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[qg] = kNoMax;
    thr[qg] = -INFINITY;  // the first unmasked score always moves the max
  }
  v8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = M::cvt(1.0f);

  // Transposing read: lane p = a + 4t of group grp addresses key 4*grp + t (+16 for the
  // second half) of the key half at d column 4a (+16db); lane 4a + c then holds
  // d = 16db + 4a + c.
  const int tr_off = (32 * kh + 4 * grp + ((lane & 15) >> 2)) * P + 4 * (lane & 3);

  u32x4_t rkA[LPT], rvA[LPT], rkB[LPT], rvB[LPT];
  f32x4_t sc[2][2];  // scores of the tile being reduced
  // Every path issues the same loads in the same order, so the compiler's wait counts stay
  // exact: writing one register set to LDS waits for that set only.
  auto step = [&](int t, u32x4_t (&rk)[LPT], u32x4_t (&rv)[LPT]) __attribute__((always_inline)) {
    const int kt = t * BN;
    if (kt + BN > nk_min) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt + 32 * kh + 16 * kb + 4 * grp + i;
            sc[qg][kb][i] = key < row_nk[qg] ? sc[qg][kb][i] : -INFINITY;
          }
    }
    // The running max moves only when some score of the row exceeds it by more than
    // kLazyRescale (log2 units): a per-lane test against thr = (m + kLazyRescale) / scale
    // decides that, and only then is the row max taken across the row's lanes.
    float lmx[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
      lmx[qg] = fmaxf(fmaxf(fmaxf(sc[qg][0][0], sc[qg][0][1]), fmaxf(sc[qg][0][2], sc[qg][0][3])),
                      fmaxf(fmaxf(sc[qg][1][0], sc[qg][1][1]), fmaxf(sc[qg][1][2], sc[qg][1][3])));
    if (__builtin_amdgcn_ballot_w64(lmx[0] > thr[0] || lmx[1] > thr[1])) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        const float mx = max_over_groups(lmx[qg]) * scale_log2;
        const bool grow = mx > m[qg] + kLazyRescale;
        const float alpha = grow ? fast_exp2(m[qg] - mx) : 1.0f;
        m[qg] = grow ? mx : m[qg];
        thr[qg] = (m[qg] + kLazyRescale) / scale_log2;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[qg][db] *= alpha;
        lsum[qg] *= alpha;
      }
    }

    f32x4_t sn[2][2];
    scores(sKV[(t + 1) & 1], sn);
    v8 pb[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[qg][i] = M::cvt(fast_exp2(fmaf(sc[qg][0][i], scale_log2, -m[qg])));
        pb[qg][4 + i] = M::cvt(fast_exp2(fmaf(sc[qg][1][i], scale_log2, -m[qg])));
      }

    const uint16_t* V = sKV[2 + (t & 1)] + tr_off;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (v4i16_t __attribute__((address_space(3)))*)(V + 16 * db));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (v4i16_t __attribute__((address_space(3)))*)(V + 16 * db + 16 * P));
      const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      o[0][db] = M::mma(a, pb[0], o[0][db]);
      o[1][db] = M::mma(a, pb[1], o[1][db]);
    }
    lsum[0] = M::mma(ones, pb[0], lsum[0]);
    lsum[1] = M::mma(ones, pb[1], lsum[1]);

    // K_{t+2} into the K buffer read last iteration, V_{t+1} into the V buffer read last
    // iteration (stale tiles past the end are written but never read).
    store(sKV[t & 1], rk);
    store(sKV[2 + ((t + 1) & 1)], rv);
    load_v(t + 3 < ntiles ? kt + 3 * BN : nk, rv);
    load_k(t + 4 < ntiles ? kt + 4 * BN : nk, rk);
    __syncthreads();
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      sc[qg][0] = sn[qg][0];
      sc[qg][1] = sn[qg][1];
    }
  };

  if (ntiles > 0) {
    // Prologue: K_0, K_1, V_0 into LDS; B = (K_2, V_1), A = (K_3, V_2) in flight.
    load_k(0, rkA);
    load_v(0, rvA);
    load_k(ntiles > 1 ? BN : nk, rkB);
    load_v(ntiles > 1 ? BN : nk, rvB);
    store(sKV[0], rkA);
    store(sKV[2], rvA);
    store(sKV[1], rkB);
    load_k(ntiles > 2 ? 2 * BN : nk, rkB);
    load_v(ntiles > 2 ? 2 * BN : nk, rvA);
    load_k(ntiles > 3 ? 3 * BN : nk, rkA);
    // Settle the Q loads here, behind the tile loads issued after them: otherwise the wait
    // for them lands in the loop header as a full drain of every load in flight.
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) asm volatile("" : "+v"(qreg[qg][ds]));
    __syncthreads();
    scores(sKV[0], sc);
    __syncthreads();  // iteration 0 overwrites buffer 0
    // Two steps per trip and no exit between them: an exit there lets the compiler sink
    // the first step's loads past it, and the wait counts at the loop header turn into
    // full drains.  With an odd tile count the last step runs past the end, where every
    // key is masked and it adds nothing.
    for (int t = 0; t < ntiles; t += 2) {
      step(t, rkB, rvB);
      step(t + 1, rkA, rvA);
    }
  }

  // Merge the key halves: waves 4..7 publish (m, l, O) of their rows, waves 0..3 combine.
  // The loop ended on a barrier, so the tile buffers are free.
  if (bad) s_bad = 1;
  float* mO = reinterpret_cast<float*>(&sKV[0][0]);
  float* mM = mO + 4 * 2 * 4 * DB * 64;
  float* mL = mM + 4 * 2 * 64;
  if (kh == 1) {
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      const int rq = (rg * 2 + qg) * 64 + lane;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) mO[((rg * 2 + qg) * 4 * DB + 4 * db + i) * 64 + lane] = o[qg][db][i];
      mM[rq] = m[qg];
      mL[rq] = lsum[qg][0];
    }
  }
  __syncthreads();
  if (kh == 1) return;
  const bool poisoned = s_bad != 0;
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const int rq = (rg * 2 + qg) * 64 + lane;
    const float m1 = mM[rq];
    const float mm = fmaxf(m[qg], m1);
    const float a0 = fast_exp2(m[qg] - mm), a1 = fast_exp2(m1 - mm);
    const float inv = poisoned ? NAN : 1.0f / (lsum[qg][0] * a0 + mL[rq] * a1);
    if (!rvalid[qg]) continue;
    uint16_t* dst = out + (qtok[qg] * HQ + hq[qg]) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = (o[qg][db][i] * a0 + mO[((rg * 2 + qg) * 4 * DB + 4 * db + i) * 64 + lane] * a1) * inv;
      uint2 pk;
      pk.x = uint32_t(M::bits(r[0])) | (uint32_t(M::bits(r[1])) << 16);
      pk.y = uint32_t(M::bits(r[2])) | (uint32_t(M::bits(r[3])) << 16);
      *reinterpret_cast<uint2*>(dst + 16 * db + 4 * grp) = pk;
    }
  }
}

}  // namespace pa
