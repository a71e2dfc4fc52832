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
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kPrefillRows = 128;     // query rows (position x head) per workgroup
constexpr int kPrefillKeys = 128;     // keys per tile
constexpr int kPrefillThreads = 512;  // 8 waves: 4 row groups x 2 key halves
constexpr int kBtCache = 2048;        // block-table entries of one sequence kept in LDS
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is moved
// Static LDS of one prefill workgroup: four K/V tile buffers, the block-table window and a flag.
constexpr int prefill_lds_bytes(int D) { return 4 * kPrefillKeys * D * 2 + kBtCache * 4 + 4; }
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
  // The hardware conversion (v_cvt_pk_bf16_f32) rounds to nearest even, as the
  // bit-level rounding of the other kernels does, in one instruction per pair.
  __device__ static uint16_t bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
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

// 16 bytes per lane from global memory straight into LDS, lane i at byte lds + 16 i
// (global_load_lds_dwordx4, LDS address in M0, the same for the whole wave).  Written as
// inline assembly so that the compiler does not hold every later LDS read of the tile
// buffers until all of these loads have landed: the caller waits for them itself
// (s_waitcnt vmcnt) before the barrier that publishes a tile.  One wait state separates
// the M0 write from the load.  The compiler reserves M0 and sets it right before each
// instruction that reads it; no code in these kernels does, so the clobber is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_to_lds(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
#pragma clang diagnostic pop

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
// the 64 keys 64*(w/4) + 0..63 of every 128-key tile (its key half).  Both query groups
// share every K and V operand read.  S^T = K Q^T per 16-key block kb = 0..3: lane holds
// the scores of its query for keys 16kb + 4*group + i of the half.  For O^T += V^T P^T
// over 32 keys at a time (ks = 0, 1), the MFMA k index (group, i) stands for key
// 32ks + 16*(i/4) + 4*group + i%4 on both operands: P comes straight from blocks 2ks and
// 2ks + 1, V^T from two transposing LDS reads.  The row sums l come from one more MFMA
// with an all-ones A operand, so they are summed from the same bf16 probabilities as the
// numerator.  The two key halves of a row keep separate (m, l, O) and are merged through
// LDS at the end.
//
// LDS: two K and two V tile buffers of 128 rows x D, unpadded; the 16-byte chunks of row r
// are permuted by XOR with swz(r), so that the 16 rows one K operand read touches (16
// lanes, one chunk each) and the 8 rows of a transposing read's half wave (two chunks
// each) fall on distinct banks.  Measured: the transposing reads run without bank
// conflicts, the 16-byte K reads with 4 conflict cycles per wave instruction (8 with the
// best padded row pitch).
//
// Pipeline: step t holds S_t in registers; it computes S_{t+1} from K tile t+1 while it
// exponentiates S_t, then accumulates V tile t.  At its start it issues K_{t+2} and
// V_{t+1} straight into the two buffers step t - 1 finished reading, and it ends with a
// wait for them and one barrier.  WIDE (block_size >= 128): every tile lies inside one
// block, so a tile's address is a scalar base plus a per-lane offset.
// The body of one workgroup item: query tile qt of sequence b for KV head g; tid is the
// thread's index in the workgroup (threadIdx.x, passed in so that a caller looping over
// items can keep the lane-dependent setup inside its loop).  MIXED: the
// batch also holds decode rows (sequences with one query), which the decode side of the
// launch handles; such a sequence is skipped here.
template <int D, int G, bool WIDE, bool MIXED, int ET>
__device__ __forceinline__ void prefill_body(
    int tid, int qt, int g, int b, uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_table, int maxb, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int total_q, int num_blocks, int bs_log2, int HQ, int HKV,
    float scale_log2, int causal) {
  using M = Mfma<ET>;
  using v8 = typename M::v8;
  constexpr int BM = kPrefillRows / G;  // positions per workgroup
  constexpr int BN = kPrefillKeys;
  constexpr int NT = kPrefillThreads;
  constexpr int BNH = BN / 2;  // keys per key half
  constexpr int KB = BNH / 16;  // 16-key blocks of S^T per key half
  constexpr int KS = BNH / 32;  // 32-key steps of O^T += V^T P^T per key half
  constexpr int DS = D / 32;  // 32-wide d steps of S^T
  constexpr int DB = D / 16;  // 16-wide d blocks of O^T
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int LPT = BN * CPR / NT;  // 16-byte loads per thread per tile (K and V each)
  // K tiles in buffers 0, 1 and V tiles in 2, 3: unpadded rows of D elements whose 16-byte
  // chunks are XOR-swizzled per row.  After the loop the same memory carries the key-half
  // partial results (4 x 2 x 32 x 64 floats of O, then m and l).
  __shared__ __attribute__((aligned(16))) uint16_t sKV[4][BN * D];
  static_assert(sizeof(sKV) >= (4 * 2 * (4 * DB + 2) * 64) * sizeof(float), "merge area");
  __shared__ int s_bt[kBtCache];
  static_assert(kBtCache % NT == 0, "block-table window split over the threads");
  __shared__ int s_bad;
  static_assert(sizeof(sKV) + sizeof(s_bt) + sizeof(s_bad) == prefill_lds_bytes(D), "LDS size");

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
  int row_nk[2];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const int row = 32 * rg + 16 * qg + qc;
    const int rpos = row / G;
    const int64_t qtok = (int64_t)q0 + pos0 + rpos;
    const bool rvalid = row < BM * G && rpos < npos && qtok >= 0 && qtok < total_q;
    row_nk[qg] = (causal && rvalid) ? prefix + pos0 + rpos + 1 : nk;
  }
  const int nk_min = causal ? min(nk, prefix + pos0 + 1) : nk;
  const int bs_mask = (1 << bs_log2) - 1;
  const int HKVD = HKV * D;  // elements between consecutive tokens of a block

  // B operand of S^T: this lane's queries, d = 32ds + 8*grp + 0..7 (read from the query
  // tile staged in LDS before the first scores).
  v8 qreg[2][DS];

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

  auto swz = [](int r) __attribute__((always_inline)) {
    return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
  };
  // Tile loads go straight into LDS: load i of wave w fills chunk positions 64 (w + 8 i) +
  // lane of the tile, i.e. row trow[i], position p, which holds global chunk p ^ swz(row).
  // The LDS destinations are wave-uniform (scalar); toff[i] is the byte offset of load i
  // within an unclamped tile.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  int trow[LPT], tcol[LPT];
  uint32_t toff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int qp = 64 * (w + 8 * i) + lane;
    trow[i] = qp / CPR;
    tcol[i] = g * D + (((qp % CPR) ^ swz(trow[i])) * 8);
    toff[i] = 2u * (uint32_t)(trow[i] * HKVD + tcol[i]);
  }
  // A tile past the last one loads the last tile's keys (clamped to key nk - 1) and is
  // never read.  WIDE: a tile is one block's rows from a scalar base; its base and the
  // count of valid rows after its first (lim) are found one step before the tile is
  // issued (Tile, locate), so that the table lookup and the address arithmetic run beside
  // the previous step's matrix work instead of holding up the step's first loads.
  struct Tile {
    const uint16_t* base;
    int lim;
  };
  auto locate = [&](const uint16_t* src, int kt) __attribute__((always_inline)) {
    const int ktc = min(kt, (ntiles - 1) * BN);
    const int blk = __builtin_amdgcn_readfirstlane(lookup(ktc >> bs_log2));
    return Tile{src + (((int64_t)blk << bs_log2) + (ktc & bs_mask)) * HKVD, nk - 1 - ktc};
  };
  auto issue_at = [&](const Tile& a, uint16_t* dst) __attribute__((always_inline)) {
    const uint16_t* base = a.base;
    const int lim = a.lim;
    if (lim >= BN - 1) {  // a whole tile: no row clamps
#pragma unroll
      for (int i = 0; i < LPT; ++i)
        load_to_lds(reinterpret_cast<const char*>(base) + toff[i],
                    (uint32_t)(uintptr_t)(dst + 512 * (wu + 8 * i)));
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i)
        load_to_lds(reinterpret_cast<const char*>(base) + (uint32_t)(2 * (min(trow[i], lim) * HKVD + tcol[i])),
                    (uint32_t)(uintptr_t)(dst + 512 * (wu + 8 * i)));
    }
  };
  auto issue = [&](const uint16_t* src, int kt, uint16_t* dst) __attribute__((always_inline)) {
    if constexpr (WIDE) {
      issue_at(locate(src, kt), dst);
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int j = min(kt + trow[i], nk - 1);
        const int64_t off = (int64_t)lookup(j >> bs_log2) * ((int64_t)HKVD << bs_log2) +
                            (int)((j & bs_mask) * HKVD + tcol[i]);
        load_to_lds(src + off, (uint32_t)(uintptr_t)(dst + 512 * (wu + 8 * i)));
      }
    }
  };
  auto issue_k = [&](int t) __attribute__((always_inline)) {
    cover(t * BN);
    issue(kc, t * BN, sKV[t & 1]);
  };
  auto issue_v = [&](int t) __attribute__((always_inline)) { issue(vc, t * BN, sKV[2 + (t & 1)]); };
  // Barrier without a memory fence: first wait for every tile load (the compiler does not
  // count them) and LDS access of this wave.
  auto bar_tiles = [&]() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  const int krow = BNH * kh + qc;  // K operand row of block kb = 0 in this wave's key half
  auto scores = [&](const uint16_t* K, f32x4_t (&s)[2][KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[0][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      s[1][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      const int r = krow + 16 * kb;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const v8 a = *reinterpret_cast<const v8*>(&K[r * D + (((4 * ds + grp) ^ swz(r)) * 8)]);
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

  // Transposing read: lane p = a + 4t of group grp addresses key 32ks + 4*grp + t (+16 for
  // the second read) of the key half at d column 4a (+16db); lane 4a + c then holds
  // d = 16db + 4a + c.  Column 16db + 4a lies in chunk 2db + a/2, at byte 8 (a & 1); rows
  // 16 apart share the swizzle.
  const int tr_row = BNH * kh + 4 * grp + ((lane & 15) >> 2);
  int tr_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    tr_off[db] = tr_row * D + (((2 * db + ((lane & 3) >> 1)) ^ swz(tr_row)) * 8) + 4 * (lane & 1);

  f32x4_t sc[2][KB];  // scores of the tile being reduced
  Tile next_v, next_k;  // WIDE: V_{t+1} and K_{t+2}, located during step t - 1
  auto step = [&](int t) __attribute__((always_inline)) {
    const int kt = t * BN;
    // V_{t+1} and K_{t+2} into the buffers step t - 1 finished reading.
    // (None past the last tile: the last steps' waits then cover no dead loads.)
    if constexpr (WIDE) {
      if (t + 1 < ntiles) issue_at(next_v, sKV[2 + ((t + 1) & 1)]);
      if (t + 2 < ntiles) issue_at(next_k, sKV[t & 1]);
    } else {
      if (t + 1 < ntiles) issue_v(t + 1);
      if (t + 2 < ntiles) issue_k(t + 2);
    }
    if (kt + BN > nk_min) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt + BNH * kh + 16 * kb + 4 * grp + i;
            sc[qg][kb][i] = key < row_nk[qg] ? sc[qg][kb][i] : -INFINITY;
          }
    }
    float lmx[2];
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      lmx[qg] = sc[qg][0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmx[qg] = fmaxf(lmx[qg], sc[qg][kb][i]);
    }
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

    // S_{t+1} = K_{t+1} Q^T interleaved with P_t = exp2(S_t c - m): KB * DS groups of one K
    // operand read two groups ahead, two MFMAs and EPG exponentials per lane (32 in all).
    constexpr int NG = KB * DS;
    constexpr int EPG = 2 * 4 * KB / NG;  // exponentials per group
    static_assert(EPG % 2 == 0 && EPG * NG == 8 * KB, "pairs of exponentials per group");
    const uint16_t* Kn = sKV[(t + 1) & 1];
    auto read_k = [&](int i) __attribute__((always_inline)) {
      const int r = krow + 16 * (i / DS);
      return *reinterpret_cast<const v8*>(&Kn[r * D + (((4 * (i % DS) + grp) ^ swz(r)) * 8)]);
    };
    f32x4_t sn[2][KB];
    v8 pb[2][KS];
    v8 kr[3];
    __builtin_amdgcn_sched_barrier(0);
    kr[0] = read_k(0);
    kr[1] = read_k(1);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (i + 2 < NG) kr[(i + 2) % 3] = read_k(i + 2);
      const int kb = i / DS, ds = i % DS;
      if (ds == 0) {
        sn[0][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        sn[1][kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
      sn[0][kb] = M::mma(kr[i % 3], qreg[0][ds], sn[0][kb]);
      sn[1][kb] = M::mma(kr[i % 3], qreg[1][ds], sn[1][kb]);
      // elements EPG i .. EPG i + EPG - 1 of this lane's 32 probabilities: element j is
      // query group j / 16, key block (j / 4) % 4, entry j % 4
#pragma unroll
      for (int j = EPG * i; j < EPG * i + EPG; ++j) {
        const int qg = j / 16, ekb = (j / 4) % 4, ii = j % 4;
        pb[qg][ekb / 2][4 * (ekb % 2) + ii] = M::cvt(fast_exp2(fmaf(sc[qg][ekb][ii], scale_log2, -m[qg])));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // The next step's tiles, located while this step's matrix work runs.  V_{t+2} lies in
    // the block window the last slide left (it starts at or before K_{t+2}'s block); the
    // window then moves for K_{t+3}.
    if constexpr (WIDE) {
      next_v = locate(vc, (t + 2) * BN);
      cover((t + 3) * BN);
      next_k = locate(kc, (t + 3) * BN);
    }

    // O^T += V^T P^T, the transposing reads of d block db + 1 issued before the MFMAs of
    // block db (and the row-sum MFMAs covering the first reads).
    const uint16_t* V = sKV[2 + (t & 1)];
    v4i16_t vr[2][2 * KS];
    auto read_v = [&](int db, v4i16_t (&r)[2 * KS]) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint16_t* Vk = V + tr_off[db] + 32 * ks * D;
        r[2 * ks] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4i16_t __attribute__((address_space(3)))*)(Vk));
        r[2 * ks + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (v4i16_t __attribute__((address_space(3)))*)(Vk + 16 * D));
      }
    };
    __builtin_amdgcn_sched_barrier(0);
    read_v(0, vr[0]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      lsum[0] = M::mma(ones, pb[0][ks], lsum[0]);
      lsum[1] = M::mma(ones, pb[1][ks], lsum[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db + 1 < DB) read_v(db + 1, vr[(db + 1) & 1]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const v8 a = __builtin_bit_cast(
            v8, __builtin_shufflevector(vr[db & 1][2 * ks], vr[db & 1][2 * ks + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[0][db] = M::mma(a, pb[0][ks], o[0][db]);
        o[1][db] = M::mma(a, pb[1][ks], o[1][db]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // V_{t+1} and K_{t+2} must have landed before the next step.
    bar_tiles();
#pragma unroll
    for (int qg = 0; qg < 2; ++qg)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sc[qg][kb] = sn[qg][kb];
  };

  if (ntiles > 0) {
    // The query tile goes through LDS (the last V buffer, free until step 0) like a K tile,
    // so that the first scores wait only for Q and K_0 while V_0 and K_1 land (Q in
    // registers would have the compiler wait for every load, as it does not count the
    // tile loads).  Rows past the sequence read a clamped (valid) token: rows never mix
    // and such a row is not stored.
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int rpos = trow[i] / G;
      const int64_t tok = min(max((int64_t)q0 + pos0 + rpos, (int64_t)0), (int64_t)total_q - 1);
      load_to_lds(q + (tok * HQ + g * G + trow[i] % G) * D + (tcol[i] - g * D),
                  (uint32_t)(uintptr_t)(sKV[3] + 512 * (wu + 8 * i)));
    }
    issue_k(0);
    issue_v(0);
    if (ntiles > 1) issue_k(1);
    if constexpr (WIDE) {
      next_v = locate(vc, BN);
      cover(2 * BN);
      next_k = locate(kc, 2 * BN);
    }
    // Loads complete in issue order: with V_0 and K_1 (LPT each) still allowed in flight,
    // this wave's parts of Q and K_0 have landed; the barrier publishes everyone's.
    asm volatile("" ::: "memory");
    if (ntiles > 1)
      __builtin_amdgcn_s_waitcnt((7 << 4) | (2 * LPT));  // vmcnt(2 LPT) expcnt(7) lgkmcnt(0)
    else
      __builtin_amdgcn_s_waitcnt((7 << 4) | LPT);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      const int r = 32 * rg + 16 * qg + qc;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qreg[qg][ds] = *reinterpret_cast<const v8*>(&sKV[3][r * D + (((4 * ds + grp) ^ swz(r)) * 8)]);
    }
    scores(sKV[0], sc);
    bar_tiles();  // V_0, K_1 landed; Q read, so step 0 may refill buffers 0 and 3
    for (int t = 0; t < ntiles; ++t) step(t);
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
  // The merged rows go to LDS in row-major order (16-byte chunks XOR-swizzled by row, so
  // that neither side conflicts) and leave in 16-byte chunks per lane: each non-temporal
  // store then writes whole 64-byte pieces of a row.  Wave rg stages its 32 rows in the
  // last tile buffer, which the merge area does not reach.
  constexpr int CR = D / 8;  // 16-byte chunks per output row
  uint16_t* stage = sKV[3] + rg * 32 * D;
  static_assert(4 * 32 * D <= BN * D, "staging area");
  static_assert((4 * 2 * (4 * DB + 2) * 64) * sizeof(float) <= 3 * BN * D * sizeof(uint16_t),
                "merge area below the staging area");
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const int rq = (rg * 2 + qg) * 64 + lane;
    const float m1 = mM[rq];
    const float mm = fmaxf(m[qg], m1);
    const float a0 = fast_exp2(m[qg] - mm), a1 = fast_exp2(m1 - mm);
    const float inv = poisoned ? NAN : 1.0f / (lsum[qg][0] * a0 + mL[rq] * a1);
    const int rl = 16 * qg + qc;  // row within the wave's 32
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r[i] = (o[qg][db][i] * a0 + mO[((rg * 2 + qg) * 4 * DB + 4 * db + i) * 64 + lane] * a1) * inv;
      const u32x2_t pk = {uint32_t(M::bits(r[0])) | (uint32_t(M::bits(r[1])) << 16),
                          uint32_t(M::bits(r[2])) | (uint32_t(M::bits(r[3])) << 16)};
      const int c = 2 * db + (grp >> 1);  // 16-byte chunk of d = 16 db + 4 grp
      *reinterpret_cast<u32x2_t*>(stage + rl * D + ((c ^ (rl % CR)) * 8) + 4 * (grp & 1)) = pk;
    }
  }
  // Each wave reads back only what it wrote (LDS keeps a wave's accesses in order).
  constexpr int RPI = 64 / CR;  // rows per pass
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rl = it * RPI + lane / CR, c = lane % CR;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stage + rl * D + ((c ^ (rl % CR)) * 8));
    const int row = 32 * rg + rl;
    const int rpos = row / G;
    const int64_t tok = (int64_t)q0 + pos0 + rpos;
    if (row < BM * G && rpos < npos && tok >= 0 && tok < total_q)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + (tok * HQ + g * G + row % G) * D + 8 * c));
  }
}

}  // namespace pa
