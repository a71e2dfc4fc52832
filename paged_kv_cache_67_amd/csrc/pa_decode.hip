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

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Element handling per storage type.  A lane owns 16 bytes of a token row:
// 8 bf16 or 4 fp32 values.  q.k uses v_dot2_f32_bf16 on the packed bf16 pairs
// (products exact, fp32 accumulation); V is widened to fp32 for the P.V sums.
template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  static constexpr int VEC = 8;
  __device__ static float dot(const uint32_t* q, const uint4& k) {
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[0]),
                                              __builtin_bit_cast(bf16x2_t, k.x), 0.0f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[1]),
                                        __builtin_bit_cast(bf16x2_t, k.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[2]),
                                        __builtin_bit_cast(bf16x2_t, k.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[3]),
                                        __builtin_bit_cast(bf16x2_t, k.w), d, false);
    return d;
  }
  __device__ static void widen(const uint4& u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  }
  __device__ static void store(void* out, int64_t idx, float v) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
  }
};
template <>
struct Elem<false> {
  static constexpr int VEC = 4;
  __device__ static float dot(const uint32_t* q, const uint4& k) {
    float d = __uint_as_float(q[0]) * __uint_as_float(k.x);
    d = fmaf(__uint_as_float(q[1]), __uint_as_float(k.y), d);
    d = fmaf(__uint_as_float(q[2]), __uint_as_float(k.z), d);
    return fmaf(__uint_as_float(q[3]), __uint_as_float(k.w), d);
  }
  __device__ static void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static void store(void* out, int64_t idx, float v) {
    reinterpret_cast<float*>(out)[idx] = v;
  }
};

#ifndef PA_DECODE_LOADS
#define PA_DECODE_LOADS 4
#endif
#ifndef PA_DECODE_WAVES_PER_CU
#define PA_DECODE_WAVES_PER_CU 8
#endif

// Load slots per chunk: wide GQA tiles hold more q / state registers, so they
// take smaller chunks to stay clear of spills.
__host__ __device__ constexpr int loads_per_chunk(int G) {
  return G > 6 ? 1 : (G > 4 ? (PA_DECODE_LOADS > 2 ? PA_DECODE_LOADS / 2 : 1) : PA_DECODE_LOADS);
}
// Head waves per workgroup: 8, or 4 for the widest tiles (a wave may then use
// up to 512 VGPRs).
__host__ __device__ constexpr int max_head_waves(int G) { return G > 6 ? 4 : 8; }
// Tokens per chunk for a kernel instance: rows per load times load slots.
__host__ __device__ constexpr int chunk_tokens(int D, bool bf16, int G) {
  return (64 / (D / (bf16 ? 8 : 4))) * loads_per_chunk(G);
}

constexpr int kHeadSlot = 0;  // partial state of a piece whose sequence began before the slice
constexpr int kTailSlot = 1;  // partial state of a piece whose sequence runs past the slice
constexpr int kMaxBalancedSeqs = 8192;  // LDS holds 2 ints per sequence

template <int U>
struct KVRegs {
  uint4 k[U], v[U];
};

// Per-wave decode state: this wave's q registers and one online-softmax state
// per row group, for G query heads of one KV head.
template <int D, bool BF16, int G>
struct DecodeWave {
  using E = Elem<BF16>;
  static constexpr int VEC = E::VEC;
  static constexpr int LANES = D / VEC;  // lanes per token row
  static constexpr int RG = 64 / LANES;  // token rows per wave load
  static constexpr int U = loads_per_chunk(G);
  static constexpr int CH = RG * U;  // tokens per chunk
  static constexpr int ESZ = BF16 ? 2 : 4;

  int r, sl;  // row group, 16-byte slice of the row
  int bs_log2, bs_mask, maxb, num_blocks;
  uint32_t row_bytes, lane_off;
  int64_t blk_bytes;
  const char* kc;
  const char* vc;
  float scale_log2;
  int bad;
  uint32_t qw[G][4];
  float m[G], l[G], acc[G][VEC];

  __device__ __forceinline__ void init(const void* kcache, const void* vcache, int g, int HKV,
                                       int bs_log2_, int maxb_, int num_blocks_, float scale) {
    const int lane = threadIdx.x & 63;
    r = lane / LANES;
    sl = lane % LANES;
    bs_log2 = bs_log2_;
    bs_mask = (1 << bs_log2_) - 1;
    maxb = maxb_;
    num_blocks = num_blocks_;
    row_bytes = (uint32_t)HKV * D * ESZ;
    lane_off = (uint32_t)(g * D + sl * VEC) * ESZ;
    blk_bytes = (int64_t)row_bytes << bs_log2_;
    kc = reinterpret_cast<const char*>(kcache);
    vc = reinterpret_cast<const char*>(vcache);
    scale_log2 = scale;
  }

  // q rows (b, h0 .. h0+G-1): this lane's 16-byte slice of each.
  __device__ __forceinline__ void load_q(const void* qptr, int64_t first_row) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(qptr) +
                                                      ((first_row + j) * D + sl * VEC) * ESZ);
      qw[j][0] = u.x; qw[j][1] = u.y; qw[j][2] = u.z; qw[j][3] = u.w;
    }
  }

  __device__ __forceinline__ void reset() {
    bad = 0;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      m[j] = -INFINITY;
      l[j] = 0.0f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] = 0.0f;
    }
  }

  // Block ids of the chunk starting at token t0 of a sequence whose keys end at
  // `end`, one per load slot.  Indices past the end are clamped to its last
  // token, so every lookup is of a live table entry.
  __device__ __forceinline__ void fetch_ids(const int32_t* bt, int t0, int end, int* ids) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jb = min(t0 + u * RG, end - 1) >> bs_log2;
      bad |= jb >= maxb;
      ids[u] = bt[min(jb, maxb - 1)];
    }
  }

  // Issue the chunk's K/V loads.  Token indices past `end` are clamped to its
  // last token (a live row) and masked in compute(); a slot's RG tokens always
  // share one block.  An out-of-range block id is replaced by block 0
  // (num_blocks >= 1) and poisons the piece through `bad`.
  __device__ __forceinline__ void issue(KVRegs<U>& X, int t0, int end, const int* ids) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + u * RG + r, end - 1);
      const bool ok = ids[u] >= 0 && ids[u] < num_blocks;
      bad |= !ok;
      const int64_t base = (int64_t)(ok ? ids[u] : 0) * blk_bytes;
      const uint32_t off = (uint32_t)(t & bs_mask) * row_bytes + lane_off;
      X.k[u] = *reinterpret_cast<const uint4*>(kc + base + off);
      X.v[u] = *reinterpret_cast<const uint4*>(vc + base + off);
    }
  }

  // Online-softmax update with the chunk's tokens t0 .. t0+CH-1 (those < end).
  __device__ __forceinline__ void compute(const KVRegs<U>& X, int t0, int end) {
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool valid = t0 + u * RG + r < end;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float d = group_sum<LANES>(E::dot(qw[j], X.k[u])) * scale_log2;
        sc[u][j] = valid ? d : -INFINITY;
      }
    }
    float ps[U][G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mx = sc[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
      const float mnew = fmaxf(m[j], mx);
      const float msafe = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = fast_exp2(m[j] - msafe);
      float psum = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ps[u][j] = fast_exp2(sc[u][j] - msafe);
        psum += ps[u][j];
      }
      l[j] = l[j] * alpha + psum;
      m[j] = mnew;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[j][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[VEC];
      E::widen(X.v[u], vf);
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[j][e] = fmaf(ps[u][j], vf[e], acc[j][e]);
    }
  }

  // Fold the row groups: rescale each to the wave max, then sum.  Afterwards
  // every lane holds the totals for its 16-byte slice (m in base-2 units).
  __device__ __forceinline__ void fold() {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float M = m[j];
#pragma unroll
      for (int o = LANES; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
      const float f = m[j] == -INFINITY ? 0.0f : fast_exp2(m[j] - M);
      float lj = l[j] * f;
#pragma unroll
      for (int o = LANES; o < 64; o <<= 1) lj += __shfl_xor(lj, o);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float a = acc[j][e] * f;
#pragma unroll
        for (int o = LANES; o < 64; o <<= 1) a += __shfl_xor(a, o);
        acc[j][e] = a;
      }
      m[j] = M;
      l[j] = lj;
    }
  }

  // After fold(): final rows out[first_row + j] = acc / l (row group 0 writes).
  __device__ __forceinline__ void store_final(void* out, int64_t first_row) const {
    if (r != 0) return;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float inv = bad ? NAN : 1.0f / l[j];
#pragma unroll
      for (int e = 0; e < VEC; ++e) E::store(out, (first_row + j) * D + sl * VEC + e, acc[j][e] * inv);
    }
  }

  // After fold(): partial state of query head j into state slot idx0 + j*stride
  // (acc unnormalised, m in natural-log units, l).
  __device__ __forceinline__ void store_state(float* ws_acc, float* ws_m, float* ws_l,
                                              int64_t idx0, int64_t stride) const {
    if (r != 0) return;
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int64_t idx = idx0 + j * stride;
      float* dst = ws_acc + idx * D + sl * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dst[e] = bad ? NAN : acc[j][e];
      if (sl == 0) {
        ws_m[idx] = m[j] * kLn2;
        ws_l[idx] = l[j];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Fixed partitions: grid = (partition, head group, sequence).  One wave = one
// (sequence, KV head, head tile, partition); the waves of a workgroup are
// consecutive KV heads of the same tokens.  split == 0: one partition per
// sequence, written straight to `out`.
template <int D, bool BF16, int G>
__global__ __launch_bounds__(max_head_waves(G) * 64) void decode_kernel(
    void* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l, const void* __restrict__ qptr, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ context_lens, int num_blocks, int bs_log2, int HQ, int HKV,
    int group, float scale_log2, int part_size, int NP, int split) {
  using W = DecodeWave<D, BF16, G>;
  using E = Elem<BF16>;
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

// ---------------------------------------------------------------------------
// Balanced split: grid = (slice, head group).  Chunk counts ceil(L_b / CH) are
// scanned into LDS (workgroup (0,0) also leaves the scan in the workspace for
// the merge); slice w of each KV head covers flat chunks [w*Cw, (w+1)*Cw).

// Position of one chunk: flat index f, sequence b, chunk j within b, b's chunk
// range [cb, ce) and key count L.  All wave-uniform.
struct Cursor {
  int f, b, j, cb, ce, L;
};

__device__ __forceinline__ int lds_uniform(const int* p) { return __builtin_amdgcn_readfirstlane(*p); }

__device__ __forceinline__ void cursor_load(Cursor& c, int b, const int* s_cuc, const int* s_len) {
  c.b = b;
  c.cb = lds_uniform(s_cuc + b);
  c.ce = lds_uniform(s_cuc + b + 1);
  c.L = lds_uniform(s_len + b);
}

// The chunk after c (past the last chunk, b becomes B).
__device__ __forceinline__ Cursor cursor_next(Cursor c, int B, const int* s_cuc, const int* s_len) {
  c.f += 1;
  c.j += 1;
  if (c.cb + c.j >= c.ce) {
    int b = c.b + 1;
    while (b < B && lds_uniform(s_cuc + b + 1) == lds_uniform(s_cuc + b)) ++b;  // skip empty sequences
    c.j = 0;
    if (b < B) cursor_load(c, b, s_cuc, s_len);
    else c.b = B;
  }
  return c;
}

template <int D, bool BF16, int G>
__global__ __launch_bounds__(max_head_waves(G) * 64) void decode_balanced_kernel(
    void* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l, int32_t* __restrict__ ws_cuc, const void* __restrict__ qptr,
    const void* __restrict__ kcache, const void* __restrict__ vcache,
    const int32_t* __restrict__ block_table, int maxb, const int32_t* __restrict__ context_lens,
    int B, int num_blocks, int bs_log2, int HQ, int HKV, int group, float scale_log2, int Wt) {
  using W = DecodeWave<D, BF16, G>;
  constexpr int CH = W::CH;
  constexpr int U = W::U;
  extern __shared__ int s_mem[];
  int* s_cuc = s_mem;          // [B + 1] exclusive prefix sums of chunk counts
  int* s_len = s_mem + B + 1;  // [B] key counts

  // Wave 0 scans the chunk counts: each lane sums a contiguous segment, a
  // wave-wide scan of the segment sums gives each segment's offset.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int seg = (B + 63) / 64;
    const int lo = min(B, lane * seg), hi = min(B, lo + seg);
    int sum = 0;
    for (int i = lo; i < hi; ++i) {
      const int L = max(context_lens[i], 0);
      s_len[i] = L;
      sum += (L + CH - 1) / CH;
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
    for (int i = lo; i < hi; ++i) {
      s_cuc[i] = run;
      run += (s_len[i] + CH - 1) / CH;
    }
    if (lane == 63) s_cuc[B] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i <= B; i += blockDim.x) ws_cuc[i] = s_cuc[i];

  const int tiles = group / G;
  const int hw = blockIdx.y * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (hw >= HKV * tiles) return;
  const int g = hw / tiles;
  const int h0 = g * group + (hw % tiles) * G;
  const int NC = lds_uniform(s_cuc + B);
  const int Cw = (NC + Wt - 1) / Wt;
  const int w = blockIdx.x;
  const int f_begin = w * Cw;
  const int f_end = min(NC, f_begin + Cw);
  if (f_begin >= f_end) return;

  // The sequence holding chunk f_begin: the largest b with s_cuc[b] <= f_begin
  // (s_cuc[0] = 0 <= f_begin < NC = s_cuc[B]).
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (lds_uniform(s_cuc + mid) <= f_begin) lo = mid;
    else hi = mid;
  }
  Cursor c0;
  cursor_load(c0, lo, s_cuc, s_len);
  c0.f = f_begin;
  c0.j = f_begin - c0.cb;

  W st;
  st.init(kcache, vcache, g, HKV, bs_log2, maxb, num_blocks, scale_log2);
  st.reset();
  st.load_q(qptr, (int64_t)c0.b * HQ + h0);

  auto bt_of = [&](const Cursor& c) { return block_table + (int64_t)c.b * maxb; };
  // After the chunk at c: if it closes a piece (its sequence's last chunk or the
  // slice's last chunk), write the piece and start the next sequence's state.
  auto finish = [&](const Cursor& c, const Cursor& next) {
    if (c.cb + c.j + 1 != c.ce && c.f + 1 != f_end) return;
    st.fold();
    if (c.cb >= f_begin && c.ce <= f_end) {
      st.store_final(out, (int64_t)c.b * HQ + h0);
    } else {
      const int slot = c.cb < f_begin ? kHeadSlot : kTailSlot;
      st.store_state(ws_acc, ws_m, ws_l, ((int64_t)h0 * Wt + w) * 2 + slot, (int64_t)Wt * 2);
    }
    st.reset();
    if (next.f < f_end) st.load_q(qptr, (int64_t)next.b * HQ + h0);
  };

  // A and B alternate as in decode_kernel; cursors c0 (in A) and c1 (in B).
  const int n = f_end - f_begin;
  KVRegs<U> A, Bv;
  int idsA[U], idsB[U];
  Cursor c1 = cursor_next(c0, B, s_cuc, s_len);
  st.fetch_ids(bt_of(c0), c0.j * CH, c0.L, idsA);
  st.issue(A, c0.j * CH, c0.L, idsA);
  if (n > 1) st.fetch_ids(bt_of(c1), c1.j * CH, c1.L, idsB);
  for (int k = 0; k < (n - 1) / 2; ++k) {
    st.issue(Bv, c1.j * CH, c1.L, idsB);
    const Cursor c2 = cursor_next(c1, B, s_cuc, s_len);
    st.fetch_ids(bt_of(c2), c2.j * CH, c2.L, idsA);
    st.compute(A, c0.j * CH, c0.L);
    finish(c0, c1);
    st.issue(A, c2.j * CH, c2.L, idsA);
    const Cursor c3 = cursor_next(c2, B, s_cuc, s_len);
    if (c3.f < f_end) st.fetch_ids(bt_of(c3), c3.j * CH, c3.L, idsB);
    st.compute(Bv, c1.j * CH, c1.L);
    finish(c1, c2);
    c0 = c2;
    c1 = c3;
  }
  if ((n - 1) & 1) {
    st.issue(Bv, c1.j * CH, c1.L, idsB);
    st.compute(A, c0.j * CH, c0.L);
    finish(c0, c1);
    st.compute(Bv, c1.j * CH, c1.L);
    finish(c1, c1);
  } else {
    st.compute(A, c0.j * CH, c0.L);
    finish(c0, c1);
  }
}

// ---------------------------------------------------------------------------
// Merges: one workgroup per (query head, sequence), one thread per element.

template <bool BF16>
__global__ __launch_bounds__(128) void merge_kernel(
    void* __restrict__ out, const float* __restrict__ ws_acc, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const int32_t* __restrict__ context_lens, int HQ, int D,
    int NP, int part_size) {
  using E = Elem<BF16>;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t bh = (int64_t)b * HQ + h;
  const int L = context_lens[b];
  int n = L > 0 ? (L + part_size - 1) / part_size : 0;
  n = min(n, NP);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    if (n == 0) {
      E::store(out, bh * D + d, 0.0f);
      continue;
    }
    float M = -INFINITY;
    for (int p = 0; p < n; ++p) M = fmaxf(M, ws_m[bh * NP + p]);
    float A = 0.0f, Lt = 0.0f;
    for (int p = 0; p < n; ++p) {
      const float f = fast_exp2((ws_m[bh * NP + p] - M) * kLog2e);
      A = fmaf(f, ws_acc[(bh * NP + p) * D + d], A);
      Lt = fmaf(f, ws_l[bh * NP + p], Lt);
    }
    E::store(out, bh * D + d, A / Lt);
  }
}

// Balanced split: sequence b spans slices w0 = cb / Cw .. w1 = (ce - 1) / Cw.
// With w0 == w1 the decode pass already wrote the row; otherwise its pieces
// are slice w0's tail state and slices w0+1 .. w1's head states.
template <bool BF16>
__global__ __launch_bounds__(128) void merge_balanced_kernel(
    void* __restrict__ out, const float* __restrict__ ws_acc, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const int32_t* __restrict__ ws_cuc, int B, int HQ, int D,
    int Wt) {
  using E = Elem<BF16>;
  const int h = blockIdx.x, b = blockIdx.y;
  const int64_t row = ((int64_t)b * HQ + h) * D;
  const int cb = ws_cuc[b], ce = ws_cuc[b + 1];
  if (cb >= ce) {  // no keys: zero row
    for (int d = threadIdx.x; d < D; d += blockDim.x) E::store(out, row + d, 0.0f);
    return;
  }
  const int NC = ws_cuc[B];
  const int Cw = (NC + Wt - 1) / Wt;
  const int w0 = cb / Cw, w1 = (ce - 1) / Cw;
  if (w0 == w1) return;
  const int64_t base = (int64_t)h * Wt * 2;
  float M = ws_m[base + w0 * 2 + kTailSlot];
  for (int w = w0 + 1; w <= w1; ++w) M = fmaxf(M, ws_m[base + w * 2 + kHeadSlot]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    int64_t s = base + w0 * 2 + kTailSlot;
    float f = fast_exp2((ws_m[s] - M) * kLog2e);
    float A = f * ws_acc[s * D + d], Lt = f * ws_l[s];
    for (int w = w0 + 1; w <= w1; ++w) {
      s = base + w * 2 + kHeadSlot;
      f = fast_exp2((ws_m[s] - M) * kLog2e);
      A = fmaf(f, ws_acc[s * D + d], A);
      Lt = fmaf(f, ws_l[s], Lt);
    }
    E::store(out, row + d, A / Lt);
  }
}

// ---------------------------------------------------------------------------
// Host side.

typedef void (*decode_fn)(void*, float*, float*, float*, const void*, const void*, const void*,
                          const int32_t*, int, const int32_t*, int, int, int, int, int, float, int,
                          int, int);
typedef void (*balanced_fn)(void*, float*, float*, float*, int32_t*, const void*, const void*,
                            const void*, const int32_t*, int, const int32_t*, int, int, int, int,
                            int, int, float, int);

template <int D, bool BF16>
static void pick_g(int G, decode_fn* f, balanced_fn* fb) {
  switch (G) {
#define PA_CASE(g)                            \
  case g:                                     \
    *f = decode_kernel<D, BF16, g>;           \
    *fb = decode_balanced_kernel<D, BF16, g>; \
    return;
    PA_CASE(1) PA_CASE(2) PA_CASE(3) PA_CASE(4) PA_CASE(5) PA_CASE(6) PA_CASE(7) PA_CASE(8)
#undef PA_CASE
  }
  *f = nullptr;
  *fb = nullptr;
}

static void pick_decode(int D, pa_dtype dt, int G, decode_fn* f, balanced_fn* fb) {
  if (dt == PA_BF16) D == 64 ? pick_g<64, true>(G, f, fb) : pick_g<128, true>(G, f, fb);
  else D == 64 ? pick_g<64, false>(G, f, fb) : pick_g<128, false>(G, f, fb);
}

// Heads per wave: the largest divisor of the GQA group that is <= 8.
static int head_tile(int group) {
  for (int t = 8; t > 1; --t)
    if (group % t == 0) return t;
  return 1;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Fixed partitions used when the balanced split is unavailable (very large
// batches): at least 256 tokens, about 64 work items per compute unit.
static int32_t auto_partition(int32_t B, int32_t HKV, int32_t max_ctx) {
  const int64_t target = 64LL * kNumCUs;
  const int64_t units = (int64_t)B * HKV;
  int64_t P = 256;
  while (P < max_ctx && units * ceil_div(max_ctx, P) > target) P *= 2;
  return (int32_t)P;
}

// How pa_decode splits a batch.
struct DecodePlan {
  enum Mode { kSingle, kFixed, kBalanced } mode;
  int32_t P;  // kFixed: partition tokens
  int NP;     // kFixed: partitions per sequence
  int Wt;     // kBalanced: slices per head wave
  int G;      // query heads per wave
  size_t ws_bytes;
};

static DecodePlan plan_decode(int32_t B, int32_t HQ, int32_t HKV, int32_t D, pa_dtype dtype,
                              int32_t max_ctx, int32_t partition_size, bool have_workspace) {
  DecodePlan pl{};
  const int group = HQ / HKV;
  pl.G = head_tile(group);
  if (partition_size == -1 || (partition_size == 0 && !have_workspace)) {
    pl.mode = DecodePlan::kSingle;
  } else if (partition_size == 0 && B <= kMaxBalancedSeqs) {
    pl.mode = DecodePlan::kBalanced;
    const int head_waves = HKV * (group / pl.G);
    const int CH = chunk_tokens(D, dtype == PA_BF16, pl.G);
    int64_t Wt = (int64_t)kNumCUs * PA_DECODE_WAVES_PER_CU / head_waves;
    Wt = Wt < 1 ? 1 : Wt;
    const int64_t max_chunks = (int64_t)B * ceil_div(max_ctx > 0 ? max_ctx : 1, CH);
    if (Wt > max_chunks) Wt = max_chunks;
    pl.Wt = (int)Wt;
    const size_t states = (size_t)HQ * pl.Wt * 2;
    pl.ws_bytes = states * (D + 2) * sizeof(float) + (size_t)(B + 1) * sizeof(int32_t);
  } else {
    pl.P = partition_size > 0 ? partition_size : auto_partition(B, HKV, max_ctx);
    if (pl.P >= max_ctx) {
      pl.mode = DecodePlan::kSingle;
    } else {
      pl.mode = DecodePlan::kFixed;
      pl.NP = (int)ceil_div(max_ctx, pl.P);
      pl.ws_bytes = (size_t)B * HQ * pl.NP * (D + 2) * sizeof(float);
    }
  }
  return pl;
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
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
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

// Workspace carving: balanced = acc | m | l | cuc; fixed = acc | m | l.
struct WsPtrs {
  float *acc, *m, *l;
  int32_t* cuc;
};
static WsPtrs carve(void* ws, const DecodePlan& pl, int32_t B, int32_t HQ, int32_t D) {
  WsPtrs p{};
  p.acc = reinterpret_cast<float*>(ws);
  const size_t states =
      pl.mode == DecodePlan::kBalanced ? (size_t)HQ * pl.Wt * 2 : (size_t)B * HQ * pl.NP;
  p.m = p.acc + states * D;
  p.l = p.m + states;
  p.cuc = reinterpret_cast<int32_t*>(p.l + states);
  return p;
}

static int launch_merge(void* out, const DecodePlan& pl, const WsPtrs& w,
                        const int32_t* context_lens, int32_t B, int32_t HQ, int32_t D,
                        pa_dtype dtype, hipStream_t s) {
  dim3 grid(HQ, B), block(D <= 128 ? D : 128);
  if (pl.mode == DecodePlan::kBalanced) {
    if (dtype == PA_BF16)
      hipLaunchKernelGGL(merge_balanced_kernel<true>, grid, block, 0, s, out, w.acc, w.m, w.l,
                         w.cuc, B, HQ, D, pl.Wt);
    else
      hipLaunchKernelGGL(merge_balanced_kernel<false>, grid, block, 0, s, out, w.acc, w.m, w.l,
                         w.cuc, B, HQ, D, pl.Wt);
  } else {
    if (dtype == PA_BF16)
      hipLaunchKernelGGL(merge_kernel<true>, grid, block, 0, s, out, w.acc, w.m, w.l, context_lens,
                         HQ, D, pl.NP, pl.P);
    else
      hipLaunchKernelGGL(merge_kernel<false>, grid, block, 0, s, out, w.acc, w.m, w.l,
                         context_lens, HQ, D, pl.NP, pl.P);
  }
  return check_launch("decode merge");
}

// First pass for any plan; kSingle writes `out` directly.
static int launch_decode(const char* fn, const DecodePlan& pl, void* out, const void* q,
                         const void* k_cache, const void* v_cache, const int32_t* block_table,
                         int32_t maxb, const int32_t* context_lens, int32_t B, int32_t NB,
                         int32_t bs, int32_t HQ, int32_t HKV, int32_t D, float scale,
                         pa_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t s) {
  if (pl.mode != DecodePlan::kSingle && (!workspace || workspace_bytes < pl.ws_bytes))
    return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes,
                pl.ws_bytes);
  decode_fn kern;
  balanced_fn bkern;
  pick_decode(D, dtype, pl.G, &kern, &bkern);
  if (!kern) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for head tile %d", fn, pl.G);
  const int group = HQ / HKV;
  const int head_waves = HKV * (group / pl.G);
  const int wpb = head_waves < max_head_waves(pl.G) ? head_waves : max_head_waves(pl.G);
  const int groups = (head_waves + wpb - 1) / wpb;
  const WsPtrs w = pl.mode == DecodePlan::kSingle ? WsPtrs{} : carve(workspace, pl, B, HQ, D);
  if (pl.mode == DecodePlan::kBalanced) {
    const size_t lds = (size_t)(2 * B + 1) * sizeof(int);
    hipLaunchKernelGGL(bkern, dim3(pl.Wt, groups), dim3(wpb * 64), lds, s, out, w.acc, w.m, w.l,
                       w.cuc, q, k_cache, v_cache, block_table, maxb, context_lens, B, NB,
                       __builtin_ctz(bs), HQ, HKV, group, scale * kLog2e, pl.Wt);
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
