// Device side of paged decode: the per-wave online-softmax machinery and the
// balanced split-K body, shared by the decode kernels and the mixed
// prefill + decode launch.  Method and design notes are in pa_decode.hip.
#pragma once

#include "pa_internal.h"

namespace pa {


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Element handling per storage type (ET = pa_dtype).  A lane owns 16 bytes of a
// token row: 8 bf16 / fp16 or 4 fp32 values.  q.k uses v_dot2_f32_bf16 or
// v_dot2_f32_f16 on the packed pairs (products exact, fp32 accumulation); V is
// widened to fp32 for the P.V sums.
template <int ET>
struct Elem;
template <>
struct Elem<PA_BF16> {
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
struct Elem<PA_F16> {
  static constexpr int VEC = 8;
  __device__ static float dot(const uint32_t* q, const uint4& k) {
    float d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q[0]),
                                     __builtin_bit_cast(f16x2_t, k.x), 0.0f, false);
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q[1]), __builtin_bit_cast(f16x2_t, k.y),
                               d, false);
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q[2]), __builtin_bit_cast(f16x2_t, k.z),
                               d, false);
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q[3]), __builtin_bit_cast(f16x2_t, k.w),
                               d, false);
    return d;
  }
  __device__ static void widen(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2_t h = __builtin_bit_cast(f16x2_t, w[i]);
      f[2 * i] = (float)h[0];
      f[2 * i + 1] = (float)h[1];
    }
  }
  __device__ static void store(void* out, int64_t idx, float v) {
    reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
  }
};
template <>
struct Elem<PA_F32> {
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
// Waves of the balanced split over the whole chip (slices x head waves, 8 per workgroup):
// a batch that may read more than the 256 MiB Infinity Cache is bound by HBM and runs
// fastest on 192 of the 256 compute units (measured on the 256-row Qwen3-0.6B decode:
// 346.5 us with 1536 waves, 355.8 us with 2048, 364.1 us with 1280; the skewed 32768 + 7 x 512
// batch: 33.2 us against 34.1 us), while a batch that fits the cache is bound by latency
// and wants every compute unit (batch 64 of Qwen2.5-0.5B: 24.5 us with 2048 waves, 25.7 us
// with 1536).
#ifndef PA_DECODE_WAVE_SLOTS
#define PA_DECODE_WAVE_SLOTS 2048
#endif
#ifndef PA_DECODE_WAVE_SLOTS_HBM
#define PA_DECODE_WAVE_SLOTS_HBM 1536
#endif
constexpr int64_t kInfinityCacheBytes = 256ll << 20;

// Load slots per chunk: wide GQA tiles hold more q / state registers, so they
// take smaller chunks to stay clear of spills and keep two waves per SIMD (a
// tile of 8 heads: one slot; of 7 heads: two, which still fit and run faster).
__host__ __device__ constexpr int loads_per_chunk(int G) {
  return G > 7 ? 1 : (G > 6 ? 2 : (G > 4 ? (PA_DECODE_LOADS > 2 ? PA_DECODE_LOADS / 2 : 1) : PA_DECODE_LOADS));
}
// Head waves per workgroup: 8, or 4 for the widest tiles (a wave may then use
// up to 512 VGPRs).
__host__ __device__ constexpr int max_head_waves(int G) { return G > 6 ? 4 : 8; }
// Tokens per chunk for a kernel instance: rows per load times load slots.
__host__ __device__ constexpr int chunk_tokens(int D, int elt_size, int G) {
  return (64 / (D / (16 / elt_size))) * loads_per_chunk(G);
}

// Query heads per decode wave: the largest divisor of the GQA group that is <= 8.
__host__ __device__ constexpr int head_tile(int group) {
  for (int t = 8; t > 1; --t)
    if (group % t == 0) return t;
  return 1;
}

constexpr int kHeadSlot = 0;  // partial state of a piece whose sequence began before the slice
constexpr int kTailSlot = 1;  // partial state of a piece whose sequence runs past the slice
constexpr int kMaxBalancedSeqs = 8192;  // LDS holds 2 ints per sequence

// The step's new K/V rows of a decode launch that also appends them to the cache: one row
// per sequence, laid out like a cache row (all KV heads), row b at key / value + b * stride
// bytes; kc / vc are the caches they go to.
struct AppendRows {
  const char* key;
  const char* value;
  int64_t key_stride, value_stride;
  char* kc;
  char* vc;
};

template <int U>
struct KVRegs {
  uint4 k[U], v[U];
};

// Per-wave decode state: this wave's q registers and one online-softmax state
// per row group, for G query heads of one KV head.
template <int D, int ET, int G>
struct DecodeWave {
  using E = Elem<ET>;
  static constexpr int VEC = E::VEC;
  static constexpr int LANES = D / VEC;  // lanes per token row
  static constexpr int RG = 64 / LANES;  // token rows per wave load
  static constexpr int U = loads_per_chunk(G);
  static constexpr int CH = RG * U;  // tokens per chunk
  static constexpr int ESZ = ET == PA_F32 ? 4 : 2;

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
      X.k[u] = load_stream16(kc + base + off);  // every K/V byte is read exactly once
      X.v[u] = load_stream16(vc + base + off);
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

  // issue() where key `fresh_t` (end - 1 in a sequence's last chunk, else -1) is the step's
  // new row: every lane whose (clamped) token is fresh_t loads it from nk / nv (the row's
  // first byte) instead of the cache, so the chunk is computed as if the row had been stored
  // first and no lane reads the slot it goes to.  One load path for every chunk: a branch
  // between two would leave the compiler's load counting conservative where they join.
  __device__ __forceinline__ void issue_last(KVRegs<U>& X, int t0, int end, const int* ids,
                                             int fresh_t, const char* nk, const char* nv) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(t0 + u * RG + r, end - 1);
      const bool ok = ids[u] >= 0 && ids[u] < num_blocks;
      bad |= !ok;
      const int64_t base = (int64_t)(ok ? ids[u] : 0) * blk_bytes;
      const uint32_t off = (uint32_t)(t & bs_mask) * row_bytes + lane_off;
      const bool fresh = t == fresh_t;
      X.k[u] = load_stream16(fresh ? nk + lane_off : kc + base + off);
      X.v[u] = load_stream16(fresh ? nv + lane_off : vc + base + off);
    }
  }

  // After the chunk issued by issue_last has been computed: the lanes that hold key end - 1
  // (unclamped) write it to its slot in block `blk` (one 16-byte piece each).  A block id out
  // of range writes nothing; the chunk's loads have already poisoned the row.
  __device__ __forceinline__ void store_new(const KVRegs<U>& X, int t0, int end, int blk,
                                            char* kcw, char* vcw) const {
    if (blk < 0 || blk >= num_blocks) return;
    const int64_t off = (int64_t)blk * blk_bytes + (int64_t)((end - 1) & bs_mask) * row_bytes + lane_off;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t0 + u * RG + r == end - 1) {
        *reinterpret_cast<uint4*>(kcw + off) = X.k[u];
        *reinterpret_cast<uint4*>(vcw + off) = X.v[u];
      }
  }
};

// ---------------------------------------------------------------------------
// Balanced split.  Chunk counts ceil(L_b / CH) are scanned into LDS (one
// workgroup also leaves the scan in the workspace for the merge); slice w of
// each head wave covers flat chunks [w*Cw, (w+1)*Cw).

// Position of one chunk: flat index f, sequence b, chunk j within b, b's chunk
// range [cb, ce), key count L and the q / out row of b.  All wave-uniform.
struct Cursor {
  int f, b, j, cb, ce, L, row;
};

__device__ __forceinline__ int lds_uniform(const int* p) { return __builtin_amdgcn_readfirstlane(*p); }

// s_row == nullptr: the row of sequence b is b.
__device__ __forceinline__ void cursor_load(Cursor& c, int b, const int* s_cuc, const int* s_len,
                                            const int* s_row) {
  c.b = b;
  c.cb = lds_uniform(s_cuc + b);
  c.ce = lds_uniform(s_cuc + b + 1);
  c.L = lds_uniform(s_len + b);
  c.row = s_row ? lds_uniform(s_row + b) : b;
}

// The chunk after c (past the last chunk, b becomes B).
__device__ __forceinline__ Cursor cursor_next(Cursor c, int B, const int* s_cuc, const int* s_len,
                                              const int* s_row) {
  c.f += 1;
  c.j += 1;
  if (c.cb + c.j >= c.ce) {
    int b = c.b + 1;
    while (b < B && lds_uniform(s_cuc + b + 1) == lds_uniform(s_cuc + b)) ++b;  // skip empty sequences
    c.j = 0;
    if (b < B) cursor_load(c, b, s_cuc, s_len, s_row);
    else c.b = B;
  }
  return c;
}

// The length scan of the balanced split, run by wave 0 (threads 0-63) of a workgroup:
// s_mem[0 .. B] = s_cuc, the exclusive prefix sums of the chunk counts ceil(L_b / CH);
// s_mem[B + 1 .. 2B] = s_len, the key counts L_b; VARLEN: s_mem[2B + 1 .. 3B] = s_row, the
// q / out rows.  Each lane sums a contiguous segment of sequences and a wave-wide scan of
// the segment sums gives each segment's offset.  VARLEN: the batch is varlen (cu_q, cu_k);
// a sequence with exactly one query (a decode row, q row cu_q[b]) attends its cu_k length
// of keys, any other sequence counts as empty here, and visit(nq, nk, L) sees each
// sequence's query and key counts and its decode key count.  Otherwise sequence b attends
// context_lens[b] keys with q / out row b.  Returns the total chunk count (every lane).
template <int CH, bool VARLEN, typename Visit>
__device__ __forceinline__ int balanced_scan(int* s_mem, const int32_t* __restrict__ context_lens,
                                              const int32_t* __restrict__ cu_q,
                                              const int32_t* __restrict__ cu_k, int total_q,
                                              int B, Visit visit) {
  int* s_cuc = s_mem;
  int* s_len = s_mem + B + 1;
  int* s_row = s_mem + 2 * B + 1;
  const int lane = threadIdx.x;
  const int seg = (B + 63) / 64;
  const int lo = min(B, lane * seg), hi = min(B, lo + seg);
  int sum = 0;
  for (int i = lo; i < hi; ++i) {
    int L;
    if constexpr (VARLEN) {
      const int q0 = cu_q[i], nq = cu_q[i + 1] - q0, nk = cu_k[i + 1] - cu_k[i];
      L = nq == 1 && q0 >= 0 && q0 < total_q ? max(nk, 0) : 0;
      s_row[i] = q0;
      visit(nq, nk, L);
    } else {
      L = max(context_lens[i], 0);
    }
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
  return __shfl(incl, 63);
}

// One wave's slice of the balanced split, after the length scan (balanced_scan) and a
// barrier: slice w of head wave hw (a KV head and a G-wide tile of its query heads), over
// the tables at s_mem.  write_cuc: this workgroup also leaves s_cuc in the workspace for
// the merge.
template <int D, int ET, int G, bool VARLEN, bool APPEND = false>
__device__ __forceinline__ void decode_balanced_run(
    const int* s_mem, int w, int hw, bool write_cuc, void* __restrict__ out,
    float* __restrict__ ws_acc, float* __restrict__ ws_m, float* __restrict__ ws_l,
    int32_t* __restrict__ ws_cuc, const void* __restrict__ qptr, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ block_table, int maxb, int B,
    int num_blocks, int bs_log2, int HQ, int HKV, int group, float scale_log2, int Wt,
    const AppendRows& ap = AppendRows{}) {
  using W = DecodeWave<D, ET, G>;
  constexpr int CH = W::CH;
  constexpr int U = W::U;
  const int* s_cuc = s_mem;
  const int* s_len = s_mem + B + 1;
  const int* s_row = VARLEN ? s_mem + 2 * B + 1 : nullptr;
  if (write_cuc)
    for (int i = threadIdx.x; i <= B; i += blockDim.x) ws_cuc[i] = s_cuc[i];

  const int tiles = group / G;
  if (hw >= HKV * tiles || w >= Wt) return;
  const int g = hw / tiles;
  const int h0 = g * group + (hw % tiles) * G;
  const int NC = lds_uniform(s_cuc + B);
  const int Cw = (NC + Wt - 1) / Wt;
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
  cursor_load(c0, lo, s_cuc, s_len, s_row);
  c0.f = f_begin;
  c0.j = f_begin - c0.cb;

  W st;
  st.init(kcache, vcache, g, HKV, bs_log2, maxb, num_blocks, scale_log2);
  st.reset();
  st.load_q(qptr, (int64_t)c0.row * HQ + h0);

  auto bt_of = [&](const Cursor& c) { return block_table + (int64_t)c.b * maxb; };
  // APPEND: the cache holds keys [0, L - 1) of each sequence and key L - 1 is the step's new
  // row, which the sequence's last chunk loads from the new rows (issue_last) and one head
  // wave per KV head then stores to its slot (store_new).
  auto iss = [&](KVRegs<U>& X, const Cursor& c, const int* ids) {
    if constexpr (APPEND)
      st.issue_last(X, c.j * CH, c.L, ids, c.cb + c.j + 1 == c.ce ? c.L - 1 : -1,
                    ap.key + (int64_t)c.b * ap.key_stride, ap.value + (int64_t)c.b * ap.value_stride);
    else
      st.issue(X, c.j * CH, c.L, ids);
  };
  // After the chunk at c (held in X): if it closes a piece (its sequence's last chunk or the
  // slice's last chunk), write the piece and start the next sequence's state.
  auto finish = [&](const Cursor& c, const Cursor& next, const KVRegs<U>& X) {
    if (c.cb + c.j + 1 != c.ce && c.f + 1 != f_end) return;
    if constexpr (APPEND)
      if (c.cb + c.j + 1 == c.ce && hw % tiles == 0) {
        const int jb = (c.L - 1) >> bs_log2;
        st.store_new(X, c.j * CH, c.L, jb < maxb ? bt_of(c)[jb] : -1, ap.kc, ap.vc);
      }
    st.fold();
    if (c.cb >= f_begin && c.ce <= f_end) {
      st.store_final(out, (int64_t)c.row * HQ + h0);
    } else {
      const int slot = c.cb < f_begin ? kHeadSlot : kTailSlot;
      st.store_state(ws_acc, ws_m, ws_l, ((int64_t)h0 * Wt + w) * 2 + slot, (int64_t)Wt * 2);
    }
    st.reset();
    if (next.f < f_end) st.load_q(qptr, (int64_t)next.row * HQ + h0);
  };

  // A and B alternate as in decode_kernel; cursors c0 (in A) and c1 (in B).
  const int n = f_end - f_begin;
  KVRegs<U> A, Bv;
  int idsA[U], idsB[U];
  Cursor c1 = cursor_next(c0, B, s_cuc, s_len, s_row);
  st.fetch_ids(bt_of(c0), c0.j * CH, c0.L, idsA);
  iss(A, c0, idsA);
  if (n > 1) st.fetch_ids(bt_of(c1), c1.j * CH, c1.L, idsB);
  for (int k = 0; k < (n - 1) / 2; ++k) {
    iss(Bv, c1, idsB);
    const Cursor c2 = cursor_next(c1, B, s_cuc, s_len, s_row);
    st.fetch_ids(bt_of(c2), c2.j * CH, c2.L, idsA);
    st.compute(A, c0.j * CH, c0.L);
    finish(c0, c1, A);
    iss(A, c2, idsA);
    const Cursor c3 = cursor_next(c2, B, s_cuc, s_len, s_row);
    if (c3.f < f_end) st.fetch_ids(bt_of(c3), c3.j * CH, c3.L, idsB);
    st.compute(Bv, c1.j * CH, c1.L);
    finish(c1, c2, Bv);
    c0 = c2;
    c1 = c3;
  }
  if ((n - 1) & 1) {
    iss(Bv, c1, idsB);
    st.compute(A, c0.j * CH, c0.L);
    finish(c0, c1, A);
    st.compute(Bv, c1.j * CH, c1.L);
    finish(c1, c1, Bv);
  } else {
    st.compute(A, c0.j * CH, c0.L);
    finish(c0, c1, A);
  }
}

// The whole balanced-split slice for a standalone launch: every wave of the workgroup
// takes part in the length scan's barrier, then runs its slice.
template <int D, int ET, int G, bool VARLEN, bool APPEND = false>
__device__ __forceinline__ void decode_balanced_body(
    int w, int hw, bool write_cuc, void* __restrict__ out, float* __restrict__ ws_acc,
    float* __restrict__ ws_m, float* __restrict__ ws_l, int32_t* __restrict__ ws_cuc,
    const void* __restrict__ qptr, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int total_q, int B, int num_blocks, int bs_log2, int HQ,
    int HKV, int group, float scale_log2, int Wt, const AppendRows& ap = AppendRows{}) {
  extern __shared__ int s_mem[];
  if (threadIdx.x < 64)
    balanced_scan<DecodeWave<D, ET, G>::CH, VARLEN>(s_mem, context_lens, cu_q, cu_k, total_q, B,
                                                     [](int, int, int) {});
  __syncthreads();
  decode_balanced_run<D, ET, G, VARLEN, APPEND>(s_mem, w, hw, write_cuc, out, ws_acc, ws_m, ws_l,
                                                ws_cuc, qptr, kcache, vcache, block_table, maxb, B,
                                                num_blocks, bs_log2, HQ, HKV, group, scale_log2,
                                                Wt, ap);
}


// Merge workgroups: 1, 2, 4 or kMergeWaves waves; each wave keeps up to kMergeUnroll pieces'
// loads in flight.
constexpr int kMergeWaves = 8;
constexpr int kMergeUnroll = 8;
// One-wave merges (short rows) run kMergeHeadsPerWG query heads per workgroup: the 256-row
// Qwen3-0.6B decode's merge dispatches 1024 workgroups instead of 4096 (step 347.4-347.6
// against 348.4 us; 8 heads gave the same).
constexpr int kMergeHeadsPerWG = 4;
// Waves per merge workgroup.  A grid of at most one workgroup per compute unit leaves most
// of the chip idle, so the widest workgroup costs nothing there, and it is what a row far
// longer than the rest (which the host cannot see) needs.  A larger grid pays for every
// wave, so it gets the fewest waves whose loads in flight take a typical row's pieces
// (pieces_per_row: the mean, or the most any row can have) in one round.
inline int merge_waves(int64_t pieces_per_row, int64_t workgroups) {
  if (workgroups <= kNumCUs) return kMergeWaves;
  int w = 1;
  while (w < kMergeWaves && (int64_t)w * kMergeUnroll < pieces_per_row) w *= 2;
  return w;
}

// Combines n partial states (m, l, acc[D]) of one output row into out[row .. row + D):
// out = sum_k e^(m_k - M) acc_k / sum_k e^(m_k - M) l_k with M = max_k m_k (m in natural-log
// units, the rescaling identity of the online softmax).  Piece k's m and l sit at ws_m /
// ws_l[idx(k)] and its acc at ws_acc[idx(k) * D].  Wave w takes pieces w, w + W, w + 2W, ...,
// kMergeUnroll at a time with all their loads issued together (slots past n load nothing
// and count zero), keeping a running (M, L, A) that is rescaled when M grows; with
// W > 1 the wave states are combined through LDS.  Lane l holds d = l and, for D = 128,
// d = l + 64.  Must be called by all 64 W threads of the workgroup.
template <int ET, int W, typename Idx>
__device__ __forceinline__ void merge_states(void* __restrict__ out, int64_t row,
                                             const float* __restrict__ ws_acc,
                                             const float* __restrict__ ws_m,
                                             const float* __restrict__ ws_l, int n, int D,
                                             Idx idx) {
  using E = Elem<ET>;
  constexpr int U = kMergeUnroll;
  const int lane = threadIdx.x & 63, w = W == 1 ? 0 : threadIdx.x >> 6;
  const bool two = D > 64;
  constexpr float kFloor = -1.0e30f;  // finite: e^(kFloor - M) is 0, never NaN
  float M = kFloor, L = 0.0f, A0 = 0.0f, A1 = 0.0f;
  for (int k0 = 0; k0 < n; k0 += U * W) {
    float m[U], l[U], a0[U], a1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kk = k0 + w + W * u;
      m[u] = kFloor;
      l[u] = a0[u] = a1[u] = 0.0f;
      if (kk < n) {  // wave-uniform
        const int64_t s = idx(kk);
        m[u] = ws_m[s];
        l[u] = ws_l[s];
        a0[u] = ws_acc[s * D + lane];
        if (two) a1[u] = ws_acc[s * D + 64 + lane];
      }
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < U; ++u) mn = fmaxf(mn, m[u]);
    const float c = fast_exp2((M - mn) * kLog2e);
    L *= c;
    A0 *= c;
    A1 *= c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = fast_exp2((m[u] - mn) * kLog2e);
      L = fmaf(f, l[u], L);
      A0 = fmaf(f, a0[u], A0);
      A1 = fmaf(f, a1[u], A1);
    }
    M = mn;
  }
  if constexpr (W == 1) {
    const float inv = 1.0f / L;
    E::store(out, row + lane, A0 * inv);
    if (two) E::store(out, row + 64 + lane, A1 * inv);
  } else {
    __shared__ float sM[W], sL[W];
    __shared__ float sA[W][128];
    if (lane == 0) {
      sM[w] = M;
      sL[w] = L;
    }
    sA[w][lane] = A0;
    if (two) sA[w][64 + lane] = A1;
    __syncthreads();
    if (w != 0) return;
    float Mt = sM[0];
#pragma unroll
    for (int j = 1; j < W; ++j) Mt = fmaxf(Mt, sM[j]);
    float f[W], Lt = 0.0f;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      f[j] = fast_exp2((sM[j] - Mt) * kLog2e);
      Lt = fmaf(f[j], sL[j], Lt);
    }
    const float inv = 1.0f / Lt;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == 1 && !two) break;
      const int d = lane + 64 * half;
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < W; ++j) a = fmaf(f[j], sA[j][d], a);
      E::store(out, row + d, a * inv);
    }
  }
}


// Balanced split: sequence b spans slices w0 = cb / Cw .. w1 = (ce - 1) / Cw.
// With w0 == w1 the decode pass already wrote the row; otherwise its pieces
// are slice w0's tail state and slices w0+1 .. w1's head states.  VARLEN: only
// the one-query sequences of a varlen batch are decode rows (row cu_q[b]); the
// others belong to the prefill side and are left alone, and the slice count is the one
// the first pass stored after its scan (Wt is then unused).
// HPW (with W = 1): query heads per workgroup, one wave each, so that a batch of short rows
// dispatches HPW times fewer workgroups.
template <int ET, bool VARLEN, int W, int HPW = 1>
__global__ __launch_bounds__(64 * W * HPW) void merge_balanced_kernel(
    void* __restrict__ out, const float* __restrict__ ws_acc, const float* __restrict__ ws_m,
    const float* __restrict__ ws_l, const int32_t* __restrict__ ws_cuc,
    const int32_t* __restrict__ cu_q, int total_q, int B, int HQ, int D, int Wt) {
  static_assert(HPW == 1 || W == 1, "several heads per workgroup only with one wave each");
  using E = Elem<ET>;
  const int h = blockIdx.x * HPW + (HPW > 1 ? (int)(threadIdx.x >> 6) : 0), b = blockIdx.y;
  if (h >= HQ) return;
  int rb = b;
  if constexpr (VARLEN) {
    rb = cu_q[b];
    if (cu_q[b + 1] - rb != 1 || rb < 0 || rb >= total_q) return;
  }
  const int64_t row = ((int64_t)rb * HQ + h) * D;
  const int cb = ws_cuc[b], ce = ws_cuc[b + 1];
  if (cb >= ce) {  // no keys: zero row
    for (int d = threadIdx.x & (64 * W - 1); d < D; d += 64 * W) E::store(out, row + d, 0.0f);
    return;
  }
  const int NC = ws_cuc[B];
  // A mixed launch picks its slice count on the device and leaves it after the scan.
  const int nw = VARLEN ? ws_cuc[B + 1] : Wt;
  const int Cw = (NC + nw - 1) / nw;
  const int w0 = cb / Cw, w1 = (ce - 1) / Cw;
  if (w0 == w1) return;
  // Piece 0 is the tail slot of slice w0, piece k >= 1 the head slot of slice w0 + k.
  const int64_t base = (int64_t)h * nw * 2 + (int64_t)w0 * 2;
  merge_states<ET, W>(out, row, ws_acc, ws_m, ws_l, w1 - w0 + 1, D, [&](int k) {
    return base + 2 * k + (k == 0 ? kTailSlot : kHeadSlot);
  });
}


}  // namespace pa
