// a3/a4: paged decode attention with split-K partitions and a log-sum-exp merge (gfx950).
//
// What is computed follows "mini-vLLM v0.4" (shadowgraph.io) section 5: for each
// query head, walk the sequence's block table, keep the online-softmax state
// (running max m, exp-sum l, weighted V sum acc) and never materialise a
// contiguous K/V copy; KV head = q head / group size.  The partition states
// are merged with the rescaling of the nano-vLLM lab manual's Fig. B-5.
//
// Work decomposition (MI355X-specific, not from the pages):
//   grid = (partition, kv head x head tile, sequence); 4 waves per workgroup.
//   One workgroup serves every query head of a GQA group, so each K/V byte is
//   fetched from HBM once.  Within a wave, LANES lanes hold one token row
//   (16 bytes each: a 128-dim bf16 row is 16 lanes), so a wave load covers RG
//   consecutive tokens with fully used 16-byte accesses; q.k is reduced over
//   the LANES lanes with DPP row moves.  The wave keeps one softmax state per
//   row group (no cross-lane max per token) and folds the row groups and the
//   waves together once, at the end.
#include "pa_internal.h"

namespace pa {

template <bool BF16>
struct Elem;
template <>
struct Elem<true> {
  static constexpr int VEC = 8;  // bf16 per 16-byte load
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
  static constexpr int VEC = 4;  // fp32 per 16-byte load
  __device__ static void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  __device__ static void store(void* out, int64_t idx, float v) {
    reinterpret_cast<float*>(out)[idx] = v;
  }
};

constexpr int kDecodeWaves = 4;
constexpr int kLoadsPerChunk = 4;

template <int D, bool BF16, int G>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_kernel(
    void* __restrict__ out, float* __restrict__ ws_acc, float* __restrict__ ws_m,
    float* __restrict__ ws_l, const void* __restrict__ qptr, const void* __restrict__ kcache,
    const void* __restrict__ vcache, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ context_lens, int num_blocks, int bs_log2, int HQ, int HKV,
    int group, float scale_log2, int part_size, int NP, int split) {
  using E = Elem<BF16>;
  constexpr int VEC = E::VEC;
  constexpr int LANES = D / VEC;  // lanes per token row
  constexpr int RG = 64 / LANES;  // token rows per wave load
  constexpr int U = kLoadsPerChunk;
  constexpr int CH = RG * U;  // tokens per wave per chunk
  constexpr int NW = kDecodeWaves;
  constexpr int ESZ = BF16 ? 2 : 4;

  __shared__ float s_acc[NW][G][D];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  __shared__ int s_bad[NW];

  const int p = blockIdx.x;
  const int tiles = group / G;
  const int g = blockIdx.y / tiles;
  const int h0 = g * group + (blockIdx.y % tiles) * G;
  const int b = blockIdx.z;
  const int L = context_lens[b];
  const int start = split ? p * part_size : 0;
  const int end = split ? min(start + part_size, L) : L;
  if (start >= end) {
    if (!split) {  // empty context: the output row is zero
      for (int i = threadIdx.x; i < G * D; i += NW * 64)
        E::store(out, ((int64_t)b * HQ + h0 + i / D) * D + i % D, 0.0f);
    }
    return;
  }

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LANES;  // row group
  const int sl = lane % LANES;  // 16-byte slice of the row
  const int bs_mask = (1 << bs_log2) - 1;

  // q for the G heads, pre-multiplied by scale * log2(e) so scores are base-2 exponents.
  float qf[G][VEC];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const char* src = reinterpret_cast<const char*>(qptr) +
                      (((int64_t)b * HQ + h0 + j) * D + sl * VEC) * ESZ;
    E::widen(*reinterpret_cast<const uint4*>(src), qf[j]);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[j][e] *= scale_log2;
  }

  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[j][e] = 0.0f;
  }
  int bad = 0;

  const char* kc = reinterpret_cast<const char*>(kcache);
  const char* vc = reinterpret_cast<const char*>(vcache);
  const int32_t* bt = block_table + (int64_t)b * maxb;

  for (int c = start + w * CH; c < end; c += NW * CH) {
    uint4 kr[U], vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok0 = c + u * RG;  // wave-uniform; RG-aligned, so one block
      const int t = tok0 + r;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      valid[u] = false;
      if (tok0 < end) {
        const int jb = tok0 >> bs_log2;
        const int blk = jb < maxb ? bt[jb] : -1;
        if (blk < 0 || blk >= num_blocks) {
          bad = 1;
        } else if (t < end) {
          const int64_t off =
              (((((int64_t)blk << bs_log2) + (t & bs_mask)) * HKV + g) * D + sl * VEC) * ESZ;
          kr[u] = *reinterpret_cast<const uint4*>(kc + off);
          vr[u] = *reinterpret_cast<const uint4*>(vc + off);
          valid[u] = true;
        }
      }
    }
    float sc[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      E::widen(kr[u], kf);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d = fmaf(qf[j][e], kf[e], d);
        d = group_sum<LANES>(d);
        sc[u][j] = valid[u] ? d : -INFINITY;
      }
    }
    float vf[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) E::widen(vr[u], vf[u]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mx = sc[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][j]);
      const float mnew = fmaxf(m[j], mx);
      const float msafe = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = fast_exp2(m[j] - msafe);
      float ps[U], psum = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ps[u] = fast_exp2(sc[u][j] - msafe);
        psum += ps[u];
      }
      l[j] = l[j] * alpha + psum;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        float a = acc[j][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) a = fmaf(ps[u], vf[u][e], a);
        acc[j][e] = a;
      }
      m[j] = mnew;
    }
  }

  // Fold the row groups of this wave: rescale to the wave max, then sum.
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
  if (r == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) s_acc[w][j][sl * VEC + e] = acc[j][e];
      if (sl == 0) {
        s_m[w][j] = m[j];
        s_l[w][j] = l[j];
      }
    }
  }
  if (lane == 0) s_bad[w] = bad;
  __syncthreads();

  // Fold the waves and write either the partition state or the final output.
  int any_bad = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) any_bad |= s_bad[v];
  for (int i = threadIdx.x; i < G * D; i += NW * 64) {
    const int j = i / D, d = i % D;
    float M = s_m[0][j];
#pragma unroll
    for (int v = 1; v < NW; ++v) M = fmaxf(M, s_m[v][j]);
    float A = 0.0f, Lt = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float f = s_m[v][j] == -INFINITY ? 0.0f : fast_exp2(s_m[v][j] - M);
      A = fmaf(f, s_acc[v][j][d], A);
      Lt = fmaf(f, s_l[v][j], Lt);
    }
    if (any_bad) A = NAN;
    const int64_t bh = (int64_t)b * HQ + h0 + j;
    if (split) {
      ws_acc[(bh * NP + p) * D + d] = A;
      if (d == 0) {
        ws_m[bh * NP + p] = M * kLn2;  // back to natural-log units
        ws_l[bh * NP + p] = Lt;
      }
    } else {
      E::store(out, bh * D + d, A / Lt);
    }
  }
}

// Second pass: one workgroup per (query head, sequence), one thread per output element.
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

typedef void (*decode_fn)(void*, float*, float*, float*, const void*, const void*, const void*,
                          const int32_t*, int, const int32_t*, int, int, int, int, int, float, int,
                          int, int);

template <int D, bool BF16>
static decode_fn pick_g(int G) {
  switch (G) {
    case 1: return decode_kernel<D, BF16, 1>;
    case 2: return decode_kernel<D, BF16, 2>;
    case 3: return decode_kernel<D, BF16, 3>;
    case 4: return decode_kernel<D, BF16, 4>;
    case 5: return decode_kernel<D, BF16, 5>;
    case 6: return decode_kernel<D, BF16, 6>;
    case 7: return decode_kernel<D, BF16, 7>;
    case 8: return decode_kernel<D, BF16, 8>;
  }
  return nullptr;
}

static decode_fn pick_decode(int D, pa_dtype dt, int G) {
  if (dt == PA_BF16) return D == 64 ? pick_g<64, true>(G) : pick_g<128, true>(G);
  return D == 64 ? pick_g<64, false>(G) : pick_g<128, false>(G);
}

// Heads per workgroup: the largest divisor of the GQA group that is <= 8.
static int head_tile(int group) {
  for (int t = 8; t > 1; --t)
    if (group % t == 0) return t;
  return 1;
}

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int32_t auto_partition(int32_t B, int32_t HKV, int32_t max_ctx) {
  // Aim for about 64 (sequence, kv head, partition) work items per compute
  // unit with partitions of at least 256 tokens.
  const int64_t target = 64LL * kNumCUs;
  const int64_t units = (int64_t)B * HKV;
  int64_t P = 256;
  while (P < max_ctx && units * ceil_div(max_ctx, P) > target) P *= 2;
  return (int32_t)P;
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

static int launch_merge(void* out, const float* acc, const float* m, const float* l,
                        const int32_t* context_lens, int32_t B, int32_t HQ, int32_t D, int NP,
                        int32_t P, pa_dtype dtype, hipStream_t stream) {
  dim3 grid(HQ, B), block(D <= 128 ? D : 128);
  if (dtype == PA_BF16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, block, 0, stream, out, acc, m, l, context_lens, HQ,
                       D, NP, P);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, block, 0, stream, out, acc, m, l, context_lens,
                       HQ, D, NP, P);
  return check_launch("decode merge");
}

// Shared by pa_decode and pa_decode_partitions.  P <= 0 or P >= max_context_len
// means one partition per sequence, written straight to `out`.
static int launch_decode(const char* fn, void* out, const void* q, const void* k_cache,
                         const void* v_cache, const int32_t* block_table, int32_t maxb,
                         const int32_t* context_lens, int32_t B, int32_t max_ctx, int32_t NB,
                         int32_t bs, int32_t HQ, int32_t HKV, int32_t D, float scale,
                         pa_dtype dtype, int32_t P, void* workspace, size_t workspace_bytes,
                         hipStream_t s, bool* split_out) {
  const bool split = P > 0 && P < max_ctx;
  *split_out = split;
  const int NP = split ? (int)ceil_div(max_ctx, P) : 1;
  float *acc = nullptr, *mm = nullptr, *ll = nullptr;
  if (split) {
    const size_t need = pa_decode_workspace_size(B, HQ, D, max_ctx, P);
    if (!workspace || workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
    acc = reinterpret_cast<float*>(workspace);
    mm = acc + (size_t)B * HQ * NP * D;
    ll = mm + (size_t)B * HQ * NP;
  }
  const int group = HQ / HKV;
  const int G = head_tile(group);
  decode_fn kern = pick_decode(D, dtype, G);
  if (!kern) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for head tile %d", fn, G);
  dim3 grid(NP, HKV * (group / G), B);
  hipLaunchKernelGGL(kern, grid, dim3(kDecodeWaves * 64), 0, s, out, acc, mm, ll, q, k_cache,
                     v_cache, block_table, maxb, context_lens, NB, __builtin_ctz(bs), HQ, HKV,
                     group, scale * kLog2e, split ? P : 0, NP, split ? 1 : 0);
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
  if (maxb <= 0 || NB < 0)
    return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq %d, num_blocks %d", fn, maxb, NB);
  if (B == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !context_lens)
    return fail(PA_ERR_NULL, "%s: null pointer", fn);
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (workspace && !aligned16(workspace)))
    return fail(PA_ERR_ALIGN, "%s: pointers must be 16-byte aligned", fn);
  return PA_OK;
}

static int32_t resolve_max_ctx(int32_t max_ctx, int32_t maxb, int32_t bs) {
  if (max_ctx > 0) return max_ctx;
  const int64_t t = (int64_t)maxb * bs;
  return (int32_t)(t < INT32_MAX ? t : INT32_MAX);
}

}  // namespace pa

using namespace pa;

extern "C" int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                            int32_t max_context_len, int32_t block_size) {
  clear_error();
  if (num_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0)
    return -fail(PA_ERR_SHAPE, "pa_decode_partition_size: bad sizes");
  if (!is_pow2(block_size)) return -fail(PA_ERR_UNSUPPORTED, "pa_decode_partition_size: block_size");
  const int32_t P = auto_partition(num_seqs, num_kv_heads, max_context_len);
  return P;
}

extern "C" size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                           int32_t head_dim, int32_t max_context_len,
                                           int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0 ||
      partition_size <= 0 || partition_size >= max_context_len)
    return 0;
  const int64_t NP = ceil_div(max_context_len, partition_size);
  return (size_t)num_seqs * num_q_heads * NP * (head_dim + 2) * sizeof(float);
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
  max_context_len = resolve_max_ctx(max_context_len, max_blocks_per_seq, block_size);
  int32_t P;
  if (partition_size == 0) {
    P = auto_partition(num_seqs, num_kv_heads, max_context_len);
    if (P < max_context_len && !workspace) P = -1;  // no workspace: single pass
  } else if (partition_size == -1) {
    P = -1;
  } else {
    if (!is_pow2(partition_size) || partition_size < 16)
      return fail(PA_ERR_UNSUPPORTED, "pa_decode: partition_size %d not a power of two >= 16",
                  partition_size);
    P = partition_size;
  }
  const hipStream_t s = (hipStream_t)stream;
  bool split = false;
  st = launch_decode("pa_decode", out, q, k_cache, v_cache, block_table, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, num_blocks, block_size, num_q_heads,
                     num_kv_heads, head_dim, scale, dtype, P, workspace, workspace_bytes, s, &split);
  if (st || !split) return st;
  const int NP = (int)ceil_div(max_context_len, P);
  const float* acc = reinterpret_cast<const float*>(workspace);
  const float* mm = acc + (size_t)num_seqs * num_q_heads * NP * head_dim;
  const float* ll = mm + (size_t)num_seqs * num_q_heads * NP;
  return launch_merge(out, acc, mm, ll, context_lens, num_seqs, num_q_heads, head_dim, NP, P,
                      dtype, s);
}

extern "C" int pa_decode_partitions(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, int32_t max_blocks_per_seq,
                                    const int32_t* context_lens, int32_t num_seqs,
                                    int32_t max_context_len, int32_t num_blocks,
                                    int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, float scale, pa_dtype dtype,
                                    int32_t partition_size, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  clear_error();
  int st = validate_decode("pa_decode_partitions", q, k_cache, v_cache, block_table,
                           max_blocks_per_seq, context_lens, num_seqs, num_blocks, block_size,
                           num_q_heads, num_kv_heads, head_dim, dtype, workspace);
  if (st || num_seqs == 0) return st;
  max_context_len = resolve_max_ctx(max_context_len, max_blocks_per_seq, block_size);
  if (!is_pow2(partition_size) || partition_size < 16 || partition_size >= max_context_len)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_decode_partitions: partition_size %d must be a power of two >= 16 and < "
                "max_context_len %d", partition_size, max_context_len);
  bool split = false;
  return launch_decode("pa_decode_partitions", nullptr, q, k_cache, v_cache, block_table,
                       max_blocks_per_seq, context_lens, num_seqs, max_context_len, num_blocks,
                       block_size, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                       partition_size, workspace, workspace_bytes, (hipStream_t)stream, &split);
}

extern "C" int pa_decode_merge(void* out, const void* workspace, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                               int32_t max_context_len, int32_t partition_size, pa_dtype dtype,
                               void* stream) {
  clear_error();
  int st = validate_common("pa_decode_merge", num_seqs, num_q_heads, 1, head_dim, dtype);
  if (st) return st;
  if (max_context_len <= 0 || partition_size <= 0)
    return fail(PA_ERR_SHAPE, "pa_decode_merge: max_context_len %d, partition_size %d",
                max_context_len, partition_size);
  if (num_seqs == 0) return PA_OK;
  if (!out || !workspace || !context_lens) return fail(PA_ERR_NULL, "pa_decode_merge: null pointer");
  if (!aligned16(out) || !aligned16(workspace))
    return fail(PA_ERR_ALIGN, "pa_decode_merge: pointers must be 16-byte aligned");
  const int NP = (int)ceil_div(max_context_len, partition_size);
  const float* acc = reinterpret_cast<const float*>(workspace);
  const float* mm = acc + (size_t)num_seqs * num_q_heads * NP * head_dim;
  const float* ll = mm + (size_t)num_seqs * num_q_heads * NP;
  return launch_merge(out, acc, mm, ll, context_lens, num_seqs, num_q_heads, head_dim, NP,
                      partition_size, dtype, (hipStream_t)stream);
}
