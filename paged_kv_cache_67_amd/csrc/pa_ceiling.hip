// Read ceiling of the decode pass (gfx950): a measurement helper beside the attention path.
//
// The decode pass reads every live K and V row of the pool once, scattered over whole pool
// blocks ("大模型推理引擎学习入门-2 ... nano-vllm 的 KV Cache 以及 Paged Attention", section
// 3.1: a block holds block_size token rows of [kv_heads][head_dim]).  This kernel makes
// exactly those reads for a list of blocks and nothing else: a wave per KV head reads that
// head's head_dim slice of every token row, 16 bytes per lane with non-temporal loads, as
// the balanced decode does, and folds what it loaded into one XOR word so that no load can
// be dropped.  Its bandwidth is what the decode's own reads can reach on the part, the
// ceiling the decode is reported against beside the vendor's 8 TB/s.
#include "pa_internal.h"

namespace pa {

constexpr int kCeilWaves = 8;  // waves per workgroup, one KV head each (heads strided)
constexpr int kCeilLoads = 8;  // 16-byte loads in flight per lane, for K and for V each

// CPR: 16-byte chunks of one head's row (head_dim * element size / 16).
template <int CPR>
__global__ __launch_bounds__(kCeilWaves * 64) void read_ceiling_kernel(
    const uint4* __restrict__ kc, const uint4* __restrict__ vc, const int32_t* __restrict__ ids,
    int num_ids, int num_blocks, int block_size, int HKV, uint32_t* __restrict__ sink) {
  constexpr int RPL = 64 / CPR;  // token rows per wave-wide load
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row_chunks = (int64_t)HKV * CPR;
  const int64_t block_chunks = (int64_t)block_size * row_chunks;
  uint32_t acc = 0;
  for (int j = blockIdx.x; j < num_ids; j += gridDim.x) {
    const int b = __builtin_amdgcn_readfirstlane(ids[j]);
    if (b < 0 || b >= num_blocks) continue;
    for (int h = wave; h < HKV; h += kCeilWaves) {
      const int64_t base = (int64_t)b * block_chunks + (int64_t)(lane / CPR) * row_chunks +
                           (int64_t)h * CPR + lane % CPR;
      for (int t0 = 0; t0 < block_size; t0 += RPL * kCeilLoads) {
        uint4 k[kCeilLoads], v[kCeilLoads];
#pragma unroll
        for (int u = 0; u < kCeilLoads; ++u) {
          // block_size is a power of two >= 8 >= RPL, so a row group starting below
          // block_size lies inside the block.
          const int t = t0 + u * RPL;
          const int64_t c = base + (int64_t)t * row_chunks;
          k[u] = t < block_size ? load_stream16(kc + c) : make_uint4(0, 0, 0, 0);
          v[u] = t < block_size ? load_stream16(vc + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kCeilLoads; ++u)
          acc ^= k[u].x ^ k[u].y ^ k[u].z ^ k[u].w ^ v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if (lane == 0) sink[(int64_t)blockIdx.x * kCeilWaves + wave] = acc;
}

}  // namespace pa

using namespace pa;

extern "C" int pa_read_ceiling(const void* k_cache, const void* v_cache, const int32_t* block_ids,
                               int32_t num_ids, int32_t num_blocks, int32_t block_size,
                               int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                               int32_t num_workgroups, uint32_t* sink, void* stream) {
  clear_error();
  const char* fn = "pa_read_ceiling";
  if (num_ids < 0 || num_blocks < 0 || num_kv_heads <= 0 || num_workgroups <= 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes", fn);
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
  if (!k_cache || !v_cache || !block_ids || !sink) return fail(PA_ERR_NULL, "%s: null pointer", fn);
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return fail(PA_ERR_ALIGN, "%s: caches must be 16-byte aligned, sink 4-byte", fn);
  const int cpr = head_dim * elt_bytes(dtype) / 16;
  const hipStream_t s = (hipStream_t)stream;
  const auto k = reinterpret_cast<const uint4*>(k_cache);
  const auto v = reinterpret_cast<const uint4*>(v_cache);
#define PA_CEIL(C)                                                                            \
  hipLaunchKernelGGL(read_ceiling_kernel<C>, dim3(num_workgroups), dim3(kCeilWaves * 64), 0, \
                     s, k, v, block_ids, num_ids, num_blocks, block_size, num_kv_heads, sink)
  if (cpr == 8) PA_CEIL(8);
  else if (cpr == 16) PA_CEIL(16);
  else PA_CEIL(32);
#undef PA_CEIL
  return check_launch(fn);
}
