// a1 slot addressing, a2 K/V scatter into the paged pool, and whole-block copies (gfx950).
//
// Slot addressing follows "大模型推理引擎学习入门-2 ... nano-vllm 的 KV Cache 以及
// Paged Attention" (juejin.cn) section 3.5: slot = block_table[p / B] * B + p % B.
// The scatter follows the store_kvcache kernel described in "MinivLLM：六步搭出
// 一个 Qwen3 推理引擎" (txtmix.com), section "注意力内核的三个分支": one row per
// token, slot -1 means "do not write".
#include <limits.h>

#include "pa_internal.h"

namespace pa {

// One workgroup per sequence; its threads stride over the sequence's new tokens.
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int32_t* __restrict__ slots, const int32_t* __restrict__ block_table, int maxb,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ lens_k, int num_tokens,
    int bs_log2, int num_blocks) {
  const int b = blockIdx.x;
  const int q0 = cu_q[b];
  const int lq = cu_q[b + 1] - q0;
  const int lk = lens_k[b];
  const int bs = 1 << bs_log2;
  const int32_t* row = block_table + (int64_t)b * maxb;
  for (int i = threadIdx.x; i < lq; i += blockDim.x) {
    const int t = q0 + i;
    if (t < 0 || t >= num_tokens) continue;
    const int p = lk - lq + i;
    int s = -1;
    if (p >= 0 && (p >> bs_log2) < maxb) {
      const int blk = row[p >> bs_log2];
      if (blk >= 0 && blk < num_blocks) s = blk * bs + (p & (bs - 1));
    }
    slots[t] = s;
  }
}

// Flat 16-byte copy: work item = (token, 16-byte chunk of its [kv_heads, head_dim] row).
__global__ __launch_bounds__(256) void store_kv_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride_bytes,
    int64_t value_stride_bytes, char* __restrict__ kc, char* __restrict__ vc,
    const int32_t* __restrict__ slots, int64_t num_items, int row_chunks, int64_t num_slots,
    int64_t row_bytes) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < num_items; i += step) {
    const int64_t t = i / row_chunks;
    const int c = int(i - t * row_chunks);
    const int s = slots[t];
    if (s < 0 || s >= num_slots) continue;
    const uint4 k = reinterpret_cast<const uint4*>(key + t * key_stride_bytes)[c];
    const uint4 v = reinterpret_cast<const uint4*>(value + t * value_stride_bytes)[c];
    reinterpret_cast<uint4*>(kc + (int64_t)s * row_bytes)[c] = k;
    reinterpret_cast<uint4*>(vc + (int64_t)s * row_bytes)[c] = v;
  }
}

// a1 and a2 in one launch.  blockIdx.y strides over the sequences and blockIdx.x x threads
// over the sequence's (new token, 16-byte chunk) items.  Each item computes its token's
// slot as slot_mapping_kernel does (every chunk of a row reads the same lengths and table
// entry, served from cache) and copies its chunk of the K and V rows.  The row loads
// depend only on the token index, so they are in flight while the table entry is read,
// instead of waiting for a separate slot pass and its reread of the slots.
__global__ __launch_bounds__(256) void store_kv_paged_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride_bytes,
    int64_t value_stride_bytes, char* __restrict__ kc, char* __restrict__ vc,
    const int32_t* __restrict__ block_table, int maxb, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ lens_k, int num_seqs, int num_tokens, int bs_log2,
    int num_blocks, int row_chunks, int64_t row_bytes, int32_t* __restrict__ slots_out) {
  const int bs = 1 << bs_log2;
  for (int b = blockIdx.y; b < num_seqs; b += gridDim.y) {
    const int q0 = cu_q ? cu_q[b] : b;  // no cu_q: one token per sequence (token b)
    const int lq = cu_q ? cu_q[b + 1] - q0 : 1;
    const int lk = lens_k[b];
    const int32_t* row = block_table + (int64_t)b * maxb;
    const int64_t items = (int64_t)(lq > 0 ? lq : 0) * row_chunks;
    for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
         it += (int64_t)gridDim.x * blockDim.x) {
      const int i = int(it / row_chunks);
      const int c = int(it - (int64_t)i * row_chunks);
      const int t = q0 + i;
      if (t < 0 || t >= num_tokens) continue;
      const uint4 k = reinterpret_cast<const uint4*>(key + (int64_t)t * key_stride_bytes)[c];
      const uint4 v = reinterpret_cast<const uint4*>(value + (int64_t)t * value_stride_bytes)[c];
      const int p = lk - lq + i;
      int s = -1;
      if (p >= 0 && (p >> bs_log2) < maxb) {
        const int blk = row[p >> bs_log2];
        if (blk >= 0 && blk < num_blocks) s = blk * bs + (p & (bs - 1));
      }
      if (slots_out && c == 0) slots_out[t] = s;
      if (s < 0) continue;
      reinterpret_cast<uint4*>(kc + (int64_t)s * row_bytes)[c] = k;
      reinterpret_cast<uint4*>(vc + (int64_t)s * row_bytes)[c] = v;
    }
  }
}

// Whole-block copy of both pools for a list of (src, dst) block pairs.  blockIdx.y strides
// over the pairs, blockIdx.x x threads over the 16-byte chunks of one block; a pair with an
// id out of range, or src == dst, copies nothing.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* kc, char* vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_pairs, int num_blocks,
                                                          int64_t block_bytes, int chunks) {
  for (int p = blockIdx.y; p < num_pairs; p += gridDim.y) {
    const int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) continue;
    const uint4* ks = reinterpret_cast<const uint4*>(kc + (int64_t)src * block_bytes);
    const uint4* vs = reinterpret_cast<const uint4*>(vc + (int64_t)src * block_bytes);
    uint4* kd = reinterpret_cast<uint4*>(kc + (int64_t)dst * block_bytes);
    uint4* vd = reinterpret_cast<uint4*>(vc + (int64_t)dst * block_bytes);
    for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += gridDim.x * blockDim.x) {
      // Source and destination are touched once: non-temporal loads and stores.
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 k = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + c));
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + c));
      __builtin_nontemporal_store(k, reinterpret_cast<u32x4*>(kd + c));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(vd + c));
    }
  }
}

// Several device copies and zero fills in one launch: the staging of a step's inputs into
// the fixed buffers a captured graph replays over ("5. 动手改造：从跑通到可测量的推理服务",
// B.4: each step's inputs are copied into the captured buffers, then the graph is replayed).
// The descriptors travel by value in the kernel arguments; each is walked in 16-byte
// chunks when its pointers and size allow, else in 4-byte words.
struct CopyList {
  pa_copy_desc d[PA_COPY_MANY_MAX];
  int n;
};

__global__ __launch_bounds__(256) void copy_many_kernel(CopyList list) {
  const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int k = 0; k < list.n; ++k) {
    const pa_copy_desc d = list.d[k];
    const bool wide = ((reinterpret_cast<uintptr_t>(d.src) | reinterpret_cast<uintptr_t>(d.dst) |
                        (uint64_t)d.bytes) & 15) == 0;
    if (wide) {
      const int64_t n = d.bytes / 16;
      const uint4* src = reinterpret_cast<const uint4*>(d.src);
      uint4* dst = reinterpret_cast<uint4*>(d.dst);
      for (int64_t i = first; i < n; i += step) dst[i] = src ? src[i] : make_uint4(0, 0, 0, 0);
    } else {
      const int64_t n = d.bytes / 4;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(d.src);
      uint32_t* dst = reinterpret_cast<uint32_t*>(d.dst);
      for (int64_t i = first; i < n; i += step) dst[i] = src ? src[i] : 0u;
    }
  }
}

}  // namespace pa

using namespace pa;

extern "C" int pa_copy_many(const pa_copy_desc* descs, int32_t count, void* stream) {
  clear_error();
  if (count < 0 || count > PA_COPY_MANY_MAX)
    return fail(PA_ERR_SHAPE, "pa_copy_many: %d descriptors (0 to %d)", count, PA_COPY_MANY_MAX);
  if (count == 0) return PA_OK;
  if (!descs) return fail(PA_ERR_NULL, "pa_copy_many: null descriptor list");
  CopyList list{};
  int64_t most = 0;
  for (int k = 0; k < count; ++k) {
    const pa_copy_desc& d = descs[k];
    if (d.bytes < 0 || d.bytes % 4)
      return fail(PA_ERR_SHAPE, "pa_copy_many: descriptor %d has %lld bytes (a multiple of 4)", k,
                  (long long)d.bytes);
    if (d.bytes > 0 && !d.dst) return fail(PA_ERR_NULL, "pa_copy_many: descriptor %d: null dst", k);
    if ((reinterpret_cast<uintptr_t>(d.src) | reinterpret_cast<uintptr_t>(d.dst)) & 3)
      return fail(PA_ERR_ALIGN, "pa_copy_many: descriptor %d: pointers must be 4-byte aligned", k);
    list.d[k] = d;
    most = d.bytes > most ? d.bytes : most;
  }
  list.n = count;
  if (most == 0) return PA_OK;
  const int64_t chunks = (most + 15) / 16;
  const int64_t blocks = (chunks + 255) / 256;
  const int grid = int(blocks < 1024 ? blocks : 1024);
  hipLaunchKernelGGL(copy_many_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, list);
  return check_launch("pa_copy_many");
}

extern "C" int pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_table,
                               int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                               const int32_t* seq_lens_k, int32_t num_seqs, int32_t num_tokens,
                               int32_t block_size, int32_t num_blocks, void* stream) {
  clear_error();
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_slot_mapping: negative size");
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "pa_slot_mapping: block_size %d not a power of two in [8,1024]",
                block_size);
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_slot_mapping: num_blocks*block_size exceeds int32 slots");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (max_blocks_per_seq == 0) return fail(PA_ERR_SHAPE, "pa_slot_mapping: max_blocks_per_seq is 0");
  if (!slot_mapping || !block_table || !cu_seqlens_q || !seq_lens_k)
    return fail(PA_ERR_NULL, "pa_slot_mapping: null pointer");
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_seqs), dim3(256), 0, (hipStream_t)stream,
                     slot_mapping, block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens_k,
                     num_tokens, __builtin_ctz(block_size), num_blocks);
  return check_launch("pa_slot_mapping");
}

extern "C" int pa_store_kv(const void* key, const void* value, int64_t key_token_stride,
                           int64_t value_token_stride, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                           int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                           pa_dtype dtype, void* stream) {
  clear_error();
  if (num_tokens < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_SHAPE, "pa_store_kv: bad size (tokens %d, blocks %d, kv_heads %d, dim %d)",
                num_tokens, num_blocks, num_kv_heads, head_dim);
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "pa_store_kv: dtype %d", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_store_kv: head_dim %d (64 or 128)", head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "pa_store_kv: block_size %d not a power of two in [8,1024]",
                block_size);
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_store_kv: num_blocks*block_size exceeds int32 slots");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "pa_store_kv: null pointer");
  const int eb = elt_bytes(dtype);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * eb;
  if (key_token_stride < (int64_t)num_kv_heads * head_dim ||
      value_token_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "pa_store_kv: token stride smaller than a row");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (key_token_stride * eb) % 16 || (value_token_stride * eb) % 16)
    return fail(PA_ERR_ALIGN, "pa_store_kv: pointers and token strides must be 16-byte aligned");
  if (debug_checks())
    if (int cs = pa_check_store_inputs(slot_mapping, num_tokens, num_blocks, block_size, stream))
      return cs;
  const int row_chunks = int(row_bytes / 16);
  const int64_t items = (int64_t)num_tokens * row_chunks;
  const int64_t blocks = (items + 255) / 256;
  const int grid = int(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(store_kv_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const char*)key, (const char*)value, key_token_stride * eb,
                     value_token_stride * eb, (char*)k_cache, (char*)v_cache, slot_mapping, items,
                     row_chunks, (int64_t)num_blocks * block_size, row_bytes);
  return check_launch("pa_store_kv");
}

namespace pa {

// The new rows of a decode batch (row b is key context_lens[b] - 1 of sequence b) into the
// cache: the fused store's kernel with one token per sequence.  Inputs already checked.
int launch_store_decode_rows(const void* key, const void* value, int64_t key_stride_bytes,
                             int64_t value_stride_bytes, void* k_cache, void* v_cache,
                             const int32_t* block_table, int32_t maxb,
                             const int32_t* context_lens, int32_t B, int32_t num_blocks,
                             int32_t block_size, int64_t row_bytes, hipStream_t s) {
  const int row_chunks = int(row_bytes / 16);
  const dim3 grid(unsigned((row_chunks + 255) / 256), unsigned(B < 65535 ? B : 65535));
  hipLaunchKernelGGL(store_kv_paged_kernel, grid, dim3(256), 0, s, (const char*)key,
                     (const char*)value, key_stride_bytes, value_stride_bytes, (char*)k_cache,
                     (char*)v_cache, block_table, maxb, nullptr, context_lens, B, B,
                     __builtin_ctz(block_size), num_blocks, row_chunks, row_bytes, nullptr);
  return check_launch("store of the new decode rows");
}

}  // namespace pa

extern "C" int pa_store_kv_paged(const void* key, const void* value, int64_t key_token_stride,
                                 int64_t value_token_stride, void* k_cache, void* v_cache,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_seqlen_q,
                                 int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                 int32_t head_dim, pa_dtype dtype, int32_t* slot_mapping,
                                 void* stream) {
  clear_error();
  const char* fn = "pa_store_kv_paged";
  if (num_seqs < 0 || num_tokens < 0 || max_seqlen_q < 0 || max_blocks_per_seq < 0 ||
      num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes", fn);
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", fn, (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (!is_pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d not a power of two in [8,1024]", fn,
                block_size);
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_SHAPE, "%s: num_blocks*block_size exceeds int32 slots", fn);
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (max_blocks_per_seq == 0) return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq is 0", fn);
  if (!key || !value || !k_cache || !v_cache || !block_table || !cu_seqlens_q || !seq_lens_k)
    return fail(PA_ERR_NULL, "%s: null pointer", fn);
  const int eb = elt_bytes(dtype);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * eb;
  if (key_token_stride < (int64_t)num_kv_heads * head_dim ||
      value_token_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PA_ERR_SHAPE, "%s: token stride smaller than a row", fn);
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (key_token_stride * eb) % 16 || (value_token_stride * eb) % 16 ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 3u))
    return fail(PA_ERR_ALIGN, "%s: pointers and token strides must be 16-byte aligned", fn);
  if (debug_checks())
    if (int cs = pa_check_store_paged_inputs(block_table, max_blocks_per_seq, cu_seqlens_q,
                                             seq_lens_k, num_seqs, num_tokens, num_blocks,
                                             block_size, stream))
      return cs;
  const int row_chunks = int(row_bytes / 16);
  const int64_t per_seq = (int64_t)(max_seqlen_q > 0 ? max_seqlen_q : 1) * row_chunks;
  const int64_t gx = (per_seq + 255) / 256;
  const dim3 grid(unsigned(gx < 1024 ? gx : 1024), unsigned(num_seqs < 65535 ? num_seqs : 65535));
  hipLaunchKernelGGL(store_kv_paged_kernel, grid, dim3(256), 0, (hipStream_t)stream,
                     (const char*)key, (const char*)value, key_token_stride * eb,
                     value_token_stride * eb, (char*)k_cache, (char*)v_cache, block_table,
                     max_blocks_per_seq, cu_seqlens_q, seq_lens_k, num_seqs, num_tokens,
                     __builtin_ctz(block_size), num_blocks, row_chunks, row_bytes, slot_mapping);
  return check_launch(fn);
}

extern "C" int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs,
                              int32_t num_pairs, int32_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                              void* stream) {
  clear_error();
  if (num_pairs < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: bad size (pairs %d, blocks %d, block %d, kv_heads "
                "%d, dim %d)", num_pairs, num_blocks, block_size, num_kv_heads, head_dim);
  if (dtype != PA_F32 && dtype != PA_BF16 && dtype != PA_F16)
    return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: dtype %d", (int)dtype);
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * elt_bytes(dtype);
  if (block_bytes % 16 || block_bytes / 16 > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: block of %lld bytes (a multiple of 16 below "
                "32 GiB)", (long long)block_bytes);
  if (num_pairs == 0 || num_blocks == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_NULL, "pa_copy_blocks: null pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_ALIGN, "pa_copy_blocks: pools must be 16-byte aligned");
  const int chunks = int(block_bytes / 16);
  const int gx = (chunks + 255) / 256;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(gx < 1024 ? gx : 1024, num_pairs < 65535 ? num_pairs : 65535),
                     dim3(256), 0, (hipStream_t)stream, (char*)k_cache, (char*)v_cache, block_pairs,
                     num_pairs, num_blocks, block_bytes, chunks);
  return check_launch("pa_copy_blocks");
}
