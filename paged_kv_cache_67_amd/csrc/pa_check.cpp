// Debug checks of the device-side contract (slot values, block ids, lengths): the
// metadata is copied to the host after the stream has drained and checked there.  The
// kernels never need these (they stay in bounds whatever the metadata holds); they name
// the first broken rule of a batch, for debugging and tests.  With the checks switched on
// (PA_DEBUG_CHECKS set to anything but "0" in the environment when the library first looks,
// or pa_set_debug_checks(1)), pa_store_kv, pa_store_kv_paged, pa_decode, pa_decode_partitions,
// pa_decode_append(_partitions), pa_prefill_paged and pa_attention_mixed run them before every
// launch, which synchronises the stream and so cannot be captured in a graph.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <unordered_set>
#include <vector>

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

// -1: not looked at yet; 0 / 1: off / on.
static std::atomic<int> g_debug{-1};

bool debug_checks() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("PA_DEBUG_CHECKS");
    const int env = e && *e && strcmp(e, "0") != 0 ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, env);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v == 1;
}

// Copies n int32 values from device memory after the stream has drained.
static int fetch(std::vector<int32_t>& dst, const int32_t* src, int64_t n, hipStream_t s,
                 const char* what) {
  dst.assign((size_t)n, 0);
  if (n == 0) return PA_OK;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(dst.data(), src, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: copy to host failed: %s", what, hipGetErrorString(e));
  return PA_OK;
}

// Block ids of the first nblk entries of each row lie in [0, num_blocks).
static int check_rows(const std::vector<int32_t>& bt, int32_t maxb, int32_t b, int64_t nblk,
                      int32_t num_blocks, const char* what) {
  if (nblk > maxb)
    return fail(PA_ERR_CONTRACT, "%s: sequence %d needs %lld blocks, table rows hold %d", what, b,
                (long long)nblk, maxb);
  for (int64_t i = 0; i < nblk; ++i) {
    const int32_t v = bt[(size_t)b * maxb + i];
    if (v < 0 || v >= num_blocks)
      return fail(PA_ERR_CONTRACT, "%s: block_table[%d][%lld] = %d outside [0, %d)", what, b,
                  (long long)i, v, num_blocks);
  }
  return PA_OK;
}

int check_append_slots(const int32_t* block_table, int32_t maxb, const int32_t* context_lens,
                       int32_t B, int32_t num_blocks, int32_t block_size, hipStream_t s) {
  const char* what = "pa_decode_append";
  std::vector<int32_t> ctx, bt;
  if (int st = fetch(ctx, context_lens, B, s, what)) return st;
  if (int st = fetch(bt, block_table, (int64_t)B * maxb, s, what)) return st;
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < B; ++b) {
    if (ctx[b] <= 0) continue;
    const int64_t p = (int64_t)ctx[b] - 1;
    if (p / block_size >= maxb) continue;  // pa_check_decode_inputs names it
    const int32_t blk = bt[(size_t)b * maxb + p / block_size];
    if (blk < 0 || blk >= num_blocks) continue;  // pa_check_decode_inputs names it
    if (!seen.insert((int64_t)blk * block_size + p % block_size).second)
      return fail(PA_ERR_CONTRACT, "%s: the new rows of two sequences share slot %lld (sequence %d)",
                  what, (long long)((int64_t)blk * block_size + p % block_size), b);
  }
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {

int pa_set_debug_checks(int on) {
  const int prev = debug_checks() ? 1 : 0;
  g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}

int pa_check_store_inputs(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                          int32_t block_size, void* stream) {
  clear_error();
  const char* what = "pa_check_store_inputs";
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes", what);
  if (num_tokens > 0 && !slot_mapping) return fail(PA_ERR_NULL, "%s: null slot_mapping", what);
  std::vector<int32_t> slots;
  if (int st = fetch(slots, slot_mapping, num_tokens, (hipStream_t)stream, what)) return st;
  const int64_t nslots = (int64_t)num_blocks * block_size;
  std::unordered_set<int32_t> seen;
  for (int32_t t = 0; t < num_tokens; ++t) {
    const int32_t s = slots[t];
    if (s == -1) continue;
    if (s < 0 || s >= nslots)
      return fail(PA_ERR_CONTRACT, "%s: slot_mapping[%d] = %d outside {-1} and [0, %lld)", what, t, s,
                  (long long)nslots);
    if (!seen.insert(s).second)
      return fail(PA_ERR_CONTRACT, "%s: slot %d appears twice (token %d)", what, s, t);
  }
  return PA_OK;
}

int pa_check_store_paged_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_blocks,
                                int32_t block_size, void* stream) {
  clear_error();
  const char* what = "pa_check_store_paged_inputs";
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0 || num_blocks < 0 ||
      block_size <= 0 || (block_size & (block_size - 1)))
    return fail(PA_ERR_SHAPE, "%s: bad sizes", what);
  if (num_seqs > 0 && (!block_table || !cu_seqlens_q || !seq_lens_k))
    return fail(PA_ERR_NULL, "%s: null pointer", what);
  if (num_seqs == 0) return PA_OK;
  std::vector<int32_t> cq, lk, bt;
  hipStream_t s = (hipStream_t)stream;
  if (int st = fetch(cq, cu_seqlens_q, num_seqs + 1, s, what)) return st;
  if (int st = fetch(lk, seq_lens_k, num_seqs, s, what)) return st;
  if (int st = fetch(bt, block_table, (int64_t)num_seqs * max_blocks_per_seq, s, what)) return st;
  if (cq[0] < 0 || cq[num_seqs] > num_tokens)
    return fail(PA_ERR_CONTRACT, "%s: cu_seqlens_q spans [%d, %d], outside [0, %d]", what, cq[0],
                cq[num_seqs], num_tokens);
  // The slots the store writes, as the kernel computes them (-1 for a token whose logical
  // block is unmapped): no two tokens may write one slot.
  std::unordered_set<int64_t> seen;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t lq = cq[b + 1] - cq[b];
    if (lq < 0) return fail(PA_ERR_CONTRACT, "%s: cu_seqlens_q decreases at sequence %d", what, b);
    for (int32_t i = 0; i < lq; ++i) {
      const int64_t p = (int64_t)lk[b] - lq + i;
      if (p < 0 || p / block_size >= max_blocks_per_seq) continue;
      const int32_t blk = bt[(size_t)b * max_blocks_per_seq + p / block_size];
      if (blk < 0 || blk >= num_blocks) continue;
      const int64_t slot = (int64_t)blk * block_size + p % block_size;
      if (!seen.insert(slot).second)
        return fail(PA_ERR_CONTRACT, "%s: slot %lld written twice (sequence %d, token %d)", what,
                    (long long)slot, b, cq[b] + i);
    }
  }
  return PA_OK;
}

int pa_check_decode_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           int32_t num_blocks, int32_t block_size, void* stream) {
  clear_error();
  const char* what = "pa_check_decode_inputs";
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes", what);
  if (num_seqs > 0 && (!block_table || !context_lens))
    return fail(PA_ERR_NULL, "%s: null pointer", what);
  std::vector<int32_t> ctx, bt;
  hipStream_t s = (hipStream_t)stream;
  if (int st = fetch(ctx, context_lens, num_seqs, s, what)) return st;
  if (int st = fetch(bt, block_table, (int64_t)num_seqs * max_blocks_per_seq, s, what)) return st;
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  const int64_t lim = max_context_len > 0 ? (max_context_len < cap ? max_context_len : cap) : cap;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (ctx[b] < 0 || ctx[b] > lim)
      return fail(PA_ERR_CONTRACT, "%s: context_lens[%d] = %d outside [0, %lld]", what, b, ctx[b],
                  (long long)lim);
    if (int st = check_rows(bt, max_blocks_per_seq, b, ((int64_t)ctx[b] + block_size - 1) / block_size,
                            num_blocks, what))
      return st;
  }
  return PA_OK;
}

int pa_check_prefill_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                            void* stream) {
  clear_error();
  const char* what = "pa_check_prefill_inputs";
  if (num_seqs < 0 || total_q < 0 || max_blocks_per_seq <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(PA_ERR_SHAPE, "%s: bad sizes", what);
  if (num_seqs > 0 && (!block_table || !cu_seqlens_q || !cu_seqlens_k))
    return fail(PA_ERR_NULL, "%s: null pointer", what);
  if (num_seqs == 0) return PA_OK;
  std::vector<int32_t> cq, ck, bt;
  hipStream_t s = (hipStream_t)stream;
  if (int st = fetch(cq, cu_seqlens_q, num_seqs + 1, s, what)) return st;
  if (int st = fetch(ck, cu_seqlens_k, num_seqs + 1, s, what)) return st;
  if (int st = fetch(bt, block_table, (int64_t)num_seqs * max_blocks_per_seq, s, what)) return st;
  if (cq[0] < 0 || cq[num_seqs] > total_q)
    return fail(PA_ERR_CONTRACT, "%s: cu_seqlens_q spans [%d, %d], outside [0, %d]", what, cq[0],
                cq[num_seqs], total_q);
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t lq = cq[b + 1] - cq[b], lk = ck[b + 1] - ck[b];
    if (lq < 0 || lk < 0)
      return fail(PA_ERR_CONTRACT, "%s: cu_seqlens decrease at sequence %d", what, b);
    if (lq > max_seqlen_q || lk > max_seqlen_k)
      return fail(PA_ERR_CONTRACT, "%s: sequence %d has %d queries / %d keys, above %d / %d", what, b,
                  lq, lk, max_seqlen_q, max_seqlen_k);
    if (lk < lq)
      return fail(PA_ERR_CONTRACT, "%s: sequence %d has fewer keys (%d) than queries (%d)", what, b,
                  lk, lq);
    if (int st = check_rows(bt, max_blocks_per_seq, b, ((int64_t)lk + block_size - 1) / block_size,
                            num_blocks, what))
      return st;
  }
  return PA_OK;
}

}  // extern "C"
