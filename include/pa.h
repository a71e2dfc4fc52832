/*
 * pa.h -- paged attention over a block-managed KV cache, for AMD Instinct
 * MI355X (gfx950).  C ABI; every function is extern "C".
 *
 * Sources cited below:
 *   [Lab]      "5. 动手改造：从跑通到可测量的推理服务", the nano-vLLM inference
 *              lab manual (duanmeng.github.io, 实验手册.html), appendix B.
 *   [mini]     "mini-vLLM v0.4 -- From-Scratch LLM Inference Serving Runtime"
 *              (shadowgraph.io/WJX3078/mini-vllm), section 5.
 *   [MinivLLM] "MinivLLM：六步搭出一个 Qwen3 推理引擎，再核清四处文档与代码的分岔"
 *              (txtmix.com), section "注意力内核的三个分支".
 *   [KVblog]   "大模型推理引擎学习入门-2：带你理解 nano-vllm 的 KV Cache 以及
 *              Paged Attention" (juejin.cn), sections 3.1, 3.5 and 4.4.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named *cache*, q, out, key, value, workspace, block_table,
 *   slot_mapping, context_lens, seq_lens_k and cu_seqlens_* are DEVICE
 *   pointers owned by the caller.  The library allocates no device memory,
 *   keeps no pointer after a call returns and has no mutable global state
 *   except a thread-local error message and the process-wide switch of the
 *   debug checks (pa_set_debug_checks, off by default).
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream): it validates its host-side arguments, enqueues its kernels and
 *   returns.  It performs no host<->device copies and no synchronisation
 *   (unless the debug checks are switched on; see pa_check_*).
 *   Inputs must stay alive and unchanged until the stream reaches the work.
 * - KV pool layout ([KVblog] 3.1: kv_cache is (2, layers, num_blocks,
 *   block_size, kv_heads, head_dim); one layer's K or V pool):
 *       cache[num_blocks][block_size][num_kv_heads][head_dim], contiguous.
 *   Logical token t of a sequence lives in block block_table[t / block_size]
 *   at row t % block_size ([MinivLLM], paged_attention_decode_kernel).
 * - block_table is int32 [num_seqs][max_blocks_per_seq], row-major, padded
 *   with -1 past each sequence's last block ([MinivLLM], prepare_decode).
 * - Element types: PA_F32 (float), PA_BF16 (bfloat16 bits) or PA_F16 (IEEE
 *   half); q, out, key, value and both caches share one type.  head_dim is 64
 *   or 128.
 *   block_size is a power of two in [8, 1024].
 * - Base pointers of q, out, key, value, caches and workspace must be 16-byte
 *   aligned.
 * - Arithmetic: fp32 accumulation; bf16 and fp16 results are rounded to
 *   nearest-even.
 * - Device-side contents (slot values, block ids, lengths) are the caller's
 *   contract and are not validated on the host: slot_mapping entries are -1
 *   or in [0, num_blocks*block_size) and distinct; block ids read for live
 *   tokens are in [0, num_blocks); 0 <= context_lens[b] <= max_context_len.
 *   The kernels never read or write outside the buffers their sizes describe
 *   even when the contract is broken: an out-of-range slot is skipped, and a
 *   live token whose block id is out of range turns that sequence's output
 *   into NaN instead of being read.
 * - Return value: a pa_status.  On failure nothing has been enqueued and
 *   pa_last_error() describes the problem.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* a size is negative or sizes are inconsistent */
  PA_ERR_UNSUPPORTED = 3, /* dtype / head_dim / block_size / head ratio without a kernel */
  PA_ERR_ALIGN = 4,       /* a pointer or stride breaks the 16-byte alignment rule */
  PA_ERR_WORKSPACE = 5,   /* workspace smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = 6,         /* the HIP runtime rejected a launch */
  PA_ERR_CAPACITY = 7,    /* block manager: not enough free blocks */
  PA_ERR_CONTRACT = 8     /* pa_check_*: device-side metadata breaks the contract */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2 } pa_dtype;

/* Library version as major*10000 + minor*100 + patch. */
int pa_version(void);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_slot_mapping -- physical cache row of every new token.
 *
 * [KVblog] 3.1 and 3.5, [Lab] B.2.3: the token at logical position p of a
 * sequence is written to row slot = block_table[p / block_size] * block_size
 * + p % block_size of the flattened pool.  Sequence b contributes the new
 * tokens cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; they are its last
 * Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] tokens out of seq_lens_k[b], so
 * new token i sits at p = seq_lens_k[b] - Lq + i (a cached prefix shifts
 * positions, [KVblog] 3.5; a decode step has Lq = 1 and p = context_len - 1,
 * [KVblog] 4.4).
 *
 *   slot_mapping  out  int32 [num_tokens]
 *   block_table   in   int32 [num_seqs][max_blocks_per_seq]
 *   cu_seqlens_q  in   int32 [num_seqs + 1], non-decreasing, cu[0] = 0,
 *                      cu[num_seqs] = num_tokens
 *   seq_lens_k    in   int32 [num_seqs], seq_lens_k[b] >= Lq of b
 *
 * A token whose logical block index is >= max_blocks_per_seq, or whose table
 * entry is outside [0, num_blocks), gets slot -1 (the pages' "do not write"
 * marker).  num_seqs = 0 or num_tokens = 0 is a no-op.
 */
int pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_table,
                    int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                    const int32_t* seq_lens_k, int32_t num_seqs, int32_t num_tokens,
                    int32_t block_size, int32_t num_blocks, void* stream);

/*
 * pa_store_kv -- scatter this step's K and V rows into the paged pool.
 *
 * [MinivLLM] store_kvcache_kernel and [KVblog] 3.1 (the physical layer):
 * for every token t with s = slot_mapping[t] != -1,
 *   k_cache[s / block_size][s % block_size][:][:] = key[t][:][:]
 *   v_cache[s / block_size][s % block_size][:][:] = value[t][:][:]
 * A bitwise copy.  Slots outside [0, num_blocks*block_size) are skipped like
 * -1.  Two tokens must not share a slot.
 *
 *   key, value   in   [num_tokens][num_kv_heads][head_dim]; the [kv_heads,
 *                     head_dim] row of a token is contiguous and consecutive
 *                     tokens are key_token_stride / value_token_stride
 *                     ELEMENTS apart (so views into a fused qkv tensor work);
 *                     the strides times the element size must be multiples
 *                     of 16 bytes
 *   k_cache, v_cache  in/out pools, layout above
 *   slot_mapping in   int32 [num_tokens]
 */
int pa_store_kv(const void* key, const void* value, int64_t key_token_stride,
                int64_t value_token_stride, void* k_cache, void* v_cache,
                const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                void* stream);

/*
 * pa_store_kv_paged -- pa_slot_mapping followed by pa_store_kv, in one launch.
 *
 * The same slots as pa_slot_mapping ([KVblog] 3.5: slot = block_table[p / B] *
 * B + p % B for the new token at position p = seq_lens_k[b] - Lq + i, -1 for
 * a token whose logical block is unmapped) and the same scatter as
 * pa_store_kv ([MinivLLM] store_kvcache_kernel), bit for bit; each token's
 * row loads are in flight while its table entry is read, so the step's store
 * costs one launch and one table round trip instead of two of each.
 *
 *   key, value, key_token_stride, value_token_stride   as for pa_store_kv
 *   block_table, max_blocks_per_seq, cu_seqlens_q, seq_lens_k, num_seqs,
 *   num_tokens, block_size, num_blocks                  as for pa_slot_mapping
 *   max_seqlen_q  largest Lq of the batch (1 for decode); it sizes the grid
 *                 only, a longer sequence is still stored whole
 *   slot_mapping  out  int32 [num_tokens], or NULL: the slots computed, as
 *                      pa_slot_mapping writes them
 *
 * Two tokens must not map to one slot.  Errors as for the two calls it
 * replaces; num_seqs = 0 or num_tokens = 0 is a no-op.
 */
int pa_store_kv_paged(const void* key, const void* value, int64_t key_token_stride,
                      int64_t value_token_stride, void* k_cache, void* v_cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* cu_seqlens_q, const int32_t* seq_lens_k, int32_t num_seqs,
                      int32_t num_tokens, int32_t max_seqlen_q, int32_t num_blocks,
                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                      int32_t* slot_mapping, void* stream);

/*
 * Split-K (flash-decoding) for decode.
 *
 * A long context is split into pieces; each piece produces the online-softmax
 * state of [mini] section 5 -- (m, l, acc): max score, exp-sum and weighted V
 * sum over its keys -- and a second kernel (pa_decode_merge) combines the
 * pieces of a sequence with the rescaling of [Lab] Fig. B-5:
 *   out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p,  M = max_p m_p.
 * partition_size selects how keys are split:
 *    0  balanced (default): every sequence's keys, in chunks of 8-32 tokens,
 *       are laid end to end and each KV head's keys are cut into equal slices,
 *       one per wave, whatever the sequence boundaries; a sequence inside one
 *       slice is finished in the first pass.  Balances mixed lengths.
 *       Needs num_seqs <= 8192; larger batches fall back to fixed partitions
 *       with an automatic size.  Without a workspace: single pass.
 *   -1  single pass: one piece per sequence, no workspace, no merge.
 *  P>0  fixed partitions: a power of two >= 16; partition p of sequence b
 *       covers keys [p*P, min((p+1)*P, L)).
 *
 * Workspace layouts (float32 unless noted, back to back):
 *  fixed, NP = ceil(max_context_len / P), written for partitions with p*P < L:
 *    acc [num_seqs][num_q_heads][NP][head_dim]   sum_j exp(s_j - m) v_j
 *    m   [num_seqs][num_q_heads][NP]             max_j s_j, s_j = scale q.k_j
 *    l   [num_seqs][num_q_heads][NP]             sum_j exp(s_j - m)
 *  balanced, W slices per KV-head wave (chosen by the library):
 *    acc [num_q_heads][W][2][head_dim], m [num_q_heads][W][2],
 *    l [num_q_heads][W][2], then int32 [num_seqs + 1] prefix sums of the
 *    per-sequence chunk counts; slot 0 of slice w holds the piece whose
 *    sequence began before the slice, slot 1 the piece that runs past it.
 */

/*
 * Bytes of workspace pa_decode needs for `partition_size` (0, -1 or P), for
 * either element type: 0 when the call runs a single pass.  Returns 0 for
 * invalid sizes.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len,
                                int32_t partition_size);

/*
 * pa_decode -- decode attention (one query token per sequence) over the pool.
 *
 * [mini] section 5 and [MinivLLM] paged_attention_decode_kernel: for sequence
 * b with L = context_lens[b] keys (L counts the token stored this step,
 * [KVblog] 4.4) and query head h served by KV head g = h / (num_q_heads /
 * num_kv_heads) (GQA, [mini] 5):
 *   out[b][h] = softmax_j(scale * q[b][h] . K_g[j]) . V_g[j],  j < L,
 * with K/V rows read through block_table and never copied to a contiguous
 * buffer.  `scale` is the final multiplier of q.k (no internal 1/sqrt(D)).
 * L = 0 gives an all-zero output row.
 *
 *   out          out  [num_seqs][num_q_heads][head_dim]
 *   q            in   [num_seqs][num_q_heads][head_dim]
 *   context_lens in   int32 [num_seqs]
 *   max_context_len   host upper bound of context_lens (sizes the split);
 *                     <= 0 means max_blocks_per_seq * block_size
 *   partition_size    0 / -1 / P, see "Split-K" above
 *   workspace         device scratch of workspace_bytes bytes (see
 *                     pa_decode_workspace_size); required by a split.
 * num_q_heads must be a multiple of num_kv_heads.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
              int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, float scale, pa_dtype dtype,
              int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_partitions -- the first pass of a split decode on its own.
 *
 * Same arguments and meaning as pa_decode; partition_size must be 0 or a P
 * that splits max_context_len, and a workspace is required.  It writes every
 * piece's online-softmax state ([mini] section 5) to the workspace in the
 * layout above; with the balanced split it also writes the final rows of the
 * sequences that no slice boundary cuts to `out` (fixed partitions do not
 * touch `out`, which may then be NULL).
 * pa_decode = pa_decode_partitions + pa_decode_merge.
 */
int pa_decode_partitions(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                         int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, float scale, pa_dtype dtype,
                         int32_t partition_size, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * pa_decode_merge -- the second pass of a split decode on its own.
 *
 * Reads piece states in the workspace layout of `partition_size` (0 or P)
 * and writes the rows the first pass left open ([Lab] Fig. B-5 rescaling;
 * a sequence without keys gives a zero row).  Exported so a merge can be
 * driven with states produced elsewhere, e.g. fixed partitions of one
 * sequence computed on several devices.
 */
int pa_decode_merge(void* out, const void* workspace, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                    pa_dtype dtype, void* stream);

/*
 * pa_decode_append -- a decode step's store and attention in one call:
 * pa_store_kv_paged of the step's new rows (one per sequence, row b at key
 * context_lens[b] - 1 of sequence b) followed by pa_decode, with the same
 * results ([MinivLLM] Attention.forward: the new K/V go to the cache, then the
 * query attends over every key including its own; [mini] section 5 for the
 * decode).  With the balanced split the store is part of the first pass: the
 * wave that finishes a sequence takes its last key from the new rows instead
 * of the cache and writes them to their slot, so the step needs no store
 * launch.  With another plan (single pass, fixed partitions) the rows are
 * stored by a launch of their own first.
 *
 *   key, value   in  [num_seqs][num_kv_heads][head_dim] rows of the step's new
 *                    token, token strides key_token_stride / value_token_stride
 *                    in elements (>= num_kv_heads * head_dim; 16-byte aligned
 *                    rows); dtype as the cache
 *   k_cache, v_cache  in/out: the pool; it holds the first context_lens[b] - 1
 *                    keys of sequence b before the call and all of them after
 *   everything else  as for pa_decode (context_lens counts the new key)
 *
 * A sequence with context_lens[b] = 0 has no new row (nothing is stored; zero
 * output row).  The new rows' slots must be distinct, and no other sequence
 * may read them.  Errors as for pa_decode and pa_store_kv_paged.
 */
int pa_decode_append(void* out, const void* q, const void* key, const void* value,
                     int64_t key_token_stride, int64_t value_token_stride, void* k_cache,
                     void* v_cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                     int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, float scale, pa_dtype dtype,
                     int32_t partition_size, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * pa_decode_append_partitions -- the first pass of pa_decode_append on its own
 * (with the store), as pa_decode_partitions is pa_decode's:
 * pa_decode_append = pa_decode_append_partitions + pa_decode_merge.
 */
int pa_decode_append_partitions(void* out, const void* q, const void* key, const void* value,
                                int64_t key_token_stride, int64_t value_token_stride,
                                void* k_cache, void* v_cache, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t max_context_len, int32_t num_blocks,
                                int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, float scale, pa_dtype dtype,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Bytes of the scratch array inside the library that pa_decode_noalloc uses (per device). */
#define PA_NOALLOC_SCRATCH_BYTES (16 << 20)

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.
 *
 * Same arguments, meaning and results as pa_decode without the workspace: the
 * split-K states go to a file-scope device array of PA_NOALLOC_SCRATCH_BYTES
 * bytes inside the library instead of a caller buffer.  Each device the library
 * runs on holds its own copy of the array until the process ends; its address is
 * looked up on the first call on that device (with that device current) and
 * kept.  Nothing is allocated and nothing needs clearing: every state a call
 * reads back was written earlier in the same call.
 *
 * Limit: a split whose workspace (pa_decode_workspace_size) exceeds
 * PA_NOALLOC_SCRATCH_BYTES is refused with PA_ERR_WORKSPACE before any work is
 * enqueued; a single-pass call (partition_size -1, or a context too short to
 * split) uses no scratch.  For the Qwen3-0.6B shape (16 Q / 8 KV heads, head_dim
 * 128) the balanced split needs about 4.3 MB at any batch up to 8192.
 *
 * Every call on one device shares that device's array: calls that overlap on a
 * device (two streams, or two host threads) race and must be ordered by the
 * caller.  Returns PA_ERR_HIP if the array's address cannot be looked up.
 */
int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                      int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, float scale, pa_dtype dtype,
                      int32_t partition_size, void* stream);

/*
 * pa_prefill_paged -- varlen (chunked) prefill attention over a cached prefix.
 *
 * [KVblog] 3.5: sequence b has Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] new
 * query tokens and Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys; the first
 * Lk - Lq keys are the cached prefix and every key is read from the pool
 * through block_table (the new chunk's rows must have been stored first,
 * [MinivLLM]: Attention.forward writes the cache, then attends).  Query i of
 * b sits at position Lk - Lq + i ([Lab] B.6) and, with causal != 0, sees keys
 * j <= Lk - Lq + i; with causal == 0 it sees all Lk keys.
 *
 *   out          out  [total_q][num_q_heads][head_dim]
 *   q            in   [total_q][num_q_heads][head_dim]
 *   cu_seqlens_q in   int32 [num_seqs + 1], cu[num_seqs] = total_q
 *   cu_seqlens_k in   int32 [num_seqs + 1], Lk >= Lq for every sequence
 *   max_seqlen_q / max_seqlen_k   host upper bounds of Lq / Lk
 *
 * dtype must be PA_BF16 or PA_F16 (the matrix-core path) and scale must be
 * > 0.
 */
int pa_prefill_paged(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                     int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                     int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal,
                     pa_dtype dtype, void* stream);

/*
 * pa_mixed_workspace_size -- bytes of workspace pa_attention_mixed needs.
 *
 * For num_seqs sequences whose key counts are at most max_seqlen_k; 0 for
 * invalid sizes, including head_dim other than 64 and 128 and more sequences
 * than pa_attention_mixed takes (2046 at head_dim 128, 7507 at head_dim 64).
 * The layout is the balanced split's of pa_decode (per query head and slice
 * two partial states, then the chunk prefix sums and the slice count the
 * launch used), covering the batch's decode rows.
 */
size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_seqlen_k);

/*
 * pa_attention_mixed -- one launch for a batch that mixes prompt chunks and
 * decode rows.
 *
 * Arguments and result are those of pa_prefill_paged with causal = 1: query
 * i of sequence b (Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b] queries,
 * Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys) sits at position Lk - Lq + i
 * and attends keys 0 .. Lk - Lq + i ([KVblog] 3.5; [Lab] B.6).  A sequence
 * with Lq = 1 is a decode row ([mini] section 5: its one query attends all Lk
 * keys); such rows take the split-K decode path and the others the matrix-core
 * prefill path, inside the same launch, followed by a small merge launch on
 * the same stream.  A decode row with Lk = 0 gives a zero row.  The launch
 * holds at most one workgroup per compute unit; each workgroup scans the
 * lengths and, with the same arithmetic in all of them, divides the
 * workgroups between the two sides so that the HBM-bound decode rows and the
 * matrix-bound prefill tiles run side by side.
 *
 *   workspace    scratch of pa_mixed_workspace_size(num_seqs, num_q_heads,
 *                num_kv_heads, head_dim, max_seqlen_k) bytes, 16-byte aligned,
 *                owned by the caller; no initialisation needed
 *
 * dtype must be PA_BF16 or PA_F16, scale > 0, num_q_heads/num_kv_heads in
 * 1..8 or 16.  num_seqs is bounded by the workgroup's LDS (160 KiB): the
 * prefill tiles hold 1024 * head_dim + 8196 bytes and the length scan
 * (3 * num_seqs + 5) * 4 bytes, so at most 2046 sequences at head_dim 128 and
 * 7507 at head_dim 64; a larger batch is refused with PA_ERR_UNSUPPORTED.
 * Errors as for pa_prefill_paged, plus PA_ERR_WORKSPACE for a missing or
 * short workspace.
 */
int pa_attention_mixed(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_table, int32_t max_blocks_per_seq,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                       pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_copy_blocks -- copy whole pool blocks (K and V), e.g. for copy-on-write.
 *
 * For each pair p: blocks block_pairs[2p] (source) -> block_pairs[2p+1]
 * (destination) of both pools, all block_size x num_kv_heads x head_dim
 * elements.  Block sharing and copy-on-write follow [KVblog] 2.2 (sequences
 * share a physical block through reference counts; a write into a shared block
 * first copies it).
 *
 *   block_pairs  in   DEVICE int32 [num_pairs][2]; a pair with an id outside
 *                     [0, num_blocks) or src == dst is skipped
 *
 * Destinations must be distinct and must not be sources of another pair.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                   int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, pa_dtype dtype, void* stream);

/*
 * pa_copy_many -- up to PA_COPY_MANY_MAX device copies and zero fills in one
 * launch.
 *
 * [Lab] B.4: a decode step replayed from a captured graph first copies its
 * inputs (q, new K/V rows, block table, lengths) into the fixed buffers the
 * graph was captured over, and marks the padding rows of its batch bucket.
 * This does all of those copies in one launch instead of one per tensor.
 *
 *   descs   HOST array of count descriptors {src, dst, bytes}: bytes >= 0 and a
 *           multiple of 4, src and dst DEVICE pointers, 4-byte aligned (16-byte
 *           aligned pointers and sizes take the 16-byte path); src NULL fills
 *           dst with zeros.  Destinations must not overlap each other or any
 *           source.
 *   count   0 .. PA_COPY_MANY_MAX
 *
 * The descriptors are passed by value to the kernel: the host array may be
 * reused as soon as the call returns.  Errors: PA_ERR_SHAPE, PA_ERR_NULL,
 * PA_ERR_ALIGN, PA_ERR_HIP.
 */
#define PA_COPY_MANY_MAX 8
typedef struct pa_copy_desc {
  const void* src;
  void* dst;
  int64_t bytes;
} pa_copy_desc;
int pa_copy_many(const pa_copy_desc* descs, int32_t count, void* stream);

/*
 * pa_read_ceiling -- measurement helper: the read bandwidth the decode pass
 * can reach.  Not part of the attention path.
 *
 * Reads every K and V byte of the pool blocks block_ids[0 .. num_ids) once
 * ([KVblog] 3.1: a block holds block_size rows of [num_kv_heads][head_dim])
 * with the decode's loads and wave-to-data mapping (one wave per KV head
 * reading that head's slice of each row, 16 bytes per lane, non-temporal) and
 * no arithmetic, and XORs what it read into sink so that no load is dropped.
 * Timing it over a pool larger than the last-level cache gives the ceiling the
 * decode pass is measured against.
 *
 *   block_ids      in   DEVICE int32 [num_ids]; ids outside [0, num_blocks)
 *                       are skipped
 *   num_workgroups      grid size (512 threads each), > 0
 *   sink           out  DEVICE uint32 [num_workgroups * 8], 4-byte aligned: the
 *                       XOR of the 32-bit words each wave read (the XOR of all
 *                       entries is the XOR of every word of the listed blocks,
 *                       a block listed twice cancelling)
 *
 * Errors: PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (head_dim, block_size, dtype as for
 * the caches), PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_HIP.
 */
int pa_read_ceiling(const void* k_cache, const void* v_cache, const int32_t* block_ids,
                    int32_t num_ids, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, pa_dtype dtype,
                    int32_t num_workgroups, uint32_t* sink, void* stream);

/*
 * Debug checks of the device-side contract stated at the top of this file.
 * Each drains `stream`, copies the metadata to the host and checks it there:
 * for debugging and tests, not for the hot path (it synchronises, so it
 * cannot be captured in a graph).  When the checks are switched on, the
 * matching check runs at the start of pa_store_kv, pa_store_kv_paged,
 * pa_decode, pa_decode_partitions, pa_decode_append(_partitions),
 * pa_prefill_paged and pa_attention_mixed, which then return its status
 * instead of launching (pa_decode_append: the decode check, then no two new
 * rows in one slot).  They start switched on
 * when the environment variable PA_DEBUG_CHECKS is set to anything but "0" at
 * the first call that looks; pa_set_debug_checks(on) switches them for the
 * whole process and returns the previous setting (0 / 1).
 *
 * pa_check_store_inputs: every slot_mapping entry is -1 or in
 *   [0, num_blocks*block_size), and no slot appears twice.
 * pa_check_store_paged_inputs: cu_seqlens_q never decreases and lies within
 *   [0, num_tokens], and no two new tokens map to one slot (the slots
 *   pa_store_kv_paged computes).
 * pa_check_decode_inputs: 0 <= context_lens[b] <= max_context_len (or
 *   max_blocks_per_seq*block_size when max_context_len <= 0, and never
 *   above it), and the first ceil(context_lens[b]/block_size) block ids of
 *   row b are in [0, num_blocks).
 * pa_check_prefill_inputs: cu_seqlens_q and cu_seqlens_k never decrease;
 *   cu_seqlens_q lies within [0, total_q]; each sequence has at most
 *   max_seqlen_q queries and max_seqlen_k keys, and at least as many keys as
 *   queries; its first ceil(keys/block_size) block ids are in
 *   [0, num_blocks).  Also covers pa_attention_mixed.
 *
 * Arguments mean what they mean for the matching call; pointers are DEVICE
 * pointers.  Returns PA_OK, PA_ERR_CONTRACT with pa_last_error() naming the
 * first violation, PA_ERR_SHAPE / PA_ERR_NULL for bad host arguments, or
 * PA_ERR_HIP if the copy fails.
 */
int pa_set_debug_checks(int on);
int pa_check_store_inputs(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                          int32_t block_size, void* stream);
int pa_check_store_paged_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                int32_t num_seqs, int32_t num_tokens, int32_t num_blocks,
                                int32_t block_size, void* stream);
int pa_check_decode_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                           int32_t num_blocks, int32_t block_size, void* stream);
int pa_check_prefill_inputs(const int32_t* block_table, int32_t max_blocks_per_seq,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                            int32_t max_seqlen_k, int32_t num_blocks, int32_t block_size,
                            void* stream);

/*
 * Host-side block manager with a chain-hash prefix cache ([KVblog] 3.3, 3.4;
 * [Lab] B.6).  Pure host code: it hands out block ids and block tables and
 * never touches device memory.  A handle is used from one thread at a time.
 *
 * pa_chain_hash: the fingerprint of one full block -- XXH64 (seed 0) over the
 *   previous block's fingerprint (8 bytes little-endian, only if has_prefix)
 *   followed by the block's token ids as 64-bit little-endian integers.
 * pa_bm_create / pa_bm_destroy: a manager of num_blocks >= 1 blocks of
 *   block_size >= 2 tokens (NULL on bad sizes).
 * pa_bm_allocate: admit a prompt (needs ceil(n / block_size) free blocks, else
 *   -PA_ERR_CAPACITY); its full blocks are looked up by fingerprint (the last
 *   block is always computed), a hit on a block in use adds a reference
 *   (REUSE), a hit on a freed block takes it back (REACTIVATE), the first miss
 *   ends the hits; returns a sequence handle >= 0 or -status.
 * pa_bm_append: one generated token; allocates a block when the token opens
 *   one, registers a block's fingerprint when the token fills it, and when the
 *   last block is shared with a fork, replaces it by a private copy and reports
 *   the pair (*cow_src, *cow_dst) for pa_copy_blocks (both -1 otherwise).
 * pa_bm_fork: a new sequence sharing all blocks of `seq` (one more reference
 *   each).
 * pa_bm_free: drop one reference per block, last block first; blocks at zero
 *   return to the back of the free list and keep their fingerprint until
 *   reallocated.  Unknown handles give -PA_ERR_SHAPE (PA_ERR_SHAPE from the
 *   int-returning calls).
 * Queries: block table (returns its length, copies up to capacity entries),
 *   sequence length, cached prompt tokens, a block's reference count, free
 *   blocks; negative status on a bad handle.
 */
typedef struct pa_block_manager pa_block_manager;
uint64_t pa_chain_hash(const int32_t* token_ids, int32_t num_tokens, int32_t has_prefix,
                       uint64_t prefix);
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);
int64_t pa_bm_allocate(pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens);
int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t token_id, int32_t* cow_src,
                 int32_t* cow_dst);
int64_t pa_bm_fork(pa_block_manager* bm, int64_t seq);
int pa_bm_free(pa_block_manager* bm, int64_t seq);
int32_t pa_bm_block_table(const pa_block_manager* bm, int64_t seq, int32_t* out,
                          int32_t capacity);
int32_t pa_bm_seq_len(const pa_block_manager* bm, int64_t seq);
int32_t pa_bm_num_cached_tokens(const pa_block_manager* bm, int64_t seq);
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id);
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
