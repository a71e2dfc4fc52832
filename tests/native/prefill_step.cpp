// A chunked-prefill step driven through the C ABI from C++, with no Python in its process:
// the chunk's new K/V rows are stored with pa_store_kv_paged, then pa_prefill_paged attends
// every new query over its sequence's cached prefix and the chunk.
//
// File layout (little-endian, written by tests/test_gpu_native.py):
//   int32 B, HQ, HKV, D, block_size, num_blocks, max_blocks_per_seq, total_q, max_seqlen_q,
//         max_seqlen_k, dtype (pa_dtype), causal;  float32 scale;
//   q [total_q][HQ][D], k_new and v_new [total_q][HKV][D], k_cache and v_cache
//   [num_blocks][block_size][HKV][D] (elements of dtype), then int32 block_table
//   [B][max_blocks_per_seq], cu_seqlens_q [B + 1], cu_seqlens_k [B + 1], seq_lens_k [B].
// Output file: out [total_q][HQ][D], then k_cache, then v_cache.
// Usage: prefill_step IN OUT.  Exit status 0 on success; a failing call prints its status and
// pa_last_error() and exits 1.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa.h"

namespace {

void* to_device(const std::vector<char>& h) {
  void* d = nullptr;
  if (hipMalloc(&d, h.size() ? h.size() : 16) != hipSuccess) return nullptr;
  if (!h.empty() && hipMemcpy(d, h.data(), h.size(), hipMemcpyHostToDevice) != hipSuccess)
    return nullptr;
  return d;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 2;
  int32_t h[12];
  float scale = 0.0f;
  if (fread(h, sizeof(h), 1, in) != 1 || fread(&scale, sizeof(scale), 1, in) != 1) return 2;
  const int32_t B = h[0], HQ = h[1], HKV = h[2], D = h[3], BS = h[4], NB = h[5], maxb = h[6];
  const int32_t T = h[7], max_q = h[8], max_k = h[9], causal = h[11];
  const pa_dtype dt = (pa_dtype)h[10];
  const size_t eb = dt == PA_F32 ? 4 : 2;
  auto take = [&](size_t n) {
    std::vector<char> v(n);
    if (n && fread(v.data(), n, 1, in) != 1) exit(2);
    return v;
  };
  const std::vector<char> q = take((size_t)T * HQ * D * eb);
  const std::vector<char> kn = take((size_t)T * HKV * D * eb), vn = take((size_t)T * HKV * D * eb);
  const size_t pool = (size_t)NB * BS * HKV * D * eb;
  const std::vector<char> kc = take(pool), vc = take(pool);
  const std::vector<char> bt = take((size_t)B * maxb * 4);
  const std::vector<char> cq = take((size_t)(B + 1) * 4), ck = take((size_t)(B + 1) * 4);
  const std::vector<char> lk = take((size_t)B * 4);
  fclose(in);

  void* dq = to_device(q);
  void* dkn = to_device(kn);
  void* dvn = to_device(vn);
  void* dkc = to_device(kc);
  void* dvc = to_device(vc);
  void* dbt = to_device(bt);
  void* dcq = to_device(cq);
  void* dck = to_device(ck);
  void* dlk = to_device(lk);
  void* dout = to_device(std::vector<char>(q.size(), (char)0xFF));  // NaN in every dtype
  if (!dq || !dkn || !dvn || !dkc || !dvc || !dbt || !dcq || !dck || !dlk || !dout) {
    fprintf(stderr, "device allocation failed\n");
    return 1;
  }
  hipStream_t s;
  if (hipStreamCreate(&s) != hipSuccess) return 1;
  const int64_t row = (int64_t)HKV * D;
  const int32_t* ibt = static_cast<const int32_t*>(dbt);
  const int32_t* icq = static_cast<const int32_t*>(dcq);
  int st = pa_store_kv_paged(dkn, dvn, row, row, dkc, dvc, ibt, maxb, icq,
                             static_cast<const int32_t*>(dlk), B, T, max_q, NB, BS, HKV, D, dt,
                             nullptr, s);
  if (st == PA_OK)
    st = pa_prefill_paged(dout, dq, dkc, dvc, ibt, maxb, icq, static_cast<const int32_t*>(dck), B,
                          T, max_q, max_k, NB, BS, HQ, HKV, D, scale, causal, dt, s);
  if (st != PA_OK) {
    fprintf(stderr, "%s (%s)\n", pa_status_string(st), pa_last_error());
    return 1;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return 1;

  std::vector<char> out(q.size()), kout(pool), vout(pool);
  if (hipMemcpy(out.data(), dout, out.size(), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(kout.data(), dkc, pool, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(vout.data(), dvc, pool, hipMemcpyDeviceToHost) != hipSuccess)
    return 1;
  FILE* o = fopen(argv[2], "wb");
  if (!o) return 1;
  fwrite(out.data(), 1, out.size(), o);
  fwrite(kout.data(), 1, kout.size(), o);
  fwrite(vout.data(), 1, vout.size(), o);
  fclose(o);
  for (void* p : {dq, dkn, dvn, dkc, dvc, dbt, dcq, dck, dlk, dout}) hipFree(p);
  hipStreamDestroy(s);
  return 0;
}
