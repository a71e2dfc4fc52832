// A decode step driven through the C ABI from C++, with no Python in the process: the
// library's own test of include/pa.h as a native caller sees it.  It reads one decode
// batch from a file, runs the step on the GPU -- pa_store_kv_paged then pa_decode (mode 0)
// or pa_decode_append (mode 1) -- and writes the output rows and both pools back.
//
// File layout (little-endian, written by tests/test_gpu_native.py):
//   int32 B, HQ, HKV, D, block_size, num_blocks, max_blocks_per_seq, max_context_len,
//         dtype (pa_dtype), mode;  float32 scale;
//   q [B][HQ][D], k_new [B][HKV][D], v_new [B][HKV][D], k_cache and v_cache
//   [num_blocks][block_size][HKV][D] (elements of dtype), block_table int32
//   [B][max_blocks_per_seq], context_lens int32 [B].
// Output file: out [B][HQ][D], then k_cache, then v_cache.
// Usage: decode_step IN OUT.  Exit status 0 on success; a failing call prints its status
// and pa_last_error() and exits 1.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa.h"

namespace {

bool read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }

void* to_device(const std::vector<char>& h) {
  void* d = nullptr;
  if (hipMalloc(&d, h.size() ? h.size() : 16) != hipSuccess) return nullptr;
  if (!h.empty() && hipMemcpy(d, h.data(), h.size(), hipMemcpyHostToDevice) != hipSuccess)
    return nullptr;
  return d;
}

int check(int st, const char* what) {
  if (st != PA_OK) fprintf(stderr, "%s: %s (%s)\n", what, pa_status_string(st), pa_last_error());
  return st;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) return 2;
  int32_t hdr[10];
  float scale = 0.0f;
  if (!read_all(in, hdr, sizeof(hdr)) || !read_all(in, &scale, sizeof(scale))) return 2;
  const int32_t B = hdr[0], HQ = hdr[1], HKV = hdr[2], D = hdr[3], BS = hdr[4], NB = hdr[5];
  const int32_t maxb = hdr[6], max_ctx = hdr[7], mode = hdr[9];
  const pa_dtype dt = (pa_dtype)hdr[8];
  const size_t eb = dt == PA_F32 ? 4 : 2;
  auto take = [&](size_t n) {
    std::vector<char> v(n);
    if (!read_all(in, v.data(), n)) exit(2);
    return v;
  };
  const std::vector<char> q = take((size_t)B * HQ * D * eb);
  const std::vector<char> kn = take((size_t)B * HKV * D * eb), vn = take((size_t)B * HKV * D * eb);
  const size_t pool = (size_t)NB * BS * HKV * D * eb;
  const std::vector<char> kc = take(pool), vc = take(pool);
  const std::vector<char> bt = take((size_t)B * maxb * 4), ctx = take((size_t)B * 4);
  fclose(in);

  std::vector<char> cu((size_t)(B + 1) * 4);
  for (int32_t i = 0; i <= B; ++i) reinterpret_cast<int32_t*>(cu.data())[i] = i;
  void* dq = to_device(q);
  void* dkn = to_device(kn);
  void* dvn = to_device(vn);
  void* dkc = to_device(kc);
  void* dvc = to_device(vc);
  void* dbt = to_device(bt);
  void* dctx = to_device(ctx);
  void* dcu = to_device(cu);
  void* dout = to_device(std::vector<char>(q.size(), (char)0xFF));  // NaN in every dtype
  const size_t ws_bytes = pa_decode_workspace_size(B, HQ, HKV, D, max_ctx, 0);
  void* dws = to_device(std::vector<char>(ws_bytes));  // 16 bytes when no split needs one
  if (!dq || !dkn || !dvn || !dkc || !dvc || !dbt || !dctx || !dcu || !dout || !dws) {
    fprintf(stderr, "device allocation failed\n");
    return 1;
  }
  hipStream_t s;
  if (hipStreamCreate(&s) != hipSuccess) return 1;
  const int64_t row = (int64_t)HKV * D;
  const int32_t* ibt = static_cast<const int32_t*>(dbt);
  const int32_t* ictx = static_cast<const int32_t*>(dctx);
  if (mode == 0) {
    if (check(pa_store_kv_paged(dkn, dvn, row, row, dkc, dvc, ibt, maxb,
                                static_cast<const int32_t*>(dcu), ictx, B, B, 1, NB, BS, HKV, D,
                                dt, nullptr, s),
              "pa_store_kv_paged") ||
        check(pa_decode(dout, dq, dkc, dvc, ibt, maxb, ictx, B, max_ctx, NB, BS, HQ, HKV, D,
                        scale, dt, 0, ws_bytes ? dws : nullptr, ws_bytes, s),
              "pa_decode"))
      return 1;
  } else if (check(pa_decode_append(dout, dq, dkn, dvn, row, row, dkc, dvc, ibt, maxb, ictx, B,
                                    max_ctx, NB, BS, HQ, HKV, D, scale, dt, 0, ws_bytes ? dws : nullptr,
                                    ws_bytes, s),
                   "pa_decode_append")) {
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
  for (void* p : {dq, dkn, dvn, dkc, dvc, dbt, dctx, dcu, dout, dws}) hipFree(p);
  hipStreamDestroy(s);
  return 0;
}
