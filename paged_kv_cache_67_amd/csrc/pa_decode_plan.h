// Host side of the decode split: how a batch is divided (single pass, fixed
// partitions or the balanced split) and how the workspace is carved.  Shared by
// pa_decode and the mixed prefill + decode launch.
#pragma once

#include "pa_decode_dev.h"

namespace pa {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Fixed partitions used when the balanced split is unavailable (very large
// batches): at least 256 tokens, about 64 work items per compute unit.
inline int32_t auto_partition(int32_t B, int32_t HKV, int32_t max_ctx) {
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

inline DecodePlan plan_decode(int32_t B, int32_t HQ, int32_t HKV, int32_t D, pa_dtype dtype,
                              int32_t max_ctx, int32_t partition_size, bool have_workspace) {
  DecodePlan pl{};
  const int group = HQ / HKV;
  pl.G = head_tile(group);
  if (partition_size == -1 || (partition_size == 0 && !have_workspace)) {
    pl.mode = DecodePlan::kSingle;
  } else if (partition_size == 0 && B <= kMaxBalancedSeqs) {
    pl.mode = DecodePlan::kBalanced;
    const int head_waves = HKV * (group / pl.G);
    const int CH = chunk_tokens(D, elt_bytes(dtype), pl.G);
    // Upper bound of the K and V bytes the batch reads (every sequence at max_ctx keys).
    const double kv_bytes = (double)B * (max_ctx > 0 ? max_ctx : 1) * HKV * D * elt_bytes(dtype) * 2;
    const int slots =
        kv_bytes > (double)kInfinityCacheBytes ? PA_DECODE_WAVE_SLOTS_HBM : PA_DECODE_WAVE_SLOTS;
    const int64_t max_chunks = (int64_t)B * ceil_div(max_ctx > 0 ? max_ctx : 1, CH);
    auto slices = [&](int64_t waves) {
      const int64_t w = waves / head_waves;
      return w < 1 ? 1 : (w > max_chunks ? max_chunks : w);
    };
    pl.Wt = (int)slices(slots);
    // The workspace covers the larger wave count whichever is used, so that its size never
    // shrinks as the batch grows (a buffer sized for the largest batch serves every smaller
    // one): states, then the chunk scan s_cuc [B + 1] and the slice count of a mixed launch.
    const int64_t Wmax = slices(PA_DECODE_WAVE_SLOTS > PA_DECODE_WAVE_SLOTS_HBM
                                    ? PA_DECODE_WAVE_SLOTS : PA_DECODE_WAVE_SLOTS_HBM);
    const size_t states = (size_t)HQ * Wmax * 2;
    pl.ws_bytes = states * (D + 2) * sizeof(float) + (size_t)(B + 2) * sizeof(int32_t);
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

// Workspace carving: balanced = acc | m | l | cuc (B + 1 scan entries, then the slice
// count of a mixed launch); fixed = acc | m | l.
struct WsPtrs {
  float *acc, *m, *l;
  int32_t* cuc;
};
inline WsPtrs carve(void* ws, const DecodePlan& pl, int32_t B, int32_t HQ, int32_t D) {
  WsPtrs p{};
  p.acc = reinterpret_cast<float*>(ws);
  const size_t states =
      pl.mode == DecodePlan::kBalanced ? (size_t)HQ * pl.Wt * 2 : (size_t)B * HQ * pl.NP;
  p.m = p.acc + states * D;
  p.l = p.m + states;
  p.cuc = reinterpret_cast<int32_t*>(p.l + states);
  return p;
}

}  // namespace pa
