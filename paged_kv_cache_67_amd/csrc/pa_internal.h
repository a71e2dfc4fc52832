// Internal helpers shared by the libpa kernels and entry points (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// ---------------------------------------------------------------------------
// Host side: error reporting.  Each entry point returns a pa_status and leaves
// a human-readable detail in a thread-local buffer.

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Check the launch that was just enqueued; returns PA_OK or PA_ERR_HIP.
int check_launch(const char* what);
// The debug checks of the device-side metadata are on (PA_DEBUG_CHECKS in the environment,
// or pa_set_debug_checks).
bool debug_checks();

// The new rows of a decode batch (row b is key context_lens[b] - 1 of sequence b) stored to
// their slots by one launch (pa_store.hip); inputs already checked.
int launch_store_decode_rows(const void* key, const void* value, int64_t key_stride_bytes,
                             int64_t value_stride_bytes, void* k_cache, void* v_cache,
                             const int32_t* block_table, int32_t maxb,
                             const int32_t* context_lens, int32_t B, int32_t num_blocks,
                             int32_t block_size, int64_t row_bytes, hipStream_t s);
// Debug check of those rows' slots (pa_check.cpp): no two sequences' new rows share one.
int check_append_slots(const int32_t* block_table, int32_t maxb, const int32_t* context_lens,
                       int32_t B, int32_t num_blocks, int32_t block_size, hipStream_t s);

inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
__host__ __device__ constexpr inline int elt_bytes(pa_dtype t) { return t == PA_F32 ? 4 : 2; }

constexpr int kNumCUs = 256;  // MI355X: 8 XCDs x 32 CUs

constexpr int kNumXCDs = 8;

constexpr int kMaxDevices = 64;  // devices one process can drive (per-device state tables)

// ---------------------------------------------------------------------------
// Device side.

// Workgroups are handed to the XCDs round-robin in launch order (id % 8).  This maps launch
// id L of N to a logical id so that each XCD receives one contiguous range of logical ids:
// XCD x gets ids [x*q + min(x, r), ...) with q = N / 8, r = N % 8 (a bijection on [0, N)).
__device__ __forceinline__ int xcd_local_id(int L, int N) {
  const int x = L % kNumXCDs, q = N / kNumXCDs, r = N % kNumXCDs;
  return x * q + min(x, r) + L / kNumXCDs;
}

// bf16 <-> fp32.  A bf16 value is the top half of an fp32, so widening is a
// shift; narrowing rounds to nearest-even (NaN stays NaN).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// DPP lane moves within a 16-lane row (all source lanes valid for these
// patterns, so bound_ctrl does not matter).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of the
// group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppRowMirror>(v);
  if constexpr (N == 32) v += __shfl_xor(v, 16);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A 16-byte load marked non-temporal (global_load_dwordx4 ... nt): for data read once,
// such as the K/V rows of a decode pass, it streams past the caches instead of
// displacing what they hold.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace pa
