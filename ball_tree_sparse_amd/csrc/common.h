// Shared device/host helpers for libbtsparse (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bt.h"

#define BT_DEV __device__ __forceinline__

// Occupancy request (waves per SIMD) for a kernel.
#ifndef BT_WAVES_PER_EU
#define BT_WAVES_PER_EU(lo, hi) __attribute__((amdgpu_waves_per_eu(lo, hi)))
#endif

// LDS address space, for the builtins that take an LDS pointer.
#ifndef BT_LDS_AS
#define BT_LDS_AS __attribute__((address_space(3)))
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace bt {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 ----
BT_DEV float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round-to-nearest-even through the gfx950 packed converter (one
// v_cvt_pk_bf16_f32 for the pair).
typedef __bf16 bf16x2_pk __attribute__((ext_vector_type(2)));
BT_DEV uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_pk v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------ float sort keys ----
// Order-preserving map of a finite float to uint32 (-0.0 is canonicalised to
// +0.0 before this is called, so equal values give equal keys).
BT_DEV uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
BT_DEV float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
BT_DEV float canon_zero(float f) { return f == 0.0f ? 0.0f : f; }

// A permutation entry used as a gather/scatter index, forced into [0, n):
// a caller that passes something other than a permutation gets wrong rows,
// never an access outside the tensor.  (n < 2^31.)
BT_DEV int64_t perm_index(int32_t p, int64_t n) {
  return (int64_t)min((uint32_t)p, (uint32_t)(n - 1));
}

// ------------------------------------------------------ wave reductions ----
template <typename T>
BT_DEV T wave_shfl_xor(T v, int m) { return __shfl_xor(v, m, kWave); }

BT_DEV float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
BT_DEV uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, kWave));
  return v;
}
BT_DEV uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, kWave));
  return v;
}
BT_DEV float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
BT_DEV uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += (uint32_t)__shfl_xor((int)v, m, kWave);
  return v;
}
// Inclusive prefix sum across the 64 lanes of a wave.
BT_DEV uint32_t wave_incl_scan_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t t = (uint32_t)__shfl_up((int)v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// -------------------------------------------- softmax shift on the MFMA ----
// Scores can leave the MFMA in log2 units with the running maximum m already
// subtracted: the queries are multiplied by log2(e)/sqrt(d) before their
// rounding to bf16 (scale_query), and a 32x32x8 MFMA of a fragment of ones
// with shift_frag(m) puts -m in every row of a lane's column, for the score
// MFMAs to accumulate onto.  shift_frag splits -m into three bf16 pieces,
// which between them hold all 24 bits of its significand, in the k rows of
// the lanes of the lower half (the lanes of the upper half hold zeros), so
// the sum over k is -m exactly.
BT_DEV bf16x8 scale_query(bf16x8 x, float scale) {
  bf16x8 y;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = (__bf16)((float)x[e] * scale);
  return y;
}
BT_DEV float log2_score_scale(int d) { return 1.4426950408889634f / sqrtf((float)d); }

BT_DEV s16x4 ones_frag() { return s16x4{0x3f80, 0x3f80, 0x3f80, 0x3f80}; }
BT_DEV s16x4 shift_frag(float m) {
  const float x = -m;
  const float hi = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
  const float r = x - hi;                                      // exact
  const float mid = __uint_as_float(__float_as_uint(r) & 0xffff0000u);
  const float lo = r - mid;                                    // exact, at most 8 bits
  const bool lower = ((threadIdx.x >> 5) & 1) == 0;
  s16x4 f;
  f[0] = lower ? (short)(__float_as_uint(hi) >> 16) : (short)0;
  f[1] = lower ? (short)(__float_as_uint(mid) >> 16) : (short)0;
  f[2] = lower ? (short)(__float_as_uint(lo) >> 16) : (short)0;
  f[3] = 0;
  return f;
}

// The same for a 32x32x16 MFMA: the three pieces in k rows 0-2, the rest 0.
BT_DEV bf16x8 ones_frag8() {
  return __builtin_bit_cast(bf16x8, s16x8{0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80, 0x3f80,
                                          0x3f80, 0x3f80});
}
BT_DEV bf16x8 shift_frag8(float m) {
  const s16x4 f = shift_frag(m);
  return __builtin_bit_cast(bf16x8, s16x8{f[0], f[1], f[2], 0, 0, 0, 0, 0});
}

}  // namespace bt

// ------------------------------------------------------------ host side ----
namespace bt {
// Records a detail message for bt_last_error() on this thread.
void set_error(const char* fmt, ...);
bt_status launch_status(const char* what);
}  // namespace bt

#define BT_REQUIRE(cond, ...)                 \
  do {                                        \
    if (!(cond)) {                            \
      bt::set_error(__VA_ARGS__);             \
      return BT_EINVAL;                       \
    }                                         \
  } while (0)
