// Host SIMT emulation of the HIP constructs that libbtsparse's kernels use,
// so that the kernel sources compile as ordinary C++ and run on the CPU
// (with AddressSanitizer) for testing.  Each workgroup runs as blockDim host
// threads; __syncthreads is a barrier over them, wave intrinsics (shuffles,
// ballot, mbcnt) exchange through a per-wave buffer and barrier, LDS
// ("__shared__") is a static array, atomics are host atomics, and the
// 32x32x16 bf16 MFMA is computed wave-wide in its lane layout:
//   A[i][k] in lane i + 32*(k/8), element k%8; B[k][j] in lane j + 32*(k/8),
//   element k%8; D[i][j] in lane j + 32*((i/4)%2), element (i/8)*4 + i%4.
// Workgroups of a launch run one after another (in a seeded random order
// when EMU_SHUFFLE is set).
#pragma once
#include <atomic>
#include <barrier>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <memory>
#include <thread>
#include <vector>
#include <algorithm>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(x)
#define BT_WAVES_PER_EU(lo, hi)
#define BT_LDS_AS
#define __shared__ static
#define __restrict__

typedef int hipError_t;
#define hipSuccess 0
typedef void* hipStream_t;
inline hipError_t hipGetLastError() { return 0; }
// A small device: launch-size heuristics then give grids of few workgroups,
// so persistent kernels walk several items each.
#define hipDeviceAttributeMultiprocessorCount 0
inline hipError_t hipGetDevice(int* d) { *d = 0; return 0; }
inline hipError_t hipDeviceGetAttribute(int* v, int, int) { *v = 2; return 0; }
inline const char* hipGetErrorString(hipError_t) { return "ok"; }

struct dim3 { unsigned x, y, z; dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {} };
struct float4 { float x, y, z, w; };
struct uint2 { unsigned x, y; };
struct int2 { int x, y; };
struct int4 { int x, y, z, w; };
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }
inline uint2 make_uint2(unsigned a, unsigned b) { return {a, b}; }

struct Idx { unsigned x, y, z; };
extern thread_local Idx threadIdx, blockIdx;
extern Idx blockDim, gridDim;

inline float __int_as_float(int i) { float f; memcpy(&f, &i, 4); return f; }
inline int __float_as_int(float f) { int i; memcpy(&i, &f, 4); return i; }
inline float __uint_as_float(unsigned i) { float f; memcpy(&f, &i, 4); return f; }
inline unsigned __float_as_uint(float f) { unsigned i; memcpy(&i, &f, 4); return i; }
inline int __clz(int x) { return x == 0 ? 32 : __builtin_clz((unsigned)x); }
inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
using std::min; using std::max;

// ---- block / wave synchronisation -------------------------------------
struct EmuBlock {
  std::unique_ptr<std::barrier<>> block_bar;
  std::vector<std::unique_ptr<std::barrier<>>> wave_bar;
  std::vector<uint64_t> xch;     // one 64-bit slot per thread
  std::atomic<int> alive{0};
};
extern EmuBlock* g_blk;
inline int emu_tid() { return threadIdx.x; }
inline void __syncthreads() { g_blk->block_bar->arrive_and_wait(); }
inline void emu_wave_sync() { g_blk->wave_bar[emu_tid() / 64]->arrive_and_wait(); }
inline void __builtin_amdgcn_wave_barrier() { emu_wave_sync(); }
// a compiler scheduling fence: nothing to do on the host
inline void __builtin_amdgcn_sched_barrier(int) {}
inline void __threadfence() { std::atomic_thread_fence(std::memory_order_seq_cst); }

template <typename T>
inline T emu_shfl_from(T v, int src_lane) {
  const int t = emu_tid(), base = t & ~63;
  uint64_t u = 0; memcpy(&u, &v, sizeof(T));
  g_blk->xch[t] = u;
  emu_wave_sync();
  uint64_t r = g_blk->xch[base + (src_lane & 63)];
  emu_wave_sync();
  T out; memcpy(&out, &r, sizeof(T));
  return out;
}
template <typename T> inline T __shfl_xor(T v, int m, int w = 64) { return emu_shfl_from(v, (emu_tid() & 63) ^ m); }
template <typename T> inline T __shfl(T v, int src, int w = 64) { return emu_shfl_from(v, src); }
template <typename T> inline T __shfl_up(T v, unsigned d, int w = 64) {
  int l = emu_tid() & 63; int s = l >= (int)d ? l - (int)d : l; return emu_shfl_from(v, s); }
// DPP move with the old value kept where the source lane is invalid or the
// row is masked off (bound_ctrl off, all banks).  Controls: quad_perm,
// row_shr:1-15, row_bcast:15, row_bcast:31.
inline int __builtin_amdgcn_update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask,
                                       bool bound_ctrl) {
  const int t = emu_tid(), base = t & ~63, l = t & 63, row = l >> 4, x = l & 15;
  g_blk->xch[t] = (uint32_t)src;
  emu_wave_sync();
  int from = -1;
  if (ctrl >= 0 && ctrl <= 0xff) from = (l & ~3) | ((ctrl >> (2 * (l & 3))) & 3);  // quad_perm
  else if (ctrl >= 0x111 && ctrl <= 0x11f) { const int k = ctrl - 0x110; if (x >= k) from = l - k; }
  else if (ctrl == 0x142) { if (row >= 1) from = 16 * row - 1; }
  else if (ctrl == 0x143) { if (row >= 2) from = 31; }
  else { fprintf(stderr, "emulator: DPP control %#x not modelled\n", ctrl); abort(); }
  int r = old;
  if (from >= 0 && ((row_mask >> row) & 1) && ((bank_mask >> (x >> 2)) & 1))
    r = (int)(uint32_t)g_blk->xch[base + from];
  emu_wave_sync();
  (void)bound_ctrl;
  return r;
}
inline int __builtin_amdgcn_mov_dpp(int src, int ctrl, int row_mask, int bank_mask,
                                    bool bound_ctrl) {
  return __builtin_amdgcn_update_dpp(0, src, ctrl, row_mask, bank_mask, bound_ctrl);
}
// ds_swizzle_b32 in bit-mask mode (offset bit 15 clear): inside each group of
// 32 lanes, lane l reads lane ((l & and) | or) ^ xor.
inline int __builtin_amdgcn_ds_swizzle(int src, int pattern) {
  if (pattern & 0x8000) { fprintf(stderr, "emulator: ds_swizzle mode not modelled\n"); abort(); }
  const int l = emu_tid() & 63, a = pattern & 31, o = (pattern >> 5) & 31, x = (pattern >> 10) & 31;
  return emu_shfl_from(src, (l & 32) | (((l & a) | o) ^ x));
}
inline int __builtin_amdgcn_readlane(int v, int lane) { return emu_shfl_from(v, lane); }
inline unsigned long long __ballot(int p) {
  const int t = emu_tid(), base = t & ~63;
  g_blk->xch[t] = p ? 1 : 0;
  emu_wave_sync();
  unsigned long long m = 0;
  for (int i = 0; i < 64; ++i) if (g_blk->xch[base + i]) m |= 1ull << i;
  emu_wave_sync();
  return m;
}
inline unsigned __builtin_amdgcn_mbcnt_lo(unsigned m, unsigned acc) {
  int l = emu_tid() & 63; unsigned mask = l >= 32 ? 0xffffffffu : ((1u << l) - 1u);
  return acc + __builtin_popcount(m & mask); }
inline unsigned __builtin_amdgcn_mbcnt_hi(unsigned m, unsigned acc) {
  int l = emu_tid() & 63; unsigned mask = l < 32 ? 0u : (l == 63 ? 0x7fffffffu : ((1u << (l - 32)) - 1u));
  if (l < 32) mask = 0;
  return acc + __builtin_popcount(m & mask); }

// ---- atomics -----------------------------------------------------------
inline unsigned atomicAdd(unsigned* p, unsigned v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
inline unsigned atomicMin(unsigned* p, unsigned v) {
  unsigned o = __atomic_load_n(p, __ATOMIC_SEQ_CST);
  while (v < o && !__atomic_compare_exchange_n(p, &o, v, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)) {}
  return o; }
inline unsigned atomicMax(unsigned* p, unsigned v) {
  unsigned o = __atomic_load_n(p, __ATOMIC_SEQ_CST);
  while (v > o && !__atomic_compare_exchange_n(p, &o, v, false, __ATOMIC_SEQ_CST, __ATOMIC_SEQ_CST)) {}
  return o; }
#define __HIP_MEMORY_SCOPE_AGENT 0
#define __hip_atomic_fetch_add(p, v, o, s) __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST)
#define __hip_atomic_load(p, o, s) __atomic_load_n(p, __ATOMIC_SEQ_CST)

// ---- math --------------------------------------------------------------
inline float __builtin_amdgcn_exp2f(float x) { return exp2f(x); }
inline float __builtin_amdgcn_rcpf(float x) { return 1.0f / x; }
inline float __expf(float x) { return expf(x); }
// v_perm_b32 for selector bytes 0-7: byte i of the result is byte sel_i of
// the 8-byte value {b (bytes 0-3), a (bytes 4-7)}.
inline unsigned __builtin_amdgcn_perm(unsigned a, unsigned b, unsigned sel) {
  const unsigned long long ab = ((unsigned long long)a << 32) | b;
  unsigned r = 0;
  for (int i = 0; i < 4; ++i) r |= (unsigned)((ab >> (8 * ((sel >> (8 * i)) & 7))) & 0xff) << (8 * i);
  return r; }
// v_dot2_f32_bf16: c + a0*b0 + a1*b1 (bf16 products are exact in fp32)
template <class V>
inline float __builtin_amdgcn_fdot2_f32_bf16(V a, V b, float c, bool) {
  return (float)((double)c + (double)(float)a[0] * (double)(float)b[0] +
                 (double)(float)a[1] * (double)(float)b[1]); }

// ds_read_b64_tr_b16 (gfx950): in each 16-lane group, lane l receives
// element l%4 of the 8-byte runs addressed by lanes l/4, l/4+4, l/4+8, l/4+12
// (the layout measured on the device).
typedef short emu_s16x4 __attribute__((ext_vector_type(4)));
inline emu_s16x4 __builtin_amdgcn_ds_read_tr16_b64_v4i16(emu_s16x4* p) {
  const int t = emu_tid(), base = t & ~63, l = t & 63, grp = l & ~15, li = l & 15;
  uint64_t u;
  memcpy(&u, p, 8);
  g_blk->xch[t] = u;
  emu_wave_sync();
  emu_s16x4 r;
  for (int e = 0; e < 4; ++e) {
    const uint64_t w = g_blk->xch[base + grp + li / 4 + 4 * e];
    r[e] = (short)((w >> (16 * (li % 4))) & 0xffffu);
  }
  emu_wave_sync();
  return r;
}

// ---- dynamic LDS -----------------------------------------------------------
extern unsigned char* g_dyn_lds;
#define HIP_DYNAMIC_SHARED(type, var) type* var = (type*)g_dyn_lds;

// ---- MFMA 32x32x16 bf16 (wave-wide) --------------------------------------
typedef __bf16 emu_bf16x8 __attribute__((ext_vector_type(8)));
typedef float emu_f32x16 __attribute__((ext_vector_type(16)));
struct EmuMfmaSlot { float a[8], b[8]; };
extern std::vector<EmuMfmaSlot> g_mfma;
inline emu_f32x16 __builtin_amdgcn_mfma_f32_32x32x16_bf16(emu_bf16x8 a, emu_bf16x8 b, emu_f32x16 c,
                                                         int, int, int) {
  const int t = emu_tid(), base = t & ~63, l = t & 63;
  for (int e = 0; e < 8; ++e) { g_mfma[t].a[e] = (float)a[e]; g_mfma[t].b[e] = (float)b[e]; }
  emu_wave_sync();
  emu_f32x16 d = c;
  const int j = l & 31, hf = l >> 5;
  for (int e = 0; e < 16; ++e) {
    const int i = (e / 4) * 8 + hf * 4 + (e % 4);
    float acc = 0.f;
    for (int k = 0; k < 16; ++k) {
      const float av = g_mfma[base + i + 32 * (k / 8)].a[k % 8];
      const float bv = g_mfma[base + j + 32 * (k / 8)].b[k % 8];
      acc += av * bv;
    }
    d[e] = c[e] + acc;
  }
  emu_wave_sync();
  return d;
}

// ---- v_permlane32_swap: lanes 32-63 of the first operand trade places with
// lanes 0-31 of the second; returns the two operands after the swap ----------
typedef unsigned emu_u32x2 __attribute__((ext_vector_type(2)));
inline emu_u32x2 __builtin_amdgcn_permlane32_swap(unsigned a, unsigned b, bool, bool) {
  const int l = emu_tid() & 63;
  const unsigned a_x = emu_shfl_from(a, l ^ 32), b_x = emu_shfl_from(b, l ^ 32);
  emu_u32x2 r;
  r[0] = l < 32 ? a : b_x;      // upper half of a takes the lower half of b
  r[1] = l < 32 ? a_x : b;      // lower half of b takes the upper half of a
  return r;
}

// ---- MFMA 32x32x8 bf16 (bf16 operands as raw 16-bit patterns) ------------
typedef short emu_s16x4 __attribute__((ext_vector_type(4)));
inline float emu_bf16_bits(short h) {
  uint32_t u = (uint32_t)(uint16_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
inline emu_f32x16 __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(emu_s16x4 a, emu_s16x4 b, emu_f32x16 c,
                                                          int, int, int) {
  const int t = emu_tid(), base = t & ~63, l = t & 63;
  for (int e = 0; e < 4; ++e) { g_mfma[t].a[e] = emu_bf16_bits(a[e]); g_mfma[t].b[e] = emu_bf16_bits(b[e]); }
  emu_wave_sync();
  emu_f32x16 d = c;
  const int j = l & 31, hf = l >> 5;
  for (int e = 0; e < 16; ++e) {
    const int i = (e / 4) * 8 + hf * 4 + (e % 4);
    float acc = 0.f;
    for (int k = 0; k < 8; ++k) {
      const float av = g_mfma[base + i + 32 * (k / 4)].a[k % 4];
      const float bv = g_mfma[base + j + 32 * (k / 4)].b[k % 4];
      acc += av * bv;
    }
    d[e] = c[e] + acc;
  }
  emu_wave_sync();
  return d;
}

// ---- launches ------------------------------------------------------------
// Runs every workgroup of the grid one after another, each with blockDim
// host threads.
void emu_launch(dim3 grid, dim3 block, size_t shm, const std::function<void()>& body);
#define hipLaunchKernelGGL(K, G, B, SHM, ST, ...) \
  emu_launch(dim3(G), dim3(B), (size_t)(SHM), [&]() { K(__VA_ARGS__); })
