// Coarsening and refinement of tree-ordered features.
//
// Erwin coarsens and then refines the ball tree while the attention ball
// size stays fixed, U-Net fashion (Erwin thread on Bluesky, post 8/N);
// because every level of the tree is stored contiguously, these operations
// reduce to views and means over consecutive tree positions (post 9/N).
// Implemented here, the non-learned half of that U-Net:
//   coarsen by s: out[j] = mean_{r < s} x[row(j*s + r)]   (tree order out)
//   refine by s:  out[row(t)] = xc[t / s]
// with row(t) = perm[t] when a permutation is given (original-order features)
// and row(t) = t otherwise.  Each thread moves one 16-byte piece of a row;
// consecutive threads walk a row, so every row is read or written whole.
// Means are summed in fp32 in a fixed order and rounded once to the output
// type (round-to-nearest-even for bf16).
#include "common.h"

namespace bt {

template <typename T> struct Piece;
template <> struct Piece<float> { static constexpr int E = 4; };
template <> struct Piece<uint16_t> { static constexpr int E = 8; };

BT_DEV void piece_add(const u32x4& x, float* acc, float) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(x[e]);
}
BT_DEV void piece_add(const u32x4& x, float* acc, uint16_t) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += bf16_to_f32((uint16_t)(x[e] & 0xffffu));
    acc[2 * e + 1] += bf16_to_f32((uint16_t)(x[e] >> 16));
  }
}
BT_DEV u32x4 piece_out(const float* acc, float f, float) {
  return u32x4{__float_as_uint(acc[0] * f), __float_as_uint(acc[1] * f),
               __float_as_uint(acc[2] * f), __float_as_uint(acc[3] * f)};
}
BT_DEV u32x4 piece_out(const float* acc, float f, uint16_t) {
  return u32x4{pack_bf16x2(acc[0] * f, acc[1] * f), pack_bf16x2(acc[2] * f, acc[3] * f),
               pack_bf16x2(acc[4] * f, acc[5] * f), pack_bf16x2(acc[6] * f, acc[7] * f)};
}

template <typename T, bool PERM>
__global__ __launch_bounds__(256) void coarsen_rows(const u32x4* __restrict__ x,
                                                    const int32_t* __restrict__ perm,
                                                    int64_t N, int32_t s, int32_t ppr,
                                                    u32x4* __restrict__ out) {
  constexpr int E = Piece<T>::E;
  const int64_t nc = N / s, total = nc * ppr;
  const float f = 1.0f / (float)s;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = i / ppr, pc = i - j * ppr;
    float acc[E] = {};
    for (int r = 0; r < s; ++r) {
      const int64_t t = j * s + r;
      const int64_t row = PERM ? perm_index(perm[t], N) : t;
      piece_add(x[row * ppr + pc], acc, T{});
    }
    out[i] = piece_out(acc, f, T{});
  }
}

template <bool PERM>
__global__ __launch_bounds__(256) void refine_rows(const u32x4* __restrict__ xc,
                                                   const int32_t* __restrict__ perm, int64_t N,
                                                   int32_t s, int32_t ppr,
                                                   u32x4* __restrict__ out) {
  const int64_t total = N * ppr;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / ppr, pc = i - t * ppr;
    const int64_t row = PERM ? perm_index(perm[t], N) : t;
    out[row * ppr + pc] = xc[(t / s) * ppr + pc];
  }
}

static dim3 pool_grid(int64_t total) {
  int64_t g = (total + 255) / 256;
  if (g > 8192) g = 8192;
  if (g < 1) g = 1;
  return dim3((unsigned)g);
}

bt_status coarsen_launch(const void* x, const int32_t* perm, int64_t N, int32_t ppr, int32_t s,
                         bt_dtype dt, void* out, hipStream_t st) {
  const dim3 grid = pool_grid(N / s * ppr), blk(256);
  const u32x4* xi = (const u32x4*)x;
  u32x4* o = (u32x4*)out;
  if (dt == BT_F32) {
    if (perm) hipLaunchKernelGGL((coarsen_rows<float, true>), grid, blk, 0, st, xi, perm, N, s, ppr, o);
    else hipLaunchKernelGGL((coarsen_rows<float, false>), grid, blk, 0, st, xi, perm, N, s, ppr, o);
  } else {
    if (perm) hipLaunchKernelGGL((coarsen_rows<uint16_t, true>), grid, blk, 0, st, xi, perm, N, s, ppr, o);
    else hipLaunchKernelGGL((coarsen_rows<uint16_t, false>), grid, blk, 0, st, xi, perm, N, s, ppr, o);
  }
  return launch_status("coarsen_rows");
}

bt_status refine_launch(const void* xc, const int32_t* perm, int64_t N, int32_t ppr, int32_t s,
                        void* out, hipStream_t st) {
  const dim3 grid = pool_grid(N * ppr), blk(256);
  if (perm)
    hipLaunchKernelGGL((refine_rows<true>), grid, blk, 0, st, (const u32x4*)xc, perm, N, s, ppr,
                       (u32x4*)out);
  else
    hipLaunchKernelGGL((refine_rows<false>), grid, blk, 0, st, (const u32x4*)xc, perm, N, s, ppr,
                       (u32x4*)out);
  return launch_status("refine_rows");
}

}  // namespace bt
