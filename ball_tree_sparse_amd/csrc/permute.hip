// Row permutation between original order and tree order.  The ball tree keeps
// every ball contiguous (Erwin thread on Bluesky, post 9/N); moving features
// between the two trees of a rotated pair is one scatter back to original
// order and one gather into the other tree's order.
//   GATHER  dst[t]       = src[perm[t]]
//   SCATTER dst[perm[t]] = src[t]
// One thread moves one 16-byte (or 4-byte) piece; consecutive threads walk
// consecutive pieces of the same row, so every row is read and written as one
// contiguous run.
#include "common.h"

namespace bt {

template <typename V, bool SCATTER>
__global__ __launch_bounds__(256) void permute_rows(const V* __restrict__ src,
                                                    const int32_t* __restrict__ perm,
                                                    int64_t n, int64_t w, V* __restrict__ dst) {
  const int64_t total = n * w;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / w;
    const int64_t e = i - t * w;
    const int64_t p = perm_index(perm[t], n);
    if (SCATTER)
      dst[p * w + e] = src[t * w + e];
    else
      dst[t * w + e] = src[p * w + e];
  }
}

// Padded permutation (a padded tree of an uneven point count): nslots
// entries, negative for an unused slot, the others row indices below nrows.
//   GATHER  dst[t] = src[perm[t]], a zero row for an unused slot
//   SCATTER dst[perm[t]] = src[t] for the used slots only
template <typename V, bool SCATTER>
__global__ __launch_bounds__(256) void permute_rows_padded(const V* __restrict__ src,
                                                           const int32_t* __restrict__ perm,
                                                           int64_t nslots, int64_t nrows, int64_t w,
                                                           V* __restrict__ dst) {
  const int64_t total = nslots * w;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / w;
    const int64_t e = i - t * w;
    const int32_t raw = perm[t];
    if (SCATTER) {
      if (raw >= 0) dst[perm_index(raw, nrows) * w + e] = src[t * w + e];
    } else {
      dst[t * w + e] = raw >= 0 ? src[perm_index(raw, nrows) * w + e] : V{};
    }
  }
}

__global__ __launch_bounds__(256) void invert_perm_kernel(const int32_t* __restrict__ perm,
                                                          int64_t n, int32_t* __restrict__ inv) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x)
    inv[perm_index(perm[t], n)] = (int32_t)t;
}

static int grid_for(int64_t work) {
  int64_t g = (work + 255) / 256;
  const int64_t cap = 256 * 64;      // grid-stride beyond 16k workgroups
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

bt_status permute_launch(const void* src, const int32_t* perm, int64_t n, int64_t row_bytes,
                         bt_perm_mode mode, void* dst, hipStream_t st) {
  if (n == 0) return BT_OK;
  const bool v16 = (row_bytes % 16 == 0) && ((uintptr_t)src % 16 == 0) &&
                   ((uintptr_t)dst % 16 == 0);
  if (v16) {
    const int64_t w = row_bytes / 16;
    if (mode == BT_SCATTER)
      hipLaunchKernelGGL((permute_rows<u32x4, true>), dim3(grid_for(n * w)), dim3(256), 0, st,
                         (const u32x4*)src, perm, n, w, (u32x4*)dst);
    else
      hipLaunchKernelGGL((permute_rows<u32x4, false>), dim3(grid_for(n * w)), dim3(256), 0, st,
                         (const u32x4*)src, perm, n, w, (u32x4*)dst);
  } else {
    const int64_t w = row_bytes / 4;
    if (mode == BT_SCATTER)
      hipLaunchKernelGGL((permute_rows<uint32_t, true>), dim3(grid_for(n * w)), dim3(256), 0, st,
                         (const uint32_t*)src, perm, n, w, (uint32_t*)dst);
    else
      hipLaunchKernelGGL((permute_rows<uint32_t, false>), dim3(grid_for(n * w)), dim3(256), 0,
                         st, (const uint32_t*)src, perm, n, w, (uint32_t*)dst);
  }
  return launch_status("bt_permute");
}

bt_status permute_padded_launch(const void* src, const int32_t* perm, int64_t nrows,
                                int64_t nslots, int64_t row_bytes, bt_perm_mode mode, void* dst,
                                hipStream_t st) {
  if (nslots == 0) return BT_OK;
  const bool v16 = (row_bytes % 16 == 0) && ((uintptr_t)src % 16 == 0) &&
                   ((uintptr_t)dst % 16 == 0);
  const int64_t w = v16 ? row_bytes / 16 : row_bytes / 4;
  const dim3 grid(grid_for(nslots * w)), blk(256);
#define BT_PP(V, SC)                                                                           \
  hipLaunchKernelGGL((permute_rows_padded<V, SC>), grid, blk, 0, st, (const V*)src, perm,     \
                     nslots, nrows, w, (V*)dst)
  if (v16) {
    if (mode == BT_SCATTER) BT_PP(u32x4, true);
    else BT_PP(u32x4, false);
  } else {
    if (mode == BT_SCATTER) BT_PP(uint32_t, true);
    else BT_PP(uint32_t, false);
  }
#undef BT_PP
  return launch_status("bt_permute_padded");
}

bt_status invert_perm_launch(const int32_t* perm, int64_t n, int32_t* inv, hipStream_t st) {
  if (n == 0) return BT_OK;
  hipLaunchKernelGGL(invert_perm_kernel, dim3(grid_for(n)), dim3(256), 0, st, perm, n, inv);
  return launch_status("bt_invert_perm");
}

}  // namespace bt
