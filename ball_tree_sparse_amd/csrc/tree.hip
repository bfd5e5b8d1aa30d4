// Ball-tree partition on the GPU.
//
// A ball tree splits the points recursively into nested sets of similar size
// and stores each ball contiguously at every level (Erwin thread on Bluesky,
// posts 6/N and 9/N; post 15/N notes the original builder is native CPU code).
// Split rule implemented here: the axis of largest fp32 spread (lowest axis on
// ties) is cut into two equal halves; the left half holds the n/2 smallest
// points in (coordinate, original index) order with -0.0 == +0.0; each node
// keeps its points in ascending original index.  This makes the permutation
// unique, so it is reproduced bit for bit.
//
// Structure:
//   up to kLdsTree (8,192) points or slots: one 16-wave workgroup reads the
//               coordinates (rotated if asked, every product and sum rounded
//               to fp32) into 16-byte LDS records {x, y, z, idx} and splits
//               every level there: segments above 1,024 points with all
//               threads (up to eight points each), 1,024-point segments by the
//               whole workgroup or, four or more at a time, by single waves,
//               smaller ones by single waves (8-bit radix select of the
//               median key from the highest byte in which the segment's
//               extreme keys differ, ballot/mbcnt partition), then
//               perm[t] = idx.
//   above that  the records go to the workspace; each level whose nodes
//               hold more than 8,192 points is one launch with a workgroup
//               per node, which streams its node from one record array to
//               the other (radix select on the 8 bits below the highest bit
//               not yet fixed, stable partition chunk by chunk, the
//               children's extents gathered on the way), down to nodes of
//               2,048 slots; then one workgroup per node finishes its
//               subtree in LDS.  No
//               workgroup ever reads what another one of the same launch
//               writes.
//   padded      an uneven point count n: the tree has leaf * 2^L slots (the
//               smallest that holds n); a node of m points gives its left
//               child the ceil(m/2) smallest, and a leaf's unused slots hold
//               -1 (built as above: in LDS up to 8,192 slots, streamed
//               above that).
#include "common.h"

// Test hook: the CPU emulation of these kernels under MemorySanitizer marks
// a workgroup's LDS arrays uninitialised when the workgroup starts (so that a
// read before any write is reported); here it is nothing.
#ifndef BT_LDS_POISON
#define BT_LDS_POISON(x)
#endif

namespace bt {

constexpr int kThreads = 256;
constexpr int kFinish = 1024;   // largest segment split by one wave

BT_DEV int axis_of(const uint32_t* e) {
  // e = {min x, min y, min z, max x, max y, max z} as order-preserving keys
  float sp0 = key_float(e[3]) - key_float(e[0]);
  float sp1 = key_float(e[4]) - key_float(e[1]);
  float sp2 = key_float(e[5]) - key_float(e[2]);
  int a = 0;
  float best = sp0;
  if (sp1 > best) { best = sp1; a = 1; }
  if (sp2 > best) { a = 2; }
  return a;
}

BT_DEV float comp(const float4& r, int a) { return a == 0 ? r.x : (a == 1 ? r.y : r.z); }

// Number of set bits of m below this lane.
BT_DEV uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---------------------------------------------------------------- ingest ----
// ((r0*x + r1*y) + r2*z) with every product and sum rounded to fp32: the
// operations are written out here, inside a scope that forbids contraction
// into fused multiply-adds.
BT_DEV float rot_row(float r0, float r1, float r2, float x, float y, float z) {
#pragma clang fp contract(off)
  const float p0 = r0 * x;
  const float p1 = r1 * y;
  const float p2 = r2 * z;
  const float s01 = p0 + p1;
  return s01 + p2;
}

__global__ __launch_bounds__(kThreads) void tree_ingest(const float* __restrict__ coords,
                                                        int64_t n, int rotate, float r00,
                                                        float r01, float r02, float r10,
                                                        float r11, float r12, float r20,
                                                        float r21, float r22,
                                                        float4* __restrict__ rec) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float x = coords[3 * i], y = coords[3 * i + 1], z = coords[3 * i + 2];
    if (rotate) {
      const float a0 = rot_row(r00, r01, r02, x, y, z);
      const float a1 = rot_row(r10, r11, r12, x, y, z);
      const float a2 = rot_row(r20, r21, r22, x, y, z);
      x = a0; y = a1; z = a2;
    }
    rec[i] = make_float4(canon_zero(x), canon_zero(y), canon_zero(z), __int_as_float((int)i));
  }
}

// ------------------------------------------------------------ LDS splits ----

// Split the m-point segment R[0..m) of a wave's LDS node in place: the left
// part takes the ceil(m/2) smallest points (m/2 for the even m of a full tree).
BT_DEV void wave_split(float4* R, int m, uint32_t* hist, int lane) {
  // extents
  uint32_t mn[3] = {~0u, ~0u, ~0u}, mx[3] = {0u, 0u, 0u};
  for (int i = lane; i < m; i += 64) {
    const float4 x = R[i];
    const uint32_t k3[3] = {float_key(x.x), float_key(x.y), float_key(x.z)};
#pragma unroll
    for (int a = 0; a < 3; ++a) { mn[a] = min(mn[a], k3[a]); mx[a] = max(mx[a], k3[a]); }
  }
  uint32_t e[6];
#pragma unroll
  for (int a = 0; a < 3; ++a) { e[a] = wave_min_u32(mn[a]); e[3 + a] = wave_max_u32(mx[a]); }
  const int axis = axis_of(e);
  const uint32_t kmin = e[axis], kmax = e[3 + axis];

  // radix select of rank m/2-1 on 8-bit digits.  Keys of the segment lie in
  // [kmin, kmax], so they share every bit above the highest bit in which
  // kmin and kmax differ; the passes start at the byte holding that bit.
  uint32_t prefix = kmin;
  uint32_t rank = (uint32_t)((m + 1) / 2 - 1);
  const uint32_t diff = kmin ^ kmax;
  if (diff) {
    const int top = 31 - __clz((int)diff);
    prefix = kmin & ~((2u << top) - 1u);          // common high bits
    for (int shift = (top / 8) * 8; shift >= 0; shift -= 8) {
      const int hi = shift + 8;
      const uint32_t hmask = hi >= 32 ? 0u : (0xffffffffu << hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) hist[lane * 4 + j] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < m; i += 64) {
        const uint32_t key = float_key(comp(R[i], axis));
        if ((key & hmask) == (prefix & hmask)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      uint32_t h[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { h[j] = hist[lane * 4 + j]; tot += h[j]; }
      const uint32_t incl = wave_incl_scan_u32(tot);
      uint32_t cum = incl - tot;
      int found = -1;
      uint32_t newrank = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (h[j] && cum <= rank && rank < cum + h[j]) { found = lane * 4 + j; newrank = rank - cum; }
        cum += h[j];
      }
      const uint64_t bf = __ballot(found >= 0);
      const int src = bf ? __builtin_ctzll(bf) : 0;
      found = __shfl(found, src, 64);
      newrank = (uint32_t)__shfl((int)newrank, src, 64);
      prefix = (prefix & ~(255u << shift)) | ((uint32_t)found << shift);
      rank = newrank;
      __builtin_amdgcn_wave_barrier();
    }
  }
  const uint32_t pivot = prefix;
  const uint32_t need_eq = rank + 1u;

  // stable partition in place: read the whole segment, then write
  constexpr int MAXR = kFinish / 64;
  float4 x[MAXR];
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr)
    if (rr * 64 < m && rr * 64 + lane < m) x[rr] = R[rr * 64 + lane];
  __builtin_amdgcn_wave_barrier();
  uint32_t E = 0, Lrun = 0, Rrun = 0;
  const uint32_t half = (uint32_t)((m + 1) / 2);
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr) {
    if (rr * 64 >= m) break;
    const bool valid = rr * 64 + lane < m;
    const int nvalid = min(64, m - rr * 64);
    uint32_t key = valid ? float_key(comp(x[rr], axis)) : 0u;
    const bool is_lt = valid && key < pivot, is_eq = valid && key == pivot;
    const uint64_t beq = __ballot(is_eq);
    const uint32_t eq_p = mbcnt64(beq);
    const bool left = is_lt || (is_eq && (E + eq_p) < need_eq);
    const uint64_t bl = __ballot(valid && left);
    const uint32_t left_p = mbcnt64(bl);
    const uint32_t ltot = (uint32_t)__popcll(bl);
    if (valid) {
      const uint32_t dest = left ? Lrun + left_p : half + Rrun + ((uint32_t)lane - left_p);
      if (dest < (uint32_t)m) R[dest] = x[rr];
    }
    Lrun += ltot;
    Rrun += (uint32_t)nvalid - ltot;
    E += (uint32_t)__popcll(beq);
  }
  __builtin_amdgcn_wave_barrier();
}

// Waves of a tree workgroup.  The segments of a level are independent, so
// the waves take the small ones in turn (wave w splits segments w, w +
// waves, ...), with a workgroup barrier between levels.
constexpr int kFinishBlockWaves = 16;

// Scratch of a block-wide split (LDS).
struct BlockSplitLds {
  uint32_t hist[256];
  uint32_t ext[kFinishBlockWaves][6];
  uint32_t cnt[kFinishBlockWaves];
  uint32_t e6[6];
  uint32_t pick[2];
};

// Exclusive count of set flags at lower thread indices over the workgroup,
// and the total.  Every thread calls it (two workgroup barriers).
BT_DEV uint32_t block_excl_count(bool f, uint32_t* wcnt, uint32_t* total) {
  const int tid = threadIdx.x, w = tid >> 6;
  const uint64_t b = __ballot(f);
  const uint32_t in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
  if ((tid & 63) == 0) wcnt[w] = (uint32_t)__popcll(b);
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int i = 0; i < kFinishBlockWaves; ++i) {
    if (i < w) before += wcnt[i];
    all += wcnt[i];
  }
  __syncthreads();                           // wcnt may be reused next
  *total = all;
  return before + in_wave;
}

// The split of wave_split (same axis, pivot and stable order, so the same
// result bit for bit) done by all kFinishBlockWaves*64 threads of the
// workgroup on one segment R[0..m), m <= kFinish: one point per thread.
BT_DEV void block_split(float4* R, int m, BlockSplitLds& L,
                        uint32_t (*whist)[256]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool act = tid < m;
  const float4 x = act ? R[tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  // extents
  uint32_t e[6];
  {
    const uint32_t k3[3] = {float_key(x.x), float_key(x.y), float_key(x.z)};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      e[a] = wave_min_u32(act ? k3[a] : ~0u);
      e[3 + a] = wave_max_u32(act ? k3[a] : 0u);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < 6; ++a) L.ext[w][a] = e[a];
  }
  __syncthreads();
  if (tid < 6) {
    uint32_t v = L.ext[0][tid];
    for (int i = 1; i < kFinishBlockWaves; ++i)
      v = tid < 3 ? min(v, L.ext[i][tid]) : max(v, L.ext[i][tid]);
    L.e6[tid] = v;
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 6; ++a) e[a] = L.e6[a];
  const int axis = axis_of(e);
  const uint32_t key = float_key(comp(x, axis));
  const uint32_t kmin = e[axis], kmax = e[3 + axis];

  // radix select of rank ceil(m/2)-1 on 8-bit digits from the highest byte
  // in which kmin and kmax differ (as wave_split)
  uint32_t prefix = kmin;
  uint32_t rank = (uint32_t)((m + 1) / 2 - 1);
  const uint32_t diff = kmin ^ kmax;
  if (diff) {
    const int top = 31 - __clz((int)diff);
    prefix = kmin & ~((2u << top) - 1u);
    for (int shift = (top / 8) * 8; shift >= 0; shift -= 8) {
      const int hi = shift + 8;
      const uint32_t hmask = hi >= 32 ? 0u : (0xffffffffu << hi);
      // per-wave histograms (atomics contend only inside a wave), then summed
#pragma unroll
      for (int j = 0; j < 4; ++j) whist[w][lane * 4 + j] = 0u;
      __builtin_amdgcn_wave_barrier();
      if (act && (key & hmask) == (prefix & hmask)) atomicAdd(&whist[w][(key >> shift) & 255u], 1u);
      __syncthreads();
      if (tid < 256) {
        uint32_t t = 0;
        for (int i = 0; i < kFinishBlockWaves; ++i) t += whist[i][tid];
        L.hist[tid] = t;
      }
      __syncthreads();
      if (w == 0) {
        uint32_t h[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { h[j] = L.hist[lane * 4 + j]; tot += h[j]; }
        const uint32_t incl = wave_incl_scan_u32(tot);
        uint32_t cum = incl - tot;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (h[j] && cum <= rank && rank < cum + h[j]) {
            L.pick[0] = (uint32_t)(lane * 4 + j);
            L.pick[1] = rank - cum;
          }
          cum += h[j];
        }
      }
      __syncthreads();
      prefix = (prefix & ~(255u << shift)) | (L.pick[0] << shift);
      rank = L.pick[1];
      __syncthreads();                       // pick is rewritten next pass
    }
  }
  const uint32_t pivot = prefix;
  const uint32_t need_eq = rank + 1u;

  // stable partition: left = keys below the pivot and the first need_eq keys
  // equal to it, in index order; then the rest in index order
  const bool is_lt = act && key < pivot, is_eq = act && key == pivot;
  uint32_t tot = 0;
  const uint32_t eq_before = block_excl_count(is_eq, L.cnt, &tot);
  const bool left = is_lt || (is_eq && eq_before < need_eq);
  const uint32_t left_before = block_excl_count(act && left, L.cnt, &tot);
  const uint32_t half = (uint32_t)((m + 1) / 2);
  const uint32_t dest = left ? left_before : half + ((uint32_t)tid - left_before);
  // every thread read its point before the barriers above
  if (act && dest < (uint32_t)m) R[dest] = x;
  __syncthreads();
}

// Padded tree: start and point count of segment s at level lev, found by
// walking down from the root (n points), the left child taking ceil(cnt/2).
BT_DEV void padded_segment(int n, int lev, int s, int* start, int* cnt) {
  int st = 0, c = n;
  for (int i = lev - 1; i >= 0; --i) {
    const int nl = c - (c >> 1);   // ceil(c/2) without overflow
    if ((s >> i) & 1) {
      st += nl;
      c -= nl;
    } else {
      c = nl;
    }
  }
  *start = st;
  *cnt = c;
}

// ------------------------------------------------ one-workgroup tree -------
// Trees of up to kLdsTree slots are built by one workgroup with every point
// in LDS (128 KB of records on a CU's 160 KB): the coordinates are read (and
// rotated) straight into LDS, every level is split there, and the
// permutation is written out.  Segments above 1,024 points are split by all
// threads, each holding up to kLdsPer points; the lower levels reuse the
// block and wave splits of the finisher.  The points of a segment of m
// points sit at R[0..m) in ascending original index, and position p of the
// segment belongs to thread p % 1024 in round p / 1024.
constexpr int kLdsTree = 8192;
constexpr int kLdsThreads = kFinishBlockWaves * 64;
constexpr int kLdsPer = kLdsTree / kLdsThreads;   // 8 points per thread

// Counts of a big split, one per (round, wave) in position order, and the
// pivot decision of its radix passes.
struct BigSplitLds {
  uint32_t rc[kLdsPer * kFinishBlockWaves];
  uint32_t pick[3];
  uint32_t total;                  // sum of rc, written by round_wave_prefix
};

// Turns the counts rc[r * waves + w] (written, then a barrier) into their
// exclusive prefix sums in position order.  Wave 0 scans; every thread
// calls it (one workgroup barrier at the end).
BT_DEV void round_wave_prefix(uint32_t* rc, uint32_t* total) {
  constexpr int kE = kLdsPer * kFinishBlockWaves;   // 128 entries, two per lane
  static_assert(kE == 128, "two entries per lane of wave 0");
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const uint32_t a = rc[2 * lane], b = rc[2 * lane + 1];
    const uint32_t incl = wave_incl_scan_u32(a + b);
    const uint32_t ex = incl - (a + b);
    rc[2 * lane] = ex;
    rc[2 * lane + 1] = ex + a;
    if (lane == 63) *total = incl;
  }
  __syncthreads();
}

// The split of block_split (same axis, pivot and stable order) on a segment
// of kFinish < m <= kLdsTree points.
BT_DEV void big_split(float4* R, int m, BlockSplitLds& L, BigSplitLds& B,
                      uint32_t (*whist)[256]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float4 x[kLdsPer];
  uint32_t mn[3] = {~0u, ~0u, ~0u}, mx[3] = {0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < kLdsPer; ++r) {
    const int p = r * kLdsThreads + tid;
    x[r] = p < m ? R[p] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (p < m) {
      const uint32_t k3[3] = {float_key(x[r].x), float_key(x[r].y), float_key(x[r].z)};
#pragma unroll
      for (int a = 0; a < 3; ++a) { mn[a] = min(mn[a], k3[a]); mx[a] = max(mx[a], k3[a]); }
    }
  }
  // extents of the segment
  uint32_t e[6];
#pragma unroll
  for (int a = 0; a < 3; ++a) { e[a] = wave_min_u32(mn[a]); e[3 + a] = wave_max_u32(mx[a]); }
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < 6; ++a) L.ext[w][a] = e[a];
  }
  __syncthreads();
  if (tid < 6) {
    uint32_t v = L.ext[0][tid];
    for (int i = 1; i < kFinishBlockWaves; ++i)
      v = tid < 3 ? min(v, L.ext[i][tid]) : max(v, L.ext[i][tid]);
    L.e6[tid] = v;
  }
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 6; ++a) e[a] = L.e6[a];
  const int axis = axis_of(e);
  // the keys are taken again from the records where needed (fewer live
  // registers than keeping them)
  auto key = [&](int r) -> uint32_t { return float_key(comp(x[r], axis)); };
  const uint32_t kmin = e[axis], kmax = e[3 + axis];

  // radix select of rank ceil(m/2)-1 on 8-bit digits from the highest byte
  // in which kmin and kmax differ (as block_split).  When the bin holding
  // that rank has a single key, that key is the pivot (it is the only key
  // equal to itself, so rank 0 among equal keys) and the passes stop.
  uint32_t prefix = kmin;
  uint32_t rank = (uint32_t)((m + 1) / 2 - 1);
  const uint32_t diff = kmin ^ kmax;
  if (diff) {
    const int top = 31 - __clz((int)diff);
    prefix = kmin & ~((2u << top) - 1u);
    for (int shift = (top / 8) * 8; shift >= 0; shift -= 8) {
      const int hi = shift + 8;
      const uint32_t hmask = hi >= 32 ? 0u : (0xffffffffu << hi);
#pragma unroll
      for (int j = 0; j < 4; ++j) whist[w][lane * 4 + j] = 0u;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < kLdsPer; ++r) {
        const int p = r * kLdsThreads + tid;
        if (p < m && (key(r) & hmask) == (prefix & hmask))
          atomicAdd(&whist[w][(key(r) >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t t = 0;
        for (int i = 0; i < kFinishBlockWaves; ++i) t += whist[i][tid];
        L.hist[tid] = t;
      }
      __syncthreads();
      if (w == 0) {
        uint32_t h[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { h[j] = L.hist[lane * 4 + j]; tot += h[j]; }
        const uint32_t incl = wave_incl_scan_u32(tot);
        uint32_t cum = incl - tot;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (h[j] && cum <= rank && rank < cum + h[j]) {
            B.pick[0] = (uint32_t)(lane * 4 + j);
            B.pick[1] = rank - cum;
            B.pick[2] = h[j];
          }
          cum += h[j];
        }
      }
      __syncthreads();
      prefix = (prefix & ~(255u << shift)) | (B.pick[0] << shift);
      rank = B.pick[1];
      const bool single = B.pick[2] == 1u && shift > 0;
      __syncthreads();                       // pick is rewritten below or next pass
      if (single) {                          // uniform: one key matches prefix above shift
        const uint32_t pmask = 0xffffffffu << shift;
#pragma unroll
        for (int r = 0; r < kLdsPer; ++r) {
          const int p = r * kLdsThreads + tid;
          if (p < m && (key(r) & pmask) == prefix) B.pick[0] = key(r);
        }
        __syncthreads();
        prefix = B.pick[0];
        rank = 0u;
        __syncthreads();
        break;
      }
    }
  }
  const uint32_t pivot = prefix;
  const uint32_t need_eq = rank + 1u;

  // stable partition in position order: left = keys below the pivot and the
  // first need_eq keys equal to it; a right point's rank is its position
  // minus the left points before it.  The ranks come from one exclusive scan
  // of per-(round, wave) counts for the pivot-equal keys, then one for the
  // left points (rounds at or past m count zero).
  uint32_t in_w[kLdsPer];
#pragma unroll
  for (int r = 0; r < kLdsPer; ++r) {
    const int p = r * kLdsThreads + tid;
    const uint64_t b = __ballot(p < m && key(r) == pivot);
    in_w[r] = mbcnt64(b);
    if (lane == 0) B.rc[r * kFinishBlockWaves + w] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  round_wave_prefix(B.rc, &B.total);
  uint32_t left_bits = 0;
#pragma unroll
  for (int r = 0; r < kLdsPer; ++r) {
    const int p = r * kLdsThreads + tid;
    const uint32_t kr = key(r);
    const bool left = p < m && (kr < pivot ||
                                (kr == pivot && B.rc[r * kFinishBlockWaves + w] + in_w[r] < need_eq));
    left_bits |= (uint32_t)left << r;
  }
  __syncthreads();                           // every thread read the pivot-equal ranks
#pragma unroll
  for (int r = 0; r < kLdsPer; ++r) {
    const uint64_t b = __ballot((left_bits >> r) & 1u);
    in_w[r] = mbcnt64(b);
    if (lane == 0) B.rc[r * kFinishBlockWaves + w] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  round_wave_prefix(B.rc, &B.total);
  const uint32_t half = (uint32_t)((m + 1) / 2);
  uint32_t dest[kLdsPer];
#pragma unroll
  for (int r = 0; r < kLdsPer; ++r) {
    const int p = r * kLdsThreads + tid;
    const uint32_t left_before = B.rc[r * kFinishBlockWaves + w] + in_w[r];
    dest[r] = p >= m ? ~0u
                     : ((left_bits >> r) & 1u) ? left_before
                                               : half + ((uint32_t)p - left_before);
  }
  // every thread read its points before the barriers above
#pragma unroll
  for (int r = 0; r < kLdsPer; ++r)
    if (dest[r] < (uint32_t)m) R[dest[r]] = x[r];
  __syncthreads();
}

// One workgroup builds the tree of n points in ncap = leaf * 2^L slots
// (kFinish < ncap <= kLdsTree; ncap == n for a full tree): a segment of c
// points gives its left child the ceil(c/2) smallest (c/2 in a full tree,
// where c is always even), and the slots of a leaf past its points get -1.
// Splits every level of the n points at srec[0..n) (a tree of ncap slots,
// kFinish < ncap <= kLdsTree) in LDS and writes the ncap permutation entries
// to perm.  Every thread of the workgroup calls it.
BT_DEV void lds_levels(float4* srec, int n, int ncap, int leaf, BlockSplitLds& bsl,
                       BigSplitLds& bgl, uint32_t (*shist)[256], int32_t* __restrict__ perm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int lev = 0;
  for (int slots = ncap; slots > leaf; slots >>= 1, ++lev) {
    // segments above 1,024 points, and up to three of 1,024, are split by
    // the whole workgroup one after another; otherwise the waves take the
    // segments in turn (four or more 1,024-point segments finish sooner as
    // parallel wave splits than as block splits in sequence)
    if (slots > kFinish || (slots == kFinish && (1 << lev) < 4)) {   // uniform
      for (int sgi = 0; sgi < (1 << lev); ++sgi) {
        int st, cnt;
        padded_segment(n, lev, sgi, &st, &cnt);
        if (cnt > kFinish) big_split(srec + st, cnt, bsl, bgl, shist);
        else if (cnt >= 2) block_split(srec + st, cnt, bsl, shist);
      }
    } else {
      for (int sgi = w; sgi < (1 << lev); sgi += kFinishBlockWaves) {
        int st, cnt;
        padded_segment(n, lev, sgi, &st, &cnt);
        if (cnt >= 2) wave_split(srec + st, cnt, shist[w], lane);
      }
      __syncthreads();
    }
  }
  for (int t = tid; t < ncap; t += kLdsThreads) {
    const int j = t / leaf, i = t - j * leaf;
    int st, cnt;
    padded_segment(n, lev, j, &st, &cnt);
    perm[t] = i < cnt ? __float_as_int(srec[st + i].w) : -1;
  }
}

__global__ __launch_bounds__(kLdsThreads) void tree_lds_build(
    const float* __restrict__ coords, int n, int ncap, int leaf, int rotate, float r00, float r01,
    float r02, float r10, float r11, float r12, float r20, float r21, float r22,
    int32_t* __restrict__ perm) {
  __shared__ float4 srec[kLdsTree];
  BT_LDS_POISON(srec);
  __shared__ uint32_t shist[kFinishBlockWaves][256];
  BT_LDS_POISON(shist);
  __shared__ BlockSplitLds bsl;
  BT_LDS_POISON(bsl);
  __shared__ BigSplitLds bgl;
  BT_LDS_POISON(bgl);
  const int tid = threadIdx.x;
  for (int i = tid; i < n; i += kLdsThreads) {
    float x = coords[3 * (int64_t)i], y = coords[3 * (int64_t)i + 1], z = coords[3 * (int64_t)i + 2];
    if (rotate) {
      const float a0 = rot_row(r00, r01, r02, x, y, z);
      const float a1 = rot_row(r10, r11, r12, x, y, z);
      const float a2 = rot_row(r20, r21, r22, x, y, z);
      x = a0; y = a1; z = a2;
    }
    srec[i] = make_float4(canon_zero(x), canon_zero(y), canon_zero(z), __int_as_float(i));
  }
  __syncthreads();
  lds_levels(srec, n, ncap, leaf, bsl, bgl, shist, perm);
}

// One workgroup per node of level lev (nodes of `slots` slots, leaf < slots
// <= kLdsTree) of the tree of n points whose records rec are in node order
// (node k holds the points padded_segment(n, lev, k) gives): the node is
// loaded into LDS, split down to its leaves there, and the permutation
// entries of its slots written.
__global__ __launch_bounds__(kLdsThreads) void tree_lds_nodes(const float4* __restrict__ rec,
                                                              int n, int lev, int slots, int leaf,
                                                              int32_t* __restrict__ perm) {
  __shared__ float4 srec[kLdsTree];
  BT_LDS_POISON(srec);
  __shared__ uint32_t shist[kFinishBlockWaves][256];
  BT_LDS_POISON(shist);
  __shared__ BlockSplitLds bsl;
  BT_LDS_POISON(bsl);
  __shared__ BigSplitLds bgl;
  BT_LDS_POISON(bgl);
  int st, cnt;
  padded_segment(n, lev, (int)blockIdx.x, &st, &cnt);
  for (int i = threadIdx.x; i < cnt; i += kLdsThreads) srec[i] = rec[st + i];
  __syncthreads();
  lds_levels(srec, cnt, slots, leaf, bsl, bgl, shist, perm + (int64_t)blockIdx.x * slots);
}

// LDS of a streamed split beyond the histograms: the children's extents per
// wave.
struct StreamLds {
  uint32_t cext[kFinishBlockWaves][12];
};

// Histogram copies per wave of a streamed split: lane l counts into copy
// l % kSubHist, so that keys of one bin collide in at most 64 / kSubHist
// lanes of an atomic (the top levels' keys crowd into few bins).
constexpr int kSubHist = 4;

// One workgroup per node of level lev of the tree of n points (node k holds
// the m points padded_segment(n, lev, k) gives, more than half of its
// slots, which are above kLdsTree): the split of big_split (left child:
// the ceil(m/2) smallest) with the node streamed from global memory in chunks of
// kLdsThreads * kLdsPer positions (position p of a chunk belongs to thread
// p % kLdsThreads in round p / kLdsThreads), the children written to out at
// the node's place and their extents to ext_out[12 node ...] (left child,
// then right).  The node's own extents come from ext_in[6 node ...] (the
// previous level's ext_out) or, with ext_in null, from a pass over the node.
// The radix digits are the 8 bits below the highest bit not yet fixed (the
// last one shorter), so that every pass resolves 8 bits that vary.  No
// workgroup reads what another one of the same launch writes.
__global__ __launch_bounds__(kLdsThreads) void tree_stream_split(
    const float4* __restrict__ in, float4* __restrict__ out, int n, int lev,
    const uint32_t* __restrict__ ext_in, uint32_t* __restrict__ ext_out) {
  __shared__ uint32_t shist[kFinishBlockWaves][kSubHist][256];
  BT_LDS_POISON(shist);
  __shared__ BlockSplitLds L;
  BT_LDS_POISON(L);
  __shared__ BigSplitLds B;
  BT_LDS_POISON(B);
  __shared__ StreamLds S;
  BT_LDS_POISON(S);
  constexpr int64_t CH = (int64_t)kLdsThreads * kLdsPer;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = lane % kSubHist;
  const int64_t node = blockIdx.x;
  int st, cnt;
  padded_segment(n, lev, (int)node, &st, &cnt);
  const int64_t base = st, m = cnt;
  const float4* R = in + base;
  float4* O = out + base;
  const int64_t nch = (m + CH - 1) / CH;

  uint32_t e[6];
  if (ext_in) {
#pragma unroll
    for (int a = 0; a < 6; ++a) e[a] = ext_in[node * 6 + a];
  } else {                                   // extents of the node: a pass over it
    uint32_t mn[3] = {~0u, ~0u, ~0u}, mx[3] = {0u, 0u, 0u};
    for (int64_t c = 0; c < nch; ++c) {
#pragma unroll
      for (int r = 0; r < kLdsPer; ++r) {
        const int64_t p = c * CH + r * kLdsThreads + tid;
        if (p < m) {
          const float4 x = R[p];
          const uint32_t k3[3] = {float_key(x.x), float_key(x.y), float_key(x.z)};
#pragma unroll
          for (int a = 0; a < 3; ++a) { mn[a] = min(mn[a], k3[a]); mx[a] = max(mx[a], k3[a]); }
        }
      }
    }
#pragma unroll
    for (int a = 0; a < 3; ++a) { e[a] = wave_min_u32(mn[a]); e[3 + a] = wave_max_u32(mx[a]); }
    if (lane == 0) {
#pragma unroll
      for (int a = 0; a < 6; ++a) L.ext[w][a] = e[a];
    }
    __syncthreads();
    if (tid < 6) {
      uint32_t v = L.ext[0][tid];
      for (int i = 1; i < kFinishBlockWaves; ++i)
        v = tid < 3 ? min(v, L.ext[i][tid]) : max(v, L.ext[i][tid]);
      L.e6[tid] = v;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 6; ++a) e[a] = L.e6[a];
  }
  const int axis = axis_of(e);
  const uint32_t kmin = e[axis], kmax = e[3 + axis];
  // the split coordinate of position p, one 4-byte load
  const float* RC = (const float*)R + axis;
  auto key_at = [&](int64_t p) -> uint32_t { return float_key(RC[4 * p]); };

  // radix select of rank ceil(m/2)-1: bits at and above hi are fixed in
  // prefix; each pass takes the (up to) 8 bits below hi
  uint32_t prefix = kmin;
  uint32_t rank = (uint32_t)((m + 1) / 2 - 1);
  const uint32_t diff = kmin ^ kmax;
  if (diff) {
    int hi = 32 - __clz((int)diff);          // the keys agree above bit hi - 1
    prefix = hi >= 32 ? 0u : (kmin & (0xffffffffu << hi));
    while (hi > 0) {
      const int shift = hi > 8 ? hi - 8 : 0;
      const uint32_t dmask = (1u << (hi - shift)) - 1u;
      const uint32_t hmask = hi >= 32 ? 0u : (0xffffffffu << hi);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int u = 0; u < kSubHist; ++u) shist[w][u][lane * 4 + j] = 0u;
      __builtin_amdgcn_wave_barrier();
      for (int64_t c = 0; c < nch; ++c) {
        uint32_t kk[kLdsPer];
#pragma unroll
        for (int r = 0; r < kLdsPer; ++r) {
          const int64_t p = c * CH + r * kLdsThreads + tid;
          kk[r] = p < m ? key_at(p) : 0u;
        }
#pragma unroll
        for (int r = 0; r < kLdsPer; ++r) {
          const int64_t p = c * CH + r * kLdsThreads + tid;
          if (p < m && (kk[r] & hmask) == (prefix & hmask))
            atomicAdd(&shist[w][sub][(kk[r] >> shift) & dmask], 1u);
        }
      }
      __syncthreads();
      if (tid < 256) {
        uint32_t t = 0;
        for (int i = 0; i < kFinishBlockWaves; ++i)
#pragma unroll
          for (int u = 0; u < kSubHist; ++u) t += shist[i][u][tid];
        L.hist[tid] = t;
      }
      __syncthreads();
      if (w == 0) {
        uint32_t h[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { h[j] = L.hist[lane * 4 + j]; tot += h[j]; }
        const uint32_t incl = wave_incl_scan_u32(tot);
        uint32_t cum = incl - tot;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (h[j] && cum <= rank && rank < cum + h[j]) {
            B.pick[0] = (uint32_t)(lane * 4 + j);
            B.pick[1] = rank - cum;
            B.pick[2] = h[j];
          }
          cum += h[j];
        }
      }
      __syncthreads();
      prefix |= B.pick[0] << shift;
      rank = B.pick[1];
      const bool single = B.pick[2] == 1u && shift > 0;
      __syncthreads();                       // pick and hist are rewritten next pass
      hi = shift;
      if (single) {                          // uniform: one key matches prefix above shift
        const uint32_t pmask = 0xffffffffu << shift;
        for (int64_t c = 0; c < nch; ++c) {
#pragma unroll
          for (int r = 0; r < kLdsPer; ++r) {
            const int64_t p = c * CH + r * kLdsThreads + tid;
            if (p < m) {
              const uint32_t key = key_at(p);
              if ((key & pmask) == prefix) B.pick[0] = key;
            }
          }
        }
        __syncthreads();
        prefix = B.pick[0];
        rank = 0u;
        __syncthreads();
        break;
      }
    }
  }
  const uint32_t pivot = prefix;
  const uint32_t need_eq = rank + 1u;

  // stable partition, chunk by chunk in position order (as big_split, with
  // the pivot-equal and left counts of the earlier chunks carried along);
  // the children's extents are gathered on the way
  const uint64_t half = (uint64_t)((m + 1) / 2);
  uint32_t E = 0, Lrun = 0;
  uint32_t cmn[2][3] = {{~0u, ~0u, ~0u}, {~0u, ~0u, ~0u}}, cmx[2][3] = {{0u, 0u, 0u}, {0u, 0u, 0u}};
  for (int64_t c = 0; c < nch; ++c) {
    float4 x[kLdsPer];
    uint32_t in_w[kLdsPer];
#pragma unroll
    for (int r = 0; r < kLdsPer; ++r) {
      const int64_t p = c * CH + r * kLdsThreads + tid;
      x[r] = p < m ? R[p] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < kLdsPer; ++r) {
      const int64_t p = c * CH + r * kLdsThreads + tid;
      const uint64_t b = __ballot(p < m && float_key(comp(x[r], axis)) == pivot);
      in_w[r] = mbcnt64(b);
      if (lane == 0) B.rc[r * kFinishBlockWaves + w] = (uint32_t)__popcll(b);
    }
    __syncthreads();
    round_wave_prefix(B.rc, &B.total);
    uint32_t left_bits = 0;
#pragma unroll
    for (int r = 0; r < kLdsPer; ++r) {
      const int64_t p = c * CH + r * kLdsThreads + tid;
      const uint32_t kr = float_key(comp(x[r], axis));
      const bool left =
          p < m && (kr < pivot ||
                    (kr == pivot && E + B.rc[r * kFinishBlockWaves + w] + in_w[r] < need_eq));
      left_bits |= (uint32_t)left << r;
      if (p < m) {
        const int side = left ? 0 : 1;
        const uint32_t k3[3] = {float_key(x[r].x), float_key(x[r].y), float_key(x[r].z)};
#pragma unroll
        for (int a = 0; a < 3; ++a) {
          cmn[side][a] = min(cmn[side][a], k3[a]);
          cmx[side][a] = max(cmx[side][a], k3[a]);
        }
      }
    }
    E += B.total;
    __syncthreads();                         // every thread read the counts and the total
#pragma unroll
    for (int r = 0; r < kLdsPer; ++r) {
      const uint64_t b = __ballot((left_bits >> r) & 1u);
      in_w[r] = mbcnt64(b);
      if (lane == 0) B.rc[r * kFinishBlockWaves + w] = (uint32_t)__popcll(b);
    }
    __syncthreads();
    round_wave_prefix(B.rc, &B.total);
#pragma unroll
    for (int r = 0; r < kLdsPer; ++r) {
      const int64_t p = c * CH + r * kLdsThreads + tid;
      if (p < m) {
        const uint64_t left_before = (uint64_t)Lrun + B.rc[r * kFinishBlockWaves + w] + in_w[r];
        const uint64_t dest = ((left_bits >> r) & 1u) ? left_before
                                                      : half + ((uint64_t)p - left_before);
        if (dest < (uint64_t)m) O[dest] = x[r];
      }
    }
    Lrun += B.total;
    __syncthreads();                         // the counts are rewritten by the next chunk
  }
  // the children's extents: {min x, min y, min z, max x, max y, max z} each
  uint32_t v12[12];
#pragma unroll
  for (int sd = 0; sd < 2; ++sd)
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      v12[6 * sd + a] = wave_min_u32(cmn[sd][a]);
      v12[6 * sd + 3 + a] = wave_max_u32(cmx[sd][a]);
    }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 12; ++j) S.cext[w][j] = v12[j];
  }
  __syncthreads();
  if (tid < 12) {
    uint32_t v = S.cext[0][tid];
    for (int i = 1; i < kFinishBlockWaves; ++i)
      v = (tid % 6) < 3 ? min(v, S.cext[i][tid]) : max(v, S.cext[i][tid]);
    ext_out[node * 12 + tid] = v;
  }
}

static bt_status tree_lds_launch(const float* coords, int64_t n, int64_t ncap, int leaf,
                                 const float* R, int32_t* perm, hipStream_t st) {
  if (ncap < 2 || ncap > kLdsTree || n > ncap || n < 1 || leaf < 1 || ncap % leaf != 0) {
    set_error("tree: %lld points in %lld slots do not fit the one-workgroup builder",
              (long long)n, (long long)ncap);
    return BT_EINVAL;
  }
  float rr[9] = {1, 0, 0, 0, 1, 0, 0, 0, 1};
  if (R) for (int i = 0; i < 9; ++i) rr[i] = R[i];
  hipLaunchKernelGGL(tree_lds_build, dim3(1), dim3(kLdsThreads), 0, st, coords, (int)n,
                     (int)ncap, leaf, R ? 1 : 0, rr[0], rr[1], rr[2], rr[3], rr[4], rr[5], rr[6],
                     rr[7], rr[8], perm);
  return launch_status("tree_lds_build");
}

// A tree that is a single leaf of ncap >= n slots: the points in index
// order, then -1.
__global__ __launch_bounds__(kThreads) void tree_single_leaf(int64_t n, int64_t ncap,
                                                             int32_t* __restrict__ perm) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < ncap;
       t += (int64_t)gridDim.x * blockDim.x)
    perm[t] = t < n ? (int32_t)t : -1;
}

static bt_status single_leaf_launch(int64_t n, int64_t ncap, int32_t* perm, hipStream_t st) {
  int64_t g = (ncap + kThreads - 1) / kThreads;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(tree_single_leaf, dim3((int)g), dim3(kThreads), 0, st, n, ncap, perm);
  return launch_status("tree_single_leaf");
}

// The leaves of level lev (leaf slots each) of the tree of n points in
// ncap slots, records in node order: slot t of leaf j holds the index of
// its t-th point, -1 past them.
__global__ __launch_bounds__(kThreads) void tree_write_perm(const float4* __restrict__ rec,
                                                            int n, int lev, int64_t ncap,
                                                            int leaf, int32_t* __restrict__ perm) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < ncap;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(t / leaf), i = (int)(t - (int64_t)j * leaf);
    int st, cnt;
    padded_segment(n, lev, j, &st, &cnt);
    perm[t] = i < cnt ? __float_as_int(rec[st + i].w) : -1;
  }
}

// -------------------------------------------------------- coordinate check ----
// Finite coordinates are a precondition of the builders; this debug check
// counts the values of x[0..n) that are NaN or infinite into *count (which
// tree_zero_count clears first, on the same stream).
__global__ void tree_zero_count(uint32_t* __restrict__ count) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *count = 0u;
}

__global__ __launch_bounds__(kThreads) void tree_count_nonfinite(const float* __restrict__ x,
                                                                 int64_t n,
                                                                 uint32_t* __restrict__ count) {
  uint32_t c = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t u = __float_as_uint(x[i]);
    c += (u & 0x7f800000u) == 0x7f800000u;         // exponent all ones: NaN or infinity
  }
  c = wave_sum_u32(c);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(count, c);
}

bt_status count_nonfinite_launch(const float* x, int64_t n, uint32_t* count, hipStream_t st) {
  hipLaunchKernelGGL(tree_zero_count, dim3(1), dim3(64), 0, st, count);
  bt_status s = launch_status("tree_zero_count");
  if (s != BT_OK || n == 0) return s;
  int64_t g = (n + kThreads - 1) / kThreads;
  if (g > 1024) g = 1024;
  hipLaunchKernelGGL(tree_count_nonfinite, dim3((int)g), dim3(kThreads), 0, st, x, n, count);
  return launch_status("tree_count_nonfinite");
}

// ------------------------------------------------------------------ host ----
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Trees above kLdsTree slots (and above one leaf) are streamed through two
// record arrays in the workspace, with two arrays of node extents (six
// words per child of the last streamed level); smaller ones need none (the
// library still asks for its 256-byte minimum).
static bool stream_tree(int64_t ncap, int leaf) { return ncap > kLdsTree && ncap > leaf; }

// A streamed build splits nodes down to this many slots before one
// workgroup per node finishes them in LDS: more, smaller nodes keep more
// CUs busy in the LDS finish (65,536 points: 395 us stopping at 8,192 slots,
// 345 us at 2,048; 262,144 points: 1.25 / 1.20 ms; 1,048,576 points about
// 5.2 ms either way).
#ifndef BT_STREAM_STOP
#define BT_STREAM_STOP 2048
#endif
constexpr int64_t kStreamStop = BT_STREAM_STOP;
static_assert(kStreamStop <= kLdsTree, "nodes finished in LDS fit it");

// Children of the last streamed level: twice its nodes.
static int64_t stream_children(int64_t ncap, int leaf) {
  int64_t slots = ncap, kids = 0;
  while (slots > leaf && slots > kStreamStop) {
    kids = 2 * (ncap / slots);
    slots >>= 1;
  }
  return kids;
}

static size_t stream_ext_bytes(int64_t ncap, int leaf) {
  return align256((size_t)stream_children(ncap, leaf) * 6 * 4);
}

static size_t stream_ws_bytes(int64_t n, int64_t ncap, int leaf) {
  return stream_tree(ncap, leaf) ? 2 * align256((size_t)n * 16) + 2 * stream_ext_bytes(ncap, leaf)
                                 : 256;
}

size_t tree_workspace_size(int64_t n, int leaf) { return stream_ws_bytes(n, n, leaf); }

// The streamed build of n points in ncap = leaf * 2^L > kLdsTree slots (ncap
// > leaf) with the records in ws (two arrays of n records, then two extent
// arrays).  Every launch is checked on the host against the arrays it
// indexes: the nodes of a level tile the slots, and the 12 extent words per
// node fit the extent array.
static bt_status tree_stream_launch(const float* coords, int64_t n, int64_t ncap, int leaf,
                                    const float* R, int32_t* perm, void* ws, hipStream_t st) {
  const size_t rb = align256((size_t)n * 16), eb = stream_ext_bytes(ncap, leaf);
  float4* rec[2] = {(float4*)ws, (float4*)((char*)ws + rb)};
  uint32_t* ext[2] = {(uint32_t*)((char*)ws + 2 * rb), (uint32_t*)((char*)ws + 2 * rb + eb)};
  float rr[9] = {1, 0, 0, 0, 1, 0, 0, 0, 1};
  if (R) for (int i = 0; i < 9; ++i) rr[i] = R[i];
  {
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(tree_ingest, dim3((int)g), dim3(kThreads), 0, st, coords, n, R ? 1 : 0,
                       rr[0], rr[1], rr[2], rr[3], rr[4], rr[5], rr[6], rr[7], rr[8], rec[0]);
    bt_status s = launch_status("tree_ingest");
    if (s != BT_OK) return s;
  }
  int64_t slots = ncap;
  int lev = 0, cur = 0;
  while (slots > leaf && slots > kStreamStop) {
    const int64_t nodes = ncap / slots;
    if (nodes * slots != ncap || nodes > INT32_MAX || (size_t)nodes * 12 * 4 > eb) {
      set_error("tree: level %d geometry does not fit the workspace", lev);
      return BT_EINVAL;
    }
    // level 0 takes its extents from a pass over the records; later levels
    // from the children's extents the level above wrote
    hipLaunchKernelGGL(tree_stream_split, dim3((unsigned)nodes), dim3(kLdsThreads), 0, st,
                       rec[cur], rec[cur ^ 1], (int)n, lev,
                       lev == 0 ? (const uint32_t*)nullptr : (const uint32_t*)ext[cur],
                       ext[cur ^ 1]);
    bt_status s = launch_status("tree_stream_split");
    if (s != BT_OK) return s;
    cur ^= 1;
    slots >>= 1;
    ++lev;
  }
  const int64_t nodes = ncap / slots;
  if (nodes * slots != ncap || nodes > INT32_MAX) {
    set_error("tree: level %d geometry does not fit the workspace", lev);
    return BT_EINVAL;
  }
  if (slots == leaf) {
    int64_t g = (ncap + kThreads - 1) / kThreads;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(tree_write_perm, dim3((int)g), dim3(kThreads), 0, st, rec[cur], (int)n,
                       lev, ncap, leaf, perm);
    return launch_status("tree_write_perm");
  }
  hipLaunchKernelGGL(tree_lds_nodes, dim3((unsigned)nodes), dim3(kLdsThreads), 0, st, rec[cur],
                     (int)n, lev, (int)slots, leaf, perm);
  return launch_status("tree_lds_nodes");
}

bt_status tree_build_launch(const float* coords, int64_t n, int leaf, const float* R,
                            int32_t* perm, void* ws, hipStream_t st) {
  if (n == leaf) return single_leaf_launch(n, n, perm, st);
  if (stream_tree(n, leaf)) return tree_stream_launch(coords, n, n, leaf, R, perm, ws, st);
  return tree_lds_launch(coords, n, n, leaf, R, perm, st);
}

int64_t tree_padded_slots(int64_t n, int leaf) {
  int64_t cap = leaf;
  while (cap < n) cap *= 2;
  return cap;
}

size_t tree_padded_workspace_size(int64_t n, int leaf) {
  return stream_ws_bytes(n, tree_padded_slots(n, leaf), leaf);
}

// Padded tree of n points: one leaf of any size, up to kLdsTree slots in
// LDS, or streamed above that.
bt_status tree_build_padded_launch(const float* coords, int64_t n, int leaf, const float* R,
                                   int32_t* perm, void* ws, hipStream_t st) {
  const int64_t ncap = tree_padded_slots(n, leaf);
  if (ncap == leaf) return single_leaf_launch(n, ncap, perm, st);
  if (stream_tree(ncap, leaf)) return tree_stream_launch(coords, n, ncap, leaf, R, perm, ws, st);
  return tree_lds_launch(coords, n, ncap, leaf, R, perm, st);
}

}  // namespace bt
