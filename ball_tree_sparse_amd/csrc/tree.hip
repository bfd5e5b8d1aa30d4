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
// Structure (all nodes of a level are handled by the same launches):
//   ingest      coords (optionally rotated, every product and sum rounded to
//               fp32) -> 16-byte records {x, y, z, idx}; root extents.
//   per level while the node size n is above kFinish (= 1024 points):
//     hist<p>     radix-select of the median key on the split axis, 11/11/10
//                 bit digits of the order-preserving uint32 key (p = 0,1,2).
//                 Workgroups own equal chunks of one node (the node halved
//                 down to at most 1-4K points while its size is even), build
//                 an LDS histogram and add it to the node's global histogram.
//     select<p>   one workgroup per node scans that histogram, fixes the next
//                 digit of the pivot (and, at p = 0, the split axis) and
//                 clears the histogram.
//     count       per chunk: keys below / equal to the pivot.
//     scatter     stable partition: per 256-point round a ballot/mbcnt scan
//                 gives each point its rank among left or right points; the
//                 pivot-equal points with the smallest indices fill the left
//                 half.  Child extents are reduced per chunk.
//     extents     one workgroup per node merges the chunk extents into the
//                 two children.
//   Workgroups never wait on each other inside a launch: every hand-over is
//   a launch boundary.
//   finish      every node of <= 1024 points is loaded into LDS and every
//               remaining level is split there by single waves (8-bit radix
//               select with an LDS histogram, ballot-scan partition), then
//               perm[t] = idx.  With few nodes a 16-wave workgroup owns a
//               node: all its threads split a 1,024-point top segment
//               together, and below that its waves split a level's
//               segments in parallel; otherwise each wave owns a node.
//   padded      an uneven point count n: the tree has leaf * 2^L slots (the
//               smallest that holds n); a node of m points gives its left
//               child the ceil(m/2) smallest, and a leaf's unused slots hold
//               -1.  Built by one workgroup in LDS (slots <= 1024).
#include "common.h"

namespace bt {

constexpr int kThreads = 256;
constexpr int kFinish = 1024;   // largest node finished in LDS by one wave
constexpr int kFinishWaves = 2;   // 2 x 16 KB of records per workgroup
constexpr int kBins = 2048;

struct NodeState {
  uint32_t prefix;   // pivot bits fixed so far
  uint32_t rank;     // rank of the median inside the bits not yet fixed
  uint32_t need_eq;  // pivot-equal points that go left (after the last pass)
  uint32_t axis;
};

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

BT_DEV uint32_t block_sum_u32(uint32_t v, uint32_t* red) {
  v = wave_sum_u32(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) t += red[i];
  return t;
}

// ------------------------------------------------------------------ init ----
__global__ void tree_init(uint32_t* zero_region, int64_t nwords, uint32_t* ext_root) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords;
       i += (int64_t)gridDim.x * blockDim.x)
    zero_region[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x < 6) ext_root[threadIdx.x] = threadIdx.x < 3 ? 0xffffffffu : 0u;
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
                                                        float4* __restrict__ rec,
                                                        uint32_t* __restrict__ ext_root,
                                                        int want_ext) {
  uint32_t mn[3] = {0xffffffffu, 0xffffffffu, 0xffffffffu}, mx[3] = {0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float x = coords[3 * i], y = coords[3 * i + 1], z = coords[3 * i + 2];
    if (rotate) {
      const float a0 = rot_row(r00, r01, r02, x, y, z);
      const float a1 = rot_row(r10, r11, r12, x, y, z);
      const float a2 = rot_row(r20, r21, r22, x, y, z);
      x = a0; y = a1; z = a2;
    }
    x = canon_zero(x); y = canon_zero(y); z = canon_zero(z);
    rec[i] = make_float4(x, y, z, __int_as_float((int)i));
    const uint32_t k[3] = {float_key(x), float_key(y), float_key(z)};
#pragma unroll
    for (int a = 0; a < 3; ++a) { mn[a] = min(mn[a], k[a]); mx[a] = max(mx[a], k[a]); }
  }
  if (!want_ext) return;
#pragma unroll
  for (int a = 0; a < 3; ++a) { mn[a] = wave_min_u32(mn[a]); mx[a] = wave_max_u32(mx[a]); }
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int a = 0; a < 3; ++a) { atomicMin(&ext_root[a], mn[a]); atomicMax(&ext_root[3 + a], mx[a]); }
  }
}

// ---------------------------------------------------------- radix passes ----
// Pass 0: bits 31..21, pass 1: bits 20..10, pass 2: bits 9..0.  Workgroups
// own one chunk of one node; they only add their LDS histogram into the
// node's global histogram.  Nothing is handed between workgroups inside a
// launch: the select of each pass is its own launch.
template <int PASS>
__global__ __launch_bounds__(kThreads) void tree_hist(const float4* __restrict__ rec, int chunk,
                                                      int cpn, const uint32_t* __restrict__ ext,
                                                      const NodeState* __restrict__ st,
                                                      uint32_t* __restrict__ hist) {
  constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr int HI = PASS == 0 ? 32 : (PASS == 1 ? 21 : 10);
  constexpr uint32_t MASK = PASS == 2 ? 1023u : 2047u;
  __shared__ uint32_t lh[kBins];
  const int tid = threadIdx.x;
  const int c = blockIdx.x;
  const int node = c / cpn;
  // pass 0 takes the axis from the node's extents; later passes from the
  // state written by the previous select
  const int axis = PASS == 0 ? axis_of(ext + 6 * node) : (int)st[node].axis;
  const uint32_t prefix = PASS == 0 ? 0u : st[node].prefix;
  for (int i = tid; i < kBins; i += kThreads) lh[i] = 0u;
  __syncthreads();
  const float4* r = rec + (int64_t)c * chunk;
  for (int i = tid; i < chunk; i += kThreads) {
    const uint32_t key = float_key(comp(r[i], axis));
    bool match = true;
    if constexpr (PASS > 0) match = (key >> HI) == (prefix >> HI);
    if (match) atomicAdd(&lh[(key >> SHIFT) & MASK], 1u);
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)node * kBins;
  for (int i = tid; i < kBins; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// One workgroup per node: find the bin holding the median's rank, fix that
// digit of the pivot, and clear the histogram for the next pass.  Pass 0
// also chooses the split axis from the node's extents.
template <int PASS>
__global__ __launch_bounds__(kThreads) void tree_select(int64_t nsize,
                                                        const uint32_t* __restrict__ ext,
                                                        NodeState* __restrict__ st,
                                                        uint32_t* __restrict__ hist) {
  constexpr int SHIFT = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr int PER = kBins / kThreads;   // 8 bins per thread
  __shared__ uint32_t red[kThreads / 64];
  __shared__ NodeState s_new;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int node = blockIdx.x;
  NodeState s;
  if (PASS == 0) {
    s.prefix = 0u;
    s.rank = (uint32_t)(nsize / 2 - 1);
    s.need_eq = 0u;
    s.axis = (uint32_t)axis_of(ext + 6 * node);
  } else {
    s = st[node];
  }
  uint32_t* gh = hist + (int64_t)node * kBins;
  uint32_t h[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) { h[j] = gh[tid * PER + j]; tot += h[j]; }
  const uint32_t incl = wave_incl_scan_u32(tot);
  if (lane == 63) red[w] = incl;
  if (tid == 0) {                     // written if no bin matches (never,
    s_new = s;                        // for a consistent histogram)
    s_new.need_eq = 1u;
  }
  __syncthreads();
  uint32_t cum = incl - tot;
  for (int i = 0; i < w; ++i) cum += red[i];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (h[j] && cum <= s.rank && s.rank < cum + h[j]) {
      NodeState t = s;
      t.prefix = s.prefix | ((uint32_t)(tid * PER + j) << SHIFT);
      t.rank = s.rank - cum;
      t.need_eq = t.rank + 1u;        // meaningful after the last pass
      s_new = t;
    }
    cum += h[j];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) gh[tid * PER + j] = 0u;
  __syncthreads();
  if (tid == 0) st[node] = s_new;
}

// ----------------------------------------------------------------- count ----
__global__ __launch_bounds__(kThreads) void tree_count(const float4* __restrict__ rec, int chunk,
                                                       int cpn, const NodeState* __restrict__ st,
                                                       uint2* __restrict__ counts) {
  __shared__ uint32_t red[kThreads / 64];
  const int c = blockIdx.x;
  const int node = c / cpn;
  const NodeState s = st[node];
  const float4* r = rec + (int64_t)c * chunk;
  uint32_t lt = 0, eq = 0;
  for (int i = threadIdx.x; i < chunk; i += kThreads) {
    const uint32_t key = float_key(comp(r[i], (int)s.axis));
    lt += key < s.prefix;
    eq += key == s.prefix;
  }
  lt = block_sum_u32(lt, red);
  eq = block_sum_u32(eq, red);
  if (threadIdx.x == 0) counts[c] = make_uint2(lt, eq);
}

// --------------------------------------------------------------- scatter ----
__global__ __launch_bounds__(kThreads) void tree_scatter(
    const float4* __restrict__ rec, float4* __restrict__ out, int64_t nsize, int chunk, int cpn,
    const NodeState* __restrict__ st, const uint2* __restrict__ counts,
    uint32_t* __restrict__ partials) {
  __shared__ uint32_t red[kThreads / 64];
  __shared__ uint32_t wlt[kThreads / 64], weq[kThreads / 64];
  __shared__ uint32_t pred[12][kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = blockIdx.x;
  const int node = c / cpn;
  const int first = node * cpn;
  const NodeState s = st[node];
  const uint32_t pivot = s.prefix, need_eq = s.need_eq;
  const int axis = (int)s.axis;

  // points of this node in earlier chunks
  uint32_t ltb = 0, eqb = 0;
  for (int i = first + tid; i < c; i += kThreads) { ltb += counts[i].x; eqb += counts[i].y; }
  ltb = block_sum_u32(ltb, red);
  eqb = block_sum_u32(eqb, red);
  const uint32_t left_before = ltb + min(eqb, need_eq);
  const uint32_t right_before = (uint32_t)(c - first) * (uint32_t)chunk - left_before;
  const int64_t nstart = (int64_t)node * nsize;
  const int64_t half = nsize / 2;

  uint32_t E = eqb, Lrun = left_before, Rrun = right_before;
  uint32_t lmin[3] = {~0u, ~0u, ~0u}, lmax[3] = {0u, 0u, 0u};
  uint32_t rmin[3] = {~0u, ~0u, ~0u}, rmax[3] = {0u, 0u, 0u};
  const float4* r = rec + (int64_t)c * chunk;
  for (int base = 0; base < chunk; base += kThreads) {
    // a chunk need not be a multiple of the workgroup: the valid lanes of
    // the last round are its first chunk - base threads
    const bool valid = base + tid < chunk;
    const int nvalid = min(kThreads, chunk - base);
    const float4 x = valid ? r[base + tid] : make_float4(0.f, 0.f, 0.f, 0.f);
    const uint32_t key = float_key(comp(x, axis));
    const bool is_lt = valid && key < pivot, is_eq = valid && key == pivot;
    const uint64_t blt = __ballot(is_lt), beq = __ballot(is_eq);
    const uint32_t lt_ex = mbcnt64(blt);
    const uint32_t eq_ex = mbcnt64(beq);
    if (lane == 0) { wlt[w] = __popcll(blt); weq[w] = __popcll(beq); }
    __syncthreads();
    uint32_t ltw = 0, eqw = 0, ltt = 0, eqt = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
      if (i < w) { ltw += wlt[i]; eqw += weq[i]; }
      ltt += wlt[i]; eqt += weq[i];
    }
    const uint32_t lt_p = ltw + lt_ex, eq_p = eqw + eq_ex;       // exclusive in round
    const uint32_t cap0 = min(E, need_eq);
    const bool left = is_lt || (is_eq && (E + eq_p) < need_eq);
    const uint32_t left_p = lt_p + (min(E + eq_p, need_eq) - cap0);
    const uint32_t left_tot = ltt + (min(E + eqt, need_eq) - cap0);
    const int64_t dest = left ? nstart + Lrun + left_p
                              : nstart + half + Rrun + ((uint32_t)tid - left_p);
    // ranks are consistent by construction; the guard keeps a broken
    // invariant from ever writing outside the node
    if (valid && dest >= nstart && dest < nstart + nsize) out[dest] = x;
    const uint32_t k3[3] = {float_key(x.x), float_key(x.y), float_key(x.z)};
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      if (!valid) continue;
      if (left) { lmin[a] = min(lmin[a], k3[a]); lmax[a] = max(lmax[a], k3[a]); }
      else { rmin[a] = min(rmin[a], k3[a]); rmax[a] = max(rmax[a], k3[a]); }
    }
    Lrun += left_tot;
    Rrun += (uint32_t)nvalid - left_tot;
    E += eqt;
    __syncthreads();
  }
  // ---- child extents of this chunk ----
  uint32_t v12[12];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    v12[a] = wave_min_u32(lmin[a]); v12[3 + a] = wave_max_u32(lmax[a]);
    v12[6 + a] = wave_min_u32(rmin[a]); v12[9 + a] = wave_max_u32(rmax[a]);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 12; ++j) pred[j][w] = v12[j];
  }
  __syncthreads();
  if (tid < 12) {
    uint32_t v = pred[tid][0];
    for (int i = 1; i < kThreads / 64; ++i)
      v = ((tid % 6) < 3) ? min(v, pred[tid][i]) : max(v, pred[tid][i]);
    partials[(int64_t)c * 12 + tid] = v;
  }
}

// One workgroup per node: merge the chunk extents into both children.
__global__ __launch_bounds__(kThreads) void tree_extents(const uint32_t* __restrict__ partials,
                                                         int cpn, uint32_t* __restrict__ ext_next) {
  __shared__ uint32_t pred[12][kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int node = blockIdx.x;
  const int first = node * cpn;
  uint32_t acc[12];
#pragma unroll
  for (int j = 0; j < 12; ++j) acc[j] = ((j % 6) < 3) ? ~0u : 0u;
  for (int i = first + tid; i < first + cpn; i += kThreads) {
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const uint32_t v = partials[(int64_t)i * 12 + j];
      acc[j] = ((j % 6) < 3) ? min(acc[j], v) : max(acc[j], v);
    }
  }
#pragma unroll
  for (int j = 0; j < 12; ++j) acc[j] = ((j % 6) < 3) ? wave_min_u32(acc[j]) : wave_max_u32(acc[j]);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < 12; ++j) pred[j][w] = acc[j];
  }
  __syncthreads();
  if (tid < 12) {
    uint32_t v = pred[tid][0];
    for (int i = 1; i < kThreads / 64; ++i)
      v = ((tid % 6) < 3) ? min(v, pred[tid][i]) : max(v, pred[tid][i]);
    ext_next[(int64_t)(2 * node) * 6 + tid] = v;   // 12 words: left child then right
  }
}

// ---------------------------------------------------------------- finish ----

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

__global__ __launch_bounds__(kFinishWaves * 64) void tree_finish(const float4* __restrict__ rec,
                                                                 int nf, int leaf, int nnodes,
                                                                 int32_t* __restrict__ perm) {
  __shared__ float4 srec[kFinishWaves][kFinish];
  __shared__ uint32_t shist[kFinishWaves][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int node = blockIdx.x * kFinishWaves + w;
  if (node >= nnodes) return;          // no workgroup barrier below
  float4* R = srec[w];
  uint32_t* hist = shist[w];
  const int64_t base = (int64_t)node * nf;
  for (int i = lane; i < nf; i += 64) R[i] = rec[base + i];
  __builtin_amdgcn_wave_barrier();
  for (int m = nf; m > leaf; m >>= 1)
    for (int o = 0; o < nf; o += m) wave_split(R + o, m, hist, lane);
  for (int i = lane; i < nf; i += 64) perm[base + i] = __float_as_int(R[i].w);
}

// One workgroup of kFinishBlockWaves waves per node of <= kFinish points:
// the segments of a level are independent, so the waves take them in turn
// (wave w splits segments w, w + waves, ...), with a workgroup barrier
// between levels.  Used when there are few nodes (a small tree has one).
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

// Segments of at least this many points are split by the whole workgroup;
// smaller ones by one wave each, the waves taking the segments in turn.  At
// 1,024 points the block-wide top split took the build from 47 to 39 us;
// block-wide splits of 256- and 512-point segments (one after another) lost
// more to barriers than they gained.
constexpr int kBlockSplitMin = 1024;

__global__ __launch_bounds__(kFinishBlockWaves * 64) void tree_finish_block(
    const float4* __restrict__ rec, int nf, int leaf, int32_t* __restrict__ perm) {
  __shared__ float4 srec[kFinish];
  __shared__ uint32_t shist[kFinishBlockWaves][256];
  __shared__ BlockSplitLds bsl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * nf;
  for (int i = tid; i < nf; i += kFinishBlockWaves * 64) srec[i] = rec[base + i];
  __syncthreads();
  for (int m = nf; m > leaf; m >>= 1) {
    const int nseg = nf / m;
    if (m >= kBlockSplitMin) {
      for (int sgi = 0; sgi < nseg; ++sgi) block_split(srec + sgi * m, m, bsl, shist);
    } else {
      for (int sgi = w; sgi < nseg; sgi += kFinishBlockWaves)
        wave_split(srec + sgi * m, m, shist[w], lane);
      __syncthreads();
    }
  }
  for (int i = tid; i < nf; i += kFinishBlockWaves * 64) perm[base + i] = __float_as_int(srec[i].w);
}

// Padded tree: start and point count of segment s at level lev, found by
// walking down from the root (n points), the left child taking ceil(cnt/2).
BT_DEV void padded_segment(int n, int lev, int s, int* start, int* cnt) {
  int st = 0, c = n;
  for (int i = lev - 1; i >= 0; --i) {
    const int nl = (c + 1) >> 1;
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

// One workgroup builds a padded tree of n <= ncap <= kFinish points: the
// points stay compacted in LDS (every segment of a level is a contiguous run),
// each level splits its segments of two or more points in place (the waves
// take them in turn), then leaf j's points go to slots j*leaf ... in order
// and the leaf's remaining slots get -1.
__global__ __launch_bounds__(kFinishBlockWaves * 64) void tree_finish_padded(
    const float4* __restrict__ rec, int n, int ncap, int leaf, int32_t* __restrict__ perm) {
  __shared__ float4 srec[kFinish];
  __shared__ uint32_t shist[kFinishBlockWaves][256];
  __shared__ BlockSplitLds bsl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < n; i += kFinishBlockWaves * 64) srec[i] = rec[i];
  __syncthreads();
  int lev = 0;
  for (int slots = ncap; slots > leaf; slots >>= 1, ++lev) {
    if (slots >= kBlockSplitMin) {           // uniform: every thread walks the segments
      for (int sgi = 0; sgi < (1 << lev); ++sgi) {
        int st, cnt;
        padded_segment(n, lev, sgi, &st, &cnt);
        if (cnt >= 2) block_split(srec + st, cnt, bsl, shist);
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
  for (int t = tid; t < ncap; t += kFinishBlockWaves * 64) {
    const int j = t / leaf, i = t - j * leaf;
    int st, cnt;
    padded_segment(n, lev, j, &st, &cnt);
    perm[t] = i < cnt ? __float_as_int(srec[st + i].w) : -1;
  }
}

// A padded tree that is a single leaf: the points in index order, then -1.
__global__ __launch_bounds__(kThreads) void tree_single_leaf_padded(int64_t n, int64_t ncap,
                                                                    int32_t* __restrict__ perm) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < ncap;
       t += (int64_t)gridDim.x * blockDim.x)
    perm[t] = t < n ? (int32_t)t : -1;
}

__global__ __launch_bounds__(kThreads) void tree_write_perm(const float4* __restrict__ rec,
                                                            int64_t n, int32_t* __restrict__ perm) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    perm[i] = __float_as_int(rec[i].w);
}

// ------------------------------------------------------------------ host ----
struct TreePlan {
  int64_t n;
  int leaf;
  int L;         // total levels
  int G;         // levels split by the global passes
  int64_t nf;    // node size handed to the finisher
  size_t off_rec0, off_rec1, off_ext0, off_ext1, off_hist, off_state, off_counts,
      off_part, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Points per chunk of a node of nsize = leaf * 2^k points: nsize halved while
// it is even and above the target, so that the chunks tile every node
// exactly.  A chunk is above half the target, or odd and above it.
static int chunk_for(int64_t n_total, int64_t nsize) {
  int64_t target = 1024;
  if (n_total >= (int64_t)1 << 19) target = 4096;
  else if (n_total >= (int64_t)1 << 18) target = 2048;
  int64_t c = nsize;
  while (c > target && (c & 1) == 0) c >>= 1;
  return (int)c;
}

static TreePlan plan_tree(int64_t n, int leaf) {
  TreePlan p{};
  p.n = n;
  p.leaf = leaf;
  int L = 0;
  while (((int64_t)leaf << L) < n) ++L;
  p.L = L;
  int G = 0;
  while (G < L && (n >> G) > kFinish) ++G;
  p.G = G;
  p.nf = n >> G;
  size_t o = 0;
  p.off_rec0 = o; o = align256(o + (size_t)n * 16);
  p.off_rec1 = o; o = align256(o + (size_t)n * 16);
  const size_t nodes_next = (size_t)1 << G;            // children of the last global level
  const size_t nodes_max = G ? ((size_t)1 << (G - 1)) : 1;
  p.off_ext0 = o; o = align256(o + nodes_next * 6 * 4);
  p.off_ext1 = o; o = align256(o + nodes_next * 6 * 4);
  p.off_hist = o; o = align256(o + nodes_max * kBins * 4);
  p.off_state = o; o = align256(o + nodes_max * sizeof(NodeState));
  size_t max_chunks = 1;
  for (int lev = 0; lev < G; ++lev) {
    const size_t nc = (size_t)(n / chunk_for(n, n >> lev));
    if (nc > max_chunks) max_chunks = nc;
  }
  p.off_counts = o; o = align256(o + max_chunks * 8);
  p.off_part = o; o = align256(o + max_chunks * 12 * 4);
  p.total = o;
  return p;
}

size_t tree_workspace_size(int64_t n, int leaf) { return plan_tree(n, leaf).total; }

bt_status tree_build_launch(const float* coords, int64_t n, int leaf, const float* R,
                            int32_t* perm, void* ws, hipStream_t st) {
  const TreePlan p = plan_tree(n, leaf);
  char* b = (char*)ws;
  float4* rec[2] = {(float4*)(b + p.off_rec0), (float4*)(b + p.off_rec1)};
  uint32_t* ext[2] = {(uint32_t*)(b + p.off_ext0), (uint32_t*)(b + p.off_ext1)};
  uint32_t* hist = (uint32_t*)(b + p.off_hist);
  NodeState* state = (NodeState*)(b + p.off_state);
  uint2* counts = (uint2*)(b + p.off_counts);
  uint32_t* part = (uint32_t*)(b + p.off_part);

  if (p.G > 0) {
    // zero every histogram and completion counter once; the last workgroup of
    // each node clears what it used, so they stay zero between passes
    const int64_t nwords = (int64_t)((p.off_state - p.off_hist) / 4);
    hipLaunchKernelGGL(tree_init, dim3(64), dim3(256), 0, st, hist, nwords, ext[0]);
    bt_status s = launch_status("tree_init");
    if (s != BT_OK) return s;
  }
  {
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 256) g = 256;
    const float* r = R;
    float rr[9] = {1, 0, 0, 0, 1, 0, 0, 0, 1};
    if (r) for (int i = 0; i < 9; ++i) rr[i] = r[i];
    hipLaunchKernelGGL(tree_ingest, dim3((int)g), dim3(kThreads), 0, st, coords, n, r ? 1 : 0,
                       rr[0], rr[1], rr[2], rr[3], rr[4], rr[5], rr[6], rr[7], rr[8], rec[0],
                       ext[0], p.G > 0 ? 1 : 0);
    bt_status s = launch_status("tree_ingest");
    if (s != BT_OK) return s;
  }
  for (int lev = 0; lev < p.G; ++lev) {
    const int64_t nsize = n >> lev;
    const int chunk = chunk_for(n, nsize);
    const int cpn = (int)(nsize / chunk);
    const int nchunks = (int)(n / chunk);
    const int nodes = 1 << lev;
    float4* cur = rec[lev & 1];
    float4* nxt = rec[(lev + 1) & 1];
    uint32_t* ec = ext[lev & 1];
    uint32_t* en = ext[(lev + 1) & 1];
    const dim3 gc(nchunks), gn(nodes), blk(kThreads);
    hipLaunchKernelGGL(tree_hist<0>, gc, blk, 0, st, cur, chunk, cpn, ec, state, hist);
    hipLaunchKernelGGL(tree_select<0>, gn, blk, 0, st, nsize, ec, state, hist);
    hipLaunchKernelGGL(tree_hist<1>, gc, blk, 0, st, cur, chunk, cpn, ec, state, hist);
    hipLaunchKernelGGL(tree_select<1>, gn, blk, 0, st, nsize, ec, state, hist);
    hipLaunchKernelGGL(tree_hist<2>, gc, blk, 0, st, cur, chunk, cpn, ec, state, hist);
    hipLaunchKernelGGL(tree_select<2>, gn, blk, 0, st, nsize, ec, state, hist);
    hipLaunchKernelGGL(tree_count, gc, blk, 0, st, cur, chunk, cpn, state, counts);
    hipLaunchKernelGGL(tree_scatter, gc, blk, 0, st, cur, nxt, nsize, chunk, cpn, state, counts,
                       part);
    hipLaunchKernelGGL(tree_extents, gn, blk, 0, st, part, cpn, en);
    bt_status s = launch_status("tree level");
    if (s != BT_OK) return s;
  }
  const float4* fin = rec[p.G & 1];
  if (p.nf == leaf) {
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(tree_write_perm, dim3((int)g), dim3(kThreads), 0, st, fin, n, perm);
    return launch_status("tree_write_perm");
  }
  const int nnodes = (int)(n / p.nf);
  if (nnodes <= 256) {                       // few nodes: a workgroup per node
    hipLaunchKernelGGL(tree_finish_block, dim3(nnodes), dim3(kFinishBlockWaves * 64), 0, st,
                       fin, (int)p.nf, leaf, perm);
    return launch_status("tree_finish_block");
  }
  hipLaunchKernelGGL(tree_finish, dim3((nnodes + kFinishWaves - 1) / kFinishWaves),
                     dim3(kFinishWaves * 64), 0, st, fin, (int)p.nf, leaf, nnodes, perm);
  return launch_status("tree_finish");
}

int64_t tree_padded_slots(int64_t n, int leaf) {
  int64_t cap = leaf;
  while (cap < n) cap *= 2;
  return cap;
}

size_t tree_padded_workspace_size(int64_t n, int leaf) {
  return tree_padded_slots(n, leaf) == leaf ? 256 : align256((size_t)n * 16);
}

// Padded tree of n points: one leaf of any size, or up to kFinish slots.
bt_status tree_build_padded_launch(const float* coords, int64_t n, int leaf, const float* R,
                                   int32_t* perm, void* ws, hipStream_t st) {
  const int64_t ncap = tree_padded_slots(n, leaf);
  if (ncap == leaf) {
    int64_t g = (ncap + kThreads - 1) / kThreads;
    if (g > 4096) g = 4096;
    hipLaunchKernelGGL(tree_single_leaf_padded, dim3((int)g), dim3(kThreads), 0, st, n, ncap,
                       perm);
    return launch_status("tree_single_leaf_padded");
  }
  if (ncap > kFinish) return BT_EINVAL;
  float4* rec = (float4*)ws;
  const float* r = R;
  float rr[9] = {1, 0, 0, 0, 1, 0, 0, 0, 1};
  if (r) for (int i = 0; i < 9; ++i) rr[i] = r[i];
  int64_t g = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(tree_ingest, dim3((int)g), dim3(kThreads), 0, st, coords, n, r ? 1 : 0,
                     rr[0], rr[1], rr[2], rr[3], rr[4], rr[5], rr[6], rr[7], rr[8], rec,
                     (uint32_t*)nullptr, 0);
  bt_status s = launch_status("tree_ingest");
  if (s != BT_OK) return s;
  hipLaunchKernelGGL(tree_finish_padded, dim3(1), dim3(kFinishBlockWaves * 64), 0, st, rec,
                     (int)n, (int)ncap, leaf, perm);
  return launch_status("tree_finish_padded");
}

}  // namespace bt
