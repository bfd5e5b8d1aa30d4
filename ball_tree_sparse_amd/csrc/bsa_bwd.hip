// Backward of Ball Sparse Attention without group compression.  The
// branches and gates of BSA are learned (Pith review of arXiv 2506.12541,
// "What carries the argument"), so training needs dq, dk, dv and the
// gradients of the gate parameters.  With out = G0 O_ball + G1 O_cmp +
// G2 O_slc and G = sigmoid(W q + b), every branch is softmax attention whose
// output gradient is G_i dO; the top-k selection is a step function and
// passes no gradient (the selection of the forward is recomputed and held
// fixed).  All work is in tree order:
//
//   prepare   the forward's pooled layouts and selection (bsa_prepare), and
//             row-major V plus K, Q and dO transposed in 32-row blocks (the
//             operand layouts of the products below); the coarse tokens
//             likewise.
//   index     for every (head, block) the groups that selected the block, in
//             ascending group order (a per-chunk count, a scan and an
//             in-order fill, so the result is deterministic).
//   queries   one wave per 32 or 64 queries, one sweep per branch: with
//             p = exp(S - m) under an online maximum m, it sums l = sum p,
//             c = sum p dP, A = K^T (p dP) and Bv = K^T p, so that dG_i =
//             dO . O_i = c / l, D_i = G_i dG_i and dQ^T = (G_i A - D_i Bv) / l
//             (S^T = K Q^T and dP^T = V dO^T are formed once per key).  The
//             gate term sum_i dz_i W[i] with dz_i = dG_i G_i (1 - G_i) is
//             added, dq is written in original order, and (m, 1/l, G_i, D_i)
//             are kept.
//   keys      one wave per 32 or 64 keys: for every query block that attends to
//             them, S = Q K^T, dP = dO V^T, P from the kept statistics, dS =
//             P (G dP - D), dV^T += dO^T (G P) and dK^T += Q^T dS.  Ball keys
//             see their ball's queries; selected blocks see the groups that
//             selected them; coarse tokens see every query (split over
//             partitions whose partial sums are added in a fixed order).
//   finish    dk = dK_ball + dK_slc + dKc[block] / l (and dv likewise),
//             rounded to bf16 and scattered to original order; the gate
//             parameter gradients are summed from per-wave partials.
//
// Products run on v_mfma_f32_32x32x16_bf16 in the operand layouts of the
// forward: p, p dP, dS and G P are rounded to bf16 for the MFMA; statistics
// and accumulators are fp32.
#include "bsa_common.h"
#include "lds_tile.h"

namespace bt {

bt_status bsa_prepare(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                      int32_t H, int32_t d, const bsa_params* p, void* ws, int32_t* sel,
                      hipStream_t st);

constexpr int kCmpParts = 16;     // query partitions of the coarse-token key pass
constexpr int kIdxChunk = 64;     // groups per chunk of the selection index

struct BsaBwdLayout {
  BsaLayout f;                      // the forward's workspace
  size_t vr, qr, dor;               // [h][t][d] row-major V, Q and dO
  size_t ktt;                       // [h][t/32][d][32]: K transposed
  size_t vcr, kctt;                 // coarse tokens: Vc row-major, Kc transposed
  size_t stats;                     // [h][3][t] float4 (m, 1/l, G_i, D_i)
  size_t dkacc, dvacc;              // [h][t][d] fp32
  size_t cpart;                     // [part][2][h][nc][d] fp32
  size_t dkc, dvc;                  // [h][nc][d] fp32
  size_t gpart;                     // [3][d + 1][H * N/32] fp32
  size_t cntc, basec, off, list;    // selection index
  size_t total;
};

static BsaBwdLayout bsa_bwd_layout(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  BsaBwdLayout L{};
  L.f = bsa_layout(N, H, d, p);
  const size_t nc = (size_t)(N / p->block), G = (size_t)(N / p->group);
  const size_t nchunk = (G + kIdxChunk - 1) / kIdxChunk;
  const size_t rows = (size_t)N * H * d;
  size_t o = L.f.total;
  L.vr = o; o = a256(o + rows * 2);
  L.qr = o; o = a256(o + rows * 2);
  L.dor = o; o = a256(o + rows * 2);
  L.ktt = o; o = a256(o + rows * 2);
  L.vcr = o; o = a256(o + nc * H * d * 2);
  L.kctt = o; o = a256(o + nc * H * d * 2);
  L.stats = o; o = a256(o + (size_t)N * H * 3 * 16);
  L.dkacc = o; o = a256(o + rows * 4);
  L.dvacc = o; o = a256(o + rows * 4);
  L.cpart = o; o = a256(o + (size_t)kCmpParts * 2 * H * nc * d * 4);
  L.dkc = o; o = a256(o + (size_t)H * nc * d * 4);
  L.dvc = o; o = a256(o + (size_t)H * nc * d * 4);
  L.gpart = o; o = a256(o + (size_t)(N / 32) * H * 3 * (d + 1) * 4);
  L.cntc = o; o = a256(o + (size_t)H * nchunk * nc * 4);
  L.basec = o; o = a256(o + (size_t)H * nchunk * nc * 4);
  L.off = o; o = a256(o + (size_t)H * (nc + 1) * 4);
  L.list = o; o = a256(o + (size_t)H * G * p->topk * 4);
  L.total = o;
  return L;
}

size_t bsa_bwd_ws_size(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  return bsa_bwd_layout(N, H, d, p).total;
}

// ------------------------------------------------------------ layouts ----
// Grid (N/32 row blocks, H), one wave: rows t0 .. t0+31 of head h gathered
// through perm.  V, Q and dO are written row-major, K also transposed per
// block, position p of a [d][32] row holding row tpos(p) (the key order of
// the forward's transposed V).
template <int D>
__global__ __launch_bounds__(64) void bsa_bwd_prep(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const uint16_t* __restrict__ dout,
                                                   const int32_t* __restrict__ perm, int32_t H,
                                                   int64_t N, uint16_t* __restrict__ vr,
                                                   uint16_t* __restrict__ qr,
                                                   uint16_t* __restrict__ dor,
                                                   uint16_t* __restrict__ ktt) {
  constexpr int CPR = D / 8;                     // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) uint16_t tl[32 * D];
  const int lane = threadIdx.x;
  const int64_t blk = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t t0 = blk * 32;
  const int64_t rs = (int64_t)H * D;
  for (int it = lane; it < 32 * CPR; it += 64) {
    const int r = it / CPR, ch = it - r * CPR;
    const int64_t src = perm_index(perm[t0 + r], N) * rs + (int64_t)h * D + ch * 8;
    const int64_t dst = ((int64_t)h * N + t0 + r) * D + ch * 8;
    *(u32x4*)(vr + dst) = *(const u32x4*)(v + src);
    *(u32x4*)(qr + dst) = *(const u32x4*)(q + src);
    *(u32x4*)(dor + dst) = *(const u32x4*)(dout + src);
    *(u32x4*)&tl[r * D + ch * 8] = *(const u32x4*)(k + src);
  }
  __syncthreads();
  for (int it = lane; it < 4 * D; it += 64) {
    const int dd = it >> 2, q8 = it & 3;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = tpos(q8 * 8 + 2 * e), r1 = tpos(q8 * 8 + 2 * e + 1);
      o[e] = uint32_t(tl[r0 * D + dd]) | (uint32_t(tl[r1 * D + dd]) << 16);
    }
    *(u32x4*)(ktt + (((int64_t)h * (N / 32) + blk) * D + dd) * 32 + q8 * 8) = o;
  }
}

// Grid (nc/32, H), one wave: coarse tokens jb*32 .. jb*32+31.  Kc (row-major
// bf16 [h][j][d]) is written transposed like K; Vc (transposed [h][j/32][d]
// [32]) is written row-major like V.
template <int D>
__global__ __launch_bounds__(64) void bsa_bwd_prep_coarse(const uint16_t* __restrict__ kcb,
                                                          const uint16_t* __restrict__ vct,
                                                          int32_t nc, uint16_t* __restrict__ vcr,
                                                          uint16_t* __restrict__ kctt) {
  const int lane = threadIdx.x;
  const int64_t jb = blockIdx.x;
  const int h = blockIdx.y;
  const uint16_t* kh = kcb + (int64_t)h * nc * D;
  const uint16_t* vb = vct + ((int64_t)h * (nc / 32) + jb) * D * 32;
  for (int it = lane; it < 32 * D; it += 64) {
    const int dd = it >> 5, p = it & 31;         // transposed Kc
    kctt[(((int64_t)h * (nc / 32) + jb) * D + dd) * 32 + p] = kh[(jb * 32 + tpos(p)) * D + dd];
    const int r = it / D, e = it - r * D;        // row-major Vc
    vcr[((int64_t)h * nc + jb * 32 + r) * D + e] = vb[e * 32 + tpos(r)];
  }
}

// ------------------------------------------------------ selection index ----
// cntc[h][c][j]: how many groups of chunk c (kIdxChunk groups) selected block
// j.  Grid (chunks, H), one wave; block indices of a group are distinct.
__global__ __launch_bounds__(64) void bsa_bwd_sel_count(const int32_t* __restrict__ sel,
                                                        int32_t nc, int32_t ngroups, int32_t topk,
                                                        uint32_t* __restrict__ cntc) {
  HIP_DYNAMIC_SHARED(uint32_t, cnt)
  const int lane = threadIdx.x;
  const int c = blockIdx.x, h = blockIdx.y, nchunk = gridDim.x;
  for (int j = lane; j < nc; j += 64) cnt[j] = 0u;
  __syncthreads();
  const int g0 = c * kIdxChunk, g1 = min(ngroups, g0 + kIdxChunk);
  for (int e = lane; e < (g1 - g0) * topk; e += 64) {
    const int j = (int)perm_index(sel[((int64_t)h * ngroups + g0) * topk + e], nc);
    atomicAdd(&cnt[j], 1u);
  }
  __syncthreads();
  uint32_t* out = cntc + ((int64_t)h * nchunk + c) * nc;
  for (int j = lane; j < nc; j += 64) out[j] = cnt[j];
}

// Grid (H), 1024 threads: off[h][j] = groups that selected blocks below j;
// basec[h][c][j] = off[h][j] + the count of chunks before c.
__global__ __launch_bounds__(1024) void bsa_bwd_sel_scan(const uint32_t* __restrict__ cntc,
                                                         int32_t nc, int32_t nchunk,
                                                         uint32_t* __restrict__ basec,
                                                         uint32_t* __restrict__ off) {
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = blockIdx.x;
  const uint32_t* ch = cntc + (int64_t)h * nchunk * nc;
  uint32_t* bh = basec + (int64_t)h * nchunk * nc;
  uint32_t* oh = off + (int64_t)h * (nc + 1);
  // each thread owns a run of consecutive blocks
  const int per = (nc + 1023) / 1024;
  const int j0 = min(nc, tid * per), j1 = min(nc, j0 + per);
  uint32_t run = 0;
  for (int j = j0; j < j1; ++j)
    for (int c = 0; c < nchunk; ++c) run += ch[(int64_t)c * nc + j];
  const uint32_t incl = wave_incl_scan_u32(run);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  uint32_t before = incl - run;
  for (int i = 0; i < w; ++i) before += wsum[i];
  for (int j = j0; j < j1; ++j) {
    oh[j] = before;
    uint32_t b = before;
    for (int c = 0; c < nchunk; ++c) {
      bh[(int64_t)c * nc + j] = b;
      b += ch[(int64_t)c * nc + j];
    }
    before = b;
  }
  if (tid == 1023) oh[nc] = before;
}

// Grid (chunks, H), one wave: the chunk's groups in ascending order append
// themselves to the lists of the blocks they selected.
__global__ __launch_bounds__(64) void bsa_bwd_sel_fill(const int32_t* __restrict__ sel,
                                                       const uint32_t* __restrict__ basec,
                                                       int32_t nc, int32_t ngroups, int32_t topk,
                                                       int32_t* __restrict__ list) {
  HIP_DYNAMIC_SHARED(uint32_t, cur)
  const int lane = threadIdx.x;
  const int c = blockIdx.x, h = blockIdx.y, nchunk = gridDim.x;
  const uint32_t* b = basec + ((int64_t)h * nchunk + c) * nc;
  for (int j = lane; j < nc; j += 64) cur[j] = b[j];
  __syncthreads();
  const int64_t cap = (int64_t)ngroups * topk;
  int32_t* lh = list + (int64_t)h * cap;
  const int g0 = c * kIdxChunk, g1 = min(ngroups, g0 + kIdxChunk);
  for (int g = g0; g < g1; ++g) {
    if (lane < topk) {
      const int j = (int)perm_index(sel[((int64_t)h * ngroups + g) * topk + lane], nc);
      const uint32_t pos = cur[j];
      cur[j] = pos + 1u;
      if ((int64_t)pos < cap) lh[pos] = g;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------- query pass ----
// One sweep per branch.  With p_k = exp(s_k - m) (online maximum m), l =
// sum p_k, c = sum p_k dP_k, A = sum p_k dP_k K_k and Bv = sum p_k K_k, the
// branch gives dG = dO . O = c / l, D = G dG and dQ = sum_k P_k (G dP_k - D)
// K_k = (G A - D Bv) / l, so S, dP and both K products are formed once per
// key (A and Bv as K^T products of the bf16-rounded p dP and p).
template <int DB>
struct QState {
  f32x16 a[DB], bv[DB];   // A^T, Bv^T: lane = query column, d in the accumulator layout
  float m;                // running maximum, log2-scaled units
  float l[2], c[2];       // partial sums of p and p dP
};

template <int DB>
BT_DEV void qstate_init(QState<DB>& q) {
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    q.a[db] = f32x16{};
    q.bv[db] = f32x16{};
  }
  q.m = -INFINITY;
  q.l[0] = q.l[1] = q.c[0] = q.c[1] = 0.f;
}

// NKB blocks of 32 keys (rows row0(kb) .. + 31) for the wave's QB query
// blocks; every K, V and K^T fragment serves all QB blocks.
template <int D, int NKB, int QB, typename RowFn>
BT_DEV void bwd_chunk(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vrh,
                      const uint16_t* __restrict__ kth, RowFn row0, const bf16x8* qf,
                      const bf16x8* dof, float c2, QState<D / 32>* st) {
  constexpr int DS = D / 16, DB = D / 32;
  const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
  bf16x8 kf[NKB][DS], vf[NKB][DS], tf[NKB][2][DB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int64_t r0 = row0(kb);
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kf[kb][s] = *(const bf16x8*)(kh + (r0 + c) * D + hf * 8 + s * 16);
      vf[kb][s] = *(const bf16x8*)(vrh + (r0 + c) * D + hf * 8 + s * 16);
    }
    const uint16_t* tb = kth + r0 * D + c * 32 + hf * 8;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        tf[kb][s2][db] = *(const bf16x8*)(tb + db * 32 * 32 + s2 * 16);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    QState<DB>& b = st[qb];
    f32x16 sa[NKB], pa[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sa[kb] = f32x16{};
      pa[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][s], qf[qb * DS + s], sa[kb], 0, 0, 0);
        pa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb][s], dof[qb * DS + s], pa[kb], 0, 0, 0);
      }
    }
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) m4[e & 3] = fmaxf(m4[e & 3], sa[kb][e]);
    float cm = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * c2;
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    // lazy rescale, as in the forward: only when a chunk maximum passes the
    // running one by more than 2^kLazyLog2, for the whole wave at once
    if (__ballot(cm > b.m + kLazyLog2)) {
      const float mn = fmaxf(b.m, cm);
      const float alpha = __builtin_amdgcn_exp2f(b.m - mn);   // 0 on the first chunk
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        b.l[i] *= alpha;
        b.c[i] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        b.a[db] *= alpha;
        b.bv[db] *= alpha;
      }
      b.m = mn;
    }
    const float mn = b.m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pb, pdb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sa[kb][s2 * 8 + e], c2, -mn));
          const float pd = pv * pa[kb][s2 * 8 + e];
          b.l[s2] += pv;
          b.c[s2] += pd;
          pb[e] = (__bf16)pv;
          pdb[e] = (__bf16)pd;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          b.a[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[kb][s2][db], pdb, b.a[db], 0, 0, 0);
          b.bv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[kb][s2][db], pb, b.bv[db], 0, 0, 0);
        }
      }
  }
}

// The branch's keys [0, len) (len a multiple of 32) in chunks of NKB blocks
// and a tail of single blocks; row0(key) gives the row of the block at key.
template <int D, int NKB, int QB, typename RowFn>
BT_DEV void bwd_range(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vrh,
                      const uint16_t* __restrict__ kth, RowFn row0, int len, const bf16x8* qf,
                      const bf16x8* dof, float c2, QState<D / 32>* st) {
  int k0 = 0;
  for (; k0 + 32 * NKB <= len; k0 += 32 * NKB)
    bwd_chunk<D, NKB, QB>(kh, vrh, kth, [&](int kb) -> int64_t { return row0(k0 + kb * 32); },
                          qf, dof, c2, st);
  if constexpr (NKB > 1) {
    for (; k0 < len; k0 += 32)
      bwd_chunk<D, 1, QB>(kh, vrh, kth, [&](int) -> int64_t { return row0(k0); }, qf, dof, c2,
                          st);
  }
}

// Grid (groups x H), NWV waves of QB blocks of 32 queries (group = 32 * NWV * QB);
// keys in chunks of NKB blocks of 32.
template <int D, int NWV, int QB, int NKB>
__global__ __launch_bounds__(NWV * 64) BT_WAVES_PER_EU(2, 8) void bsa_bwd_q(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
    const int32_t* __restrict__ perm, const uint16_t* __restrict__ kt,
    const uint16_t* __restrict__ vr, const uint16_t* __restrict__ ktt,
    const uint16_t* __restrict__ kcb, const uint16_t* __restrict__ vcr,
    const uint16_t* __restrict__ kctt, const int32_t* __restrict__ sel,
    const float* __restrict__ gate_w, const float* __restrict__ gate_b, float gc0, float gc1,
    float gc2, int32_t H, int64_t N, int32_t nc, int32_t ngroups, int32_t ball, int32_t block,
    int32_t topk, int32_t xcd_map, float4* __restrict__ stats, float* __restrict__ gpart,
    uint16_t* __restrict__ dq) {
  constexpr int DS = D / 16, DB = D / 32;
  __shared__ int32_t ssel[64];
  const int total = ngroups * H;
  int pair = blockIdx.x;
  if (xcd_map) pair = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int h = pair / ngroups;
  const int g = pair - h * ngroups;
  const int group = NWV * QB * 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, c = lane & 31;
  const int64_t rs = (int64_t)H * D;
  if (tid < topk)
    ssel[tid] = (int32_t)perm_index(sel[((int64_t)h * ngroups + g) * topk + tid], nc);

  // query block qb of this wave: tree positions t0 + qb*32 + c
  const int64_t t0 = (int64_t)g * group + w * (QB * 32);
  int64_t pq[QB];
  bf16x8 qf[QB * DS], dof[QB * DS];
  float G[QB][3];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    pq[qb] = perm_index(perm[t0 + qb * 32 + c], N);
    const uint16_t* qrow = q + pq[qb] * rs + (int64_t)h * D;
    const uint16_t* drow = dout + pq[qb] * rs + (int64_t)h * D;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[qb * DS + s] = *(const bf16x8*)(qrow + s * 16 + hf * 8);
      dof[qb * DS + s] = *(const bf16x8*)(drow + s * 16 + hf * 8);
    }
    G[qb][0] = gc0;
    G[qb][1] = gc1;
    G[qb][2] = gc2;
    if (gate_w) {
      float z[3] = {0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dd = s * 16 + hf * 8 + e;
          const float x = (float)qf[qb * DS + s][e];
#pragma unroll
          for (int i = 0; i < 3; ++i) z[i] = fmaf(gate_w[i * D + dd], x, z[i]);
        }
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        z[i] += __shfl_xor(z[i], 32, 64);
        if (gate_b) z[i] += gate_b[i];
        G[qb][i] = 1.0f / (1.0f + __expf(-z[i]));
      }
    }
  }
  __syncthreads();   // ssel

  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* kh = kt + (int64_t)h * N * D;
  const uint16_t* vrh = vr + (int64_t)h * N * D;
  const uint16_t* kth = ktt + (int64_t)h * N * D;
  const uint16_t* kch = kcb + (int64_t)h * nc * D;
  const uint16_t* vcrh = vcr + (int64_t)h * nc * D;
  const uint16_t* kcth = kctt + (int64_t)h * nc * D;
  const int64_t b0 = ((int64_t)g * group / ball) * ball;
  auto row_ball = [&](int key) -> int64_t { return b0 + key; };
  auto row_cmp = [&](int key) -> int64_t { return key; };
  auto row_slc = [&](int key) -> int64_t {
    return (int64_t)ssel[key / block] * block + (key % block);
  };

  // dQ^T per lane, kept in LDS between branches (registers go to the
  // branch state); lane-consecutive words, so free of bank conflicts
  __shared__ float sdq[NWV][QB][DB][16][64];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) sdq[w][qb][db][e][lane] = 0.f;
  float dG[QB][3];
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    QState<DB> S[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qstate_init<DB>(S[qb]);
    if (br == 0) bwd_range<D, NKB, QB>(kh, vrh, kth, row_ball, ball, qf, dof, c2, S);
    else if (br == 1) bwd_range<D, NKB, QB>(kch, vcrh, kcth, row_cmp, nc, qf, dof, c2, S);
    else bwd_range<D, NKB, QB>(kh, vrh, kth, row_slc, topk * block, qf, dof, c2, S);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float l = S[qb].l[0] + S[qb].l[1];
      float cc = S[qb].c[0] + S[qb].c[1];
      l += __shfl_xor(l, 32, 64);
      cc += __shfl_xor(cc, 32, 64);
      const float linv = __builtin_amdgcn_rcpf(l);
      const float dg = cc * linv;                 // dO . O_i
      const float gi = G[qb][br], dv = gi * dg;
      dG[qb][br] = dg;
      const float fa = gi * linv, fb = dv * linv;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          sdq[w][qb][db][e][lane] += fa * S[qb].a[db][e] - fb * S[qb].bv[db][e];
      if (hf == 0)
        stats[((int64_t)h * 3 + br) * N + t0 + qb * 32 + c] = make_float4(S[qb].m, linv, gi, dv);
    }
  }

  // dq = dQ / sqrt(d) + sum_i dz_i W[i]
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float dz[3] = {0.f, 0.f, 0.f};
    if (gate_w) {
#pragma unroll
      for (int i = 0; i < 3; ++i) dz[i] = dG[qb][i] * G[qb][i] * (1.0f - G[qb][i]);
    }
    uint16_t* orow = dq + pq[qb] * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dd = db * 32 + gq * 8 + hf * 4 + e;
          x[e] = sdq[w][qb][db][gq * 4 + e][lane] * scale;
          if (gate_w)
            x[e] = fmaf(dz[0], gate_w[dd],
                        fmaf(dz[1], gate_w[D + dd], fmaf(dz[2], gate_w[2 * D + dd], x[e])));
        }
        u32x2 pk;
        pk[0] = pack_bf16x2(x[0], x[1]);
        pk[1] = pack_bf16x2(x[2], x[3]);
        *(u32x2*)(orow + db * 32 + gq * 8 + hf * 4) = pk;
      }

    // gate parameters: this block's sums of dz_i q[d] and dz_i over its 32
    // queries, output-major ([3*(d+1)][blocks]) so the final sums read
    // contiguous memory
    if (gate_w && gpart) {
      const int64_t nblk = (int64_t)H * (N / 32);
      const int64_t wv = (int64_t)h * (N / 32) + (t0 / 32) + qb;
#pragma unroll
      for (int i = 0; i < 3; ++i) {
#pragma unroll
        for (int s = 0; s < DS; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x = dz[i] * (float)qf[qb * DS + s][e];
#pragma unroll
            for (int m = 1; m < 32; m <<= 1) x += __shfl_xor(x, m, 64);
            if (c == 0) gpart[(int64_t)(i * (D + 1) + s * 16 + hf * 8 + e) * nblk + wv] = x;
          }
        float y = dz[i];
#pragma unroll
        for (int m = 1; m < 32; m <<= 1) y += __shfl_xor(y, m, 64);
        if (lane == 0) gpart[(int64_t)(i * (D + 1) + D) * nblk + wv] = y;
      }
    }
  }
}

// ------------------------------------------------------------ key pass ----
// One wave per NKB blocks of 32 keys (rows r0 .. r0 + 32*NKB - 1 of the key
// source, row-major): over the query blocks given by qblock(i) (tree
// position of the block's first query) for i < nqb, accumulate dK^T and dV^T
// of branch BR into acc[kb][0..DB) (dK^T, scaled) and acc[kb][DB..2DB)
// (dV^T).  A query block's Q and dO rows (one contiguous run each in the
// tree-ordered copies qr, dor) are staged in the wave's LDS tiles tq, td
// (td is followed by the block's 32 statistics): row reads give the A
// operands of S = Q K^T and dP = dO V^T, transposed reads the Q^T and dO^T
// operands.  The next block's rows and statistics are fetched into
// registers while the current one is computed.  The tiles are private to the wave, whose
// LDS accesses complete in program order, so wave barriers (which only keep
// the compiler from moving accesses across them) suffice.
template <int D, int BR, int NKB, typename QFn>
BT_DEV void kv_sweep(const uint16_t* __restrict__ qr, const uint16_t* __restrict__ dor,
                     const float4* __restrict__ stats, const uint16_t* __restrict__ krow,
                     const uint16_t* __restrict__ vrow, int64_t N, int h, int nqb, QFn qblock,
                     uint16_t* tq, uint16_t* td, f32x16 (*acc)[2 * (D / 32)]) {
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  bf16x8 kB[NKB][DS], vB[NKB][DS];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      kB[kb][s] = *(const bf16x8*)(krow + (kb * 32 + c) * D + hf * 8 + s * 16);
      vB[kb][s] = *(const bf16x8*)(vrow + (kb * 32 + c) * D + hf * 8 + s * 16);
    }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) acc[kb][i] = f32x16{};
  const float4* sh = stats + ((int64_t)h * 3 + BR) * N;
  const uint16_t* qh = qr + (int64_t)h * N * D;
  const uint16_t* dh = dor + (int64_t)h * N * D;
  // the next block's rows and statistics are fetched into registers while
  // the current one is computed, then put into the wave's LDS tiles
  constexpr int PPL = 32 * CPR / 64;            // 16-byte pieces per lane and tensor
  float4* sst = (float4*)(td + 32 * D);          // statistics of the block's 32 queries
  u32x4 fq[PPL], fd[PPL];
  float4 fs = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fetch = [&](int64_t q0) {
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int it = lane + u * 64, r = it / CPR, p = it - r * CPR;
      fq[u] = *(const u32x4*)(qh + (q0 + r) * D + p * 8);
      fd[u] = *(const u32x4*)(dh + (q0 + r) * D + p * 8);
    }
    if (lane < 32) fs = sh[q0 + lane];
  };
  if (nqb > 0) fetch(qblock(0));
  for (int i = 0; i < nqb; ++i) {
    __builtin_amdgcn_wave_barrier();   // the wave's reads of the last block came first
#pragma unroll
    for (int u = 0; u < PPL; ++u) {
      const int it = lane + u * 64, r = it / CPR, p = it - r * CPR;
      const int t = tile_off<D>(r, p);
      *(u32x4*)&tq[t] = fq[u];
      *(u32x4*)&td[t] = fd[u];
    }
    if (lane < 32) sst[lane] = fs;
    __builtin_amdgcn_wave_barrier();
    if (i + 1 < nqb) fetch(qblock(i + 1));
    bf16x8 qA[DS], dA[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qA[s] = *(const bf16x8*)&tq[tile_off<D>(c, s * 2 + hf)];
      dA[s] = *(const bf16x8*)&td[tile_off<D>(c, s * 2 + hf)];
    }
    f32x16 sa[NKB], pa[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sa[kb] = f32x16{};
      pa[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qA[s], kB[kb][s], sa[kb], 0, 0, 0);
        pa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dA[s], vB[kb][s], pa[kb], 0, 0, 0);
      }
    }
    // element e holds query 8*(e/4) + 4*hf + e%4 of the block
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 gpf[NKB], dsf[NKB];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ee = s2 * 8 + e;
        const float4 st = sst[8 * (ee / 4) + 4 * hf + (ee % 4)];   // (m, 1/l, G, D)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sa[kb][ee], c2, -st.x)) * st.y;
          gpf[kb][e] = (__bf16)(st.z * p);
          dsf[kb][e] = (__bf16)(p * fmaf(st.z, pa[kb][ee], -st.w));
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 qT = tr_operand<D>(tq, s2, db);
        const bf16x8 dT = tr_operand<D>(td, s2, db);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          acc[kb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qT, dsf[kb], acc[kb][db], 0, 0, 0);
          acc[kb][DB + db] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(dT, gpf[kb], acc[kb][DB + db], 0, 0, 0);
        }
      }
    }
  }
  const float scale = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[kb][db] *= scale;
}

// Writes (ADD = false) or adds a wave's dK^T / dV^T (acc as kv_sweep leaves
// it) into [.][rows][D] fp32 at rows r0 .. r0 + 32*NKB - 1.
template <int D, int NKB, bool ADD>
BT_DEV void kv_store(f32x16 (*acc)[2 * (D / 32)], int64_t r0, float* __restrict__ dk,
                     float* __restrict__ dv) {
  constexpr int DB = D / 32;
  const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float* base = (x == 0 ? dk : dv) + (r0 + kb * 32 + c) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float4* p = (float4*)(base + db * 32 + gq * 8 + hf * 4);
          const f32x16& a = acc[kb][x * DB + db];
          float4 v = make_float4(a[gq * 4 + 0], a[gq * 4 + 1], a[gq * 4 + 2], a[gq * 4 + 3]);
          if (ADD) {
            const float4 o = *p;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *p = v;
        }
    }
}

// Key blocks per wave of the key passes: two at d = 32 (their loads of a
// query block are shared), one at d = 64 (register budget).
template <int D>
constexpr int kv_nkb() { return D == 32 ? 2 : 1; }

// Ball branch: grid (balls, H), ball/(32*NKB) waves; wave w owns keys
// w*32*NKB.. of the ball and visits the ball's query blocks.
template <int D, int NKB>
__global__ __launch_bounds__(512) void bsa_bwd_kv_ball(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ dor,
    const float4* __restrict__ stats, const uint16_t* __restrict__ kt,
    const uint16_t* __restrict__ vr, int64_t N, int32_t ball, float* __restrict__ dkacc,
    float* __restrict__ dvacc) {
  constexpr int DB = D / 32;
  const int w = threadIdx.x >> 6, h = blockIdx.y;
  const int64_t b0 = (int64_t)blockIdx.x * ball;
  const int64_t r0 = b0 + w * 32 * NKB;
  f32x16 acc[NKB][2 * DB];
  HIP_DYNAMIC_SHARED(uint16_t, tiles)
  uint16_t* tq = tiles + (size_t)w * (2 * 32 * D + 256);
  kv_sweep<D, 0, NKB>(qr, dor, stats, kt + ((int64_t)h * N + r0) * D,
                      vr + ((int64_t)h * N + r0) * D, N, h, ball / 32,
                      [&](int i) -> int64_t { return b0 + i * 32; }, tq, tq + 32 * D, acc);
  kv_store<D, NKB, false>(acc, r0, dkacc + (int64_t)h * N * D, dvacc + (int64_t)h * N * D);
}

// Selection branch: grid (blocks, H), block/(32*NKB) waves; wave w owns keys
// w*32*NKB.. of block j and visits the query blocks of every group that
// selected j.
template <int D, int NKB>
__global__ __launch_bounds__(512) void bsa_bwd_kv_slc(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ dor,
    const float4* __restrict__ stats, const uint16_t* __restrict__ kt,
    const uint16_t* __restrict__ vr, const uint32_t* __restrict__ off,
    const int32_t* __restrict__ list, int64_t N, int32_t nc, int32_t ngroups, int32_t group,
    int32_t block, int32_t topk, float* __restrict__ dkacc, float* __restrict__ dvacc) {
  constexpr int DB = D / 32;
  const int w = threadIdx.x >> 6, h = blockIdx.y;
  const int64_t j = blockIdx.x;
  const int64_t r0 = j * block + w * 32 * NKB;
  const int64_t cap = (int64_t)ngroups * topk;
  const uint32_t* oh = off + (int64_t)h * (nc + 1);
  const int64_t e0 = min((int64_t)oh[j], cap), e1 = min((int64_t)oh[j + 1], cap);
  const int32_t* lh = list + (int64_t)h * cap;
  const int per = group / 32;
  const int nqb = e1 > e0 ? (int)(e1 - e0) * per : 0;
  f32x16 acc[NKB][2 * DB];
  HIP_DYNAMIC_SHARED(uint16_t, tiles)
  uint16_t* tq = tiles + (size_t)w * (2 * 32 * D + 256);
  kv_sweep<D, 2, NKB>(qr, dor, stats, kt + ((int64_t)h * N + r0) * D,
                      vr + ((int64_t)h * N + r0) * D, N, h, nqb,
                      [&](int i) -> int64_t {
                        const int e = i / per, qb = i - e * per;
                        const int64_t gg = perm_index(lh[e0 + e], ngroups);
                        return gg * group + qb * 32;
                      },
                      tq, tq + 32 * D, acc);
  kv_store<D, NKB, true>(acc, r0, dkacc + (int64_t)h * N * D, dvacc + (int64_t)h * N * D);
}

// Compression branch: grid (nc/(32*NKB), H, kCmpParts/4), 4 waves; wave w
// takes query partition z*4 + w of all N/32 query blocks for the coarse
// tokens jb*32*NKB.. and writes its partial dKc / dVc.
// (two waves per SIMD at d = 32: 7 registers spill, and it still beats one wave)
template <int D, int NKB>
__global__ __launch_bounds__(256) BT_WAVES_PER_EU(D == 32 ? 2 : 1, 8) void bsa_bwd_kv_cmp(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ dor,
    const float4* __restrict__ stats, const uint16_t* __restrict__ kcb,
    const uint16_t* __restrict__ vcr, int32_t H, int64_t N, int32_t nc,
    float* __restrict__ cpart) {
  constexpr int DB = D / 32;
  const int w = threadIdx.x >> 6, h = blockIdx.y;
  const int part = blockIdx.z * 4 + w;
  const int64_t r0 = (int64_t)blockIdx.x * 32 * NKB;
  const int64_t nqb = N / 32;
  const int64_t i0 = nqb * part / kCmpParts, i1 = nqb * (part + 1) / kCmpParts;
  f32x16 acc[NKB][2 * DB];
  HIP_DYNAMIC_SHARED(uint16_t, tiles)
  uint16_t* tq = tiles + (size_t)w * (2 * 32 * D + 256);
  kv_sweep<D, 1, NKB>(qr, dor, stats, kcb + ((int64_t)h * nc + r0) * D,
                      vcr + ((int64_t)h * nc + r0) * D, N, h, (int)(i1 - i0),
                      [&](int i) -> int64_t { return (i0 + i) * 32; }, tq, tq + 32 * D, acc);
  float* pk = cpart + (((int64_t)part * 2 + 0) * H + h) * nc * D;
  float* pv = cpart + (((int64_t)part * 2 + 1) * H + h) * nc * D;
  kv_store<D, NKB, false>(acc, r0, pk, pv);
}

// dKc, dVc [h][j][d] = the sum of the partitions' partials, in order.
__global__ __launch_bounds__(256) void bsa_bwd_cmp_reduce(const float* __restrict__ cpart,
                                                          int64_t per, float* __restrict__ dkc,
                                                          float* __restrict__ dvc) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < per;
       i += (int64_t)gridDim.x * blockDim.x) {
    float sk = 0.f, sv = 0.f;
    for (int p = 0; p < kCmpParts; ++p) {
      sk += cpart[((int64_t)p * 2 + 0) * per + i];
      sv += cpart[((int64_t)p * 2 + 1) * per + i];
    }
    dkc[i] = sk;
    dvc[i] = sv;
  }
}

// dk[perm[t]][h] = bf16(dK_ball + dK_slc + dKc[h][t / block] / block), dv
// likewise; one thread per 8 elements of a row.
template <int D>
__global__ __launch_bounds__(256) void bsa_bwd_finish(const float* __restrict__ dkacc,
                                                      const float* __restrict__ dvacc,
                                                      const float* __restrict__ dkc,
                                                      const float* __restrict__ dvc,
                                                      const int32_t* __restrict__ perm,
                                                      int32_t H, int64_t N, int32_t nc,
                                                      int32_t block, uint16_t* __restrict__ dk,
                                                      uint16_t* __restrict__ dv) {
  constexpr int P8 = D / 8;
  const int64_t total = N * H * P8;
  const float inv = 1.0f / (float)block;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int pc = (int)(i % P8);
    const int64_t th = i / P8;
    const int h = (int)(th % H);
    const int64_t t = th / H;
    const int64_t src = ((int64_t)h * N + t) * D + pc * 8;
    const int64_t csrc = ((int64_t)h * nc + t / block) * D + pc * 8;
    const int64_t dst = perm_index(perm[t], N) * H * D + (int64_t)h * D + pc * 8;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const float* a = (x == 0 ? dkacc : dvacc) + src;
      const float* cc = (x == 0 ? dkc : dvc) + csrc;
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf16x2(fmaf(cc[2 * e], inv, a[2 * e]), fmaf(cc[2 * e + 1], inv, a[2 * e + 1]));
      *(u32x4*)((x == 0 ? dk : dv) + dst) = o;
    }
  }
}

// Grid (3 * (D + 1)), 256 threads: output o of (dW [3][D], db [3]) summed over
// the per-block partials (gpart[o][block], contiguous) in a fixed order.
__global__ __launch_bounds__(256) void bsa_bwd_gate_reduce(const float* __restrict__ gpart,
                                                           int64_t nblk, int32_t d,
                                                           float* __restrict__ dgw,
                                                           float* __restrict__ dgb) {
  __shared__ float red[256];
  const int o = blockIdx.x, tid = threadIdx.x;
  const float* src = gpart + (int64_t)o * nblk;
  float s = 0.f;
  for (int64_t i = tid; i < nblk; i += 256) s += src[i];
  red[tid] = s;
  __syncthreads();
  for (int m = 128; m > 0; m >>= 1) {
    if (tid < m) red[tid] += red[tid + m];
    __syncthreads();
  }
  if (tid == 0) {
    const int i = o / (d + 1), e = o - i * (d + 1);
    if (e < d) {
      if (dgw) dgw[i * d + e] = red[0];
    } else if (dgb) {
      dgb[i] = red[0];
    }
  }
}

// ------------------------------------------------------------------ host ----
template <int D>
static bt_status bwd_launch_d(const void* q, const void* k, const void* v, const void* dout,
                              const int32_t* perm, int64_t N,
                              int32_t H, const bsa_params* p, const float* gate_w,
                              const float* gate_b, const float* gate_const, void* dq, void* dk,
                              void* dv, float* dgate_w, float* dgate_b, const BsaBwdLayout& L,
                              char* b, const int32_t* sel, hipStream_t st) {
  const int32_t nc = (int32_t)(N / p->block), ngroups = (int32_t)(N / p->group);
  const int nchunk = (ngroups + kIdxChunk - 1) / kIdxChunk;
  const uint16_t* kt = (const uint16_t*)(b + L.f.kt);
  const uint16_t* kcb = (const uint16_t*)(b + L.f.kcb);
  const uint16_t* vct = (const uint16_t*)(b + L.f.vcb);
  uint16_t* vr = (uint16_t*)(b + L.vr);
  uint16_t* qr = (uint16_t*)(b + L.qr);
  uint16_t* dor = (uint16_t*)(b + L.dor);
  uint16_t* ktt = (uint16_t*)(b + L.ktt);
  uint16_t* vcr = (uint16_t*)(b + L.vcr);
  uint16_t* kctt = (uint16_t*)(b + L.kctt);
  float4* stats = (float4*)(b + L.stats);
  float* dkacc = (float*)(b + L.dkacc);
  float* dvacc = (float*)(b + L.dvacc);
  float* cpart = (float*)(b + L.cpart);
  float* dkc = (float*)(b + L.dkc);
  float* dvc = (float*)(b + L.dvc);
  float* gpart = (float*)(b + L.gpart);
  uint32_t* cntc = (uint32_t*)(b + L.cntc);
  uint32_t* basec = (uint32_t*)(b + L.basec);
  uint32_t* off = (uint32_t*)(b + L.off);
  int32_t* list = (int32_t*)(b + L.list);
  const uint16_t* kin = (const uint16_t*)k;
  const uint16_t* vin = (const uint16_t*)v;

  const dim3 w1(64);
  hipLaunchKernelGGL((bsa_bwd_prep<D>), dim3((unsigned)(N / 32), H), w1, 0, st,
                     (const uint16_t*)q, kin, vin, (const uint16_t*)dout, perm, H, N, vr, qr, dor,
                     ktt);
  hipLaunchKernelGGL((bsa_bwd_prep_coarse<D>), dim3(nc / 32, H), w1, 0, st, kcb, vct, nc, vcr,
                     kctt);
  const size_t idx_lds = (size_t)nc * 4;
  hipLaunchKernelGGL(bsa_bwd_sel_count, dim3(nchunk, H), w1, idx_lds, st, sel, nc, ngroups,
                     p->topk, cntc);
  hipLaunchKernelGGL(bsa_bwd_sel_scan, dim3(H), dim3(1024), 0, st, cntc, nc, nchunk, basec, off);
  hipLaunchKernelGGL(bsa_bwd_sel_fill, dim3(nchunk, H), w1, idx_lds, st, sel, basec, nc, ngroups,
                     p->topk, list);
  bt_status s = launch_status("bsa_bwd prepare");
  if (s != BT_OK) return s;

  const float g0 = gate_const ? gate_const[0] : 0.f, g1 = gate_const ? gate_const[1] : 0.f,
              g2 = gate_const ? gate_const[2] : 0.f;
  const int total = ngroups * H;
  const int xmap = (total % 8 == 0) ? 1 : 0;
  float* gp = (gate_w && (dgate_w || dgate_b)) ? gpart : nullptr;
#define BT_BWDQ(NW, QBB)                                                                       \
  hipLaunchKernelGGL((bsa_bwd_q<D, NW, QBB, QNKB>), dim3(total), dim3(NW * 64), 0, st,                \
                     (const uint16_t*)q, (const uint16_t*)dout, perm, kt, vr, ktt, kcb, vcr,    \
                     kctt, sel, gate_w, gate_b, g0, g1, g2, H, N, nc, ngroups, p->ball,     \
                     p->block, p->topk, xmap, stats, gp, (uint16_t*)dq)
  constexpr int QNKB = 1;   // 64-key chunks measured no faster
  // two query blocks per wave at d = 32 (their key fragments are shared)
  if constexpr (D == 32) {
    switch (p->group) {
      case 32: BT_BWDQ(1, 1); break;
      case 64: BT_BWDQ(1, 2); break;
      case 128: BT_BWDQ(2, 2); break;
      default: BT_BWDQ(4, 2); break;
    }
  } else {
    switch (p->group) {
      case 32: BT_BWDQ(1, 1); break;
      case 64: BT_BWDQ(2, 1); break;
      case 128: BT_BWDQ(4, 1); break;
      default: BT_BWDQ(8, 1); break;
    }
  }
#undef BT_BWDQ
  s = launch_status("bsa_bwd_q");
  if (s != BT_OK) return s;

  // two key blocks per wave where the block sizes allow it
  constexpr int NK = kv_nkb<D>();
  const bool ball2 = NK == 2 && p->ball % 64 == 0, blk2 = NK == 2 && p->block % 64 == 0,
             cmp2 = NK == 2 && nc % 64 == 0;
  // each wave stages a query block's Q and dO rows in two tiles of its own,
  // followed by the block's statistics
  const size_t tl_bytes = (size_t)2 * 32 * D * sizeof(uint16_t) + 32 * sizeof(float4);
#define BT_KVB(K)                                                                             \
  hipLaunchKernelGGL((bsa_bwd_kv_ball<D, K>), dim3((unsigned)(N / p->ball), H),               \
                     dim3(p->ball / (32 * K) * 64), p->ball / (32 * K) * tl_bytes, st, qr, dor, \
                     stats, kt, vr, N, p->ball, dkacc, dvacc)
#define BT_KVS(K)                                                                             \
  hipLaunchKernelGGL((bsa_bwd_kv_slc<D, K>), dim3(nc, H), dim3(p->block / (32 * K) * 64),     \
                     p->block / (32 * K) * tl_bytes, st, qr, dor, stats, kt, vr, off, list, N, nc, \
                     ngroups, p->group, p->block, p->topk, dkacc, dvacc)
#define BT_KVC(K)                                                                             \
  hipLaunchKernelGGL((bsa_bwd_kv_cmp<D, K>), dim3(nc / (32 * K), H, kCmpParts / 4), dim3(256), \
                     4 * tl_bytes, st, qr, dor, stats, kcb, vcr, H, N, nc, cpart)
  if (ball2) BT_KVB(NK); else BT_KVB(1);
  if (blk2) BT_KVS(NK); else BT_KVS(1);
  if (cmp2) BT_KVC(NK); else BT_KVC(1);
#undef BT_KVB
#undef BT_KVS
#undef BT_KVC
  s = launch_status("bsa_bwd keys");
  if (s != BT_OK) return s;

  const int64_t per = (int64_t)H * nc * D;
  const int64_t gr = (per + 255) / 256 < 2048 ? (per + 255) / 256 : 2048;
  hipLaunchKernelGGL(bsa_bwd_cmp_reduce, dim3((unsigned)gr), dim3(256), 0, st, cpart, per, dkc,
                     dvc);
  const int64_t fin = N * H * (D / 8);
  const int64_t gf = (fin + 255) / 256 < 8192 ? (fin + 255) / 256 : 8192;
  hipLaunchKernelGGL((bsa_bwd_finish<D>), dim3((unsigned)gf), dim3(256), 0, st, dkacc, dvacc, dkc,
                     dvc, perm, H, N, nc, p->block, (uint16_t*)dk, (uint16_t*)dv);
  if (gp)
    hipLaunchKernelGGL(bsa_bwd_gate_reduce, dim3(3 * (D + 1)), dim3(256), 0, st, gp,
                       (int64_t)H * (N / 32), D, dgate_w, dgate_b);
  return launch_status("bsa_bwd finish");
}

bt_status bsa_bwd_launch(const void* q, const void* k, const void* v, const int32_t* perm,
                         const void* dout, int64_t N, int32_t H, int32_t d, const bsa_params* p,
                         const float* gate_w, const float* gate_b, const float* gate_const,
                         void* dq, void* dk, void* dv, float* dgate_w, float* dgate_b, void* ws,
                         hipStream_t st) {
  const BsaBwdLayout L = bsa_bwd_layout(N, H, d, p);
  char* b = (char*)ws;
  int32_t* sel = (int32_t*)(b + L.f.sel);
  bt_status s = bsa_prepare(q, k, v, perm, N, H, d, p, ws, sel, st);
  if (s != BT_OK) return s;
  if (d == 32)
    return bwd_launch_d<32>(q, k, v, dout, perm, N, H, p, gate_w, gate_b, gate_const, dq, dk, dv,
                            dgate_w, dgate_b, L, b, sel, st);
  return bwd_launch_d<64>(q, k, v, dout, perm, N, H, p, gate_w, gate_b, gate_const, dq, dk, dv,
                          dgate_w, dgate_b, L, b, sel, st);
}

}  // namespace bt
