// Backward pass of ball attention.  The branches of BSA and Erwin's layers
// are learned (Pith review of arXiv 2506.12541, "What carries the argument";
// Erwin thread on Bluesky, post 7/N), so training needs dQ, dK, dV.  Per ball
// b and head h, with S = Q K^T / sqrt(d), P = softmax(S), O = P V and the
// incoming gradient dO (all rows gathered through perm):
//     D_i = dO_i . O_i,  dS = P * (dO V^T - D),
//     dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d),  dV = P^T dO,
// scattered back to original order.
//
// ball_attn_bwd_valu<T, D>: fp32 arithmetic for every dtype, one workgroup per
// (ball, head), 256 threads.
//   query pass (thread per query): one sweep over the keys recomputes the
//     forward online softmax -- row maximum m_i, sum l_i and O_i -- so D_i
//     needs no stored forward output; a second sweep accumulates dQ_i.  m, l
//     and D of every query of the ball stay in LDS.
//   key pass (thread per key): a sweep over the queries (staged in LDS with
//     their dO rows) accumulates dK_j and dV_j.
// Rows are staged through LDS in chunks of 64 as fp32.
#include "lds_tile.h"

namespace bt {

template <typename T>
BT_DEV float ld(const T* p);
template <>
BT_DEV float ld<float>(const float* p) { return *p; }
template <>
BT_DEV float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
BT_DEV void st(T* p, float x);
template <>
BT_DEV void st<float>(float* p, float x) { *p = x; }
template <>
BT_DEV void st<uint16_t>(uint16_t* p, float x) {
  const __bf16 b = (__bf16)x;
  *p = __builtin_bit_cast(uint16_t, b);
}

constexpr int kBwdThreads = 256;
constexpr int kBwdChunk = 64;
constexpr int kBwdMaxBall = 1024;

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads) void ball_attn_bwd_valu(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const int32_t* __restrict__ perm, int64_t N, int32_t H,
    int32_t ball, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float sa[kBwdChunk][D + 1];
  __shared__ float sb[kBwdChunk][D + 1];
  __shared__ float sm[kBwdMaxBall], sl[kBwdMaxBall], sd[kBwdMaxBall];
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int64_t base = (int64_t)b * ball;
  const int64_t rs = (int64_t)H * D;
  const float scale = 1.0f / sqrtf((float)D);
  const int tid = threadIdx.x;
  auto row = [&](int i) -> int64_t { return perm ? perm_index(perm[base + i], N) : base + i; };
  // stage rows r0 .. r0+n-1 of x and y (head h) into sa, sb
  auto stage = [&](const T* x, const T* y, int r0, int n) {
    __syncthreads();
    for (int i = tid; i < n * D; i += kBwdThreads) {
      const int j = i / D, e = i - j * D;
      const int64_t pr = row(r0 + j) * rs + h * D + e;
      sa[j][e] = ld<T>(x + pr);
      sb[j][e] = ld<T>(y + pr);
    }
    __syncthreads();
  };

  // ---- query pass ---------------------------------------------------------
  for (int q0 = 0; q0 < ball; q0 += kBwdThreads) {
    const int qi = q0 + tid;
    const bool active = qi < ball;
    float qv[D], dov[D], acc[D];
    float m = -INFINITY, l = 0.f;
    int64_t pq = 0;
    if (active) {
      pq = row(qi);
#pragma unroll
      for (int e = 0; e < D; ++e) {
        qv[e] = ld<T>(q + pq * rs + h * D + e);
        dov[e] = ld<T>(dout + pq * rs + h * D + e);
      }
    }
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = 0.f;
    // sweep 1: forward online softmax -> m, l, O
    for (int c0 = 0; c0 < ball; c0 += kBwdChunk) {
      const int nk = min(kBwdChunk, ball - c0);
      stage(k, v, c0, nk);
      if (!active) continue;
      for (int j = 0; j < nk; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = fmaf(qv[e], sa[j][e], s);
        s *= scale;
        const float mn = fmaxf(m, s);
        const float corr = expf(m - mn);        // 0 on the first key
        const float p = expf(s - mn);
        l = l * corr + p;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = fmaf(p, sb[j][e], acc[e] * corr);
        m = mn;
      }
    }
    float dd = 0.f;
    if (active) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int e = 0; e < D; ++e) dd = fmaf(dov[e], acc[e] * inv, dd);
      sm[qi] = m;
      sl[qi] = l;
      sd[qi] = dd;
    }
    // sweep 2: dQ_i = scale * sum_j P_ij (dO_i . V_j - D_i) K_j
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = 0.f;
    for (int c0 = 0; c0 < ball; c0 += kBwdChunk) {
      const int nk = min(kBwdChunk, ball - c0);
      stage(k, v, c0, nk);
      if (!active) continue;
      const float inv = 1.0f / l;
      for (int j = 0; j < nk; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          s = fmaf(qv[e], sa[j][e], s);
          dp = fmaf(dov[e], sb[j][e], dp);
        }
        const float p = expf(s * scale - m) * inv;
        const float ds = p * (dp - dd);
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, sa[j][e], acc[e]);
      }
    }
    if (active)
#pragma unroll
      for (int e = 0; e < D; ++e) st<T>(dq + pq * rs + h * D + e, acc[e] * scale);
  }
  __syncthreads();   // m, l, D of every query are in LDS

  // ---- key pass -------------------------------------------------------------
  for (int k0 = 0; k0 < ball; k0 += kBwdThreads) {
    const int kj = k0 + tid;
    const bool active = kj < ball;
    float kv[D], vv[D], gk[D], gv[D];
    int64_t pk = 0;
    if (active) {
      pk = row(kj);
#pragma unroll
      for (int e = 0; e < D; ++e) {
        kv[e] = ld<T>(k + pk * rs + h * D + e);
        vv[e] = ld<T>(v + pk * rs + h * D + e);
      }
    }
#pragma unroll
    for (int e = 0; e < D; ++e) { gk[e] = 0.f; gv[e] = 0.f; }
    for (int c0 = 0; c0 < ball; c0 += kBwdChunk) {
      const int nq = min(kBwdChunk, ball - c0);
      stage(q, dout, c0, nq);              // sa = Q rows, sb = dO rows
      if (!active) continue;
      for (int i = 0; i < nq; ++i) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          s = fmaf(sa[i][e], kv[e], s);
          dp = fmaf(sb[i][e], vv[e], dp);
        }
        const int qi = c0 + i;
        const float p = expf(s * scale - sm[qi]) / sl[qi];
        const float ds = p * (dp - sd[qi]);
#pragma unroll
        for (int e = 0; e < D; ++e) {
          gv[e] = fmaf(p, sb[i][e], gv[e]);
          gk[e] = fmaf(ds, sa[i][e], gk[e]);
        }
      }
    }
    if (active)
#pragma unroll
      for (int e = 0; e < D; ++e) {
        st<T>(dk + pk * rs + h * D + e, gk[e] * scale);
        st<T>(dv + pk * rs + h * D + e, gv[e]);
      }
  }
}

// --------------------------------------------------------------------------
// bf16 MFMA kernel (v_mfma_f32_32x32x16_bf16; operand layouts as in the
// forward kernel: A[i][kk] lane i + 32*(kk/8) element kk%8, B[kk][j] lane
// j + 32*(kk/8) element kk%8, C[i][j] lane j + 32*((i/4)%2) element
// (i/8)*4 + i%4).  One workgroup per (ball, head), one wave per 32 rows.
// Q, K, V and dO of the ball are staged once into LDS as row-major tiles
// without padding; the 16-byte pieces of a row are permuted by a function of
// the row (tile_off) so that both access patterns below are free of bank
// conflicts:
//  * row reads (ds_read_b128): a lane reads 8 consecutive d of one row, the
//    A operand of S^T = K Q^T and similar products;
//  * transposed reads (ds_read_b64_tr_b16, gfx950): in each 16-lane group,
//    lane l receives element l%4 of the 8-byte runs addressed by lanes l/4,
//    l/4+4, l/4+8, l/4+12, so four rows x 16 d become 4 keys for each of 16
//    d: the K^T, Q^T and dO^T operands, read from the same tiles.
// Key positions inside a 16-key slice follow the order in which a C tile
// feeds a B operand (bits 2 and 3 of the position swapped), and the
// transposed reads fetch rows in that order.
//  query pass (lane = query column): a first sweep over the key blocks forms
//    the row maximum, the normaliser and D_i = sum_j P_ij dP_ij with
//    dP^T = V dO^T (equal to dO_i . O_i, so O is not needed) by an online
//    rescaling; a second sweep recomputes S^T and dP^T per block, forms
//    dS^T = P^T (dP^T - D) and accumulates dQ^T += K^T dS^T.  The statistics
//    go to LDS.
//  key pass (lane = key column): per 32-query block S = Q K^T, P from the
//    stored statistics, dP = dO V^T, dS = P (dP - D); dV^T += dO^T P and
//    dK^T += Q^T dS.
// P and dS are rounded to bf16 for the MFMA; everything else is fp32.

// lane (c, hf) holds C^T[d][c] of a 32-column block for d = db*32 + 8*g +
// 4*hf + 0..3 in acc[db][g*4 + 0..3]; write row `row` (d contiguous) scaled,
// as 16-byte runs after one exchange with lane c^32.
template <int D>
BT_DEV void store_cols(const f32x16* acc, float f, uint16_t* __restrict__ row) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    u32x2 pg[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      pg[g][0] = pack_bf16x2(acc[db][g * 4 + 0] * f, acc[db][g * 4 + 1] * f);
      pg[g][1] = pack_bf16x2(acc[db][g * 4 + 2] * f, acc[db][g * 4 + 3] * f);
    }
    const u32x2 sa = hf ? pg[0] : pg[1], sb = hf ? pg[2] : pg[3];
    u32x2 ra, rb;
    ra[0] = (uint32_t)__shfl_xor((int)sa[0], 32, 64);
    ra[1] = (uint32_t)__shfl_xor((int)sa[1], 32, 64);
    rb[0] = (uint32_t)__shfl_xor((int)sb[0], 32, 64);
    rb[1] = (uint32_t)__shfl_xor((int)sb[1], 32, 64);
    u32x4 c0, c1;
    if (hf == 0) {
      c0 = u32x4{pg[0][0], pg[0][1], ra[0], ra[1]};
      c1 = u32x4{pg[2][0], pg[2][1], rb[0], rb[1]};
    } else {
      c0 = u32x4{ra[0], ra[1], pg[1][0], pg[1][1]};
      c1 = u32x4{rb[0], rb[1], pg[3][0], pg[3][1]};
    }
    *(u32x4*)(row + db * 32 + hf * 8) = c0;
    *(u32x4*)(row + db * 32 + 16 + hf * 8) = c1;
  }
}

template <int D, int BALL>
__global__ __launch_bounds__(BALL / 32 * 64) void ball_attn_bwd_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const int32_t* __restrict__ perm, int64_t N, int32_t H, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv) {
  constexpr int NT = BALL / 32 * 64, KB = BALL / 32, DS = D / 16, DB = D / 32, CPR = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t ql[BALL * D], kl[BALL * D], vl[BALL * D],
      dl[BALL * D];
  __shared__ __attribute__((aligned(16))) float smc[BALL], sli[BALL], sdd[BALL];
  // Workgroups go round-robin to the 8 XCDs (the grid is a multiple of 8 when
  // the item count is): XCD x runs items x*total/8 ... in order, so the heads
  // of one ball, which share the 128-byte lines of its rows, are fetched
  // through the same L2 at about the same time.
  const int total = (int)gridDim.x;
  const int item = (total & 7) ? (int)blockIdx.x
                               : ((int)blockIdx.x & 7) * (total >> 3) + ((int)blockIdx.x >> 3);
  const int b = item / H, h = item - (item / H) * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, c = lane & 31;
  const int64_t base = (int64_t)b * BALL, rs = (int64_t)H * D;
  auto row_of = [&](int i) -> int64_t { return perm ? perm_index(perm[base + i], N) : base + i; };

  // ---- stage the ball's rows of Q, K, V, dO ----------------------------------
#pragma unroll
  for (int it = tid; it < BALL * CPR; it += NT) {
    const int r = it / CPR, p = it - r * CPR;
    const int64_t o = row_of(r) * rs + (int64_t)h * D + p * 8;
    const u32x4 a0 = *(const u32x4*)(q + o), a1 = *(const u32x4*)(k + o);
    const u32x4 a2 = *(const u32x4*)(v + o), a3 = *(const u32x4*)(dout + o);
    const int t = tile_off<D>(r, p);
    *(u32x4*)&ql[t] = a0;
    *(u32x4*)&kl[t] = a1;
    *(u32x4*)&vl[t] = a2;
    *(u32x4*)&dl[t] = a3;
  }
  __syncthreads();
  const float c2 = 1.4426950408889634f / sqrtf((float)D);   // log2(e)/sqrt(d)
  const float scale = 1.0f / sqrtf((float)D);

  // ---- query pass: row w*32 + c is this lane's query ---------------------------
  {
    const int qr = w * 32 + c;
    bf16x8 qf[DS], df[DS];
#pragma unroll
    for (int s2 = 0; s2 < DS; ++s2) {
      qf[s2] = *(const bf16x8*)&ql[tile_off<D>(qr, s2 * 2 + hf)];
      df[s2] = *(const bf16x8*)&dl[tile_off<D>(qr, s2 * 2 + hf)];
    }
    // S^T and dP^T of key block kb for this lane's query
    auto blocks = [&](int kb, f32x16& sa, f32x16& pa) {
      sa = f32x16{};
      pa = f32x16{};
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        const int t = tile_off<D>(kb * 32 + c, s2 * 2 + hf);
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&kl[t], qf[s2], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&vl[t], df[s2], pa, 0, 0, 0);
      }
    };
    // sweep 1: maximum (log2 units), normaliser and sum_j p_j dP_j, rescaled
    // as the maximum grows; both lane halves keep the same running maximum
    float m = -INFINITY, l = 0.f, dacc = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 sa, pa;
      blocks(kb, sa, pa);
      float bm = sa[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) bm = fmaxf(bm, sa[e]);
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64)) * c2;
      const float mn = fmaxf(m, bm);
      const float sc = __builtin_amdgcn_exp2f(m - mn);      // 0 on the first block
      l *= sc;
      dacc *= sc;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sa[e], c2, -mn));
        l += p;
        dacc = fmaf(p, pa[e], dacc);
      }
      m = mn;
    }
    l += __shfl_xor(l, 32, 64);
    dacc += __shfl_xor(dacc, 32, 64);
    const float inv = 1.0f / l;
    const float di = dacc * inv;
    if (hf == 0) { smc[qr] = m; sli[qr] = inv; sdd[qr] = di; }
    // sweep 2: dS^T per block, dQ^T += K^T dS^T
    f32x16 gq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) gq[db] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x16 sa, pa;
      blocks(kb, sa, pa);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 sf;                         // dS^T operand
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sa[s2 * 8 + e], c2, -m)) * inv;
          sf[e] = (__bf16)(p * (pa[s2 * 8 + e] - di));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
          gq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(kl, kb * 2 + s2, db), sf,
                                                           gq[db], 0, 0, 0);
      }
    }
    store_cols<D>(gq, scale, dq + row_of(qr) * rs + (int64_t)h * D);
  }
  __syncthreads();   // row statistics of every query in LDS

  // ---- key pass: row w*32 + c is this lane's key -------------------------------
  {
    const int kr = w * 32 + c;
    bf16x8 kf[DS], vf[DS];
#pragma unroll
    for (int s2 = 0; s2 < DS; ++s2) {
      kf[s2] = *(const bf16x8*)&kl[tile_off<D>(kr, s2 * 2 + hf)];
      vf[s2] = *(const bf16x8*)&vl[tile_off<D>(kr, s2 * 2 + hf)];
    }
    f32x16 gk[DB], gv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) { gk[db] = f32x16{}; gv[db] = f32x16{}; }
#pragma unroll
    for (int qb = 0; qb < KB; ++qb) {
      f32x16 sq = {}, dp = {};
#pragma unroll
      for (int s2 = 0; s2 < DS; ++s2) {
        const int t = tile_off<D>(qb * 32 + c, s2 * 2 + hf);
        sq = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&ql[t], kf[s2], sq, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&dl[t], vf[s2], dp, 0, 0, 0);
      }
      // element e is query qb*32 + 8*(e/4) + 4*hf + e%4
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pf, sf;
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
          const int q0 = qb * 32 + 16 * s2 + 8 * g4 + 4 * hf;
          const f32x4 mm = *(const f32x4*)&smc[q0];
          const f32x4 li = *(const f32x4*)&sli[q0];
          const f32x4 dd = *(const f32x4*)&sdd[q0];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ee = s2 * 8 + g4 * 4 + i;
            const float p = __builtin_amdgcn_exp2f(fmaf(sq[ee], c2, -mm[i])) * li[i];
            pf[g4 * 4 + i] = (__bf16)p;
            sf[g4 * 4 + i] = (__bf16)(p * (dp[ee] - dd[i]));
          }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          gv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(dl, qb * 2 + s2, db), pf,
                                                           gv[db], 0, 0, 0);
          gk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(ql, qb * 2 + s2, db), sf,
                                                           gk[db], 0, 0, 0);
        }
      }
    }
    const int64_t orow = row_of(kr) * rs + (int64_t)h * D;
    store_cols<D>(gk, scale, dk + orow);
    store_cols<D>(gv, 1.0f, dv + orow);
  }
}

bool ball_attn_bwd_uses_mfma(bt_dtype dt, int32_t ball, int32_t d) {
  return dt == BT_BF16 && (d == 32 || d == 64) &&
         (ball == 32 || ball == 64 || ball == 128 || ball == 256);
}

bt_status ball_attn_bwd_launch(const void* q, const void* k, const void* v, const void* dout,
                               const int32_t* perm, int64_t N, int32_t ball, int32_t H,
                               int32_t d, bt_dtype dt, void* dq, void* dk, void* dv,
                               hipStream_t st) {
  const dim3 grid((unsigned)((N / ball) * H));
  if (ball_attn_bwd_uses_mfma(dt, ball, d)) {
#define BT_BWDM(DD, BB)                                                                        \
  hipLaunchKernelGGL((ball_attn_bwd_mfma<DD, BB>), grid, dim3(BB / 32 * 64), 0, st,           \
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,              \
                     (const uint16_t*)dout, perm, N, H, (uint16_t*)dq, (uint16_t*)dk,         \
                     (uint16_t*)dv)
    if (d == 32 && ball == 32) BT_BWDM(32, 32);
    else if (d == 32 && ball == 64) BT_BWDM(32, 64);
    else if (d == 32 && ball == 128) BT_BWDM(32, 128);
    else if (d == 32) BT_BWDM(32, 256);
    else if (ball == 32) BT_BWDM(64, 32);
    else if (ball == 64) BT_BWDM(64, 64);
    else if (ball == 128) BT_BWDM(64, 128);
    else BT_BWDM(64, 256);
#undef BT_BWDM
    return launch_status("ball_attn_bwd_mfma");
  }
  const dim3 blk(kBwdThreads);
#define BT_BWD(TT, DD)                                                                         \
  hipLaunchKernelGGL((ball_attn_bwd_valu<TT, DD>), grid, blk, 0, st, (const TT*)q,            \
                     (const TT*)k, (const TT*)v, (const TT*)dout, perm, N, H, ball, (TT*)dq,   \
                     (TT*)dk, (TT*)dv)
  if (dt == BT_F32) {
    if (d == 16) BT_BWD(float, 16);
    else if (d == 32) BT_BWD(float, 32);
    else BT_BWD(float, 64);
  } else {
    if (d == 16) BT_BWD(uint16_t, 16);
    else if (d == 32) BT_BWD(uint16_t, 32);
    else BT_BWD(uint16_t, 64);
  }
#undef BT_BWD
  return launch_status("ball_attn_bwd_valu");
}

}  // namespace bt
