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
#include "common.h"

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

bt_status ball_attn_bwd_launch(const void* q, const void* k, const void* v, const void* dout,
                               const int32_t* perm, int64_t N, int32_t ball, int32_t H,
                               int32_t d, bt_dtype dt, void* dq, void* dk, void* dv,
                               hipStream_t st) {
  const dim3 grid((unsigned)((N / ball) * H)), blk(kBwdThreads);
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
