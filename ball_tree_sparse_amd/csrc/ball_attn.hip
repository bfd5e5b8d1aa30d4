// Ball attention: scaled dot-product attention restricted to each ball of the
// tree (Erwin thread on Bluesky, post 7/N; Pith review of arXiv 2506.12541,
// "What carries the argument").  For ball b and head h:
//     O = softmax(Q_b K_b^T / sqrt(d)) V_b,   out[perm[t]] = O[t].
//
// Two kernels:
//  * ball_attn_mfma<D, BALL>: bf16 inputs, one workgroup per (ball, head),
//    one wave per 32-query strip.  S^T = K Q^T and O^T = V^T P^T run on
//    v_mfma_f32_32x32x16_bf16; the softmax is fp32 in registers (each lane
//    owns one query column, so a row reduction is a lane-local loop plus one
//    exchange with lane^32).  K and Q fragments are loaded straight from HBM
//    in the MFMA operand layout; V is staged transposed in LDS.
//  * ball_attn_valu<T, D>: fp32 arithmetic for any ball, one thread per query,
//    K/V chunks of 64 keys staged in LDS, exact online softmax with expf.
#include "common.h"

namespace bt {

// --------------------------------------------------------------------------
// fp32 VALU kernel
// --------------------------------------------------------------------------
template <typename T>
BT_DEV float load_elem(const T* p);
template <>
BT_DEV float load_elem<float>(const float* p) { return *p; }
template <>
BT_DEV float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T>
BT_DEV void store_elem(T* p, float x);
template <>
BT_DEV void store_elem<float>(float* p, float x) { *p = x; }
template <>
BT_DEV void store_elem<uint16_t>(uint16_t* p, float x) {
  __bf16 b = (__bf16)x;
  *p = __builtin_bit_cast(uint16_t, b);
}

constexpr int kValuThreads = 256;
constexpr int kValuChunk = 64;

template <typename T, int D>
__global__ __launch_bounds__(kValuThreads) void ball_attn_valu(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ perm, int64_t N, int32_t H, int32_t ball,
    T* __restrict__ out) {
  __shared__ float ks[kValuChunk][D + 1];
  __shared__ float vs[kValuChunk][D + 1];
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int64_t base = (int64_t)b * ball;
  const int64_t rs = (int64_t)H * D;
  const float scale = 1.0f / sqrtf((float)D);
  const int nthr = blockDim.x;

  for (int q0 = 0; q0 < ball; q0 += nthr) {
    const int qi = q0 + threadIdx.x;
    const bool active = qi < ball;
    int64_t pq = 0;
    float qv[D], acc[D];
    float m = -INFINITY, l = 0.f;
    if (active) {
      pq = perm ? perm_index(perm[base + qi], N) : base + qi;
#pragma unroll
      for (int e = 0; e < D; ++e) qv[e] = load_elem<T>(q + pq * rs + h * D + e);
    }
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] = 0.f;

    for (int c0 = 0; c0 < ball; c0 += kValuChunk) {
      const int nk = min(kValuChunk, ball - c0);
      __syncthreads();
      for (int i = threadIdx.x; i < nk * D; i += nthr) {
        const int j = i / D, e = i - j * D;
        const int64_t pk = perm ? perm_index(perm[base + c0 + j], N) : base + c0 + j;
        ks[j][e] = load_elem<T>(k + pk * rs + h * D + e);
        vs[j][e] = load_elem<T>(v + pk * rs + h * D + e);
      }
      __syncthreads();
      if (!active) continue;
      // online softmax over sub-chunks of 16 keys (scores stay in registers)
      for (int j0 = 0; j0 < nk; j0 += 16) {
        float sc[16];
        float cm = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          float t = -INFINITY;
          if (j0 + jj < nk) {
            t = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) t = fmaf(qv[e], ks[j0 + jj][e], t);
            t *= scale;
          }
          sc[jj] = t;
          cm = fmaxf(cm, t);
        }
        const float mn = fmaxf(m, cm);
        const float corr = expf(m - mn);        // 0 on the first sub-chunk
        l *= corr;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] *= corr;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          if (j0 + jj < nk) {
            const float p = expf(sc[jj] - mn);
            l += p;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] = fmaf(p, vs[j0 + jj][e], acc[e]);
          }
        }
        m = mn;
      }
    }
    if (active) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int e = 0; e < D; ++e) store_elem<T>(out + pq * rs + h * D + e, acc[e] * inv);
    }
  }
}

// --------------------------------------------------------------------------
// bf16 MFMA kernel
// --------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16 operand layout (lane l, hf = l/32, c = l%32):
//   A[i][kk]: lane i + 32*(kk/8), element kk%8      (32 rows x 16 K)
//   B[kk][j]: lane j + 32*(kk/8), element kk%8      (16 K x 32 cols)
//   C[i][j] : lane j + 32*((i/4)%2), element (i/8)*4 + i%4
// S^T = K Q^T: A = 32 keys x 16 d (K rows), B = 16 d x 32 queries (Q rows),
// so a lane of C owns query column c and 16 of the 32 keys of the block:
// key = 8*(e/4) + 4*hf + e%4.  For O^T = V^T P^T the same lane feeds P^T as
// the B operand; the K index of that product walks keys in the order above,
// which V^T in LDS matches by swapping bits 2 and 3 of the key index inside
// each group of 16 keys.
BT_DEV int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

BT_DEV uint16_t u16_of(const u32x4& r, int e) {
  const uint32_t w = r[e >> 1];
  return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu));
}

template <int D, int BALL>
__global__ __launch_bounds__(BALL / 32 * 64) void ball_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
    int32_t H, int32_t nballs, int32_t xcd_map, uint16_t* __restrict__ out) {
  const int64_t N = (int64_t)nballs * BALL;
  constexpr int NW = BALL / 32;      // waves = 32-query strips
  constexpr int NT = NW * 64;
  constexpr int KB = BALL / 32;      // 32-key blocks
  constexpr int DS = D / 16;         // K steps of S^T
  constexpr int DB = D / 32;         // 32-row blocks of O^T
  constexpr int VTS = BALL + 8;      // V^T row stride in bf16 (16 B pad)
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VTS];
  __shared__ int32_t sperm[BALL];

  // Workgroups are dispatched round-robin over the 8 XCDs; with xcd_map the
  // 8*k-th..8*k+7-th launches of one XCD take the heads of the same balls, so
  // the two 64-byte halves of a 128-byte line meet in one L2.
  int pair = blockIdx.x;
  if (xcd_map) {
    const int total = nballs * H;
    pair = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  }
  const int b = pair / H;
  const int h = pair - b * H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, c = lane & 31;
  const int64_t rs = (int64_t)H * D;
  const int64_t hoff = (int64_t)h * D;

  for (int i = tid; i < BALL; i += NT)
    sperm[i] = perm ? (int32_t)perm_index(perm[b * BALL + i], N) : b * BALL + i;
  __syncthreads();

  // ---- stage V^T: 4 keys x 8 d per item, written as 8-byte runs ----------
  for (int it = tid; it < (BALL / 4) * (D / 8); it += NT) {
    const int kq = it / (D / 8), dc = it - kq * (D / 8);
    u32x4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      r[u] = *(const u32x4*)(v + (int64_t)sperm[kq * 4 + u] * rs + hoff + dc * 8);
    const int key0 = kq * 4;
    const int pos0 = (key0 & ~15) + swap23(key0 & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 pk;
      pk[0] = uint32_t(u16_of(r[0], e)) | (uint32_t(u16_of(r[1], e)) << 16);
      pk[1] = uint32_t(u16_of(r[2], e)) | (uint32_t(u16_of(r[3], e)) << 16);
      *(u32x2*)&vt[(dc * 8 + e) * VTS + pos0] = pk;
    }
  }

  // ---- S^T = K Q^T for this wave's 32 queries ----------------------------
  const int qrow = w * 32 + c;
  const int64_t pq = sperm[qrow];
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = *(const bf16x8*)(q + pq * rs + hoff + s * 16 + hf * 8);

  f32x16 sacc[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t pk = sperm[kb * 32 + c];
    bf16x8 kf[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) kf[s] = *(const bf16x8*)(k + pk * rs + hoff + s * 16 + hf * 8);
    f32x16 a = {};
#pragma unroll
    for (int s = 0; s < DS; ++s) a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], a, 0, 0, 0);
    sacc[kb] = a;
  }

  // ---- softmax over the keys of query column c (fp32) --------------------
  const float c2 = 1.4426950408889634f / sqrtf((float)D);   // log2(e)/sqrt(d)
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[kb][e]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float moff = -mx * c2;
  float sum = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], c2, moff));
      sacc[kb][e] = p;
      sum += p;
    }
  sum += __shfl_xor(sum, 32, 64);

  __syncthreads();   // V^T staged

  // ---- O^T = V^T P^T ------------------------------------------------------
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sacc[kb][s2 * 8 + e];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x8 vf = *(const bf16x8*)&vt[(db * 32 + c) * VTS + (kb * 2 + s2) * 16 + hf * 8];
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store: lane owns dd = db*32 + 8*g + 4*hf + 0..3 -----
  const float inv = 1.0f / sum;
  uint16_t* orow = out + pq * rs + hoff;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 pk;
      pk[0] = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
      pk[1] = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
      *(u32x2*)(orow + db * 32 + g * 8 + hf * 4) = pk;
    }
}

// --------------------------------------------------------------------------
// host launchers
// --------------------------------------------------------------------------
template <typename T>
static bt_status launch_valu(const void* q, const void* k, const void* v, const int32_t* perm,
                             int64_t N, int32_t ball, int32_t H, int32_t d, void* out,
                             hipStream_t st) {
  const int nb = (int)(N / ball);
  const int thr = ball >= kValuThreads ? kValuThreads : ((ball + 63) / 64) * 64;
  dim3 grid(nb * H), block(thr);
#define BT_VALU(DD)                                                                        \
  case DD:                                                                                 \
    hipLaunchKernelGGL((ball_attn_valu<T, DD>), grid, block, 0, st, (const T*)q,           \
                       (const T*)k, (const T*)v, perm, N, H, ball, (T*)out);                 \
    break;
  switch (d) {
    BT_VALU(16)
    BT_VALU(32)
    BT_VALU(64)
    default:
      return BT_EINVAL;
  }
#undef BT_VALU
  return launch_status("ball_attn_valu");
}

template <int D>
static bt_status launch_mfma_d(const void* q, const void* k, const void* v, const int32_t* perm,
                               int64_t N, int32_t ball, int32_t H, void* out, hipStream_t st) {
  const int nb = (int)(N / ball);
  const int total = nb * H;
  const int xmap = (total % 8 == 0) ? 1 : 0;
  dim3 grid(total);
#define BT_MF(BB)                                                                           \
  case BB:                                                                                  \
    hipLaunchKernelGGL((ball_attn_mfma<D, BB>), grid, dim3(BB / 32 * 64), 0, st,           \
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, perm, H, \
                       nb, xmap, (uint16_t*)out);                                           \
    break;
  switch (ball) {
    BT_MF(32)
    BT_MF(64)
    BT_MF(128)
    BT_MF(256)
    default:
      return BT_EINVAL;
  }
#undef BT_MF
  return launch_status("ball_attn_mfma");
}

bool ball_attn_uses_mfma(bt_dtype dt, int32_t ball, int32_t d) {
  return dt == BT_BF16 && (d == 32 || d == 64) && (ball == 32 || ball == 64 || ball == 128 ||
                                                   ball == 256);
}

bt_status ball_attn_launch(const void* q, const void* k, const void* v, const int32_t* perm,
                           int64_t N, int32_t ball, int32_t H, int32_t d, bt_dtype dt,
                           void* out, hipStream_t st) {
  if (ball_attn_uses_mfma(dt, ball, d)) {
    if (d == 32) return launch_mfma_d<32>(q, k, v, perm, N, ball, H, out, st);
    return launch_mfma_d<64>(q, k, v, perm, N, ball, H, out, st);
  }
  if (dt == BT_F32) return launch_valu<float>(q, k, v, perm, N, ball, H, d, out, st);
  return launch_valu<uint16_t>(q, k, v, perm, N, ball, H, d, out, st);
}

}  // namespace bt
