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
// With MASK (the padded tree of an uneven point count) a negative permutation
// entry marks an unused slot: its key takes no weight and no output row is
// written for it; row indices are clamped to the nrows input rows.
#include <type_traits>

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

template <typename T, int D, bool MASK>
__global__ __launch_bounds__(kValuThreads) void ball_attn_valu(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ perm, int64_t N, int32_t H, int32_t ball,
    T* __restrict__ out) {
  __shared__ float ks[kValuChunk][D + 1];
  __shared__ float vs[kValuChunk][D + 1];
  __shared__ uint8_t kok[kValuChunk];       // the key holds a point (MASK)
  const int b = blockIdx.x / H;
  const int h = blockIdx.x - b * H;
  const int64_t base = (int64_t)b * ball;
  const int64_t rs = (int64_t)H * D;
  const float scale = 1.0f / sqrtf((float)D);
  const int nthr = blockDim.x;

  for (int q0 = 0; q0 < ball; q0 += nthr) {
    const int qi = q0 + threadIdx.x;
    bool active = qi < ball;
    if (MASK && active) active = perm[base + qi] >= 0;
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
        if (MASK && e == 0) kok[j] = perm[base + c0 + j] >= 0;
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
          if (j0 + jj < nk && (!MASK || kok[j0 + jj])) {
            t = 0.f;
#pragma unroll
            for (int e = 0; e < D; ++e) t = fmaf(qv[e], ks[j0 + jj][e], t);
            t *= scale;
          }
          sc[jj] = t;
          cm = fmaxf(cm, t);
        }
        const float mn = fmaxf(m, cm);
        if (MASK && mn == -INFINITY) continue;  // no key with a point so far
        const float corr = expf(m - mn);        // 0 on the first sub-chunk
        l *= corr;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] *= corr;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          if (j0 + jj < nk && (!MASK || kok[j0 + jj])) {
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

// Halves e of two 16-byte pieces as one word: (lo[e], hi[e]).
BT_DEV uint32_t pair_u16(const u32x4& lo, const u32x4& hi, int e) {
  // byte selectors of v_perm_b32: result bytes 0,1 from lo, 2,3 from hi
  return __builtin_amdgcn_perm(hi[e >> 1], lo[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the eight bf16 values of an MFMA operand, added to acc.
BT_DEV float sum_bf16x8(bf16x8 x, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
}

// An item is one ball and HPW adjacent heads (HPW = 2 when H is even): the
// rows of two heads are one 128-byte line, and random 128-byte gathers run
// about a quarter faster than 64-byte ones.  The workgroup has one wave per
// 32-query strip; each wave computes the item's heads in turn.  K (row-major,
// padded) and V^T of the heads sit in LDS.
//
// Softmax: the probabilities are rounded to bf16 once, for the P V product,
// and the normaliser is the sum of those rounded values, so the output is a
// weighted mean of V rows whose weights sum to one up to fp32 rounding.
//
// With PIPE the kernel is persistent and software-pipelined: a workgroup
// walks items j = blockIdx.x, blockIdx.x + gridDim.x, ...; while item j is
// computed, the Q/K/V pieces of the next item are in flight into registers
// and the permutation entries of the one after are in flight too.  Without
// PIPE a workgroup runs one item.
template <int D, int BALL, int HPW>
struct AttnGeom {
  static constexpr int NW = BALL / 32;      // waves = 32-query strips
  static constexpr int NT = NW * 64;
  static constexpr int KB = BALL / 32;      // 32-key blocks
  static constexpr int DS = D / 16;         // K steps of S^T
  static constexpr int DB = D / 32;         // 32-row blocks of O^T
  static constexpr int VTS = BALL + 8;      // V^T row stride (bf16), 16-byte pad
  static constexpr int KS = D + 8;          // K row stride (bf16), 16-byte pad
  static constexpr int KPI = D / 16;        // keys per staging piece
  static constexpr int CPR = HPW * D / 8;   // 16-byte chunks per row of an item
  static constexpr int IPT = HPW;           // staging pieces per thread
  static_assert((BALL / KPI) * CPR == NT * IPT, "staging pieces tile the threads");
};

template <int D, int BALL, int HPW, bool PERM, bool PIPE, bool MASK>
__global__ __launch_bounds__(BALL / 32 * 64)
BT_WAVES_PER_EU((BALL >= 256 ? (D == 32 ? 4 : 2) : (PIPE ? 3 : 4)), 8)
void ball_attn_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                    const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
                    int64_t nrows, int32_t H, int32_t nballs, int32_t xcd_map,
                    uint16_t* __restrict__ out) {
  static_assert(PERM || !MASK, "the mask comes from the permutation");
  using Gm = AttnGeom<D, BALL, HPW>;
  constexpr int NT = Gm::NT, KB = Gm::KB, DS = Gm::DS, DB = Gm::DB, VTS = Gm::VTS;
  constexpr int KS = Gm::KS, KPI = Gm::KPI, CPR = Gm::CPR, IPT = Gm::IPT;
  __shared__ __attribute__((aligned(16))) uint16_t ks[HPW][BALL * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vt[HPW][D * VTS];
  // MASK: 1 where the key slot holds a point (read four keys at a time)
  __shared__ __attribute__((aligned(16))) uint8_t kok[MASK ? BALL : 4];
  // unmasked 256-point balls: largest squared key norm per wave and head
  constexpr bool kShift = BALL >= 256 && !MASK;
  __shared__ __attribute__((aligned(16))) float knorm2[kShift ? HPW : 1][kShift ? NT / 64 : 1];

  const int64_t N = nrows;
  const int hgroups = H / HPW;
  const int total = nballs * hgroups;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, c = lane & 31;
  const int64_t rs = (int64_t)H * D;

  // Workgroups are dispatched round-robin over the 8 XCDs, and item j runs
  // on XCD j % 8 (the grid is a multiple of 8).  With xcd_map, the items an
  // XCD runs at the same time are consecutive (ball, head group) pairs, so
  // the lines of one point row are fetched at about the same time.
  auto pair_of = [&](int j) -> int { return xcd_map ? (j & 7) * (total >> 3) + (j >> 3) : j; };

  // Permutation entries of an item for this thread, as loaded: they are
  // clamped only where row addresses are formed, so that no wait for them is
  // placed ahead of the rows of the item in flight before them.
  struct Rows { int32_t q; int32_t kv[IPT][KPI]; int32_t h0; };
  auto load_rows = [&](int j) -> Rows {
    Rows r;
    const int pair = pair_of(j);
    const int b = pair / hgroups;
    r.h0 = (pair - b * hgroups) * HPW;
    const int64_t base = (int64_t)b * BALL;
    if constexpr (PERM) r.q = perm[base + w * 32 + c];
    else r.q = (int32_t)(base + w * 32 + c);
#pragma unroll
    for (int ii = 0; ii < IPT; ++ii) {
      const int kq = (tid + ii * NT) / CPR;
      if constexpr (PERM) {
        if constexpr (KPI == 2) {
          const int2 pp = *(const int2*)(perm + base + kq * 2);
          r.kv[ii][0] = pp.x;
          r.kv[ii][1] = pp.y;
        } else {
          const int4 pp = *(const int4*)(perm + base + kq * 4);
          r.kv[ii][0] = pp.x;
          r.kv[ii][1] = pp.y;
          r.kv[ii][2] = pp.z;
          r.kv[ii][3] = pp.w;
        }
      } else {
#pragma unroll
        for (int u = 0; u < KPI; ++u) r.kv[ii][u] = (int32_t)(base + kq * KPI + u);
      }
    }
    return r;
  };
  auto row_of = [&](int32_t p) -> int64_t { return PERM ? perm_index(p, N) : (int64_t)p; };

  bf16x8 qn[HPW][DS];                // next item: Q fragments (B operand of S^T)
  u32x4 kn[IPT][KPI], vn[IPT][KPI];  // next item: this thread's K and V pieces
  auto load_data = [&](const Rows& r) {
    const uint16_t* qrow = q + row_of(r.q) * rs + (int64_t)r.h0 * D + hf * 8;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int s = 0; s < DS; ++s) qn[hh][s] = *(const bf16x8*)(qrow + hh * D + s * 16);
#pragma unroll
    for (int ii = 0; ii < IPT; ++ii) {
      const int ch = (tid + ii * NT) % CPR;        // 16-byte chunk of the item row
      const int64_t off = (int64_t)r.h0 * D + ch * 8;
#pragma unroll
      for (int u = 0; u < KPI; ++u) {
        const int64_t row = row_of(r.kv[ii][u]) * rs + off;
        kn[ii][u] = *(const u32x4*)(k + row);
        vn[ii][u] = *(const u32x4*)(v + row);
      }
    }
  };
  auto stage = [&](const Rows& r) {
    float kmax2 = 0.f;
#pragma unroll
    for (int ii = 0; ii < IPT; ++ii) {
      const int it = tid + ii * NT;
      const int kq = it / CPR, ch = it - kq * CPR;
      const int hh = ch / (D / 8), dc = ch - hh * (D / 8);
      const int key0 = kq * KPI;
      if constexpr (MASK) {
        if (ch == 0) {
#pragma unroll
          for (int u = 0; u < KPI; ++u) kok[key0 + u] = r.kv[ii][u] >= 0 ? 1 : 0;
        }
      }
#pragma unroll
      for (int u = 0; u < KPI; ++u) *(u32x4*)&ks[hh][(key0 + u) * KS + dc * 8] = kn[ii][u];
      if constexpr (kShift) {
        // squared norm of each key's head slice: this thread's 8 elements,
        // then the D/8 adjacent lanes holding the rest of the slice
        float nk = 0.f;
#pragma unroll
        for (int u = 0; u < KPI; ++u) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wd = kn[ii][u][e];
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wd),
                                                __builtin_bit_cast(bf16x2, wd), t, false);
          }
#pragma unroll
          for (int m = 1; m < D / 8; m <<= 1) t += __shfl_xor(t, m, 64);
          nk = fmaxf(nk, t);
        }
        kmax2 = ii == 0 ? nk : fmaxf(kmax2, nk);
      }
      const int pos0 = (key0 & ~15) + swap23(key0 & 15);   // keeps bits 0,1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (KPI == 2) {
          *(uint32_t*)&vt[hh][(dc * 8 + e) * VTS + pos0] = pair_u16(vn[ii][0], vn[ii][1], e);
        } else {
          u32x2 pk2;
          pk2[0] = pair_u16(vn[ii][0], vn[ii][1], e);
          pk2[1] = pair_u16(vn[ii][2], vn[ii][3], e);
          *(u32x2*)&vt[hh][(dc * 8 + e) * VTS + pos0] = pk2;
        }
      }
    }
    if constexpr (kShift) {
      // lanes CPR apart hold the same head; lane hh * D/8 writes head hh
#pragma unroll
      for (int m = CPR; m < 64; m <<= 1) kmax2 = fmaxf(kmax2, __shfl_xor(kmax2, m, 64));
      if (lane < CPR && lane % (D / 8) == 0) knorm2[lane / (D / 8)][w] = kmax2;
    }
  };

  const float c2 = 1.4426950408889634f / sqrtf((float)D);   // log2(e)/sqrt(d)
  // Unmasked 256-point balls (their softmax binds with the gathers) take the
  // scores from the MFMA in log2 units with a shift already subtracted
  // (scale_query and shift_frag, common.h).  The shift is |q| * max_k |k|
  // (log2 units, the queries scaled): no score exceeds it (Cauchy-Schwarz),
  // so no maximum is taken.  When that bound is above kBound for a query of
  // the wave, the largest weight could fall below 2^(-2 kBound) and the wave
  // takes a running maximum instead, raised only when a chunk passes it by
  // more than kLazy (the weights stay below 2^kLazy).
  constexpr float kLazy = 8.f;
  constexpr float kBound = 48.f;
  bf16x8 qc[HPW][DS];
  float qnorm2[HPW];                 // kShift: squared norm of each head's scaled query
  auto take_queries = [&]() {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float nq = 0.f;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        qc[hh][s] = kShift ? scale_query(qn[hh][s], c2) : qn[hh][s];
        if constexpr (kShift) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 pr = {qc[hh][s][2 * e], qc[hh][s][2 * e + 1]};
            nq = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, nq, false);
          }
        }
      }
      if constexpr (kShift) nq += __shfl_xor(nq, 32, 64);
      qnorm2[hh] = nq;
    }
  };
  // attention of the staged item for its HPW heads and this wave's queries
  auto attend = [&](const Rows& rc) {
    uint16_t* orow0 = out + row_of(rc.q) * rs + (int64_t)rc.h0 * D;
    // kShift: the bound |q| max|k| of every head, up front
    float bnd_q[HPW];
    bool bnd_ok[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      bnd_q[hh] = 0.f;
      bnd_ok[hh] = false;
      if constexpr (kShift) {
        const float nq = qnorm2[hh];
        float nk = knorm2[hh][0];
#pragma unroll
        for (int i = 1; i < NT / 64; ++i) nk = fmaxf(nk, knorm2[hh][i]);
        bnd_q[hh] = __builtin_sqrtf(nq * nk);
        bnd_ok[hh] = __ballot(!(bnd_q[hh] <= kBound)) == 0;   // NaN or Inf: not bounded
      }
    }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      // Keys go in chunks of CH 32-key blocks with an online softmax: one
      // chunk for balls up to 128; 64-key chunks for 256-point balls keep a
      // wave's score and probability registers small enough for two
      // workgroups per CU.
      constexpr int CH = BALL >= 256 ? 2 : KB;
      f32x16 oacc[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
      float s4[4] = {0.f, 0.f, 0.f, 0.f};   // four chains of the normaliser
      float mrun = -INFINITY;               // running maximum (raw scores; kShift: log2 units)
      bf16x8 shf = {};                      // kShift: shift_frag8(mrun)
      const bool bounded = kShift && bnd_ok[hh];
      if (bounded) {
        mrun = bnd_q[hh];
        shf = shift_frag8(mrun);
      }
      auto chunks = [&](auto bnd) {
        constexpr bool BND = decltype(bnd)::value;
#pragma unroll
        for (int c0 = 0; c0 < KB; c0 += CH) {
          // ---- S^T = K Q^T --------------------------------------------------
          f32x16 sacc[CH];
#pragma unroll
          for (int kb = 0; kb < CH; ++kb) {
            f32x16 a = {};
            if constexpr (kShift) {
              if (BND || c0 > 0)
                a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones_frag8(), shf, a, 0, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < DS; ++s) {
              const bf16x8 kf =
                  *(const bf16x8*)&ks[hh][((c0 + kb) * 32 + c) * KS + s * 16 + hf * 8];
              a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qc[hh][s], a, 0, 0, 0);
            }
            sacc[kb] = a;
          }
          if constexpr (MASK) {
            // element e holds key kb*32 + 8*(e/4) + 4*hf + e%4
#pragma unroll
            for (int kb = 0; kb < CH; ++kb)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const uint32_t ok4 = *(const uint32_t*)&kok[(c0 + kb) * 32 + 8 * g + 4 * hf];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (!((ok4 >> (8 * i)) & 0xffu)) sacc[kb][g * 4 + i] = -INFINITY;
              }
          }
          // ---- softmax over the keys of query column c ----------------------
          // Four independent chains for the maximum and the sum (BND: the
          // maximum is not used).
          float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
          for (int kb = 0; kb < CH; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) m4[e & 3] = fmaxf(m4[e & 3], sacc[kb][e]);
          float mx = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          float moff = -mx * c2;
          if constexpr (BND) {
            (void)mx;
          } else if constexpr (kShift) {
            // the scores are relative to mrun (on the first chunk, raw)
            if (c0 == 0 || __ballot(mx > kLazy)) {
              float delta;
              if (c0 == 0) {
                delta = mx;
                mrun = mx;
              } else {
                const float mn = mrun + fmaxf(mx, 0.f);
                delta = mn - mrun;
                const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
                for (int i = 0; i < 4; ++i) s4[i] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                  for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
                mrun = mn;
              }
              shf = shift_frag8(mrun);
#pragma unroll
              for (int kb = 0; kb < CH; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[kb][e] -= delta;
            }
          } else if constexpr (CH < KB) {
            const float mn = fmaxf(mrun, mx);
            // nothing to rescale before the first chunk with a key; a chunk
            // whose keys are all unused slots leaves the maximum at -inf
            const float alpha =
                mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mrun - mn) * c2);
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
              for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            mrun = mn;
            moff = mn == -INFINITY ? 0.f : -mn * c2;
          }
          bf16x8 pf[CH][2];                // P^T operands, rounded once
#pragma unroll
          for (int kb = 0; kb < CH; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                pf[kb][s2][e] = (__bf16)__builtin_amdgcn_exp2f(
                    kShift ? sacc[kb][s2 * 8 + e] : fmaf(sacc[kb][s2 * 8 + e], c2, moff));
              s4[(kb * 2 + s2) & 3] = sum_bf16x8(pf[kb][s2], s4[(kb * 2 + s2) & 3]);
            }
          // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
          for (int kb = 0; kb < CH; ++kb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
              for (int db = 0; db < DB; ++db) {
                const bf16x8 vf = *(const bf16x8*)&vt[hh][(db * 32 + c) * VTS +
                                                          ((c0 + kb) * 2 + s2) * 16 + hf * 8];
                oacc[db] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb][s2], oacc[db], 0, 0, 0);
              }
        }
      };
      if (kShift && bounded) chunks(std::true_type{});
      else chunks(std::false_type{});
      float sum = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      sum += __shfl_xor(sum, 32, 64);
      // ---- normalise, regroup across the lane halves, store 16-byte runs ---
      // Lane (c, hf) holds d = db*32 + 8*g + 4*hf + 0..3 for g = 0..3.  After
      // one exchange with lane c^32, the hf = 0 lane holds d 0-7 and 16-23
      // and the hf = 1 lane holds d 8-15 and 24-31 of each 32-column block.
      const float inv = __builtin_amdgcn_rcpf(sum);
      uint16_t* orow = orow0 + hh * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        u32x2 pg[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          pg[g][0] = pack_bf16x2(oacc[db][g * 4 + 0] * inv, oacc[db][g * 4 + 1] * inv);
          pg[g][1] = pack_bf16x2(oacc[db][g * 4 + 2] * inv, oacc[db][g * 4 + 3] * inv);
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
        if (!MASK || rc.q >= 0) {          // no output for an unused slot
          *(u32x4*)(orow + db * 32 + hf * 8) = c0;
          *(u32x4*)(orow + db * 32 + 16 + hf * 8) = c1;
        }
      }
    }
  };

  const int G = gridDim.x;
  int j = blockIdx.x;
  if (j >= total) return;                    // uniform over the workgroup
  Rows rc = load_rows(j);
  load_data(rc);
  stage(rc);
  take_queries();
  if constexpr (!PIPE) {                     // one item per workgroup
    __syncthreads();
    attend(rc);
    return;
  }
  int jn = j + G;
  Rows rn = rc;
  if (jn < total) rn = load_rows(jn);

  for (;;) {
    const bool has_next = jn < total;
    if (has_next) load_data(rn);             // rows of the next item
    const int jnn = jn + G;
    Rows rnn = rn;
    if (jnn < total) rnn = load_rows(jnn);   // permutation of the one after
    __syncthreads();                         // the current item is staged
    attend(rc);
    if (!has_next) break;
    __syncthreads();                         // everyone is done with LDS
    stage(rn);                               // waits for the next item's rows
    take_queries();
    rc = rn;
    rn = rnn;
    jn = jnn;
  }
}

// --------------------------------------------------------------------------
// host launchers
// --------------------------------------------------------------------------
template <typename T, bool MASK>
static bt_status launch_valu(const void* q, const void* k, const void* v, const int32_t* perm,
                             int64_t nrows, int64_t nslots, int32_t ball, int32_t H, int32_t d,
                             void* out, hipStream_t st) {
  const int nb = (int)(nslots / ball);
  const int thr = ball >= kValuThreads ? kValuThreads : ((ball + 63) / 64) * 64;
  dim3 grid(nb * H), block(thr);
#define BT_VALU(DD)                                                                        \
  case DD:                                                                                 \
    hipLaunchKernelGGL((ball_attn_valu<T, DD, MASK>), grid, block, 0, st, (const T*)q,     \
                       (const T*)k, (const T*)v, perm, nrows, H, ball, (T*)out);             \
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

// Workgroups of the MFMA kernel: at most kGridPerCu per CU (a multiple of 8
// for the XCD map), or one per item when there are fewer items.  With more
// items than that the pipelined form runs.  At 65,536 points, ball 128 and 8
// heads (2,048 head-pair items; about 3 workgroups fit per CU at once), 5
// per CU measured best among 3 to 8 in steps of a half.
constexpr int kGridPerCu = 5;

// CU count of the current device, cached per device (a relaxed atomic per
// slot: concurrent first calls store the same value).
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static int cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  if (cached) __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  return n;
}

static int attn_grid(int total) {
  int g = device_cus() * kGridPerCu;
  g -= g % 8;
  if (g < 8) g = 8;
  return total < g ? total : g;
}

template <int D, int BB, int HPW, bool MASK>
static bt_status launch_mfma(const void* q, const void* k, const void* v, const int32_t* perm,
                             int64_t nrows, int64_t nslots, int32_t H, void* out,
                             hipStream_t st) {
  const int nb = (int)(nslots / BB);
  const int total = nb * (H / HPW);
  const int xmap = (total % 8 == 0) ? 1 : 0;
  // the masked kernel and 256-point balls run one item per workgroup: their
  // persistent form would need more registers than the waves per SIMD that
  // hide the gathers allow (256-point balls: two 8-wave workgroups per CU)
  const int g = (MASK || BB >= 256) ? total : attn_grid(total);
  const bool pipe = g < total;
  dim3 grid(g), block(BB / 32 * 64);
#define BT_MF(PERM, PIPE, MK)                                                                \
  hipLaunchKernelGGL((ball_attn_mfma<D, BB, HPW, PERM, PIPE, MK>), grid, block, 0, st,      \
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, perm, nrows, \
                     H, nb, xmap, (uint16_t*)out)
  if constexpr (MASK) {
    BT_MF(true, false, true);
  } else if constexpr (BB >= 256) {
    if (perm) BT_MF(true, false, false);
    else BT_MF(false, false, false);
  } else if (perm) {
    if (pipe) BT_MF(true, true, false);
    else BT_MF(true, false, false);
  } else {
    if (pipe) BT_MF(false, true, false);
    else BT_MF(false, false, false);
  }
#undef BT_MF
  return launch_status("ball_attn_mfma");
}

// Head pairs when H is even: at d = 32 two heads' slices of a row are one
// 128-byte line.  At d = 64 one head's slice already is a line, and from
// 128-point balls on a pair's registers leave one wave per SIMD, so single
// heads run there (65,536 points, 8 heads, ball 128: 69 us against 84 us).
template <int D, bool MASK>
static bt_status launch_mfma_d(const void* q, const void* k, const void* v, const int32_t* perm,
                               int64_t nrows, int64_t nslots, int32_t ball, int32_t H, void* out,
                               hipStream_t st) {
  const bool pair = H % 2 == 0 && (D == 32 || ball <= 64);
  switch (ball) {
    case 32:
      return pair ? launch_mfma<D, 32, 2, MASK>(q, k, v, perm, nrows, nslots, H, out, st)
                  : launch_mfma<D, 32, 1, MASK>(q, k, v, perm, nrows, nslots, H, out, st);
    case 64:
      return pair ? launch_mfma<D, 64, 2, MASK>(q, k, v, perm, nrows, nslots, H, out, st)
                  : launch_mfma<D, 64, 1, MASK>(q, k, v, perm, nrows, nslots, H, out, st);
    case 128:
      return pair ? launch_mfma<D, 128, 2, MASK>(q, k, v, perm, nrows, nslots, H, out, st)
                  : launch_mfma<D, 128, 1, MASK>(q, k, v, perm, nrows, nslots, H, out, st);
    case 256:   // head pairs at d = 32 (at d = 64 their LDS would leave one workgroup per CU)
      if constexpr (D == 32) {
        if (pair) return launch_mfma<D, 256, 2, MASK>(q, k, v, perm, nrows, nslots, H, out, st);
      }
      return launch_mfma<D, 256, 1, MASK>(q, k, v, perm, nrows, nslots, H, out, st);
    default:
      return BT_EINVAL;
  }
}

bool ball_attn_uses_mfma(bt_dtype dt, int32_t ball, int32_t d) {
  return dt == BT_BF16 && (d == 32 || d == 64) && (ball == 32 || ball == 64 || ball == 128 ||
                                                   ball == 256);
}

bt_status ball_attn_launch(const void* q, const void* k, const void* v, const int32_t* perm,
                           int64_t N, int32_t ball, int32_t H, int32_t d, bt_dtype dt,
                           void* out, hipStream_t st) {
  if (ball_attn_uses_mfma(dt, ball, d)) {
    if (d == 32) return launch_mfma_d<32, false>(q, k, v, perm, N, N, ball, H, out, st);
    return launch_mfma_d<64, false>(q, k, v, perm, N, N, ball, H, out, st);
  }
  if (dt == BT_F32) return launch_valu<float, false>(q, k, v, perm, N, N, ball, H, d, out, st);
  return launch_valu<uint16_t, false>(q, k, v, perm, N, N, ball, H, d, out, st);
}

// Padded tree: nslots permutation entries (ball | nslots), negative for an
// unused slot, the others in [0, nrows).
bt_status ball_attn_padded_launch(const void* q, const void* k, const void* v,
                                  const int32_t* perm, int64_t nrows, int64_t nslots,
                                  int32_t ball, int32_t H, int32_t d, bt_dtype dt, void* out,
                                  hipStream_t st) {
  if (ball_attn_uses_mfma(dt, ball, d)) {
    if (d == 32) return launch_mfma_d<32, true>(q, k, v, perm, nrows, nslots, ball, H, out, st);
    return launch_mfma_d<64, true>(q, k, v, perm, nrows, nslots, ball, H, out, st);
  }
  if (dt == BT_F32)
    return launch_valu<float, true>(q, k, v, perm, nrows, nslots, ball, H, d, out, st);
  return launch_valu<uint16_t, true>(q, k, v, perm, nrows, nslots, ball, H, d, out, st);
}

}  // namespace bt
