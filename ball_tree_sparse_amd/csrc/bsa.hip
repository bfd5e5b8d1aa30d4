// Ball Sparse Attention (Pith review of arXiv 2506.12541: "What carries the
// argument", "Core claim", Figure 1 and Figure 3 captions; referee report,
// major comments 1 and 2 on Eqs. 10-15).  Everything runs in tree order:
//
//   pool    K, V -> head-major tree-ordered copies (K row-major [h][t][d];
//           V transposed in 32-key blocks [h][t/32][d][32], the operand
//           layout of the P V product), block means of K in fp32 ([h][d][j],
//           for the scores) and bf16 ([h][j][d]) and of V in bf16 (transposed
//           like V) over blocks of l tree positions; Q -> fp32 group means
//           qbar (the pooled query); the largest squared key norm per block
//           and head.
//   select  s[g, j] = qbar_g . Kc_j / sqrt(d) in fp32; blocks inside the
//           group's own ball are excluded; top-k per (group, head), ties to
//           the smaller block index: a wave bitonic sort of the 64 lane
//           maxima gives the k-th best of them, a lower bound of the k-th
//           score; the (score, block) pairs at least that good (k or a few
//           more) are gathered through LDS and sorted the same way, best
//           first.  Only when more than 64 pairs tie with the bound does the
//           wave fall back to repeated arg-max.  One workgroup per head also
//           reduces the block norm maxima to the head's.
//   fused   one workgroup per (group, head), one wave per 32 queries: the
//           ball, compression and selection branches run one after another
//           as online-softmax attention over 64-key chunks (S^T = K Q^T and
//           O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, both operands read
//           straight from the pooled layouts, so waves never wait on each
//           other), and are merged with G = sigmoid(W q + b) before one
//           scatter of the bf16 result to original order.  The softmax shift
//           is the bound |q| max|k| of every score when that bound is small
//           enough (no maximum is taken), else a running maximum.
#include "bsa_common.h"

namespace bt {

size_t bsa_ws_size(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  return bsa_layout(N, H, d, p).total;
}

// ------------------------------------------------------------------ pool ----

// Workgroup (block j of `len` tree positions, head group hg of HP heads),
// 256 threads.  Rows of K and V are gathered through perm (HP*D*2 bytes
// each, a whole 128-byte line for two heads at d = 32) into LDS (lds: 2 len
// HP D bf16); K is written back row-major to kt[h][t][:], V transposed to
// vt[h][t/32][:][tpos(t%32)]; the block means are summed from LDS in a fixed
// order (deterministic).
template <int D, int HP>
BT_DEV void pool_kv_block(int64_t j, int hg, uint16_t* lds, const uint16_t* __restrict__ k,
                          const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
                          int32_t H, int32_t len, int64_t N, uint16_t* __restrict__ kt,
                          uint16_t* __restrict__ vtt, float* __restrict__ kc32,
                          uint16_t* __restrict__ kcb, uint16_t* __restrict__ vct,
                          float* __restrict__ kbmax) {
  __shared__ float snorm[4][HP];      // largest squared key norm per wave and head
  constexpr int CPR = HP * D / 8;                 // 16-byte chunks per gathered row
  uint16_t* kl = lds;                             // [len][HP*D]
  uint16_t* vl = lds + (size_t)len * HP * D;      // [len][HP*D]
  const int tid = threadIdx.x;
  const int h0 = hg * HP;
  const int64_t nc = N / len;
  const int64_t rs = (int64_t)H * D;
  // Squared norms of the key head rows: a thread's 8 elements, summed over
  // the D/8 adjacent lanes of the row; the largest per thread (256 is a
  // multiple of CPR, so a thread keeps one head).  len * CPR is a multiple of
  // 64 (len is a multiple of 32), so every lane of a wave runs the same
  // iterations.
  float n2max = 0.f;
  for (int it = tid; it < len * CPR; it += 256) {
    const int r = it / CPR, ch = it - r * CPR;
    const int64_t t = j * len + r;
    const int64_t pt = perm_index(perm[t], N);
    const int64_t off = pt * rs + (int64_t)h0 * D + ch * 8;
    const u32x4 xk = *(const u32x4*)(k + off);
    const u32x4 xv = *(const u32x4*)(v + off);
    const int hh = ch / (D / 8), dc = ch - hh * (D / 8);
    *(u32x4*)(kt + ((int64_t)(h0 + hh) * N + t) * D + dc * 8) = xk;
    *(u32x4*)(kl + r * (HP * D) + ch * 8) = xk;
    *(u32x4*)(vl + r * (HP * D) + ch * 8) = xv;
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bsa_bf16x2, xk[e]),
                                           __builtin_bit_cast(bsa_bf16x2, xk[e]), n2, false);
#pragma unroll
    for (int m = 1; m < D / 8; m <<= 1) n2 += __shfl_xor(n2, m, 64);
    n2max = fmaxf(n2max, n2);
  }
  // lanes CPR apart hold the same head
#pragma unroll
  for (int m = CPR; m < 64; m <<= 1) n2max = fmaxf(n2max, __shfl_xor(n2max, m, 64));
  if ((tid & 63) < CPR && (tid & 63) % (D / 8) == 0)
    snorm[tid >> 6][(tid & 63) / (D / 8)] = n2max;
  __syncthreads();
  // V transposed: 16-byte runs of 8 positions of one (head, 32-key block, d)
  const int nkb = len / 32;
  for (int it = tid; it < HP * nkb * D * 4; it += 256) {
    const int q8 = it & 3;
    const int dd = (it >> 2) % D;
    const int kb = (it >> 2) / D % nkb;
    const int hh = (it >> 2) / D / nkb;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = kb * 32 + tpos(q8 * 8 + 2 * e), r1 = kb * 32 + tpos(q8 * 8 + 2 * e + 1);
      o[e] = uint32_t(vl[r0 * (HP * D) + hh * D + dd]) |
             (uint32_t(vl[r1 * (HP * D) + hh * D + dd]) << 16);
    }
    const int64_t blk = (j * len) / 32 + kb;
    *(u32x4*)(vtt + (((int64_t)(h0 + hh) * (N / 32) + blk) * D + dd) * 32 + q8 * 8) = o;
  }
  if (tid < HP)
    kbmax[(int64_t)(h0 + tid) * nc + j] =
        fmaxf(fmaxf(snorm[0][tid], snorm[1][tid]), fmaxf(snorm[2][tid], snorm[3][tid]));
  // block means of K (fp32 and bf16) and V (bf16, transposed layout)
  for (int it = tid; it < 2 * HP * D; it += 256) {
    const int isv = it / (HP * D), hd = it - isv * (HP * D);
    const int hh = hd / D, dd = hd - hh * D;
    const uint16_t* col = (isv ? vl : kl) + hd;
    float sum = 0.f;
    for (int r = 0; r < len; ++r) sum += bf16_to_f32(col[r * (HP * D)]);
    const float m = sum * (1.0f / (float)len);
    const int h = h0 + hh;
    if (!isv) {
      kc32[((int64_t)h * D + dd) * nc + j] = m;
      kcb[((int64_t)h * nc + j) * D + dd] = (uint16_t)(pack_bf16x2(m, 0.f) & 0xffffu);
    } else {
      vct[(((int64_t)h * (nc / 32) + j / 32) * D + dd) * 32 + tpos((int)(j % 32))] =
          (uint16_t)(pack_bf16x2(m, 0.f) & 0xffffu);
    }
  }
}

// Workgroup (group j, column slice sy), 256 threads: fp32 means of Q over
// groups of `len` tree positions.  A column is 8 consecutive bf16 of one
// head; thread (col, rg) sums rows rg, rg+RG, ...; the RG partial sums
// (part: 256 x 9 floats of LDS) are added in a fixed order.
BT_DEV void pool_q_group(int64_t j, int sy, float (*part)[9], const uint16_t* __restrict__ src,
                         const int32_t* __restrict__ perm, int32_t H, int32_t d, int32_t len,
                         int64_t N, float* __restrict__ mean32) {
  const int cols = H * d / 8;
  const int slice = cols < 64 ? cols : 64;
  const int RG = 256 / slice;
  const int tid = threadIdx.x;
  const int colw = tid % slice, rg = tid / slice;
  const int col = sy * slice + colw;
  const int h = (col * 8) / d, dd = (col * 8) % d;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (rg < RG && col < cols) {
    for (int r = rg; r < len; r += RG) {
      const int64_t t = j * len + r;
      const int64_t pt = perm_index(perm[t], N);
      const u32x4 x = *(const u32x4*)(src + pt * H * d + col * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_to_f32((uint16_t)(x[e] & 0xffffu));
        acc[2 * e + 1] += bf16_to_f32((uint16_t)(x[e] >> 16));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[tid][e] = acc[e];
  __syncthreads();
  if (rg == 0 && col < cols) {
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = part[colw][e];
    for (int g = 1; g < RG; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += part[g * slice + colw][e];
    const float inv = 1.0f / (float)len;
    const int64_t nb = N / len;
    float* m32 = mean32 + ((int64_t)h * nb + j) * d + dd;
#pragma unroll
    for (int e = 0; e < 8; ++e) m32[e] = s[e] * inv;
  }
}

// Grid (groups, column slices): the query means alone.
__global__ __launch_bounds__(256) void bsa_pool_q(const uint16_t* __restrict__ src,
                                                  const int32_t* __restrict__ perm, int32_t H,
                                                  int32_t d, int32_t len, int64_t N,
                                                  float* __restrict__ mean32) {
  __shared__ float part[256][9];
  pool_q_group(blockIdx.x, blockIdx.y, part, src, perm, H, d, len, N, mean32);
}

// One launch for the pooling of a BSA step: workgroups 0 .. nc*H/HP - 1
// pool K and V (block j = id % nc, head group id / nc), the rest the group
// means of Q (group id' % ngroups, column slice id' / ngroups), so that the
// lighter query pooling fills the tail of the K and V gathers.  Dynamic LDS:
// the larger of 2 len HP D bf16 and 256 x 9 floats.
template <int D, int HP>
__global__ __launch_bounds__(256) void bsa_pool(const uint16_t* __restrict__ q,
                                                const uint16_t* __restrict__ k,
                                                const uint16_t* __restrict__ v,
                                                const int32_t* __restrict__ perm, int32_t H,
                                                int32_t block, int32_t group, int64_t N,
                                                uint16_t* __restrict__ kt,
                                                uint16_t* __restrict__ vtt,
                                                float* __restrict__ kc32,
                                                uint16_t* __restrict__ kcb,
                                                uint16_t* __restrict__ vct,
                                                float* __restrict__ kbmax,
                                                float* __restrict__ qbar) {
  HIP_DYNAMIC_SHARED(uint16_t, lds)
  const int64_t nc = N / block, ngroups = N / group;
  const int64_t nkv = nc * (H / HP);
  const int64_t id = blockIdx.x;          // uniform over the workgroup
  if (id < nkv) {
    pool_kv_block<D, HP>(id % nc, (int)(id / nc), lds, k, v, perm, H, block, N, kt, vtt, kc32,
                         kcb, vct, kbmax);
  } else {
    const int64_t iq = id - nkv;
    pool_q_group(iq % ngroups, (int)(iq / ngroups), (float (*)[9])lds, q, perm, H, D, group, N,
                 qbar);
  }
}

// ---------------------------------------------------------------- select ----
// One step of a wave arg-max over (v, i): take the partner's pair if its
// value is larger, or equal with a smaller index.  DPP moves with the lane's
// own value as the fallback, so lanes without a partner keep their pair.
#define BT_ARGMAX_DPP(CTRL, ROWS)                                                          \
  {                                                                                        \
    const float ov = __int_as_float(                                                       \
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xf, \
                                    false));                                               \
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROWS, 0xf, false);              \
    const bool take = (ov > v) | ((ov == v) & (oi < i));                                   \
    v = take ? ov : v;                                                                     \
    i = take ? oi : i;                                                                     \
  }

// Wave arg-max: the largest v, ties to the smallest i, returned to every
// lane.  row_shr 1, 2, 4, 8 leave each row's result in its lane 15; the two
// row broadcasts gather the four rows into lane 63.
BT_DEV void wave_argmax(float& v, int& i) {
  BT_ARGMAX_DPP(0x111, 0xf)    // row_shr:1
  BT_ARGMAX_DPP(0x112, 0xf)    // row_shr:2
  BT_ARGMAX_DPP(0x114, 0xf)    // row_shr:4
  BT_ARGMAX_DPP(0x118, 0xf)    // row_shr:8
  BT_ARGMAX_DPP(0x142, 0xa)    // row_bcast:15 into rows 1 and 3
  BT_ARGMAX_DPP(0x143, 0xc)    // row_bcast:31 into rows 2 and 3
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  i = __builtin_amdgcn_readlane(i, 63);
}
#undef BT_ARGMAX_DPP

// (score, block) pairs: a is better than b if its score is larger, or equal
// with a smaller block index.
BT_DEV bool sel_better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

// The value of lane (this lane) ^ J.  Distances 1 and 2 are DPP quad
// permutes and 4, 8, 16 ds_swizzle bit-mask moves inside each half-wave, so
// only distance 32 goes through ds_bpermute.
template <int J>
BT_DEV int lane_xor(int x) {
  if constexpr (J == 1) return __builtin_amdgcn_mov_dpp(x, 0xb1, 0xf, 0xf, false);  // [1,0,3,2]
  else if constexpr (J == 2) return __builtin_amdgcn_mov_dpp(x, 0x4e, 0xf, 0xf, false);  // [2,3,0,1]
  else if constexpr (J < 32) return __builtin_amdgcn_ds_swizzle(x, (J << 10) | 0x1f);
  else {   // lanes 32 apart: the two halves swapped on the VALU
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return (int)((threadIdx.x & 32) ? r[0] : r[1]);
  }
}

template <int K, int J>
BT_DEV void sort_step(float& v, int& i, int lane) {
  const float ov = __int_as_float(lane_xor<J>(__float_as_int(v)));
  const int oi = lane_xor<J>(i);
  // the lower lane of a pair keeps the better pair in a best-first run
  // (lane & K == 0) and the worse one in a worst-first run
  const bool keep_better = ((lane & J) == 0) == ((lane & K) == 0);
  const bool ob = sel_better(ov, oi, v, i);
  if (ob == keep_better) {
    v = ov;
    i = oi;
  }
}

template <int K, int J>
BT_DEV void sort_stage(float& v, int& i, int lane) {
  sort_step<K, J>(v, i, lane);
  if constexpr (J > 1) sort_stage<K, J / 2>(v, i, lane);
}

// Bitonic sort of one (score, block) pair per lane across the wave, best
// first: lane 0 ends with the best pair.  Pairs must be distinct.
BT_DEV void wave_sort_best_first(float& v, int& i) {
  const int lane = threadIdx.x & 63;
  sort_stage<2, 1>(v, i, lane);
  sort_stage<4, 2>(v, i, lane);
  sort_stage<8, 4>(v, i, lane);
  sort_stage<16, 8>(v, i, lane);
  sort_stage<32, 16>(v, i, lane);
  sort_stage<64, 32>(v, i, lane);
}

// Lanes below this one with their bit of m set.
BT_DEV uint32_t sel_lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Workgroup = (head, tile of TG groups).  Scores of the tile live in LDS;
// the waves take the tile's groups in turn for the top-k (a chain of
// dependent wave reductions per group, so one group per wave keeps more of
// them in flight).
template <int D>
__global__ __launch_bounds__(kSelThreads) void bsa_select(const float* __restrict__ qbar,
                                                  const float* __restrict__ kc32, int32_t H,
                                                  int32_t nc, int32_t ngroups,
                                                  int32_t tg, int32_t group, int32_t ball,
                                                  int32_t block, int32_t topk, int32_t mask,
                                                  int32_t* __restrict__ sel,
                                                  const float* __restrict__ kbmax,
                                                  float* __restrict__ kmax2) {
  HIP_DYNAMIC_SHARED(float, smem)
  constexpr int d = D;
  float* sc = smem + tg * d;           // [tg][nc] (after tg*d floats kept for the layout)
  float* cand = sc + tg * nc;          // [waves][128]: top-k candidates of a wave
  const int h = blockIdx.y;
  const int g0 = blockIdx.x * tg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ng = min(tg, ngroups - g0);
  const float scale = 1.0f / sqrtf((float)d);
  if (blockIdx.x == 0) {
    // the head's largest squared key norm, for the attention's softmax shift
    // (smem[0 .. 7] lie in the tg*d floats that the scores leave unused)
    float m = 0.f;
    for (int jb = tid; jb < nc; jb += kSelThreads) m = fmaxf(m, kbmax[(int64_t)h * nc + jb]);
    m = wave_max(m);
    if (lane == 0) smem[w] = m;
    __syncthreads();
    if (tid == 0) {
      float x = smem[0];
      for (int i = 1; i < kSelThreads / 64; ++i) x = fmaxf(x, smem[i]);
      kmax2[h] = x;
    }
    __syncthreads();
  }
  const float* kh = kc32 + (int64_t)h * D * nc;   // [d][nc]: lanes read consecutive blocks
  // the pooled query of a group is the same for every lane: it is read with
  // scalar loads (SGPR operands of the FMAs), not from LDS once per lane
  const float* qh = qbar + ((int64_t)h * ngroups + g0) * d;
  for (int jb = tid; jb < nc; jb += kSelThreads) {
    float kr[D];
#pragma unroll
    for (int e = 0; e < D; ++e) kr[e] = kh[(int64_t)e * nc + jb];
    for (int g = 0; g < ng; ++g) {
      const float* qg = qh + g * D;
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = fmaf(qg[e], kr[e], s);
      sc[g * nc + jb] = s * scale;
    }
  }
  __syncthreads();
  for (int g = w; g < ng; g += kSelThreads / 64) {
    float* s = sc + g * nc;
    const int gg = g0 + g;
    if (mask) {
      // blocks overlapping a ball that holds a position of the group
      const int64_t t0 = (int64_t)gg * group, t1 = t0 + group;
      const int64_t lo = (t0 / ball) * ball, hi = ((t1 - 1) / ball + 1) * ball;
      for (int64_t jb = lo / block + lane; jb < hi / block; jb += 64) s[jb] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    if (nc <= 64 * kSelRegs) {
      // scores of block jb = lane + 64*i held in registers
      float r[kSelRegs];
#pragma unroll
      for (int i = 0; i < kSelRegs; ++i) {
        const int jb = lane + 64 * i;
        r[i] = jb < nc ? s[jb] : -INFINITY;
      }
      // Threshold: the topk-th best of the 64 lane maxima.  At least topk
      // pairs are as good as it, so every one of the topk best pairs is.
      float lv = r[0];
      int li = lane;
#pragma unroll
      for (int u = 1; u < kSelRegs; ++u)
        if (r[u] > lv) { lv = r[u]; li = lane + 64 * u; }  // ascending index: first max kept
      wave_sort_best_first(lv, li);
      const float tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), topk - 1));
      const int ti = __builtin_amdgcn_readlane(li, topk - 1);
      uint32_t cnt = 0;
#pragma unroll
      for (int u = 0; u < kSelRegs; ++u) cnt += !sel_better(tv, ti, r[u], lane + 64 * u);
      // exclusive prefix of the candidate counts (at most 16: five bits)
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int bit = 0; bit < 5; ++bit) {
        const uint64_t m = __ballot((cnt >> bit) & 1u);
        before += sel_lanes_below(m) << bit;
        total += (uint32_t)__popcll(m) << bit;
      }
      if (total <= 64) {
        // gather the candidates, one per lane, and sort them: the first
        // topk lanes hold the selection, best first
        float* cv = cand + w * 128;
        int* ci = (int*)(cv + 64);
        uint32_t pos = before;
#pragma unroll
        for (int u = 0; u < kSelRegs; ++u)
          if (!sel_better(tv, ti, r[u], lane + 64 * u)) {
            cv[pos] = r[u];
            ci[pos] = lane + 64 * u;
            ++pos;
          }
        __builtin_amdgcn_wave_barrier();
        float v = (uint32_t)lane < total ? cv[lane] : -INFINITY;
        int i = (uint32_t)lane < total ? ci[lane] : 0x40000000 + lane;   // after every block
        __builtin_amdgcn_wave_barrier();
        wave_sort_best_first(v, i);
        if (lane < topk) sel[((int64_t)h * ngroups + gg) * topk + lane] = i;
      } else {
        // many pairs tie with the threshold: repeated wave arg-max
        for (int it = 0; it < topk; ++it) {
          float v = -INFINITY;
          int i = 0x7fffffff;
#pragma unroll
          for (int u = 0; u < kSelRegs; ++u)
            if (r[u] > v) { v = r[u]; i = lane + 64 * u; }   // ascending index: first max kept
          wave_argmax(v, i);
          if (lane == 0) sel[((int64_t)h * ngroups + gg) * topk + it] = i;
          if ((i & 63) == lane) {
#pragma unroll
            for (int u = 0; u < kSelRegs; ++u)
              if (u == (i >> 6)) r[u] = -INFINITY;
          }
        }
      }
    } else {
      for (int it = 0; it < topk; ++it) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        for (int jb = lane; jb < nc; jb += 64) {
          const float x = s[jb];
          if (x > v) { v = x; i = jb; }          // ascending jb: first max kept
        }
        wave_argmax(v, i);
        if (lane == 0) {
          sel[((int64_t)h * ngroups + gg) * topk + it] = i;
          if (i < nc) s[i] = -INFINITY;
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

// ------------------------------------------------------ group compression ----
// Pooled (fp32) query rows times scale -> the B operand of S^T = K Q^T,
// rounded to bf16 once.
template <int D>
BT_DEV void pooled_query_frags(const float* __restrict__ row, float scale, bf16x8* qf) {
  const int hf = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const float4 a = *(const float4*)(row + s * 16 + hf * 8);
    const float4 b = *(const float4*)(row + s * 16 + hf * 8 + 4);
    qf[s] = bf16x8{(__bf16)(a.x * scale), (__bf16)(a.y * scale), (__bf16)(a.z * scale),
                   (__bf16)(a.w * scale), (__bf16)(b.x * scale), (__bf16)(b.y * scale),
                   (__bf16)(b.z * scale), (__bf16)(b.w * scale)};
  }
}

// Compression branch of group compression: 32 block-mean queries of a head
// per workgroup, all attending to every coarse token.  The coarse tokens are
// split into kQcWaves contiguous ranges (multiples of 32), one per wave, and
// the waves' partial results (running maximum, normaliser, unnormalised
// output) are merged through LDS.  Grid (nc/32, H).
constexpr int kQcWaves = 4;

template <int D>
__global__ __launch_bounds__(kQcWaves * 64) void bsa_qc_cmp(const float* __restrict__ qc,
                                                            const uint16_t* __restrict__ kcb,
                                                            const uint16_t* __restrict__ vct,
                                                            int32_t nc,
                                                            float* __restrict__ ocmp) {
  constexpr int DB = D / 32;
  __shared__ float pm[kQcWaves][64], pl[kQcWaves][64], po[kQcWaves][DB * 16][64];
  const int h = blockIdx.y, lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 31;
  const int64_t j = (int64_t)blockIdx.x * 32 + c;          // this lane's coarse query
  bf16x8 qf[D / 16];
  pooled_query_frags<D>(qc + ((int64_t)h * nc + j) * D, log2_score_scale(D), qf);
  Branch<DB> br;
  branch_init<D>(br);
  const int seg = ((nc / 32 + kQcWaves - 1) / kQcWaves) * 32;  // keys per wave
  const int k0 = w * seg, len = max(0, min(nc - k0, seg));
  attend_range<D, 1>(kcb + (int64_t)h * nc * D, vct + (int64_t)h * nc * D,
                     [&](int key) -> int64_t { return k0 + key; }, len, qf, &br);
  const float l = xor32_sum(branch_l(br));
  pm[w][lane] = br.m;
  pl[w][lane] = l;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) po[w][db * 16 + e][lane] = br.o[db][e];
  __syncthreads();
  if (w != 0) return;
  float mt = -INFINITY;
#pragma unroll
  for (int u = 0; u < kQcWaves; ++u) mt = fmaxf(mt, pm[u][lane]);
  float lt = 0.f, f[kQcWaves];
#pragma unroll
  for (int u = 0; u < kQcWaves; ++u) {
    // a wave without keys has m = -inf and contributes nothing
    f[u] = pm[u][lane] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm[u][lane] - mt);
    lt = fmaf(f[u], pl[u][lane], lt);
  }
  const float inv = __builtin_amdgcn_rcpf(lt);
  const int hf = lane >> 5;
  float* row = ocmp + ((int64_t)h * nc + j) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < kQcWaves; ++u) a = fmaf(f[u], po[u][db * 16 + g * 4 + i][lane], a);
        x[i] = a * inv;
      }
      *(float4*)(row + db * 32 + g * 8 + hf * 4) = make_float4(x[0], x[1], x[2], x[3]);
    }
}

// Selection branch of group compression: one wave per (group, head) and a
// single query -- the group's mean query (fp32) -- over the union of the
// group's selected blocks, on the vector units (one query would fill 1/32
// of an MFMA tile).  Keys go in chunks of 1,024 with an online softmax: lane
// l scores keys l, l+64, ... of the chunk; the weights go to LDS in the
// position order of the transposed V blocks; then lane (dd, half) adds
// p * V[., dd] over half of every 32-key block.  Grid (ngroups, H).
constexpr int kQcsChunk = 1024;

template <int D>
__global__ __launch_bounds__(64) void bsa_qc_slc(const float* __restrict__ qbar,
                                                 const uint16_t* __restrict__ kt,
                                                 const uint16_t* __restrict__ vtt,
                                                 const int32_t* __restrict__ sel, int64_t N,
                                                 int32_t nc, int32_t ngroups, int32_t block,
                                                 int32_t topk, float* __restrict__ oslc) {
  __shared__ int32_t ssel[64];
  __shared__ __attribute__((aligned(16))) float ps[kQcsChunk];
  const int g = blockIdx.x, h = blockIdx.y, lane = threadIdx.x & 63;
  const int dd = lane & 31, half = lane >> 5;
  if (lane < topk)   // block indices are forced into range like perm entries
    ssel[lane] = (int32_t)perm_index(sel[((int64_t)h * ngroups + g) * topk + lane], nc);
  float qv[D];
  const float* qrow = qbar + ((int64_t)h * ngroups + g) * D;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const float4 x = *(const float4*)(qrow + e);
    qv[e] = x.x; qv[e + 1] = x.y; qv[e + 2] = x.z; qv[e + 3] = x.w;
  }
  __syncthreads();   // ssel
  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* kh = kt + (int64_t)h * N * D;
  const uint16_t* vh = vtt + (int64_t)h * N * D;
  auto row_of = [&](int key) -> int64_t {
    return (int64_t)ssel[key / block] * block + (key % block);
  };
  const int nsel = topk * block;
  float m = -INFINITY, l = 0.f;
  float o[D / 32] = {};
  for (int k0 = 0; k0 < nsel; k0 += kQcsChunk) {
    const int nk = min(kQcsChunk, nsel - k0);          // a multiple of 32
    // ---- scores of this lane's keys
    float sc[kQcsChunk / 64];
    float cm = -INFINITY;
#pragma unroll
    for (int i = 0; i < kQcsChunk / 64; ++i) {
      const int kl = i * 64 + lane;
      sc[i] = -INFINITY;
      if (kl < nk) {
        const uint16_t* kr = kh + row_of(k0 + kl) * D;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < D; e += 8) {
          const u32x4 x = *(const u32x4*)(kr + e);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            s = fmaf(qv[e + 2 * u], bf16_to_f32((uint16_t)(x[u] & 0xffffu)), s);
            s = fmaf(qv[e + 2 * u + 1], bf16_to_f32((uint16_t)(x[u] >> 16)), s);
          }
        }
        sc[i] = s * c2;
        cm = fmaxf(cm, sc[i]);
      }
    }
    cm = wave_max(cm);
    const float mn = fmaxf(m, cm);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);          // 0 on the first chunk
    m = mn;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < kQcsChunk / 64; ++i) {
      const int kl = i * 64 + lane;
      if (kl < nk) {
        const float p = __builtin_amdgcn_exp2f(sc[i] - mn);
        ls += p;
        ps[(kl & ~31) + tpos(kl & 31)] = p;                  // V^T position order
      }
    }
    l = l * alpha + ls;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    __builtin_amdgcn_wave_barrier();                          // one wave: LDS in order
    // ---- o[dd] += sum over half of every 32-key block of p * V[., dd]
    for (int kb = 0; kb < nk / 32; ++kb) {
      const int64_t tb = row_of(k0 + kb * 32) / 32;           // transposed V block
      const float* pp = ps + kb * 32 + half * 16;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const uint16_t* vr = vh + (tb * D + db * 32 + dd) * 32 + half * 16;
        const u32x4 v0 = *(const u32x4*)vr, v1 = *(const u32x4*)(vr + 8);
        const float4 p0 = *(const float4*)pp, p1 = *(const float4*)(pp + 4);
        const float4 p2 = *(const float4*)(pp + 8), p3 = *(const float4*)(pp + 12);
        const float pv[16] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w,
                              p2.x, p2.y, p2.z, p2.w, p3.x, p3.y, p3.z, p3.w};
        float acc = o[db];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc = fmaf(pv[2 * u], bf16_to_f32((uint16_t)(v0[u] & 0xffffu)), acc);
          acc = fmaf(pv[2 * u + 1], bf16_to_f32((uint16_t)(v0[u] >> 16)), acc);
          acc = fmaf(pv[8 + 2 * u], bf16_to_f32((uint16_t)(v1[u] & 0xffffu)), acc);
          acc = fmaf(pv[8 + 2 * u + 1], bf16_to_f32((uint16_t)(v1[u] >> 16)), acc);
        }
        o[db] = acc;
      }
    }
    __builtin_amdgcn_wave_barrier();                          // ps reused by the next chunk
  }
  l = wave_sum_f32(l);
  const float inv = __builtin_amdgcn_rcpf(l);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const float tot = o[db] + __shfl_xor(o[db], 32, 64);     // the two halves
    if (half == 0) oslc[((int64_t)h * ngroups + g) * D + db * 32 + dd] = tot * inv;
  }
}

// QC (group compression): only the ball branch runs here; the compression
// and selection results of the token's block and group come from ocmp and
// oslc (fp32, computed by bsa_qc_cmp / bsa_qc_slc).
// A workgroup owns one (group, head); each of its NWV waves owns QB blocks of
// 32 queries (group = NWV * QB * 32).
template <int D, int NWV, bool QC, int QB>
__global__ __launch_bounds__(NWV * 64) BT_WAVES_PER_EU((QC || D > 32 ? 2 : 3), 8) void bsa_fused(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ perm,
    const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vtt,
    const uint16_t* __restrict__ kcb, const uint16_t* __restrict__ vct,
    const int32_t* __restrict__ sel, const float* __restrict__ gate_w,
    const float* __restrict__ gate_b, float gc0, float gc1, float gc2, int32_t H, int64_t N,
    int32_t nc, int32_t ngroups, int32_t ball, int32_t block, int32_t topk, int32_t xcd_map,
    const float* __restrict__ ocmp, const float* __restrict__ oslc,
    const float* __restrict__ kmax2, uint16_t* __restrict__ out) {
  constexpr int DS = D / 16, DB = D / 32;
  __shared__ int32_t ssel[64];
  // Without group compression the merged output and the gates of a wave's
  // queries wait in LDS while the three branches run (lane-major,
  // conflict-free), so the registers hold only the branch state: three waves
  // per SIMD instead of two.  With it (one branch, then the block and group
  // results) the merged output stays in registers.
  __shared__ float sacc_out[QC ? 1 : NWV][QC ? 1 : QB][QC ? 1 : DB * 16][64];
  __shared__ float sgate[NWV][QB][3][64];
  f32x16 accr[QC ? QB : 1][QC ? DB : 1];
  const int total = ngroups * H;
  int pair = blockIdx.x;
  if (xcd_map) pair = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int h = pair / ngroups;
  const int g = pair - h * ngroups;
  const int group = NWV * QB * 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, c = lane & 31;
  const int64_t rs = (int64_t)H * D;
  if (tid < topk)   // block indices are forced into range like perm entries
    ssel[tid] = (int32_t)perm_index(sel[((int64_t)h * ngroups + g) * topk + tid], nc);

  // queries of this wave: tree positions t0 .. t0 + QB*32 - 1, block qb at
  // t0 + qb*32 + c for lane column c
  const int64_t t0 = (int64_t)g * group + w * (QB * 32);
  bf16x8 qf[QB * DS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t pq = perm_index(perm[t0 + qb * 32 + c], N);
#pragma unroll
    for (int s = 0; s < DS; ++s)
      qf[qb * DS + s] = *(const bf16x8*)(q + pq * rs + (int64_t)h * D + s * 16 + hf * 8);
  }

  // gates: G = sigmoid(W q + b), one W [3, d] for every head
  float G[QB][3];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    G[qb][0] = gc0;
    G[qb][1] = gc1;
    G[qb][2] = gc2;
    if (gate_w) {
      float z0 = 0.f, z1 = 0.f, z2 = 0.f;
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int dd = s * 16 + hf * 8 + e;
          const float x = (float)qf[qb * DS + s][e];
          z0 = fmaf(gate_w[dd], x, z0);
          z1 = fmaf(gate_w[D + dd], x, z1);
          z2 = fmaf(gate_w[2 * D + dd], x, z2);
        }
      z0 += __shfl_xor(z0, 32, 64);
      z1 += __shfl_xor(z1, 32, 64);
      z2 += __shfl_xor(z2, 32, 64);
      if (gate_b) { z0 += gate_b[0]; z1 += gate_b[1]; z2 += gate_b[2]; }
      G[qb][0] = 1.0f / (1.0f + __expf(-z0));
      G[qb][1] = 1.0f / (1.0f + __expf(-z1));
      G[qb][2] = 1.0f / (1.0f + __expf(-z2));
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) sgate[w][qb][i][lane] = G[qb][i];
  }
  __syncthreads();   // ssel
  // from here on the queries are scaled: their scores come out in log2 units
#pragma unroll
  for (int i = 0; i < QB * DS; ++i) qf[i] = scale_query(qf[i], log2_score_scale(D));
  // The shift of every branch is the bound |q| max|k| when it is at most
  // kBoundLog2 for every query of the wave (the largest weight is then at
  // least 2^(-2 kBoundLog2), a normal float); otherwise the branches keep a
  // running maximum.
  float bound[QB];
  bool bounded = true;
  {
    const float k2 = kmax2[h];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float n2 = 0.f;
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bsa_bf16x2 pr = {qf[qb * DS + s][2 * e], qf[qb * DS + s][2 * e + 1]};
          n2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, n2, false);
        }
      n2 = xor32_sum(n2);
      bound[qb] = __builtin_sqrtf(n2 * k2);
      bounded = bounded && __ballot(!(bound[qb] <= kBoundLog2)) == 0;   // NaN: not bounded
    }
  }

  const uint16_t* kh = kt + (int64_t)h * N * D;
  const uint16_t* vh = vtt + (int64_t)h * N * D;
  Branch<DB> br[QB];
  // out_slot = (first ? 0 : out_slot) + gate * o / l for every query block
  auto merge = [&](int gi, bool first) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l = xor32_sum(branch_l(br[qb]));
      const float f = sgate[w][qb][gi][lane] * __builtin_amdgcn_rcpf(l);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if constexpr (QC) {
            accr[qb][db][e] = br[qb].o[db][e] * f;      // QC: the ball branch only
          } else {
            float& x = sacc_out[w][qb][db * 16 + e][lane];
            x = first ? br[qb].o[db][e] * f : fmaf(br[qb].o[db][e], f, x);
          }
        }
    }
  };

  auto init = [&](auto bnd) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if constexpr (decltype(bnd)::value) branch_init_bound<D>(br[qb], bound[qb]);
      else branch_init<D>(br[qb]);
    }
  };
  auto branches = [&](auto bnd) {
    constexpr bool BND = decltype(bnd)::value;
    // ---- ball branch: the ball holding this group (group | ball) ----------
    {
      init(bnd);
      const int64_t b0 = ((int64_t)g * group / ball) * ball;
      attend_range<D, QB, BND>(kh, vh, [&](int key) -> int64_t { return b0 + key; }, ball, qf, br);
      merge(0, true);
    }
    if constexpr (QC) {
      // ---- group compression: the token's block and group results --------
      const float* rsl = oslc + ((int64_t)h * ngroups + g) * D;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int64_t t = t0 + qb * 32 + c;
        const float* rc = ocmp + ((int64_t)h * nc + t / block) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const float4 a = *(const float4*)(rc + db * 32 + gq * 8 + hf * 4);
            const float4 b = *(const float4*)(rsl + db * 32 + gq * 8 + hf * 4);
            const float g1 = G[qb][1], g2 = G[qb][2];
            f32x16& x = accr[qb][db];
            x[gq * 4 + 0] = fmaf(g2, b.x, fmaf(g1, a.x, x[gq * 4 + 0]));
            x[gq * 4 + 1] = fmaf(g2, b.y, fmaf(g1, a.y, x[gq * 4 + 1]));
            x[gq * 4 + 2] = fmaf(g2, b.z, fmaf(g1, a.z, x[gq * 4 + 2]));
            x[gq * 4 + 3] = fmaf(g2, b.w, fmaf(g1, a.w, x[gq * 4 + 3]));
          }
      }
    } else {
      // ---- compression branch: every coarse token ---------------------------
      {
        init(bnd);
        const uint16_t* kch = kcb + (int64_t)h * nc * D;
        const uint16_t* vch = vct + (int64_t)h * nc * D;
        attend_range<D, QB, BND>(kch, vch, [&](int key) -> int64_t { return key; }, nc, qf, br);
        merge(1, false);
      }
      // ---- selection branch: the union of the selected blocks ---------------
      {
        init(bnd);
        attend_range<D, QB, BND>(kh, vh,
                                 [&](int key) -> int64_t {
                                   return (int64_t)ssel[key / block] * block + (key % block);
                                 },
                                 topk * block, qf, br);
        merge(2, false);
      }
    }
  };
  if (bounded) branches(std::true_type{});
  else branches(std::false_type{});

  // ---- store: lane owns d = db*32 + 8*gq + 4*hf + 0..3 of its query -------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t pq = perm_index(perm[t0 + qb * 32 + c], N);
    uint16_t* orow = out + pq * rs + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (QC) y[r] = accr[qb][db][gq * 4 + r];
          else y[r] = sacc_out[w][qb][db * 16 + gq * 4 + r][lane];
        }
        u32x2 pk;
        pk[0] = pack_bf16x2(y[0], y[1]);
        pk[1] = pack_bf16x2(y[2], y[3]);
        *(u32x2*)(orow + db * 32 + gq * 8 + hf * 4) = pk;
      }
  }
}

// ------------------------------------------------------------------ host ----
template <int D, bool QC>
static void launch_fused(int group, dim3 grid, hipStream_t st, const uint16_t* q,
                         const int32_t* perm, const uint16_t* kt, const uint16_t* vt,
                         const uint16_t* kcb, const uint16_t* vcb, const int32_t* sel,
                         const float* gw, const float* gb, const float* gc, int32_t H, int64_t N,
                         int32_t nc, int32_t ngroups, int32_t ball, int32_t block, int32_t topk,
                         int32_t xmap, const float* ocmp, const float* oslc, const float* kmax2,
                         uint16_t* out) {
  const float g0 = gc ? gc[0] : 0.f, g1 = gc ? gc[1] : 0.f, g2 = gc ? gc[2] : 0.f;
#define BT_FUSED(NW, QBB)                                                                     \
  hipLaunchKernelGGL((bsa_fused<D, NW, QC, QBB>), grid, dim3(NW * 64), 0, st, q, perm, kt,    \
                     vt, kcb, vcb, sel, gw, gb, g0, g1, g2, H, N, nc, ngroups, ball, block,     \
                     topk, xmap, ocmp, oslc, kmax2, out)
  // d = 32 and groups of 64 or more: each wave owns two 32-query blocks, so
  // every K and V fragment it loads serves 64 queries (at d = 64 the second
  // block's state would not fit the registers)
  if constexpr (D == 32) {
    switch (group) {
      case 32: BT_FUSED(1, 1); break;
      case 64: BT_FUSED(1, 2); break;
      case 128: BT_FUSED(2, 2); break;
      case 256: BT_FUSED(4, 2); break;
      default: break;
    }
  } else {
    switch (group) {
      case 32: BT_FUSED(1, 1); break;
      case 64: BT_FUSED(2, 1); break;
      case 128: BT_FUSED(4, 1); break;
      case 256: BT_FUSED(8, 1); break;
      default: break;
    }
  }
#undef BT_FUSED
}

// Tree-ordered copies of K and V (V transposed), block means, the pooled
// group queries and the selection: the part of BSA that the forward and the
// backward share.  sel: [H, N/group, topk] int32.
bt_status bsa_prepare(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                      int32_t H, int32_t d, const bsa_params* p, void* ws, int32_t* sel,
                      hipStream_t st) {
  const BsaLayout L = bsa_layout(N, H, d, p);
  char* b = (char*)ws;
  uint16_t* kt = (uint16_t*)(b + L.kt);
  uint16_t* vt = (uint16_t*)(b + L.vt);
  float* kc32 = (float*)(b + L.kc32);
  uint16_t* kcb = (uint16_t*)(b + L.kcb);
  uint16_t* vcb = (uint16_t*)(b + L.vcb);
  float* qbar = (float*)(b + L.qbar);
  float* kbmax = (float*)(b + L.kbmax);
  float* kmax2 = (float*)(b + L.kmax2);
  const int32_t nc = (int32_t)(N / p->block), ngroups = (int32_t)(N / p->group);
  const int cols = H * d / 8;
  const int slice = cols < 64 ? cols : 64;
  const dim3 pblk(256);

  // K, V: tree-ordered copies (V transposed) and block means; Q: fp32 group
  // means (the pooled queries that score the blocks); one launch
  const int hp = (H % 2 == 0 && d == 32) ? 2 : 1;
  size_t pool_lds = (size_t)2 * p->block * hp * d * sizeof(uint16_t);
  if (pool_lds < 256 * 9 * sizeof(float)) pool_lds = 256 * 9 * sizeof(float);
  const int64_t npool = (int64_t)nc * (H / hp) + (int64_t)ngroups * ((cols + slice - 1) / slice);
  const dim3 gp((unsigned)npool);
#define BT_POOL(DD, HH)                                                                       \
  hipLaunchKernelGGL((bsa_pool<DD, HH>), gp, pblk, pool_lds, st, (const uint16_t*)q,          \
                     (const uint16_t*)k, (const uint16_t*)v, perm, H, p->block, p->group, N, kt, \
                     vt, kc32, kcb, vcb, kbmax, qbar)
  if (d == 32 && hp == 2) BT_POOL(32, 2);
  else if (d == 32) BT_POOL(32, 1);
  else BT_POOL(64, 1);
#undef BT_POOL
  bt_status s = launch_status("bsa_pool");
  if (s != BT_OK) return s;

  int tg = 8192 / nc;                  // scores of a tile: <= 32 KB of LDS
  if (tg > 16) tg = 16;
  if (tg < 1) tg = 1;
  const size_t smem = (size_t)(tg * d + tg * nc + kSelThreads / 64 * 128) * sizeof(float);
  const dim3 gs((ngroups + tg - 1) / tg, H);
  if (d == 32)
    hipLaunchKernelGGL(bsa_select<32>, gs, dim3(kSelThreads), smem, st, qbar, kc32, H, nc, ngroups, tg,
                       p->group, p->ball, p->block, p->topk, p->mask_own_ball, sel, kbmax, kmax2);
  else
    hipLaunchKernelGGL(bsa_select<64>, gs, dim3(kSelThreads), smem, st, qbar, kc32, H, nc, ngroups, tg,
                       p->group, p->ball, p->block, p->topk, p->mask_own_ball, sel, kbmax, kmax2);
  return launch_status("bsa_select");
}

bt_status bsa_launch(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                     int32_t H, int32_t d, const bsa_params* p, const float* gate_w,
                     const float* gate_b, const float* gate_const, int32_t* sel_out, void* ws,
                     void* out, hipStream_t st) {
  const BsaLayout L = bsa_layout(N, H, d, p);
  char* b = (char*)ws;
  uint16_t* kt = (uint16_t*)(b + L.kt);
  uint16_t* vt = (uint16_t*)(b + L.vt);
  uint16_t* kcb = (uint16_t*)(b + L.kcb);
  uint16_t* vcb = (uint16_t*)(b + L.vcb);
  float* qbar = (float*)(b + L.qbar);
  const float* kmax2 = (const float*)(b + L.kmax2);
  int32_t* sel = sel_out ? sel_out : (int32_t*)(b + L.sel);
  const int32_t nc = (int32_t)(N / p->block), ngroups = (int32_t)(N / p->group);
  const int cols = H * d / 8;
  const int slice = cols < 64 ? cols : 64;
  const dim3 pblk(256);
  bt_status s = bsa_prepare(q, k, v, perm, N, H, d, p, ws, sel, st);
  if (s != BT_OK) return s;

  // group compression: block-mean queries over all coarse tokens, group-mean
  // queries over their selected blocks
  const bool qcm = p->query_compression != 0;
  float* ocmp = qcm ? (float*)(b + L.ocmp) : nullptr;
  float* oslc = qcm ? (float*)(b + L.oslc) : nullptr;
  if (qcm) {
    float* qc = (float*)(b + L.qc);
    const dim3 gqc(nc, (cols + slice - 1) / slice);
    hipLaunchKernelGGL(bsa_pool_q, gqc, pblk, 0, st, (const uint16_t*)q, perm, H, d, p->block, N,
                       qc);
    const dim3 gcm(nc / 32, H), gsl(ngroups, H);
    if (d == 32) {
      hipLaunchKernelGGL(bsa_qc_cmp<32>, gcm, dim3(kQcWaves * 64), 0, st, qc, kcb, vcb, nc, ocmp);
      hipLaunchKernelGGL(bsa_qc_slc<32>, gsl, dim3(64), 0, st, qbar, kt, vt, sel, N, nc, ngroups,
                         p->block, p->topk, oslc);
    } else {
      hipLaunchKernelGGL(bsa_qc_cmp<64>, gcm, dim3(kQcWaves * 64), 0, st, qc, kcb, vcb, nc, ocmp);
      hipLaunchKernelGGL(bsa_qc_slc<64>, gsl, dim3(64), 0, st, qbar, kt, vt, sel, N, nc, ngroups,
                         p->block, p->topk, oslc);
    }
    s = launch_status("bsa_qc");
    if (s != BT_OK) return s;
  }

  const int total = ngroups * H;
  const int xmap = (total % 8 == 0) ? 1 : 0;
#define BT_FUSED_CALL(DD, QCM)                                                                \
  launch_fused<DD, QCM>(p->group, dim3(total), st, (const uint16_t*)q, perm, kt, vt, kcb, vcb, sel, \
                        gate_w, gate_b, gate_const, H, N, nc, ngroups, p->ball, p->block,     \
                        p->topk, xmap, ocmp, oslc, kmax2, (uint16_t*)out)
  if (d == 32) {
    if (qcm) BT_FUSED_CALL(32, true);
    else BT_FUSED_CALL(32, false);
  } else {
    if (qcm) BT_FUSED_CALL(64, true);
    else BT_FUSED_CALL(64, false);
  }
#undef BT_FUSED_CALL
  return launch_status("bsa_fused");
}

}  // namespace bt
