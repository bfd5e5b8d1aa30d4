// Ball Sparse Attention (Pith review of arXiv 2506.12541: "What carries the
// argument", "Core claim", Figure 1 and Figure 3 captions; referee report,
// major comments 1 and 2 on Eqs. 10-15).  Everything runs in tree order:
//
//   pool    K, V -> block means Kc (fp32 and bf16), Vc (bf16) over blocks of
//           l tree positions, plus head-major tree-ordered copies Kt, Vt so
//           that every later read of a ball or a selected block is one
//           contiguous run; Q -> fp32 group means qbar (the pooled query).
//   select  s[g, j] = qbar_g . Kc_j / sqrt(d) in fp32; blocks inside the
//           group's own ball are excluded; top-k per (group, head) by
//           repeated wave arg-max (ties to the smaller block index).
//   fused   one workgroup per (group, head), one wave per 32 queries: the
//           ball, compression and selection branches run one after another
//           as online-softmax attention over 128-key chunks (S^T = K Q^T and
//           O^T = V^T P^T on v_mfma_f32_32x32x16_bf16, V^T staged in LDS),
//           and are merged with G = sigmoid(W q + b) before one scatter of
//           the bf16 result to original order.
#include "common.h"

namespace bt {

constexpr int kChunk = 128;            // keys per online-softmax step

struct BsaLayout {
  size_t kt, vt, kc32, kcb, vcb, qbar, sel, total;
};

static size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

static BsaLayout bsa_layout(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  BsaLayout L{};
  const size_t nc = (size_t)(N / p->block), G = (size_t)(N / p->group);
  size_t o = 0;
  L.kt = o; o = a256(o + (size_t)N * H * d * 2);
  L.vt = o; o = a256(o + (size_t)N * H * d * 2);
  L.kc32 = o; o = a256(o + nc * H * d * 4);
  L.kcb = o; o = a256(o + nc * H * d * 2);
  L.vcb = o; o = a256(o + nc * H * d * 2);
  L.qbar = o; o = a256(o + G * H * d * 4);
  L.sel = o; o = a256(o + G * H * (size_t)p->topk * 4);
  L.total = o;
  return L;
}

size_t bsa_ws_size(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  return bsa_layout(N, H, d, p).total;
}

// ------------------------------------------------------------------ pool ----
// Grid (blocks of `len` tree positions, column slices).  A column is 8
// consecutive bf16 of one head.  Thread (col, rg) sums rows rg, rg+RG, ...;
// the RG partial sums are then added in a fixed order, so the result is
// deterministic.  With COPY the rows are also written to the head-major
// tree-ordered copy dst[h][t][:].
template <bool COPY, bool F32OUT, bool BF16OUT>
__global__ __launch_bounds__(256) void bsa_pool(const uint16_t* __restrict__ src,
                                                const int32_t* __restrict__ perm, int32_t H,
                                                int32_t d, int32_t len, int64_t N,
                                                uint16_t* __restrict__ copy,
                                                float* __restrict__ mean32,
                                                uint16_t* __restrict__ meanb) {
  __shared__ float part[256][9];
  const int cols = H * d / 8;
  const int slice = cols < 64 ? cols : 64;
  const int RG = 256 / slice;
  const int tid = threadIdx.x;
  const int colw = tid % slice, rg = tid / slice;
  const int col = blockIdx.y * slice + colw;
  const int64_t j = blockIdx.x;
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
      if (COPY) *(u32x4*)(copy + ((int64_t)h * N + t) * d + dd) = x;
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
    if (F32OUT) {
      float* m32 = mean32 + ((int64_t)h * nb + j) * d + dd;
#pragma unroll
      for (int e = 0; e < 8; ++e) m32[e] = s[e] * inv;
    }
    if (BF16OUT) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(s[2 * e] * inv, s[2 * e + 1] * inv);
      *(u32x4*)(meanb + ((int64_t)h * nb + j) * d + dd) = o;
    }
  }
}

// ---------------------------------------------------------------- select ----
// Workgroup = (head, tile of TG groups).  Scores of the tile live in LDS.
template <int D>
__global__ __launch_bounds__(256) void bsa_select(const float* __restrict__ qbar,
                                                  const float* __restrict__ kc32, int32_t H,
                                                  int32_t nc, int32_t ngroups,
                                                  int32_t tg, int32_t group, int32_t ball,
                                                  int32_t block, int32_t topk, int32_t mask,
                                                  int32_t* __restrict__ sel) {
  HIP_DYNAMIC_SHARED(float, smem)
  constexpr int d = D;
  float* qs = smem;                    // [tg][d]
  float* sc = smem + tg * d;           // [tg][nc]
  const int h = blockIdx.y;
  const int g0 = blockIdx.x * tg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ng = min(tg, ngroups - g0);
  for (int i = tid; i < ng * d; i += 256)
    qs[i] = qbar[((int64_t)h * ngroups + g0) * d + i];
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)d);
  const float* kh = kc32 + (int64_t)h * nc * d;
  for (int jb = tid; jb < nc; jb += 256) {
    float kr[D];
#pragma unroll
    for (int e = 0; e < D; ++e) kr[e] = kh[(int64_t)jb * D + e];
    for (int g = 0; g < ng; ++g) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = fmaf(qs[g * D + e], kr[e], s);
      sc[g * nc + jb] = s * scale;
    }
  }
  __syncthreads();
  for (int g = w; g < ng; g += 4) {
    float* s = sc + g * nc;
    const int gg = g0 + g;
    if (mask) {
      // blocks overlapping a ball that holds a position of the group
      const int64_t t0 = (int64_t)gg * group, t1 = t0 + group;
      const int64_t lo = (t0 / ball) * ball, hi = ((t1 - 1) / ball + 1) * ball;
      for (int64_t jb = lo / block + lane; jb < hi / block; jb += 64) s[jb] = -INFINITY;
    }
    __builtin_amdgcn_wave_barrier();
    for (int it = 0; it < topk; ++it) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int jb = lane; jb < nc; jb += 64) {
        const float v = s[jb];
        if (v > bv) { bv = v; bi = jb; }          // ascending jb: first max kept
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (lane == 0) {
        sel[((int64_t)h * ngroups + gg) * topk + it] = bi;
        if (bi < nc) s[bi] = -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// ----------------------------------------------------------------- fused ----
BT_DEV int swap23b(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

BT_DEV uint16_t u16_at(const u32x4& r, int e) {
  const uint32_t x = r[e >> 1];
  return (uint16_t)((e & 1) ? (x >> 16) : (x & 0xffffu));
}

// Running state of one branch for the lane's query column.
template <int DB>
struct Branch {
  f32x16 o[DB];
  float m;      // running max in log2-scaled units
  float l;      // lane-local partial sum of exp2
};

template <int D, int NWV>
struct FusedCtx {
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int VTS = kChunk + 8;
};

// One online-softmax step over a chunk of nkb*32 keys whose rows are
// rowbase(kb) + c for 32-key block kb (rows of a head-major [rows][D] array).
template <int D, int NT, typename RowFn>
BT_DEV void attend_chunk(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                         RowFn rowbase, int nkb, const bf16x8* qf, float c2, Branch<D / 32>& br,
                         uint16_t* vt) {
  constexpr int DS = D / 16, DB = D / 32, VTS = kChunk + 8;
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, c = lane & 31;
  // stage V^T of the chunk (4 keys x 8 d per item)
  for (int it = tid; it < nkb * 8 * (D / 8); it += NT) {
    const int kq = it / (D / 8), dc = it - kq * (D / 8);
    const int key0 = kq * 4;
    const int64_t row0 = rowbase(key0 >> 5) + (key0 & 31);
    u32x4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = *(const u32x4*)(vh + (row0 + u) * D + dc * 8);
    const int pos0 = (key0 & ~15) + swap23b(key0 & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 pk;
      pk[0] = uint32_t(u16_at(r[0], e)) | (uint32_t(u16_at(r[1], e)) << 16);
      pk[1] = uint32_t(u16_at(r[2], e)) | (uint32_t(u16_at(r[3], e)) << 16);
      *(u32x2*)&vt[(dc * 8 + e) * VTS + pos0] = pk;
    }
  }
  // S^T blocks
  f32x16 sacc[kChunk / 32];
#pragma unroll
  for (int kb = 0; kb < kChunk / 32; ++kb) {
    if (kb < nkb) {
      const int64_t row = rowbase(kb) + c;
      f32x16 a = {};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 kf = *(const bf16x8*)(kh + row * D + s * 16 + hf * 8);
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], a, 0, 0, 0);
      }
      sacc[kb] = a;
    }
  }
  float cm = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < kChunk / 32; ++kb)
    if (kb < nkb)
#pragma unroll
      for (int e = 0; e < 16; ++e) cm = fmaxf(cm, sacc[kb][e] * c2);
  cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
  const float mn = fmaxf(br.m, cm);
  const float alpha = __builtin_amdgcn_exp2f(br.m - mn);     // 0 on the first chunk
  br.l *= alpha;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) br.o[db][e] *= alpha;
  br.m = mn;
#pragma unroll
  for (int kb = 0; kb < kChunk / 32; ++kb)
    if (kb < nkb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][e], c2, -mn));
        sacc[kb][e] = p;
        br.l += p;
      }
  __syncthreads();                                        // V^T staged
#pragma unroll
  for (int kb = 0; kb < kChunk / 32; ++kb) {
    if (kb < nkb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (__bf16)sacc[kb][s2 * 8 + e];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf =
              *(const bf16x8*)&vt[(db * 32 + c) * VTS + (kb * 2 + s2) * 16 + hf * 8];
          br.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, br.o[db], 0, 0, 0);
        }
      }
    }
  }
  __syncthreads();                                        // V^T free again
}

template <int D>
BT_DEV void branch_init(Branch<D / 32>& br) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) br.o[db] = f32x16{};
  br.m = -INFINITY;
  br.l = 0.f;
}

template <int D>
BT_DEV void branch_merge(const Branch<D / 32>& br, float gate, f32x16* acc) {
  const float l = br.l + __shfl_xor(br.l, 32, 64);
  const float f = gate / l;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = fmaf(br.o[db][e], f, acc[db][e]);
}

template <int D, int NWV>
__global__ __launch_bounds__(NWV * 64) void bsa_fused(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ perm,
    const uint16_t* __restrict__ kt, const uint16_t* __restrict__ vt_g,
    const uint16_t* __restrict__ kcb, const uint16_t* __restrict__ vcb,
    const int32_t* __restrict__ sel, const float* __restrict__ gate_w,
    const float* __restrict__ gate_b, float gc0, float gc1, float gc2, int32_t H, int64_t N,
    int32_t nc, int32_t ngroups, int32_t ball, int32_t block, int32_t topk, int32_t xcd_map,
    uint16_t* __restrict__ out) {
  constexpr int NT = NWV * 64;
  constexpr int DS = D / 16, DB = D / 32, VTS = kChunk + 8;
  __shared__ __attribute__((aligned(16))) uint16_t vts[D * VTS];
  __shared__ int32_t ssel[64];
  const int total = ngroups * H;
  int pair = blockIdx.x;
  if (xcd_map) pair = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int h = pair / ngroups;
  const int g = pair - h * ngroups;
  const int group = NWV * 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, c = lane & 31;
  const int64_t rs = (int64_t)H * D;
  if (tid < topk)   // block indices are forced into range like perm entries
    ssel[tid] = (int32_t)perm_index(sel[((int64_t)h * ngroups + g) * topk + tid], nc);

  // queries of this wave: tree positions t0 .. t0+31
  const int64_t t0 = (int64_t)g * group + w * 32;
  const int64_t pq = perm_index(perm[t0 + c], N);
  bf16x8 qf[DS];
#pragma unroll
  for (int s = 0; s < DS; ++s) qf[s] = *(const bf16x8*)(q + pq * rs + (int64_t)h * D + s * 16 + hf * 8);

  // gates: G = sigmoid(W q + b), one W [3, d] for every head
  float G0 = gc0, G1 = gc1, G2 = gc2;
  if (gate_w) {
    float z0 = 0.f, z1 = 0.f, z2 = 0.f;
#pragma unroll
    for (int s = 0; s < DS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dd = s * 16 + hf * 8 + e;
        const float x = (float)qf[s][e];
        z0 = fmaf(gate_w[dd], x, z0);
        z1 = fmaf(gate_w[D + dd], x, z1);
        z2 = fmaf(gate_w[2 * D + dd], x, z2);
      }
    z0 += __shfl_xor(z0, 32, 64);
    z1 += __shfl_xor(z1, 32, 64);
    z2 += __shfl_xor(z2, 32, 64);
    if (gate_b) { z0 += gate_b[0]; z1 += gate_b[1]; z2 += gate_b[2]; }
    G0 = 1.0f / (1.0f + __expf(-z0));
    G1 = 1.0f / (1.0f + __expf(-z1));
    G2 = 1.0f / (1.0f + __expf(-z2));
  }
  __syncthreads();   // ssel

  const float c2 = 1.4426950408889634f / sqrtf((float)D);
  const uint16_t* kh = kt + (int64_t)h * N * D;
  const uint16_t* vh = vt_g + (int64_t)h * N * D;
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  Branch<DB> br;

  // ---- ball branch: the ball holding this group (group | ball) ----------
  {
    branch_init<D>(br);
    const int64_t b0 = ((int64_t)g * group / ball) * ball;
    for (int k0 = 0; k0 < ball; k0 += kChunk) {
      const int nkb = min(kChunk, ball - k0) / 32;
      attend_chunk<D, NT>(kh, vh, [&](int kb) -> int64_t { return b0 + k0 + kb * 32; }, nkb,
                          qf, c2, br, vts);
    }
    branch_merge<D>(br, G0, acc);
  }
  // ---- compression branch: every coarse token ---------------------------
  {
    branch_init<D>(br);
    const uint16_t* kch = kcb + (int64_t)h * nc * D;
    const uint16_t* vch = vcb + (int64_t)h * nc * D;
    for (int k0 = 0; k0 < nc; k0 += kChunk) {
      const int nkb = min(kChunk, nc - k0) / 32;
      attend_chunk<D, NT>(kch, vch, [&](int kb) -> int64_t { return (int64_t)k0 + kb * 32; },
                          nkb, qf, c2, br, vts);
    }
    branch_merge<D>(br, G1, acc);
  }
  // ---- selection branch: the union of the selected blocks ---------------
  {
    branch_init<D>(br);
    const int nsel = topk * block;
    for (int k0 = 0; k0 < nsel; k0 += kChunk) {
      const int nkb = min(kChunk, nsel - k0) / 32;
      attend_chunk<D, NT>(kh, vh,
                          [&](int kb) -> int64_t {
                            const int idx = k0 + kb * 32;
                            return (int64_t)ssel[idx / block] * block + (idx % block);
                          },
                          nkb, qf, c2, br, vts);
    }
    branch_merge<D>(br, G2, acc);
  }

  // ---- store: lane owns d = db*32 + 8*gq + 4*hf + 0..3 of query c -------
  uint16_t* orow = out + pq * rs + (int64_t)h * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[db][gq * 4 + 0], acc[db][gq * 4 + 1]);
      pk[1] = pack_bf16x2(acc[db][gq * 4 + 2], acc[db][gq * 4 + 3]);
      *(u32x2*)(orow + db * 32 + gq * 8 + hf * 4) = pk;
    }
}

// ------------------------------------------------------------------ host ----
template <int D>
static void launch_fused(int nwv, dim3 grid, hipStream_t st, const uint16_t* q,
                         const int32_t* perm, const uint16_t* kt, const uint16_t* vt,
                         const uint16_t* kcb, const uint16_t* vcb, const int32_t* sel,
                         const float* gw, const float* gb, const float* gc, int32_t H, int64_t N,
                         int32_t nc, int32_t ngroups, int32_t ball, int32_t block, int32_t topk,
                         int32_t xmap, uint16_t* out) {
  const float g0 = gc ? gc[0] : 0.f, g1 = gc ? gc[1] : 0.f, g2 = gc ? gc[2] : 0.f;
#define BT_FUSED(NW)                                                                          \
  case NW:                                                                                    \
    hipLaunchKernelGGL((bsa_fused<D, NW>), grid, dim3(NW * 64), 0, st, q, perm, kt, vt, kcb, \
                       vcb, sel, gw, gb, g0, g1, g2, H, N, nc, ngroups, ball, block, topk,   \
                       xmap, out);                                                            \
    break;
  switch (nwv) {
    BT_FUSED(1)
    BT_FUSED(2)
    BT_FUSED(4)
    BT_FUSED(8)
    default:
      break;
  }
#undef BT_FUSED
}

bt_status bsa_launch(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                     int32_t H, int32_t d, const bsa_params* p, const float* gate_w,
                     const float* gate_b, const float* gate_const, int32_t* sel_out, void* ws,
                     void* out, hipStream_t st) {
  const BsaLayout L = bsa_layout(N, H, d, p);
  char* b = (char*)ws;
  uint16_t* kt = (uint16_t*)(b + L.kt);
  uint16_t* vt = (uint16_t*)(b + L.vt);
  float* kc32 = (float*)(b + L.kc32);
  uint16_t* kcb = (uint16_t*)(b + L.kcb);
  uint16_t* vcb = (uint16_t*)(b + L.vcb);
  float* qbar = (float*)(b + L.qbar);
  int32_t* sel = sel_out ? sel_out : (int32_t*)(b + L.sel);
  const int32_t nc = (int32_t)(N / p->block), ngroups = (int32_t)(N / p->group);
  const int cols = H * d / 8;
  const int slice = cols < 64 ? cols : 64;
  const dim3 pblk(256);

  // K: tree-ordered copy, fp32 and bf16 block means; V: copy and bf16 means;
  // Q: fp32 group means (the pooled queries that score the blocks)
  const dim3 gk(nc, (cols + slice - 1) / slice), gq(ngroups, (cols + slice - 1) / slice);
  hipLaunchKernelGGL((bsa_pool<true, true, true>), gk, pblk, 0, st, (const uint16_t*)k, perm, H,
                     d, p->block, N, kt, kc32, kcb);
  hipLaunchKernelGGL((bsa_pool<true, false, true>), gk, pblk, 0, st, (const uint16_t*)v, perm, H,
                     d, p->block, N, vt, (float*)nullptr, vcb);
  hipLaunchKernelGGL((bsa_pool<false, true, false>), gq, pblk, 0, st, (const uint16_t*)q, perm,
                     H, d, p->group, N, (uint16_t*)nullptr, qbar, (uint16_t*)nullptr);
  bt_status s = launch_status("bsa_pool");
  if (s != BT_OK) return s;

  int tg = 8192 / nc;                  // scores of a tile: <= 32 KB of LDS
  if (tg > 16) tg = 16;
  if (tg < 1) tg = 1;
  const size_t smem = (size_t)(tg * d + tg * nc) * sizeof(float);
  const dim3 gs((ngroups + tg - 1) / tg, H);
  if (d == 32)
    hipLaunchKernelGGL(bsa_select<32>, gs, dim3(256), smem, st, qbar, kc32, H, nc, ngroups, tg,
                       p->group, p->ball, p->block, p->topk, p->mask_own_ball, sel);
  else
    hipLaunchKernelGGL(bsa_select<64>, gs, dim3(256), smem, st, qbar, kc32, H, nc, ngroups, tg,
                       p->group, p->ball, p->block, p->topk, p->mask_own_ball, sel);
  s = launch_status("bsa_select");
  if (s != BT_OK) return s;

  const int nwv = p->group / 32;
  const int total = ngroups * H;
  const int xmap = (total % 8 == 0) ? 1 : 0;
  if (d == 32)
    launch_fused<32>(nwv, dim3(total), st, (const uint16_t*)q, perm, kt, vt, kcb, vcb, sel, gate_w,
                     gate_b, gate_const, H, N, nc, ngroups, p->ball, p->block, p->topk, xmap,
                     (uint16_t*)out);
  else
    launch_fused<64>(nwv, dim3(total), st, (const uint16_t*)q, perm, kt, vt, kcb, vcb, sel, gate_w,
                     gate_b, gate_const, H, N, nc, ngroups, p->ball, p->block, p->topk, xmap,
                     (uint16_t*)out);
  return launch_status("bsa_fused");
}

}  // namespace bt
