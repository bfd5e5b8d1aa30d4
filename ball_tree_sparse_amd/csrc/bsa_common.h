// Pieces of Ball Sparse Attention shared by the forward and backward
// kernels: workspace layout, the transposed-block key order and the
// online-softmax attention over 32-key blocks read straight from the
// tree-ordered K and transposed V.
#pragma once
#include "common.h"

namespace bt {

constexpr int kChunk = 64;             // keys per online-softmax step
constexpr int kSelRegs = 16;           // scores per lane held in registers by select
constexpr int kSelThreads = 512;       // select: eight waves, one group of a tile each
constexpr float kLazyLog2 = 8.0f;      // online softmax: rescale only past 2^8

struct BsaLayout {
  size_t kt, vt, kc32, kcb, vcb, qbar, sel;   // vt, vcb: transposed blocks
  size_t qc, ocmp, oslc;                      // group compression only
  size_t total;
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
  if (p->query_compression) {
    L.qc = o; o = a256(o + nc * H * d * 4);
    L.ocmp = o; o = a256(o + nc * H * d * 4);
    L.oslc = o; o = a256(o + G * H * d * 4);
  }
  L.total = o;
  return L;
}


// Position of key r (0..31) inside a transposed 32-key block.  The P V
// product feeds a lane's 8 keys of P^T in the order that the S^T tile gives
// them (key = 8*(e/4) + 4*hf + e%4 within 16), which is the natural order
// with bits 2 and 3 of the key index swapped; the mapping is its own inverse.
BT_DEV int tpos(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// ----------------------------------------------------------------- fused ----
typedef __bf16 bsa_bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the eight bf16 values of an MFMA operand, added to acc.
BT_DEV float bsa_sum8(bf16x8 x, float acc) {
  const bsa_bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), one, acc, false);
}

// Running state of one branch for the lane's query column.  The softmax
// weights are rounded once to bf16 for the P V product and the normaliser
// sums those rounded weights (four chains, lane-local until the merge).
template <int DB>
struct Branch {
  f32x16 o[DB];
  float m;      // running max in log2-scaled units
  float l[4];   // partial sums of the rounded weights
};

// One online-softmax step over NKB 32-key blocks for QB query blocks of 32
// (qf: QB x D/16 B-operand fragments, br: QB branch states).  Block kb's keys
// are rows row0(kb) .. row0(kb)+31 of the head's row-major K (kh) and of its
// transposed V blocks (vh: [rows/32][D][32]); row0(kb) is a multiple of 32.
// Every K and V fragment of the chunk is requested before the first MFMA and
// then serves all QB query blocks, so the cache traffic per query falls by QB.
template <int D, int NKB, int QB, typename RowFn>
BT_DEV void attend_chunk(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                         RowFn row0, const bf16x8* qf, float c2, Branch<D / 32>* br) {
  constexpr int DS = D / 16, DB = D / 32;
  const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
  bf16x8 kf[NKB][DS], vf[NKB][2][DB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int64_t r0 = row0(kb);
    const uint16_t* krow = kh + (r0 + c) * D + hf * 8;
#pragma unroll
    for (int s = 0; s < DS; ++s) kf[kb][s] = *(const bf16x8*)(krow + s * 16);
    const uint16_t* vblk = vh + r0 * D + c * 32 + hf * 8;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        vf[kb][s2][db] = *(const bf16x8*)(vblk + db * 32 * 32 + s2 * 16);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    Branch<DB>& b = br[qb];
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 a = {};
#pragma unroll
      for (int s = 0; s < DS; ++s)
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][s], qf[qb * DS + s], a, 0, 0, 0);
      sacc[kb] = a;
    }
    // chunk maximum of the raw scores (scaling by c2 > 0 keeps the order)
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) m4[e & 3] = fmaxf(m4[e & 3], sacc[kb][e]);
    float cm = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])) * c2;
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
    // The running maximum is raised (and the state rescaled) only when a
    // chunk maximum exceeds it by more than kLazyLog2, for every lane of the
    // wave at once; the weights then stay below 2^kLazyLog2, and the
    // normalised result is the same up to rounding.
    if (__ballot(cm > b.m + kLazyLog2)) {
      const float mn = fmaxf(b.m, cm);
      const float alpha = __builtin_amdgcn_exp2f(b.m - mn);   // 0 on the first chunk
#pragma unroll
      for (int i = 0; i < 4; ++i) b.l[i] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) b.o[db][e] *= alpha;
      b.m = mn;
    }
    const float mn = b.m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kb][s2 * 8 + e], c2, -mn));
        b.l[(kb * 2 + s2) & 3] = bsa_sum8(pf, b.l[(kb * 2 + s2) & 3]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          b.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb][s2][db], pf, b.o[db], 0, 0, 0);
      }
  }
}

// Online softmax over keys [0, len) of a branch in kChunk-key chunks (len is
// a multiple of 32); row0(key) gives the row of the 32-key block at key.
template <int D, int QB, typename RowFn>
BT_DEV void attend_range(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                         RowFn row0, int len, const bf16x8* qf, float c2, Branch<D / 32>* br) {
  constexpr int KB = kChunk / 32;
  int k0 = 0;
  for (; k0 + kChunk <= len; k0 += kChunk)
    attend_chunk<D, KB, QB>(kh, vh, [&](int kb) -> int64_t { return row0(k0 + kb * 32); }, qf, c2,
                            br);
  for (; k0 < len; k0 += 32)                 // a tail of 32-key blocks
    attend_chunk<D, 1, QB>(kh, vh, [&](int kb) -> int64_t { return row0(k0); }, qf, c2, br);
}

template <int D>
BT_DEV void branch_init(Branch<D / 32>& br) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) br.o[db] = f32x16{};
  br.m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) br.l[i] = 0.f;
}

template <int D>
BT_DEV void branch_merge(const Branch<D / 32>& br, float gate, f32x16* acc) {
  float l = (br.l[0] + br.l[1]) + (br.l[2] + br.l[3]);
  l += __shfl_xor(l, 32, 64);
  const float f = gate * __builtin_amdgcn_rcpf(l);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = fmaf(br.o[db][e], f, acc[db][e]);
}


}  // namespace bt
