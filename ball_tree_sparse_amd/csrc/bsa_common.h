// Pieces of Ball Sparse Attention shared by the forward and backward
// kernels: workspace layout, the transposed-block key order and the
// online-softmax attention over 32-key blocks read straight from the
// tree-ordered K and transposed V.
#pragma once
#include <type_traits>

#include "common.h"

namespace bt {

constexpr int kChunk = 64;             // keys per online-softmax step
constexpr int kSelRegs = 16;           // scores per lane held in registers by select
constexpr int kSelThreads = 512;       // select: eight waves, one group of a tile each
constexpr float kLazyLog2 = 8.0f;      // online softmax: rescale only past 2^8
constexpr float kBoundLog2 = 48.0f;    // largest bound taken as the fixed softmax shift
constexpr int kLChains = 2;            // chains of the softmax normaliser

struct BsaLayout {
  size_t kt, vt, kc32, kcb, vcb, qbar, sel;   // vt, vcb: transposed blocks
  size_t kbmax, kmax2;                        // largest squared key norm: per block, per head
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
  L.kbmax = o; o = a256(o + nc * H * 4);
  L.kmax2 = o; o = a256(o + (size_t)H * 4);
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

// x combined with its value in lane ^ 32, through gfx950's v_permlane32_swap
// (a VALU exchange of the wave's two halves) rather than an LDS permute.
// With both operands x, the swap returns each lane's own value and its
// partner's, so the max and the sum are the same in both lanes of a pair.
BT_DEV float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
BT_DEV float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
// sums those rounded weights (kLChains chains, lane-local until the merge).
template <int DB>
struct Branch {
  f32x16 o[DB];
  float m;      // running max in log2-scaled units (-inf before the first chunk)
  float l[kLChains];   // partial sums of the rounded weights
  s16x4 shf;    // shift_frag(m)
};

// The scores reach the exponential without a pass over them on the VALU:
// the queries are multiplied by log2(e)/sqrt(d) before their rounding to bf16
// (scale_query), so S^T = K Q^T is already in log2 units, and the running
// maximum m is subtracted inside the MFMAs (shift_frag, common.h).
//
// BND: m is fixed before the first chunk at a bound on every score of the
// query, |q| * max_k |k| (Cauchy-Schwarz; the mean of keys is no longer than
// the longest key, so the compressed tokens are covered too), and the chunks
// take no maximum and never rescale.

// Fragments of NKB 32-key blocks: block kb's keys are rows row0(kb) ..
// row0(kb)+31 of the head's row-major K (kh) and of its transposed V blocks
// (vh: [rows/32][D][32]); row0(kb) is a multiple of 32.  kf are A operands of
// S^T = K Q^T, vf A operands of O^T = V^T P^T.
template <int D, int NKB, typename RowFn>
BT_DEV void load_kfrags(const uint16_t* __restrict__ kh, RowFn row0, bf16x8 (&kf)[NKB][D / 16]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const uint16_t* krow = kh + (row0(kb) + c) * D + hf * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) kf[kb][s] = *(const bf16x8*)(krow + s * 16);
  }
}
template <int D, int NKB, typename RowFn>
BT_DEV void load_vfrags(const uint16_t* __restrict__ vh, RowFn row0,
                        bf16x8 (&vf)[NKB][2][D / 32]) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, c = lane & 31;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const uint16_t* vblk = vh + row0(kb) * D + c * 32 + hf * 8;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        vf[kb][s2][db] = *(const bf16x8*)(vblk + db * 32 * 32 + s2 * 16);
  }
}

// S^T of NKB key blocks for one query block (qf: its D/16 B-operand
// fragments of scaled queries), shifted by -m (not on the branch's first
// chunk, FIRST, unless m is a fixed bound, BND).
template <int D, int NKB, bool FIRST, bool BND = false>
BT_DEV void chunk_scores(const bf16x8 (&kf)[NKB][D / 16], const bf16x8* qf,
                         const Branch<D / 32>& b, f32x16 (&sacc)[NKB]) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    f32x16 a = {};
    if constexpr (!FIRST || BND)
      a = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ones_frag(), b.shf, a, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][s], qf[s], a, 0, 0, 0);
    sacc[kb] = a;
  }
}

// The online-softmax update of one query block's branch state with the
// chunk's scores, and O^T += V^T P^T.  FIRST: the branch's first chunk (its
// maximum sets m; nothing is accumulated yet).  BND: m is a fixed bound and
// the update is the weights alone.
template <int D, int NKB, bool FIRST, bool BND = false>
BT_DEV void chunk_softmax_pv(f32x16 (&sacc)[NKB], const bf16x8 (&vf)[NKB][2][D / 32],
                             Branch<D / 32>& b) {
  constexpr int DB = D / 32;
  if constexpr (!BND) {
    // chunk maximum of the shifted scores (of the scores on the first chunk)
    float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) m4[e & 3] = fmaxf(m4[e & 3], sacc[kb][e]);
    const float cm = xor32_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
    // The running maximum is raised (and the state rescaled) only when a
    // chunk maximum exceeds it by more than kLazyLog2, for every lane of the
    // wave at once; the weights then stay below 2^kLazyLog2, and the
    // normalised result is the same up to rounding.
    if (FIRST || __ballot(cm > kLazyLog2)) {
      float delta;                                  // taken off this chunk's scores
      if constexpr (FIRST) {
        delta = cm;
        b.m = cm;
      } else {
        const float mn = b.m + fmaxf(cm, 0.f);
        delta = mn - b.m;
        const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
        for (int i = 0; i < kLChains; ++i) b.l[i] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) b.o[db][e] *= alpha;
        b.m = mn;
      }
      b.shf = shift_frag(b.m);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] -= delta;
    }
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (__bf16)__builtin_amdgcn_exp2f(sacc[kb][s2 * 8 + e]);
      b.l[(kb * 2 + s2) % kLChains] = bsa_sum8(pf, b.l[(kb * 2 + s2) % kLChains]);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        b.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kb][s2][db], pf, b.o[db], 0, 0, 0);
    }
}

// One online-softmax step over NKB 32-key blocks for QB query blocks of 32
// (qf: QB x D/16 fragments, br: QB branch states), its fragments loaded here.
// Every K and V fragment of the chunk serves all QB query blocks, so the
// cache traffic per query falls by QB.
template <int D, int NKB, int QB, bool FIRST, bool BND, typename RowFn>
BT_DEV void attend_chunk(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                         RowFn row0, const bf16x8* qf, Branch<D / 32>* br) {
  bf16x8 kf[NKB][D / 16], vf[NKB][2][D / 32];
  load_kfrags<D, NKB>(kh, row0, kf);
  load_vfrags<D, NKB>(vh, row0, vf);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    f32x16 sacc[NKB];
    chunk_scores<D, NKB, FIRST, BND>(kf, qf + qb * (D / 16), br[qb], sacc);
    chunk_softmax_pv<D, NKB, FIRST, BND>(sacc, vf, br[qb]);
  }
}

// Online softmax over keys [0, len) of a branch (len a multiple of 32);
// row0(key) gives the row of the 32-key block at key.  Full kChunk-key chunks
// are software-pipelined without extra registers: the next chunk's K
// fragments are requested as soon as the last query block's score MFMAs have
// taken theirs, and its V fragments once the last P V MFMAs have, so each
// load is in flight while part of a chunk is computed.  A tail of 32-key
// blocks follows unpipelined.
template <int D, int QB, bool BND = false, typename RowFn>
BT_DEV void attend_range(const uint16_t* __restrict__ kh, const uint16_t* __restrict__ vh,
                         RowFn row0, int len, const bf16x8* qf, Branch<D / 32>* br) {
  constexpr int KB = kChunk / 32, DS = D / 16;
  const int nfull = len / kChunk;
  int k0 = 0;
  if (nfull > 0) {
    bf16x8 kf[KB][DS], vf[KB][2][D / 32];
    load_kfrags<D, KB>(kh, [&](int kb) -> int64_t { return row0(kb * 32); }, kf);
    load_vfrags<D, KB>(vh, [&](int kb) -> int64_t { return row0(kb * 32); }, vf);
    // The loads are unconditional (the last chunk requests itself again,
    // from the cache, and the values go unused): with loads under a branch
    // the compiler's wait counts at the loop head also covered the V loads
    // just issued.
    auto step = [&](auto first, int ci) {
      constexpr bool FIRST = decltype(first)::value;
      const int kn = min(ci + 1, nfull - 1) * kChunk;   // the next chunk's first key
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        f32x16 sacc[KB];
        chunk_scores<D, KB, FIRST, BND>(kf, qf + qb * DS, br[qb], sacc);
        if (qb == QB - 1)                      // the last scores have taken kf
          load_kfrags<D, KB>(kh, [&](int kb) -> int64_t { return row0(kn + kb * 32); }, kf);
        chunk_softmax_pv<D, KB, FIRST, BND>(sacc, vf, br[qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      load_vfrags<D, KB>(vh, [&](int kb) -> int64_t { return row0(kn + kb * 32); }, vf);
    };
    step(std::true_type{}, 0);
    for (int ci = 1; ci < nfull; ++ci) step(std::false_type{}, ci);
    k0 = nfull * kChunk;
  }
  if (k0 < len) {                            // a tail of 32-key blocks
    if (k0 == 0)
      attend_chunk<D, 1, QB, true, BND>(kh, vh, [&](int kb) -> int64_t { return row0(0); }, qf,
                                        br);
    else
      attend_chunk<D, 1, QB, false, BND>(kh, vh, [&](int kb) -> int64_t { return row0(k0); },
                                         qf, br);
    for (k0 += 32; k0 < len; k0 += 32)
      attend_chunk<D, 1, QB, false, BND>(kh, vh, [&](int kb) -> int64_t { return row0(k0); },
                                         qf, br);
  }
}

// The lane's part of a branch's normaliser (the chains added in order).
template <int DB>
BT_DEV float branch_l(const Branch<DB>& br) {
  float l = br.l[0];
#pragma unroll
  for (int i = 1; i < kLChains; ++i) l += br.l[i];
  return l;
}

template <int D>
BT_DEV void branch_init(Branch<D / 32>& br) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) br.o[db] = f32x16{};
  br.m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kLChains; ++i) br.l[i] = 0.f;
  br.shf = s16x4{0, 0, 0, 0};
}
// A branch whose shift is fixed at the bound m (BND).
template <int D>
BT_DEV void branch_init_bound(Branch<D / 32>& br, float m) {
  branch_init<D>(br);
  br.m = m;
  br.shf = shift_frag(m);
}

template <int D>
BT_DEV void branch_merge(const Branch<D / 32>& br, float gate, f32x16* acc) {
  const float l = xor32_sum(branch_l(br));
  const float f = gate * __builtin_amdgcn_rcpf(l);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = fmaf(br.o[db][e], f, acc[db][e]);
}


}  // namespace bt
