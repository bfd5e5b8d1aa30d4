// C ABI of libbtsparse: host-side validation, workspace sizing and launches.
// Every argument check runs before any HIP call, so a rejected call never
// touches the device (and can be exercised on a machine without a GPU).
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace bt {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

bt_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return BT_EHIP;
  }
  return BT_OK;
}

// implemented in the kernel units
size_t tree_workspace_size(int64_t n, int leaf);
bt_status tree_build_launch(const float* coords, int64_t n, int leaf, const float* R,
                            int32_t* perm, void* ws, hipStream_t st);
bt_status permute_launch(const void* src, const int32_t* perm, int64_t n, int64_t row_bytes,
                         bt_perm_mode mode, void* dst, hipStream_t st);
bt_status invert_perm_launch(const int32_t* perm, int64_t n, int32_t* inv, hipStream_t st);
bt_status count_nonfinite_launch(const float* x, int64_t n, uint32_t* count, hipStream_t st);
bt_status ball_attn_launch(const void* q, const void* k, const void* v, const int32_t* perm,
                           int64_t N, int32_t ball, int32_t H, int32_t d, bt_dtype dt,
                           void* out, hipStream_t st);
size_t bsa_ws_size(int64_t N, int32_t H, int32_t d, const bsa_params* p);
bt_status ball_attn_bwd_launch(const void* q, const void* k, const void* v, const void* dout,
                               const int32_t* perm, int64_t N, int32_t ball, int32_t H,
                               int32_t d, bt_dtype dt, void* dq, void* dk, void* dv,
                               hipStream_t st);
bt_status coarsen_launch(const void* x, const int32_t* perm, int64_t N, int32_t ppr, int32_t s,
                         bt_dtype dt, void* out, hipStream_t st);
bt_status refine_launch(const void* xc, const int32_t* perm, int64_t N, int32_t ppr, int32_t s,
                        void* out, hipStream_t st);
int64_t tree_padded_slots(int64_t n, int leaf);
size_t tree_padded_workspace_size(int64_t n, int leaf);
bt_status tree_build_padded_launch(const float* coords, int64_t n, int leaf, const float* R,
                                   int32_t* perm, void* ws, hipStream_t st);
bt_status permute_padded_launch(const void* src, const int32_t* perm, int64_t nrows,
                                int64_t nslots, int64_t row_bytes, bt_perm_mode mode, void* dst,
                                hipStream_t st);
bt_status ball_attn_padded_launch(const void* q, const void* k, const void* v,
                                  const int32_t* perm, int64_t nrows, int64_t nslots,
                                  int32_t ball, int32_t H, int32_t d, bt_dtype dt, void* out,
                                  hipStream_t st);
bt_status bsa_launch(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                     int32_t H, int32_t d, const bsa_params* p, const float* gate_w,
                     const float* gate_b, const float* gate_const, int32_t* sel_out, void* ws,
                     void* out, hipStream_t st);

size_t bsa_bwd_ws_size(int64_t N, int32_t H, int32_t d, const bsa_params* p);
bt_status bsa_bwd_launch(const void* q, const void* k, const void* v, const int32_t* perm,
                         const void* dout, int64_t N, int32_t H, int32_t d, const bsa_params* p,
                         const float* gate_w, const float* gate_b, const float* gate_const,
                         void* dq, void* dk, void* dv, float* dgate_w, float* dgate_b, void* ws,
                         hipStream_t st);

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }


static bool valid_tree_shape(int64_t N, int32_t leaf) {
  return N >= 1 && leaf >= 1 && N < ((int64_t)1 << 31) && N % leaf == 0 && is_pow2(N / leaf);
}

static bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const char* x = (const char*)a;
  const char* y = (const char*)b;
  return x < y + bn && y < x + an;
}

}  // namespace bt

using namespace bt;

extern "C" {

const char* bt_status_str(bt_status s) {
  switch (s) {
    case BT_OK: return "ok";
    case BT_EINVAL: return "invalid argument";
    case BT_EHIP: return "HIP runtime error";
    case BT_ENOMEM: return "workspace too small";
  }
  return "unknown status";
}

const char* bt_last_error(void) { return g_err; }

const char* bt_version(void) { return "btsparse 0.1 (gfx950)"; }

size_t bt_build_workspace_size(int64_t N, int32_t leaf) {
  if (!valid_tree_shape(N, leaf)) return 0;
  return tree_workspace_size(N, leaf);
}

static bt_status build_common(const float* coords, int64_t N, int32_t leaf, const float* R,
                              int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  BT_REQUIRE(coords && perm, "coords and perm must be non-null");
  BT_REQUIRE(N >= 1 && leaf >= 1, "need N >= 1 and leaf >= 1 (N=%lld, leaf=%d)", (long long)N,
             leaf);
  BT_REQUIRE(N < ((int64_t)1 << 31), "N must be below 2^31");
  BT_REQUIRE(N % leaf == 0 && is_pow2(N / leaf), "N must be leaf * 2^L (N=%lld, leaf=%d)",
             (long long)N, leaf);
  BT_REQUIRE(ws != nullptr, "workspace must be non-null");
  BT_REQUIRE(((uintptr_t)ws & 255) == 0, "workspace must be 256-byte aligned");
  const size_t need = tree_workspace_size(N, leaf);
  if (ws_bytes < need) {
    set_error("workspace holds %zu bytes, bt_build needs %zu", ws_bytes, need);
    return BT_ENOMEM;
  }
  return tree_build_launch(coords, N, leaf, R, perm, ws, (hipStream_t)stream);
}

bt_status bt_build(const float* coords, int64_t N, int32_t leaf, int32_t* perm, void* ws,
                   size_t ws_bytes, void* stream) {
  return build_common(coords, N, leaf, nullptr, perm, ws, ws_bytes, stream);
}

bt_status bt_rotate_build(const float* coords, int64_t N, int32_t leaf, const float* R_host,
                          int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  BT_REQUIRE(R_host != nullptr, "rotation matrix must be non-null");
  for (int i = 0; i < 9; ++i)
    BT_REQUIRE(R_host[i] == R_host[i] && R_host[i] - R_host[i] == 0.0f,
               "rotation matrix must be finite");
  return build_common(coords, N, leaf, R_host, perm, ws, ws_bytes, stream);
}

bt_status bt_permute(const void* src, const int32_t* perm, int64_t N, int64_t row_bytes,
                     bt_perm_mode mode, void* dst, void* stream) {
  BT_REQUIRE(N >= 0, "N must be >= 0");
  BT_REQUIRE(N < ((int64_t)1 << 31), "N must be below 2^31");
  BT_REQUIRE(row_bytes > 0 && row_bytes % 4 == 0, "row_bytes must be a positive multiple of 4");
  BT_REQUIRE(mode == BT_GATHER || mode == BT_SCATTER, "mode must be BT_GATHER or BT_SCATTER");
  if (N == 0) return BT_OK;
  BT_REQUIRE(src && dst && perm, "src, dst and perm must be non-null");
  BT_REQUIRE(!overlaps(src, (size_t)(N * row_bytes), dst, (size_t)(N * row_bytes)),
             "src and dst must not overlap");
  return permute_launch(src, perm, N, row_bytes, mode, dst, (hipStream_t)stream);
}

bt_status bt_count_nonfinite(const float* x, int64_t n, uint32_t* count, void* stream) {
  BT_REQUIRE(n >= 0, "need n >= 0");
  BT_REQUIRE(count != nullptr && (x != nullptr || n == 0), "x and count must be non-null");
  BT_REQUIRE(((uintptr_t)count & 3) == 0, "count must be 4-byte aligned");
  return count_nonfinite_launch(x, n, count, (hipStream_t)stream);
}

bt_status bt_invert_perm(const int32_t* perm, int64_t N, int32_t* inv, void* stream) {
  BT_REQUIRE(N >= 0 && N < ((int64_t)1 << 31), "need 0 <= N < 2^31");
  if (N == 0) return BT_OK;
  BT_REQUIRE(perm && inv, "perm and inv must be non-null");
  BT_REQUIRE(!overlaps(perm, (size_t)N * 4, inv, (size_t)N * 4), "perm and inv must not overlap");
  return invert_perm_launch(perm, N, inv, (hipStream_t)stream);
}

// Shared checks of bt_coarsen / bt_refine; sets *ppr to the 16-byte pieces
// per row.
static bt_status check_pool(int64_t N, int32_t H, int32_t d, int32_t s, bt_dtype dt,
                            int32_t* ppr) {
  BT_REQUIRE(dt == BT_F32 || dt == BT_BF16, "dtype must be BT_F32 or BT_BF16");
  BT_REQUIRE(H >= 1 && d >= 1, "need H >= 1 and d >= 1");
  BT_REQUIRE(s >= 1 && N >= 0 && N % s == 0, "s must divide N (N=%lld, s=%d)", (long long)N, s);
  BT_REQUIRE(N * H * d < ((int64_t)1 << 31), "N*H*d must be below 2^31");
  const int64_t row = (int64_t)H * d * (dt == BT_F32 ? 4 : 2);
  BT_REQUIRE(row % 16 == 0, "a row (H*d elements) must be a multiple of 16 bytes");
  *ppr = (int32_t)(row / 16);
  return BT_OK;
}

bt_status bt_coarsen(const void* x, const int32_t* perm, int64_t N, int32_t H, int32_t d,
                     int32_t s, bt_dtype dt, void* out, void* stream) {
  int32_t ppr = 0;
  const bt_status st = check_pool(N, H, d, s, dt, &ppr);
  if (st != BT_OK) return st;
  if (N == 0) return BT_OK;
  BT_REQUIRE(x && out, "x and out must be non-null");
  BT_REQUIRE((((uintptr_t)x | (uintptr_t)out) & 15) == 0, "x and out must be 16-byte aligned");
  BT_REQUIRE(!overlaps(x, (size_t)N * ppr * 16, out, (size_t)(N / s) * ppr * 16),
             "out must not overlap x");
  return coarsen_launch(x, perm, N, ppr, s, dt, out, (hipStream_t)stream);
}

bt_status bt_refine(const void* xc, const int32_t* perm, int64_t N, int32_t H, int32_t d,
                    int32_t s, bt_dtype dt, void* out, void* stream) {
  int32_t ppr = 0;
  const bt_status st = check_pool(N, H, d, s, dt, &ppr);
  if (st != BT_OK) return st;
  if (N == 0) return BT_OK;
  BT_REQUIRE(xc && out, "xc and out must be non-null");
  BT_REQUIRE((((uintptr_t)xc | (uintptr_t)out) & 15) == 0, "xc and out must be 16-byte aligned");
  BT_REQUIRE(!overlaps(xc, (size_t)(N / s) * ppr * 16, out, (size_t)N * ppr * 16),
             "out must not overlap xc");
  return refine_launch(xc, perm, N, ppr, s, out, (hipStream_t)stream);
}

bt_status ball_attn(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                    int32_t ball, int32_t H, int32_t d, bt_dtype dt, void* out, void* stream) {
  BT_REQUIRE(dt == BT_F32 || dt == BT_BF16, "dtype must be BT_F32 or BT_BF16");
  BT_REQUIRE(d == 16 || d == 32 || d == 64, "d must be 16, 32 or 64 (d=%d)", d);
  BT_REQUIRE(H >= 1, "H must be >= 1");
  BT_REQUIRE(N >= 0 && ball >= 1 && N % ball == 0, "ball must divide N (N=%lld, ball=%d)",
             (long long)N, ball);
  BT_REQUIRE(ball <= 4096, "ball must be <= 4096");
  if (N == 0) return BT_OK;                 // no points: nothing to do
  BT_REQUIRE(q && k && v && out, "q, k, v and out must be non-null");
  BT_REQUIRE(N * H * d < ((int64_t)1 << 31), "N*H*d must be below 2^31");
  BT_REQUIRE((N / ball) * H < ((int64_t)1 << 31), "too many (ball, head) pairs");
  const size_t bytes = (size_t)(N * H * d) * (dt == BT_F32 ? 4 : 2);
  BT_REQUIRE(!overlaps(out, bytes, q, bytes) && !overlaps(out, bytes, k, bytes) &&
                 !overlaps(out, bytes, v, bytes),
             "out must not alias q, k or v");
  if (dt == BT_BF16) {
    BT_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 == 0,
               "bf16 tensors must be 16-byte aligned");
  } else {
    BT_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 4 == 0,
               "fp32 tensors must be 4-byte aligned");
  }
  // the MFMA kernel reads a ball's permutation entries 2 or 4 at a time
  BT_REQUIRE(((uintptr_t)perm & 15) == 0, "perm must be 16-byte aligned");
  return ball_attn_launch(q, k, v, perm, N, ball, H, d, dt, out, (hipStream_t)stream);
}

bt_status ball_attn_bwd(const void* q, const void* k, const void* v, const void* dout,
                        const int32_t* perm, int64_t N, int32_t ball, int32_t H, int32_t d,
                        bt_dtype dt, void* dq, void* dk, void* dv, void* stream) {
  BT_REQUIRE(dt == BT_F32 || dt == BT_BF16, "dtype must be BT_F32 or BT_BF16");
  BT_REQUIRE(d == 16 || d == 32 || d == 64, "d must be 16, 32 or 64 (d=%d)", d);
  BT_REQUIRE(H >= 1, "H must be >= 1");
  BT_REQUIRE(N >= 0 && ball >= 1 && N % ball == 0, "ball must divide N (N=%lld, ball=%d)",
             (long long)N, ball);
  BT_REQUIRE(ball <= 1024, "ball_attn_bwd takes ball <= 1024 (ball=%d)", ball);
  if (N == 0) return BT_OK;
  BT_REQUIRE(q && k && v && dout && dq && dk && dv, "tensors must be non-null");
  BT_REQUIRE(N * H * d < ((int64_t)1 << 31), "N*H*d must be below 2^31");
  BT_REQUIRE((N / ball) * H < ((int64_t)1 << 31), "too many (ball, head) pairs");
  const size_t bytes = (size_t)(N * H * d) * (dt == BT_F32 ? 4 : 2);
  const void* ins[4] = {q, k, v, dout};
  void* outs[3] = {dq, dk, dv};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      BT_REQUIRE(!overlaps(outs[o], bytes, ins[i], bytes), "gradients must not alias the inputs");
    for (int o2 = o + 1; o2 < 3; ++o2)
      BT_REQUIRE(!overlaps(outs[o], bytes, outs[o2], bytes), "dq, dk and dv must not overlap");
  }
  return ball_attn_bwd_launch(q, k, v, dout, perm, N, ball, H, d, dt, dq, dk, dv,
                              (hipStream_t)stream);
}

int64_t bt_padded_size(int64_t N, int32_t leaf) {
  if (N < 1 || leaf < 1 || N >= ((int64_t)1 << 31)) return -1;
  const int64_t s = tree_padded_slots(N, leaf);
  return s < ((int64_t)1 << 31) ? s : -1;
}

size_t bt_build_padded_workspace_size(int64_t N, int32_t leaf) {
  if (bt_padded_size(N, leaf) < 0) return 0;
  return tree_padded_workspace_size(N, leaf);
}

bt_status bt_build_padded(const float* coords, int64_t N, int32_t leaf, const float* R_host,
                          int32_t* perm, void* ws, size_t ws_bytes, void* stream) {
  BT_REQUIRE(coords && perm, "coords and perm must be non-null");
  const int64_t S = bt_padded_size(N, leaf);
  BT_REQUIRE(S > 0, "need N >= 1, leaf >= 1 and fewer than 2^31 slots (N=%lld, leaf=%d)",
             (long long)N, leaf);
  if (R_host) {
    for (int i = 0; i < 9; ++i)
      BT_REQUIRE(R_host[i] == R_host[i] && R_host[i] - R_host[i] == 0.0f,
                 "rotation matrix must be finite");
  }
  BT_REQUIRE(ws != nullptr, "workspace must be non-null");
  BT_REQUIRE(((uintptr_t)ws & 255) == 0, "workspace must be 256-byte aligned");
  const size_t need = tree_padded_workspace_size(N, leaf);
  if (ws_bytes < need) {
    set_error("workspace holds %zu bytes, bt_build_padded needs %zu", ws_bytes, need);
    return BT_ENOMEM;
  }
  return tree_build_padded_launch(coords, N, leaf, R_host, perm, ws, (hipStream_t)stream);
}

bt_status bt_permute_padded(const void* src, const int32_t* perm, int64_t n_rows,
                            int64_t n_slots, int64_t row_bytes, bt_perm_mode mode, void* dst,
                            void* stream) {
  BT_REQUIRE(n_slots >= 0 && n_slots < ((int64_t)1 << 31), "need 0 <= n_slots < 2^31");
  BT_REQUIRE(row_bytes > 0 && row_bytes % 4 == 0, "row_bytes must be a positive multiple of 4");
  BT_REQUIRE(mode == BT_GATHER || mode == BT_SCATTER, "mode must be BT_GATHER or BT_SCATTER");
  if (n_slots == 0) return BT_OK;
  BT_REQUIRE(n_rows >= 1 && n_rows <= n_slots, "need 1 <= n_rows <= n_slots (n_rows=%lld)",
             (long long)n_rows);
  BT_REQUIRE(src && dst && perm, "src, dst and perm must be non-null");
  const size_t sb = (size_t)((mode == BT_GATHER ? n_rows : n_slots) * row_bytes);
  const size_t db = (size_t)((mode == BT_GATHER ? n_slots : n_rows) * row_bytes);
  BT_REQUIRE(!overlaps(src, sb, dst, db), "src and dst must not overlap");
  return permute_padded_launch(src, perm, n_rows, n_slots, row_bytes, mode, dst,
                               (hipStream_t)stream);
}

bt_status ball_attn_padded(const void* q, const void* k, const void* v, const int32_t* perm,
                           int64_t n_rows, int64_t n_slots, int32_t ball, int32_t H, int32_t d,
                           bt_dtype dt, void* out, void* stream) {
  BT_REQUIRE(dt == BT_F32 || dt == BT_BF16, "dtype must be BT_F32 or BT_BF16");
  BT_REQUIRE(d == 16 || d == 32 || d == 64, "d must be 16, 32 or 64 (d=%d)", d);
  BT_REQUIRE(H >= 1, "H must be >= 1");
  BT_REQUIRE(ball >= 1 && ball <= 4096, "need 1 <= ball <= 4096 (ball=%d)", ball);
  BT_REQUIRE(n_slots >= 1 && n_slots % ball == 0, "ball must divide n_slots (n_slots=%lld)",
             (long long)n_slots);
  BT_REQUIRE(n_rows >= 1 && n_rows <= n_slots, "need 1 <= n_rows <= n_slots (n_rows=%lld)",
             (long long)n_rows);
  BT_REQUIRE(q && k && v && out && perm, "q, k, v, out and perm must be non-null");
  BT_REQUIRE(n_slots * H * d < ((int64_t)1 << 31), "n_slots*H*d must be below 2^31");
  const size_t bytes = (size_t)(n_rows * H * d) * (dt == BT_F32 ? 4 : 2);
  BT_REQUIRE(!overlaps(out, bytes, q, bytes) && !overlaps(out, bytes, k, bytes) &&
                 !overlaps(out, bytes, v, bytes),
             "out must not alias q, k or v");
  if (dt == BT_BF16) {
    BT_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 == 0,
               "bf16 tensors must be 16-byte aligned");
  } else {
    BT_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 4 == 0,
               "fp32 tensors must be 4-byte aligned");
  }
  BT_REQUIRE(((uintptr_t)perm & 15) == 0, "perm must be 16-byte aligned");
  return ball_attn_padded_launch(q, k, v, perm, n_rows, n_slots, ball, H, d, dt, out,
                                 (hipStream_t)stream);
}

static bt_status check_bsa(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  BT_REQUIRE(p != nullptr, "bsa_params must be non-null");
  BT_REQUIRE(d == 32 || d == 64, "BSA supports d = 32 or 64 (d=%d)", d);
  BT_REQUIRE(H >= 1, "H must be >= 1");
  BT_REQUIRE(N >= 1 && N < ((int64_t)1 << 31) && N * H * d < ((int64_t)1 << 31),
             "N*H*d must be below 2^31");
  const int32_t ball = p->ball, block = p->block, group = p->group, topk = p->topk;
  BT_REQUIRE(ball >= 32 && block >= 32 && group >= 32 && ball % 32 == 0 && block % 32 == 0 &&
                 group % 32 == 0,
             "ball, block and group must be positive multiples of 32");
  BT_REQUIRE(ball <= 256, "ball must be <= 256");
  BT_REQUIRE(group <= 256, "group must be <= 256");
  BT_REQUIRE(N % ball == 0 && ball % block == 0 && N % group == 0,
             "need ball | N, block | ball and group | N");
  BT_REQUIRE(group == 32 || group == 64 || group == 128 || group == 256,
             "group must be 32, 64, 128 or 256");
  BT_REQUIRE(ball % group == 0, "group must divide ball");
  const int64_t nc = N / block;
  BT_REQUIRE(nc % 32 == 0 && nc <= 8192, "N/block must be a multiple of 32 and <= 8192");
  BT_REQUIRE(p->query_compression == 0 || p->query_compression == 1,
             "query_compression must be 0 or 1");
  const int64_t masked = p->mask_own_ball ? ball / block : 0;
  BT_REQUIRE(topk >= 1 && topk <= 64 && topk <= nc - masked,
             "need 1 <= topk <= 64 and topk <= N/block - masked blocks (%lld)",
             (long long)(nc - masked));
  return BT_OK;
}

size_t bsa_workspace_size(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  if (check_bsa(N, H, d, p) != BT_OK) return 0;
  return bsa_ws_size(N, H, d, p);
}

bt_status bsa_attn(const void* q, const void* k, const void* v, const int32_t* perm, int64_t N,
                   int32_t H, int32_t d, bt_dtype dt, const bsa_params* p, const float* gate_w,
                   const float* gate_b, const float* gate_const_host, int32_t* sel_out, void* ws,
                   size_t ws_bytes, void* out, void* stream) {
  BT_REQUIRE(q && k && v && out && perm, "q, k, v, perm and out must be non-null");
  BT_REQUIRE(dt == BT_BF16, "bsa_attn supports bf16 inputs");
  bt_status s = check_bsa(N, H, d, p);
  if (s != BT_OK) return s;
  BT_REQUIRE((gate_w == nullptr) != (gate_const_host == nullptr),
             "give exactly one of gate_w and gate_const");
  if (gate_const_host)
    for (int i = 0; i < 3; ++i)
      BT_REQUIRE(gate_const_host[i] == gate_const_host[i], "gate_const must not be NaN");
  const size_t bytes = (size_t)(N * H * d) * 2;
  BT_REQUIRE(!overlaps(out, bytes, q, bytes) && !overlaps(out, bytes, k, bytes) &&
                 !overlaps(out, bytes, v, bytes),
             "out must not alias q, k or v");
  BT_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 == 0,
             "bf16 tensors must be 16-byte aligned");
  BT_REQUIRE(ws != nullptr && ((uintptr_t)ws & 255) == 0,
             "workspace must be non-null and 256-byte aligned");
  const size_t need = bsa_ws_size(N, H, d, p);
  if (ws_bytes < need) {
    set_error("workspace holds %zu bytes, bsa_attn needs %zu", ws_bytes, need);
    return BT_ENOMEM;
  }
  return bsa_launch(q, k, v, perm, N, H, d, p, gate_w, gate_b, gate_const_host, sel_out, ws, out,
                    (hipStream_t)stream);
}

size_t bsa_attn_bwd_workspace_size(int64_t N, int32_t H, int32_t d, const bsa_params* p) {
  if (check_bsa(N, H, d, p) != BT_OK || p->query_compression != 0) return 0;
  return bsa_bwd_ws_size(N, H, d, p);
}

bt_status bsa_attn_bwd(const void* q, const void* k, const void* v, const int32_t* perm,
                       const void* dout, int64_t N, int32_t H, int32_t d, bt_dtype dt,
                       const bsa_params* p, const float* gate_w, const float* gate_b,
                       const float* gate_const_host, void* dq, void* dk, void* dv,
                       float* dgate_w, float* dgate_b, void* ws, size_t ws_bytes, void* stream) {
  BT_REQUIRE(q && k && v && perm && dout && dq && dk && dv,
             "q, k, v, perm, dout, dq, dk and dv must be non-null");
  BT_REQUIRE(dt == BT_BF16, "bsa_attn_bwd supports bf16 inputs");
  bt_status s = check_bsa(N, H, d, p);
  if (s != BT_OK) return s;
  BT_REQUIRE(p->query_compression == 0,
             "bsa_attn_bwd does not cover group compression (query_compression must be 0)");
  BT_REQUIRE((gate_w == nullptr) != (gate_const_host == nullptr),
             "give exactly one of gate_w and gate_const");
  BT_REQUIRE(gate_w || (dgate_w == nullptr && dgate_b == nullptr),
             "constant gates have no parameter gradients: dgate_w and dgate_b must be NULL");
  if (gate_const_host)
    for (int i = 0; i < 3; ++i)
      BT_REQUIRE(gate_const_host[i] == gate_const_host[i], "gate_const must not be NaN");
  const size_t bytes = (size_t)(N * H * d) * 2;
  const void* ins[5] = {q, k, v, dout, nullptr};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      BT_REQUIRE(!overlaps(outs[i], bytes, ins[j], bytes),
                 "dq, dk and dv must not alias q, k, v or dout");
    for (int j = i + 1; j < 3; ++j)
      BT_REQUIRE(!overlaps(outs[i], bytes, outs[j], bytes), "dq, dk and dv must not overlap");
  }
  BT_REQUIRE(((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)dout | (uintptr_t)dq |
              (uintptr_t)dk | (uintptr_t)dv) % 16 == 0,
             "bf16 tensors must be 16-byte aligned");
  BT_REQUIRE(ws != nullptr && ((uintptr_t)ws & 255) == 0,
             "workspace must be non-null and 256-byte aligned");
  const size_t need = bsa_bwd_ws_size(N, H, d, p);
  if (ws_bytes < need) {
    set_error("workspace holds %zu bytes, bsa_attn_bwd needs %zu", ws_bytes, need);
    return BT_ENOMEM;
  }
  return bsa_bwd_launch(q, k, v, perm, dout, N, H, d, p, gate_w, gate_b, gate_const_host, dq, dk,
                        dv, dgate_w, dgate_b, ws, (hipStream_t)stream);
}

}  // extern "C"
