/*
 * bt.h -- C ABI of libbtsparse: ball-tree partition, ball attention and Ball
 * Sparse Attention (BSA) on AMD MI355X (gfx950).
 *
 * Conventions (all entry points)
 * ------------------------------
 * - Every call returns a bt_status.  Arguments are validated on the host
 *   before anything is launched; a rejected call returns BT_EINVAL and
 *   launches nothing.  A failed launch returns BT_EHIP.  bt_last_error()
 *   gives a human-readable detail of the last failure on the calling thread.
 * - Every call that launches work is asynchronous on `stream` (a hipStream_t
 *   passed as void*; NULL = the null stream).  No call synchronises the
 *   stream or copies between host and device.
 * - Ownership: every tensor argument is device memory owned by the caller.
 *   The library allocates nothing; calls that need scratch memory take a
 *   caller-provided workspace whose size is given by the matching
 *   *_workspace_size function.  Calls are stateless; concurrent calls on
 *   different streams need different workspaces.
 * - Layouts: coords is [N,3] fp32 row-major.  q, k, v and out are [N,H,d]
 *   row-major and contiguous, in ORIGINAL point order when a permutation is
 *   given and in tree order when perm == NULL.  perm[t] is the original index
 *   of the point at tree position t (int32).
 * - Element types: BT_F32 (fp32 arithmetic throughout) or BT_BF16 (bf16
 *   inputs and output, fp32 accumulation and softmax).
 */
#ifndef BT_H
#define BT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BT_OK = 0,
  BT_EINVAL = 1,   /* bad argument; nothing was launched */
  BT_EHIP = 2,     /* the HIP runtime reported an error at launch */
  BT_ENOMEM = 3,   /* workspace smaller than *_workspace_size() */
} bt_status;

typedef enum { BT_F32 = 0, BT_BF16 = 1 } bt_dtype;

typedef enum { BT_GATHER = 0, BT_SCATTER = 1 } bt_perm_mode;

/* BSA hyper-parameters: ball = local attention ball size, block = compression
 * and selection block size (l), group = contiguous query group size (g),
 * topk = selected blocks per group (k*), mask_own_ball = 1 to exclude blocks
 * inside the group's own ball(s) from selection, query_compression = 1 for
 * BSA with group compression (queries pooled before the compression and
 * selection branches; see bsa_attn). */
typedef struct {
  int32_t ball;
  int32_t block;
  int32_t group;
  int32_t topk;
  int32_t mask_own_ball;
  int32_t query_compression;
} bsa_params;

const char* bt_status_str(bt_status s);
/* Detail of the last error raised on the calling thread ("" if none). */
const char* bt_last_error(void);
/* Library version, for logs. */
const char* bt_version(void);

/* ------------------------------------------------------------------------
 * Ball tree (Erwin thread on Bluesky, posts 6/N and 9/N: a ball tree splits
 * the points recursively into nested sets of similar size and stores every
 * ball contiguously; post 15/N: the tree is built by native code).
 *
 * Split rule: at every node the axis of largest fp32 spread (max - min,
 * lowest axis on ties) is split into two equal halves; the left half holds
 * the n/2 smallest points in (coordinate, original index) order, -0.0 equal
 * to +0.0; points keep ascending original index inside each node.  The
 * result is unique and bit-reproducible.
 *
 * bt_build: coords [N,3] fp32 (device), N = leaf * 2^L with 1 <= leaf,
 *   N < 2^31; writes perm [N] int32 (device).  ws: device workspace of at
 *   least bt_build_workspace_size(N, leaf) bytes, 256-byte aligned.
 *   Coordinates must be finite (not checked here; bt_count_nonfinite is the
 *   debug check).
 *   Up to 8,192 points one workgroup builds the tree in LDS (from 1,025
 *   points straight from coords: the workspace size is then the 256-byte
 *   minimum); above that each node is split by one workgroup, streamed
 *   through two record arrays in ws (with two small arrays of node
 *   extents), until the nodes have at most 8,192 points, which one
 *   workgroup each finishes in LDS.
 *   Errors: BT_EINVAL for null pointers, N not leaf*2^L, N >= 2^31;
 *   BT_ENOMEM for a short workspace.
 * ---------------------------------------------------------------------- */
size_t bt_build_workspace_size(int64_t N, int32_t leaf);
bt_status bt_build(const float* coords, int64_t N, int32_t leaf, int32_t* perm,
                   void* ws, size_t ws_bytes, void* stream);

/* bt_count_nonfinite: the debug check of the builders' precondition.  Writes
 * to *count (a device uint32) the number of the n fp32 values x[0..n) (pass
 * coords and n = 3 N) that are NaN or infinite; 0 means the coordinates may
 * be passed to bt_build.  Asynchronous on stream: *count is cleared and then
 * accumulated by kernels on that stream, so read it after the stream.
 * Errors: BT_EINVAL for n < 0, a null count (or a null x with n > 0), or a
 * count that is not 4-byte aligned. */
bt_status bt_count_nonfinite(const float* x, int64_t n, uint32_t* count, void* stream);

/* bt_rotate_build: the second tree of a rotated pair (Erwin thread: trees are
 * rotated instead of shifting windows, so that alternate layers exchange
 * information across balls).  The tree is built on x' = R x with R a 3x3
 * row-major fp32 matrix in HOST memory; each product and sum is rounded to
 * fp32 separately: x'_a = ((R[a][0]*x + R[a][1]*y) + R[a][2]*z).  R must be
 * finite (orthogonality is not checked).  Same arguments and errors as
 * bt_build otherwise. */
bt_status bt_rotate_build(const float* coords, int64_t N, int32_t leaf,
                          const float* R_host, int32_t* perm, void* ws,
                          size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Permutation of rows (Erwin thread, post 9/N: tree-ordered storage; the
 * rotated pair moves features from one tree order to the other).
 * GATHER:  dst[t]       = src[perm[t]]
 * SCATTER: dst[perm[t]] = src[t]
 * Rows are row_bytes bytes (a multiple of 4; multiples of 16 use 128-bit
 * accesses).  src and dst are device buffers of N rows that must not
 * overlap; perm must be a permutation of 0..N-1 (not checked).
 * Errors: BT_EINVAL for null pointers, N < 0, bad row_bytes, src == dst.
 * ---------------------------------------------------------------------- */
bt_status bt_permute(const void* src, const int32_t* perm, int64_t N,
                     int64_t row_bytes, bt_perm_mode mode, void* dst,
                     void* stream);

/* inv[perm[t]] = t for t < N (device buffers). */
bt_status bt_invert_perm(const int32_t* perm, int64_t N, int32_t* inv,
                         void* stream);

/* ------------------------------------------------------------------------
 * Backward pass of ball attention (the layers around it are learned: Pith
 * review of arXiv 2506.12541, "What carries the argument"; Erwin thread,
 * post 7/N).  For the output gradient dout of ball_attn(q, k, v, perm, ...),
 * per ball and head, with S = Q K^T / sqrt(d), P = softmax(S), O = P V:
 *   D_i = dO_i . O_i,  dS = P * (dO V^T - D),
 *   dq = dS K / sqrt(d),  dk = dS^T Q / sqrt(d),  dv = P^T dO,
 * in the inputs' order (original order when perm != NULL).  O is recomputed,
 * so the forward output is not an argument.  Outputs in dt.  bf16 with d = 32
 * and ball in {32, 64, 128}, or d = 64 and ball in {32, 64}, runs the MFMA
 * kernel (bf16 operands with P and dS rounded to bf16; fp32 softmax
 * statistics and accumulation); every other shape runs in fp32 arithmetic.
 * Requirements: as ball_attn, with ball <= 1024; dq, dk, dv must not alias
 * the inputs or each other.  N = 0 is a no-op.  Errors: BT_EINVAL for a
 * violated requirement or a null pointer with N > 0; BT_EHIP if the launch
 * fails.  Asynchronous on stream; nothing is allocated.
 * ---------------------------------------------------------------------- */
bt_status ball_attn_bwd(const void* q, const void* k, const void* v,
                        const void* dout, const int32_t* perm, int64_t N,
                        int32_t ball, int32_t H, int32_t d, bt_dtype dt,
                        void* dq, void* dk, void* dv, void* stream);

/* ------------------------------------------------------------------------
 * Coarsening and refinement (Erwin thread, post 8/N: the ball tree is
 * coarsened and then refined while the attention ball size stays fixed;
 * post 9/N: every level is contiguous, so these are means over consecutive
 * tree positions).  Features are [N,H,d] rows of dtype dt; row(t) = perm[t]
 * when perm != NULL (features in original order), else t (tree order).
 *   bt_coarsen: out[j] = mean_{r < s} x[row(j*s + r)] for j < N/s; out is the
 *               coarse level [N/s,H,d] in tree order (fp32 sums in a fixed
 *               order, rounded once to dt).
 *   bt_refine:  out[row(t)] = xc[t / s] for t < N (xc: [N/s,H,d]).
 * Requirements: s >= 1 divides N; H, d >= 1; a row (H*d elements) a multiple
 * of 16 bytes; N*H*d < 2^31; device buffers, 16-byte aligned, out not
 * overlapping the input.  N = 0 is a no-op.  Errors: BT_EINVAL for a
 * violated requirement or a null pointer with N > 0; BT_EHIP if a launch
 * fails.  Asynchronous on stream; nothing is allocated.
 * ---------------------------------------------------------------------- */
bt_status bt_coarsen(const void* x, const int32_t* perm, int64_t N, int32_t H,
                     int32_t d, int32_t s, bt_dtype dt, void* out, void* stream);
bt_status bt_refine(const void* xc, const int32_t* perm, int64_t N, int32_t H,
                    int32_t d, int32_t s, bt_dtype dt, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Ball attention (Erwin thread, post 7/N: attention inside the balls of a
 * chosen tree level, all balls in parallel; Pith review of arXiv 2506.12541,
 * "What carries the argument": scaled dot-product attention within each
 * ball).  For every ball b (tree positions [b*ball, (b+1)*ball)) and head h:
 *   O = softmax(Q_b K_b^T / sqrt(d)) V_b,
 * no mask, no bias, non-causal.  out[perm[t]] = O[t] (out in the same order
 * and dtype as the inputs).
 * Requirements: ball >= 1 divides N; 1 <= H; d in {16, 32, 64};
 * ball <= 4096; N*H*d < 2^31; out does not alias q, k or v; perm (when
 * given) 16-byte aligned.  N = 0 is a no-op (pointers are not used).  Errors: BT_EINVAL for a violated
 * requirement or a null pointer with N > 0; BT_EHIP if the launch fails.
 * bf16 with d in {32, 64} and ball a multiple of 32 up to 256 runs the MFMA
 * kernel; every other supported shape runs the fp32-VALU kernel.
 * ---------------------------------------------------------------------- */
bt_status ball_attn(const void* q, const void* k, const void* v,
                    const int32_t* perm, int64_t N, int32_t ball, int32_t H,
                    int32_t d, bt_dtype dt, void* out, void* stream);

/* ------------------------------------------------------------------------
 * Uneven point counts (Erwin thread, post 6/N: the sets are of similar size;
 * post 9/N: equal contiguous balls make ball operations views and means).
 * The padded tree of N points has S = bt_padded_size(N, leaf) slots, the
 * smallest leaf * 2^L >= N.  At every node of m points the split axis is
 * chosen as in bt_build and the left child takes the ceil(m/2) smallest
 * points in (coordinate, index) order; a leaf stores its points first, in
 * ascending index, and -1 in its unused slots.  For N = leaf * 2^L this is
 * exactly bt_build.
 *
 * bt_padded_size: S, or -1 when N < 1, leaf < 1 or S >= 2^31.
 * bt_build_padded: coords [N,3] fp32 (device); R_host NULL (no rotation) or
 *   a finite 3x3 row-major fp32 rotation in host memory, applied as in
 *   bt_rotate_build; writes perm [S] int32 (device).  ws: device workspace of
 *   bt_build_padded_workspace_size(N, leaf) bytes, 256-byte aligned (the
 *   256-byte minimum up to 8,192 slots, which one workgroup builds in LDS;
 *   two record arrays of N points above that, built as bt_build does).
 *   Errors: BT_EINVAL for null pointers or a violated limit, BT_ENOMEM for a
 *   short workspace.
 * bt_permute_padded: perm has n_slots entries, negative for an unused slot,
 *   the others row indices below n_rows (not checked beyond clamping).
 *   GATHER:  dst[t] = src[perm[t]] (dst [n_slots] rows, src [n_rows] rows),
 *            a zero row for an unused slot;
 *   SCATTER: dst[perm[t]] = src[t] for the used slots (src [n_slots] rows,
 *            dst [n_rows] rows; rows no slot names are left unchanged).
 *   Requirements: 1 <= n_rows <= n_slots < 2^31 (n_slots = 0 is a no-op);
 *   row_bytes a positive multiple of 4; src and dst do not overlap.
 * ball_attn_padded: ball attention on a padded tree: q, k, v, out [n_rows,
 *   H, d] in original order; perm [n_slots] as above (required); the keys of
 *   a ball are its used slots, and out[perm[t]] is written for every used
 *   slot t only.  Requirements: ball | n_slots; 1 <= n_rows <= n_slots;
 *   perm 16-byte aligned; otherwise as ball_attn.  Errors: BT_EINVAL for a violated requirement or
 *   a null pointer; BT_EHIP if the launch fails.
 * All three are asynchronous on stream and allocate nothing.
 * ---------------------------------------------------------------------- */
int64_t bt_padded_size(int64_t N, int32_t leaf);
size_t bt_build_padded_workspace_size(int64_t N, int32_t leaf);
bt_status bt_build_padded(const float* coords, int64_t N, int32_t leaf,
                          const float* R_host, int32_t* perm, void* ws,
                          size_t ws_bytes, void* stream);
bt_status bt_permute_padded(const void* src, const int32_t* perm,
                            int64_t n_rows, int64_t n_slots, int64_t row_bytes,
                            bt_perm_mode mode, void* dst, void* stream);
bt_status ball_attn_padded(const void* q, const void* k, const void* v,
                           const int32_t* perm, int64_t n_rows, int64_t n_slots,
                           int32_t ball, int32_t H, int32_t d, bt_dtype dt,
                           void* out, void* stream);

/* ------------------------------------------------------------------------
 * Ball Sparse Attention (Pith review of arXiv 2506.12541: "What carries the
 * argument", "Core claim", Figure 1 and Figure 3 captions; referee report
 * major comments 1 and 2, Eqs. 10-15).  In tree order:
 *   O_ball: ball attention with ball size p->ball;
 *   Kc, Vc: means of K, V over contiguous blocks of p->block positions;
 *   O_cmp:  softmax(q Kc^T / sqrt(d)) Vc over all N/block coarse tokens;
 *   s[g,h,j] = mean_{t in group g}(q_t) . Kc_j / sqrt(d) in fp32; blocks
 *           overlapping a ball that holds a position of g are excluded when
 *           p->mask_own_ball; the p->topk best blocks are kept (ties to the
 *           smaller block index);
 *   O_slc:  each query of g attends once over the union of its selected
 *           blocks at full resolution;
 *   with p->query_compression (group compression: the pages' optional
 *   coarsening step that pools queries before selection and compression,
 *   "Core claim"; Eq. 15 over Q_cmp): O_cmp of a token is the attention of
 *   its block's mean query over all coarse tokens, and O_slc of a token is
 *   the attention of its group's mean query over the group's selected
 *   blocks (the block-mean queries are rounded to bf16 for the MFMA; the
 *   group-mean query's selection attention runs in fp32);
 *   out = G0*O_ball + G1*O_cmp + G2*O_slc with G = sigmoid(W q + b)
 *         (gate_w [3,d] fp32 device, gate_b [3] fp32 device or NULL for 0),
 *         or G = gate_const (host [3]) when gate_w == NULL.
 * sel_out (device [H, N/group, topk] int32, or NULL) receives the selected
 * blocks of every group and head, best first.
 * Requirements: dt == BT_BF16; d in {32, 64}; perm non-NULL; ball and block
 * multiples of 32 with ball <= 256, block | ball and ball | N; group in
 * {32, 64, 128, 256} with group | ball; N/block a multiple of 32 and
 * <= 8192; 1 <= topk <= 64 and topk <= N/block minus the masked blocks of a
 * group; exactly one of gate_w and gate_const non-NULL; query_compression 0
 * or 1.
 * ws: device workspace of at least bsa_workspace_size() bytes.
 * ---------------------------------------------------------------------- */
size_t bsa_workspace_size(int64_t N, int32_t H, int32_t d, const bsa_params* p);
bt_status bsa_attn(const void* q, const void* k, const void* v,
                   const int32_t* perm, int64_t N, int32_t H, int32_t d,
                   bt_dtype dt, const bsa_params* p, const float* gate_w,
                   const float* gate_b, const float* gate_const_host,
                   int32_t* sel_out, void* ws, size_t ws_bytes, void* out,
                   void* stream);

/* ------------------------------------------------------------------------
 * bsa_attn without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same computation, arguments, requirements and errors
 * as bsa_attn, without the workspace arguments: the workspace is a static
 * device array of bsa_attn_noalloc_max_bytes() bytes (80 MiB) that the
 * library holds on every GPU it runs on until the process ends.  A call whose
 * bsa_workspace_size() exceeds it returns BT_EINVAL (the BSA workload of
 * 65,536 points, 8 heads of 32 needs 67.5 MiB, 70.5 MiB with group
 * compression).  Calls on one GPU share the array: calls that overlap on one
 * GPU (other streams, other threads) race.  Allocates nothing; asynchronous
 * on stream.
 * ---------------------------------------------------------------------- */
size_t bsa_attn_noalloc_max_bytes(void);
bt_status bsa_attn_noalloc(const void* q, const void* k, const void* v,
                           const int32_t* perm, int64_t N, int32_t H, int32_t d,
                           bt_dtype dt, const bsa_params* p,
                           const float* gate_w, const float* gate_b,
                           const float* gate_const_host, int32_t* sel_out,
                           void* out, void* stream);

/* ------------------------------------------------------------------------
 * Backward of BSA without group compression (the branches and the gates are
 * learned: Pith review of arXiv 2506.12541, "What carries the argument").
 * For the output gradient dout [N,H,d] (original order, bf16) it writes
 *   dq, dk, dv [N,H,d] bf16 in original order, and with learned gates
 *   dgate_w [3,d] and dgate_b [3] (fp32 device; either may be NULL to skip
 *   it; both must be NULL with gate_const).
 * Every branch is softmax attention with output gradient G_i dout; the
 * gates give dG_i = dout . O_i and, when learned, dz_i = dG_i G_i (1 - G_i)
 * with dq += sum_i dz_i W[i], dW[i] = sum_{t,h} dz_i q_{t,h} and db[i] =
 * sum_{t,h} dz_i.  Compression passes dKc[j] / block to every token of block
 * j; selected blocks collect the gradient of every group that selected them.
 * The top-k selection passes no gradient: it is recomputed exactly as the
 * forward's and held fixed.  The softmax weights, their products with dP,
 * dS and G*P are rounded to bf16 for the matrix products; everything else
 * accumulates in fp32.
 * Arguments and requirements as bsa_attn, plus p->query_compression == 0;
 * dq, dk and dv must not overlap each other or q, k, v, dout, and must be
 * 16-byte aligned.  ws: device workspace of at least
 * bsa_attn_bwd_workspace_size() bytes (0 for invalid parameters), 256-byte
 * aligned.  Errors: BT_EINVAL for a violated requirement or a null pointer;
 * BT_ENOMEM for a short workspace; BT_EHIP if a launch fails.  Asynchronous
 * on stream; allocates nothing.
 * ---------------------------------------------------------------------- */
size_t bsa_attn_bwd_workspace_size(int64_t N, int32_t H, int32_t d,
                                   const bsa_params* p);
bt_status bsa_attn_bwd(const void* q, const void* k, const void* v,
                       const int32_t* perm, const void* dout, int64_t N,
                       int32_t H, int32_t d, bt_dtype dt, const bsa_params* p,
                       const float* gate_w, const float* gate_b,
                       const float* gate_const_host, void* dq, void* dk,
                       void* dv, float* dgate_w, float* dgate_b, void* ws,
                       size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BT_H */
