// Runs the rotated-pair pipeline on the host under the SIMT emulation, with
// every array in an allocation of its own (exact size, so AddressSanitizer
// reports an access one element past any of them, including between the
// tree's workspace arrays):
//   tree A = build(coords), tree B = build(R coords)
//   o1  = ball_attn(q, k, v, perm A)                  (original order)
//   qb, kb, vb = gather(q, B), gather(k, B), gather(o1, B)
//   o2b = ball_attn(qb, kb, vb, NULL)                 (tree order B)
//   o2  = scatter(o2b, B);  inv = invert(B)
// usage: pipeline_sim N leaf ball H d   (reads coords.bin R.bin q.bin k.bin
// v.bin; writes pa.bin pb.bin o1.bin o2.bin inv.bin)
#include <cstdarg>
#include <string>
#include "hip/hip_runtime.h"
#include "../../ball_tree_sparse_amd/csrc/common.h"
namespace bt {
void set_error(const char* fmt, ...) { va_list ap; va_start(ap, fmt); vfprintf(stderr, fmt, ap); va_end(ap); }
bt_status launch_status(const char*) { return BT_OK; }
}
#include "../../ball_tree_sparse_amd/csrc/tree.hip"
#include "../../ball_tree_sparse_amd/csrc/ball_attn.hip"
#include "../../ball_tree_sparse_amd/csrc/permute.hip"

// An allocation of exactly n bytes, 64-byte aligned, filled with garbage
// like an uninitialised device buffer.
static void* exact(size_t n) {
  void* p = nullptr;
  if (posix_memalign(&p, 64, n ? n : 1) != 0) { fprintf(stderr, "alloc\n"); exit(2); }
  for (size_t i = 0; i < n; ++i) ((unsigned char*)p)[i] = (unsigned char)(i * 131 + 7);
  return p;
}

static void* load(const char* path, size_t n) {
  void* p = exact(n);
  FILE* f = fopen(path, "rb");
  if (!f || fread(p, 1, n, f) != n) { fprintf(stderr, "read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

static void save(const char* path, const void* p, size_t n) {
  FILE* f = fopen(path, "wb");
  fwrite(p, 1, n, f);
  fclose(f);
}

int main(int argc, char** argv) {
  if (argc < 6) { fprintf(stderr, "usage: pipeline_sim N leaf ball H d\n"); return 2; }
  const long long n = atoll(argv[1]);
  const int leaf = atoi(argv[2]), ball = atoi(argv[3]), H = atoi(argv[4]), d = atoi(argv[5]);
  const size_t rowb = (size_t)H * d * 2, featb = (size_t)n * rowb;
  const float* coords = (const float*)load("coords.bin", (size_t)n * 12);
  float R[9];
  { FILE* f = fopen("R.bin", "rb"); if (!f || fread(R, 4, 9, f) != 9) return 2; fclose(f); }
  void* q = load("q.bin", featb);
  void* k = load("k.bin", featb);
  void* v = load("v.bin", featb);
  int32_t* pa = (int32_t*)exact((size_t)n * 4);
  int32_t* pb = (int32_t*)exact((size_t)n * 4);
  int32_t* inv = (int32_t*)exact((size_t)n * 4);
  void *o1 = exact(featb), *qb = exact(featb), *kb = exact(featb), *vb = exact(featb),
       *o2b = exact(featb), *o2 = exact(featb);

  // each tree its own workspace of exactly the size the library asks for
  const size_t wsb = bt::tree_workspace_size(n, leaf);
  void* wa = exact(wsb);
  void* wb = exact(wsb);
  int st = 0;
  st |= bt::tree_build_launch(coords, n, leaf, nullptr, pa, wa, nullptr);
  st |= bt::tree_build_launch(coords, n, leaf, R, pb, wb, nullptr);
  st |= bt::ball_attn_launch(q, k, v, pa, n, ball, H, d, BT_BF16, o1, nullptr);
  st |= bt::permute_launch(q, pb, n, (int64_t)rowb, BT_GATHER, qb, nullptr);
  st |= bt::permute_launch(k, pb, n, (int64_t)rowb, BT_GATHER, kb, nullptr);
  st |= bt::permute_launch(o1, pb, n, (int64_t)rowb, BT_GATHER, vb, nullptr);
  st |= bt::ball_attn_launch(qb, kb, vb, nullptr, n, ball, H, d, BT_BF16, o2b, nullptr);
  st |= bt::permute_launch(o2b, pb, n, (int64_t)rowb, BT_SCATTER, o2, nullptr);
  st |= bt::invert_perm_launch(pb, n, inv, nullptr);
  if (st != 0) { fprintf(stderr, "a call returned an error\n"); return 3; }
  save("pa.bin", pa, (size_t)n * 4);
  save("pb.bin", pb, (size_t)n * 4);
  save("inv.bin", inv, (size_t)n * 4);
  save("o1.bin", o1, featb);
  save("o2.bin", o2, featb);
  for (void* x : {(void*)coords, q, k, v, (void*)pa, (void*)pb, (void*)inv, o1, qb, kb, vb, o2b, o2,
                  wa, wb})
    free(x);
  printf("done pipeline n=%lld leaf=%d ws=%zu\n", n, leaf, wsb);
  return 0;
}
