// Runs the tree.hip kernels on the host under the SIMT emulation.
// usage: tree_sim [padded] coords.bin N leaf out.bin [R.bin]
#include <cstdarg>
#include <string>
#include "hip/hip_runtime.h"
namespace bt {
void set_error(const char* fmt, ...) { va_list ap; va_start(ap, fmt); vfprintf(stderr, fmt, ap); va_end(ap); }
}
#include "../../ball_tree_sparse_amd/csrc/tree.hip"
namespace bt { bt_status launch_status(const char*) { return BT_OK; } }

int main(int argc, char** argv) {
  // argv: [padded] coords.bin N leaf out.bin [R.bin]
  const bool padded = std::string(argv[1]) == "padded";
  if (padded) { ++argv; --argc; }
  const char* cpath = argv[1];
  long long n = atoll(argv[2]);
  int leaf = atoi(argv[3]);
  std::vector<float> coords(3 * n);
  FILE* f = fopen(cpath, "rb"); fread(coords.data(), 4, 3 * n, f); fclose(f);
  float R[9]; bool rot = argc > 5;
  if (rot) { f = fopen(argv[5], "rb"); fread(R, 4, 9, f); fclose(f); }
  if (padded) {
    const long long S = bt::tree_padded_slots(n, leaf);
    size_t ws = bt::tree_padded_workspace_size(n, leaf);
    void* w = nullptr;
    if (posix_memalign(&w, 256, ws) != 0) return 2;
#ifndef BT_SIM_UNINIT_WS
    for (size_t i = 0; i < ws; ++i) ((unsigned char*)w)[i] = (unsigned char)(i * 131 + 7);
#endif
    std::vector<int32_t> perm(S, -7);
    const bt_status st = bt::tree_build_padded_launch(coords.data(), n, leaf, rot ? R : nullptr,
                                                      perm.data(), w, nullptr);
    free(w);
    if (st != BT_OK) { fprintf(stderr, "status %d\n", (int)st); return 3; }
    f = fopen(argv[4], "wb"); fwrite(perm.data(), 4, S, f); fclose(f);
    printf("done padded n=%lld leaf=%d slots=%lld\n", n, leaf, S);
    return 0;
  }
  size_t ws = bt::tree_workspace_size(n, leaf);
  // exactly ws bytes, 256-byte aligned (ws is a multiple of 256), so that an
  // access one byte past the workspace is caught; filled with garbage, like an
  // uninitialised device buffer
  void* w = nullptr;
  if (posix_memalign(&w, 256, ws) != 0) return 2;
#ifndef BT_SIM_UNINIT_WS   // (MemorySanitizer builds track it as uninitialised instead)
  for (size_t i = 0; i < ws; ++i) ((unsigned char*)w)[i] = (unsigned char)(i * 131 + 7);
#endif
  std::vector<int32_t> perm(n, -1);
  const bt_status st = bt::tree_build_launch(coords.data(), n, leaf, rot ? R : nullptr,
                                             perm.data(), w, nullptr);
  if (st != BT_OK) { free(w); fprintf(stderr, "status %d\n", (int)st); return 3; }
  free(w);
  f = fopen(argv[4], "wb"); fwrite(perm.data(), 4, n, f); fclose(f);
  printf("done n=%lld leaf=%d ws=%zu\n", n, leaf, ws);
  return 0;
}
