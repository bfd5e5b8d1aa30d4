// Runs the ball_attn.hip, ball_attn_bwd.hip, bsa.hip and bsa_bwd.hip kernels
// on the host under the SIMT emulation.  Inputs and outputs are raw files in
// the working directory (q.bin, k.bin, v.bin, perm.bin, w.bin, b.bin, do.bin
// -> out.bin, sel.out, dq.bin, dk.bin, dv.bin, dw.bin, db.bin).
#include <cstdarg>
#include "hip/hip_runtime.h"
#include "../../ball_tree_sparse_amd/csrc/common.h"
namespace bt {
void set_error(const char* fmt, ...) { va_list ap; va_start(ap, fmt); vfprintf(stderr, fmt, ap); va_end(ap); }
bt_status launch_status(const char*) { return BT_OK; }
}
// Built twice (the two builds run in parallel): with BT_SIM_BSA_BWD only the
// BSA backward, otherwise the rest.
#ifdef BT_SIM_BSA_BWD
#include "../../ball_tree_sparse_amd/csrc/bsa.hip"
#include "../../ball_tree_sparse_amd/csrc/bsa_bwd.hip"
#else
#include "../../ball_tree_sparse_amd/csrc/ball_attn.hip"
#include "../../ball_tree_sparse_amd/csrc/bsa.hip"
#include "../../ball_tree_sparse_amd/csrc/ball_attn_bwd.hip"
#endif

template <typename T> std::vector<T> rd(const char* p, size_t n) {
  std::vector<T> v(n); FILE* f = fopen(p, "rb"); fread(v.data(), sizeof(T), n, f); fclose(f); return v; }
template <typename T> void wr(const char* p, const std::vector<T>& v) {
  FILE* f = fopen(p, "wb"); fwrite(v.data(), sizeof(T), v.size(), f); fclose(f); }

int main(int argc, char** argv) {
  // mode N H d ball dt [block group topk mask gatemode]
  std::string mode = argv[1];
  long long N = atoll(argv[2]); int H = atoi(argv[3]), d = atoi(argv[4]), ball = atoi(argv[5]);
  int dt = atoi(argv[6]);
  size_t ne = (size_t)N * H * d, es = dt == BT_F32 ? 4 : 2;
  auto q = rd<unsigned char>("q.bin", ne * es), k = rd<unsigned char>("k.bin", ne * es),
       v = rd<unsigned char>("v.bin", ne * es);
  const long long nslots = mode == "ball_padded" ? atoll(argv[7]) : N;
  auto perm = rd<int32_t>("perm.bin", nslots);
  std::vector<unsigned char> out(ne * es, 0xcd);
#ifdef BT_SIM_BSA_BWD
  if (mode == "bsa_bwd") {
    // ... block group topk mask gatemode (0: W and b, 1: gates (0.3, 0.5, 0.7),
    // 2 + i: gate i alone)
    bsa_params p{ball, atoi(argv[7]), atoi(argv[8]), atoi(argv[9]), atoi(argv[10]), 0};
    const int gm = atoi(argv[11]);
    auto dout = rd<unsigned char>("do.bin", ne * es);
    auto W = rd<float>("w.bin", 3 * d);
    auto Bv = rd<float>("b.bin", 3);
    float gc[3] = {0.3f, 0.5f, 0.7f};
    if (gm >= 2)
      for (int i = 0; i < 3; ++i) gc[i] = i == gm - 2 ? 1.f : 0.f;
    std::vector<unsigned char> g[3];
    for (auto& x : g) x.assign(ne * es, 0xcd);
    std::vector<float> dw(3 * d, -7.f), db(3, -7.f);
    const size_t ws = bt::bsa_bwd_ws_size(N, H, d, &p);
    void* w = nullptr;
    if (posix_memalign(&w, 256, ws) != 0) return 2;
    memset(w, 0xab, ws);
    bt::bsa_bwd_launch(q.data(), k.data(), v.data(), perm.data(), dout.data(), N, H, d, &p,
                       gm == 0 ? W.data() : nullptr, gm == 0 ? Bv.data() : nullptr,
                       gm == 0 ? nullptr : gc, g[0].data(), g[1].data(), g[2].data(),
                       gm == 0 ? dw.data() : nullptr, gm == 0 ? db.data() : nullptr, w, nullptr);
    free(w);
    wr("dq.bin", g[0]);
    wr("dk.bin", g[1]);
    wr("dv.bin", g[2]);
    wr("dw.bin", dw);
    wr("db.bin", db);
    printf("done bsa_bwd\n");
    return 0;
  }
  return 3;
#else
  if (mode == "bwd") {
    auto dout = rd<unsigned char>("do.bin", ne * es);
    std::vector<unsigned char> g[3];
    for (auto& x : g) x.assign(ne * es, 0xcd);
    bt::ball_attn_bwd_launch(q.data(), k.data(), v.data(), dout.data(), perm.data(), N, ball, H,
                             d, (bt_dtype)dt, g[0].data(), g[1].data(), g[2].data(), nullptr);
    wr("dq.bin", g[0]);
    wr("dk.bin", g[1]);
    wr("dv.bin", g[2]);
    printf("done bwd %d\n", (int)bt::ball_attn_bwd_uses_mfma((bt_dtype)dt, ball, d));
    return 0;
  }
  if (mode == "ball_padded") {
    bt::ball_attn_padded_launch(q.data(), k.data(), v.data(), perm.data(), N, nslots, ball, H, d,
                                (bt_dtype)dt, out.data(), nullptr);
  } else if (mode == "ball" || mode == "ball_noperm") {
    bt::ball_attn_launch(q.data(), k.data(), v.data(), mode == "ball" ? perm.data() : nullptr, N,
                         ball, H, d, (bt_dtype)dt, out.data(), nullptr);
  } else {
    bsa_params p{ball, atoi(argv[7]), atoi(argv[8]), atoi(argv[9]), atoi(argv[10]),
                 argc > 12 ? atoi(argv[12]) : 0};
    int gm = atoi(argv[11]);
    auto W = rd<float>("w.bin", 3 * d);
    float gc[3] = {1, 0, 0};
    if (gm == 2) { gc[0] = 0; gc[1] = 1; }
    if (gm == 3) { gc[0] = 0; gc[2] = 1; }
    size_t ws = bt::bsa_ws_size(N, H, d, &p);
    // exactly ws bytes (a multiple of 256), filled with garbage
    void* w = nullptr;
    if (posix_memalign(&w, 256, ws) != 0) return 2;
    memset(w, 0xab, ws);
    std::vector<int32_t> sel((size_t)H * (N / p.group) * p.topk, -1);
    bt::bsa_launch(q.data(), k.data(), v.data(), perm.data(), N, H, d, &p,
                   gm == 0 ? W.data() : nullptr, nullptr, gm == 0 ? nullptr : gc, sel.data(), w,
                   out.data(), nullptr);
    wr("sel.out", sel);
    free(w);
  }
  wr("out.bin", out);
  printf("done %s\n", mode.c_str());
  return 0;
#endif
}
