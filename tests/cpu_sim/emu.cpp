#include "hip/hip_runtime.h"
thread_local Idx threadIdx, blockIdx;
Idx blockDim, gridDim;
EmuBlock* g_blk;
unsigned char* g_dyn_lds;
std::vector<EmuMfmaSlot> g_mfma;

void emu_launch(dim3 grid, dim3 block, size_t shm, const std::function<void()>& body) {
  std::vector<unsigned char> dyn(shm + 16);
  g_dyn_lds = dyn.data();
  const unsigned nt = block.x;
  g_mfma.assign(((nt + 63) / 64) * 64, EmuMfmaSlot{});
  gridDim = {grid.x, grid.y, grid.z};
  blockDim = {block.x, block.y, block.z};
  // one host thread per emulated thread, reused for every workgroup of the
  // launch; workgroups run one after another
  std::barrier<> outer(nt + 1);
  std::vector<std::unique_ptr<EmuBlock>> blocks;
  const unsigned nblk = grid.x * grid.y * grid.z;
  for (unsigned b = 0; b < nblk; ++b) {
    auto eb = std::make_unique<EmuBlock>();
    eb->block_bar = std::make_unique<std::barrier<>>(nt);
    for (unsigned w = 0; w < (nt + 63) / 64; ++w)
      eb->wave_bar.push_back(std::make_unique<std::barrier<>>(std::min(64u, nt - 64 * w)));
    eb->xch.assign(nt, 0);
    blocks.push_back(std::move(eb));
  }
  // With EMU_SHUFFLE=<seed> the workgroups run in a seeded random order (a
  // different order in every launch): results must not depend on it.
  std::vector<unsigned> order(nblk);
  for (unsigned b = 0; b < nblk; ++b) order[b] = b;
  if (const char* sh = getenv("EMU_SHUFFLE")) {
    static unsigned long long state = 0;
    if (state == 0) state = 0x9e3779b97f4a7c15ull ^ strtoull(sh, nullptr, 10);
    for (unsigned b = nblk; b > 1; --b) {        // Fisher-Yates, splitmix64 draws
      unsigned long long z = (state += 0x9e3779b97f4a7c15ull);
      z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
      z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
      z ^= z >> 31;
      std::swap(order[b - 1], order[z % b]);
    }
  }
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([&, t]() {
      for (unsigned bi = 0; bi < nblk; ++bi) {
        outer.arrive_and_wait();                 // workgroup order[bi] may start
        const unsigned b = order[bi];
        threadIdx = {t, 0, 0};
        blockIdx = {b % grid.x, (b / grid.x) % grid.y, b / (grid.x * grid.y)};
        body();
        // a finished thread leaves this workgroup's barriers
        g_blk->block_bar->arrive_and_drop();
        g_blk->wave_bar[t / 64]->arrive_and_drop();
        outer.arrive_and_wait();                 // workgroup b done
      }
    });
  for (unsigned bi = 0; bi < nblk; ++bi) {
    g_blk = blocks[order[bi]].get();
    outer.arrive_and_wait();
    outer.arrive_and_wait();
  }
  for (auto& x : th) x.join();
}
