// BSA without allocation: bsa_attn with its workspace in a file-scope device
// array, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` exists once per GPU the library runs on and is held
// until the process ends.  Host code never uses its name as an address: the
// device address is looked up once per device with hipGetSymbolAddress (with
// that device current) and kept per device; kernels receive that pointer.
// Every call on one GPU shares the array and it keeps the last call's
// contents (bsa_attn writes every workspace byte it reads, so nothing needs
// clearing); calls that overlap on one GPU (different streams or threads)
// race on it.
#include <mutex>

#include "common.h"

namespace bt {

// Largest workspace served: the BSA workload of 65,536 points, 8 heads of 32
// (with or without group compression) needs 67.5 / 70.5 MiB.
constexpr size_t kScratchBytes = (size_t)80 << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this device's copy of `scratch` (looked up on the first
// call on the device, with the device current).
static bt_status scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("bsa_attn_noalloc: no usable current device (%d)", dev);
    return BT_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("bsa_attn_noalloc: hipGetSymbolAddress failed: %s", hipGetErrorString(e));
      return BT_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return BT_OK;
}

}  // namespace bt

using namespace bt;

extern "C" {

size_t bsa_attn_noalloc_max_bytes(void) { return kScratchBytes; }

bt_status bsa_attn_noalloc(const void* q, const void* k, const void* v, const int32_t* perm,
                           int64_t N, int32_t H, int32_t d, bt_dtype dt, const bsa_params* p,
                           const float* gate_w, const float* gate_b,
                           const float* gate_const_host, int32_t* sel_out, void* out,
                           void* stream) {
  // bsa_workspace_size is 0 for invalid parameters: bsa_attn reports those
  const size_t need = bsa_workspace_size(N, H, d, p);
  if (need > kScratchBytes) {
    set_error("bsa_attn_noalloc: this call needs %zu bytes of workspace, the static scratch "
              "holds %zu",
              need, kScratchBytes);
    return BT_EINVAL;
  }
  void* ws = nullptr;
  if (need > 0) {
    const bt_status s = scratch_address(&ws);
    if (s != BT_OK) return s;
  }
  return bsa_attn(q, k, v, perm, N, H, d, dt, p, gate_w, gate_b, gate_const_host, sel_out, ws,
                  kScratchBytes, out, stream);
}

}  // extern "C"
