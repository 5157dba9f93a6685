// rv_lm_head_accept_noalloc: the LM head + accept with its scratch memory in
// a static device array instead of a caller workspace, for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid allocation).
//
// The slab partials of the LM head (16 bytes per packed row and 64-column
// vocabulary slab) live in `scratch`, one copy per GPU, held until the process
// ends.  Host code never uses the array's name as an address: on the first
// call on a device, with that device current, hipGetSymbolAddress gives the
// device address of that GPU's copy, which is kept per device and passed to
// the kernels.  Every call on one GPU shares its copy, so calls that overlap
// on one GPU (concurrent streams, or threads) race on it.

#include <mutex>

#include "rv_common.h"

namespace rv {

// 64 MiB: the latent batch (2048 packed rows of vocabulary 129280) needs
// 63.1 MiB of slab partials plus the status header.
constexpr size_t kNoAllocScratchBytes = RV_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];   // device address of each GPU's copy of scratch

// The current device's copy of `scratch`, looked up once per device.
rv_status scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RV_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return RV_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_addr[dev]);
  return RV_OK;
}

}  // namespace
}  // namespace rv

using namespace rv;

extern "C" rv_status rv_lm_head_accept_noalloc(const rv_lm_args* a, void* stream) {
  const rv_status st = lm_args_check(a);
  if (st != RV_OK) return st;
  if (a->workspace && a->workspace_bytes < (size_t)kStatusBytes) return RV_ERR_WORKSPACE;
  const size_t need = kStatusBytes + lm_scratch_bytes(a->B, a->gamma, a->V);
  if (need > kNoAllocScratchBytes) return RV_ERR_SCRATCH;
  char* base = nullptr;
  const rv_status sst = scratch_of_current_device(&base);
  if (sst != RV_OK) return sst;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* status = status_ptr(a->workspace);
  if (status == nullptr) {
    // no status word from the caller: the header of scratch takes it,
    // cleared first (it keeps the previous call's value)
    status = status_ptr(base);
    if (launch_clear_status(base, s) != hipSuccess) return RV_ERR_HIP;
  }
  return launch_lm(*a, base + kStatusBytes, status, s) == hipSuccess ? RV_OK : RV_ERR_HIP;
}
