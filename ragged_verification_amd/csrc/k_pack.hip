// Stage 2: ragged front-packing and capture-tier rounding (the device body
// is in pack_body.h; DSpark-in-SGLang page, section A2 "ragged verify over a
// full CUDA graph" and Fig. 2).

#include "pack_body.h"

namespace rv {
namespace {

__global__ __launch_bounds__(kScanThreads) void k_pack(PackParams p) { pack_body(p); }

}  // namespace

hipError_t launch_pack(const rv_pack_args& a, hipStream_t s) {
  hipLaunchKernelGGL(k_pack, dim3(1), dim3(kScanThreads), 0, s, make_pack_params(a));
  return hipGetLastError();
}

}  // namespace rv
