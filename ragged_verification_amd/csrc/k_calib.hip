// Observability: calibration of the draft confidences against the target's
// per-token verdicts (DSpark-in-SGLang page, section A2 "observability and
// ceiling recovery": per-request confidence and calibration metrics such as
// ECE).  Only verified drafts carry a verdict: the scheduled window under
// compact, the whole block under cap-accept.
//
// One workgroup: each thread takes whole requests, counts its verified and
// matching drafts, and adds each draft to its confidence bin in LDS (32-bit
// counts, 64-bit fixed-point confidence sums: integer atomics, so the sums
// are exact and independent of order).  The ECE numerator is an exact int64
// reduction over the bins; the two fp64 divides follow in a fixed order.

#include <math.h>

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kCalThreads = 256;
constexpr int kCalFixShift = 48;

struct CalibParams {
  const float* conf;
  const int32_t* drafts;
  const int32_t* pred;
  const int32_t* cu;
  const int32_t* w_verify;
  int B, gamma, rows_cap, n_bins;
  int64_t* bin_count;
  int64_t* bin_match;
  int64_t* bin_conf_fx;
  double* ece;
  int32_t* req_verified;
  int32_t* req_matched;
  int32_t* status;
};

__global__ __launch_bounds__(kCalThreads) void k_calibration(CalibParams p) {
  __shared__ unsigned s_count[RV_MAX_CALIB_BINS];
  __shared__ unsigned s_match[RV_MAX_CALIB_BINS];
  __shared__ unsigned long long s_conf[RV_MAX_CALIB_BINS];
  __shared__ unsigned long long s_num[kCalThreads / 64];
  __shared__ unsigned s_n[kCalThreads / 64];
  const int tid = threadIdx.x;
  for (int b = tid; b < p.n_bins; b += kCalThreads) {
    s_count[b] = 0u;
    s_match[b] = 0u;
    s_conf[b] = 0ull;
  }
  __syncthreads();
  const int g1 = p.gamma - 1;
  const double scale = (double)(1ll << kCalFixShift);
  for (int i = tid; i < p.B; i += kCalThreads) {
    const int w = p.w_verify[i];
    int nv = 0, nm = 0;
    if (w < 1 || w > p.gamma) {
      set_status(p.status, RV_DEV_BAD_WINDOW);
    } else {
      const int c0 = p.cu[i];
      for (int j = 1; j < w; ++j) {
        const int r = c0 + j - 1;
        if (r < 0 || r >= p.rows_cap) {
          set_status(p.status, RV_DEV_BAD_WINDOW);
          break;
        }
        const double c = (double)p.conf[(size_t)i * g1 + j - 1];
        const int label = p.drafts[(size_t)i * g1 + j - 1] == p.pred[r] ? 1 : 0;
        int b = (int)floor(c * (double)p.n_bins);
        b = b < 0 ? 0 : (b > p.n_bins - 1 ? p.n_bins - 1 : b);
        atomicAdd(&s_count[b], 1u);
        if (label) atomicAdd(&s_match[b], 1u);
        atomicAdd(&s_conf[b], (unsigned long long)floor(c * scale));
        ++nv;
        nm += label;
      }
    }
    if (p.req_verified) p.req_verified[i] = nv;
    if (p.req_matched) p.req_matched[i] = nm;
  }
  __syncthreads();
  // bins out; ECE numerator sum_b |match_b * 2^48 - conf_b| as an exact int64
  unsigned long long num = 0ull;
  unsigned n = 0u;
  for (int b = tid; b < p.n_bins; b += kCalThreads) {
    const long long m = (long long)s_match[b] << kCalFixShift;
    const long long cf = (long long)s_conf[b];
    num += (unsigned long long)(m > cf ? m - cf : cf - m);
    n += s_count[b];
    p.bin_count[b] = s_count[b];
    p.bin_match[b] = s_match[b];
    p.bin_conf_fx[b] = cf;
  }
  for (int off = 32; off > 0; off >>= 1) {
    num += __shfl_xor(num, off);
    n += __shfl_xor(n, off);
  }
  if ((tid & 63) == 0) {
    s_num[tid >> 6] = num;
    s_n[tid >> 6] = n;
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long tot = 0ull;
    unsigned nn = 0u;
    for (int k = 0; k < kCalThreads / 64; ++k) {
      tot += s_num[k];
      nn += s_n[k];
    }
    p.ece[0] = nn ? ((double)tot / scale) / (double)nn : 0.0;
  }
}

}  // namespace

hipError_t launch_calibration(const rv_calib_args& a, hipStream_t s) {
  CalibParams p;
  p.conf = a.conf;
  p.drafts = a.drafts;
  p.pred = a.pred;
  p.cu = a.cu;
  p.w_verify = a.w_verify;
  p.B = a.B;
  p.gamma = a.gamma;
  p.rows_cap = a.rows_cap;
  p.n_bins = a.n_bins;
  p.bin_count = a.bin_count;
  p.bin_match = a.bin_match;
  p.bin_conf_fx = a.bin_conf_fx;
  p.ece = a.ece;
  p.req_verified = a.req_verified;
  p.req_matched = a.req_matched;
  p.status = status_ptr(a.workspace);
  hipLaunchKernelGGL(k_calibration, dim3(1), dim3(kCalThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace rv
