// Stage 2 device body (ragged front-packing and capture-tier rounding),
// shared by the pack launch and the launch that also builds the attention
// plan.  DSpark-in-SGLang page, section A2 "ragged verify over a full CUDA
// graph" and Fig. 2: each request's window is front-packed into one compact
// buffer in a cu_seqlens-style variable-length layout (no per-request
// padding) and only the total is rounded up to the nearest captured tier.
//
// One workgroup of kScanThreads: an exclusive scan of the windows gives cu[],
// the tier lookup gives M_pad, then every request writes its rows' metadata
// (request, position, token, KV slot through the device page table).
#pragma once

#include "rv_common.h"

namespace rv {
namespace {

struct PackParams {
  const int32_t* w;
  const int32_t* anchor;
  const int32_t* drafts;
  const int32_t* ctx;
  const int32_t* page_table;
  int32_t* cu;
  int32_t* mm;
  int32_t* row_req;
  int32_t* row_pos;
  int32_t* tok;
  int32_t* slot;
  int32_t* status;
  int B, gamma, max_pages, page_size, num_pages, n_tiers;
  int tiers[RV_MAX_TIERS];
};

// every thread of the (kScanThreads) workgroup calls this
__device__ __forceinline__ void pack_body(const PackParams& p) {
  constexpr int kThreads = kScanThreads;
  __shared__ int s_buf[kScanWaves];
  __shared__ int s_M, s_Mpad;
  const int t = threadIdx.x;
  const int B = p.B;
  const int seg = (B + kThreads - 1) / kThreads;
  const int i0 = t * seg;

  int local[8];
  int run = 0;
  for (int s = 0; s < seg; ++s) {
    const int i = i0 + s;
    int w = 0;
    if (i < B) {
      w = p.w[i];
      if (w < 1 || w > p.gamma) {
        set_status(p.status, RV_DEV_BAD_WINDOW);
        w = w < 1 ? 1 : p.gamma;
      }
    }
    local[s] = w;
    run += w;
  }
  int v1[1] = {run}, ex1[1], tot1[1];
  block_excl_scan<1>(v1, ex1, tot1, s_buf);
  int pre = ex1[0];
  if (t == kThreads - 1) {
    const int M = tot1[0];
    int Mpad = M;
    if (p.n_tiers > 0) {
      int found = -1;
      for (int k = 0; k < p.n_tiers; ++k)
        if (p.tiers[k] >= M) { found = p.tiers[k]; break; }
      if (found < 0) set_status(p.status, RV_DEV_TIER_OVERFLOW);
      else Mpad = found;
    }
    s_M = M;
    s_Mpad = Mpad;
    p.mm[0] = M;
    p.mm[1] = Mpad;
    p.cu[B] = M;
  }

  const int g1 = p.gamma - 1;
  const int P = p.page_size;
  for (int s = 0; s < seg; ++s) {
    const int i = i0 + s;
    if (i >= B) break;
    p.cu[i] = pre;
    const int c = p.ctx[i];
    const int w = local[s];
    // all loads of the request first (the stores could alias them, which
    // would otherwise serialise one round trip per row)
    int pgv[RV_MAX_GAMMA], tokv[RV_MAX_GAMMA];
#pragma unroll
    for (int k = 0; k < RV_MAX_GAMMA; ++k) {
      pgv[k] = -1;
      tokv[k] = -1;
      if (k < w) {
        const int pos = c + k;
        const int pg_idx = pos / P;
        if (pos >= 0 && pg_idx < p.max_pages) pgv[k] = p.page_table[(size_t)i * p.max_pages + pg_idx];
        tokv[k] = (k == 0) ? p.anchor[i] : p.drafts[(size_t)i * g1 + (k - 1)];
      }
    }
#pragma unroll
    for (int k = 0; k < RV_MAX_GAMMA; ++k) {
      if (k >= w) break;
      const int r = pre + k;
      const int pos = c + k;
      const int pg = pgv[k];
      int sl = -1;
      if (pg >= 0 && pg < p.num_pages) sl = pg * P + pos % P;
      else set_status(p.status, RV_DEV_BAD_PAGE);
      p.row_req[r] = i;
      p.row_pos[r] = pos;
      p.tok[r] = tokv[k];
      p.slot[r] = sl;
    }
    pre += w;
  }
  __syncthreads();
  for (int r = s_M + t; r < s_Mpad; r += kThreads) {
    p.row_req[r] = -1;
    p.row_pos[r] = -1;
    p.tok[r] = -1;
    p.slot[r] = -1;
  }
}

}  // namespace

inline PackParams make_pack_params(const rv_pack_args& a) {
  PackParams p;
  p.w = a.w_verify;
  p.anchor = a.anchor;
  p.drafts = a.drafts;
  p.ctx = a.ctx;
  p.page_table = a.page_table;
  p.cu = a.cu;
  p.mm = a.mm;
  p.row_req = a.row_req;
  p.row_pos = a.row_pos;
  p.tok = a.tok;
  p.slot = a.slot;
  p.status = status_ptr(a.workspace);
  p.B = a.B;
  p.gamma = a.gamma;
  p.max_pages = a.max_pages;
  p.page_size = a.page_size;
  p.num_pages = a.num_pages;
  p.n_tiers = a.n_tiers;
  for (int k = 0; k < RV_MAX_TIERS; ++k) p.tiers[k] = k < a.n_tiers ? a.tiers[k] : 0;
  return p;
}

}  // namespace rv
