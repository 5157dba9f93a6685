// Stage 5: compact scatter of the committed tokens and KV slots.
//
// DSpark-in-SGLang page, section A2 "performance and zero-overhead
// scheduling": small per-step ops, among them the compact scatter, run as
// fused kernels, and the page table stays on the device so no per-step host
// sync is needed.
//
// One workgroup: two exclusive scans (committed tokens a+1, released slots
// w-a-1) give every request its output offsets; each request then writes its
// committed tokens and KV slots, its req_to_token entries and history, and
// advances ctx and the anchor in place.

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kThreads = 1024;

struct ScatterParams {
  rv_scatter_args a;
  int32_t* status;
};

// rows packed for request i; cu is the authority, w_verify must agree
// (0 for a corrupt packing: such a request commits and releases nothing)
__device__ inline int rows_of(const rv_scatter_args& p, int i, int32_t* status) {
  int wv = p.cu[i + 1] - p.cu[i];
  if (wv < 1 || wv > p.gamma) wv = 0;
  if (status && wv != p.w_verify[i]) set_status(status, RV_DEV_BAD_WINDOW);
  return wv;
}

__global__ __launch_bounds__(kThreads) void k_scatter(ScatterParams sp) {
  const rv_scatter_args& p = sp.a;
  static_assert(kThreads == kScanThreads, "block_excl_scan's workgroup");
  __shared__ int s_buf[kScanWaves * 2];
  const int t = threadIdx.x;
  const int B = p.B;
  const int seg = (B + kThreads - 1) / kThreads;
  const int i0 = t * seg;
  int acc[8];
  int nc = 0, nf = 0;
  for (int s = 0; s < seg; ++s) {
    const int i = i0 + s;
    int a = 0;
    if (i < B) {
      const int wv = rows_of(p, i, sp.status);
      a = p.accept[i];
      if (wv == 0) {
        a = -1;
      } else if (a < 0 || a > wv - 1) {
        set_status(sp.status, RV_DEV_BAD_WINDOW);
        a = a < 0 ? 0 : wv - 1;
      }
      nc += a + 1;
      nf += wv - a - 1;
    }
    acc[s] = a;
  }
  int v2[2] = {nc, nf}, ex2[2], tot2[2];
  block_excl_scan<2>(v2, ex2, tot2, s_buf);
  int co = ex2[0];
  int fo = ex2[1];
  if (t == kThreads - 1) {
    p.commit_cu[B] = tot2[0];
    p.free_count[0] = tot2[1];
  }
  const int g1 = p.gamma - 1;
  for (int s = 0; s < seg; ++s) {
    const int i = i0 + s;
    if (i >= B) break;
    const int a = acc[s];
    const int wv = rows_of(p, i, nullptr);
    const int base = p.cu[i];
    const int c = p.ctx[i];
    const int b = p.bonus[i];
    p.commit_cu[i] = co;
    const bool r2t_ok = c >= 0 && c + a < p.r2t_stride;
    int hl = 0;
    bool hist_ok = false;
    if (p.hist) {
      hl = p.hist_len[i];
      hist_ok = hl >= 0 && hl + a < p.hist_stride;
    }
    if (!r2t_ok || (p.hist && !hist_ok)) set_status(sp.status, RV_DEV_HIST_OVERFLOW);
    // all loads of the request first (the stores could alias them, which
    // would otherwise serialise one round trip per row)
    int tokv[RV_MAX_GAMMA], slv[RV_MAX_GAMMA];
#pragma unroll
    for (int j = 0; j < RV_MAX_GAMMA; ++j) {
      tokv[j] = b;
      slv[j] = -1;
      if (j < wv) {
        slv[j] = p.slot[base + j];
        if (j < a) tokv[j] = p.drafts[(size_t)i * g1 + j];
      }
    }
#pragma unroll
    for (int j = 0; j < RV_MAX_GAMMA; ++j) {
      if (j > a) break;
      p.commit_tok[co + j] = tokv[j];
      p.commit_slot[co + j] = slv[j];
      if (r2t_ok) p.req_to_token[(size_t)i * p.r2t_stride + c + j] = slv[j];
      if (hist_ok) p.hist[(size_t)i * p.hist_stride + hl + j] = tokv[j];
    }
#pragma unroll
    for (int j = 0; j < RV_MAX_GAMMA; ++j)
      if (j > a && j < wv) p.free_slots[fo + (j - a - 1)] = slv[j];
    if (a < 0) continue;   // corrupt packing: state left unchanged
    if (p.hist) p.hist_len[i] = hl + a + 1;
    p.ctx[i] = c + a + 1;
    p.anchor[i] = b;
    co += a + 1;
    fo += wv - a - 1;
  }
}

}  // namespace

hipError_t launch_scatter(const rv_scatter_args& a, hipStream_t s) {
  ScatterParams sp;
  sp.a = a;
  sp.status = status_ptr(a.workspace);
  hipLaunchKernelGGL(k_scatter, dim3(1), dim3(kThreads), 0, s, sp);
  return hipGetLastError();
}

}  // namespace rv
