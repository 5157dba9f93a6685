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
  __shared__ int sc_c[kThreads], sc_f[kThreads];
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
  sc_c[t] = nc;
  sc_f[t] = nf;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int x = t >= off ? sc_c[t - off] : 0;
    const int y = t >= off ? sc_f[t - off] : 0;
    __syncthreads();
    sc_c[t] += x;
    sc_f[t] += y;
    __syncthreads();
  }
  int co = sc_c[t] - nc;
  int fo = sc_f[t] - nf;
  if (t == kThreads - 1) {
    p.commit_cu[B] = sc_c[t];
    p.free_count[0] = sc_f[t];
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
    for (int j = 0; j <= a; ++j) {
      const int tok = (j < a) ? p.drafts[(size_t)i * g1 + j] : b;
      const int sl = p.slot[base + j];
      p.commit_tok[co + j] = tok;
      p.commit_slot[co + j] = sl;
      if (r2t_ok) p.req_to_token[(size_t)i * p.r2t_stride + c + j] = sl;
      if (hist_ok) p.hist[(size_t)i * p.hist_stride + hl + j] = tok;
    }
    for (int j = a + 1; j < wv; ++j) p.free_slots[fo + (j - a - 1)] = p.slot[base + j];
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
