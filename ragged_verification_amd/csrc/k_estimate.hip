// Observability: the block-accept estimator of the ceiling that truncation
// hides (DSpark-in-SGLang page, section A2 "the ceiling estimator under
// truncation").
//
// Compact mode verifies only the scheduled window, so what the full block
// would have accepted is not observed.  A request whose window was truncated
// and whose verified drafts were all accepted opens a probe on its
// counterfactual tail (drafts d_w .. d_{gamma-1}, proposals for positions
// ctx + w ..).  Later steps commit those positions; the row of a later step
// that predicts a committed position is the target there on the realised
// prefix (taken for the counterfactual one), and its verdict on the tail
// draft is an acceptance probability: 1 or 0 under greedy (draft equals the
// row's prediction), min(1, p(d)/q(d)) under rejection sampling.  Survival
// products of those verdicts give the expected tail; the probe closes when
// every tail position is resolved or a verdict is 0, and its estimate is
// (w - 1) + the sum of the survivals.
//
// One workgroup of 256 threads per request.  The control flow is uniform
// (every thread holds the same probe state); under the rejection rule all
// threads reduce the row's log-sum-exp for the target probability.

#include <float.h>

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kEstThreads = 256;

struct EstParams {
  const int32_t* cu;
  const int32_t* w_verify;
  const int32_t* accept;
  const int32_t* drafts;
  const int32_t* ctx;
  const int32_t* pred;
  const float* logits;
  const float* q_rows;
  int32_t* pos;
  int32_t* left;
  int32_t* done;
  int32_t* base;
  int32_t* count;
  float* S;
  float* E;
  float* last;
  double* sum;
  int32_t* tok;
  float* lq;
  int32_t* status;
  int B, gamma, rows_cap, V, rule;
};

// natural log-sum-exp of one logits row, all threads (one pass, per-thread
// running max and rescaled sum, merged in LDS)
__device__ float row_lse(const float* z, int V, float* s_m, float* s_s) {
  const int t = threadIdx.x;
  float m = -INFINITY, s = 0.f;
  for (int v = t; v < V; v += kEstThreads) {
    const float x = z[v];
    if (x > m) {
      s = s * __expf(m - x) + 1.f;   // exp(-inf) = 0 on the first element
      m = x;
    } else {
      s += __expf(x - m);
    }
  }
  __syncthreads();   // s_m / s_s free
  s_m[t] = m;
  s_s[t] = s;
  __syncthreads();
  for (int w = kEstThreads / 2; w > 0; w >>= 1) {
    if (t < w) {
      const float m2 = s_m[t + w], s2 = s_s[t + w];
      const float mm = fmaxf(s_m[t], m2);
      if (mm > -INFINITY) {
        s_s[t] = s_s[t] * __expf(s_m[t] - mm) + s2 * __expf(m2 - mm);
        s_m[t] = mm;
      }
    }
    __syncthreads();
  }
  return s_m[0] + __logf(s_s[0]);
}

__global__ __launch_bounds__(kEstThreads) void k_estimate(EstParams p) {
  __shared__ float s_m[kEstThreads], s_s[kEstThreads];
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  if (i >= p.B) return;
  const int g1 = p.gamma - 1;
  const int row0 = p.cu[i];
  const int wv = p.w_verify[i];
  const int c = p.ctx[i];
  int a = p.accept[i];
  if (wv < 1 || wv > p.gamma || a < 0 || a > wv - 1 || row0 < 0 || row0 + wv > p.rows_cap) {
    if (t == 0) set_status(p.status, RV_DEV_BAD_WINDOW);
    return;
  }

  // the probe state, identical in every thread
  int pos = p.pos[i], left = p.left[i], done = p.done[i], base = p.base[i], cnt = p.count[i];
  float S = p.S[i], E = p.E[i], lastv = p.last[i];
  double sumv = p.sum[i];
  if (left > 0 && pos <= c) left = 0;   // passed unresolved (steps skipped): dropped
  const bool greedy = (p.rule == RV_GREEDY);

  // verdict of row `row` on tail draft d whose draft log-probability is lq
  auto alpha = [&](int row, int d, float lq) -> float {
    if (greedy) return p.pred[row] == d ? 1.f : 0.f;
    if (d < 0 || d >= p.V) return 0.f;
    const float* z = p.logits + (size_t)row * p.V;
    const float lse = row_lse(z, p.V, s_m, s_s);
    return fminf(1.f, __expf(z[d] - lse - lq));
  };
  auto resolve = [&](int row, int P, int d, float lq) {
    if (left == 0 || P != pos) return;
    const float al = alpha(row, d, lq);
    S *= al;
    E += S;
    ++done;
    --left;
    ++pos;
    if (S == 0.f) left = 0;   // the tail is cut at this draft
    if (left == 0) {
      const float est = (float)base + E;
      ++cnt;
      lastv = est;
      sumv += (double)est;
    }
  };

  // rows 0..a predict positions c+1 .. c+a+1, all committed this step; the
  // open probe's tail drafts come from the state (written by an earlier
  // launch)
  for (int k = 0; k <= a; ++k)
    if (left > 0 && c + k + 1 == pos)
      resolve(row0 + k, c + k + 1, p.tok[(size_t)i * g1 + done], greedy ? 0.f : p.lq[(size_t)i * g1 + done]);
  if (left == 0 && wv < p.gamma && a == wv - 1) {
    const int n = p.gamma - wv;
    pos = c + wv;
    left = n;
    done = 0;
    base = wv - 1;
    S = 1.f;
    E = 0.f;
    // log q of tail draft j (rejection), from the step's draft distributions
    auto log_q = [&](int j, int d) -> float {
      if (greedy) return 0.f;
      if (d < 0 || d >= p.V) return 0.f;
      return __logf(p.q_rows[((size_t)i * g1 + wv - 1 + j) * p.V + d]);
    };
    // the tail drafts into the state for later steps (after every thread
    // has read the old probe's drafts)
    __syncthreads();
    for (int j = t; j < g1; j += kEstThreads) {
      const int d = j < n ? p.drafts[(size_t)i * g1 + wv - 1 + j] : 0;
      if (!greedy && j < n && (d < 0 || d >= p.V)) set_status(p.status, RV_DEV_BAD_TOKEN);
      p.tok[(size_t)i * g1 + j] = d;
      p.lq[(size_t)i * g1 + j] = j < n ? log_q(j, d) : 0.f;
    }
    // this step's row a predicts the first tail position (the bonus)
    const int d0 = p.drafts[(size_t)i * g1 + wv - 1];
    resolve(row0 + a, c + a + 1, d0, log_q(0, d0));
  }
  __syncthreads();   // every thread is done reading the old state
  if (t == 0) {
    p.pos[i] = pos;
    p.left[i] = left;
    p.done[i] = done;
    p.base[i] = base;
    p.count[i] = cnt;
    p.S[i] = S;
    p.E[i] = E;
    p.last[i] = lastv;
    p.sum[i] = sumv;
  }
}

}  // namespace

size_t estimator_state_bytes(int B, int gamma) { return (size_t)40 * B + (size_t)8 * B * (gamma - 1); }

hipError_t launch_estimate(const rv_estimate_args& a, hipStream_t s) {
  char* st = static_cast<char*>(a.state);
  const size_t B = (size_t)a.B, G = (size_t)(a.gamma - 1);
  EstParams p;
  p.cu = a.cu;
  p.w_verify = a.w_verify;
  p.accept = a.accept;
  p.drafts = a.drafts;
  p.ctx = a.ctx;
  p.pred = a.pred;
  p.logits = a.logits;
  p.q_rows = a.q_rows;
  p.pos = reinterpret_cast<int32_t*>(st);
  p.left = reinterpret_cast<int32_t*>(st + 4 * B);
  p.done = reinterpret_cast<int32_t*>(st + 8 * B);
  p.base = reinterpret_cast<int32_t*>(st + 12 * B);
  p.count = reinterpret_cast<int32_t*>(st + 16 * B);
  p.S = reinterpret_cast<float*>(st + 20 * B);
  p.E = reinterpret_cast<float*>(st + 24 * B);
  p.last = reinterpret_cast<float*>(st + 28 * B);
  p.sum = reinterpret_cast<double*>(st + 32 * B);
  p.tok = reinterpret_cast<int32_t*>(st + 40 * B);
  p.lq = reinterpret_cast<float*>(st + 40 * B + 4 * B * G);
  p.status = status_ptr(a.workspace);
  p.B = a.B;
  p.gamma = a.gamma;
  p.rows_cap = a.rows_cap;
  p.V = a.V;
  p.rule = a.rule;
  hipLaunchKernelGGL(k_estimate, dim3(a.B), dim3(kEstThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace rv
