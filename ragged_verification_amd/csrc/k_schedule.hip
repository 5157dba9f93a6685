// Stage 1: confidence scheduler.
//
// DSpark-in-SGLang page, section A2: the confidence head scores each draft,
// the product of the scores over the block is the block's survival
// probability, and the confidence scheduler turns survival into per-request
// verify budgets each step; section 速读 / A2 "cost-table profiling": the
// step time is modelled as T(bs, K) = bias + alpha(bs) + theta(bs + K) and the
// scheduler's argmax trades expected accepted tokens against that marginal
// cost.
//
// One workgroup of 1024 threads does the whole batch in LDS (at most 4096
// candidates): survival products, a bitonic sort of the candidates by
// (survival desc, request asc, position asc), an int64 fixed-point prefix sum
// of the ranked survivals, the ratio E(K)/T(K) for every K, and the first
// arg-max.  Every operation is order independent or sequential per request,
// so the result is bit-identical to a sequential evaluation: fp64 products in
// position order, floor(S * 2^40) as int64, exact integer sums, two fp64 adds
// and one IEEE fp64 divide per K.  Contraction is disabled in this file.
#pragma clang fp contract(off)

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kThreads = 1024;
constexpr int kMaxCand = RV_MAX_SCHED_CANDIDATES;
constexpr int kShift = 40;

struct SchedParams {
  const float* conf;
  const double* alpha;
  const double* theta;
  int32_t* w_commit;
  int32_t* w_verify;
  int32_t* k_star;
  double* e_star;
  int32_t* status;
  double bias;
  int B, gamma, mode;
};

__device__ inline long long fixed_of(double s) {
  // s in [0,1]: s * 2^40 is exact, floor of a non-negative value is a cast
  return static_cast<long long>(floor(s * 1099511627776.0));
}

// Inclusive scan of one int64 per thread: wave shuffles, then one pass over
// the 16 wave totals (integer adds, so the order does not matter).  *total
// gets the workgroup total.  buf holds kThreads / 64 values.
__device__ long long block_scan_incl(long long v, long long* buf, long long* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  __syncthreads();   // buf is free
  if (lane == 63) buf[wv] = v;
  __syncthreads();
  long long before = 0, all = 0;
  for (int u = 0; u < kThreads / 64; ++u) {
    const long long x = buf[u];
    before += u < wv ? x : 0;
    all += x;
  }
  *total = all;
  return before + v;
}

__global__ __launch_bounds__(kThreads) void k_schedule(SchedParams p) {
  __shared__ uint64_t key[kMaxCand];      // ~bits(S): ascending = S descending
  __shared__ uint16_t cid[kMaxCand];      // candidate id = i*(gamma-1) + (k-1)
  __shared__ uint16_t rank_of[kMaxCand];  // sorted position of each candidate
  __shared__ long long scan_buf[kThreads / 64];
  __shared__ double red_r[kThreads / 64];
  __shared__ int red_k[kThreads / 64];
  __shared__ int bad_cost;

  const int t = threadIdx.x;
  const int B = p.B, g1 = p.gamma - 1;
  const int n = B * g1;
  if (t == 0) bad_cost = 0;

  // The cost-table entries this thread evaluates after the sort (K = j+1
  // for its ranked slots j, and K = 0 on thread 0), loaded now so that their
  // latency overlaps the survival products and the sort.
  const int seg = (n + kThreads - 1) / kThreads;  // <= 4
  const int j0 = t * seg;
  constexpr int kSegMax = kMaxCand / kThreads;
  double th[kSegMax];
  double alpha_b = 0.0, theta0 = 0.0;
  if (p.mode == RV_COMPACT || p.mode == RV_CAP_ACCEPT) {
#pragma unroll
    for (int u = 0; u < kSegMax; ++u) th[u] = (u < seg && j0 + u < n) ? p.theta[B + j0 + u + 1] : 0.0;
    alpha_b = p.alpha[B];
    if (t == 0) theta0 = p.theta[B];
  }

  // ---- survival products, sequential per request ----------------------------
  long long local_sum = 0;
  auto survive = [&](int i) {
    // all of the request's confidences in flight at once, then the products
    float cv[RV_MAX_GAMMA - 1];
#pragma unroll
    for (int k = 1; k < RV_MAX_GAMMA; ++k) cv[k - 1] = k <= g1 ? p.conf[i * g1 + (k - 1)] : 0.0f;
    double S = 1.0;
#pragma unroll
    for (int k = 1; k < RV_MAX_GAMMA; ++k) {
      if (k > g1) break;
      float c = cv[k - 1];
      if (!(c >= 0.0f && c <= 1.0f)) {
        set_status(p.status, RV_DEV_BAD_CONF);
        c = 0.0f;
      }
      // -0.0 is a valid zero; as +0.0 its survival key sorts with the other
      // zeros (the sort compares bit patterns)
      if (c == 0.0f) c = 0.0f;
      S = S * static_cast<double>(c);
      const int id = i * g1 + (k - 1);
      if (p.mode == RV_COMPACT || p.mode == RV_CAP_ACCEPT) {
        key[id] = ~static_cast<uint64_t>(__double_as_longlong(S));
        cid[id] = static_cast<uint16_t>(id);
      } else {
        local_sum += fixed_of(S);
      }
    }
  };
  // the first request of each thread outside any loop, so that its loads
  // share one round trip with the cost-table loads above (a loop head would
  // wait for those first)
  if (t < B) survive(t);
  for (int i = t + kThreads; i < B; i += kThreads) survive(i);
  const long long base = static_cast<long long>(B) << kShift;

  if (p.mode == RV_STATIC || p.mode == RV_NO_TRIM) {
    long long all = 0;
    block_scan_incl(local_sum, scan_buf, &all);
    for (int i = t; i < B; i += kThreads) {
      p.w_commit[i] = p.gamma;
      p.w_verify[i] = p.gamma;
    }
    if (t == 0) {
      p.k_star[0] = n;
      p.e_star[0] = static_cast<double>(base + all) * (1.0 / 1099511627776.0);
    }
    return;
  }

  // ---- bitonic sort of (key, cid) ascending ---------------------------------
  int N = 1;
  while (N < n) N <<= 1;
  for (int j = n + t; j < N; j += kThreads) {
    key[j] = ~0ull;
    cid[j] = 0xffff;
  }
  __syncthreads();
  // Thread t compares pairs q = t, t+1024, ...; with stride <= 64 both
  // elements of every pair lie in the 128-element block 2q/128, which only
  // the wave of t touches, so such a stage needs only the wave's own LDS
  // operations to be done before the next; a workgroup barrier follows any
  // stage that crosses waves and any stage before one that does.
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = t; q < N / 2; q += kThreads) {
        const int lo = 2 * q - (q & (stride - 1));
        const int hi = lo + stride;
        const bool up = ((lo & size) == 0);
        const uint64_t ka = key[lo], kb = key[hi];
        const uint16_t ia = cid[lo], ib = cid[hi];
        const bool a_gt_b = (ka > kb) || (ka == kb && ia > ib);
        if (a_gt_b == up) {
          key[lo] = kb; key[hi] = ka;
          cid[lo] = ib; cid[hi] = ia;
        }
      }
      const int next_stride = stride > 1 ? stride >> 1 : size;   // first stride of the next size
      if (stride >= 128 || (next_stride >= 128 && size < N)) {
        __syncthreads();
      } else {
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  __syncthreads();

  // ---- fixed-point prefix sums in ranked order ------------------------------
  long long run = 0;
  for (int j = j0; j < j0 + seg && j < n; ++j) {
    const double S = __longlong_as_double(static_cast<long long>(~key[j]));
    run += fixed_of(S);
    rank_of[cid[j]] = static_cast<uint16_t>(j);
  }
  long long run_total = 0;
  const long long incl = block_scan_incl(run, scan_buf, &run_total);
  long long pre = incl - run;  // exclusive prefix before j0

  // ---- ratio for every K, first arg-max -------------------------------------
  const double ba = p.bias + alpha_b;
  double best_r = -1.0;
  int best_k = 0x7fffffff;
  bool bad = false;
  auto eval = [&](int K, long long nk, double theta) {
    const double T = ba + theta;
    if (!(T > 0.0) || !(T < 1e300)) { bad = true; return; }
    const double r = static_cast<double>(nk) / T;
    if (r > best_r) { best_r = r; best_k = K; }
  };
  if (t == 0) eval(0, base, theta0);
#pragma unroll
  for (int u = 0; u < kSegMax; ++u) {
    const int j = j0 + u;
    if (u >= seg || j >= n) break;
    const double S = __longlong_as_double(static_cast<long long>(~key[j]));
    pre += fixed_of(S);
    eval(j + 1, base + pre, th[u]);  // K = j+1 takes the first j+1 ranked candidates
  }
  if (bad) atomicOr(&bad_cost, 1);
  // first arg-max: the larger ratio, the smaller K on ties (an exact order,
  // so the shuffle tree gives the sequential answer)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double rb = __shfl_xor(best_r, off);
    const int kb = __shfl_xor(best_k, off);
    if (rb > best_r || (rb == best_r && kb < best_k)) { best_r = rb; best_k = kb; }
  }
  if ((t & 63) == 0) {
    red_r[t >> 6] = best_r;
    red_k[t >> 6] = best_k;
  }
  __syncthreads();
  double rbest = red_r[0];
  int kst = red_k[0];
  for (int u = 1; u < kThreads / 64; ++u) {
    const double rb = red_r[u];
    const int kb = red_k[u];
    if (rb > rbest || (rb == rbest && kb < kst)) { rbest = rb; kst = kb; }
  }
  if (bad_cost) {
    kst = 0;
    if (t == 0) set_status(p.status, RV_DEV_BAD_COST);
  }
  // N_{K*}: the inclusive prefix at position K*-1 (recomputed by its owner)
  if (t == 0 && kst == 0) p.e_star[0] = static_cast<double>(base) * (1.0 / 1099511627776.0);
  {
    long long pre2 = incl - run;
    for (int j = j0; j < j0 + seg && j < n; ++j) {
      const double S = __longlong_as_double(static_cast<long long>(~key[j]));
      pre2 += fixed_of(S);
      if (j + 1 == kst) p.e_star[0] = static_cast<double>(base + pre2) * (1.0 / 1099511627776.0);
    }
  }
  if (t == 0) p.k_star[0] = kst;

  // ---- windows ---------------------------------------------------------------
  for (int i = t; i < B; i += kThreads) {
    int w = 1;
    for (int k = 1; k <= g1; ++k) w += (rank_of[i * g1 + (k - 1)] < kst) ? 1 : 0;
    p.w_commit[i] = w;
    p.w_verify[i] = (p.mode == RV_CAP_ACCEPT) ? p.gamma : w;
  }
}

}  // namespace

hipError_t launch_schedule(const rv_schedule_args& a, hipStream_t s) {
  SchedParams p;
  p.conf = a.conf;
  p.alpha = a.cost_alpha;
  p.theta = a.cost_theta;
  p.w_commit = a.w_commit;
  p.w_verify = a.w_verify;
  p.k_star = a.k_star;
  p.e_star = a.e_star;
  p.status = status_ptr(a.workspace);
  p.bias = a.cost_bias;
  p.B = a.B;
  p.gamma = a.gamma;
  p.mode = a.mode;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace rv
