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
// One workgroup (1 to 16 waves, at most 4096 candidates):
//  1. survival products, sequential per request in fp64 (-0.0 made +0.0);
//  2. a bitonic sort of the survivals alone, descending, 2 to 8 per lane in
//     registers: strides inside a lane are fmax/fmin pairs, strides up to 63
//     lanes go through DPP, swizzles or permutes, strides across waves
//     through LDS (one barrier each).  A single wave sorts up to 64 survivals;
//     from 65 on the work is spread over at least four waves, one per SIMD;
//  3. the fixed-point prefix sums of floor(S * 2^40) in ranked order, the
//     ratio E(K)/T(K) for every K, and the first arg-max K*;
//  4. the windows: candidates whose survival exceeds the K*-th largest S*
//     are in; of those equal to it, the first ones in (request, position)
//     order fill the remaining places (a scan over requests, only when S* is
//     not unique), which is the order the ranking (S desc, request asc,
//     position asc) gives equal survivals.
// Equal survivals have equal fixed-point values, so ranking survivals
// without candidate ids leaves every E(K) unchanged.  Every operation is
// order independent or sequential per request, so the result is
// bit-identical to a sequential evaluation: fp64 products in position order,
// floor(S * 2^40), exact sums (fp64 adds of integers whose partial sums stay
// at most 2^53, int64 in the full-block modes), two fp64 adds and one IEEE
// fp64 divide per K.
// Contraction is disabled in this file.
#pragma clang fp contract(off)

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kMaxCand = RV_MAX_SCHED_CANDIDATES;    // 8 waves x 64 lanes x 8
constexpr int kShift = 40;
constexpr double kFix = 1099511627776.0;            // 2^40
static_assert(kMaxCand == 8 * 64 * 8, "candidate limit is the 8-wave sort");

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
  return static_cast<long long>(floor(s * kFix));
}

// the value lane (lane ^ M) holds, M < 64
template <int M>
__device__ inline uint32_t xchg32(uint32_t v) {
  const int x = static_cast<int>(v);
  if constexpr (M == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);    // quad_perm 1,0,3,2
  else if constexpr (M == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true); // quad_perm 2,3,0,1
  else if constexpr (M == 3) return __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, true); // quad_perm 3,2,1,0
  else if constexpr (M == 7) return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true); // row_half_mirror
  else if constexpr (M == 15) return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true); // row_mirror
  else if constexpr (M < 32) return __builtin_amdgcn_ds_swizzle(x, 0x1F | (M << 10));   // xor within 32
  else return __builtin_amdgcn_ds_bpermute(static_cast<int>(((threadIdx.x & 63) ^ M) << 2), x);
}
template <int M>
__device__ inline double xchg(double v) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = xchg32<M>(static_cast<uint32_t>(b));
  const uint32_t hi = xchg32<M>(static_cast<uint32_t>(b >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sort keys are the survivals themselves (S in [0, 1], -0.0 made +0.0, no
// NaN), padding -1.  One compare-exchange stage of the descending bitonic
// network over positions p = I * g + j (g = thread, j < I in registers):
// p meets p ^ m and the lower position keeps the larger key; m = size - 1 is
// the mirror stage that starts the merge of a size block, a power of two m
// a half-cleaner.
template <int W, int I, int m>
__device__ inline void stage(double (&v)[I], double* xbuf, int& flip) {
  if constexpr (m < I) {
#pragma unroll
    for (int j = 0; j < I; ++j) {
      const int jj = j ^ m;
      if (j < jj) {
        const double a = v[j], b = v[jj];
        v[j] = fmax(a, b);
        v[jj] = fmin(a, b);
      }
    }
  } else {
    constexpr int lgI = (I == 2) ? 1 : (I == 4) ? 2 : (I == 8) ? 3 : 4;
    constexpr int M = m >> lgI;            // lane distance
    constexpr int jm = m & (I - 1);        // 0 (half-cleaner) or I-1 (mirror)
    constexpr int hb = (jm == I - 1) ? (M + 1) >> 1 : M;   // the bit that orders the pair
    const bool upper = (threadIdx.x & hb) != 0;
    double o[I];
    if constexpr (M < 64) {
#pragma unroll
      for (int j = 0; j < I; ++j) o[j] = xchg<M>(v[j ^ jm]);
    } else {
      // across waves: every lane publishes its keys, one barrier, the partner
      // lane's keys are read back (two buffers in turn, so the next such stage
      // may write before the last reader of this one is done)
      double* b = xbuf + (flip & 1) * (64 * W * I);
      ++flip;
      double2* mine = reinterpret_cast<double2*>(b + I * threadIdx.x);
#pragma unroll
      for (int j = 0; j < I; j += 2) mine[j / 2] = make_double2(v[j], v[j + 1]);
      __syncthreads();
      const double2* part = reinterpret_cast<const double2*>(b + I * (threadIdx.x ^ M));
#pragma unroll
      for (int j = 0; j < I; j += 2) {
        const double2 q = part[(j ^ jm) / 2];
        if constexpr (jm == 0) {
          o[j] = q.x;
          o[j + 1] = q.y;
        } else {
          o[j] = q.y;
          o[j + 1] = q.x;
        }
      }
    }
    // the lower lane of the pair keeps the larger key, the upper the smaller
#pragma unroll
    for (int j = 0; j < I; ++j) v[j] = ((v[j] > o[j]) != upper) ? v[j] : o[j];
  }
}

template <int W, int I, int ST>
__device__ inline void cleaners(double (&v)[I], double* xbuf, int& flip) {
  if constexpr (ST >= 1) {
    stage<W, I, ST>(v, xbuf, flip);
    cleaners<W, I, ST / 2>(v, xbuf, flip);
  }
}

// sorts the first N positions (N a power of two, uniform) for sizes S.. N
template <int W, int I, int S>
__device__ inline void sort_sizes(double (&v)[I], int N, double* xbuf, int& flip) {
  if constexpr (S <= 64 * W * I) {
    if (S > N) return;
    stage<W, I, S - 1>(v, xbuf, flip);
    cleaners<W, I, S / 4>(v, xbuf, flip);
    sort_sizes<W, I, S * 2>(v, N, xbuf, flip);
  }
}

// Exclusive scan of one value per thread in thread order (butterfly over the
// wave, then the wave totals); *total gets the sum.  Exact for integers, and
// for doubles whose partial sums are integers below 2^53.  buf holds W values
// and must not be read by a scan still in progress (callers alternate).
template <int M, typename V>
__device__ inline V xchg_any(V x) {
  if constexpr (sizeof(V) == 8) {
    const uint64_t b = static_cast<uint64_t>(__builtin_bit_cast(long long, x));
    const uint32_t lo = xchg32<M>(static_cast<uint32_t>(b));
    const uint32_t hi = xchg32<M>(static_cast<uint32_t>(b >> 32));
    return __builtin_bit_cast(V, static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
  } else {
    return __builtin_bit_cast(V, xchg32<M>(__builtin_bit_cast(uint32_t, x)));
  }
}
template <int W, typename V>
__device__ inline V block_scan_excl(V x, V* buf, V* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  V pre = 0, tot = x;
  auto step = [&](V t, int bit) {
    if (lane & bit) pre += t;
    tot += t;
  };
  step(xchg_any<1>(tot), 1);
  step(xchg_any<2>(tot), 2);
  step(xchg_any<4>(tot), 4);
  step(xchg_any<8>(tot), 8);
  step(xchg_any<16>(tot), 16);
  step(xchg_any<32>(tot), 32);
  if (lane == 0) buf[wv] = tot;
  __syncthreads();
  V before = 0, all = 0;
#pragma unroll
  for (int u = 0; u < W; ++u) {
    const V y = buf[u];
    before += u < wv ? y : 0;
    all += y;
  }
  *total = all;
  return before + pre;
}

template <int W, int I>
__global__ __launch_bounds__(64 * W) void k_schedule(SchedParams p) {
  constexpr int T = 64 * W;
  __shared__ __align__(16) double orig[T * I];     // survival of candidate i*(gamma-1) + k-1
  __shared__ __align__(16) double xbuf[(W > 1) ? 2 * T * I : T * I];
  __shared__ double scan_d[W];
  __shared__ long long scan_l[2][W];
  __shared__ double red_r[W];
  __shared__ int red_k[W], red_bad[W];

  const int g = threadIdx.x;
  const int lane = g & 63, wv = g >> 6;
  const int B = p.B, g1 = p.gamma - 1;
  const int n = B * g1;
  const bool ranked = (p.mode == RV_COMPACT || p.mode == RV_CAP_ACCEPT);
  const int R = (B + T - 1) / T;                 // requests per thread, in order
  const int i0 = g * R, i1 = min(i0 + R, B);

  // The first request's confidences, then the cost-table entries for
  // K = I*g+j+1 and K = 0, all issued before any is used and without
  // branches (indices clamped into range, the values masked later), so the
  // two sets of loads share one round trip.
  auto load_conf = [&](int i, float (&cv)[RV_MAX_GAMMA - 1]) {
#pragma unroll
    for (int k = 0; k < RV_MAX_GAMMA - 1; ++k) cv[k] = p.conf[i * g1 + min(k, g1 - 1)];
  };
  float cv0[RV_MAX_GAMMA - 1];
  load_conf(i0 < i1 ? i0 : 0, cv0);
  double th[I];
  double alpha_b = 0.0, theta0 = 0.0;
  if (ranked) {
#pragma unroll
    for (int j = 0; j < I; ++j) th[j] = p.theta[B + min(I * g + j + 1, n)];   // B + n < theta_len
    alpha_b = p.alpha[B];
    theta0 = p.theta[B];
  }

  // ---- 1. survival products, sequential per request ----------------------------
  long long local_sum = 0;
  for (int i = i0; i < i1; ++i) {
    float cv[RV_MAX_GAMMA - 1];
    if (i == i0) {
#pragma unroll
      for (int k = 0; k < RV_MAX_GAMMA - 1; ++k) cv[k] = cv0[k];
    } else {
      load_conf(i, cv);
    }
    double S = 1.0;
#pragma unroll
    for (int k = 1; k < RV_MAX_GAMMA; ++k) {
      if (k > g1) break;
      float c = cv[k - 1];
      if (!(c >= 0.0f && c <= 1.0f)) {
        set_status(p.status, RV_DEV_BAD_CONF);
        c = 0.0f;
      }
      if (c == 0.0f) c = 0.0f;   // -0.0 as +0.0: zero survivals compare equal in every form
      S = S * static_cast<double>(c);
      if (ranked) orig[i * g1 + (k - 1)] = S;
      else local_sum += fixed_of(S);
    }
  }
  const long long base = static_cast<long long>(B) << kShift;

  if (!ranked) {
    long long all = 0;
    block_scan_excl<W, long long>(local_sum, scan_l[0], &all);
    for (int i = g; i < B; i += T) {
      p.w_commit[i] = p.gamma;
      p.w_verify[i] = p.gamma;
    }
    if (g == 0) {
      p.k_star[0] = n;
      p.e_star[0] = static_cast<double>(base + all) * (1.0 / kFix);
    }
    return;
  }
  __syncthreads();

  // ---- 2. sort the survivals, descending ---------------------------------------
  int N = I;
  while (N < n) N <<= 1;
  double v[I];
#pragma unroll
  for (int j = 0; j < I; j += 2) {
    const double2 q = reinterpret_cast<const double2*>(orig + I * g)[j / 2];
    v[j] = I * g + j < n ? q.x : -1.0;
    v[j + 1] = I * g + j + 1 < n ? q.y : -1.0;
  }
  int flip = 0;
  sort_sizes<W, I, 2>(v, N, xbuf, flip);
  // the ranked survivals into the exchange buffer the last cross-wave stage
  // did not use (every reader of it passed that stage's barrier); published
  // by the arg-max barrier below
  double* srt = xbuf + (flip & 1) * (T * I);
#pragma unroll
  for (int j = 0; j < I; j += 2) reinterpret_cast<double2*>(srt + I * g)[j / 2] = make_double2(v[j], v[j + 1]);

  // ---- 3. fixed-point prefix sums in ranked order, first arg-max ---------------
  // floor(S * 2^40) as doubles: every partial sum (with the base B * 2^40) is
  // an integer at most 2^53, so the fp64 adds are exact and equal the int64 sums
  double f[I];
  double mine = 0.0;
#pragma unroll
  for (int j = 0; j < I; ++j) {
    f[j] = I * g + j < n ? floor(v[j] * kFix) : 0.0;
    mine += f[j];
  }
  double tot = 0.0;
  const double pre = block_scan_excl<W, double>(mine, scan_d, &tot);
  const double based = static_cast<double>(base);

  const double ba = p.bias + alpha_b;
  double best_r = -1.0;
  int best_k = 0x7fffffff;
  bool bad = false;
  // branch-free, so the divides of the lane's K values overlap
  auto eval = [&](int K, double nk, double theta, bool valid) {
    const double Tm = ba + theta;
    const bool ok = (Tm > 0.0) && (Tm < 1e300);
    bad = bad || (valid && !ok);
    const double r = nk / (ok ? Tm : 1.0);
    const bool take = valid && ok && r > best_r;
    best_r = take ? r : best_r;
    best_k = take ? K : best_k;
  };
  eval(0, based, theta0, g == 0);
  double run = pre;
#pragma unroll
  for (int j = 0; j < I; ++j) {
    const int K = I * g + j + 1;
    run += f[j];
    eval(K, based + run, th[j], K <= n);   // K takes the first K ranked candidates
  }
  // first arg-max: the largest ratio; of equal ratios the smallest K, which
  // is the lowest lane holding it (K grows with the lane) and then the first
  // wave (K grows with the wave)
  double rmax = best_r;
  rmax = fmax(rmax, xchg<1>(rmax));
  rmax = fmax(rmax, xchg<2>(rmax));
  rmax = fmax(rmax, xchg<4>(rmax));
  rmax = fmax(rmax, xchg<8>(rmax));
  rmax = fmax(rmax, xchg<16>(rmax));
  rmax = fmax(rmax, xchg<32>(rmax));
  const uint64_t at = __ballot(best_r == rmax);
  const int first = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(at)));
  const int kw = __shfl(best_k, first);
  const bool wave_bad = __ballot(bad) != 0;
  if (lane == 0) {
    red_r[wv] = rmax;
    red_k[wv] = kw;
    red_bad[wv] = wave_bad ? 1 : 0;
  }
  __syncthreads();
  double rbest = red_r[0];
  int kst = red_k[0];
  int any_bad = red_bad[0];
#pragma unroll
  for (int u = 1; u < W; ++u) {
    const double rb = red_r[u];
    if (rb > rbest) { rbest = rb; kst = red_k[u]; }
    any_bad |= red_bad[u];
  }
  if (any_bad) {
    kst = 0;
    if (g == 0) set_status(p.status, RV_DEV_BAD_COST);
  }
  if (g == 0) {
    p.k_star[0] = kst;
    if (kst == 0) p.e_star[0] = based * (1.0 / kFix);
  }
  // E(K*) from the owner of ranked position K*-1
  if (kst > 0 && (kst - 1) / I == g) {
    const int jst = (kst - 1) % I;
    double e = pre;
#pragma unroll
    for (int j = 0; j < I; ++j)
      if (j <= jst) e += f[j];
    p.e_star[0] = (based + e) * (1.0 / kFix);
  }

  // ---- 4. windows ----------------------------------------------------------------
  if (kst == 0) {
    for (int i = g; i < B; i += T) {
      p.w_commit[i] = 1;
      p.w_verify[i] = (p.mode == RV_CAP_ACCEPT) ? p.gamma : 1;
    }
    return;
  }
  // S*: the K*-th largest survival.  Every survival above it is in; equal
  // survivals are adjacent in ranked order, so S* is unique when its two
  // ranked neighbours differ from it, and then the survivals >= S* are
  // exactly the first K*.
  const double sstar = srt[kst - 1];
  const bool unique = (kst < 2 || srt[kst - 2] != sstar) && (kst >= n || srt[kst] != sstar);
  // a request's survivals, unrolled over the longest block (indices clamped
  // into the array, positions past the block masked)
  auto count_req = [&](int i, int& gt, int& eq) {
    gt = 0;
    eq = 0;
#pragma unroll
    for (int k = 0; k < RV_MAX_GAMMA - 1; ++k) {
      const double sv = orig[min(i * g1 + k, T * I - 1)];
      gt += (k < g1 && sv > sstar) ? 1 : 0;
      eq += (k < g1 && sv == sstar) ? 1 : 0;
    }
  };
  if (unique) {
    for (int i = i0; i < i1; ++i) {
      int gt, eq;
      count_req(i, gt, eq);
      const int w = 1 + gt + eq;
      p.w_commit[i] = w;
      p.w_verify[i] = (p.mode == RV_CAP_ACCEPT) ? p.gamma : w;
    }
    return;
  }
  // Equal survivals at the boundary: G ranked strictly before S* (binary
  // search for the first ranked position holding S*), and the remaining
  // K* - G places go to the candidates equal to S* in (request, position)
  // order: a scan of their counts over the requests.
  int lo = 0, hi = kst - 1;     // srt[hi] == S*, srt[i] > S* for i < G
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (srt[mid] > sstar) lo = mid + 1;
    else hi = mid;
  }
  const int r = kst - lo;
  long long eq_mine = 0;
  for (int i = i0; i < i1; ++i) {
    int gt, eq;
    count_req(i, gt, eq);
    eq_mine += eq;
  }
  long long eq_all = 0;
  int eq_before = static_cast<int>(block_scan_excl<W, long long>(eq_mine, scan_l[1], &eq_all));
  for (int i = i0; i < i1; ++i) {
    int gt, eq;
    count_req(i, gt, eq);
    const int take = min(max(r - eq_before, 0), eq);
    eq_before += eq;
    const int w = 1 + gt + take;
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
  // waves x keys per lane: all four SIMDs from 65 candidates on
  const long long n = (long long)a.B * (a.gamma - 1);
  if (n <= 128) hipLaunchKernelGGL((k_schedule<1, 2>), dim3(1), dim3(64), 0, s, p);
  else if (n <= 512) hipLaunchKernelGGL((k_schedule<4, 2>), dim3(1), dim3(256), 0, s, p);
  else if (n <= 1024) hipLaunchKernelGGL((k_schedule<4, 4>), dim3(1), dim3(256), 0, s, p);
  else if (n <= 2048) hipLaunchKernelGGL((k_schedule<8, 4>), dim3(1), dim3(512), 0, s, p);
  else hipLaunchKernelGGL((k_schedule<8, 8>), dim3(1), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace rv
