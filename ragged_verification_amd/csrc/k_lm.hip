// Stage 4: target LM head over the packed rows and the acceptance rule.
//
// The verify forward ends in the target's vocabulary projection of every
// packed row; drafts are checked against it (lshu.cn DSpark explainer, section
// 1.2: keep drafts up to the first disagreement; sections 2.3 and 3.3: keep
// draft x with probability min(1, p(x)/q(x))).  cap-accept verifies the whole
// block but commits up to the scheduled window and reports the ceiling
// (DSpark-in-SGLang page, section A2 "verify modes" and "observability").
//
// Design (gfx950):
//  * k_lm_gemm: z = X W^T with bf16 32x32x16 MFMAs (fp32 accumulation), a
//    128x128 output tile per workgroup (four waves of 64x64), K-loop of 64
//    staged through double-buffered LDS with register prefetch.  Workgroups
//    whose rows lie past the packed total exit at once, so the work follows
//    the real row count M, not the tier.  The epilogue never materialises the
//    logits unless asked: per 64-column slab it reduces each row to (max,
//    lowest argmax, sum of exp(z - max)) with cross-lane shuffles and writes
//    16 bytes.  Column tiles of one vocabulary block sit on one XCD so the
//    weight tile is fetched from HBM once per XCD-resident row tile group.
//  * k_lm_f32: the same partials from fp32 inputs (plain dot products).
//  * k_accept: one workgroup per request merges the slab partials of its
//    rows, runs the greedy or rejection scan, and for rejection draws the
//    bonus token by an inverse CDF over the vocabulary (fp64 chunk sums, one
//    block scan, one sequential walk inside the chunk that holds the target).

#include <float.h>

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kSlab = 64;                 // columns per partial
constexpr int kGemmThreads = 256;
constexpr int kAStride = kBK + 8;         // bf16 per LDS row (16-byte pad)

struct GemmParams {
  const bf16_t* x;     // [rows][H]
  const bf16_t* w;     // [V][H]
  const int32_t* mm;
  float4* part;        // [rows][n_slabs]
  float* logits;       // optional [rows][V]
  int H, V, n_slabs, n_mt, n_vt;
  int with_sum;
};

__device__ inline void merge_best(float& v, int& idx, float ov, int oidx) {
  if (ov > v || (ov == v && oidx < idx)) { v = ov; idx = oidx; }
}

__global__ __launch_bounds__(kGemmThreads) void k_lm_gemm(GemmParams p) {
  __shared__ __align__(16) bf16_t As[2][kBM * kAStride];
  __shared__ __align__(16) bf16_t Bs[2][kBN * kAStride];

  // XCD-aware tile order: consecutive logical tiles stay on one XCD, and the
  // row tiles of a vocabulary tile are consecutive.
  const int n_tiles = p.n_mt * p.n_vt;
  const int per_xcd = (n_tiles + 7) / 8;
  const int kloc = blockIdx.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + kloc;
  if (kloc >= per_xcd || logical >= n_tiles) return;
  const int vt = logical / p.n_mt;
  const int mt = logical % p.n_mt;
  const int M = p.mm[0];
  const int m0 = mt * kBM;
  if (m0 >= M) return;
  const int v0 = vt * kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  // global -> register prefetch: 1024 chunks of 16 B per operand tile
  u32x4_t ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = tid + e * kGemmThreads;
      const int r = ch >> 3, c = (ch & 7) * 8;
      const int gr = m0 + r;
      ra[e] = (gr < M) ? *reinterpret_cast<const u32x4_t*>(p.x + (size_t)gr * p.H + k0 + c)
                       : u32x4_t{0u, 0u, 0u, 0u};
      const int gv = v0 + r;
      rb[e] = (gv < p.V) ? *reinterpret_cast<const u32x4_t*>(p.w + (size_t)gv * p.H + k0 + c)
                         : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ch = tid + e * kGemmThreads;
      const int r = ch >> 3, c = (ch & 7) * 8;
      *reinterpret_cast<u32x4_t*>(&As[buf][r * kAStride + c]) = ra[e];
      *reinterpret_cast<u32x4_t*>(&Bs[buf][r * kAStride + c]) = rb[e];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  const int nk = p.H / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4_t af[2], bfr[2];
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
        af[bm] = *reinterpret_cast<const u32x4_t*>(
            &As[cur][(wm * 64 + bm * 32 + l32) * kAStride + ks * 16 + lh * 8]);
#pragma unroll
      for (int bn = 0; bn < 2; ++bn)
        bfr[bn] = *reinterpret_cast<const u32x4_t*>(
            &Bs[cur][(wn * 64 + bn * 32 + l32) * kAStride + ks * 16 + lh * 8]);
#pragma unroll
      for (int bm = 0; bm < 2; ++bm)
#pragma unroll
        for (int bn = 0; bn < 2; ++bn) acc[bm][bn] = mfma32(af[bm], bfr[bn], acc[bm][bn]);
    }
    if (kt + 1 < nk) {
      sstore(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds column (l32) of rows 8*(j/4) + 4*lh + j%4 ------
  const int slab = (v0 + wn * 64) / kSlab;
#pragma unroll
  for (int bm = 0; bm < 2; ++bm) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int rl = wm * 64 + bm * 32 + (j / 4) * 8 + lh * 4 + (j % 4);
      const int row = m0 + rl;
      const int c0 = v0 + wn * 64 + l32;
      const int c1 = c0 + 32;
      float z0 = acc[bm][0][j], z1 = acc[bm][1][j];
      if (p.logits && row < M) {
        if (c0 < p.V) p.logits[(size_t)row * p.V + c0] = z0;
        if (c1 < p.V) p.logits[(size_t)row * p.V + c1] = z1;
      }
      if (c0 >= p.V) z0 = -INFINITY;
      if (c1 >= p.V) z1 = -INFINITY;
      float best = z0;
      int bi = c0;
      merge_best(best, bi, z1, c1);
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) {
        const float ov = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        merge_best(best, bi, ov, oi);
      }
      float se = 0.f;
      if (p.with_sum) {
        se = (z0 == -INFINITY ? 0.f : __expf(z0 - best)) + (z1 == -INFINITY ? 0.f : __expf(z1 - best));
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) se += __shfl_xor(se, off);
      }
      if (l32 == 0 && row < M && v0 + wn * 64 < p.V)
        p.part[(size_t)row * p.n_slabs + slab] = make_float4(best, __int_as_float(bi), se, 0.f);
    }
  }
}

// ---- fp32 path ------------------------------------------------------------------
struct F32LmParams {
  const float* x;
  const float* w;
  const int32_t* mm;
  float4* part;
  float* logits;
  int H, V, n_slabs;
};

// grid (rows_cap, ceil(V/256)); each wave owns one 64-column slab
__global__ __launch_bounds__(256) void k_lm_f32(F32LmParams p) {
  const int row = blockIdx.x;
  if (row >= p.mm[0]) return;
  const int col = blockIdx.y * 256 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  float z = -INFINITY;
  if (col < p.V) {
    const float* xr = p.x + (size_t)row * p.H;
    const float* wr = p.w + (size_t)col * p.H;
    float s = 0.f;
    for (int h = 0; h < p.H; ++h) s = fmaf(xr[h], wr[h], s);
    z = s;
    if (p.logits) p.logits[(size_t)row * p.V + col] = s;
  }
  float best = z;
  int bi = col;
  for (int off = 1; off < 64; off <<= 1) {
    const float ov = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    merge_best(best, bi, ov, oi);
  }
  float se = (z == -INFINITY) ? 0.f : __expf(z - best);
  for (int off = 1; off < 64; off <<= 1) se += __shfl_xor(se, off);
  const int slab = col / kSlab;
  if (lane == 0 && slab * kSlab < p.V) p.part[(size_t)row * p.n_slabs + slab] = make_float4(best, __int_as_float(bi), se, 0.f);
}

// ---- accept ------------------------------------------------------------------------
struct AcceptParams {
  const float4* part;
  const float* logits;
  const int32_t* mm;
  const int32_t* cu;
  const int32_t* w_commit;
  const int32_t* w_verify;
  const int32_t* drafts;
  const float* q_rows;
  const float* u;
  const float* u_bonus;
  int32_t* pred;
  int32_t* accept;
  int32_t* bonus;
  int32_t* ceiling;
  int32_t* status;
  int B, gamma, V, n_slabs, rule;
};

constexpr int kAccThreads = 256;

__global__ __launch_bounds__(kAccThreads) void k_accept(AcceptParams p) {
  __shared__ float s_val[kAccThreads];
  __shared__ int s_idx[kAccThreads];
  __shared__ double s_sum[kAccThreads];
  __shared__ int s_pred[RV_MAX_GAMMA];
  __shared__ float s_lse[RV_MAX_GAMMA];
  __shared__ int s_row, s_qrow, s_c, s_a;
  const int tid = threadIdx.x;

  if (blockIdx.x == p.B) {  // padding rows [M, M_pad)
    const int M = p.mm[0], Mpad = p.mm[1];
    for (int r = M + tid; r < Mpad; r += kAccThreads) p.pred[r] = -1;
    return;
  }
  const int i = blockIdx.x;
  const int base = p.cu[i];
  int wv = p.w_verify[i], wc = p.w_commit[i];
  const int packed = p.cu[i + 1] - base;      // rows actually packed for request i
  if (packed < 1 || packed > p.gamma) {       // corrupt packing: touch no rows
    if (tid == 0) {
      set_status(p.status, RV_DEV_BAD_WINDOW);
      p.accept[i] = 0;
      p.ceiling[i] = 0;
      p.bonus[i] = -1;
    }
    return;
  }
  if (wv != packed || wc < 1 || wc > packed) {
    if (tid == 0) set_status(p.status, RV_DEV_BAD_WINDOW);
    wv = packed;
    wc = min(max(wc, 1), wv);
  }
  const int g1 = p.gamma - 1;

  // merge slab partials: argmax (lowest index on ties) and log-sum-exp
  for (int k = 0; k < wv; ++k) {
    const float4* pr = p.part + (size_t)(base + k) * p.n_slabs;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int s = tid; s < p.n_slabs; s += kAccThreads) {
      const float4 q = pr[s];
      merge_best(best, bi, q.x, __float_as_int(q.y));
    }
    s_val[tid] = best;
    s_idx[tid] = bi;
    __syncthreads();
    for (int off = kAccThreads / 2; off > 0; off >>= 1) {
      if (tid < off) {
        float b = s_val[tid];
        int bb = s_idx[tid];
        merge_best(b, bb, s_val[tid + off], s_idx[tid + off]);
        s_val[tid] = b;
        s_idx[tid] = bb;
      }
      __syncthreads();
    }
    const float mx = s_val[0];
    if (tid == 0) {
      s_pred[k] = s_idx[0];
      p.pred[base + k] = s_idx[0];
    }
    if (p.rule == RV_REJECTION) {
      double acc = 0.0;
      for (int s = tid; s < p.n_slabs; s += kAccThreads) {
        const float4 q = pr[s];
        acc += (double)q.z * exp((double)q.x - (double)mx);
      }
      s_sum[tid] = acc;
      __syncthreads();
      for (int off = kAccThreads / 2; off > 0; off >>= 1) {
        if (tid < off) s_sum[tid] += s_sum[tid + off];
        __syncthreads();
      }
      if (tid == 0) s_lse[k] = mx + (float)log(s_sum[0]);
    }
    __syncthreads();
  }

  if (p.rule == RV_GREEDY) {
    if (tid == 0) {
      int c = 0;
      while (c < wv - 1) {
        const int d = p.drafts[(size_t)i * g1 + c];
        if (d < 0 || d >= p.V) { set_status(p.status, RV_DEV_BAD_TOKEN); break; }
        if (d != s_pred[c]) break;
        ++c;
      }
      const int a = min(c, wc - 1);
      p.ceiling[i] = c;
      p.accept[i] = a;
      p.bonus[i] = s_pred[a];
    }
    return;
  }

  // ---- rejection sampling -------------------------------------------------------
  if (tid == 0) {
    int c = 0;
    while (c < wv - 1) {
      const int j = c + 1;
      const int d = p.drafts[(size_t)i * g1 + (j - 1)];
      if (d < 0 || d >= p.V) { set_status(p.status, RV_DEV_BAD_TOKEN); break; }
      const float zd = p.logits[(size_t)(base + j - 1) * p.V + d];
      const float pd = expf(zd - s_lse[j - 1]);
      const float qd = p.q_rows[((size_t)i * g1 + (j - 1)) * p.V + d];
      if (p.u[(size_t)i * g1 + (j - 1)] * qd < pd) ++c;
      else break;
    }
    const int a = min(c, wc - 1);
    s_c = c;
    s_a = a;
    if (c < wc - 1) {          // rejected inside the commit window: residual
      s_row = c;
      s_qrow = c;
    } else {                   // all committed drafts accepted: target row wc-1
      s_row = wc - 1;
      s_qrow = -1;
    }
  }
  __syncthreads();
  const int rrow = s_row, qrow = s_qrow;
  const float lse = s_lse[rrow];
  const float* z = p.logits + (size_t)(base + rrow) * p.V;
  const float* qd = qrow >= 0 ? p.q_rows + ((size_t)i * g1 + qrow) * p.V : nullptr;
  auto weight = [&](int v) -> float {
    const float pv = expf(z[v] - lse);
    return qd ? fmaxf(0.f, pv - qd[v]) : pv;
  };
  const int per = (p.V + kAccThreads - 1) / kAccThreads;
  const int v_lo = tid * per;
  const int v_hi = min(v_lo + per, p.V);
  double csum = 0.0;
  int last_pos = -1;
  for (int v = v_lo; v < v_hi; ++v) {
    const float r = weight(v);
    csum += (double)r;
    if (r > 0.f) last_pos = v;
  }
  // inclusive scan of chunk sums
  s_sum[tid] = csum;
  s_idx[tid] = last_pos;
  __syncthreads();
  for (int off = 1; off < kAccThreads; off <<= 1) {
    const double add = tid >= off ? s_sum[tid - off] : 0.0;
    const int li = tid >= off ? s_idx[tid - off] : -1;
    __syncthreads();
    s_sum[tid] += add;
    s_idx[tid] = max(s_idx[tid], li);
    __syncthreads();
  }
  const double total = s_sum[kAccThreads - 1];
  const int last_any = s_idx[kAccThreads - 1];
  const double target = (double)p.u_bonus[i] * total;
  // exclusive prefix taken from the neighbour's inclusive value, so the
  // per-thread intervals [excl, incl) tile the line without gaps or overlap
  const double excl = tid > 0 ? s_sum[tid - 1] : 0.0;
  __shared__ int s_bonus;
  if (tid == 0) s_bonus = last_any;   // target at or past the end: last positive
  __syncthreads();
  if (excl <= target && target < s_sum[tid] && csum > 0.0) {
    double run = excl;
    int pick = last_pos;               // rounding left the walk short: chunk's last
    for (int v = v_lo; v < v_hi; ++v) {
      run += (double)weight(v);
      if (run > target) { pick = v; break; }
    }
    s_bonus = pick;
  }
  __syncthreads();
  if (tid == 0) {
    p.ceiling[i] = s_c;
    p.accept[i] = s_a;
    p.bonus[i] = s_bonus;
  }
}

}  // namespace

size_t lm_scratch_bytes(int B, int gamma, int V) {
  const size_t n_slabs = (size_t)(V + kSlab - 1) / kSlab;
  return align_up(sizeof(float4) * (size_t)B * gamma * n_slabs, 256);
}

hipError_t launch_lm(const rv_lm_args& a, hipStream_t s) {
  const int n_slabs = (a.V + kSlab - 1) / kSlab;
  float4* part = reinterpret_cast<float4*>(static_cast<char*>(a.workspace) + kStatusBytes);
  const bool rej = (a.rule == RV_REJECTION);
  hipError_t e;
  if (a.dtype == RV_BF16) {
    GemmParams g;
    g.x = static_cast<const bf16_t*>(a.hidden);
    g.w = static_cast<const bf16_t*>(a.W);
    g.mm = a.mm;
    g.part = part;
    g.logits = a.logits;
    g.H = a.H;
    g.V = a.V;
    g.n_slabs = n_slabs;
    const int rows = a.B * a.gamma;   // real rows never exceed one full block each
    g.n_mt = (rows + kBM - 1) / kBM;
    g.n_vt = (a.V + kBN - 1) / kBN;
    g.with_sum = rej ? 1 : 0;
    const int n_tiles = g.n_mt * g.n_vt;
    const int grid = ((n_tiles + 7) / 8) * 8;
    hipLaunchKernelGGL(k_lm_gemm, dim3(grid), dim3(kGemmThreads), 0, s, g);
  } else {
    F32LmParams f;
    f.x = static_cast<const float*>(a.hidden);
    f.w = static_cast<const float*>(a.W);
    f.mm = a.mm;
    f.part = part;
    f.logits = a.logits;
    f.H = a.H;
    f.V = a.V;
    f.n_slabs = n_slabs;
    hipLaunchKernelGGL(k_lm_f32, dim3(a.B * a.gamma, (a.V + 255) / 256), dim3(256), 0, s, f);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  AcceptParams ap;
  ap.part = part;
  ap.logits = a.logits;
  ap.mm = a.mm;
  ap.cu = a.cu;
  ap.w_commit = a.w_commit;
  ap.w_verify = a.w_verify;
  ap.drafts = a.drafts;
  ap.q_rows = a.q_rows;
  ap.u = a.u;
  ap.u_bonus = a.u_bonus;
  ap.pred = a.pred;
  ap.accept = a.accept;
  ap.bonus = a.bonus;
  ap.ceiling = a.ceiling;
  ap.status = status_ptr(a.workspace);
  ap.B = a.B;
  ap.gamma = a.gamma;
  ap.V = a.V;
  ap.n_slabs = n_slabs;
  ap.rule = a.rule;
  hipLaunchKernelGGL(k_accept, dim3(a.B + 1), dim3(kAccThreads), 0, s, ap);
  return hipGetLastError();
}

}  // namespace rv
