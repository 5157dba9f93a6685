// librv C ABI: argument validation, workspace sizing, launches.
//
// Every entry point checks what the host can check before anything is
// enqueued and returns a negative rv_status on failure; see include/rv.h for
// the contract of each call.

#include <math.h>
#include <stddef.h>

#include <vector>

#include "rv_common.h"

namespace rv {
namespace {

__global__ void k_clear_status(int32_t* status) {
  if (threadIdx.x == 0) status[0] = 0;
}

bool ws_ok(const void* ws, size_t bytes, size_t need) { return ws != nullptr && bytes >= need; }

bool block_ok(int B, int gamma) {
  return B >= 1 && gamma >= 2 && gamma <= RV_MAX_GAMMA && (long long)B * gamma <= RV_MAX_ROWS;
}

rv_status hip_status(hipError_t e) { return e == hipSuccess ? RV_OK : RV_ERR_HIP; }

}  // namespace

rv_status lm_args_check(const rv_lm_args* a) {
  if (!a || !a->hidden || !a->W || !a->mm || !a->cu || !a->w_commit || !a->w_verify || !a->drafts ||
      !a->pred || !a->accept || !a->bonus || !a->ceiling)
    return RV_ERR_INVALID_ARG;
  if (a->rule != RV_GREEDY && a->rule != RV_REJECTION) return RV_ERR_INVALID_ARG;
  if (a->rule == RV_REJECTION && (!a->q_rows || !a->u || !a->u_bonus || !a->logits)) return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if ((long long)a->rows_cap < (long long)a->B * a->gamma) return RV_ERR_INVALID_ARG;
  if (a->H < 1 || a->V < 1) return RV_ERR_INVALID_ARG;
  if (a->rule == RV_REJECTION && a->V > kMaxVocabRejection) return RV_ERR_UNSUPPORTED;
  if (a->dtype != RV_F32 && a->dtype != RV_BF16) return RV_ERR_INVALID_ARG;
  if (a->dtype == RV_BF16 && a->H % 64 != 0) return RV_ERR_UNSUPPORTED;
  if (a->w_layout != RV_W_ROWS && a->w_layout != RV_W_TILED) return RV_ERR_INVALID_ARG;
  if (a->w_layout == RV_W_TILED && (a->dtype != RV_BF16 || a->H % 128 != 0)) return RV_ERR_UNSUPPORTED;
  return RV_OK;
}

hipError_t launch_clear_status(void* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_clear_status, dim3(1), dim3(64), 0, s, status_ptr(ws));
  return hipGetLastError();
}

}  // namespace rv

using namespace rv;

extern "C" {

const char* rv_version(void) { return "librv 0.1.0 gfx950 (ragged confidence-driven verify)"; }

rv_status rv_workspace_size(const rv_dims* d, size_t* bytes) {
  if (!d || !bytes) return RV_ERR_INVALID_ARG;
  if (d->B < 0 || d->gamma < 0 || d->Hq < 0 || d->Hkv < 0 || d->Dqk < 0 || d->Dv < 0 || d->V < 0)
    return RV_ERR_INVALID_ARG;
  size_t need = 0;
  if (d->B > 0 && d->gamma > 0 && d->Hq > 0 && d->Hkv > 0 && d->Dqk > 0 && d->Dv > 0)
    need = attn_scratch_bytes(d->B, d->gamma, d->Hq, d->Hkv, d->Dqk, d->Dv, d->dtype);
  if (d->B > 0 && d->gamma > 0 && d->V > 0) {
    const size_t lm = lm_scratch_bytes(d->B, d->gamma, d->V);
    if (lm > need) need = lm;
  }
  *bytes = (size_t)kStatusBytes + need;
  return RV_OK;
}

rv_status rv_device_status(const void* workspace, int32_t* code, void* stream) {
  if (!workspace || !code) return RV_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(code, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return RV_ERR_HIP;
  return hip_status(hipStreamSynchronize(s));
}

rv_status rv_clear_status(void* workspace, void* stream) {
  if (!workspace) return RV_ERR_INVALID_ARG;
  return hip_status(launch_clear_status(workspace, static_cast<hipStream_t>(stream)));
}

rv_status rv_schedule(const rv_schedule_args* a, void* stream) {
  if (!a || !a->conf || !a->cost_alpha || !a->cost_theta || !a->w_commit || !a->w_verify ||
      !a->k_star || !a->e_star)
    return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if (a->mode < RV_STATIC || a->mode > RV_NO_TRIM) return RV_ERR_INVALID_ARG;
  if ((a->mode == RV_COMPACT || a->mode == RV_CAP_ACCEPT) &&
      (long long)a->B * (a->gamma - 1) > RV_MAX_SCHED_CANDIDATES)
    return RV_ERR_UNSUPPORTED;
  if (a->alpha_len <= a->B || (long long)a->theta_len <= (long long)a->B * a->gamma) return RV_ERR_INVALID_ARG;
  if (!isfinite(a->cost_bias)) return RV_ERR_INVALID_ARG;
  if (!ws_ok(a->workspace, a->workspace_bytes, kStatusBytes)) return RV_ERR_WORKSPACE;
  return hip_status(launch_schedule(*a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

rv_status pack_args_check(const rv_pack_args* a) {
  if (!a || !a->w_verify || !a->anchor || !a->drafts || !a->ctx || !a->page_table || !a->cu ||
      !a->mm || !a->row_req || !a->row_pos || !a->tok || !a->slot)
    return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if (a->page_size < 1 || a->max_pages < 1 || a->num_pages < 1) return RV_ERR_INVALID_ARG;
  if ((long long)a->rows_cap < (long long)a->B * a->gamma) return RV_ERR_INVALID_ARG;
  if (a->n_tiers < 0 || a->n_tiers > RV_MAX_TIERS) return RV_ERR_TIER;
  if (a->n_tiers > 0) {
    if (!a->tiers) return RV_ERR_TIER;
    for (int k = 0; k < a->n_tiers; ++k) {
      if (a->tiers[k] < 1 || (k > 0 && a->tiers[k] <= a->tiers[k - 1])) return RV_ERR_TIER;
    }
    if (a->tiers[a->n_tiers - 1] > a->rows_cap) return RV_ERR_TIER;
  }
  if (!ws_ok(a->workspace, a->workspace_bytes, kStatusBytes)) return RV_ERR_WORKSPACE;
  return RV_OK;
}

rv_status attn_args_check(const rv_attn_args* a) {
  if (!a || !a->q || !a->k_cache || !a->page_table || !a->ctx || !a->cu || !a->mm || !a->o)
    return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if ((long long)a->rows_cap < (long long)a->B * a->gamma) return RV_ERR_INVALID_ARG;
  if (a->page_size < 1 || a->max_pages < 1 || a->num_pages < 1) return RV_ERR_INVALID_ARG;
  if (a->Hq < 1 || a->Hkv < 1 || a->Dqk < 1 || a->Dv < 1 || a->Hq % a->Hkv != 0) return RV_ERR_INVALID_ARG;
  if (a->dtype != RV_F32 && a->dtype != RV_BF16) return RV_ERR_INVALID_ARG;
  if (!isfinite(a->sm_scale) || a->window < 0) return RV_ERR_INVALID_ARG;
  const bool latent = (a->v_cache == nullptr);
  if (latent && (a->Hkv != 1 || a->Dv > a->Dqk)) return RV_ERR_UNSUPPORTED;
  if (!attn_shape_supported(a->Hq, a->Hkv, a->Dqk, a->Dv, a->dtype, latent)) return RV_ERR_UNSUPPORTED;
  if (a->topk_idx && (!latent || a->dtype != RV_BF16 || a->window != 0)) return RV_ERR_UNSUPPORTED;
  if (a->topk_idx && (a->topk < 1 || a->topk > RV_MAX_TOPK)) return RV_ERR_INVALID_ARG;
  if (a->topk_idx && (long long)a->num_pages * a->page_size >= (1ll << 31)) return RV_ERR_UNSUPPORTED;
  if (a->max_pages > attn_max_pages_limit(a->dtype, latent)) return RV_ERR_UNSUPPORTED;
  const size_t need = kStatusBytes + attn_scratch_bytes(a->B, a->gamma, a->Hq, a->Hkv, a->Dqk, a->Dv, a->dtype);
  if (!ws_ok(a->workspace, a->workspace_bytes, need)) return RV_ERR_WORKSPACE;
  return RV_OK;
}

}  // namespace

extern "C" {

rv_status rv_pack(const rv_pack_args* a, void* stream) {
  const rv_status st = pack_args_check(a);
  if (st != RV_OK) return st;
  return hip_status(launch_pack(*a, static_cast<hipStream_t>(stream)));
}

rv_status rv_verify_attn(const rv_attn_args* a, void* stream) {
  const rv_status st = attn_args_check(a);
  if (st != RV_OK) return st;
  return hip_status(launch_attn(*a, static_cast<hipStream_t>(stream)));
}

rv_status rv_pack_plan(const rv_pack_args* pack, const rv_attn_args* attn, void* stream) {
  rv_status st = pack_args_check(pack);
  if (st != RV_OK) return st;
  if ((st = attn_args_check(attn)) != RV_OK) return st;
  // the plan reads the pack's outputs for the same requests
  if (attn->cu != pack->cu || attn->mm != pack->mm || attn->ctx != pack->ctx || attn->B != pack->B ||
      attn->gamma != pack->gamma)
    return RV_ERR_INVALID_ARG;
  return hip_status(launch_pack_plan(*pack, *attn, static_cast<hipStream_t>(stream)));
}

rv_status rv_verify_attn_planned(const rv_attn_args* a, void* stream) {
  const rv_status st = attn_args_check(a);
  if (st != RV_OK) return st;
  return hip_status(launch_attn(*a, static_cast<hipStream_t>(stream), true));
}

rv_status rv_lm_head_accept(const rv_lm_args* a, void* stream) {
  const rv_status st = lm_args_check(a);
  if (st != RV_OK) return st;
  const size_t need = kStatusBytes + lm_scratch_bytes(a->B, a->gamma, a->V);
  if (!ws_ok(a->workspace, a->workspace_bytes, need)) return RV_ERR_WORKSPACE;
  return hip_status(launch_lm(*a, static_cast<char*>(a->workspace) + kStatusBytes, status_ptr(a->workspace),
                              static_cast<hipStream_t>(stream)));
}

rv_status rv_lm_tiled_weight_bytes(int32_t V, int32_t H, int32_t dtype, size_t* bytes) {
  if (!bytes || V < 1 || H < 128 || H % 128 != 0) return RV_ERR_INVALID_ARG;
  if (dtype != RV_BF16) return RV_ERR_UNSUPPORTED;
  *bytes = lm_tiled_weight_bytes(V, H);
  return RV_OK;
}

rv_status rv_lm_tile_weight(const void* W, void* W_tiled, int32_t V, int32_t H, int32_t dtype, void* stream) {
  if (!W || !W_tiled || V < 1 || H < 128 || H % 128 != 0) return RV_ERR_INVALID_ARG;
  if (dtype != RV_BF16) return RV_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(W) % 16 != 0 || reinterpret_cast<uintptr_t>(W_tiled) % 16 != 0)
    return RV_ERR_INVALID_ARG;
  return hip_status(launch_lm_tile_weight(W, W_tiled, V, H, static_cast<hipStream_t>(stream)));
}

rv_status rv_calibration(const rv_calib_args* a, void* stream) {
  if (!a || !a->conf || !a->drafts || !a->pred || !a->cu || !a->w_verify || !a->bin_count || !a->bin_match ||
      !a->bin_conf_fx || !a->ece)
    return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if (a->n_bins < 1 || a->n_bins > RV_MAX_CALIB_BINS) return RV_ERR_INVALID_ARG;
  if ((long long)a->rows_cap < (long long)a->B * a->gamma) return RV_ERR_INVALID_ARG;
  if (!ws_ok(a->workspace, a->workspace_bytes, kStatusBytes)) return RV_ERR_WORKSPACE;
  return hip_status(launch_calibration(*a, static_cast<hipStream_t>(stream)));
}

rv_status rv_estimator_state_bytes(int32_t B, int32_t gamma, size_t* bytes) {
  if (!bytes || !block_ok(B, gamma)) return RV_ERR_INVALID_ARG;
  *bytes = estimator_state_bytes(B, gamma);
  return RV_OK;
}

rv_status rv_block_accept_estimate(const rv_estimate_args* a, void* stream) {
  if (!a || !a->cu || !a->w_verify || !a->accept || !a->drafts || !a->ctx || !a->state) return RV_ERR_INVALID_ARG;
  if (a->rule != RV_GREEDY && a->rule != RV_REJECTION) return RV_ERR_INVALID_ARG;
  if (a->rule == RV_GREEDY && !a->pred) return RV_ERR_INVALID_ARG;
  if (a->rule == RV_REJECTION && (!a->logits || !a->q_rows)) return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if ((long long)a->rows_cap < (long long)a->B * a->gamma || a->V < 1) return RV_ERR_INVALID_ARG;
  if (!ws_ok(a->workspace, a->workspace_bytes, kStatusBytes)) return RV_ERR_WORKSPACE;
  return hip_status(launch_estimate(*a, static_cast<hipStream_t>(stream)));
}

rv_status rv_fit_cost_model(const double* bs, const double* M, const double* t, int32_t n, double* coef,
                            double* alpha, int32_t alpha_len, double* theta, int32_t theta_len) {
  if (!bs || !M || !t || !coef || n < 3) return RV_ERR_INVALID_ARG;
  if ((alpha && alpha_len < 0) || (theta && theta_len < 0)) return RV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!isfinite(bs[i]) || !isfinite(M[i]) || !isfinite(t[i])) return RV_ERR_INVALID_ARG;
  // columns of the design matrix: 1, bs, M; orthonormalised in place
  std::vector<double> q[3];
  for (int j = 0; j < 3; ++j) q[j].resize(n);
  for (int32_t i = 0; i < n; ++i) {
    q[0][i] = 1.0;
    q[1][i] = bs[i];
    q[2][i] = M[i];
  }
  auto dot = [n](const std::vector<double>& x, const std::vector<double>& y) {
    double acc = 0.0;
    for (int32_t i = 0; i < n; ++i) acc += x[i] * y[i];
    return acc;
  };
  double R[3][3] = {{0.0}};
  for (int j = 0; j < 3; ++j) {
    const double norm0 = sqrt(dot(q[j], q[j]));
    for (int pass = 0; pass < 2; ++pass)   // Gram-Schmidt twice keeps Q orthogonal
      for (int k = 0; k < j; ++k) {
        const double r = dot(q[k], q[j]);
        R[k][j] += r;
        for (int32_t i = 0; i < n; ++i) q[j][i] -= r * q[k][i];
      }
    R[j][j] = sqrt(dot(q[j], q[j]));
    if (!(norm0 > 0.0) || !(R[j][j] > 1e-12 * norm0)) return RV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) q[j][i] /= R[j][j];
  }
  std::vector<double> tv(t, t + n);
  double y[3], x[3];
  for (int j = 0; j < 3; ++j) y[j] = dot(q[j], tv);
  for (int j = 2; j >= 0; --j) {
    double acc = y[j];
    for (int k = j + 1; k < 3; ++k) acc -= R[j][k] * x[k];
    x[j] = acc / R[j][j];
  }
  for (int j = 0; j < 3; ++j) coef[j] = x[j];
  if (alpha)
    for (int32_t b = 0; b < alpha_len; ++b) alpha[b] = x[1] * (double)b;
  if (theta)
    for (int32_t m = 0; m < theta_len; ++m) theta[m] = x[2] * (double)m;
  return RV_OK;
}

rv_status rv_compact_scatter(const rv_scatter_args* a, void* stream) {
  if (!a || !a->cu || !a->w_verify || !a->accept || !a->bonus || !a->drafts || !a->slot || !a->ctx ||
      !a->anchor || !a->req_to_token || !a->commit_cu || !a->commit_tok || !a->commit_slot ||
      !a->free_slots || !a->free_count)
    return RV_ERR_INVALID_ARG;
  if ((a->hist == nullptr) != (a->hist_len == nullptr)) return RV_ERR_INVALID_ARG;
  if (!block_ok(a->B, a->gamma)) return RV_ERR_INVALID_ARG;
  if (a->r2t_stride < 1 || (a->hist && a->hist_stride < 1)) return RV_ERR_INVALID_ARG;
  if (!ws_ok(a->workspace, a->workspace_bytes, kStatusBytes)) return RV_ERR_WORKSPACE;
  return hip_status(launch_scatter(*a, static_cast<hipStream_t>(stream)));
}

#define RV_OFF(S, f) (int64_t) offsetof(S, f)

int32_t rv_abi_layout(int32_t which, int64_t* out, int32_t cap) {
  int64_t v[48];
  int n = 0;
  switch (which) {
    case 0: {
      typedef rv_schedule_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, conf), RV_OFF(S, B), RV_OFF(S, gamma), RV_OFF(S, mode),
                     RV_OFF(S, alpha_len), RV_OFF(S, theta_len), RV_OFF(S, _pad0), RV_OFF(S, cost_bias),
                     RV_OFF(S, cost_alpha), RV_OFF(S, cost_theta), RV_OFF(S, w_commit), RV_OFF(S, w_verify),
                     RV_OFF(S, k_star), RV_OFF(S, e_star), RV_OFF(S, workspace), RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 1: {
      typedef rv_pack_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, w_verify), RV_OFF(S, anchor), RV_OFF(S, drafts), RV_OFF(S, ctx),
                     RV_OFF(S, page_table), RV_OFF(S, B), RV_OFF(S, gamma), RV_OFF(S, max_pages),
                     RV_OFF(S, page_size), RV_OFF(S, num_pages), RV_OFF(S, n_tiers), RV_OFF(S, tiers),
                     RV_OFF(S, rows_cap), RV_OFF(S, _pad0), RV_OFF(S, cu), RV_OFF(S, mm), RV_OFF(S, row_req),
                     RV_OFF(S, row_pos), RV_OFF(S, tok), RV_OFF(S, slot), RV_OFF(S, workspace),
                     RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 2: {
      typedef rv_attn_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, q), RV_OFF(S, k_cache), RV_OFF(S, v_cache), RV_OFF(S, page_table),
                     RV_OFF(S, ctx), RV_OFF(S, cu), RV_OFF(S, mm), RV_OFF(S, B), RV_OFF(S, gamma),
                     RV_OFF(S, rows_cap), RV_OFF(S, max_pages), RV_OFF(S, page_size), RV_OFF(S, num_pages),
                     RV_OFF(S, Hq), RV_OFF(S, Hkv), RV_OFF(S, Dqk), RV_OFF(S, Dv), RV_OFF(S, dtype),
                     RV_OFF(S, sm_scale), RV_OFF(S, window), RV_OFF(S, topk), RV_OFF(S, topk_idx), RV_OFF(S, o), RV_OFF(S, lse), RV_OFF(S, workspace),
                     RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 3: {
      typedef rv_lm_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, hidden), RV_OFF(S, W), RV_OFF(S, mm), RV_OFF(S, cu),
                     RV_OFF(S, w_commit), RV_OFF(S, w_verify), RV_OFF(S, drafts), RV_OFF(S, q_rows),
                     RV_OFF(S, u), RV_OFF(S, u_bonus), RV_OFF(S, B), RV_OFF(S, gamma), RV_OFF(S, rows_cap),
                     RV_OFF(S, H), RV_OFF(S, V), RV_OFF(S, dtype), RV_OFF(S, rule), RV_OFF(S, w_layout),
                     RV_OFF(S, pred), RV_OFF(S, accept), RV_OFF(S, bonus), RV_OFF(S, ceiling),
                     RV_OFF(S, logits), RV_OFF(S, workspace), RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 4: {
      typedef rv_scatter_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, cu), RV_OFF(S, w_verify), RV_OFF(S, accept), RV_OFF(S, bonus),
                     RV_OFF(S, drafts), RV_OFF(S, slot), RV_OFF(S, B), RV_OFF(S, gamma), RV_OFF(S, r2t_stride),
                     RV_OFF(S, hist_stride), RV_OFF(S, ctx), RV_OFF(S, anchor), RV_OFF(S, req_to_token),
                     RV_OFF(S, hist), RV_OFF(S, hist_len), RV_OFF(S, commit_cu), RV_OFF(S, commit_tok),
                     RV_OFF(S, commit_slot), RV_OFF(S, free_slots), RV_OFF(S, free_count),
                     RV_OFF(S, workspace), RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 6: {
      typedef rv_calib_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, conf), RV_OFF(S, drafts), RV_OFF(S, pred), RV_OFF(S, cu),
                     RV_OFF(S, w_verify), RV_OFF(S, B), RV_OFF(S, gamma), RV_OFF(S, rows_cap), RV_OFF(S, n_bins),
                     RV_OFF(S, bin_count), RV_OFF(S, bin_match), RV_OFF(S, bin_conf_fx), RV_OFF(S, ece),
                     RV_OFF(S, req_verified), RV_OFF(S, req_matched), RV_OFF(S, workspace),
                     RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 7: {
      typedef rv_estimate_args S;
      int64_t t[] = {sizeof(S), RV_OFF(S, cu), RV_OFF(S, w_verify), RV_OFF(S, accept), RV_OFF(S, drafts),
                     RV_OFF(S, ctx), RV_OFF(S, pred), RV_OFF(S, logits), RV_OFF(S, q_rows), RV_OFF(S, B),
                     RV_OFF(S, gamma), RV_OFF(S, rows_cap), RV_OFF(S, V), RV_OFF(S, rule), RV_OFF(S, _pad0),
                     RV_OFF(S, state), RV_OFF(S, workspace), RV_OFF(S, workspace_bytes)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    case 5: {
      typedef rv_dims S;
      int64_t t[] = {sizeof(S), RV_OFF(S, B), RV_OFF(S, gamma), RV_OFF(S, Hq), RV_OFF(S, Hkv),
                     RV_OFF(S, Dqk), RV_OFF(S, Dv), RV_OFF(S, V), RV_OFF(S, dtype)};
      n = sizeof(t) / sizeof(t[0]);
      for (int k = 0; k < n; ++k) v[k] = t[k];
      break;
    }
    default:
      return -1;
  }
  if (!out || cap < n) return -1;
  for (int k = 0; k < n; ++k) out[k] = v[k];
  return n;
}

}  // extern "C"
