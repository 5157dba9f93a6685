/*
 * rv.h -- C ABI of the ragged, confidence-driven verify step (librv.so).
 *
 * The step is the verify half of DSpark speculative decoding as described on
 * the page "DSpark in SGLang: Speculative Decoding with Confidence-Driven,
 * Variable-Length Verification" (papercache.org summary of the LMSYS blog,
 * below: the DSpark-in-SGLang page).  Five calls, run in this order on one
 * stream:
 *
 *   rv_schedule        per-request verify windows from draft confidences
 *   rv_pack            front-pack the windows into a cu_seqlens buffer
 *   rv_verify_attn     varlen causal attention of packed rows, paged KV
 *   rv_pack_plan, rv_verify_attn_planned
 *                      the same two stages with the attention plan built in
 *                      the pack launch
 *   rv_lm_head_accept  target LM head, argmax / min(1,p/q) accept
 *   rv_compact_scatter write committed tokens and KV slots back
 *
 * Conventions shared by every call
 * --------------------------------
 * - All array pointers are DEVICE memory owned by the caller unless a field
 *   says "host".  Arrays are dense, row-major, with the shapes given per field.
 *   Integers are int32, confidences/uniforms float32, cost tables float64.
 * - Block layout: each request has a block of `gamma` positions; position 0 is
 *   the anchor (the last committed token, whose KV is written but not yet
 *   committed) and positions 1..gamma-1 hold drafts d_1..d_{gamma-1}.  A window
 *   w in [1, gamma] counts packed rows.  Row k of request i sits at sequence
 *   position ctx[i] + k and its prediction checks draft d_{k+1}.
 * - Every call only enqueues work on `stream` (a hipStream_t, NULL = default
 *   stream) and returns; nothing is synchronised and nothing is allocated.
 *   Scratch memory comes from `workspace` (size from rv_workspace_size); the
 *   first 256 bytes of a workspace hold a sticky device status word.
 *   Distinct workspaces make concurrent calls independent.
 * - Host-checkable problems (NULL pointers, sizes out of range, unsupported
 *   shapes, workspace too small) return a negative rv_status before anything
 *   is enqueued.  Data problems found on the device (confidence outside [0,1],
 *   window outside [1,gamma], page or token index out of range, packed total
 *   above the largest tier, history overflow, non-positive step time) set the
 *   sticky device status (first error wins, read with rv_device_status); the
 *   kernels then keep every access in bounds and give the offending request a
 *   defined result, as stated per call.
 * - Nothing in the library aborts the process.
 */
#ifndef RV_H_
#define RV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes (host return values) ---------------------------------- */
#define RV_OK 0
#define RV_ERR_INVALID_ARG (-1)   /* NULL pointer or size out of range */
#define RV_ERR_UNSUPPORTED (-2)   /* shape/dtype combination not built */
#define RV_ERR_TIER (-3)          /* tier list not ascending, or too long */
#define RV_ERR_WORKSPACE (-4)     /* workspace NULL or smaller than needed */
#define RV_ERR_HIP (-5)           /* a HIP runtime call failed */
#define RV_ERR_SCRATCH (-6)       /* problem larger than rv_lm_head_accept_noalloc's
                                     static scratch (RV_NOALLOC_SCRATCH_BYTES) */
typedef int32_t rv_status;

/* ---- sticky device status codes (rv_device_status) ---------------------- */
#define RV_DEV_OK 0
#define RV_DEV_BAD_CONF 1         /* confidence NaN or outside [0, 1] */
#define RV_DEV_BAD_COST 2         /* step time not positive (or NaN) */
#define RV_DEV_BAD_WINDOW 3       /* window outside [1, gamma] */
#define RV_DEV_TIER_OVERFLOW 4    /* packed total above the largest tier */
#define RV_DEV_BAD_PAGE 5         /* page-table entry outside [0, num_pages) */
#define RV_DEV_BAD_TOKEN 6        /* token id outside [0, V) */
#define RV_DEV_HIST_OVERFLOW 7    /* history or req_to_token row too short */

/* ---- enums ---------------------------------------------------------------- */
/* Verify modes, DSpark-in-SGLang page, section A2 (verify modes) and A3
 * (no-trim): static verifies and commits full blocks; compact verifies and
 * commits the scheduled windows; cap-accept verifies full blocks and commits up
 * to the scheduled window; no-trim is compact without a cost table (full
 * windows, ragged path). */
#define RV_STATIC 0
#define RV_COMPACT 1
#define RV_CAP_ACCEPT 2
#define RV_NO_TRIM 3

/* Acceptance rules: greedy (drafts kept up to the first disagreement with
 * the target argmax) and rejection sampling (keep x with probability
 * min(1, p(x)/q(x))); lshu.cn DSpark explainer, sections 1.2, 2.3, 3.3. */
#define RV_GREEDY 0
#define RV_REJECTION 1

/* Element types of the floating-point payloads. */
#define RV_F32 0
#define RV_BF16 1

/* LM-head weight layout (rv_lm_args.w_layout) */
#define RV_W_ROWS 0    /* W is [V][H], row-major */
#define RV_W_TILED 1   /* W is the tiled copy written by rv_lm_tile_weight (bf16) */

/* Limits of this build. */
#define RV_MAX_GAMMA 16
#define RV_MAX_TIERS 16
#define RV_MAX_SCHED_CANDIDATES 4096   /* B * (gamma - 1), compact/cap-accept */
#define RV_MAX_ROWS 8192               /* B * gamma */
#define RV_MAX_TOPK 2048               /* sparse latent attention: index entries per row */

/* ---- sizing ------------------------------------------------------------- */
/* Upper bounds of the problem a workspace must serve.  Any field may be 0 when
 * the corresponding call is never made with that workspace (e.g. H = V = 0 if
 * rv_lm_head_accept is not used). */
typedef struct {
  int32_t B;          /* requests */
  int32_t gamma;      /* block width (anchor + drafts) */
  int32_t Hq;         /* query heads */
  int32_t Hkv;        /* KV heads (1 for the latent layout) */
  int32_t Dqk;        /* query/key head dim */
  int32_t Dv;         /* value head dim */
  int32_t V;          /* vocabulary size */
  int32_t dtype;      /* RV_F32 or RV_BF16 */
} rv_dims;

/* Library version string (static storage). */
const char* rv_version(void);

/* Bytes of workspace the five calls need for problems bounded by *dims.
 * Host-only, pure.  Returns RV_ERR_INVALID_ARG on NULL or negative fields. */
rv_status rv_workspace_size(const rv_dims* dims, size_t* bytes);

/* Copies the sticky device status of `workspace` to *code (host) after
 * synchronising `stream`.  Returns RV_ERR_HIP if the copy fails. */
rv_status rv_device_status(const void* workspace, int32_t* code, void* stream);

/* Enqueues a reset of the sticky device status to RV_DEV_OK (a kernel, not a
 * memset, so the call may sit inside a captured graph). */
rv_status rv_clear_status(void* workspace, void* stream);

/* ---- stage 1: confidence scheduler -------------------------------------- */
/* DSpark-in-SGLang page: section A2 (the confidence head scores each draft;
 * the product of scores over the block is its survival probability; the
 * scheduler turns survival into per-request verify budgets), section 速读 and
 * A2 "cost-table profiling" (T(bs,K) = bias + alpha(bs) + theta(M), M = bs+K;
 * the argmax trades expected accepted tokens against marginal cost).
 *
 * Computes S[i,k] = prod_{j<=k} conf[i,j] left to right in fp64, ranks all
 * (i,k), k>=1, by (S desc, i asc, k asc), and for K = 0..B*(gamma-1) evaluates
 * R(K) = (B*2^40 + sum_{first K} floor(S*2^40)) / ((bias + alpha[B]) +
 * theta[B+K]) with int64 sums and one fp64 divide; K* is the first maximiser
 * and w_i = 1 + #{ranked-first-K* candidates of request i}.  static / no-trim:
 * w = gamma.  Outputs are bit-identical to a sequential evaluation. */
typedef struct {
  const float* conf;         /* [B][gamma-1] draft confidences in [0,1] */
  int32_t B;                 /* 1..RV_MAX_ROWS/gamma */
  int32_t gamma;             /* 2..RV_MAX_GAMMA */
  int32_t mode;              /* RV_STATIC / RV_COMPACT / RV_CAP_ACCEPT / RV_NO_TRIM */
  int32_t alpha_len;         /* entries of cost_alpha, must exceed B */
  int32_t theta_len;         /* entries of cost_theta, must exceed B*gamma */
  int32_t _pad0;
  double cost_bias;          /* host value, ms */
  const double* cost_alpha;  /* [alpha_len] alpha(bs), ms */
  const double* cost_theta;  /* [theta_len] theta(M), ms */
  int32_t* w_commit;         /* out [B] rows whose verdicts may be committed */
  int32_t* w_verify;         /* out [B] rows packed and verified */
  int32_t* k_star;           /* out [1] extra verify tokens K* */
  double* e_star;            /* out [1] expected committed tokens at K* */
  void* workspace;
  size_t workspace_bytes;
} rv_schedule_args;
/* Device errors: BAD_CONF (that confidence counts as 0), BAD_COST (windows
 * fall back to 1). */
rv_status rv_schedule(const rv_schedule_args* a, void* stream);

/* ---- stage 2: ragged front-packing -------------------------------------- */
/* DSpark-in-SGLang page, section A2 "ragged verify over a full CUDA graph"
 * and Fig. 2: windows are front-packed into one compact cu_seqlens-style
 * buffer with no per-request padding, and only the total is rounded up to the
 * nearest captured tier.
 *
 * cu = exclusive scan of w_verify (cu[B] = M); M_pad = smallest tier >= M (M
 * when n_tiers == 0).  For row r = cu[i] + k: row_req = i, row_pos = ctx[i]+k,
 * tok = anchor[i] (k == 0) or drafts[i][k-1], slot = page_table[i][pos/P]*P +
 * pos%P.  Rows [M, M_pad) get -1 in all four arrays; rows >= M_pad are not
 * written. */
typedef struct {
  const int32_t* w_verify;   /* [B] windows from rv_schedule */
  const int32_t* anchor;     /* [B] anchor token per request */
  const int32_t* drafts;     /* [B][gamma-1] */
  const int32_t* ctx;        /* [B] committed tokens before the anchor */
  const int32_t* page_table; /* [B][max_pages] KV page per page_size positions */
  int32_t B, gamma;
  int32_t max_pages;         /* row stride of page_table */
  int32_t page_size;         /* positions per page, >= 1 */
  int32_t num_pages;         /* pages in the KV cache (bounds check) */
  int32_t n_tiers;           /* 0..RV_MAX_TIERS */
  const int32_t* tiers;      /* HOST [n_tiers], strictly ascending, > 0 */
  int32_t rows_cap;          /* rows of the four row arrays, >= B*gamma */
  int32_t _pad0;
  int32_t* cu;               /* out [B+1] */
  int32_t* mm;               /* out [2] = {M, M_pad} */
  int32_t* row_req;          /* out [rows_cap] */
  int32_t* row_pos;          /* out [rows_cap] */
  int32_t* tok;              /* out [rows_cap] */
  int32_t* slot;             /* out [rows_cap] */
  void* workspace;
  size_t workspace_bytes;
} rv_pack_args;
/* Device errors: BAD_WINDOW (window clamped to [1,gamma]), TIER_OVERFLOW
 * (M_pad = M, still within rows_cap), BAD_PAGE (slot = -1). */
rv_status rv_pack(const rv_pack_args* a, void* stream);

/* ---- stage 3: verify attention ------------------------------------------ */
/* DSpark-in-SGLang page, section A2: the packed buffer uses a cu_seqlens-style
 * variable-length layout so compact verify reuses the backend's varlen
 * attention (native sparse-MLA on DeepSeek-V4); each backend rebuilds its
 * varlen metadata for the packed layout.
 *
 * For every real row r (request i, row k, position p = ctx[i]+k) and query
 * head h (KV head g = h / (Hq/Hkv)): o[r,h] = softmax_j(sm_scale * q[r,h] .
 * K[i,j,g]) V[i,j,g] over keys j = 0..p read through the page table (with
 * window W > 0, the sliding-window layers' attention: keys j = max(0,p-W+1)..p;
 * with topk_idx, sparse latent attention as on the DeepSeek-V4 path (the
 * page names its sparse-MLA kernel): the keys are the positions
 * topk_idx[r][0..topk-1] in list order, entries outside 0..p (e.g. -1 for
 * unused slots) skipped; a repeated position counts once per entry; latent
 * bf16 layout only, topk <= 2048, window 0);
 * lse[r,h] = natural log of the softmax normaliser.  Latent layout
 * (v_cache == NULL, Hkv == 1): V[i,j] = first Dv entries of K[i,j].  Rows
 * [M, M_pad) get o = 0, lse = -inf; rows >= M_pad are not written.
 *
 * Built shapes: dtype RV_BF16 with (Dqk,Dv) = (576,512) latent, Hq % 64 == 0,
 * or (128,128) with Hq/Hkv in {1,2,4,8,16}, both with max_pages <= 2047 (the
 * bf16 kernels hold a request's page-table entries in an LDS window); dtype
 * RV_F32 with Dqk = Dv <= 128 (any group).  bf16 accumulates in fp32. */
typedef struct {
  const void* q;             /* [rows_cap][Hq][Dqk] packed queries, dtype */
  const void* k_cache;       /* [num_pages][page_size][Hkv][Dqk], dtype */
  const void* v_cache;       /* [num_pages][page_size][Hkv][Dv] or NULL (latent) */
  const int32_t* page_table; /* [B][max_pages] */
  const int32_t* ctx;        /* [B] */
  const int32_t* cu;         /* [B+1] from rv_pack */
  const int32_t* mm;         /* [2] {M, M_pad} from rv_pack */
  int32_t B, gamma;          /* requests; block width (bounds every window) */
  int32_t rows_cap, max_pages, page_size, num_pages;
  int32_t Hq, Hkv, Dqk, Dv, dtype;
  float sm_scale;            /* multiplies q.k (e.g. 1/sqrt(Dqk)) */
  int32_t window;            /* sliding window in keys; 0 = full causal */
  int32_t topk;              /* entries per row of topk_idx */
  const int32_t* topk_idx;   /* NULL, or [rows_cap][topk] sparse key positions */
  void* o;                   /* out [rows_cap][Hq][Dv], dtype */
  float* lse;                /* out [rows_cap][Hq] or NULL */
  void* workspace;
  size_t workspace_bytes;
} rv_attn_args;
/* Device errors: BAD_PAGE (the key is read from page 0 instead). */
rv_status rv_verify_attn(const rv_attn_args* a, void* stream);

/* Stage 2 with the plan of stage 3 in the same launch.  The attention call's
 * device-side plan (how the packed rows' tiles and key chunks are dealt to
 * the persistent workgroups; DSpark-in-SGLang page, section A2: each backend
 * rebuilds its varlen metadata for the packed layout) depends only on cu[],
 * ctx[] and the call's shape, so one workgroup can pack and then plan.
 * rv_pack_plan(pack, attn) does what rv_pack(pack) does and leaves in
 * attn->workspace the plan that rv_verify_attn(attn) would build; attn must
 * name the pack's cu, mm and ctx arrays and the same B and gamma (otherwise
 * RV_ERR_INVALID_ARG), and both argument sets are checked as by rv_pack and
 * rv_verify_attn.  rv_verify_attn_planned(attn) is then stage 3 without its
 * plan launch: it must follow rv_pack_plan with the same attention arguments
 * on the same stream, with nothing written to the workspace in between (the
 * plan is not checked).  For RV_F32 attention, which has no plan,
 * rv_pack_plan is rv_pack and rv_verify_attn_planned is rv_verify_attn. */
rv_status rv_pack_plan(const rv_pack_args* pack, const rv_attn_args* attn, void* stream);
rv_status rv_verify_attn_planned(const rv_attn_args* a, void* stream);

/* ---- stage 4: LM head + accept ------------------------------------------ */
/* Target LM head over the packed rows (z = W h, fp32 accumulation) and the
 * acceptance rule (lshu.cn DSpark explainer: section 1.2 greedy first-mismatch,
 * sections 2.3/3.3 min(1,p/q)); cap-accept ceiling (DSpark-in-SGLang page,
 * section A2 "verify modes" and "observability").
 *
 * pred[r] = lowest index of the maximal logit of real row r; -1 for rows
 * [M, M_pad).  Per request i (rows cu[i]..cu[i]+w_verify[i]-1):
 *  greedy:    ceiling = leading j with drafts[i][j-1] == pred[cu[i]+j-1];
 *  rejection: p = softmax(z) (T=1), accept draft j iff
 *             u[i][j-1] * q_rows[i][j-1][d_j] < p_{row j-1}(d_j), stop at the
 *             first reject;
 *  accept = min(ceiling, w_commit[i]-1);
 *  bonus (greedy) = pred at row accept; bonus (rejection) = inverse-CDF draw
 *  with u_bonus[i] from max(0, p_{row c} - q_{c+1}) after a reject at draft
 *  c+1 <= w_commit-1, else from p at row w_commit-1 (smallest v whose running
 *  mass exceeds u_bonus * total). */
typedef struct {
  const void* hidden;        /* [rows_cap][H] packed final hidden states, dtype */
  const void* W;             /* [V][H] LM-head weight, dtype; or its tiled
                                copy (w_layout = RV_W_TILED) */
  const int32_t* mm;         /* [2] {M, M_pad} */
  const int32_t* cu;         /* [B+1] */
  const int32_t* w_commit;   /* [B] */
  const int32_t* w_verify;   /* [B] */
  const int32_t* drafts;     /* [B][gamma-1] */
  const float* q_rows;       /* [B][gamma-1][V] draft distributions (rejection) */
  const float* u;            /* [B][gamma-1] uniforms (rejection) */
  const float* u_bonus;      /* [B] uniforms (rejection) */
  int32_t B, gamma, rows_cap, H, V, dtype, rule;
  int32_t w_layout;          /* RV_W_ROWS, or RV_W_TILED (bf16, H % 128 == 0) */
  int32_t* pred;             /* out [rows_cap] */
  int32_t* accept;           /* out [B] accepted drafts */
  int32_t* bonus;            /* out [B] bonus token */
  int32_t* ceiling;          /* out [B] accepts over all verified rows */
  float* logits;             /* out [rows_cap][V] fp32 (required for
                                rejection, optional for greedy, real rows) */
  void* workspace;
  size_t workspace_bytes;
} rv_lm_args;
/* Host errors: UNSUPPORTED for the rejection rule with V above 2^22.
 * Device errors: BAD_TOKEN for a draft outside [0,V) (it never matches;
 * under rejection it is rejected), BAD_WINDOW. */
rv_status rv_lm_head_accept(const rv_lm_args* a, void* stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): rv_lm_head_accept
 * with the same arguments and results, but its scratch memory (the slab
 * partials: 16 bytes per row of B*gamma and 64-column vocabulary slab) is a
 * static device array of RV_NOALLOC_SCRATCH_BYTES held by the library, one
 * copy per GPU, until the process ends; the call allocates nothing.
 * `workspace` is optional here: NULL, or a caller buffer of at least 256
 * bytes that receives the sticky device status (read it with
 * rv_device_status); with NULL the status goes to the static array and is
 * not readable.  Host errors: those of rv_lm_head_accept, RV_ERR_WORKSPACE
 * for a status buffer under 256 bytes, RV_ERR_SCRATCH when
 * 256 + 16 * B*gamma * ceil(V/64), rounded up to 256, exceeds
 * RV_NOALLOC_SCRATCH_BYTES.  Every call on one GPU shares its static array:
 * calls that overlap on one GPU (other streams, other threads) race, so a
 * caller serialises them. */
#define RV_NOALLOC_SCRATCH_BYTES (64u << 20)
rv_status rv_lm_head_accept_noalloc(const rv_lm_args* a, void* stream);

/* The LM-head weight in MFMA fragment order, made once when the weight is
 * loaded (as a serving system lays out its weights for its kernels), so that
 * rv_lm_head_accept with w_layout = RV_W_TILED loads each wave's weight
 * operand straight into registers with whole-line reads.  Layout: blocks of
 * 32 vocabulary rows (V rounded up to a multiple of 32; the padding rows are
 * zero), each a run of H/16 fragments of 1 KB; lane l (0..63) of fragment f
 * of block cb holds the 8 bf16 W[32*cb + l%32][16*f + 8*(l/32) .. +7] at byte
 * offset ((cb*(H/16) + f)*64 + l)*16.
 *
 * rv_lm_tiled_weight_bytes: host only, the size of that copy.
 * rv_lm_tile_weight: W [V][H] bf16 (device, caller-owned) -> W_tiled
 * (device, caller-owned, rv_lm_tiled_weight_bytes bytes, 16-byte aligned);
 * enqueued on stream.  Host errors: NULL pointer, V < 1, H < 128 or H not a
 * multiple of 128 (INVALID_ARG); dtype other than bf16 (UNSUPPORTED). */
rv_status rv_lm_tiled_weight_bytes(int32_t V, int32_t H, int32_t dtype, size_t* bytes);
rv_status rv_lm_tile_weight(const void* W, void* W_tiled, int32_t V, int32_t H, int32_t dtype, void* stream);

/* ---- observability: confidence calibration ------------------------------- */
/* DSpark-in-SGLang page, section A2 "observability and ceiling recovery":
 * per-request confidence and calibration metrics (ECE) for post-hoc
 * analysis.  Compact verifies only the scheduled window, so only drafts
 * 1..w_verify-1 carry a verdict; cap-accept verifies the whole block.
 *
 * Per verified draft j of request i (1 <= j <= w_verify[i]-1): confidence
 * c = conf[i][j-1], label = (drafts[i][j-1] == pred[cu[i]+j-1]) (the greedy
 * per-token verdict), bin b = min(floor(c * n_bins), n_bins-1) with c*n_bins
 * one fp64 product.  Outputs (device, caller-owned, written in full):
 * bin_count[b], bin_match[b], bin_conf_fx[b] = sum of floor(c * 2^48) (int64
 * fixed point, so sums are exact and order-free), ece[0] =
 * (sum_b |bin_match[b]*2^48 - bin_conf_fx[b]|) / 2^48 / N (0 when N = 0),
 * and, when not NULL, req_verified[i] (drafts verified) and req_matched[i]
 * (verified drafts equal to the target's prediction).
 * Host errors: NULL required pointer, bad B/gamma, n_bins outside
 * [1, RV_MAX_CALIB_BINS], rows_cap < B*gamma, small workspace.  Device
 * errors: BAD_WINDOW (a w_verify outside [1, gamma]: that request is
 * skipped). */
#define RV_MAX_CALIB_BINS 1024
typedef struct {
  const float* conf;         /* [B][gamma-1] */
  const int32_t* drafts;     /* [B][gamma-1] */
  const int32_t* pred;       /* [rows_cap] from rv_lm_head_accept */
  const int32_t* cu;         /* [B+1] from rv_pack */
  const int32_t* w_verify;   /* [B] */
  int32_t B, gamma, rows_cap, n_bins;
  int64_t* bin_count;        /* out [n_bins] */
  int64_t* bin_match;        /* out [n_bins] */
  int64_t* bin_conf_fx;      /* out [n_bins] */
  double* ece;               /* out [1] */
  int32_t* req_verified;     /* out [B] or NULL */
  int32_t* req_matched;      /* out [B] or NULL */
  void* workspace;           /* status word at its start */
  size_t workspace_bytes;
} rv_calib_args;
rv_status rv_calibration(const rv_calib_args* a, void* stream);

/* ---- observability: block-accept estimator -------------------------------- */
/* DSpark-in-SGLang page, section A2 "the ceiling estimator under truncation":
 * compact mode hides how many tokens the full block would have accepted; the
 * estimator recovers that ceiling from the compact run itself, using the
 * target's token usage and log-probabilities in later steps under the
 * assumption that the anchor behaves alike with and without truncation, as
 * an interval on the counterfactual tail.
 *
 * Called once per step after rv_lm_head_accept and before rv_compact_scatter
 * (ctx = the step's anchor positions).  Per request i, with a = accept[i],
 * w = w_verify[i], rows r0 = cu[i] ..:
 *  - an open probe (next tail position `pos`) is resolved by the rows k in
 *    0..a whose predicted position ctx+k+1 equals pos, in order: verdict
 *    alpha = (pred[r0+k] == tail draft) under greedy, min(1, p(d)/q(d))
 *    under rejection (p = softmax of logits row r0+k, q = the censored
 *    step's draft distribution, stored as log q); S *= alpha; E += S; the
 *    probe closes when its tail is exhausted or S == 0, adding
 *    (w_censored - 1) + E to `sum`, setting `last` and counting it;
 *  - a probe whose next position is <= ctx[i] (steps skipped) is dropped;
 *  - with no probe open and a censored request (w < gamma, a == w - 1), a
 *    probe opens on drafts d_w .. d_{gamma-1} (positions ctx+w ..) and row
 *    r0+a resolves its first draft at once.
 * The open probe's interval is [base + E, base + E + S * left].
 *
 * State: caller-owned device memory of rv_estimator_state_bytes(B, gamma)
 * bytes, zero-filled before the first step (no probe open), structure of
 * arrays with G = gamma-1: int32 pos[B], left[B], done[B], base[B],
 * count[B]; float S[B], E[B], last[B]; double sum[B]; int32 tok[B][G];
 * float lq[B][G] (byte offsets 0, 4B, 8B, 12B, 16B, 20B, 24B, 28B, 32B,
 * 40B, 40B + 4BG).
 * Host errors: NULL required pointer (pred for greedy; logits and q_rows for
 * rejection), bad B/gamma, rows_cap < B*gamma, V < 1, unknown rule, small
 * workspace.  Device errors: BAD_WINDOW (window or accept out of range: that
 * request is skipped), BAD_TOKEN (a tail draft outside [0, V) under
 * rejection: its verdict is 0). */
typedef struct {
  const int32_t* cu;         /* [B+1] this step's packing */
  const int32_t* w_verify;   /* [B] */
  const int32_t* accept;     /* [B] from rv_lm_head_accept */
  const int32_t* drafts;     /* [B][gamma-1] this step's drafts */
  const int32_t* ctx;        /* [B] anchor positions (before the scatter) */
  const int32_t* pred;       /* [rows_cap] row predictions (greedy) */
  const float* logits;       /* [rows_cap][V] (rejection) */
  const float* q_rows;       /* [B][gamma-1][V] draft distributions (rejection) */
  int32_t B, gamma, rows_cap, V, rule;
  int32_t _pad0;
  void* state;               /* in/out, rv_estimator_state_bytes(B, gamma) */
  void* workspace;           /* status word at its start */
  size_t workspace_bytes;
} rv_estimate_args;
rv_status rv_estimator_state_bytes(int32_t B, int32_t gamma, size_t* bytes);
rv_status rv_block_accept_estimate(const rv_estimate_args* a, void* stream);

/* ---- cost-table profiling (outside the per-step path) -------------------- */
/* DSpark-in-SGLang page, section A2 "cost-table profiling and modelling"
 * (with the additive model of section 速读): the step time
 * T(bs, K) = bias + alpha(bs) + theta(M), M = bs + K, is profiled and the
 * scheduler reads the resulting table.  The pages give neither the form of
 * alpha and theta nor the fitting method; here both are linear and fitted by
 * ordinary least squares: t ~ bias + a*bs + th*M over n recorded samples,
 * solved by modified Gram-Schmidt QR (with one reorthogonalisation) in fp64.
 *
 * Host only, pure; every pointer is host memory.  In: bs[n], M[n], t[n].
 * Out: coef[3] = {bias, a, th}; when alpha (theta) is not NULL,
 * alpha[b] = a*b for b < alpha_len (theta[m] = th*m for m < theta_len): the
 * tables rv_schedule_args takes, with bias as cost_bias.
 * Errors (nothing is written): NULL bs/M/t/coef, n < 3, a negative table
 * length, a non-finite sample, or samples that do not determine the three
 * coefficients (a column within 1e-12 of the span of the previous ones):
 * INVALID_ARG. */
rv_status rv_fit_cost_model(const double* bs, const double* M, const double* t, int32_t n, double* coef,
                            double* alpha, int32_t alpha_len, double* theta, int32_t theta_len);

/* ---- stage 5: compact scatter ------------------------------------------- */
/* DSpark-in-SGLang page, section A2 "performance and zero-overhead
 * scheduling": a fused compact-scatter kernel writes the accepted results
 * back; the page table stays on the device.
 *
 * commit_cu = exclusive scan of accept+1.  Request i commits tokens
 * d_1..d_a, bonus at commit_tok[commit_cu[i]..] and the KV slots of rows
 * 0..a at commit_slot[...]; req_to_token[i][ctx[i]+k] = slot of row k
 * (k <= a); hist[i][hist_len[i]+k] = committed token k and hist_len += a+1
 * (when hist != NULL); ctx[i] += a+1; anchor[i] = bonus.  Slots of rows
 * a+1..w_verify-1 are listed in free_slots (in request order), their count in
 * *free_count. */
typedef struct {
  const int32_t* cu;         /* [B+1] */
  const int32_t* w_verify;   /* [B] */
  const int32_t* accept;     /* [B] */
  const int32_t* bonus;      /* [B] */
  const int32_t* drafts;     /* [B][gamma-1] */
  const int32_t* slot;       /* [rows_cap] from rv_pack */
  int32_t B, gamma;
  int32_t r2t_stride;        /* row length of req_to_token */
  int32_t hist_stride;       /* row length of hist (ignored if hist NULL) */
  int32_t* ctx;              /* in/out [B] */
  int32_t* anchor;           /* in/out [B] */
  int32_t* req_to_token;     /* in/out [B][r2t_stride] */
  int32_t* hist;             /* in/out [B][hist_stride] or NULL */
  int32_t* hist_len;         /* in/out [B] or NULL */
  int32_t* commit_cu;        /* out [B+1] */
  int32_t* commit_tok;       /* out [B*gamma] */
  int32_t* commit_slot;      /* out [B*gamma] */
  int32_t* free_slots;       /* out [B*gamma] */
  int32_t* free_count;       /* out [1] */
  void* workspace;
  size_t workspace_bytes;
} rv_scatter_args;
/* Device errors: HIST_OVERFLOW (the request's req_to_token / hist writes are
 * skipped; counters still advance), BAD_WINDOW (accept clamped). */
rv_status rv_compact_scatter(const rv_scatter_args* a, void* stream);

/* ---- ABI self-description ----------------------------------------------- */
/* Fills out[0] = sizeof(struct), out[1..] = offsetof of each field in
 * declaration order, for struct `which` (0 schedule, 1 pack, 2 attn, 3 lm,
 * 4 scatter, 5 dims, 6 calibration, 7 estimate).  Returns the number of values written, or -1 if `cap`
 * is too small or `which` unknown.  Host-only; lets a binding verify its
 * struct mirror. */
int32_t rv_abi_layout(int32_t which, int64_t* out, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* RV_H_ */
