// Stage 3: varlen causal verify attention over a paged KV cache.
//
// DSpark-in-SGLang page, section A2 "ragged verify over a full CUDA graph":
// the packed buffer is a cu_seqlens-style variable-length batch, so verify
// reuses ordinary varlen causal attention (native sparse-MLA on DeepSeek-V4);
// each backend rebuilds its varlen metadata from the packed layout.
//
// Design (gfx950).  Every kernel reads keys through the page table and
// moves them into LDS by direct global->LDS DMA (global_load_lds, 16 bytes
// per lane) into a ring of stages; scores and outputs use bf16 MFMAs with
// fp32 accumulation.
//  * Plans (one workgroup each, launched alone or appended to the pack
//    launch: k_pack_plan) rebuild the varlen metadata on the device from
//    cu[] and ctx[].  k_attn_plan cuts every request into tiles of query
//    vectors that share one KV head and, when the batch alone cannot fill the
//    chip, splits the key range into chunks (split-KV), ordered request-major
//    and per XCD so that the tiles reading one KV chunk share it through L2.
//    k_attn_plan_bal (GQA) lays every tile's 64-key super-tiles out as one
//    cost sequence and gives each persistent workgroup an equal contiguous
//    range of it.
//  * GQA (k_attn_gqa_bal, persistent): four waves, two query-vector groups x
//    two key groups, each super-tile's two 32-key halves in a four-stage
//    ring; S^T = K Q^T and O^T += V^T P^T on 16x16x32 MFMAs with an online
//    base-2 softmax (each lane owns one query vector; P^T feeds the PV MFMA
//    from registers; V^T comes from the row-major value rows through
//    gfx950's transposing LDS reads).  The two key groups merge through LDS
//    at the end of a range; a range that covers part of a tile writes fp32
//    partials to its slot.  k_attn_gqa is the same range code over the
//    chunked plan's work list.
//  * Latent (MLA-style) layout: one 576-wide row per key, its first 512
//    entries the value.  k_attn_mla_row takes one packed row with all 128
//    heads per workgroup (each 32-key tile DMA'd once per row): QK on
//    32x32x16 MFMAs with the queries' 512 value dims in registers and the 64
//    rope dims in LDS, probabilities exchanged between the four waves through
//    LDS, each wave accumulating 128 output columns of all 128 heads; a fixed
//    softmax reference from the first tile, with one rerun when a later score
//    leaves its range.  With per-row key lists (sparse) the same kernel runs
//    over each item's visible list entries, compacted in list order, each
//    DMA lane reading its slot's row.  k_attn_mla (64 heads per workgroup)
//    serves other head counts and page sizes.
//  * k_attn_combine merges split partials (O, max, normaliser) and writes
//    the rows between the packed count and the tier (k_attn_pad does that
//    for the fp32 kernel).
//  * fp32 inputs take a plain vector kernel (k_attn_f32).

#include <float.h>

#include <algorithm>
#include <mutex>

#include "pack_body.h"
#include "rv_common.h"

namespace rv {
namespace {

constexpr int kNK = 32;            // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnShape {
  int Hq, Hkv, G;        // G = Hq / Hkv
  int QT;                // query vectors per tile (16 per wave)
  int NH;                // heads per tile
  int RT;                // rows per tile
  int n_hb;              // head blocks per KV head = G / NH
  int tpr_max;           // tiles per request at most
  int target;            // work items the plan aims for
};

// Work header written by the plan: [0] items, [1] chunk, [2] partial slots
// used, [8 + x] / [16 + x] start and length of XCD x's item list, [24 + x]
// that list's take counter (zeroed by the plan, advanced by the workers);
// the shared tail list: start [40], length [41], take counter [24 + 8].
constexpr int kHdrXOff = 8, kHdrXLen = 16, kHdrCtr = 24, kHdrTOff = 40, kHdrTLen = 41;
// share of the work (by rank, the shortest chunks) that goes to the tail list
constexpr int kTailPct = 35;
// Header of the balanced GQA plan: total super-tiles, super-tiles per
// virtual worker, virtual workers, tiles, partial slots used.
constexpr int kBalS = 0, kBalQ = 1, kBalVw = 2, kBalTiles = 3, kBalParts = 4;
// Both plans: the number of tiles with split partials (listed in split[]).
constexpr int kHdrSplit = 6;
constexpr int kBalSuper = 64;   // keys per super-tile of the GQA kernel (two 32-key sub-tiles)
// A range's prologue (page window, queries, first DMA) costs about 2.4
// super-tiles of streaming (3.4-3.6 us against 1.44 us per super-tile,
// measured), so the balanced plan charges each tile three on top of its
// super-tiles (two and four measured slower on both GQA batches).
constexpr int kBalPro = 3;

struct PlanParams {
  const int32_t* cu;
  const int32_t* ctx;
  const int32_t* mm;
  int4* req_info;        // per request: {n_splits, chunk (keys), part_off, tiles}
  int4* items;           // {request, tile, split, 0}, grouped by XCD list
  int2* grp;             // scratch: {request, split} of each group by rank
  int2* split;           // {request, tile} of every tile with split partials
  int32_t* hdr;
  int B, gamma, item_cap, part_cap, target;
  int n_workers;         // persistent workgroups of the main kernel
  int window;            // sliding window (keys), 0 = full causal
  int topk;              // sparse latent attention: index entries per row (0: dense)
  AttnShape sh;
};

__device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Sliding window of W keys (W > 0): the row at position p sees keys
// [p - W + 1, p].  A request's key range then starts at its first row's
// bound, aligned down to 64 keys so that tiles and super-tiles stay aligned
// (page-uniform DMA); keys below a row's bound are masked.  W = 0: full causal.
__device__ inline int win_origin(int ctx, int W) { return W > 0 ? (max(0, ctx - W + 1) & ~63) : 0; }
// lowest visible key of the row at position pos (INT_MIN without a window)
__device__ inline int win_low(int pos, int W) { return W > 0 ? pos - W + 1 : INT32_MIN; }

// ---- plan: device-side varlen metadata -------------------------------------
//
// One workgroup of 1024 threads; thread t owns requests [t*seg, t*seg+seg)
// (seg = ceil(B/1024)), whose (window, keys) pairs it caches in LDS.  Every
// block-wide reduction and scan is a wave-level shuffle scan plus one pass
// over the 16 wave totals (block_excl_scan), so each costs two barriers.
constexpr int kPlanThreads = kScanThreads;
constexpr int kPlanWaves = kScanWaves;
constexpr int kPlanMaxB = RV_MAX_ROWS / 2;   // gamma >= 2

__device__ __forceinline__ void plan_chunked_body(const PlanParams& p) {
  __shared__ int2 s_wl[kPlanMaxB];            // per request: window, keys (ctx + window)
  __shared__ int s_ci[kPlanMaxB];             // per request: its chunk
  __shared__ int s_buf[kPlanWaves * 8];
  __shared__ long long s_red[kPlanWaves];
  __shared__ int hist[64];
  __shared__ int hwork[64];
  __shared__ int s_rs;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int B = p.B;
  const AttnShape& sh = p.sh;
  const int seg = ceil_div(B, kPlanThreads);
  const int i0 = t * seg;
  const int i1 = min(i0 + seg, B);
  auto tiles_of_w = [&](int w) { return ceil_div(w, sh.RT) * sh.Hkv * sh.n_hb; };

  // total work: sum over tiles of keys visible to the tile's last row
  long long work = 0;
  for (int i = i0; i < i1; ++i) {
    const int w = p.cu[i + 1] - p.cu[i];
    // keys from the origin; sparse: each row's tile walks its topk index slots
    const int L = p.topk > 0 ? p.topk : p.ctx[i] + w - win_origin(p.ctx[i], p.window);
    s_wl[i] = make_int2(w, L);
    work += (long long)tiles_of_w(w) * L;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) work += __shfl_xor(work, off);
  if (lane == 0) s_red[t >> 6] = work;
  if (t < 64) hist[t] = 0;
  __syncthreads();
  long long all_work = 0;
  for (int u = 0; u < kPlanWaves; ++u) all_work += s_red[u];
  long long c0 = (all_work + p.target - 1) / p.target;
  c0 = (c0 + kNK - 1) / kNK * kNK;
  if (c0 < kMinChunk) c0 = kMinChunk;
  if (c0 > (1 << 30)) c0 = 1 << 30;
  int C = (int)c0;

  // grow the chunk until items and partial slots fit their buffers (both
  // counts fall as the chunk grows)
  for (int iter = 0; iter < 32; ++iter) {
    int cnt[2] = {0, 0}, ex[2], tot[2];
    for (int i = i0; i < i1; ++i) {
      const int2 wl = s_wl[i];
      const int tiles = tiles_of_w(wl.x);
      const int ns = wl.y > 0 ? ceil_div(wl.y, C) : 1;
      cnt[0] += ns * tiles;
      cnt[1] += ns > 1 ? ns * tiles : 0;
    }
    block_excl_scan<2>(cnt, ex, tot, s_buf);
    if ((tot[0] <= p.item_cap && tot[1] <= p.part_cap) || C >= (1 << 29)) break;
    C *= 2;
  }

  // Per-request chunks (req_info.y).  When the work ends on items that are
  // long next to a worker's share (equal-length requests, e.g. under a
  // sliding window or with key lists: 815 equal items on 256 workers run 3.2
  // rounds and most workers idle through the fourth), the requests with the
  // shortest key ranges get a chunk m times finer, enough of them that about
  // one finer piece per worker ends the longest-first schedule.  "Long" is
  // judged at the request that completes the shortest n_workers tiles.
  for (int i = i0; i < i1; ++i) s_ci[i] = C;
  {
    __shared__ int s_cut[3];
    int lmin = INT32_MAX, lmax = 0;
    for (int i = i0; i < i1; ++i) {
      lmin = min(lmin, s_wl[i].y);
      lmax = max(lmax, s_wl[i].y);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lmin = min(lmin, __shfl_xor(lmin, off));
      lmax = max(lmax, __shfl_xor(lmax, off));
    }
    __syncthreads();   // s_buf is free
    if (lane == 0) {
      s_buf[(t >> 6) * 2] = lmin;
      s_buf[(t >> 6) * 2 + 1] = lmax;
    }
    if (t < 64) hist[t] = 0;
    __syncthreads();
    for (int u = 0; u < kPlanWaves; ++u) {
      lmin = min(lmin, s_buf[u * 2]);
      lmax = max(lmax, s_buf[u * 2 + 1]);
    }
    // tiles by key-range length: 64 buckets over [lmin, lmax]
    const long long span = (long long)lmax - lmin + 1;
    auto lb = [&](int L) { return (int)(((long long)(L - lmin) * 64) / span); };
    for (int i = i0; i < i1; ++i) atomicAdd(&hist[lb(s_wl[i].y)], tiles_of_w(s_wl[i].x));
    __syncthreads();
    if (t < 64) {   // wave 0: cumulative tiles over the buckets
      int h[1] = {hist[t]};
      wave_incl_scan<1>(h);
      // first bucket whose cumulative count reaches x (63 if none), and the
      // count before it
      auto first_reach = [&](int x, int& before) {
        const unsigned long long hit = __ballot(h[0] >= x);
        const int b = hit ? __ffsll((long long)hit) - 1 : 63;
        before = __shfl(h[0], b > 0 ? b - 1 : 0);
        if (b == 0) before = 0;
        return b;
      };
      const long long share = p.n_workers > 0 ? all_work / p.n_workers : 0;   // tile-keys per worker
      int m = 1, bc = 0, before = 0;
      if (share > 0) {
        const int b = first_reach(p.n_workers, before);
        const long long lk = min((long long)C, lmin + ((long long)(b + 1) * span + 63) / 64);   // that request's item length, at most
        if (lk * 8 > share) m = (int)min(8LL, (lk * 8 + share - 1) / share);
      }
      const int need = ceil_div(max(p.n_workers, 1), m);
      if (m >= 2) bc = first_reach(need, before);
      if (t == 0) {
        s_cut[0] = m;
        s_cut[1] = bc;              // buckets below bc: all chosen
        s_cut[2] = need - before;   // tiles still wanted from bucket bc, in request order
      }
    }
    __syncthreads();
    const int m = s_cut[0], bcut = s_cut[1], rem = s_cut[2];
    if (m >= 2) {
      int in_b[1] = {0}, ex_b[1], tot_b[1];
      for (int i = i0; i < i1; ++i)
        if (lb(s_wl[i].y) == bcut) in_b[0] += tiles_of_w(s_wl[i].x);
      block_excl_scan<1>(in_b, ex_b, tot_b, s_buf);
      int before = ex_b[0];
      for (int i = i0; i < i1; ++i) {
        const int2 wl = s_wl[i];
        const int b = lb(wl.y);
        bool pick = b < bcut;
        if (b == bcut) {
          pick = before < rem;
          before += tiles_of_w(wl.x);
        }
        if (pick && wl.y > 0) s_ci[i] = max(ceil_div(ceil_div(min(C, wl.y), m), kNK) * kNK, kNK);
      }
      // keep the finer chunks only if items and partial slots still fit
      int cnt[2] = {0, 0}, ex[2], tot[2];
      for (int i = i0; i < i1; ++i) {
        const int2 wl = s_wl[i];
        const int tiles = tiles_of_w(wl.x);
        const int ns = wl.y > 0 ? ceil_div(wl.y, s_ci[i]) : 1;
        cnt[0] += ns * tiles;
        cnt[1] += ns > 1 ? ns * tiles : 0;
      }
      block_excl_scan<2>(cnt, ex, tot, s_buf);
      if (tot[0] > p.item_cap || tot[1] > p.part_cap)
        for (int i = i0; i < i1; ++i) s_ci[i] = C;
    }
    __syncthreads();
    if (t < 64) hist[t] = 0;
    __syncthreads();
  }

  // A group is the set of tiles of one request that read one key chunk; its
  // tiles run on one XCD, one after another in that XCD's list, so the chunk
  // is fetched into that XCD's L2 once.  Groups are ranked longest chunk
  // first (counting sort over 64 length buckets) and dealt to the 8 lists in
  // snake order (ranks 8c..8c+7 go to XCDs 0..7 for even c, 7..0 for odd c),
  // which balances the lists and starts the longest items first.
  int mine[3] = {0, 0, 0}, off2[3], tot2[3];
  for (int i = i0; i < i1; ++i) {
    const int2 wl = s_wl[i];
    const int ns = wl.y > 0 ? ceil_div(wl.y, s_ci[i]) : 1;
    mine[0] += ns;
    mine[1] += ns > 1 ? ns * tiles_of_w(wl.x) : 0;
    mine[2] += ns > 1 ? tiles_of_w(wl.x) : 0;
  }
  block_excl_scan<3>(mine, off2, tot2, s_buf);
  const int n_groups = tot2[0];
  const int n_parts = tot2[1];
  int part_off = off2[1], split_off = off2[2];
  // bucket of a chunk of `len` keys: 0 for a full chunk, up to 63 for the shortest
  auto bucket = [&](int len) { return (int)(((long long)(C - len) * 64) / C); };
  if (t < 64) hwork[t] = 0;
  __syncthreads();
  for (int i = i0; i < i1; ++i) {
    const int L = s_wl[i].y, ci = s_ci[i];
    const int ns = L > 0 ? ceil_div(L, ci) : 1;
    const int tiles = tiles_of_w(s_wl[i].x);
    for (int sp = 0; sp < ns; ++sp) {
      const int len = max(min(ci, L - sp * ci), 1);
      atomicAdd(&hist[bucket(len)], 1);
      atomicAdd(&hwork[bucket(len)], tiles * ceil_div(len, kNK));   // work in 32-key tiles
    }
  }
  __syncthreads();
  // The ranks from rs on (the shortest chunks, from the first bucket at
  // which about 100 - kTailPct percent of the work, counted in 32-key tiles,
  // lies before it) form a shared tail list, which every worker takes from
  // once its own XCD's list is empty.  The XCD lists are dealt by group
  // count and a group is one to eight rows, so their work differs; without
  // a shared tail the last items taken are wherever the fullest list had got
  // to (on the latent batch workers then ended up to 0.3 ms apart; a fifth
  // of the work in the tail was not enough, 35% to 70% measured alike).
  if (t < 64) {   // wave 0: exclusive scans of the bucket counts and works
    int h[2] = {hist[t], hwork[t]};
    const int own_c = h[0], own_w = h[1];
    wave_incl_scan<2>(h);
    hist[t] = h[0] - own_c;
    const int wall = __shfl(h[1], 63);
    const int thresh = wall - (int)((long long)wall * kTailPct / 100);
    // the bucket in which the threshold falls; within it, the groups (of
    // about equal chunk length) are cut by count in proportion
    const unsigned long long hit = __ballot(h[1] >= thresh && own_c > 0);
    const int bt = hit ? __ffsll((long long)hit) - 1 : 63;
    const int src = bt;
    const int start_bt = __shfl(h[0] - own_c, src);   // first rank of bucket bt
    const int cnt_bt = __shfl(own_c, src);
    const int wex_bt = __shfl(h[1] - own_w, src);
    const int w_bt = __shfl(own_w, src);
    if (t == 0) {
      int r = n_groups;
      if (hit && w_bt > 0)
        r = start_bt + (int)min((long long)cnt_bt,
                                ((long long)(thresh - wex_bt) * cnt_bt + w_bt - 1) / w_bt);
      s_rs = r;
    }
  }
  __syncthreads();
  for (int i = i0; i < i1; ++i) {
    const int2 wl = s_wl[i];
    const int tiles = tiles_of_w(wl.x);
    const int L = wl.y, ci = s_ci[i];
    const int ns = L > 0 ? ceil_div(L, ci) : 1;
    p.req_info[i] = make_int4(ns, ci, ns > 1 ? part_off : -1, tiles);
    if (ns > 1)
      for (int tl = 0; tl < tiles; ++tl) p.split[split_off++] = make_int2(i, tl);
    for (int sp = 0; sp < ns; ++sp) {
      const int rank = atomicAdd(&hist[bucket(max(min(ci, L - sp * ci), 1))], 1);
      p.grp[rank] = make_int2(i, sp);
    }
    part_off += ns > 1 ? ns * tiles : 0;
  }
  __syncthreads();   // the ranked groups are visible to the whole workgroup
  const int rs = s_rs;
  const int segr = ceil_div(n_groups, kPlanThreads);
  const int r0 = min(t * segr, n_groups), r1 = min(r0 + segr, n_groups);

  // items per (cycle, XCD) slot, scanned along the cycles of each XCD
  const int nc = ceil_div(rs, 8);
  const int segc = ceil_div(nc, kPlanThreads);
  auto rank_of = [](int c, int x) { return 8 * c + ((c & 1) ? 7 - x : x); };
  int cnt[8], pos[8], xlen[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) cnt[x] = 0;
  for (int cc = 0; cc < segc; ++cc) {
    const int c = t * segc + cc;
    if (c >= nc) break;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int r = rank_of(c, x);
      if (r < rs) cnt[x] += tiles_of_w(s_wl[p.grp[r].x].x);
    }
  }
  block_excl_scan<8>(cnt, pos, xlen, s_buf);
  int xoff[8];
  int total = 0;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    xoff[x] = total;
    total += xlen[x];
    pos[x] += xoff[x];
  }
  for (int cc = 0; cc < segc; ++cc) {
    const int c = t * segc + cc;
    if (c >= nc) break;
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int r = rank_of(c, x);
      if (r >= rs) continue;
      const int2 g = p.grp[r];
      const int tiles = tiles_of_w(s_wl[g.x].x);
      for (int tl = 0; tl < tiles; ++tl) p.items[pos[x] + tl] = make_int4(g.x, tl, g.y, 0);
      pos[x] += tiles;
    }
  }
  // the tail list after the XCD lists, in rank order (longest first)
  int tv[1] = {0}, tex[1], ttot[1];
  for (int r = max(r0, rs); r < r1; ++r) tv[0] += tiles_of_w(s_wl[p.grp[r].x].x);
  block_excl_scan<1>(tv, tex, ttot, s_buf);
  {
    int q = total + tex[0];
    for (int r = max(r0, rs); r < r1; ++r) {
      const int2 g = p.grp[r];
      const int tiles = tiles_of_w(s_wl[g.x].x);
      for (int tl = 0; tl < tiles; ++tl) p.items[q + tl] = make_int4(g.x, tl, g.y, 0);
      q += tiles;
    }
  }
  if (t == 0) {
    p.hdr[0] = total + ttot[0];
    p.hdr[1] = C;
    p.hdr[2] = n_parts;
    p.hdr[kHdrSplit] = tot2[2];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      p.hdr[kHdrXOff + x] = xoff[x];
      p.hdr[kHdrXLen + x] = xlen[x];
      p.hdr[kHdrCtr + x] = 0;
    }
    p.hdr[kHdrTOff] = total;
    p.hdr[kHdrTLen] = ttot[0];
    p.hdr[kHdrCtr + 8] = 0;
  }
}

// ---- balanced plan (GQA) ----------------------------------------------------
//
// The tiles of all requests, request-major, each cut into 64-key super-tiles
// and charged kBalPro units of prologue before them, form one cost sequence
// of S units; virtual worker v takes [v*q, v*q+q) with q = ceil(S /
// workers), so the workers' loads differ by about one unit.  Outputs:
// req_info[i] = {tiles, first tile, 0, 0}; per tile T (in items[]) {cost
// position of its first super-tile, super-tiles, first partial slot or -1,
// request}; after the n_tiles entries of items[], the first tile of each
// virtual worker.  A tile whose super-tiles fall to k > 1 workers owns k
// consecutive partial slots, one per worker in order.
__device__ __forceinline__ void plan_bal_body(const PlanParams& p) {
  __shared__ int2 s_wc[kPlanMaxB];            // per request: window, context
  __shared__ int2 s_off[kPlanMaxB];           // per request: first tile, first cost unit
  __shared__ int s_buf[kPlanWaves * 8];
  const int t = threadIdx.x;
  const int B = p.B;
  const AttnShape& sh = p.sh;
  const int seg = ceil_div(B, kPlanThreads);
  const int i0 = t * seg;
  const int i1 = min(i0 + seg, B);
  const int per_rb = sh.Hkv * sh.n_hb;   // tiles per row block
  // super-tiles of one tile of row block rb
  auto nst = [&](int w, int c, int rb) {
    const int L_tile = c + min((rb + 1) * sh.RT, w);
    return ceil_div(L_tile - win_origin(c, p.window), kBalSuper);
  };

  // per request: tiles and cost units (super-tiles plus kBalPro per tile)
  int cnt[2] = {0, 0}, off[2], tot[2];
  for (int i = i0; i < i1; ++i) {
    const int w = p.cu[i + 1] - p.cu[i];
    const int c = p.ctx[i];
    s_wc[i] = make_int2(w, c);
    const int n_rb = ceil_div(w, sh.RT);
    cnt[0] += n_rb * per_rb;
    for (int rb = 0; rb < n_rb; ++rb) cnt[1] += per_rb * (nst(w, c, rb) + kBalPro);
  }
  block_excl_scan<2>(cnt, off, tot, s_buf);
  const int n_tiles = tot[0], S = tot[1];
  const int q = max(1, ceil_div(S, max(p.n_workers, 1)));
  const int n_vw = ceil_div(S, q);
  {
    int T = off[0], st = off[1];
    for (int i = i0; i < i1; ++i) {
      const int2 wc = s_wc[i];
      const int n_rb = ceil_div(wc.x, sh.RT);
      s_off[i] = make_int2(T, st);
      p.req_info[i] = make_int4(n_rb * per_rb, T, 0, 0);
      T += n_rb * per_rb;
      for (int rb = 0; rb < n_rb; ++rb) st += per_rb * (nst(wc.x, wc.y, rb) + kBalPro);
    }
  }
  __syncthreads();

  // per tile, in parallel (a contiguous run of tiles per thread): its
  // request (binary search over the requests' first tiles), row block and
  // cost position; a tile split over k > 1 workers takes k partial slots
  const int segT = ceil_div(n_tiles, kPlanThreads);
  const int T0 = min(t * segT, n_tiles), T1 = min(T0 + segT, n_tiles);
  struct TileAt { int i, n, st; };
  auto tile_at = [&](int T) {
    int lo = 0, hi = B - 1;   // last request whose first tile is at or before T
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid].x <= T) lo = mid; else hi = mid - 1;
    }
    const int2 wc = s_wc[lo];
    const int u = T - s_off[lo].x;
    const int rb = u / per_rb, k = u % per_rb;
    int st = s_off[lo].y;
    for (int r = 0; r < rb; ++r) st += per_rb * (nst(wc.x, wc.y, r) + kBalPro);
    const int n = nst(wc.x, wc.y, rb);
    st += k * (n + kBalPro);
    return TileAt{lo, n, st};
  };
  int parts[2] = {0, 0}, poff[2], ptot[2];
  for (int T = T0; T < T1; ++T) {
    const TileAt ta = tile_at(T);
    const int s0 = ta.st + kBalPro;   // cost position of the tile's first super-tile
    const int kseg = (s0 + ta.n - 1) / q - s0 / q + 1;
    parts[0] += kseg > 1 ? kseg : 0;
    parts[1] += kseg > 1 ? 1 : 0;
  }
  block_excl_scan<2>(parts, poff, ptot, s_buf);

  int* vw_first = reinterpret_cast<int*>(p.items + n_tiles);
  int slot = poff[0], split_at = poff[1];
  for (int T = T0; T < T1; ++T) {
    const TileAt ta = tile_at(T);
    const int s0 = ta.st + kBalPro;
    const int v_first = s0 / q, v_last = (s0 + ta.n - 1) / q;
    const int kseg = v_last - v_first + 1;
    p.items[T] = make_int4(s0, ta.n, kseg > 1 ? slot : -1, ta.i);
    slot += kseg > 1 ? kseg : 0;
    if (kseg > 1) p.split[split_at++] = make_int2(ta.i, T - s_off[ta.i].x);
    // workers whose range starts inside this tile
    for (int v = ceil_div(ta.st, q); v <= v_last; ++v) vw_first[v] = T;
  }
  if (t == 0) {
    p.hdr[kBalS] = S;
    p.hdr[kBalQ] = q;
    p.hdr[kBalVw] = n_vw;
    p.hdr[kBalTiles] = n_tiles;
    p.hdr[kBalParts] = ptot[0];
    p.hdr[kHdrSplit] = ptot[1];
  }
}

__global__ __launch_bounds__(kPlanThreads) void k_attn_plan(PlanParams p) { plan_chunked_body(p); }
__global__ __launch_bounds__(kPlanThreads) void k_attn_plan_bal(PlanParams p) { plan_bal_body(p); }

// Stage 2 and stage 3's plan in one launch (one workgroup): the plan reads
// the cu[] this workgroup has just written.
template <bool BAL>
__global__ __launch_bounds__(kPlanThreads) void k_pack_plan(PackParams pk, PlanParams pp) {
  static_assert(kPlanThreads == kScanThreads, "the pack body's workgroup");
  pack_body(pk);
  __syncthreads();   // cu[] and mm[] written by this workgroup are visible to all of it
  if constexpr (BAL) plan_bal_body(pp);
  else plan_chunked_body(pp);
}

// ---- bf16 attention kernels: shared parameters ---------------------------------
struct MainParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;        // nullptr for the latent layout
  const int32_t* page_table;
  const int32_t* ctx;
  const int32_t* cu;
  const int4* req_info;
  const int4* items;
  const int32_t* hdr;
  int32_t* ctr;           // hdr + kHdrCtr: per-XCD take counters
  bf16_t* o;
  float* lse;
  float* part_o;          // [part_cap][QT][DV]
  float* part_ml;         // [part_cap][QT][2]
  int32_t* status;
  int max_pages, page_size, num_pages, Hq, Hkv, G, NH, RT, n_hb, part_cap;
  int log2P;              // log2(page_size) when it is a power of two, else -1
  int window;             // sliding window (keys), 0 = full causal
  const int32_t* topk_idx;  // sparse latent attention: [rows][topk] key positions, or nullptr
  int topk;
  float scale_log2;       // sm_scale * log2(e)
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// gfx950 transposing LDS read at a raw 32-bit LDS byte address: within each
// 16-lane group, lane 4s+e receives element e of the 4-element blocks
// addressed by lanes s, 4+s, 8+s, 12+s.  With lane r of the group addressing
// row (key0 + r/4), columns c0 + 4*(r%4) of a row-major tile, lane m receives
// column c0 + m of rows key0..key0+3: the k-contiguous MFMA operand fragment
// of a [keys x dims] tile.
__device__ inline uint2 lds_tr16(uint32_t addr) {
  s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(size_t)addr);
  return __builtin_bit_cast(uint2, v);
}

// Persistent workers: the hardware places workgroup b on XCD b % 8.  A
// workgroup takes the next item of its XCD's list (longest first) and, once
// that list is empty, of the other lists; it returns -1 when all are empty,
// so every workgroup ends after at most one failed take per list.  (Taking
// the following item one item ahead, to hide the atomic's round trip, was
// measured slower: it commits items early and unbalances the tail.)
__device__ inline int next_item(const MainParams& p, int* s_item, unsigned& done) {
  __syncthreads();   // every thread has read the previous item
  if (threadIdx.x == 0) {
    // this XCD's list, then the shared tail list (8), then the other XCDs'
    const int x = blockIdx.x & 7;
    int it = -1;
    for (int probe = 0; probe < 9 && it < 0; ++probe) {
      const int y = probe == 0 ? x : probe == 1 ? 8 : (x + probe - 1) & 7;
      if (done & (1u << y)) continue;
      const int k = atomicAdd(p.ctr + y, 1);
      const int len = y == 8 ? p.hdr[kHdrTLen] : p.hdr[kHdrXLen + y];
      if (k < len) it = (y == 8 ? p.hdr[kHdrTOff] : p.hdr[kHdrXOff + y]) + k;
      else done |= 1u << y;
    }
    *s_item = it;
  }
  __syncthreads();
  // every lane read the same value: tell the compiler, so that the item's
  // metadata loads and the arithmetic on them stay scalar
  return __builtin_amdgcn_readfirstlane(*s_item);
}

// ---- latent (MLA-style) bf16 kernel: LDS DMA ring ---------------------------------
//
// One workgroup = four waves against one latent KV head and 64 query vectors
// (e.g. half of a 128-head row).  Keys arrive through direct global->LDS DMA
// (global_load_lds_dwordx4) into a ring of kMlaStages 32-key stages issued two
// tiles ahead, so no registers stage the data and the latency of the next
// tiles hides behind the MFMA work of the current one.  The DMA is issued from
// inline assembly because the compiler would otherwise wait for every
// outstanding DMA before each LDS read; the kernel tracks the vector-memory
// counter itself (loads complete in issue order).
//
// LDS layout of a stage: 32 rows of 1152 bytes (576 bf16, no padding) whose
// 16-byte chunks are XOR-swizzled within aligned groups of eight
// (physical = logical ^ ((row >> 1) & 7)) so that fragment reads of sixteen
// consecutive rows hit distinct banks.  The request's page-table entries for
// the item's key range sit in an LDS window.  The softmax reference of each
// query vector is fixed by the first tile; if the visible scores of the item
// end up far above (overflow risk) or far below (underflow risk) it, the item
// runs once more with the true maximum, so the O accumulators are never
// rescaled.

constexpr int kMlaD = 576, kMlaDv = 512;
constexpr int kMlaRowBytes = kMlaD * 2;                    // 1152
constexpr int kMlaStageBytes = kNK * kMlaRowBytes;         // 36864
constexpr int kMlaStages = 3;
constexpr int kPageWin = 2048;
constexpr int kMlaChunksPerRow = kMlaD / 8;                // 72
constexpr int kMlaDmaPerWave = kNK * kMlaChunksPerRow / 256;  // 9 per wave per tile
constexpr int kMlaQT = 64;                                 // query vectors per tile (2 wave pairs x 32)

__device__ inline int swz(int row) { return (row >> 1) & 7; }
// A per-lane value the compiler must treat as computed here: LDS addresses
// formed as opaque(base) + constant keep the constant in the instruction's
// offset field instead of re-adding a scalar base to a lane offset per read.
__device__ inline uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
// Swizzle of the latent kernels' 1152-byte key rows.  Rows alternate between
// the two halves of the 64 banks (1152 = 4.5 x 256 bytes), and the XOR with
// the bit-reversed pair index gives (a) 16 consecutive rows at one chunk:
// 16 distinct 16-byte bank slots (QK fragment reads), and (b) 4 consecutive
// rows at an aligned group of 4 chunks: rows r and r+2 in opposite halves of
// the 8 chunk slots (transposing V^T reads), which (row >> 1) & 7 maps to the
// same banks.
__device__ inline int lswz(int row) {
  const int x = (row >> 1) & 7;
  return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
}

__device__ inline uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};   // v_cvt_pk_bf16_f32 (RNE)
  return __builtin_bit_cast(uint32_t, v);
}

// FAST: page size is a power of two >= 32, so a 32-key tile lies in one page.
//
// Work split inside a workgroup (4 waves, 64 query vectors in four 16-wide
// blocks): waves 2p and 2p+1 form pair p, which owns blocks 2p and 2p+1.
// Wave h of the pair scores keys [16h, 16h+16) of every 32-key tile for its
// pair's 32 vectors over all 576 head dims and turns them into bf16
// probabilities, which every wave then reads from LDS.  Wave w accumulates
// all 32 keys for all 64 vectors into its quarter of the output columns,
// [128w, 128w+128).  Every K fragment read from LDS feeds two MFMAs and every
// transposed V fragment four; no partial scores cross waves and no wave
// repeats another's softmax.
//
// Software pipeline, one barrier per 32-key tile: iteration t scores tile t+1
// (QK), then accumulates tile t (PV) while the new scores become
// probabilities, and publishes them; the barrier of iteration t+1 makes them
// visible to the partner.  The DMA of tile t+2 is issued right after the
// barrier into the stage that tile t-1 used.
constexpr int kMlaXBytes = 2 * 4 * 64 * 16;       // probabilities [buffer][block][lane], 16 B each
constexpr int kMlaRedBytes = 2 * 4 * 2 * 16 * 4;   // column max and sum [wave][block][16]
constexpr int kMaxTopk = RV_MAX_TOPK;   // sparse latent attention: index entries per row at most
constexpr int kMlaLdsBytes = kMlaStages * kMlaStageBytes + kMlaXBytes + kMlaRedBytes + kPageWin * 4 + kMaxTopk * 4;
static_assert(kMlaLdsBytes <= 160 * 1024, "latent kernel LDS");

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) f32x4_t lds_f32x4_t;
__device__ inline uint2 lds_b64(uint32_t addr) {
  return __builtin_bit_cast(uint2, *(const lds_u32x2_t*)(size_t)addr);
}
__device__ inline void lds_st_b64(uint32_t addr, uint32_t lo, uint32_t hi) {
  *(lds_u32x2_t*)(size_t)addr = u32x2_t{lo, hi};
}

template <bool FAST, bool SPARSE>
__device__ __forceinline__ void attn_mla_item(const MainParams& p, int item, unsigned char* smem);

// SPARSE: each row attends to the key positions its index list names (the
// rows of a latent tile are one row: 64 heads), walked in list order.
template <bool FAST, bool SPARSE>
__global__ __launch_bounds__(256) void k_attn_mla(MainParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_item;
  unsigned done = 0;
  for (;;) {
    const int item = next_item(p, &s_item, done);
    if (item < 0) break;
    attn_mla_item<FAST, SPARSE>(p, item, smem);
  }
}

template <bool FAST, bool SPARSE>
__device__ __forceinline__ void attn_mla_item(const MainParams& p, int item, unsigned char* smem) {
  static_assert(!(FAST && SPARSE), "sparse keys do not lie in one page per tile");
  constexpr int kRing = kMlaStages * kMlaStageBytes;
  float* red_m = reinterpret_cast<float*>(smem + kRing + kMlaXBytes);
  float* red_l = red_m + 4 * 2 * 16;
  int* pwin = reinterpret_cast<int*>(smem + kRing + kMlaXBytes + kMlaRedBytes);
  int* sidx = pwin + kPageWin;   // SPARSE: the item's index slots as cache rows, -1 where masked

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wid >> 1;
  const int half = wid & 1;
  const int n16 = lane & 15;
  const int grp = lane >> 4;

  const int4 rec = p.items[item];
  const int i = rec.x, tile = rec.y, sp = rec.z;
  const int4 info = p.req_info[i];
  const int ns = info.x;
  const int row_start = p.cu[i];
  const int w = p.cu[i + 1] - row_start;
  const int c = p.ctx[i];
  const int rb = tile / p.n_hb;          // one KV head
  const int hb = tile % p.n_hb;
  const int row0 = rb * p.RT;
  const int rows_here = min(p.RT, w - row0);
  // SPARSE: keys [kv_begin, kv_end) are index slots of the tile's one row,
  // whose positions lie in 0 .. c + row0
  const int L_tile = SPARSE ? p.topk : c + row0 + rows_here;
  const int chunk = info.y;   // this request's chunk
  const int kv_begin = (SPARSE ? 0 : win_origin(c, p.window)) + sp * chunk;
  const int kv_end = min(kv_begin + chunk, L_tile);
  const int P = p.page_size;

  // page-table window for keys [kv_begin, kv_end) (SPARSE: every page up to
  // the row's position)
  const int pg0 = SPARSE ? 0 : kv_begin / P;
  int npg = SPARSE ? 0 : (kv_end > kv_begin ? (kv_end - 1) / P - pg0 + 1 : 0);
  if (npg > kPageWin) {                 // context longer than the page table allows
    if (tid == 0) set_status(p.status, RV_DEV_BAD_PAGE);
    npg = kPageWin;
  }
  const int* pt_row = p.page_table + (size_t)i * p.max_pages;
  for (int x = tid; x < npg; x += 256) {
    int pg = (pg0 + x < p.max_pages) ? pt_row[pg0 + x] : -1;
    if (pg < 0 || pg >= p.num_pages) { set_status(p.status, RV_DEV_BAD_PAGE); pg = 0; }
    pwin[x] = pg;
  }
  if constexpr (SPARSE) {
    // the row's index slots of this item as cache rows (page table read
    // directly); positions outside 0 .. its own position (and -1 entries)
    // are -1, masked
    const int32_t* src = p.topk_idx + (size_t)(row_start + row0) * p.topk;
    for (int x = tid; x < kv_end - kv_begin; x += 256) {
      const int j = src[kv_begin + x];
      int r = -1;
      if (j >= 0 && j <= c + row0) {
        int pg = (j / P < p.max_pages) ? pt_row[j / P] : -1;
        if (pg < 0 || pg >= p.num_pages) { set_status(p.status, RV_DEV_BAD_PAGE); pg = 0; }
        r = pg * P + j % P;
      }
      sidx[x] = r;
    }
  }

  // query fragments: both 16-vector blocks of the pair, all 576 dims
  int q_row[2], head[2], lim[2], low[2];
  bool q_valid[2];
  u32x4_t qf[2][18];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qv = pair * 32 + qb * 16 + n16;
    const int rl = qv / p.NH;
    head[qb] = hb * p.NH + (qv % p.NH);
    q_valid[qb] = rl < rows_here;
    q_row[qb] = row_start + row0 + (q_valid[qb] ? rl : 0);
    lim[qb] = SPARSE ? kv_end - 1 : min(c + row0 + rl, kv_end - 1);   // last key (slot) it may see here
    low[qb] = SPARSE ? INT32_MIN : win_low(c + row0 + rl, p.window);  // first key it may see
    const bf16_t* qsrc = p.q + ((size_t)q_row[qb] * p.Hq + head[qb]) * kMlaD + grp * 8;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qf[qb][ks] = *reinterpret_cast<const u32x4_t*>(qsrc + ks * 32);
  }
  // tiles ending at or before this key need no mask for any valid vector;
  // with a window, neither do tiles starting at or after every row's bound
  const int full_lim = min(c + row0, kv_end - 1);
  const int low_max = win_low(c + row0 + rows_here - 1, p.window);
  auto is_full = [&](int t0) { return !SPARSE && t0 + kNK - 1 <= full_lim && t0 >= low_max; };
  wait_vm<0>();
  __syncthreads();   // page window visible

  const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + kNK - 1) / kNK : 0;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const uint32_t xbase = smem_lds + kRing;
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(smem_lds + wid * kMlaDmaPerWave * 1024);

  // DMA chunks: wave wid issues chunks (wid*9 + e)*64 + lane of a tile; chunk
  // c lands at row c/72, physical position c%72 and holds logical chunk
  // (c%72) ^ lswz(row)
  const int cbase = wid * kMlaDmaPerWave * 64 + lane;
  const int last = kv_end - 1;   // keys past the end read this valid row (masked later)

  // FAST: this lane's source byte offsets relative to a tile's first row.  A
  // tile lies in one page, so a DMA is a uniform base plus these offsets;
  // rows past the item's last key are clamped to that key's final 16 bytes
  // (finite data; those keys are masked).
  uint32_t dma_off[kMlaDmaPerWave];
#pragma unroll
  for (int e = 0; e < kMlaDmaPerWave; ++e) {
    const int cidx = cbase + e * 64;
    const int row = cidx / kMlaChunksPerRow;
    dma_off[e] = (uint32_t)(row * kMlaRowBytes + ((cidx - row * kMlaChunksPerRow) ^ lswz(row)) * 16);
  }
  struct DmaTile {
    const void* base;   // the tile's first row
    uint32_t lim;       // largest source offset (last valid row's final chunk)
    uint32_t lds0;      // this wave's destination in the stage
  };
  auto dma_tile = [&](int t, int st, int pg) {
    const int t0 = kv_begin + t * kNK;
    DmaTile d;
    d.base = uniform_ptr(reinterpret_cast<const unsigned char*>(p.k) +
                         ((size_t)pg * P + (t0 & (P - 1))) * kMlaRowBytes);
    d.lim = (uint32_t)(min(last - t0, kNK - 1) * kMlaRowBytes + kMlaRowBytes - 16);
    d.lds0 = wave_lds + st * kMlaStageBytes;
    return d;
  };
  auto dma_one = [&](const DmaTile& d, int e) { dma16_s(min(dma_off[e], d.lim), d.base, d.lds0 + e * 1024); };
  // FAST: window index of tile t's page
  auto page_at = [&](int t) { return pwin[((kv_begin + t * kNK) >> p.log2P) - pg0]; };

  auto issue = [&](int t, int st) {
    const int t0 = kv_begin + t * kNK;
    const uint32_t lds0 = wave_lds + st * kMlaStageBytes;
    if constexpr (FAST) {
      const DmaTile d = dma_tile(t, st, __builtin_amdgcn_readfirstlane(page_at(t)));
#pragma unroll
      for (int e = 0; e < kMlaDmaPerWave; ++e) dma_one(d, e);
    } else {
      // every source row first (the LDS reads overlap), then the DMAs: the
      // asm statements order memory, so reads between them would serialise
      int krow[kMlaDmaPerWave];
#pragma unroll
      for (int e = 0; e < kMlaDmaPerWave; ++e) {
        const int row = (cbase + e * 64) / kMlaChunksPerRow;
        const int j = min(t0 + row, last);
        if constexpr (SPARSE) {
          krow[e] = max(sidx[j - kv_begin], 0);   // masked slots read cache row 0
        } else {
          krow[e] = pwin[min(j / P - pg0, npg - 1)] * P + (j % P);
        }
      }
#pragma unroll
      for (int e = 0; e < kMlaDmaPerWave; ++e) {
        const int cidx = cbase + e * 64;
        const int row = cidx / kMlaChunksPerRow;
        const uint32_t lg = (uint32_t)(((cidx - row * kMlaChunksPerRow) ^ lswz(row)) * 16);
        dma16(reinterpret_cast<const unsigned char*>(p.k) + (size_t)krow[e] * kMlaRowBytes + lg, lds0 + e * 1024);
      }
    }
  };

  // per-lane LDS byte offsets of the fragment reads (swizzle precomputed)
  // QK: A rows 16*half + n16 (this wave's keys), logical chunk 4*ks + grp; the
  // swizzle only touches the low three chunk bits, so the pattern repeats every 2 ks
  int qk_off[2];
  {
    const int r = half * 16 + n16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) qk_off[kk] = r * kMlaRowBytes + ((4 * kk + grp) ^ lswz(r)) * 16;
  }
  // PV (transposing reads): rows kb + n16/4 (kb = 4*grp or 16 + 4*grp), elements
  // 128*wid + 16*mb + 4*(n16 & 3): logical chunk 16*wid + 2*mb + ((n16 & 3) >> 1);
  // the pattern repeats every 4 mb (one aligned group of 8 chunks = 128 bytes)
  int pv_off[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = hh * 16 + grp * 4 + (n16 >> 2);
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      const int lc = 16 * wid + 2 * mm + ((n16 & 3) >> 1);
      pv_off[hh][mm] = r * kMlaRowBytes + (lc ^ lswz(r)) * 16 + (n16 & 1) * 8;
    }
  }
  // probability exchange: buffer b, block B (0..3), 16 bytes per lane = the
  // PV B operand of that block; the wave scoring keys [16h, 16h+16) fills
  // bytes [8h, 8h+8)
  auto xaddr = [&](int b, int blk) { return xbase + (uint32_t)(((b * 4 + blk) * 64 + lane) * 16); };

  // S^T of this wave's 16 keys x 32 vectors for the tile in stage `stg`
  // `between(ks)` runs after step ks's MFMAs (used to spread a tile's DMA)
  auto qk_tile = [&](uint32_t stg, f32x4_t (&sc)[2], auto&& between) {
    sc[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sc[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t a0 = stg + qk_off[0], a1 = stg + qk_off[1];
    u32x4_t fa[4];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) fa[ks] = lds_b128(((ks & 1) ? a1 : a0) + (ks >> 1) * 128);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      if (ks + 3 < 18) {
        const int kn = ks + 3;
        fa[kn & 3] = lds_b128(((kn & 1) ? a1 : a0) + (kn >> 1) * 128);
      }
      sc[0] = mfma16(fa[ks & 3], qf[0][ks], sc[0]);
      sc[1] = mfma16(fa[ks & 3], qf[1][ks], sc[1]);
      between(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_op = [](int) {};

  // own keys of this lane within a tile: 16*half + 4*grp + j; their
  // probabilities fill k-slots 8*grp + 4*half + j of the PV B operand
  const int key_lane = half * 16 + grp * 4;
  f32x4_t oacc[4][8];   // [block][16-column group of this wave's quarter]
  float m_ref[2] = {0.f, 0.f}, l_part[2], m_seen[2];
  float l_all[2] = {0.f, 0.f};

  // Softmax reference: each query vector's reference m_ref is the max of the
  // first tile's scaled scores (whole tile, both waves, mask ignored).
  // Probabilities are exp2(score - m_ref), so the O accumulators are never
  // rescaled.  After a pass the true max of the visible scores is known; if it
  // lies more than 2^32 above the reference (overflow risk) or more than 2^64
  // below it (underflow risk) the item runs once more with the true max.
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) oacc[blk][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      l_part[qb] = 0.f;
      m_seen[qb] = -INFINITY;
    }

    // scaled scores -> probabilities, one 16-vector block (4 keys per lane)
    auto soft = [&](const f32x4_t& sc, int qb, int t0, bool full, uint32_t (&out)[2]) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = sc[j] * p.scale_log2;
      if (!full) {   // edge tile: keys outside this vector's [low, lim] get probability 0
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = t0 + key_lane + j;
          bool out = k > lim[qb] || k < low[qb];
          if constexpr (SPARSE) out = out || sidx[min(k, kv_end - 1) - kv_begin] < 0;
          if (out) v[j] = -INFINITY;
        }
      }
      m_seen[qb] = fmaxf(m_seen[qb], fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_exp2f(v[j] - m_ref[qb]);   // exp2(-inf) = 0
      l_part[qb] += (e[0] + e[1]) + (e[2] + e[3]);
      out[0] = cvt_bf16x2(e[0], e[1]);
      out[1] = cvt_bf16x2(e[2], e[3]);
    };

    if (n_tiles > 0) {
      // prologue: tiles 0 and 1 in flight, probabilities of tile 0 published
      issue(0, 0);
      if (n_tiles > 1) issue(1, 1);
      if (n_tiles > 1) wait_vm<kMlaDmaPerWave>(); else wait_vm<0>();
      __syncthreads();
      f32x4_t sc[2];
      qk_tile(smem_lds, sc, no_op);
      if (pass == 0) {
        float mx[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          mx[qb] = fmaxf(fmaxf(sc[qb][0], sc[qb][1]), fmaxf(sc[qb][2], sc[qb][3])) * p.scale_log2;
          mx[qb] = fmaxf(mx[qb], __shfl_xor(mx[qb], 16));
          mx[qb] = fmaxf(mx[qb], __shfl_xor(mx[qb], 32));
          if (grp == 0) red_m[(wid * 2 + qb) * 16 + n16] = mx[qb];
        }
        __syncthreads();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) m_ref[qb] = fmaxf(mx[qb], red_m[((wid ^ 1) * 2 + qb) * 16 + n16]);
      }
      const bool full0 = is_full(kv_begin);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        uint32_t po[2];
        soft(sc[qb], qb, kv_begin, full0, po);
        lds_st_b64(xaddr(0, 2 * pair + qb) + half * 8, po[0], po[1]);
      }
    }

    // FAST: page of the tile the next iteration fetches, read one iteration ahead
    int pg_pref = 0;
    if constexpr (FAST)
      if (n_tiles > 0) pg_pref = page_at(min(2, n_tiles - 1));
    int st_cur = 0;                    // stage of tile t
    for (int t = 0; t < n_tiles; ++t) {
      // tile t+1 (next QK) must have landed; it is the only DMA in flight
      wait_vm<0>();
      __syncthreads();
      // DMA of tile t+2 into the stage tile t-1 used.  FAST spreads it over
      // the QK steps below; near the end it refetches the last tile into that
      // (dead) stage, which keeps the QK loop free of branches.
      DmaTile dnext{};
      if constexpr (FAST) {
        dnext = dma_tile(min(t + 2, n_tiles - 1), (t + 2) % kMlaStages, __builtin_amdgcn_readfirstlane(pg_pref));
        pg_pref = page_at(min(t + 3, n_tiles - 1));
      } else {
        if (t + 2 < n_tiles) issue(t + 2, (t + 2) % kMlaStages);
      }

      // the probabilities of tile t, all four blocks
      u32x4_t pb[4];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) pb[blk] = lds_b128(xaddr(t & 1, blk));

      const uint32_t stg = smem_lds + st_cur * kMlaStageBytes;
      st_cur = (st_cur == kMlaStages - 1) ? 0 : st_cur + 1;
      const uint32_t stg_next = smem_lds + st_cur * kMlaStageBytes;
      const bool more = t + 1 < n_tiles;   // uniform
      const int t0n = kv_begin + (t + 1) * kNK;
      const bool full_n = is_full(t0n);

      f32x4_t sc[2];
      auto spread_dma = [&](int ks) {
        if constexpr (FAST)
          if ((ks & 1) == 0) dma_one(dnext, ks >> 1);
      };
      if (more) {
        qk_tile(stg_next, sc, spread_dma);
      } else if constexpr (FAST) {
#pragma unroll
        for (int e = 0; e < kMlaDmaPerWave; ++e) dma_one(dnext, e);
      }

      // O^T[this wave's 128 columns] += V^T P^T; each transposed V fragment
      // feeds all four blocks.  The next tile's softmax runs between MFMAs so
      // that its VALU work overlaps them.
      uint32_t pn[2][2];
      {
        uint32_t av[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) av[hh][mm] = stg + pv_off[hh][mm];
        u32x4_t va[4];
        auto rd_v = [&](int mb) {
          const uint2 lo = lds_tr16(av[0][mb & 3] + (mb >> 2) * 128);
          const uint2 hi = lds_tr16(av[1][mb & 3] + (mb >> 2) * 128);
          return u32x4_t{lo.x, lo.y, hi.x, hi.y};
        };
#pragma unroll
        for (int mb = 0; mb < 3; ++mb) va[mb] = rd_v(mb);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          if (mb + 3 < 8) va[(mb + 3) & 3] = rd_v(mb + 3);
#pragma unroll
          for (int blk = 0; blk < 4; ++blk) oacc[blk][mb] = mfma16(va[mb & 3], pb[blk], oacc[blk][mb]);
          if (more && (mb == 1 || mb == 4)) soft(sc[mb >> 2], mb >> 2, t0n, full_n, pn[mb >> 2]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (more) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          lds_st_b64(xaddr((t + 1) & 1, 2 * pair + qb) + half * 8, pn[qb][0], pn[qb][1]);
      }
    }

    wait_vm<0>();   // no DMA in flight past the pass
    // column max of the visible scores and column sums, over the lane groups
    // and then over the pair
    float mcol[2], lcol[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mcol[qb] = fmaxf(m_seen[qb], __shfl_xor(m_seen[qb], 16));
      mcol[qb] = fmaxf(mcol[qb], __shfl_xor(mcol[qb], 32));
      lcol[qb] = l_part[qb] + __shfl_xor(l_part[qb], 16);
      lcol[qb] += __shfl_xor(lcol[qb], 32);
      if (grp == 0) {
        red_m[(wid * 2 + qb) * 16 + n16] = mcol[qb];
        red_l[(wid * 2 + qb) * 16 + n16] = lcol[qb];
      }
    }
    __syncthreads();
    int need = 0;
    float m_all[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      m_all[qb] = fmaxf(mcol[qb], red_m[((wid ^ 1) * 2 + qb) * 16 + n16]);
      l_all[qb] = lcol[qb] + red_l[((wid ^ 1) * 2 + qb) * 16 + n16];
      if (pass == 0 && q_valid[qb] && m_all[qb] > -INFINITY &&
          (m_all[qb] > m_ref[qb] + 32.f || m_all[qb] < m_ref[qb] - 64.f))
        need = 1;
    }
    if (!__syncthreads_or(need)) break;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
      if (m_all[qb] > -INFINITY) m_ref[qb] = m_all[qb];
  }   // pass

  // the scoring pair's statistics (lse, partial max and sum) for its own
  // blocks; the sums of the other pair's blocks come from its column sums
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (!q_valid[qb] || grp != 0 || half != 0) continue;
    const float l_tot = l_all[qb];
    const int qv = pair * 32 + qb * 16 + n16;
    if (ns == 1) {
      if (p.lse)
        p.lse[(size_t)q_row[qb] * p.Hq + head[qb]] = l_tot > 0.f ? (m_ref[qb] + log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int slot = info.z + sp * info.w + tile;
      if (slot >= 0 && slot < p.part_cap) {
        float* pml = p.part_ml + ((size_t)slot * kMlaQT + qv) * 2;
        pml[0] = l_tot > 0.f ? m_ref[qb] : -INFINITY;
        pml[1] = l_tot;
      }
    }
  }
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int qv = blk * 16 + n16;
    const int rl = qv / p.NH;
    if (rl >= rows_here) continue;
    const int row = row_start + row0 + rl;
    const int hd = hb * p.NH + (qv % p.NH);
    // column sum: the two scoring waves of the block's pair, in a fixed order
    const int pw = (blk >> 1) * 2;
    const float l_tot = red_l[(pw * 2 + (blk & 1)) * 16 + n16] + red_l[((pw + 1) * 2 + (blk & 1)) * 16 + n16];
    if (ns == 1) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      bf16_t* dst = p.o + ((size_t)row * p.Hq + hd) * kMlaDv + wid * 128;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        uint2 pk;
        pk.x = cvt_bf16x2(oacc[blk][mb][0] * inv, oacc[blk][mb][1] * inv);
        pk.y = cvt_bf16x2(oacc[blk][mb][2] * inv, oacc[blk][mb][3] * inv);
        *reinterpret_cast<uint2*>(dst + mb * 16 + grp * 4) = pk;
      }
    } else {
      const int slot = info.z + sp * info.w + tile;
      if (slot < 0 || slot >= p.part_cap) continue;
      float* po_ = p.part_o + ((size_t)slot * kMlaQT + qv) * kMlaDv + wid * 128;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
        *reinterpret_cast<f32x4_t*>(po_ + mb * 16 + grp * 4) = oacc[blk][mb];
    }
  }
}

// ---- latent kernel, one workgroup per packed row (all 128 heads) -----------------
//
// The 64-vector kernel above needs two workgroups for a 128-head row, so each
// 32-key tile is DMA'd into LDS twice and its value columns are read twice.
// Here one workgroup of four waves takes the whole row:
//  * QK: wave w scores vectors [32w, 32w+32) against all 32 keys of the tile
//    over the 576 dims with 32x32x16 MFMAs, S^T = K Q^T (K rows straight from
//    LDS, Q^T in 144 VGPRs); each K fragment feeds one MFMA.
//  * The 32x32 output layout gives lane l sixteen keys of vector l%32:
//    keys 8q + 4(l/32) + r (q, r < 4).  The PV MFMA's B operand (P^T, a
//    16-key step) wants eight keys per lane, so step s takes the keys of
//    q = 2s, 2s+1: each lane's own probabilities form its B operand with no
//    lane exchange, provided the V^T operand uses the same key order.  The
//    wave publishes its 32 vectors' probabilities (32 bytes per lane) for
//    the other waves.
//  * PV: wave w accumulates output columns [128w, 128w+128) for all 128
//    vectors, O^T += V^T P^T: four 32-column blocks x four 32-vector blocks
//    of 32x32x16 MFMAs (256 accumulators), V^T fragments from the row-major
//    key rows through transposing LDS reads (keys 16s + 4(l/32) + r and
//    16s + 8 + 4(l/32) + r of column l%32), each feeding four MFMAs.
// Per 32-key tile and row the LDS carries 36 KB of DMA, 144 KB of K
// fragment reads, 32 KB of V^T reads and 40 KB of probability exchange, about
// a quarter less than two 64-vector workgroups, with half the MFMA
// instructions.  Pipeline, softmax reference and rerun rule as above.
// Power-of-two pages of at least 32 keys (a tile lies in one page).
constexpr int kRowQT = 128;
constexpr int kRowKRing = 3;          // K fragment registers (read that many minus one MFMAs ahead)
constexpr int kRowXBytes = 2 * 4 * 2 * 64 * 16;   // probabilities [buffer][vector block][step][lane], 16 B
constexpr int kRowRedBytes = 4 * 32 * 4;      // per-vector sums [vector block][32]
constexpr int kRowQrBytes = 4 * 4 * 64 * 16;   // rope query fragments [wave][step][lane], 16 B
constexpr int kRowLdsBytes = kMlaStages * kMlaStageBytes + kRowXBytes + kRowRedBytes + kPageWin * 4 + kRowQrBytes;
static_assert(kRowLdsBytes <= 160 * 1024, "latent row kernel LDS");
static_assert(kMaxTopk <= kPageWin && kMaxTopk % 256 == 0, "a key list's slots fit the page-window area");

// SPARSE: the row attends to its key list (topk_idx); the item's slice of
// the list, less the entries that name no visible position, is compacted in
// list order into cache rows in the page-window area, and the tile loop runs
// over those slots as over dense keys, each DMA lane reading its slot's row.
template <bool SPARSE>
__device__ __forceinline__ void attn_mla_row_item(const MainParams& p, int item, unsigned char* smem) {
  constexpr int kRing = kMlaStages * kMlaStageBytes;
  float* red_l = reinterpret_cast<float*>(smem + kRing + kRowXBytes);
  int* pwin = reinterpret_cast<int*>(smem + kRing + kRowXBytes + kRowRedBytes);
  int* sidx = pwin;   // SPARSE: the compacted slots' cache rows (no page window then)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n32 = lane & 31;   // vector (QK) or column (PV) within a 32-block
  const int hl = lane >> 5;    // lane half: which keys of a step

  const int4 rec = p.items[item];
  const int i = rec.x, tile = rec.y, sp = rec.z;
  const int4 info = p.req_info[i];
  const int ns = info.x;
  const int row_start = p.cu[i];
  const int c = p.ctx[i];
  const int rl = tile / p.n_hb;          // the tile's packed row within the request
  const int hb = tile % p.n_hb;          // its block of 128 heads
  const int row = row_start + rl;
  const int pos = c + rl;                // the row's position: keys 0..pos are visible
  const int chunk = info.y;   // this request's chunk
  // keys [kv_begin, kv_end): positions, or (SPARSE) compacted slots
  const int kv_begin = SPARSE ? sp * chunk : win_origin(c, p.window) + sp * chunk;
  int kv_end = SPARSE ? min(kv_begin + chunk, p.topk) : min(kv_begin + chunk, pos + 1);
  const int P = p.page_size;
  const int* pt_row = p.page_table + (size_t)i * p.max_pages;

  const int pg0 = kv_begin / P;
  int npg = 0;
  if constexpr (SPARSE) {
    // list entries [kv_begin, kv_end) of this row (at most kMaxTopk, eight
    // per thread): those naming a position in 0..pos, in list order, as
    // cache rows; the other entries (-1 pads, later positions) are dropped
    const int32_t* src = p.topk_idx + (size_t)row * p.topk;
    int rr[kMaxTopk / 256], cnt[1] = {0};
#pragma unroll
    for (int k = 0; k < kMaxTopk / 256; ++k) {
      const int x = tid * (kMaxTopk / 256) + k;
      int r = -1;
      if (x < kv_end - kv_begin) {
        const int j = src[kv_begin + x];
        if (j >= 0 && j <= pos) {
          int pg = (j / P < p.max_pages) ? pt_row[j / P] : -1;
          if (pg < 0 || pg >= p.num_pages) { set_status(p.status, RV_DEV_BAD_PAGE); pg = 0; }
          r = pg * P + j % P;
        }
      }
      rr[k] = r;
      cnt[0] += r >= 0 ? 1 : 0;
    }
    // exclusive scan of the counts over the 256 threads (wave scan, then the
    // four wave totals through LDS)
    wave_incl_scan<1>(cnt);
    int* wtot = reinterpret_cast<int*>(red_l);
    if (lane == 63) wtot[wid] = cnt[0];
    __syncthreads();
    int off = cnt[0] - 0, all = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = wtot[u];
      off += u < wid ? v : 0;
      all += v;
    }
    int own = 0;
#pragma unroll
    for (int k = 0; k < kMaxTopk / 256; ++k) own += rr[k] >= 0 ? 1 : 0;
    off -= own;
#pragma unroll
    for (int k = 0; k < kMaxTopk / 256; ++k)
      if (rr[k] >= 0) sidx[off++] = rr[k];
    kv_end = kv_begin + all;   // the item's keys are now slots kv_begin .. kv_begin + all - 1
  } else {
    npg = kv_end > kv_begin ? (kv_end - 1) / P - pg0 + 1 : 0;
    if (npg > kPageWin) {
      if (tid == 0) set_status(p.status, RV_DEV_BAD_PAGE);
      npg = kPageWin;
    }
    for (int x = tid; x < npg; x += 256) {
      int pg = (pg0 + x < p.max_pages) ? pt_row[pg0 + x] : -1;
      if (pg < 0 || pg >= p.num_pages) { set_status(p.status, RV_DEV_BAD_PAGE); pg = 0; }
      pwin[x] = pg;
    }
  }
  const int lim = kv_end - 1;            // last key (slot) this item may see
  const int low = SPARSE ? INT32_MIN : win_low(pos, p.window);

  // query fragments: vector 32*wid + n32, dims 16*ks + 8*hl .. +7; the 512
  // value dims in registers, the 64 rope dims (steps 32..35) in this wave's
  // LDS area (each lane reads back only what it wrote)
  const int head = hb * kRowQT + wid * 32 + n32;
  const uint32_t qr_lds = (uint32_t)(uintptr_t)smem + kMlaStages * kMlaStageBytes + kRowXBytes + kRowRedBytes +
                          kPageWin * 4 + (uint32_t)((wid * 4 * 64 + lane) * 16);
  u32x4_t qf[32];
  {
    const bf16_t* qsrc = p.q + ((size_t)row * p.Hq + head) * kMlaD + hl * 8;
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qf[ks] = *reinterpret_cast<const u32x4_t*>(qsrc + ks * 16);
#pragma unroll
    for (int ks = 32; ks < 36; ++ks)
      *(lds_u32x4_t*)(size_t)(qr_lds + (ks - 32) * 1024) = *reinterpret_cast<const u32x4_t*>(qsrc + ks * 16);
  }
  auto is_full = [&](int t0) { return t0 + kNK - 1 <= lim && t0 >= low; };
  wait_vm<0>();
  __syncthreads();   // page window (SPARSE: compacted slots) visible

  const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + kNK - 1) / kNK : 0;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)smem;
  const uint32_t xbase = smem_lds + kRing;
  const uint32_t wave_lds = __builtin_amdgcn_readfirstlane(smem_lds + wid * kMlaDmaPerWave * 1024);
  const int cbase = wid * kMlaDmaPerWave * 64 + lane;
  const int last = kv_end - 1;
  // per DMA instruction e of this lane: its row r of the tile and chunk; the
  // byte offset r * row + swizzled chunk (SPARSE: r | chunk byte offset << 8)
  uint32_t dma_off[kMlaDmaPerWave];
#pragma unroll
  for (int e = 0; e < kMlaDmaPerWave; ++e) {
    const int cidx = cbase + e * 64;
    const int r = cidx / kMlaChunksPerRow;
    const uint32_t cb = (uint32_t)(((cidx - r * kMlaChunksPerRow) ^ lswz(r)) * 16);
    dma_off[e] = SPARSE ? (uint32_t)r | (cb << 8) : (uint32_t)(r * kMlaRowBytes) + cb;
  }
  struct DmaTile {
    const void* base;
    uint32_t lim;
    uint32_t lds0;
    int t0;
  };
  auto dma_tile = [&](int t, int st, int pg) {
    const int t0 = kv_begin + t * kNK;
    DmaTile d;
    d.base = SPARSE ? p.k
                    : uniform_ptr(reinterpret_cast<const unsigned char*>(p.k) +
                                  ((size_t)pg * P + (t0 & (P - 1))) * kMlaRowBytes);
    d.lim = (uint32_t)(min(last - t0, kNK - 1) * kMlaRowBytes + kMlaRowBytes - 16);
    d.lds0 = wave_lds + st * kMlaStageBytes;
    d.t0 = t0;
    return d;
  };
  // SPARSE: the cache row of the slot that DMA e of tile d reads (slots past
  // the item's last read the last one: finite data, masked)
  auto slot_row = [&](const DmaTile& d, int e) {
    return sidx[min(d.t0 + (int)(dma_off[e] & 255u), last) - kv_begin];
  };
  // (the chunk offset is taken through opaque() inside the loop: hoisted,
  // base + chunk would hold a 64-bit pair per DMA and the kernel would spill)
  auto dma_row = [&](const DmaTile& d, int e, int krow) {
    const uint64_t off = (uint64_t)(uint32_t)krow * kMlaRowBytes + (opaque(dma_off[e]) >> 8);
    dma16(reinterpret_cast<const unsigned char*>(p.k) + off, d.lds0 + e * 1024);
  };
  auto dma_one = [&](const DmaTile& d, int e) {
    if constexpr (SPARSE) dma_row(d, e, slot_row(d, e));
    else dma16_s(min(dma_off[e], d.lim), d.base, d.lds0 + e * 1024);
  };
  auto page_at = [&](int t) { return SPARSE ? 0 : pwin[((kv_begin + t * kNK) >> p.log2P) - pg0]; };
  auto issue = [&](int t, int st) {
    const DmaTile d = dma_tile(t, st, __builtin_amdgcn_readfirstlane(page_at(t)));
    if constexpr (SPARSE) {
      // every slot's row first (the LDS reads overlap), then the DMAs
      int kr[kMlaDmaPerWave];
#pragma unroll
      for (int e = 0; e < kMlaDmaPerWave; ++e) kr[e] = slot_row(d, e);
#pragma unroll
      for (int e = 0; e < kMlaDmaPerWave; ++e) dma_row(d, e, kr[e]);
    } else {
#pragma unroll
      for (int e = 0; e < kMlaDmaPerWave; ++e) dma_one(d, e);
    }
  };

  // QK fragment offsets: row n32, logical chunk 2*ks + hl; the swizzle
  // touches the low three chunk bits, so the pattern repeats every 4 ks
  uint32_t qk_off[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qk_off[kk] = n32 * kMlaRowBytes + ((2 * kk + hl) ^ lswz(n32)) * 16;
  // V^T reads: read `which` of step s covers keys 16s + 8*which + 4*hl + 0..3;
  // lane r of each 16-lane group addresses row key0 + (r&15)/4 and columns
  // c0 + 4*(r%4) with c0 = 128*wid + 32*cb + 16*((lane>>4)&1).  The row's
  // swizzle does not depend on s, and the column chunk's low bits only on cb&1.
  uint32_t pv_off[2][2];
#pragma unroll
  for (int wh = 0; wh < 2; ++wh) {
    const int r = 8 * wh + 4 * hl + ((lane & 15) >> 2);
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1) {
      const int lc = 4 * c1 + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);   // low chunk bits
      pv_off[wh][c1] = r * kMlaRowBytes + ((lc ^ lswz(r)) + 16 * wid) * 16 + (lane & 1) * 8;
    }
  }
  // probability exchange: [buffer][vector block][step][lane], 16 bytes each
  auto xaddr = [&](int b, int vb, int s2) { return xbase + (uint32_t)((((b * 4 + vb) * 2 + s2) * 64 + lane) * 16); };

  // K fragments (and, for the rope steps, Q fragments) read kRowKRing - 1
  // MFMAs ahead; the scheduling barrier keeps each read before the MFMA it
  // precedes (left alone, the compiler sinks it below, leaving one read in
  // flight)
  auto qk_tile = [&](uint32_t stg, f32x16_t& sc, auto&& between) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sc[j] = 0.f;
    u32x4_t fa[kRowKRing], qa[kRowKRing];
    uint32_t kb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kb[kk] = opaque(stg + qk_off[kk]);
    const uint32_t qrb = opaque(qr_lds);
    auto rd = [&](int kn) {
      fa[kn % kRowKRing] = lds_b128(kb[kn & 3] + (kn >> 2) * 128);
      if (kn >= 32) qa[kn % kRowKRing] = lds_b128(qrb + (kn - 32) * 1024);
    };
#pragma unroll
    for (int ks = 0; ks < kRowKRing - 1; ++ks) rd(ks);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      if (ks + kRowKRing - 1 < 36) rd(ks + kRowKRing - 1);
      __builtin_amdgcn_sched_barrier(0);
      sc = mfma32(fa[ks % kRowKRing], ks < 32 ? qf[ks < 32 ? ks : 0] : qa[ks % kRowKRing], sc);
      between(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_op = [](int) {};

  f32x16_t oacc[4][4];   // [32-column block][32-vector block]
  float m_ref = 0.f, l_part = 0.f, m_rel = -INFINITY, l_all = 0.f;

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[cb][vb][j] = 0.f;
    l_part = 0.f;
    m_rel = -INFINITY;   // largest visible scaled score less the reference

    // scaled scores -> the PV B operands of steps 0 and 1, for this lane's
    // 16 keys (key t0 + 8*(j/4) + 4*hl + j%4 of the tile), in registers of
    // their own (writing them back into the score accumulators would cost a
    // move each).  A full tile needs no mask: one fma per key forms the
    // exponent relative to the reference, and the largest exponent is the
    // tile's largest scaled score less the reference.  An edge tile masks
    // keys outside [low, lim].  The branch is uniform.
    auto soft = [&](const f32x16_t& sc, int t0, bool full, u32x4_t (&out)[2]) {
      float x[16];
      if (full) {
        const float mr = -m_ref;
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(sc[j], p.scale_log2, mr);
        float mx = x[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, x[j]);
        m_rel = fmaxf(m_rel, mx);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          x[j] = __builtin_amdgcn_exp2f(x[j]);
          sum += x[j];
        }
        l_part += sum;
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float v = sc[j] * p.scale_log2;
          const int k = t0 + 8 * (j >> 2) + 4 * hl + (j & 3);
          if (k > lim || k < low) v = -INFINITY;
          v -= m_ref;
          m_rel = fmaxf(m_rel, v);
          v = __builtin_amdgcn_exp2f(v);   // exp2(-inf) = 0
          l_part += v;
          x[j] = v;
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        out[s2] = u32x4_t{cvt_bf16x2(x[8 * s2 + 0], x[8 * s2 + 1]), cvt_bf16x2(x[8 * s2 + 2], x[8 * s2 + 3]),
                          cvt_bf16x2(x[8 * s2 + 4], x[8 * s2 + 5]), cvt_bf16x2(x[8 * s2 + 6], x[8 * s2 + 7])};
    };

    if (n_tiles > 0) {
      issue(0, 0);
      if (n_tiles > 1) issue(1, 1);
      if (n_tiles > 1) wait_vm<kMlaDmaPerWave>(); else wait_vm<0>();
      __syncthreads();
      f32x16_t sc;
      qk_tile(smem_lds, sc, no_op);
      if (pass == 0) {
        // reference: the max of the first tile's scaled scores (mask ignored)
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sc[j]);
        mx *= p.scale_log2;
        m_ref = fmaxf(mx, __shfl_xor(mx, 32));
      }
      u32x4_t po[2];
      soft(sc, kv_begin, is_full(kv_begin), po);
      *(lds_u32x4_t*)(size_t)(xaddr(0, wid, 0)) = po[0];
      *(lds_u32x4_t*)(size_t)(xaddr(0, wid, 1)) = po[1];
    }

    int pg_pref = 0;
    if (n_tiles > 0) pg_pref = page_at(min(2, n_tiles - 1));
    int st_cur = 0;
    for (int t = 0; t < n_tiles; ++t) {
      wait_vm<0>();
      __syncthreads();
      const DmaTile dnext =
          dma_tile(min(t + 2, n_tiles - 1), (t + 2) % kMlaStages, __builtin_amdgcn_readfirstlane(pg_pref));
      pg_pref = page_at(min(t + 3, n_tiles - 1));

      const uint32_t stg = smem_lds + st_cur * kMlaStageBytes;
      st_cur = (st_cur == kMlaStages - 1) ? 0 : st_cur + 1;
      const uint32_t stg_next = smem_lds + st_cur * kMlaStageBytes;
      const bool more = t + 1 < n_tiles;
      const int t0n = kv_begin + (t + 1) * kNK;
      const bool full_n = is_full(t0n);

      f32x16_t sc;
      // the next tile's DMA, one instruction every fourth QK step (issued
      // all at once, or during PV, it measured slower)
      // SPARSE: each DMA's slot row is read one DMA ahead
      int kr_next = 0;
      if constexpr (SPARSE) kr_next = slot_row(dnext, 0);
      auto spread_dma = [&](int ks) {
        if ((ks & 3) == 0) {
          const int e = ks >> 2;
          if constexpr (SPARSE) {
            const int kr = kr_next;
            if (e + 1 < kMlaDmaPerWave) kr_next = slot_row(dnext, e + 1);
            dma_row(dnext, e, kr);
          } else {
            dma_one(dnext, e);
          }
        }
      };
      if (more) {
        qk_tile(stg_next, sc, spread_dma);
      } else {
#pragma unroll
        for (int e = 0; e < kMlaDmaPerWave; ++e) dma_one(dnext, e);
      }

      // O^T[this wave's 128 columns][all vectors] += V^T P^T, step by step;
      // the next tile's softmax runs between the MFMAs of step 1
      u32x4_t pn[2];
      const uint32_t xb = opaque(xaddr(t & 1, 0, 0));
      uint32_t vbase[2][2];
#pragma unroll
      for (int wh = 0; wh < 2; ++wh)
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1) vbase[wh][c1] = opaque(stg + pv_off[wh][c1]);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        u32x4_t pb[4];
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) pb[vb] = lds_b128(xb + (vb * 2 + s2) * 1024);
        auto rd_v = [&](int cb) {
          const uint32_t c0 = s2 * 16 * kMlaRowBytes + (cb >> 1) * 128;
          const uint2 lo = lds_tr16(vbase[0][cb & 1] + c0);
          const uint2 hi = lds_tr16(vbase[1][cb & 1] + c0);
          return u32x4_t{lo.x, lo.y, hi.x, hi.y};
        };
        u32x4_t va[2];
        va[0] = rd_v(0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          if (cb + 1 < 4) va[(cb + 1) & 1] = rd_v(cb + 1);
#pragma unroll
          for (int vb = 0; vb < 4; ++vb) {
            if (cb == 3 && vb == 3) {
              // this block's accumulator is pinned to VGPRs: the other 15
              // (240 AGPRs) leave 16 AGPRs for the scores, so the compiler
              // no longer parks an output block in VGPRs around every QK
              // (48 accumulator moves a tile).  Its operands come straight
              // from LDS loads (waited on by the compiler); the block is
              // read again only by this MFMA (same accumulator, back to
              // back) and after the guard that follows the tile loop.
              asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                           : "+v"(oacc[3][3])
                           : "v"(va[cb & 1]), "v"(pb[vb]));
            } else {
              oacc[cb][vb] = mfma32(va[cb & 1], pb[vb], oacc[cb][vb]);
            }
          }
          // the next tile's softmax as one block after four MFMAs of step 1
          // (spread one key per MFMA, or sliced with a branch per slice, it
          // measured slower: the scheduling barriers and branch boundaries
          // cost the V^T reads their lead)
          if (more && s2 == 1 && cb == 0) soft(sc, t0n, full_n, pn);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (more) {
        *(lds_u32x4_t*)(size_t)(xaddr((t + 1) & 1, wid, 0)) = pn[0];
        *(lds_u32x4_t*)(size_t)(xaddr((t + 1) & 1, wid, 1)) = pn[1];
      }
    }
    // the pinned block's last MFMA (32 cycles) completes before anything
    // else reads or writes its registers: 32 wait states, ordered after it
    // by the operand
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(oacc[3][3]));

    wait_vm<0>();
    // each vector's visible max and sum: the two lane halves hold its keys
    const float m_seen = m_rel + m_ref;   // -inf when no key was visible
    const float m_all = fmaxf(m_seen, __shfl_xor(m_seen, 32));
    l_all = l_part + __shfl_xor(l_part, 32);
    const int need = (pass == 0 && m_all > -INFINITY && (m_all > m_ref + 32.f || m_all < m_ref - 64.f)) ? 1 : 0;
    if (!__syncthreads_or(need)) break;
    if (m_all > -INFINITY) m_ref = m_all;
  }   // pass

  // No spill reload among the output stores (each would wait for every store
  // issued before it): the VGPR-held accumulator block is brought back into
  // registers here, and the lane-dependent values come from an opaque lane
  // id (formed before the tile loop they would be held across it, spilled).
  asm volatile("" : "+v"(oacc[3][3]));
  const int le = (int)opaque((uint32_t)lane);
  const int n32e = le & 31, hle = le >> 5;
  // sums of every vector for the normalisation (block vb from wave vb)
  if (hle == 0) red_l[wid * 32 + n32e] = l_all;
  if (hle == 0) {
    if (ns == 1) {
      if (p.lse)
        p.lse[(size_t)row * p.Hq + hb * kRowQT + wid * 32 + n32e] =
            l_all > 0.f ? (m_ref + log2f(l_all)) * kLn2 : -INFINITY;
    } else {
      const int slot = info.z + sp * info.w + tile;
      if (slot >= 0 && slot < p.part_cap) {
        float* pml = p.part_ml + ((size_t)slot * kRowQT + wid * 32 + n32e) * 2;
        pml[0] = l_all > 0.f ? m_ref : -INFINITY;
        pml[1] = l_all;
      }
    }
  }
  __syncthreads();
  if (ns == 1) {
    // One vector block (32 vectors x 512 columns) at a time through the idle
    // ring: each wave writes its accumulators into LDS as they are (rows
    // padded by 16 bytes), then each thread scales 64 columns of one vector
    // by that vector's 1/sum and writes them as bf16, eight threads to a
    // 1 KB output row.  (Scaled where they sit, the compiler copies every
    // block out of the accumulator registers at once and spills them, and
    // each reload waits for the stores issued before it.)
    constexpr int kStRow = kMlaDv + 4;   // floats per staged row
    static_assert(32 * kStRow * 4 <= kRing, "a staged vector block fits the ring");
    const int sv = tid >> 3, sq = tid & 7;   // read-back: vector, column group
#pragma unroll
    for (int vb = 0; vb < 4; ++vb) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(lds_f32x4_t*)(size_t)(smem_lds + (uint32_t)(n32e * kStRow + wid * 128 + 32 * cb + 8 * q4 + 4 * hle) * 4) =
              f32x4_t{oacc[cb][vb][4 * q4], oacc[cb][vb][4 * q4 + 1], oacc[cb][vb][4 * q4 + 2],
                      oacc[cb][vb][4 * q4 + 3]};
      __syncthreads();
      const float l_tot = red_l[vb * 32 + sv];
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      bf16_t* dst = p.o + ((size_t)row * p.Hq + hb * kRowQT + vb * 32 + sv) * kMlaDv;
#pragma unroll
      for (int k = 0; k < kMlaDv / 32; ++k) {
        const int col = (k * 8 + sq) * 4;
        const f32x4_t x = *(const lds_f32x4_t*)(size_t)(smem_lds + (uint32_t)(sv * kStRow + col) * 4);
        uint2 pk;
        pk.x = cvt_bf16x2(x[0] * inv, x[1] * inv);
        pk.y = cvt_bf16x2(x[2] * inv, x[3] * inv);
        *reinterpret_cast<uint2*>(dst + col) = pk;
      }
      __syncthreads();   // the block is read before the next one is written
    }
  } else {
    const int slot = info.z + sp * info.w + tile;
    if (slot >= 0 && slot < p.part_cap) {
      float* po0 = p.part_o + ((size_t)slot * kRowQT + n32e) * kMlaDv + wid * 128 + 4 * hle;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        float* po_ = po0 + (size_t)vb * 32 * kMlaDv;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<f32x4_t*>(po_ + 32 * cb + 8 * q4) =
                f32x4_t{oacc[cb][vb][4 * q4], oacc[cb][vb][4 * q4 + 1], oacc[cb][vb][4 * q4 + 2],
                        oacc[cb][vb][4 * q4 + 3]};
      }
    }
  }
}

template <bool SPARSE>
__global__ __launch_bounds__(256) void k_attn_mla_row(MainParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_item;
  unsigned done = 0;
  for (;;) {
    const int item = next_item(p, &s_item, done);
    if (item < 0) break;
    attn_mla_row_item<SPARSE>(p, item, smem);
  }
}

// Max over lanes l, l^16, l^32, l^48 through gfx950's lane-swap moves (VALU,
// no LDS round trip): permlane32_swap exchanges the two 32-lane halves and
// permlane16_swap the odd and even 16-lane rows; each returns both swapped
// registers, so the max of the pair is the max over the partner lanes.
__device__ inline float max_lanes_xor16_32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---- GQA bf16 kernel (head dim 128): LDS DMA ring -------------------------------
//
// One workgroup = NV*KS waves against 16*NV query vectors (rows x query
// heads) of one KV head and one key chunk.  Wave w serves vector group
// w % NV and key group w / NV: the keys advance in super-tiles of KS*32 keys
// and key group k takes the k-th 32-key sub-tile of each, with an online
// softmax of its own; the KS states of a vector are merged through LDS at
// the end of the item.  Splitting the keys between waves puts a wave on
// every SIMD of the CU while one workgroup per CU keeps the bytes in flight
// (and so the memory latency) moderate.
//
// K and V sub-tiles arrive by direct global->LDS DMA into a ring of kStages
// super-tiles issued one stage short of the ring ahead; rows of 256 bytes
// whose 16-byte chunks are XOR-swizzled by (row >> 1) & 7; the request's
// page-table entries for the chunk sit in an LDS window (with power-of-two
// pages of at least 4 keys each DMA instruction's four rows share a page, so
// the DMA is a uniform page base plus lane offsets).  Per sub-tile the
// scores S^T = K Q^T and O^T += V^T P^T run on bf16 16x16x32 MFMAs (V^T
// fragments through transposing LDS reads); the accumulators are rescaled
// only when some vector's running max grows.
constexpr int kGqaD = 128;
constexpr int kGqaRow = kGqaD * 2;                         // bytes per K or V row
constexpr int kGqaSub = 2 * kNK * kGqaRow;                 // one sub-tile: K rows then V rows, 16 KB
constexpr int kGqaKS = 2;                                  // key groups per workgroup
template <int NV>
struct GqaCfg {
  static constexpr int kWaves = NV * kGqaKS;
  static constexpr int kStages = 4;
  static constexpr int kStage = kGqaKS * kGqaSub;
  static constexpr int kLds = kStages * kStage + kPageWin * 4;
  // the merge buffer (kGqaKS - 1 partner states of NV waves: 64 lanes x
  // (32 accumulators + max + sum) floats) reuses the ring after the loop
  static_assert((kGqaKS - 1) * NV * 64 * 34 * 4 <= kStages * kStage, "merge buffer");
};

// Keys [kv_lo, min(kv_hi, the tile's key count)) of tile `tile` of request
// i (context c, packed rows row_start .. row_start + w - 1).  slot < 0: the
// range is the tile's whole key range and the normalised output is written;
// otherwise fp32 partials go to partial slot `slot`.
template <int NV, bool FAST>
__device__ __forceinline__ void attn_gqa_range(const MainParams& p, int i, int tile, int c, int row_start, int w,
                                               int kv_lo, int kv_hi, int slot, unsigned char* smem) {
  using Cfg = GqaCfg<NV>;
  constexpr int NST = Cfg::kStages;
  constexpr int NWV = Cfg::kWaves;
  constexpr int kDmaPer = Cfg::kStage / 1024 / NWV;   // 1 KB DMA instructions per wave and super-tile
  constexpr int kChunksRow = kGqaRow / 16;            // 16
  constexpr int kInstSub = kGqaSub / 1024;            // 16 instructions per sub-tile
  constexpr int kSuper = kGqaKS * kNK;                // keys per super-tile
  int* pwin = reinterpret_cast<int*>(smem + NST * Cfg::kStage);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vg = wid % NV;   // vector group
  const int kg = wid / NV;   // key group
  const int n16 = lane & 15;
  const int grp = lane >> 4;

  const int rb = tile / (p.Hkv * p.n_hb);
  const int rem = tile % (p.Hkv * p.n_hb);
  const int g = rem / p.n_hb;
  const int hb = rem % p.n_hb;
  const int row0 = rb * p.RT;
  const int rows_here = min(p.RT, w - row0);
  const int L_tile = c + row0 + rows_here;
  const int kv_begin = kv_lo;
  const int kv_end = min(kv_hi, L_tile);
  const int P = p.page_size;

  // page-table window for keys [kv_begin, kv_end)
  const int pg0 = kv_begin / P;
  int npg = kv_end > kv_begin ? (kv_end - 1) / P - pg0 + 1 : 0;
  if (npg > kPageWin) {                 // context longer than the page table allows
    if (tid == 0) set_status(p.status, RV_DEV_BAD_PAGE);
    npg = kPageWin;
  }
  const int* pt_row = p.page_table + (size_t)i * p.max_pages;
  for (int x = tid; x < npg; x += 64 * NWV) {
    int pg = (pg0 + x < p.max_pages) ? pt_row[pg0 + x] : -1;
    if (pg < 0 || pg >= p.num_pages) { set_status(p.status, RV_DEV_BAD_PAGE); pg = 0; }
    pwin[x] = pg;
  }

  // this lane's query vector
  const int qv = vg * 16 + n16;
  const int q_row_local = qv / p.NH;
  const int head = g * p.G + hb * p.NH + (qv % p.NH);
  const bool q_valid = q_row_local < rows_here;
  const int q_row = row_start + row0 + q_row_local;
  const int limit = c + row0 + q_row_local;   // last visible key position
  const int low = win_low(limit, p.window);   // first visible key position
  // sub-tiles ending at or before this key need no mask for any real row;
  // with a window, neither do sub-tiles starting at or after every row's bound
  const int full_lim = min(c + row0, kv_end - 1);
  const int low_max = win_low(c + row0 + rows_here - 1, p.window);
  u32x4_t qf[kGqaD / 32];
#pragma unroll
  for (int ks = 0; ks < kGqaD / 32; ++ks) {
    if (q_valid) {
      const bf16_t* src = p.q + ((size_t)q_row * p.Hq + head) * kGqaD + ks * 32 + grp * 8;
      qf[ks] = *reinterpret_cast<const u32x4_t*>(src);
    } else {
      qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  wait_vm<0>();
  __syncthreads();   // page window visible

  const int n_tiles = kv_end > kv_begin ? (kv_end - kv_begin + kSuper - 1) / kSuper : 0;
  const uint32_t lds = (uint32_t)(uintptr_t)smem;
  const int last = kv_end - 1;   // keys past the end read this valid row (masked later)
  const size_t kv_head = (size_t)p.Hkv * kGqaD;   // elements between consecutive key rows

  // DMA of super-tile t into stage st: this wave's instruction e is
  // instruction q = wid*kDmaPer + e of the stage, i.e. instruction q % 16 of
  // sub-tile q / 16, moving chunks (q % 16)*64 + lane of that sub-tile (K
  // rows 0..31, then V rows); chunk cc of a row sits at physical position cc
  // and holds logical chunk cc ^ swz(row).  Per lane: the key offset within
  // the super-tile and the logical chunk (bytes) of each instruction.
  int dkey[kDmaPer], dlc[kDmaPer];
#pragma unroll
  for (int e = 0; e < kDmaPer; ++e) {
    const int q = wid * kDmaPer + e;
    const int c_ = (q % kInstSub) * 64 + lane;
    const int row = (c_ / kChunksRow) % kNK;
    dkey[e] = (q / kInstSub) * kNK + row;
    dlc[e] = ((c_ % kChunksRow) ^ swz(row)) * 16;
  }
  const unsigned char* gk = reinterpret_cast<const unsigned char*>(p.k + (size_t)g * kGqaD);
  const unsigned char* gv = reinterpret_cast<const unsigned char*>(p.v + (size_t)g * kGqaD);
  const uint64_t page_bytes = (uint64_t)P * kv_head * 2;
  const uint32_t row_bytes = (uint32_t)(kv_head * 2);

  // FAST: instruction q's four rows lie in one page, clamped rows included,
  // so its DMA is a uniform page base plus a 32-bit lane offset; the page
  // reads of a super-tile are issued together ahead of the fragment reads
  auto pages = [&](int t, int (&pgv)[kDmaPer]) {
    const int t0 = kv_begin + t * kSuper;
#pragma unroll
    for (int e = 0; e < kDmaPer; ++e) {
      const int q = wid * kDmaPer + e;
      const int jb = min(t0 + (q / kInstSub) * kNK + 4 * (q % (kNK / 4)), last);
      pgv[e] = pwin[min((jb >> p.log2P) - pg0, npg - 1)];
    }
  };
  auto issue = [&](int t, int st, const int (&pgv)[kDmaPer]) {
    const int t0 = kv_begin + t * kSuper;
    if constexpr (FAST) {
#pragma unroll
      for (int e = 0; e < kDmaPer; ++e) {
        const int q = wid * kDmaPer + e;
        const bool is_v = (q % kInstSub) >= kInstSub / 2;   // uniform: the V rows follow the K rows
        const uint32_t pg = (uint32_t)__builtin_amdgcn_readfirstlane(pgv[e]);   // validated: >= 0
        const void* base = uniform_ptr((is_v ? gv : gk) + (uint64_t)pg * page_bytes);
        const int j = min(t0 + dkey[e], last);
        // in-page row times row bytes: both below 2^24 (checked on the host)
        dma16_s(__umul24((uint32_t)(j & (P - 1)), row_bytes) + (uint32_t)dlc[e], base,
                __builtin_amdgcn_readfirstlane(lds + st * Cfg::kStage + q * 1024));
      }
    } else {
      (void)pgv;
      // every source row first (the LDS reads overlap), then the DMAs: the
      // asm statements order memory, so reads between them would serialise
      int tok[kDmaPer];
#pragma unroll
      for (int e = 0; e < kDmaPer; ++e) {
        const int j = min(t0 + dkey[e], last);
        tok[e] = pwin[min(j / P - pg0, npg - 1)] * P + (j % P);
      }
#pragma unroll
      for (int e = 0; e < kDmaPer; ++e) {
        const int q = wid * kDmaPer + e;
        const bool is_v = (q % kInstSub) >= kInstSub / 2;
        dma16((is_v ? gv : gk) + (size_t)tok[e] * row_bytes + dlc[e],
              __builtin_amdgcn_readfirstlane(lds + st * Cfg::kStage + q * 1024));
      }
    }
  };

  // fragment offsets within a sub-tile: QK A rows 16*mb + n16, logical
  // chunk 4*ks + grp; V^T transposing reads rows kb + n16/4 (kb = 4*grp or
  // 16 + 4*grp), elements 16*mb + 4*(n16 & 3): logical chunk 2*mb + ((n16 & 3) >> 1)
  auto k_addr = [&](uint32_t sub, int mb, int ks) {
    const int r = mb * 16 + n16;
    return sub + (uint32_t)(r * kGqaRow + ((4 * ks + grp) ^ swz(r)) * 16);
  };
  auto v_addr = [&](uint32_t sub, int hh, int mb) {
    const int r = hh * 16 + grp * 4 + (n16 >> 2);
    const int lc = 2 * mb + ((n16 & 3) >> 1);
    return sub + (uint32_t)(kNK * kGqaRow + r * kGqaRow + (lc ^ swz(r)) * 16 + (n16 & 1) * 8);
  };

  f32x4_t oacc[kGqaD / 16];
#pragma unroll
  for (int mb = 0; mb < kGqaD / 16; ++mb) oacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_part = 0.f;

  // prologue: super-tiles 0 .. NST-2 in flight
#pragma unroll
  for (int u = 0; u < NST - 1; ++u) {
    if (u < n_tiles) {
      int pgv[kDmaPer];
      if constexpr (FAST) pages(u, pgv);
      issue(u, u, pgv);
    }
  }
  int st = 0;
  for (int t = 0; t < n_tiles; ++t) {
    // super-tile t has landed once at most the NST-2 younger ones remain
    if (t + NST - 2 < n_tiles) wait_vm<(NST - 2) * kDmaPer>();
    else wait_vm<0>();
    __syncthreads();   // super-tile t visible; every wave is done with t-1
    const bool more = t + NST - 1 < n_tiles;
    int pgv[kDmaPer];
    if constexpr (FAST) {
      if (more) pages(t + NST - 1, pgv);
    }
    const uint32_t sub = lds + st * Cfg::kStage + kg * kGqaSub;
    // all K fragments of the sub-tile in flight before the DMA issue and the MFMAs
    u32x4_t kf[kNK / 16][kGqaD / 32];
#pragma unroll
    for (int mb = 0; mb < kNK / 16; ++mb)
#pragma unroll
      for (int ks = 0; ks < kGqaD / 32; ++ks) kf[mb][ks] = lds_b128(k_addr(sub, mb, ks));
    if (more) issue(t + NST - 1, (t + NST - 1) % NST, pgv);
    __builtin_amdgcn_sched_barrier(0);
    st = (st == NST - 1) ? 0 : st + 1;
    const int t0 = kv_begin + t * kSuper + kg * kNK;   // this wave's first key

    // S^T (keys x query vectors): lane holds keys 16*mb + 4*grp + j of query n16
    f32x4_t sacc[kNK / 16];
#pragma unroll
    for (int mb = 0; mb < kNK / 16; ++mb) sacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kGqaD / 32; ++ks)
#pragma unroll
      for (int mb = 0; mb < kNK / 16; ++mb) sacc[mb] = mfma16(kf[mb][ks], qf[ks], sacc[mb]);
    float tmax = -INFINITY;
    const bool full = (t0 + kNK - 1 <= full_lim) && t0 >= low_max;   // uniform: no key outside any real row's range
#pragma unroll
    for (int mb = 0; mb < kNK / 16; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s = sacc[mb][j] * p.scale_log2;
        if (!full) {
          const int kpos = t0 + mb * 16 + grp * 4 + j;
          if (kpos >= kv_end || kpos > limit || kpos < low) s = -INFINITY;
        }
        sacc[mb][j] = s;
        tmax = fmaxf(tmax, s);
      }
    }
    tmax = max_lanes_xor16_32(tmax);
    // no branch around the MFMAs: a fully masked query gets p = 0
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < kNK / 16; ++mb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pr = __builtin_amdgcn_exp2f(sacc[mb][j] - m_use);   // exp2(-inf) = 0
        sacc[mb][j] = pr;
        psum += pr;
      }
    }
    // rescale only when some vector's running max grew
    if (__any(m_new > m_run)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int mb = 0; mb < kGqaD / 16; ++mb) oacc[mb] *= alpha;
    }
    l_part += psum;
    m_run = m_new;
    // P^T as the B operand: k-slots 8*grp+x <-> keys 4*grp+x (x<4), 16+4*grp+x-4
    u32x4_t pb;
    pb[0] = cvt_bf16x2(sacc[0][0], sacc[0][1]);
    pb[1] = cvt_bf16x2(sacc[0][2], sacc[0][3]);
    pb[2] = cvt_bf16x2(sacc[1][0], sacc[1][1]);
    pb[3] = cvt_bf16x2(sacc[1][2], sacc[1][3]);
#pragma unroll
    for (int mb = 0; mb < kGqaD / 16; ++mb) {
      const uint2 lo = lds_tr16(v_addr(sub, 0, mb));
      const uint2 hi = lds_tr16(v_addr(sub, 1, mb));
      oacc[mb] = mfma16(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pb, oacc[mb]);
    }
  }
  wait_vm<0>();   // no DMA in flight past the item

  // normaliser over the four lane groups that share a query vector
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);

  // merge the key groups: groups 1.. publish (accumulators, max, sum) per
  // lane, group 0 rescales all of them to the common max and adds
  __syncthreads();   // every wave is done reading the ring
  float* xch = reinterpret_cast<float*>(smem);
  if (kg > 0) {
    float* dst = xch + ((size_t)((kg - 1) * NV + vg) * 64) * 34;
#pragma unroll
    for (int mb = 0; mb < kGqaD / 16; ++mb)
      *reinterpret_cast<f32x4_t*>(dst + (mb * 64 + lane) * 4) = oacc[mb];
    dst[32 * 64 + lane] = m_run;
    dst[33 * 64 + lane] = l_tot;
  }
  __syncthreads();
  if (kg > 0) return;
#pragma unroll
  for (int k = 1; k < kGqaKS; ++k) {
    const float* src = xch + ((size_t)((k - 1) * NV + vg) * 64) * 34;
    const float m_o = src[32 * 64 + lane];
    const float l_o = src[33 * 64 + lane];
    const float m_c = fmaxf(m_run, m_o);
    const float a_s = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_c);
    const float a_o = (m_o == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_o - m_c);
#pragma unroll
    for (int mb = 0; mb < kGqaD / 16; ++mb)
      oacc[mb] = oacc[mb] * a_s + *reinterpret_cast<const f32x4_t*>(src + (mb * 64 + lane) * 4) * a_o;
    l_tot = l_tot * a_s + l_o * a_o;
    m_run = m_c;
  }
  if (!q_valid) return;

  if (slot < 0) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16_t* dst = p.o + ((size_t)q_row * p.Hq + head) * kGqaD;
#pragma unroll
    for (int mb = 0; mb < kGqaD / 16; ++mb) {
      uint2 pk;
      pk.x = cvt_bf16x2(oacc[mb][0] * inv, oacc[mb][1] * inv);
      pk.y = cvt_bf16x2(oacc[mb][2] * inv, oacc[mb][3] * inv);
      *reinterpret_cast<uint2*>(dst + mb * 16 + grp * 4) = pk;
    }
    if (p.lse && grp == 0)
      p.lse[(size_t)q_row * p.Hq + head] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  } else {
    if (slot >= p.part_cap) return;   // the plans keep slots below the cap
    float* po = p.part_o + ((size_t)slot * (16 * NV) + qv) * kGqaD;
#pragma unroll
    for (int mb = 0; mb < kGqaD / 16; ++mb)
      *reinterpret_cast<f32x4_t*>(po + mb * 16 + grp * 4) = oacc[mb];
    if (grp == 0) {
      float* pml = p.part_ml + ((size_t)slot * (16 * NV) + qv) * 2;
      pml[0] = m_run;
      pml[1] = l_tot;
    }
  }
}

template <int NV, bool FAST>
__device__ __forceinline__ void attn_gqa_item(const MainParams& p, int item, unsigned char* smem) {
  const int4 rec = p.items[item];
  const int i = rec.x, tile = rec.y, sp = rec.z;
  const int4 info = p.req_info[i];
  const int chunk = info.y;   // this request's chunk
  const int kv_lo = win_origin(p.ctx[i], p.window) + sp * chunk;
  const int kv_hi = (int)min((long long)kv_lo + chunk, (long long)INT32_MAX);
  const int slot = info.x == 1 ? -1 : (info.z < 0 ? INT32_MAX : info.z + sp * info.w + tile);
  const int r0 = p.cu[i];
  attn_gqa_range<NV, FAST>(p, i, tile, p.ctx[i], r0, p.cu[i + 1] - r0, kv_lo, kv_hi, slot, smem);
}

// Balanced schedule: virtual worker v takes super-tiles [v*q, v*q+q) of the
// request-major sequence of every tile's 64-key super-tiles (the plan's
// k_attn_plan_bal), one contiguous range per worker, so every workgroup
// streams the same number of keys.  A range may start and end inside a
// tile; a tile covered by several ranges writes one partial per range.
template <int NV, bool FAST>
__global__ __launch_bounds__(64 * GqaCfg<NV>::kWaves) void k_attn_gqa_bal(MainParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kSuper = kGqaKS * kNK;
  static_assert(kSuper == kBalSuper, "the plan's super-tile is the kernel's");
  const int S = p.hdr[kBalS], q = p.hdr[kBalQ], n_vw = p.hdr[kBalVw], n_tiles = p.hdr[kBalTiles];
  const int4* tinfo = p.items;                                          // per tile
  const int* vw_first = reinterpret_cast<const int*>(p.items + n_tiles);
  const int4 none = make_int4(INT32_MAX, 0, 0, 0);
  for (int vw = blockIdx.x; vw < n_vw; vw += gridDim.x) {
    const int a = vw * q;
    const int b = min(a + q, S);
    // records read at clamped indices and replaced by `none` past the end
    // (a select between the loaded values, not between addresses)
    int T = vw_first[vw];
    int4 ti = tinfo[max(min(T, n_tiles - 1), 0)];   // {first super-tile, super-tiles, first slot or -1, request}
    if (T >= n_tiles) ti = none;
    for (; T < n_tiles && ti.x < b; ++T) {
      // the next tile's record is in flight while this range runs
      int4 ti_next = tinfo[min(T + 1, n_tiles - 1)];
      const int s0 = max(a, ti.x) - ti.x, s1 = min(b, ti.x + ti.y) - ti.x;
      if (s1 > s0) {
        // the request's values in one round of loads, ahead of the barrier
        const int i = ti.w;
        const int first = p.req_info[i].y, c = p.ctx[i], r0 = p.cu[i], r1 = p.cu[i + 1];
        const int slot = ti.z < 0 ? -1 : ti.z + (vw - ti.x / q);
        const int org = win_origin(c, p.window);
        __syncthreads();   // the previous range's merge and stores are done with the LDS
        attn_gqa_range<NV, FAST>(p, i, T - first, c, r0, r1 - r0, org + s0 * kSuper, org + s1 * kSuper, slot,
                                 smem);
      }
      // first read of the prefetched record here (the compiler would move it
      // to scalar registers, and so wait for it, right after the load)
      asm volatile("" : "+v"(ti_next.x), "+v"(ti_next.y), "+v"(ti_next.z), "+v"(ti_next.w));
      // (the same record in every lane: uniform again for what follows)
      ti = T + 1 < n_tiles ? make_int4(__builtin_amdgcn_readfirstlane(ti_next.x), __builtin_amdgcn_readfirstlane(ti_next.y),
                                       __builtin_amdgcn_readfirstlane(ti_next.z), __builtin_amdgcn_readfirstlane(ti_next.w))
                           : none;
    }
  }
}

template <int NV, bool FAST>
__global__ __launch_bounds__(64 * GqaCfg<NV>::kWaves) void k_attn_gqa(MainParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_item;
  unsigned done = 0;
  for (;;) {
    const int item = next_item(p, &s_item, done);
    if (item < 0) break;
    attn_gqa_item<NV, FAST>(p, item, smem);
  }
}

// ---- combine split partials ----------------------------------------------------
struct CombineParams {
  const int32_t* cu;
  const int4* req_info;
  const int4* tinfo;      // balanced plan: per tile {first super-tile, super-tiles, first slot or -1, request}
  const int2* split;      // {request, tile} of the tiles with split partials
  const int32_t* hdr;
  int bal;                // 1: slots from the balanced plan, 0: from the chunked plan
  const float* part_o;
  const float* part_ml;
  bf16_t* o;
  float* lse;
  const int32_t* mm;      // {M, M_pad}: rows [M, M_pad) are padding
  int Hq, Hkv, G, NH, RT, n_hb, QT, DV, tpr_max, part_cap, rows_cap;
};

// One workgroup per (request, tile with split keys, group of 8 query
// vectors).  The partials' maxima and sums give each vector its combined max
// m and sum l; each split's weight 2^(m_s - m) / l goes to LDS (in rounds of
// kCombRound splits) and every output element is the weighted sum of its
// partials, read as float4 runs.
constexpr int kCombVec = 8;       // query vectors per workgroup
constexpr int kCombRound = 512;   // split weights held in LDS at once

template <int DV>
__device__ __forceinline__ void combine_unit(const CombineParams& p, int i, int tile, int v0,
                                             float* s_red, float (*s_w)[kCombVec]) {
  constexpr int kPer = kCombVec * DV / 4 / 256;   // float4 runs per thread
  const int4 info = p.req_info[i];
  // partials of this tile: ns slots at slot0 + s * sstride
  int ns, slot0, sstride;
  if (p.bal) {
    if (tile >= info.x) return;
    const int4 ti = p.tinfo[info.y + tile];
    if (ti.z < 0) return;   // one worker covered the tile: written directly
    const int q = p.hdr[kBalQ];
    ns = (ti.x + ti.y - 1) / q - ti.x / q + 1;
    slot0 = ti.z;
    sstride = 1;
  } else {
    ns = info.x;
    if (ns <= 1 || tile >= info.w || info.z < 0) return;
    slot0 = info.z + tile;
    sstride = info.w;
  }
  if (slot0 + (ns - 1) * sstride >= p.part_cap) return;
  const int row_start = p.cu[i];
  const int w = p.cu[i + 1] - row_start;
  const int rb = tile / (p.Hkv * p.n_hb);
  const int rem = tile % (p.Hkv * p.n_hb);
  const int g = rem / p.n_hb;
  const int hb = rem % p.n_hb;
  const int row0 = rb * p.RT;
  const int rows_here = min(p.RT, w - row0);
  const int t = threadIdx.x;
  const int vl = t % kCombVec, ss = t / kCombVec;   // 32 split lanes per vector
  constexpr int kLanes = 256 / kCombVec;
  const int qv = v0 + vl;
  auto slot = [&](int s_) { return (size_t)(slot0 + s_ * sstride); };
  auto ml = [&](int s_) { return p.part_ml + (slot(s_) * p.QT + qv) * 2; };

  // combined max and sum (empty partials carry max -inf and sum 0)
  float m = -INFINITY;
  for (int s_ = ss; s_ < ns; s_ += kLanes) m = fmaxf(m, ml(s_)[0]);
  s_red[t] = m;
  __syncthreads();
  m = s_red[vl];
  for (int k = 1; k < kLanes; ++k) m = fmaxf(m, s_red[vl + k * kCombVec]);
  __syncthreads();
  float l = 0.f;
  if (m != -INFINITY)
    for (int s_ = ss; s_ < ns; s_ += kLanes) {
      const float ms = ml(s_)[0];
      if (ms != -INFINITY) l += exp2f(ms - m) * ml(s_)[1];
    }
  s_red[t] = l;
  __syncthreads();
  l = 0.f;
  for (int k = 0; k < kLanes; ++k) l += s_red[vl + k * kCombVec];
  const int rl = qv / p.NH;
  if (ss == 0 && rl < rows_here && p.lse) {
    const int head = g * p.G + hb * p.NH + (qv % p.NH);
    p.lse[(size_t)(row_start + row0 + rl) * p.Hq + head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }

  // this thread's float4 runs: element e = 4 * (t + 256 k) of the group
  float4 acc[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) acc[k] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int r0 = 0; r0 < ns; r0 += kCombRound) {
    const int nr = min(kCombRound, ns - r0);
    for (int s_ = ss; s_ < nr; s_ += kLanes) {
      const float ms = ml(r0 + s_)[0];
      s_w[s_][vl] = (l > 0.f && ms != -INFINITY) ? exp2f(ms - m) / l : 0.f;
    }
    __syncthreads();
    for (int s_ = 0; s_ < nr; ++s_) {
      const float4* src = reinterpret_cast<const float4*>(p.part_o + (slot(r0 + s_) * p.QT + v0) * DV);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int e = 4 * (t + 256 * k);
        const float wt = s_w[s_][e / DV];
        const float4 x = src[t + 256 * k];
        acc[k].x += wt * x.x;
        acc[k].y += wt * x.y;
        acc[k].z += wt * x.z;
        acc[k].w += wt * x.w;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = 4 * (t + 256 * k);
    const int v = v0 + e / DV;
    const int rv_ = v / p.NH;
    if (rv_ >= rows_here) continue;
    const int head = g * p.G + hb * p.NH + (v % p.NH);
    bf16_t* dst = p.o + ((size_t)(row_start + row0 + rv_) * p.Hq + head) * DV + (e % DV);
    uint2 pk;
    pk.x = pack_bf16x2(acc[k].x, acc[k].y);
    pk.y = pack_bf16x2(acc[k].z, acc[k].w);
    *reinterpret_cast<uint2*>(dst) = pk;
  }
}

// Grid-stride over (tile with split partials, group of 8 query vectors); the
// plan lists those tiles, so the grid is a fixed few workgroups per CU
// instead of one per possible tile.
template <int DV>
__global__ __launch_bounds__(256) void k_attn_combine(CombineParams p) {
  __shared__ float s_red[256];
  __shared__ float s_w[kCombRound][kCombVec];
  const int groups = p.QT / kCombVec;
  const int n_units = p.hdr[kHdrSplit] * groups;
  for (int u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int2 it = p.split[u / groups];
    __syncthreads();   // the previous unit is done with the LDS
    combine_unit<DV>(p, it.x, it.y, (u % groups) * kCombVec, s_red, s_w);
  }
  // padding rows [M, M_pad): o = 0 (16-byte stores; a row is Hq*DV bf16, a
  // multiple of 16 bytes), lse = -inf
  const int M = p.mm[0], Mpad = min(p.mm[1], p.rows_cap);
  const size_t n16 = (size_t)p.Hq * DV * 2 / 16;
  for (int r = max(M, 0) + blockIdx.x; r < Mpad; r += gridDim.x) {
    uint4* d = reinterpret_cast<uint4*>(p.o + (size_t)r * p.Hq * DV);
    for (size_t k = threadIdx.x; k < n16; k += 256) d[k] = make_uint4(0u, 0u, 0u, 0u);
    if (p.lse)
      for (int h = threadIdx.x; h < p.Hq; h += 256) p.lse[(size_t)r * p.Hq + h] = -INFINITY;
  }
}

// ---- padding rows [M, M_pad): o = 0, lse = -inf --------------------------------
__global__ __launch_bounds__(256) void k_attn_pad(const int32_t* mm, void* o, float* lse,
                                                  int Hq, int Dv, int elem_bytes, int rows_cap) {
  const int M = mm[0], Mpad = mm[1];
  const int row = M + blockIdx.x;
  if (row < 0 || row >= Mpad || row >= rows_cap) return;
  const size_t row_bytes = (size_t)Hq * Dv * elem_bytes;   // a whole number of 32-bit words
  char* base = static_cast<char*>(o) + (size_t)row * row_bytes;
  size_t done = 0;
  if (((uintptr_t)base % 16) == 0) {   // 16-byte stores over the aligned body
    uint4* d16 = reinterpret_cast<uint4*>(base);
    const size_t n16 = row_bytes / 16;
    for (size_t k = threadIdx.x; k < n16; k += blockDim.x) d16[k] = make_uint4(0u, 0u, 0u, 0u);
    done = n16 * 16;
  }
  uint32_t* d4 = reinterpret_cast<uint32_t*>(base + done);
  for (size_t k = threadIdx.x; k < (row_bytes - done) / 4; k += blockDim.x) d4[k] = 0u;
  if (lse)
    for (int h = threadIdx.x; h < Hq; h += blockDim.x) lse[(size_t)row * Hq + h] = -INFINITY;
}

// ---- fp32 path: one workgroup per (row, head) --------------------------------
struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* page_table;
  const int32_t* ctx;
  const int32_t* cu;
  const int32_t* mm;
  float* o;
  float* lse;
  int32_t* status;
  int B, max_pages, page_size, num_pages, Hq, Hkv, D, Dv;
  int window;             // sliding window (keys), 0 = full causal
  float sm_scale;
};

__global__ __launch_bounds__(128) void k_attn_f32(F32Params p) {
  __shared__ float sc[128];
  __shared__ float red[128];
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  if (row >= p.mm[0]) return;   // padding rows are written by k_attn_pad
  int lo = 0, hi = p.B - 1;     // request containing this row
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (p.cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int i = lo;
  const int pos = p.ctx[i] + (row - p.cu[i]);
  const int g = h / (p.Hq / p.Hkv);
  const float* qv = p.q + ((size_t)row * p.Hq + h) * p.D;
  const int P = p.page_size;
  float m = -INFINITY, l = 0.f, acc = 0.f;   // thread tid owns output dim tid
  const int j_lo = max(0, win_low(pos, p.window));
  for (int j0 = j_lo; j0 <= pos; j0 += 128) {
    const int j = j0 + tid;
    float s = -INFINITY;
    if (j <= pos) {
      int pg = (j / P < p.max_pages) ? p.page_table[(size_t)i * p.max_pages + j / P] : -1;
      if (pg < 0 || pg >= p.num_pages) { set_status(p.status, RV_DEV_BAD_PAGE); pg = 0; }
      const float* kr = p.k + (((size_t)pg * P + j % P) * p.Hkv + g) * p.D;
      float dot = 0.f;
      for (int d = 0; d < p.D; ++d) dot += qv[d] * kr[d];
      s = dot * p.sm_scale;
    }
    sc[tid] = s;
    red[tid] = s;
    __syncthreads();
    for (int off = 64; off > 0; off >>= 1) {
      if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
      __syncthreads();
    }
    const float m_new = fmaxf(m, red[0]);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    __syncthreads();
    const int n = min(128, pos + 1 - j0);
    float psum = 0.f, vacc = 0.f;
    for (int jj = 0; jj < n; ++jj) {
      const float pr = expf(sc[jj] - m_new);
      psum += pr;
      if (tid < p.Dv) {
        const int jk = j0 + jj;
        int pg = (jk / P < p.max_pages) ? p.page_table[(size_t)i * p.max_pages + jk / P] : -1;
        if (pg < 0 || pg >= p.num_pages) pg = 0;
        const float* vr = (p.v ? p.v : p.k) + (((size_t)pg * P + jk % P) * p.Hkv + g) * (p.v ? p.Dv : p.D);
        vacc += pr * vr[tid];
      }
    }
    l = l * alpha + psum;
    acc = acc * alpha + vacc;
    m = m_new;
    __syncthreads();
  }
  if (tid < p.Dv) p.o[((size_t)row * p.Hq + h) * p.Dv + tid] = acc / l;
  if (tid == 0 && p.lse) p.lse[(size_t)row * p.Hq + h] = m + logf(l);
}

// ---- host side -----------------------------------------------------------------
// row_tile (latent only): one tile per packed row and block of 128 heads,
// for the row kernel (Hq a multiple of 128)
bool pick_shape(int Hq, int Hkv, int Dqk, int Dv, int gamma, bool latent, AttnShape* sh, int* nw,
                bool row_tile = false) {
  if (Hkv <= 0 || Hq % Hkv != 0) return false;
  const int G = Hq / Hkv;
  if (latent) {
    if (!(Dqk == 576 && Dv == 512 && Hkv == 1 && Hq % 64 == 0)) return false;
    if (row_tile && Hq % kRowQT != 0) return false;
    *nw = (row_tile ? kRowQT : kMlaQT) / 16;   // 16 query vectors per block
  } else {
    if (!(Dqk == 128 && Dv == 128)) return false;
    if (!(G == 1 || G == 2 || G == 4 || G == 8 || G == 16)) return false;
    *nw = (G * gamma <= 32) ? 2 : 4;
  }
  const int QT = 16 * *nw;   // query vectors per tile
  sh->Hq = Hq;
  sh->Hkv = Hkv;
  sh->G = G;
  sh->QT = QT;
  sh->NH = G < QT ? G : QT;
  sh->RT = QT / sh->NH;
  sh->n_hb = G / sh->NH;
  sh->tpr_max = ((gamma + sh->RT - 1) / sh->RT) * Hkv * sh->n_hb;
  sh->target = latent ? (row_tile ? kTargetItemsLatentRow : kTargetItemsLatent) : kTargetItemsGqa;
  return true;
}

struct AttnScratch {
  size_t hdr, req_info, items, grp, split, part_ml, part_o, total;
  int item_cap, part_slots;
};

AttnScratch attn_layout(int B, const AttnShape& sh, int Dv) {
  AttnScratch L;
  L.item_cap = sh.target + B * sh.tpr_max;
  L.part_slots = (int)std::min<size_t>(kPartSlotsMax, kPartBytes / ((size_t)sh.QT * Dv * sizeof(float)));
  size_t off = 0;
  L.hdr = off; off = align_up(off + 256, 256);
  L.req_info = off; off = align_up(off + sizeof(int4) * (size_t)B, 256);
  L.items = off; off = align_up(off + sizeof(int4) * (size_t)L.item_cap, 256);
  L.grp = off; off = align_up(off + sizeof(int2) * (size_t)L.item_cap, 256);
  L.split = off; off = align_up(off + sizeof(int2) * (size_t)B * sh.tpr_max, 256);
  L.part_ml = off; off = align_up(off + sizeof(float) * 2 * (size_t)L.part_slots * sh.QT, 256);
  L.part_o = off; off = align_up(off + sizeof(float) * (size_t)L.part_slots * sh.QT * Dv, 256);
  L.total = off;
  return L;
}

// Workgroups that fit on the device at once (the persistent grid), rounded up
// to whole rounds of the 8 XCDs; cached per device and kernel.
hipError_t persistent_grid(const void* kern, int threads, int lds, int* grid) {
  struct Entry { const void* kern; int dev, grid; };
  static std::mutex mu;
  static Entry cache[32];
  static int n_cache = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(mu);
    for (int j = 0; j < n_cache; ++j)
      if (cache[j].kern == kern && cache[j].dev == dev) { *grid = cache[j].grid; return hipSuccess; }
  }
  int cus = 0, occ = 0;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, lds)) != hipSuccess) return e;
  const int g = ((std::max(cus, 1) * std::max(occ, 1) + 7) / 8) * 8;
  std::lock_guard<std::mutex> lk(mu);
  if (n_cache < 32) cache[n_cache++] = Entry{kern, dev, g};
  *grid = g;
  return hipSuccess;
}

template <int NV, bool FAST>
hipError_t launch_gqa_t(const MainParams& mp, hipStream_t s) {
  const void* kern = reinterpret_cast<const void*>(k_attn_gqa<NV, FAST>);
  constexpr int lds = GqaCfg<NV>::kLds;
  constexpr int threads = 64 * GqaCfg<NV>::kWaves;
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int grid = 0;
  if ((e = persistent_grid(kern, threads, lds, &grid)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_attn_gqa<NV, FAST>), dim3(grid), dim3(threads), lds, s, mp);
  return hipGetLastError();
}

template <int NV, bool FAST>
const void* gqa_bal_kernel() { return reinterpret_cast<const void*>(k_attn_gqa_bal<NV, FAST>); }

const void* gqa_bal_kernel(int nv, bool fast) {
  if (nv == 2) return fast ? gqa_bal_kernel<2, true>() : gqa_bal_kernel<2, false>();
  return fast ? gqa_bal_kernel<4, true>() : gqa_bal_kernel<4, false>();
}

// Persistent grid of the balanced GQA kernel (its LDS attribute set first).
hipError_t gqa_bal_grid(int nv, bool fast, int* grid) {
  const void* kern = gqa_bal_kernel(nv, fast);
  const int lds = nv == 2 ? GqaCfg<2>::kLds : GqaCfg<4>::kLds;
  const int threads = 64 * (nv == 2 ? GqaCfg<2>::kWaves : GqaCfg<4>::kWaves);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  return persistent_grid(kern, threads, lds, grid);
}

template <int NV, bool FAST>
hipError_t launch_gqa_bal_t(const MainParams& mp, int grid, hipStream_t s) {
  constexpr int lds = GqaCfg<NV>::kLds;
  constexpr int threads = 64 * GqaCfg<NV>::kWaves;
  hipLaunchKernelGGL((k_attn_gqa_bal<NV, FAST>), dim3(grid), dim3(threads), lds, s, mp);
  return hipGetLastError();
}

hipError_t launch_gqa_bal(const MainParams& mp, int nv, bool fast, int grid, hipStream_t s) {
  if (nv == 2) return fast ? launch_gqa_bal_t<2, true>(mp, grid, s) : launch_gqa_bal_t<2, false>(mp, grid, s);
  return fast ? launch_gqa_bal_t<4, true>(mp, grid, s) : launch_gqa_bal_t<4, false>(mp, grid, s);
}

// GQA bf16 (head dim 128): 16*nv query vectors per tile (nv = 2 or 4); FAST:
// power-of-two pages of at least 4 keys
hipError_t launch_gqa(const MainParams& mp, int nv, bool fast, hipStream_t s) {
  if (nv == 2) return fast ? launch_gqa_t<2, true>(mp, s) : launch_gqa_t<2, false>(mp, s);
  return fast ? launch_gqa_t<4, true>(mp, s) : launch_gqa_t<4, false>(mp, s);
}

}  // namespace

int attn_max_pages_limit(int dtype, bool latent) {
  return (dtype == RV_BF16) ? kPageWin - 1 : (1 << 30);   // bf16 kernels hold a page window
}

bool attn_shape_supported(int Hq, int Hkv, int Dqk, int Dv, int dtype, bool latent) {
  if (dtype == RV_F32) return Dqk <= 128 && Dv <= 128 && Dqk > 0 && Dv > 0 && Hkv > 0 && Hq % Hkv == 0 &&
                              (!latent || Dv <= Dqk);
  AttnShape sh;
  int nw;
  return pick_shape(Hq, Hkv, Dqk, Dv, 2, latent, &sh, &nw);
}

size_t attn_scratch_bytes(int B, int gamma, int Hq, int Hkv, int Dqk, int Dv, int dtype) {
  if (dtype == RV_F32 || B <= 0) return 0;
  AttnShape sh;
  int nw;
  const bool latent = (Dqk == 576);
  if (!pick_shape(Hq, Hkv, Dqk, Dv, gamma, latent, &sh, &nw)) return 0;
  size_t need = attn_layout(B, sh, Dv).total;
  if (latent && pick_shape(Hq, Hkv, Dqk, Dv, gamma, latent, &sh, &nw, true))
    need = std::max(need, attn_layout(B, sh, Dv).total);   // the row kernel's plan
  return need;
}

// What the plan and the main kernels of one bf16 attention call share: the
// kernel choice, the shape, the workspace layout and the plan's parameters.
struct AttnPrep {
  bool latent, row_kernel, bal, fast_gqa;
  int nw, bal_grid;
  AttnShape sh;
  AttnScratch L;
  char* base;
  PlanParams pp;
};

hipError_t prep_attn(const rv_attn_args& a, AttnPrep& P) {
  const bool latent = (a.v_cache == nullptr);
  char* ws = static_cast<char*>(a.workspace);
  hipError_t e;
  // latent: the row kernel for a multiple of 128 heads, with key lists
  // (sparse) or dense over power-of-two pages of at least 32 keys; the
  // 64-vector kernel otherwise
  const bool pow2_pages = (a.page_size & (a.page_size - 1)) == 0;
  const bool row_kernel = latent && a.Hq % kRowQT == 0 &&
                          (a.topk_idx != nullptr || (pow2_pages && a.page_size >= 32));
  AttnShape sh;
  int nw = 0;
  if (!pick_shape(a.Hq, a.Hkv, a.Dqk, a.Dv, a.gamma, latent, &sh, &nw, row_kernel)) return hipErrorInvalidValue;
  if (a.B > kPlanMaxB) return hipErrorInvalidValue;   // the plan caches one pair per request in LDS
  const AttnScratch L = attn_layout(a.B, sh, a.Dv);
  char* base = ws + kStatusBytes;

  // GQA: FAST DMA needs power-of-two pages of 4 .. 2^16 keys and rows under
  // 2^24 bytes (24-bit in-page offsets).  The balanced schedule applies when
  // its partial slots (at most workers + tiles) and worker list fit.
  const int log2P = ((a.page_size & (a.page_size - 1)) == 0) ? __builtin_ctz((unsigned)a.page_size) : -1;
  const bool fast_gqa = !latent && log2P >= 2 && log2P <= 16 && (long long)a.Hkv * kGqaD * 2 < (1 << 24);
  int bal_grid = 0;
  bool bal = false;
  if (!latent) {
    if ((e = gqa_bal_grid(nw, fast_gqa, &bal_grid)) != hipSuccess) return e;
    const long long tiles_max = (long long)a.B * sh.tpr_max;
    const long long st_max = ((long long)a.max_pages * a.page_size + kBalSuper - 1) / kBalSuper + kBalPro;
    bal = bal_grid <= 4 * (L.item_cap - tiles_max) && bal_grid + tiles_max <= L.part_slots &&
          tiles_max * st_max < INT32_MAX;
  }

  PlanParams& pp = P.pp;
  pp.cu = a.cu;
  pp.ctx = a.ctx;
  pp.mm = a.mm;
  pp.req_info = reinterpret_cast<int4*>(base + L.req_info);
  pp.items = reinterpret_cast<int4*>(base + L.items);
  pp.hdr = reinterpret_cast<int32_t*>(base + L.hdr);
  pp.grp = reinterpret_cast<int2*>(base + L.grp);
  pp.split = reinterpret_cast<int2*>(base + L.split);
  pp.B = a.B;
  pp.gamma = a.gamma;
  pp.item_cap = L.item_cap;
  pp.part_cap = L.part_slots;
  pp.target = sh.target;
  // workers of the main kernel (the chunked plan sizes its finer chunks by
  // them; 0 for the GQA fallback, which keeps one chunk length)
  int chunk_workers = 0;
  if (!bal && latent) {
    const bool sparse = a.topk_idx != nullptr;
    const bool fast = !sparse && (a.page_size & (a.page_size - 1)) == 0 && a.page_size >= 32;
    const void* kern = row_kernel ? (sparse ? reinterpret_cast<const void*>(k_attn_mla_row<true>)
                                            : reinterpret_cast<const void*>(k_attn_mla_row<false>))
                       : sparse ? reinterpret_cast<const void*>(k_attn_mla<false, true>)
                       : fast   ? reinterpret_cast<const void*>(k_attn_mla<true, false>)
                                : reinterpret_cast<const void*>(k_attn_mla<false, false>);
    const int lds = row_kernel ? kRowLdsBytes : kMlaLdsBytes;
    if ((e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds)) != hipSuccess) return e;
    if ((e = persistent_grid(kern, 256, lds, &chunk_workers)) != hipSuccess) return e;
  }
  pp.n_workers = bal ? bal_grid : chunk_workers;
  pp.window = a.window;
  pp.topk = a.topk_idx ? a.topk : 0;
  pp.sh = sh;
  P.latent = latent;
  P.row_kernel = row_kernel;
  P.bal = bal;
  P.fast_gqa = fast_gqa;
  P.nw = nw;
  P.bal_grid = bal_grid;
  P.sh = sh;
  P.L = L;
  P.base = base;
  return hipSuccess;
}

hipError_t launch_pack_plan(const rv_pack_args& pk, const rv_attn_args& a, hipStream_t s) {
  if (a.dtype == RV_F32) return launch_pack(pk, s);   // the fp32 kernel has no plan
  AttnPrep P;
  hipError_t e = prep_attn(a, P);
  if (e != hipSuccess) return e;
  if (P.bal) hipLaunchKernelGGL(k_pack_plan<true>, dim3(1), dim3(kPlanThreads), 0, s, make_pack_params(pk), P.pp);
  else hipLaunchKernelGGL(k_pack_plan<false>, dim3(1), dim3(kPlanThreads), 0, s, make_pack_params(pk), P.pp);
  return hipGetLastError();
}

hipError_t launch_attn(const rv_attn_args& a, hipStream_t s, bool planned) {
  int32_t* status = status_ptr(a.workspace);
  hipError_t e;

  if (a.dtype == RV_F32) {
    // padding rows here; the bf16 path's combine kernel writes them
    hipLaunchKernelGGL(k_attn_pad, dim3(a.rows_cap), dim3(256), 0, s, a.mm, a.o, a.lse, a.Hq, a.Dv, 4,
                       a.rows_cap);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    F32Params f;
    f.q = static_cast<const float*>(a.q);
    f.k = static_cast<const float*>(a.k_cache);
    f.v = static_cast<const float*>(a.v_cache);
    f.page_table = a.page_table;
    f.ctx = a.ctx;
    f.cu = a.cu;
    f.mm = a.mm;
    f.o = static_cast<float*>(a.o);
    f.lse = a.lse;
    f.status = status;
    f.B = a.B;
    f.max_pages = a.max_pages;
    f.page_size = a.page_size;
    f.num_pages = a.num_pages;
    f.Hq = a.Hq;
    f.Hkv = a.Hkv;
    f.D = a.Dqk;
    f.Dv = a.Dv;
    f.window = a.window;
    f.sm_scale = a.sm_scale;
    hipLaunchKernelGGL(k_attn_f32, dim3(a.rows_cap, a.Hq), dim3(128), 0, s, f);
    return hipGetLastError();
  }

  AttnPrep P;
  if ((e = prep_attn(a, P)) != hipSuccess) return e;
  const bool latent = P.latent, row_kernel = P.row_kernel, bal = P.bal, fast_gqa = P.fast_gqa;
  const int nw = P.nw, bal_grid = P.bal_grid;
  const AttnShape& sh = P.sh;
  const AttnScratch& L = P.L;
  char* base = P.base;
  const PlanParams& pp = P.pp;
  if (!planned) {   // else the pack launch built this call's plan (launch_pack_plan)
    if (bal) hipLaunchKernelGGL(k_attn_plan_bal, dim3(1), dim3(kPlanThreads), 0, s, pp);
    else hipLaunchKernelGGL(k_attn_plan, dim3(1), dim3(kPlanThreads), 0, s, pp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  MainParams mp;
  mp.q = static_cast<const bf16_t*>(a.q);
  mp.k = static_cast<const bf16_t*>(a.k_cache);
  mp.v = static_cast<const bf16_t*>(a.v_cache);
  mp.page_table = a.page_table;
  mp.ctx = a.ctx;
  mp.cu = a.cu;
  mp.req_info = pp.req_info;
  mp.items = pp.items;
  mp.hdr = pp.hdr;
  mp.o = static_cast<bf16_t*>(a.o);
  mp.lse = a.lse;
  mp.part_o = reinterpret_cast<float*>(base + L.part_o);
  mp.part_ml = reinterpret_cast<float*>(base + L.part_ml);
  mp.status = status;
  mp.max_pages = a.max_pages;
  mp.page_size = a.page_size;
  mp.num_pages = a.num_pages;
  mp.Hq = a.Hq;
  mp.Hkv = a.Hkv;
  mp.G = sh.G;
  mp.NH = sh.NH;
  mp.RT = sh.RT;
  mp.n_hb = sh.n_hb;
  mp.part_cap = L.part_slots;
  mp.log2P = -1;
  if ((a.page_size & (a.page_size - 1)) == 0) {
    int l2 = 0;
    while ((1 << l2) < a.page_size) ++l2;
    mp.log2P = l2;
  }
  mp.scale_log2 = a.sm_scale * kLog2e;
  mp.window = a.window;
  mp.topk_idx = a.topk_idx;
  mp.topk = a.topk_idx ? a.topk : 0;
  mp.ctr = pp.hdr + kHdrCtr;

  if (row_kernel) {
    const bool sparse = a.topk_idx != nullptr;
    const void* kern = sparse ? reinterpret_cast<const void*>(k_attn_mla_row<true>)
                              : reinterpret_cast<const void*>(k_attn_mla_row<false>);
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kRowLdsBytes);
    if (e != hipSuccess) return e;
    int grid = 0;
    if ((e = persistent_grid(kern, 256, kRowLdsBytes, &grid)) != hipSuccess) return e;
    if (sparse) hipLaunchKernelGGL(k_attn_mla_row<true>, dim3(grid), dim3(256), kRowLdsBytes, s, mp);
    else hipLaunchKernelGGL(k_attn_mla_row<false>, dim3(grid), dim3(256), kRowLdsBytes, s, mp);
    e = hipGetLastError();
  } else if (latent) {
    const bool sparse = a.topk_idx != nullptr;
    const bool fast = !sparse && mp.log2P >= 5;   // power-of-two pages of at least 32 keys
    const void* kern = sparse ? reinterpret_cast<const void*>(k_attn_mla<false, true>)
                       : fast ? reinterpret_cast<const void*>(k_attn_mla<true, false>)
                              : reinterpret_cast<const void*>(k_attn_mla<false, false>);
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kMlaLdsBytes);
    if (e != hipSuccess) return e;
    int grid = 0;
    if ((e = persistent_grid(kern, 256, kMlaLdsBytes, &grid)) != hipSuccess) return e;
    if (sparse) hipLaunchKernelGGL((k_attn_mla<false, true>), dim3(grid), dim3(256), kMlaLdsBytes, s, mp);
    else if (fast) hipLaunchKernelGGL((k_attn_mla<true, false>), dim3(grid), dim3(256), kMlaLdsBytes, s, mp);
    else hipLaunchKernelGGL((k_attn_mla<false, false>), dim3(grid), dim3(256), kMlaLdsBytes, s, mp);
    e = hipGetLastError();
  } else {
    e = bal ? launch_gqa_bal(mp, nw, fast_gqa, bal_grid, s) : launch_gqa(mp, nw, fast_gqa, s);
  }
  if (e != hipSuccess) return e;

  CombineParams cp;
  cp.cu = a.cu;
  cp.req_info = pp.req_info;
  cp.tinfo = pp.items;
  cp.split = pp.split;
  cp.hdr = pp.hdr;
  cp.bal = bal ? 1 : 0;
  cp.part_o = mp.part_o;
  cp.part_ml = mp.part_ml;
  cp.o = mp.o;
  cp.lse = a.lse;
  cp.Hq = a.Hq;
  cp.Hkv = a.Hkv;
  cp.G = sh.G;
  cp.NH = sh.NH;
  cp.RT = sh.RT;
  cp.n_hb = sh.n_hb;
  cp.QT = sh.QT;
  cp.DV = a.Dv;
  cp.tpr_max = sh.tpr_max;
  cp.part_cap = L.part_slots;
  cp.mm = a.mm;
  cp.rows_cap = a.rows_cap;
  int cus = 0, dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
  const dim3 cgrid((unsigned)std::max(1LL, std::min((long long)a.B * sh.tpr_max * (sh.QT / kCombVec),
                                                     4LL * std::max(cus, 1))));
  if (a.Dv == 512) hipLaunchKernelGGL(k_attn_combine<512>, cgrid, dim3(256), 0, s, cp);
  else hipLaunchKernelGGL(k_attn_combine<128>, cgrid, dim3(256), 0, s, cp);
  return hipGetLastError();
}

}  // namespace rv
