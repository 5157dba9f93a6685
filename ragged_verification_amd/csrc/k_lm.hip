// Stage 4: target LM head over the packed rows and the acceptance rule.
//
// The verify forward ends in the target's vocabulary projection of every
// packed row; drafts are checked against it (lshu.cn DSpark explainer, section
// 1.2: keep drafts up to the first disagreement; sections 2.3 and 3.3: keep
// draft x with probability min(1, p(x)/q(x))).  cap-accept verifies the whole
// block but commits up to the scheduled window and reports the ceiling
// (DSpark-in-SGLang page, section A2 "verify modes" and "observability").
//
// Design (gfx950).  z = X W^T on bf16 32x32x16 MFMAs with fp32
// accumulation; the epilogue of every GEMM goes through an LDS transpose and
// reduces each (row, 64-column slab) to (max, lowest argmax, sum of
// exp(z - max)) in 16 bytes, writing the logits (row-contiguous float4
// runs) only when asked.  Workgroups past the packed row count M exit at
// once, so the work follows M, not the tier.
//  * k_lm_tile_weight (once per weight, model-load work) writes W in MFMA
//    fragment order: blocks of 32 vocabulary rows, each a run of H/16
//    fragments of 1 KB, so a wave's B operand for one MFMA is one fully
//    coalesced 1 KB load straight into registers.
//  * k_lm_gemm_tiled (the path for more than 256 row slots): 128 rows x 512
//    (or 256) vocabulary columns per workgroup, each wave 128 x 128 in 256
//    accumulators; its weight fragments come into an 8-deep register ring
//    seven 16-wide K sub-steps ahead, the hidden rows through a four-stage
//    LDS ring (128-byte rows XOR-swizzled by (row >> 1) & 7); the row tiles
//    of one vocabulary tile are consecutive on one XCD so they share its
//    weights through L2; MFMAs only for the 32-row blocks that hold packed
//    rows.
//  * k_lm_gemm_rows (33 to 256 row slots): all packed rows in one tile
//    against 128 columns, each wave one 32-column block and every row block,
//    so each weight byte is loaded by one wave once (16-deep register ring);
//    above 224 packed rows it switches to two 128-row tiles.
//  * k_lm_gemm_small (at most 32 row slots): one-wave 32 x 64 tiles streaming
//    the weight, both operands straight into 16-deep register rings.
//  * k_lm_gemm: the row-major weight, both operands by DMA into a
//    three-stage LDS ring (used when no tiled copy is given).
//  * k_lm_f32: the same partials from fp32 inputs (plain dot products).
//  * k_accept: one workgroup per request merges the slab partials of its
//    rows, runs the greedy or rejection scan, and for rejection draws the
//    bonus token by an inverse CDF over the vocabulary (fp64 sums of
//    4096-token segments, a scan of them, then a walk inside the segment
//    that holds the target).

#include <float.h>

#include "rv_common.h"

namespace rv {
namespace {

constexpr int kBM = 128, kBK = 64;             // workgroup rows and K step
constexpr int kSlab = 64;                        // columns per partial
constexpr int kGemmThreads = 256;
constexpr int kGRow = kBK * 2;                   // bytes per LDS row: 8 chunks of 16, one 128-byte line
constexpr int kGChunks = kGRow / 16;
constexpr int kGBOff = kBM * kGRow;              // B rows follow the A rows in a stage
constexpr int kGDmaA = kBM * kGChunks / 64;      // 1 KB DMA instructions per stage: A
constexpr int kGKs = kBK / 16;                   // 32x32x16 MFMA steps per K step
constexpr int kGDmaGap = 2;                      // MFMAs between a wave's DMA instructions

// Workgroup tile 128 rows x BN vocabulary columns (each wave 128 x BN/4).
// The launch uses BN = 256 (three 48 KB stages); BN = 512 (each wave
// 128 x 128 in 256 accumulators, two 80 KB stages) compiles as well.
constexpr int kGemmBN = 256;   // the launched tile width

template <int BN>
struct GemmCfg {
  static constexpr int kWN = BN / 4;                          // columns per wave
  static constexpr int kNB = kWN / 32;                        // 32-column blocks per wave
  static constexpr int kStage = (kBM + BN) * kGRow;           // 80 KB / 48 KB
  // ring stages: two 80 KB (the whole LDS) or three 48 KB, so the narrow
  // tiles keep two steps in flight (they stream weights with few MFMAs)
  static constexpr int kStages = BN == 512 ? 2 : 3;
  static constexpr int kLds = kStages * kStage;               // 160 KB / 144 KB
  static constexpr int kDma = (kBM + BN) * kGChunks / 64;     // 1 KB DMA instructions per stage
  static constexpr int kDmaPerWave = kDma / 4;
  static constexpr int kERow = kWN + 4;                       // floats per padded epilogue row
  static constexpr int kSlabs = kWN / kSlab;                  // partial slabs per wave
  static_assert(kDma % 4 == 0, "DMA split over waves");
  static_assert(kDmaPerWave * kGDmaGap <= kGKs * 4 * kNB, "DMA spread fits the step");
  static_assert(kGemmThreads / 64 * 32 * kERow * 4 <= kLds, "epilogue fits the ring");
};

struct GemmParams {
  const bf16_t* x;     // [rows][H]
  const bf16_t* w;     // [V][H]
  const int32_t* mm;
  float4* part;        // [rows][n_slabs]
  float* logits;       // optional [rows][V]
  int H, V, n_slabs, n_mt, n_vt;
  int with_sum;
  int ncb;             // 32-column blocks of the tiled weight
  int cus;             // compute units of the device
  size_t w_bytes;      // bytes of the tiled weight
};

__device__ inline void merge_best(float& v, int& idx, float ov, int oidx) {
  if (ov > v || (ov == v && oidx < idx)) { v = ov; idx = oidx; }
}

// 128-byte LDS rows: chunk c of row r sits at c ^ gswz(r), so the 16 rows
// that one quarter-wave reads at one logical chunk (two rows per 256-byte
// bank line) fall on 16 distinct bank groups
__device__ inline int gswz(int row) { return (row >> 1) & 7; }

// Epilogue of both GEMM kernels, through LDS (the operand ring is free): for
// each 32-row block the wave writes its 32 x WN fp32 tile (rows padded to
// WN + 4 floats), then lane t reduces row t % 32 over its 64-column slab
// t / 32 to (max, lowest argmax, sum of exp(z - max)).  Accumulator lane l
// holds column l % 32 of rows 8*(j/4) + 4*(l/32) + j%4.
template <int WN, int BMB = 4>
__device__ __forceinline__ void lm_epilogue(f32x16_t (&acc)[BMB][WN / 32], unsigned char* smem,
                                            const GemmParams& p, int wid, int lane, int m0, int v0, int M) {
  constexpr int kNB = WN / 32;
  const int l32 = lane & 31, lh = lane >> 5;
  constexpr int kERow = WN + 4;               // floats per padded LDS row
  float* et = reinterpret_cast<float*>(smem) + wid * 32 * kERow;
  const int er = lane & 31, es = lane >> 5;       // reduced row and slab
  // float4 logits stores when every row starts 16-byte aligned
  const bool vec_logits = (p.V % 4) == 0 && ((uintptr_t)p.logits % 16) == 0;
  const int cslab = v0 + wid * WN + es * kSlab;  // first column of the slab
  const bool reducer = es < WN / kSlab;          // lanes with a slab to reduce
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm) {
#pragma unroll
    for (int bn = 0; bn < kNB; ++bn)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        et[((j / 4) * 8 + lh * 4 + (j % 4)) * kERow + bn * 32 + l32] = acc[bm][bn][j];
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const int row = m0 + bm * 32 + er;
    const float* src = et + er * kERow + (reducer ? es : 0) * kSlab;
    float z[kSlab];
#pragma unroll
    for (int i = 0; i < kSlab; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      z[i] = v.x; z[i + 1] = v.y; z[i + 2] = v.z; z[i + 3] = v.w;
    }
    float best = -INFINITY;
    int bi = cslab;
#pragma unroll
    for (int i = 0; i < kSlab; ++i) {
      if (cslab + i >= p.V) z[i] = -INFINITY;
      if (z[i] > best) { best = z[i]; bi = cslab + i; }   // strict: lowest index wins ties
    }
    float se = 0.f;
    if (p.with_sum && best != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kSlab; ++i) se += (z[i] == -INFINITY) ? 0.f : __expf(z[i] - best);
    }
    if (reducer && row < M && cslab < p.V)
      p.part[(size_t)row * p.n_slabs + cslab / kSlab] = make_float4(best, __int_as_float(bi), se, 0.f);
    if (p.logits) {
      // row-contiguous stores of the wave's 32 x WN block: WN/4 lanes
      // write one row's columns as float4 runs, the other lanes the next rows
      constexpr int kLanesRow = WN / 4;
      constexpr int kRowsPer = 64 / kLanesRow;
      const int c4 = (lane % kLanesRow) * 4;
      const int gcol = v0 + wid * WN + c4;
#pragma unroll 4
      for (int rr = 0; rr < 32 / kRowsPer; ++rr) {
        const int rl = kRowsPer * rr + lane / kLanesRow;
        const int grow = m0 + bm * 32 + rl;
        if (grow >= M) continue;
        const float4 v = *reinterpret_cast<const float4*>(et + rl * kERow + c4);
        float* dst = p.logits + (size_t)grow * p.V + gcol;
        if (vec_logits && gcol + 3 < p.V) {
          *reinterpret_cast<float4*>(dst) = v;
        } else {
          const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (gcol + c < p.V) dst[c] = e4[c];
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);   // reads done before the next block overwrites
  }
}

template <int BN>
__global__ __launch_bounds__(kGemmThreads) void k_lm_gemm(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  using Cfg = GemmCfg<BN>;
  constexpr int kGStage = Cfg::kStage;
  constexpr int kGDmaPerWave = Cfg::kDmaPerWave;
  constexpr int kNB = Cfg::kNB;
  constexpr int kWN = Cfg::kWN;
  constexpr int kGStages = Cfg::kStages;

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
  const int v0 = vt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const uint32_t lds = (uint32_t)(uintptr_t)smem;

  // DMA: instruction q (0 .. kGDma-1) of a stage moves chunks 64q .. 64q+63
  // (A rows first, then B rows), eight whole 128-byte rows per instruction
  // (a full cache line per row: half-line rows halve the DMA rate); wave w
  // issues q = w*kGDmaPerWave + e.  Chunk c sits at row c/8, physical
  // position c%8 and holds logical chunk (c%8) ^ gswz(row).  Rows past the
  // real ones read the last real row.
  const unsigned char* baseA = reinterpret_cast<const unsigned char*>(p.x + (size_t)m0 * p.H);
  const unsigned char* baseB = reinterpret_cast<const unsigned char*>(p.w + (size_t)v0 * p.H);
  uint32_t doff[kGDmaPerWave];
#pragma unroll
  for (int e = 0; e < kGDmaPerWave; ++e) {
    const int q = wid * kGDmaPerWave + e;
    const bool is_a = q < kGDmaA;
    const int c = (is_a ? q : q - kGDmaA) * 64 + lane;
    const int row = c / kGChunks;
    const int lc = (c % kGChunks) ^ gswz(row);
    const int r = is_a ? min(row, M - 1 - m0) : min(row, p.V - 1 - v0);
    doff[e] = (uint32_t)r * (uint32_t)(p.H * 2) + (uint32_t)lc * 16u;
  }
  auto dma = [&](int kt, int st, int e) {
    const int q = wid * kGDmaPerWave + e;
    const bool is_a = q < kGDmaA;   // uniform
    const void* base = uniform_ptr((is_a ? baseA : baseB) + (size_t)kt * kGRow);
    dma16_s(doff[e], base, __builtin_amdgcn_readfirstlane(lds + st * kGStage + q * 1024));
  };

  // fragment reads: row 32*b + l32 of A (rows) or of this wave's B columns,
  // logical chunk 2*ks + lh
  uint32_t foff[kGKs];
#pragma unroll
  for (int ks = 0; ks < kGKs; ++ks) foff[ks] = (uint32_t)(l32 * kGRow + (((2 * ks + lh) ^ gswz(l32)) * 16));
  const uint32_t bq = (uint32_t)(kGBOff + wid * kWN * kGRow);

  f32x16_t acc[4][kNB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  const int nk = p.H / kBK;
  // ring: steps kt+1 .. kt+kGStages-1 are in flight while step kt is
  // multiplied; the DMA of step kt+kGStages-1 is spread over its MFMAs
  // (past the end: the last step again, into a dead stage)
#pragma unroll
  for (int u = 0; u < kGStages - 1; ++u)
#pragma unroll
    for (int e = 0; e < kGDmaPerWave; ++e) dma(min(u, nk - 1), u, e);
  wait_vm<(kGStages - 2) * kGDmaPerWave>();
  __syncthreads();

  int st = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const uint32_t stg = lds + st * kGStage;
    u32x4_t fa[2][4], fb[2][kNB];
#pragma unroll
    for (int b = 0; b < 4; ++b) fa[0][b] = lds_b128(stg + b * 32 * kGRow + foff[0]);
#pragma unroll
    for (int b = 0; b < kNB; ++b) fb[0][b] = lds_b128(stg + bq + b * 32 * kGRow + foff[0]);
    // the stage of step kt+kGStages-1 is the one step kt-1 used
    const int kn = min(kt + kGStages - 1, nk - 1);
    const int st_dma = (st == 0) ? kGStages - 1 : st - 1;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kGKs; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kGKs) {
#pragma unroll
        for (int b = 0; b < 4; ++b) fa[cur ^ 1][b] = lds_b128(stg + b * 32 * kGRow + foff[ks + 1]);
#pragma unroll
        for (int b = 0; b < kNB; ++b) fb[cur ^ 1][b] = lds_b128(stg + bq + b * 32 * kGRow + foff[ks + 1]);
      }
      // the next sub-step's fragment reads go out before this sub-step's
      // MFMAs (left to itself the scheduler sinks them behind most of them)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bm = 0; bm < 4; ++bm)
#pragma unroll
        for (int bn = 0; bn < kNB; ++bn) {
          acc[bm][bn] = mfma32(fa[cur][bm], fb[cur][bn], acc[bm][bn]);
          // the next step's DMA, one instruction every kGDmaGap MFMAs: the
          // address unit takes about one 1 KB instruction per 16 clocks
          // per CU, so a burst would hold the MFMAs back
          const int slot = (ks * 4 + bm) * kNB + bn;
          if (slot % kGDmaGap == 0 && slot / kGDmaGap < kGDmaPerWave) dma(kn, st_dma, slot / kGDmaGap);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // step kt+1 has landed (later steps may still be in flight); every wave
    // is done with stage kt before it is refilled
    wait_vm<(kGStages - 2) * kGDmaPerWave>();
    __syncthreads();
    st = (st == kGStages - 1) ? 0 : st + 1;
  }
  wait_vm<0>();
  __syncthreads();   // the ring is free

  lm_epilogue<kWN>(acc, smem, p, wid, lane, m0, v0, M);
}

// ---- LM head over the tiled weight ----------------------------------------------
// The tiled weight (rv_lm_tile_weight) stores W in MFMA fragment order:
// 32-column blocks, each a run of H/16 fragments of 1 KB, where lane l of
// fragment f of block cb holds W[32*cb + l%32][16*f + 8*(l/32) .. +7] (rows
// past V are zero).  One wave's B operand for one 32x32x16 MFMA is then a
// single fully coalesced 1 KB load straight into registers.  No other wave
// reads those weights, so they skip LDS altogether: LDS carries only the
// hidden rows, which all four waves share (16 KB of DMA-free staging and
// 64 KB of fragment reads per 64-wide K step, against 2x64 KB more for
// weights staged through LDS).
constexpr int kBufFlags = 0x00020000;   // buffer resource word 3 (gfx9 family: 32-bit data format)
constexpr int kTRing = 8;             // weight sub-steps (16-wide K) held in registers
constexpr int kTDist = kTRing - 1;    // sub-steps between a weight load and its MFMAs

template <int WN>
struct TiledCfg {
  static constexpr int kNB = WN / 32;                 // 32-column blocks per wave
  static constexpr int kBN = 4 * WN;                  // workgroup columns
  static constexpr int kStage = kBM * kGRow;          // 16 KB of hidden rows per K step
  static constexpr int kEpi = 4 * 32 * (WN + 4) * 4;  // epilogue transpose area
  static constexpr int kLds = 4 * kStage > kEpi ? 4 * kStage : kEpi;   // four-stage ring
};

__device__ inline void lds_w128(uint32_t addr, const u32x4_t& v) { *(lds_u32x4_t*)(size_t)addr = v; }

// BMB: 32-row blocks of the tile that hold packed rows (1, 2 or 4); the
// MFMAs, fragment reads and epilogue of the blocks past them are skipped
template <int WN, int BMB>
__device__ __forceinline__ void lm_tiled_body(const GemmParams& p, unsigned char* smem, int m0, int v0, int M) {
  using Cfg = TiledCfg<WN>;
  constexpr int kNB = Cfg::kNB;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const uint32_t lds = (uint32_t)(uintptr_t)smem;
  const int nk = p.H / kBK;      // even (H % 128 == 0)
  const int nsub = p.H / 16;     // fragments per column block

  // hidden rows: wave w stages rows 32w .. 32w+31 of every K step, four
  // 16-byte chunks per lane, eight lanes per 128-byte row (whole lines);
  // rows past the packed total read the last real row.  Buffer loads: the
  // tile's rows as one resource, the K step as the scalar offset.
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(p.x) + (size_t)m0 * p.H, 0, kBM * p.H * 2, kBufFlags);
  uint32_t aoff[4], adst[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int rl = 32 * wid + 8 * e + (lane >> 3);
    const int c = lane & 7;
    aoff[e] = (uint32_t)(min(rl, M - 1 - m0) * p.H * 2 + c * 16);
    adst[e] = (uint32_t)(rl * kGRow + ((c ^ gswz(rl)) * 16));
  }
  auto load_a = [&](u32x4_t (&ar)[4], int kt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) ar[e] = __builtin_amdgcn_raw_buffer_load_b128(xr, aoff[e], kt * kGRow, 0);
  };

  // weights: this wave's kNB column blocks as one buffer resource ending at
  // the tiled weight's end, so blocks past it read as zeros (their columns
  // are masked in the epilogue); the sub-step is the scalar offset
  const size_t wbase = (size_t)((v0 + wid * WN) / 32) * nsub * 1024;
  const size_t wspan = (size_t)kNB * nsub * 1024;
  const size_t wleft = p.w_bytes > wbase ? p.w_bytes - wbase : 0;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<unsigned char*>(const_cast<bf16_t*>(p.w)) + (wleft ? wbase : 0), 0,
      (int)(wleft < wspan ? wleft : wspan), kBufFlags);
  uint32_t woff[kNB];
#pragma unroll
  for (int bn = 0; bn < kNB; ++bn) woff[bn] = (uint32_t)(bn * nsub * 1024 + lane * 16);
  auto load_w = [&](u32x4_t (&dst)[kNB], int sub) {
#pragma unroll
    for (int bn = 0; bn < kNB; ++bn) dst[bn] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[bn], sub * 1024, 0);
  };

  // fragment reads of the hidden rows: row 32*b + l32, logical chunk 2*ks + lh
  uint32_t foff[kGKs];
#pragma unroll
  for (int ks = 0; ks < kGKs; ++ks) foff[ks] = (uint32_t)(l32 * kGRow + (((2 * ks + lh) ^ gswz(l32)) * 16));

  f32x16_t acc[BMB][kNB];
#pragma unroll
  for (int a = 0; a < BMB; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  // register ring of weight fragments: sub-step s sits in slot s % kTRing
  // and is loaded kTDist sub-steps before its MFMAs (past the end: the last
  // sub-step again).  Hidden rows: a four-stage LDS ring, step k in stage
  // k % 4, written during step k-2 from registers ar[k % 2] that were loaded
  // during step k-4; so one barrier per two steps suffices (it separates the
  // reads of stage k % 4 during steps k and k+1 from its refill during step
  // k+2, and that refill from its reads), and waiting for hidden rows never
  // waits for weights loaded less than seven sub-steps ahead.  The prologue
  // issues its loads in the order the loop does (scheduling barriers keep
  // it), so that the compiler's load counting sees the same queue on entry as
  // around the loop.
  u32x4_t br[kTRing][kNB];
  u32x4_t ar[2][4], ar0[4], ar1[4];
  load_a(ar0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_a(ar1, min(1, nk - 1));
  __builtin_amdgcn_sched_barrier(0);
  load_w(br[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  load_a(ar[0], min(2, nk - 1));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 1; j < 5; ++j) {
    load_w(br[j], min(j, nsub - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  load_a(ar[1], min(3, nk - 1));
  __builtin_amdgcn_sched_barrier(0);
  load_w(br[5], min(5, nsub - 1));
  __builtin_amdgcn_sched_barrier(0);
  load_w(br[6], min(6, nsub - 1));
  __builtin_amdgcn_sched_barrier(0);
  // hidden rows of steps 0 and 1 into stages 0 and 1
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lds_w128(lds + adst[e], ar0[e]);
    lds_w128(lds + Cfg::kStage + adst[e], ar1[e]);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; kt += 2) {
    const uint32_t half = (uint32_t)(kt & 2) * Cfg::kStage;   // stages of steps kt, kt+1
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = kt + u;
      const uint32_t stg = lds + half + u * Cfg::kStage;                   // stage k % 4
      const uint32_t nxt = lds + (half ^ (2 * Cfg::kStage)) + u * Cfg::kStage;   // stage (k+2) % 4
      u32x4_t fa[2][BMB];
#pragma unroll
      for (int b = 0; b < BMB; ++b) fa[0][b] = lds_b128(stg + b * 32 * kGRow + foff[0]);
#pragma unroll
      for (int ks = 0; ks < kGKs; ++ks) {
        const int j = 4 * u + ks;                      // ring slot of this sub-step
        const int jn = (j + kTDist) % kTRing;          // slot of the sub-step kTDist ahead
        load_w(br[jn], min(4 * k + ks + kTDist, nsub - 1));
        if (ks == 1) {
          // step k+2's hidden rows (ar[u]) into stage (k+2) % 4, then step
          // k+4 into the same registers
#pragma unroll
          for (int e = 0; e < 4; ++e) lds_w128(nxt + adst[e], ar[u][e]);
          load_a(ar[u], min(k + 4, nk - 1));
        }
        if (ks + 1 < kGKs) {
#pragma unroll
          for (int b = 0; b < BMB; ++b) fa[(ks + 1) & 1][b] = lds_b128(stg + b * 32 * kGRow + foff[ks + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
          for (int bn = 0; bn < kNB; ++bn) acc[bm][bn] = mfma32(fa[ks & 1][bm], br[j][bn], acc[bm][bn]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // steps kt+2 and kt+3 are in LDS; every wave is done with the stages of
    // steps kt and kt+1
    __syncthreads();
  }

  lm_epilogue<WN, BMB>(acc, smem, p, wid, lane, m0, v0, M);
}

template <int WN>
__global__ __launch_bounds__(kGemmThreads) void k_lm_gemm_tiled(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // XCD-aware tile order as in k_lm_gemm: the row tiles of one vocabulary
  // tile run on one XCD at about the same time, so its weights come from HBM
  // once and from that XCD's L2 for the other row tiles
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
  const int v0 = vt * TiledCfg<WN>::kBN;
  // The last row tile of a ragged batch is mostly padding: MFMAs only for
  // its 32-row blocks that hold packed rows.  Except when every live tile
  // runs at once (one round on the CUs) and a vocabulary tile has several
  // row tiles: then the short tile would run ahead of its partners, fetch the
  // weights from HBM on its own, and gain nothing, as the full tiles set the
  // time (GQA shapes, 148 rows x 32000: 86 -> 96 us with accept; 48 rows,
  // one row tile: 74 -> 63 us; 278 rows, a round and a half: 122 -> 116 us).
  const int live_mt = (M + kBM - 1) / kBM;
  const bool lockstep = live_mt > 1 && live_mt * p.n_vt <= p.cus;
  const int rows = lockstep ? kBM : M - m0;
  if (rows > 64) lm_tiled_body<WN, 4>(p, smem, m0, v0, M);
  else if (rows > 32) lm_tiled_body<WN, 2>(p, smem, m0, v0, M);
  else lm_tiled_body<WN, 1>(p, smem, m0, v0, M);
}

// ---- LM head with every packed row in one tile (at most 256 rows) -------------------
// With 128-row tiles a batch of 129..256 rows has two row tiles per
// vocabulary tile: both stream the same weights (shared through L2 only
// while they keep pace) and the second is mostly padding.  Here one
// workgroup takes all rows (up to 224) against 128 vocabulary columns: each
// wave owns one 32-column block and all 32-row blocks that hold packed rows
// (BMB), so every weight byte is loaded by one wave only, once, and a
// weight fragment feeds BMB MFMAs.  The hidden rows reach LDS by DMA (no
// registers) three K steps ahead into a four-stage ring; the weights come
// straight into a 16-deep register ring, loaded fifteen sub-steps ahead (a
// wait for a hidden-row DMA three steps old never waits for weights needed
// later than the next step; the compiler's own waits before the MFMAs count
// only the weight loads, so they also wait for the DMAs issued since, which
// shortens the weights' lead when BMB is large).  The epilogue writes the
// fp32 tile to LDS and reduces each (row, 64-column slab) in column order,
// as the other kernels do.
constexpr int kRRing = 16, kRDist = 15, kRAhead = 3;
constexpr int kRMaxRows = 256;
constexpr int kRBN = 128;                             // columns per workgroup
constexpr int kRStage = kRMaxRows * kGRow;            // 32 KB of hidden rows per K step
constexpr int kRERow = kRBN + 4;                      // floats per padded epilogue row
constexpr int kREpi = kRMaxRows * kRERow * 4;         // the fp32 tile of all rows
constexpr int kRLds = 4 * kRStage > kREpi ? 4 * kRStage : kREpi;

template <int BMB>
__device__ __forceinline__ void lm_rows_body(const GemmParams& p, unsigned char* smem, int v0, int M) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  const uint32_t lds = (uint32_t)(uintptr_t)smem;
  const int nk = p.H / kBK;      // a multiple of 4 (H % 256 == 0)
  const int nsub = p.H / 16;

  // hidden rows: DMA instruction e of wave w moves chunks (BMB*w + e)*64 +
  // lane of the step (BMB*32 rows of eight 16-byte chunks); chunk c goes to
  // row c/8 at physical position c%8 and holds logical chunk (c%8) ^
  // gswz(row); rows past the packed total read the last real row
  const unsigned char* xa = reinterpret_cast<const unsigned char*>(p.x);
  uint32_t doff[BMB];
#pragma unroll
  for (int e = 0; e < BMB; ++e) {
    const int c = (wid * BMB + e) * 64 + lane;
    const int row = c / kGChunks;
    const int lc = (c % kGChunks) ^ gswz(row);
    doff[e] = (uint32_t)min(row, M - 1) * (uint32_t)(p.H * 2) + (uint32_t)lc * 16u;
  }
  auto dma_a = [&](int kt) {   // K step kt into stage kt % 4
    const void* base = uniform_ptr(xa + (size_t)min(kt, nk - 1) * kGRow);
    const uint32_t dst = lds + (uint32_t)((kt & 3) * kRStage);
#pragma unroll
    for (int e = 0; e < BMB; ++e)
      dma16_s(doff[e], base, __builtin_amdgcn_readfirstlane(dst + (wid * BMB + e) * 1024));
  };

  // weights: this wave's column block as one buffer resource ending at the
  // tiled weight's end (a block past it reads as zeros, masked below)
  const size_t wbase = (size_t)((v0 + wid * 32) / 32) * nsub * 1024;
  const size_t wspan = (size_t)nsub * 1024;
  const size_t wleft = p.w_bytes > wbase ? p.w_bytes - wbase : 0;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<unsigned char*>(const_cast<bf16_t*>(p.w)) + (wleft ? wbase : 0), 0,
      (int)(wleft < wspan ? wleft : wspan), kBufFlags);
  const uint32_t woff = (uint32_t)(lane * 16);
  auto load_w = [&](u32x4_t& dst, int sub) { dst = __builtin_amdgcn_raw_buffer_load_b128(wr, woff, sub * 1024, 0); };

  uint32_t foff[kGKs];
#pragma unroll
  for (int ks = 0; ks < kGKs; ++ks) foff[ks] = (uint32_t)(l32 * kGRow + (((2 * ks + lh) ^ gswz(l32)) * 16));

  f32x16_t acc[BMB];
#pragma unroll
  for (int a = 0; a < BMB; ++a)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[a][j] = 0.f;

  // prologue in the loop's order (the compiler's load counting then sees
  // the same queue at the loop head as inside it)
  u32x4_t br[kRRing];
#pragma unroll
  for (int k = 0; k < kRAhead; ++k) dma_a(k);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kRDist; ++j) {
    load_w(br[j], min(j, nsub - 1));
    __builtin_amdgcn_sched_barrier(0);
  }
  // step 0 landed: the DMAs of steps 1 and 2 and the fifteen weight loads
  // may still be in flight
  wait_vm<(kRAhead - 1) * BMB + kRDist>();
  __syncthreads();

  for (int kt = 0; kt < nk; kt += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = kt + u;
      const uint32_t stg = lds + (uint32_t)(u * kRStage);   // stage k % 4 (kt % 4 == 0)
      // step k+3 into stage (k+3) % 4, last read during step k-1, before the
      // last barrier (past the end: the last step again, never read)
      dma_a(k + kRAhead);
      u32x4_t fa[2][BMB];
#pragma unroll
      for (int b = 0; b < BMB; ++b) fa[0][b] = lds_b128(stg + b * 32 * kGRow + foff[0]);
#pragma unroll
      for (int ks = 0; ks < kGKs; ++ks) {
        const int j = 4 * u + ks;   // ring slot of sub-step 4k + ks
        load_w(br[(j + kRDist) % kRRing], min(4 * k + ks + kRDist, nsub - 1));
        if (ks + 1 < kGKs) {
#pragma unroll
          for (int b = 0; b < BMB; ++b) fa[(ks + 1) & 1][b] = lds_b128(stg + b * 32 * kGRow + foff[ks + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int bm = 0; bm < BMB; ++bm) acc[bm] = mfma32(fa[ks & 1][bm], br[j], acc[bm]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // step k+1's DMA (issued at the start of step k-2) has landed: after
      // it this wave issued four weight loads in each of steps k-2 .. k and
      // the DMAs of steps k+2 and k+3
      wait_vm<(kRAhead - 1) * BMB + kRAhead * kGKs>();
      __syncthreads();
    }
  }
  wait_vm<0>();
  __syncthreads();   // the ring is free for the epilogue

  // epilogue: the fp32 tile [rows][128] into LDS, then one thread per
  // (row, 64-column slab): max, lowest argmax, sum of exp(z - max)
  float* et = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int bm = 0; bm < BMB; ++bm)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      et[(bm * 32 + (j / 4) * 8 + lh * 4 + (j % 4)) * kRERow + wid * 32 + l32] = acc[bm][j];
  __syncthreads();
  const int rows = min(M, BMB * 32);
  // four lanes per (row, slab), 16 columns each read as float4 runs; the
  // lanes' (max, lowest argmax, sum of exp) merge through two lane swaps
  // (one lane scanning 64 columns one float at a time took 8 us of the
  // 156-row batch's 60)
  constexpr int kQ = kSlab / 16;
  const int n_items = rows * (kRBN / kSlab);
  for (int q0 = 0; q0 < n_items * kQ; q0 += kGemmThreads) {   // uniform trip count
    const int qq = q0 + tid;
    const int q = qq / kQ, part = qq % kQ;
    const bool live = q < n_items;
    const int row = live ? q / (kRBN / kSlab) : 0, sl = live ? q % (kRBN / kSlab) : 0;
    const int cslab = v0 + sl * kSlab;
    const int c0 = cslab + part * 16;
    const float* src = et + row * kRERow + sl * kSlab + part * 16;
    float z[16];
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      const float4 v = *reinterpret_cast<const float4*>(src + i);
      z[i] = v.x; z[i + 1] = v.y; z[i + 2] = v.z; z[i + 3] = v.w;
    }
    float best = -INFINITY;
    int bi = c0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (c0 + i >= p.V) z[i] = -INFINITY;
      if (z[i] > best) { best = z[i]; bi = c0 + i; }   // strict: lowest index wins ties
    }
    float se = 0.f;
    if (p.with_sum && best != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) se += (z[i] == -INFINITY) ? 0.f : __expf(z[i] - best);
    }
#pragma unroll
    for (int off = 1; off < kQ; off <<= 1) {
      const float ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bi, off);
      const float os = __shfl_xor(se, off);
      const float m = fmaxf(best, ob);
      if (p.with_sum && m != -INFINITY)
        se = (best == -INFINITY ? 0.f : se * __expf(best - m)) + (ob == -INFINITY ? 0.f : os * __expf(ob - m));
      merge_best(best, bi, ob, oi);
    }
    if (live && part == 0 && cslab < p.V)
      p.part[(size_t)row * p.n_slabs + cslab / kSlab] = make_float4(best, __int_as_float(bi), se, 0.f);
  }
  if (p.logits) {
    // row-contiguous float4 runs: 32 lanes per row, eight rows per pass
    const bool vec_logits = (p.V % 4) == 0 && ((uintptr_t)p.logits % 16) == 0;
    const int c4 = (tid & 31) * 4;
    const int gcol = v0 + c4;
    for (int r = tid >> 5; r < rows; r += kGemmThreads / 32) {
      const float4 v = *reinterpret_cast<const float4*>(et + r * kRERow + c4);
      float* dst = p.logits + (size_t)r * p.V + gcol;
      if (vec_logits && gcol + 3 < p.V) {
        *reinterpret_cast<float4*>(dst) = v;
      } else {
        const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (gcol + c < p.V) dst[c] = e4[c];
      }
    }
  }
}

// Past seven 32-row blocks the fragment reads (every wave reads every
// block) outweigh what the single tile saves: 256 rows took 96 us here
// against 89 us for two 128-row tiles in lockstep (GQA shapes, with accept),
// 148 rows 63 against 79 us.  So the packed count, known only on the device,
// picks the layout: the grid covers both (2 * ceil(V/256) >= ceil(V/128)).
constexpr int kRTiledAbove = 224;

__global__ __launch_bounds__(kGemmThreads) void k_lm_gemm_rows(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  // at most kRMaxRows rows (the launcher's B*gamma bound); the clamp only
  // keeps a corrupt count inside the LDS tile
  const int M = min(p.mm[0], kRMaxRows);
  if (M <= 0) return;
  if (M > kRTiledAbove) {
    // two 128-row tiles per 256 columns, XCD-aware as in k_lm_gemm_tiled;
    // both hold more than 96 rows, so all four blocks of each are computed
    const int n_vt = (p.V + TiledCfg<64>::kBN - 1) / TiledCfg<64>::kBN;
    const int n_tiles = 2 * n_vt;
    const int per_xcd = (n_tiles + 7) / 8;
    const int kloc = blockIdx.x / 8;
    const int logical = (blockIdx.x % 8) * per_xcd + kloc;
    if (kloc >= per_xcd || logical >= n_tiles) return;
    lm_tiled_body<64, 4>(p, smem, (logical % 2) * kBM, (logical / 2) * TiledCfg<64>::kBN, M);
    return;
  }
  const int vt = blockIdx.x;
  if (vt >= p.n_vt) return;
  const int v0 = vt * kRBN;
  switch ((M + 31) / 32) {
    case 1: lm_rows_body<1>(p, smem, v0, M); break;
    case 2: lm_rows_body<2>(p, smem, v0, M); break;
    case 3: lm_rows_body<3>(p, smem, v0, M); break;
    case 4: lm_rows_body<4>(p, smem, v0, M); break;
    case 5: lm_rows_body<5>(p, smem, v0, M); break;
    case 6: lm_rows_body<6>(p, smem, v0, M); break;
    default: lm_rows_body<7>(p, smem, v0, M); break;
  }
}

// ---- LM head for at most 32 rows over the tiled weight ---------------------------
// With so few rows the MFMAs are cheap and the stage streams the weight: its
// speed is the weight bytes in flight.  One wave per workgroup owns a
// 32-row x 64-column tile (the 128-row tiles would multiply mostly padding,
// and four waves per workgroup would halve the workgroups); both operands
// come straight from memory into a 16-deep register ring (hidden-row
// fragments are 16 bytes per lane, L2-resident), so every wait is for loads
// issued fifteen sub-steps earlier.  Two waves fit per SIMD.
constexpr int kSmallRing = 16;

__global__ __launch_bounds__(64) void k_lm_gemm_small(GemmParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kNB = 2, kRows = 32, kCols = 64;
  constexpr int kRing = kSmallRing, kDist = kSmallRing - 1;
  const int n_tiles = p.n_mt * p.n_vt;
  const int per_xcd = (n_tiles + 7) / 8;
  const int kloc = blockIdx.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + kloc;
  if (kloc >= per_xcd || logical >= n_tiles) return;
  const int vt = logical / p.n_mt;
  const int mt = logical % p.n_mt;
  const int M = p.mm[0];
  const int m0 = mt * kRows;
  if (m0 >= M) return;
  const int v0 = vt * kCols;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, lh = lane >> 5;
  const int nsub = p.H / 16;   // a multiple of kRing (H % 256 == 0)

  // hidden rows: lane l reads row m0 + l%32 (rows past M: the last real
  // row), 8 bf16 at K = 16*s + 8*(l/32) for sub-step s
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(p.x) + (size_t)m0 * p.H, 0, kRows * p.H * 2, kBufFlags);
  const uint32_t aoff = (uint32_t)(min(l32, M - 1 - m0) * p.H * 2 + lh * 16);
  // weights: the tile's two column blocks, ending at the tiled weight's end
  const size_t wbase = (size_t)(v0 / 32) * nsub * 1024;
  const size_t wspan = (size_t)kNB * nsub * 1024;
  const size_t wleft = p.w_bytes > wbase ? p.w_bytes - wbase : 0;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<unsigned char*>(const_cast<bf16_t*>(p.w)) + (wleft ? wbase : 0), 0,
      (int)(wleft < wspan ? wleft : wspan), kBufFlags);
  const uint32_t woff0 = (uint32_t)(lane * 16), woff1 = (uint32_t)(nsub * 1024 + lane * 16);

  u32x4_t ra[kRing], rb[kRing][kNB];
  auto load = [&](int slot, int sub) {
    ra[slot] = __builtin_amdgcn_raw_buffer_load_b128(xr, aoff, sub * 32, 0);
    rb[slot][0] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff0, sub * 1024, 0);
    rb[slot][1] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff1, sub * 1024, 0);
  };
  f32x16_t acc[1][kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[0][b][j] = 0.f;
#pragma unroll
  for (int j = 0; j < kDist; ++j) {
    load(j, j);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int s0 = 0; s0 < nsub; s0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      load((j + kDist) % kRing, min(s0 + j + kDist, nsub - 1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int bn = 0; bn < kNB; ++bn) acc[0][bn] = mfma32(ra[j], rb[j][bn], acc[0][bn]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lm_epilogue<kCols, 1>(acc, smem, p, 0, lane, m0, v0, M);
}

// W [V][H] -> tiled copy: one thread per (fragment, lane), 16 bytes each
__global__ __launch_bounds__(256) void k_lm_tile_weight(const bf16_t* __restrict__ w, u32x4_t* __restrict__ out,
                                                        int V, int H, long long n_chunks) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int lane = (int)(i & 63);
  const long long frag = i >> 6;
  const int nsub = H / 16;
  const int cb = (int)(frag / nsub);
  const int f = (int)(frag % nsub);
  const int row = cb * 32 + (lane & 31);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < V) v = *reinterpret_cast<const u32x4_t*>(w + (size_t)row * H + f * 16 + 8 * (lane >> 5));
  out[i] = v;
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

constexpr int kAccThreads = 512;   // eight waves: one per row of a gamma-8 window
constexpr int kAccDepth = 16;     // slab partials per lane in flight while merging
constexpr int kAccSeg = 4096;      // tokens per vocabulary segment of the bonus draw
constexpr int kAccMaxSeg = kMaxVocabRejection / kAccSeg;

__global__ __launch_bounds__(kAccThreads) void k_accept(AcceptParams p) {
  __shared__ int s_pred[RV_MAX_GAMMA];
  __shared__ float s_lse[RV_MAX_GAMMA];
  __shared__ int s_flag[RV_MAX_GAMMA];
  __shared__ int s_sel;
  __shared__ float s_w[kAccSeg + kAccSeg / 64];   // the selected segment's token weights
  __shared__ int s_row, s_qrow, s_c, s_a, s_bonus;
  __shared__ double s_seg[kAccMaxSeg], s_total;
  __shared__ int s_seg_last[kAccMaxSeg];
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

  // merge slab partials, one wave per row (rows in parallel, no workgroup
  // barrier per row): argmax (lowest index on ties, an exact merge whose
  // result does not depend on the order) and, for the rejection rule,
  // log-sum-exp in fp64
  const int lane = tid & 63, wv_id = tid >> 6;
  for (int k = wv_id; k < wv; k += kAccThreads / 64) {
    const float4* pr = p.part + (size_t)(base + k) * p.n_slabs;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    // kAccDepth loads per lane in flight, then their merges
    for (int s0 = lane; s0 < p.n_slabs; s0 += 64 * kAccDepth) {
      float4 q[kAccDepth];
#pragma unroll
      for (int u = 0; u < kAccDepth; ++u) {
        const int s = s0 + 64 * u;
        q[u] = s < p.n_slabs ? pr[s] : make_float4(-INFINITY, __int_as_float(0x7fffffff), 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kAccDepth; ++u) merge_best(best, bi, q[u].x, __float_as_int(q[u].y));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bi, off);
      merge_best(best, bi, ob, oi);
    }
    if (lane == 0) {
      s_pred[k] = bi;
      p.pred[base + k] = bi;
    }
    if (p.rule == RV_REJECTION) {
      double acc = 0.0;
      for (int s0 = lane; s0 < p.n_slabs; s0 += 64 * kAccDepth) {
        float4 q[kAccDepth];
#pragma unroll
        for (int u = 0; u < kAccDepth; ++u) {
          const int s = s0 + 64 * u;
          q[u] = s < p.n_slabs ? pr[s] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < kAccDepth; ++u)
          if (s0 + 64 * u < p.n_slabs) acc += (double)q[u].z * exp((double)q[u].x - (double)best);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
      if (lane == 0) s_lse[k] = best + (float)log(acc);
    }
  }
  __syncthreads();

  // Every draft's test at once (lane t: draft t against row t), then the scan
  // for the first failure: 2 = invalid token, 1 = kept, 0 = stop.
  if (tid < wv - 1) {
    const int t = tid;
    const int d = p.drafts[(size_t)i * g1 + t];
    int f = 2;
    if (d >= 0 && d < p.V) {
      if (p.rule == RV_GREEDY) {
        f = d == s_pred[t] ? 1 : 0;
      } else {
        const float zd = p.logits[(size_t)(base + t) * p.V + d];
        const float pd = expf(zd - s_lse[t]);
        const float qd = p.q_rows[((size_t)i * g1 + t) * p.V + d];
        f = p.u[(size_t)i * g1 + t] * qd < pd ? 1 : 0;
      }
    }
    s_flag[t] = f;
  }
  __syncthreads();
  auto scan = [&]() {
    int c = 0;
    while (c < wv - 1) {
      if (s_flag[c] == 2) { set_status(p.status, RV_DEV_BAD_TOKEN); break; }
      if (s_flag[c] == 0) break;
      ++c;
    }
    return c;
  };

  if (p.rule == RV_GREEDY) {
    if (tid == 0) {
      const int c = scan();
      const int a = min(c, wc - 1);
      p.ceiling[i] = c;
      p.accept[i] = a;
      p.bonus[i] = s_pred[a];
    }
    return;
  }

  // ---- rejection sampling -------------------------------------------------------
  if (tid == 0) {
    const int c = scan();
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
  // The vocabulary in segments of kAccSeg consecutive tokens; wave w sums
  // segments w, w+8, ... with lane l reading the float4 runs l, l+64, ...
  // of the segment (coalesced 1 KB loads, all in flight together).
  const int n_seg = (p.V + kAccSeg - 1) / kAccSeg;
  // float4 runs when every row starts 16-byte aligned
  const bool vec4 = (p.V % 4) == 0 && ((uintptr_t)p.logits % 16) == 0 && ((uintptr_t)p.q_rows % 16) == 0;
  for (int sg = wv_id; sg < n_seg; sg += kAccThreads / 64) {
    double acc = 0.0;
    int lastp = -1;
    const int s0 = sg * kAccSeg;
    if (vec4 && s0 + kAccSeg <= p.V) {
      float4 zv[kAccSeg / 256], qv[kAccSeg / 256];
#pragma unroll
      for (int u = 0; u < kAccSeg / 256; ++u) {
        zv[u] = *reinterpret_cast<const float4*>(z + s0 + 4 * (lane + 64 * u));
        if (qd) qv[u] = *reinterpret_cast<const float4*>(qd + s0 + 4 * (lane + 64 * u));
      }
#pragma unroll
      for (int u = 0; u < kAccSeg / 256; ++u) {
        const float zz[4] = {zv[u].x, zv[u].y, zv[u].z, zv[u].w};
        const float qq[4] = {qd ? qv[u].x : 0.f, qd ? qv[u].y : 0.f, qd ? qv[u].z : 0.f, qd ? qv[u].w : 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float pv = expf(zz[c] - lse);
          const float r = qd ? fmaxf(0.f, pv - qq[c]) : pv;
          acc += (double)r;
          if (r > 0.f) lastp = s0 + 4 * (lane + 64 * u) + c;
        }
      }
    } else {
      for (int v = s0 + lane; v < min(s0 + kAccSeg, p.V); v += 64) {
        const float r = weight(v);
        acc += (double)r;
        if (r > 0.f) lastp = v;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      acc += __shfl_xor(acc, off);
      lastp = max(lastp, __shfl_xor(lastp, off));
    }
    if (lane == 0) {
      s_seg[sg] = acc;
      s_seg_last[sg] = lastp;
    }
  }
  __syncthreads();
  // inclusive scan of the segment sums by wave 0 (each lane a run of
  // consecutive segments), and the last token of positive weight
  if (wv_id == 0) {
    const int per = (n_seg + 63) / 64;
    const int k0 = lane * per, k1 = min(k0 + per, n_seg);
    double run = 0.0;
    int lastp = -1;
    for (int k = k0; k < k1; ++k) {
      run += s_seg[k];
      lastp = max(lastp, s_seg_last[k]);
    }
    double incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) lastp = max(lastp, __shfl_xor(lastp, off));
    const double up = __shfl_up(incl, 1);
    double pre = lane > 0 ? up : 0.0;   // exclusive prefix: the previous lane's inclusive
    for (int k = k0; k < k1; ++k) {
      pre += s_seg[k];
      s_seg[k] = pre;   // inclusive prefix through segment k
    }
    if (lane == 63) s_total = incl;
    if (lane == 0) s_bonus = lastp;   // target at or past the end: last positive token
  }
  __syncthreads();
  const double total = s_total;
  const double target = (double)p.u_bonus[i] * total;
  // the segment whose interval [excl, incl) holds the target; its token
  // weights are staged in LDS by the whole workgroup (one coalesced pass),
  // then lane l of wave 0 sums its 64-token block of them, a wave scan finds
  // the block that crosses the target, and that block's lane walks it token
  // by token
  if (wv_id == 0) {
    int sel = -1;
    for (int k = lane; k < n_seg; k += 64) {
      const double excl = k > 0 ? s_seg[k - 1] : 0.0;
      if (excl <= target && target < s_seg[k] && s_seg[k] > excl) sel = k;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sel = max(sel, __shfl_xor(sel, off));
    if (lane == 0) s_sel = sel;
  }
  __syncthreads();
  const int sel = s_sel;
  const int sbase = sel * kAccSeg;
  // token t of the segment at t + t/64: the 64 lanes' blocks start in
  // different banks
  auto wslot = [](int t) { return t + (t >> 6); };
  if (sel >= 0) {
    for (int t = tid; t < kAccSeg; t += kAccThreads) s_w[wslot(t)] = sbase + t < p.V ? weight(sbase + t) : 0.f;
  }
  __syncthreads();
  if (wv_id == 0) {
    if (sel >= 0) {
      const double excl = sel > 0 ? s_seg[sel - 1] : 0.0;
      const int b0 = sbase + 64 * lane;
      const int b1 = min(b0 + 64, p.V);
      double bs = 0.0;
      for (int v = b0; v < b1; ++v) bs += (double)s_w[wslot(v - sbase)];
      double incl = bs;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const unsigned long long hit = __ballot(excl + incl > target && bs > 0.0);
      int pick = s_seg_last[sel];      // rounding left the walk short: the segment's last
      if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        if (lane == L) {
          double run = excl + incl - bs;
          int pk = -1;
          for (int v = b0; v < b1; ++v) {
            run += (double)s_w[wslot(v - sbase)];
            if (run > target) { pk = v; break; }
          }
          if (pk < 0) {                // rounding: this block's last positive token
            for (int v = b1 - 1; v >= b0; --v)
              if (s_w[wslot(v - sbase)] > 0.f) { pk = v; break; }
          }
          s_bonus = pk;
        }
      } else if (lane == 0) {
        s_bonus = pick;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    p.ceiling[i] = s_c;
    p.accept[i] = s_a;
    p.bonus[i] = s_bonus;
  }
}

}  // namespace

size_t lm_tiled_weight_bytes(int V, int H) { return (size_t)((V + 31) / 32) * 32 * (size_t)H * 2; }

hipError_t launch_lm_tile_weight(const void* W, void* W_tiled, int V, int H, hipStream_t s) {
  const long long n_chunks = (long long)((V + 31) / 32) * (H / 16) * 64;
  const long long grid = (n_chunks + 255) / 256;
  hipLaunchKernelGGL(k_lm_tile_weight, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16_t*>(W),
                     static_cast<u32x4_t*>(W_tiled), V, H, n_chunks);
  return hipGetLastError();
}

size_t lm_scratch_bytes(int B, int gamma, int V) {
  const size_t n_slabs = (size_t)(V + kSlab - 1) / kSlab;
  return align_up(sizeof(float4) * (size_t)B * gamma * n_slabs, 256);
}

hipError_t launch_lm(const rv_lm_args& a, void* part_mem, int32_t* status, hipStream_t s) {
  const int n_slabs = (a.V + kSlab - 1) / kSlab;
  float4* part = static_cast<float4*>(part_mem);
  const bool rej = (a.rule == RV_REJECTION);
  hipError_t e;
  if (a.dtype == RV_BF16 && a.w_layout == RV_W_TILED) {
    GemmParams g{};
    g.x = static_cast<const bf16_t*>(a.hidden);
    g.w = static_cast<const bf16_t*>(a.W);
    g.mm = a.mm;
    g.part = part;
    g.logits = a.logits;
    g.H = a.H;
    g.V = a.V;
    g.n_slabs = n_slabs;
    g.n_mt = (a.B * a.gamma + kBM - 1) / kBM;   // real rows never exceed one full block each
    g.with_sum = rej ? 1 : 0;
    g.ncb = (a.V + 31) / 32;
    g.w_bytes = lm_tiled_weight_bytes(a.V, a.H);
    // 128 x 512 tiles; 128 x 256 tiles when they need no more rounds of one
    // tile per CU (counted at the B*gamma row bound): small batches, whose
    // 512-wide grid leaves CUs idle (the 156-row GQA batch: 118 -> 87 us,
    // before the all-rows kernel took row bounds up to 256; the latent
    // batch's 815 rows: 1.73 ms with 256-wide tiles, 1.52 ms with 512-wide
    // ones)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    g.cus = cus;
    const int t512 = g.n_mt * ((a.V + 511) / 512), t256 = g.n_mt * ((a.V + 255) / 256);
    const bool narrow = (t256 + cus - 1) / cus <= (t512 + cus - 1) / cus;
    auto launch = [&](auto kern, int bn, int lds_bytes) -> hipError_t {
      g.n_vt = (a.V + bn - 1) / bn;
      const int grid = ((g.n_mt * g.n_vt + 7) / 8) * 8;
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
      if (err != hipSuccess) return err;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), lds_bytes, s, g);
      return hipSuccess;
    };
    if (a.B * a.gamma <= 32 && a.H % 256 == 0) {
      // one row tile's worth of rows: one-wave 32 x 64 tiles streaming the
      // weight (batch 1 of the GQA shapes, 8 rows x 4096 x 32000: 77 -> 60 us
      // with accept; with two row tiles the weight is streamed twice and
      // the 128 x 256 tiles win)
      g.n_mt = 1;
      g.n_vt = (a.V + 63) / 64;
      const int grid = ((g.n_mt * g.n_vt + 7) / 8) * 8;
      constexpr int kSmallLds = 32 * (64 + 4) * 4;   // the epilogue's transpose
      hipLaunchKernelGGL(k_lm_gemm_small, dim3(grid), dim3(64), kSmallLds, s, g);
      e = hipSuccess;
    } else if (a.B * a.gamma <= kRMaxRows && a.H % 256 == 0) {
      g.n_mt = 1;
      g.n_vt = (a.V + kRBN - 1) / kRBN;
      const int n_t = 2 * ((a.V + TiledCfg<64>::kBN - 1) / TiledCfg<64>::kBN);
      const int grid = ((g.n_vt > n_t ? g.n_vt : n_t) + 7) / 8 * 8;
      constexpr int kLds = kRLds > TiledCfg<64>::kLds ? kRLds : TiledCfg<64>::kLds;
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_lm_gemm_rows),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
      if (e == hipSuccess) hipLaunchKernelGGL(k_lm_gemm_rows, dim3(grid), dim3(kGemmThreads), kLds, s, g);
    } else {
      e = narrow ? launch(k_lm_gemm_tiled<64>, TiledCfg<64>::kBN, TiledCfg<64>::kLds)
                 : launch(k_lm_gemm_tiled<128>, TiledCfg<128>::kBN, TiledCfg<128>::kLds);
    }
    if (e != hipSuccess) return e;
  } else if (a.dtype == RV_BF16) {
    GemmParams g{};
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
    g.with_sum = rej ? 1 : 0;
    // 128 x 256 tiles with three 48 KB stages: measured at or below the
    // 128 x 512 double-buffered tiles on every workload but one (config 3,
    // +2%): latent batch 1.75 against 1.81 ms, config 2 95 against 154 us
    g.n_vt = (a.V + kGemmBN - 1) / kGemmBN;
    const int grid = ((g.n_mt * g.n_vt + 7) / 8) * 8;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_lm_gemm<kGemmBN>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, GemmCfg<kGemmBN>::kLds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_lm_gemm<kGemmBN>, dim3(grid), dim3(kGemmThreads), GemmCfg<kGemmBN>::kLds, s, g);
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
  ap.status = status;
  ap.B = a.B;
  ap.gamma = a.gamma;
  ap.V = a.V;
  ap.n_slabs = n_slabs;
  ap.rule = a.rule;
  hipLaunchKernelGGL(k_accept, dim3(a.B + 1), dim3(kAccThreads), 0, s, ap);
  return hipGetLastError();
}

}  // namespace rv
