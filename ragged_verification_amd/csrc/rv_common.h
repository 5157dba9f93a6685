// Internal helpers shared by the librv kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rv.h"

namespace rv {

constexpr int kStatusBytes = 256;        // status word + padding at workspace start
constexpr int kTargetItemsLatent = 1024; // latent attention: work items aimed for per launch
constexpr int kTargetItemsLatentRow = 512;  // latent row kernel (128-head tiles)
constexpr int kTargetItemsGqa = 512;     // GQA attention: about two items per persistent workgroup
constexpr size_t kPartBytes = 128u << 20; // split-KV partial outputs held in workspace
constexpr int kPartSlotsMax = 8192;      // split-KV partial tiles at most
constexpr int kMaxVocabRejection = 1 << 22;  // vocabulary limit of the rejection rule
constexpr int kMinChunk = 256;           // smallest split-KV chunk (keys)

// ---- sticky device status: first error wins --------------------------------
__device__ inline void set_status(int32_t* status, int32_t code) {
  if (status) atomicCAS(status, 0, code);
}

// ---- bf16 <-> f32 ------------------------------------------------------------
typedef uint16_t bf16_t;

__device__ inline float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// round to nearest even; NaN kept quiet
__device__ inline bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<bf16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// ---- MFMA operand types (gfx950 bf16 MFMAs take 8 bf16 per lane) ------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// D(16x16, fp32) += A(16x32) * B(32x16).  Lane l: A row l%16, B column l%16,
// both holding k = 8*(l/16) .. 8*(l/16)+7; D column l%16, rows 4*(l/16)+j.
__device__ inline f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16) * B(16x32).  Lane l: A row l%32, B column l%32,
// both holding k = 8*(l/32) .. +7; D column l%32, rows 8*(j/4) + 4*(l/32) + j%4.
__device__ inline f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// 16-byte LDS read at a raw 32-bit LDS byte address (constant parts fold
// into the instruction's offset field)
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
__device__ inline u32x4_t lds_b128(uint32_t addr) { return *(const lds_u32x4_t*)(size_t)addr; }

// ---- direct global -> LDS loads ----------------------------------------------
// Issued from inline assembly so that the compiler does not wait for every
// outstanding load before each LDS read; callers track the vector-memory
// counter themselves with wait_vm (loads complete in issue order).
// DMA of 16 bytes per lane: global (64-bit address) -> LDS at m0 + 16*lane
__device__ inline void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr) : "memory", "m0");
}
// same with a wave-uniform 64-bit base and a per-lane 32-bit byte offset
__device__ inline void dma16_s(uint32_t off, const void* base, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_addr)
               : "memory", "m0");
}

__device__ inline const void* uniform_ptr(const void* x) {
  const uint64_t v = reinterpret_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding)
template <int N>
__device__ inline void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__host__ __device__ inline int32_t* status_ptr(void* ws) { return reinterpret_cast<int32_t*>(ws); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---- launchers (defined next to their kernels) -------------------------------
struct SchedLaunch;
hipError_t launch_schedule(const rv_schedule_args& a, hipStream_t s);
hipError_t launch_pack(const rv_pack_args& a, hipStream_t s);
hipError_t launch_attn(const rv_attn_args& a, hipStream_t s, bool planned = false);
// stage 2 and the plan of the stage-3 call described by `attn`, in one launch
hipError_t launch_pack_plan(const rv_pack_args& pack, const rv_attn_args& attn, hipStream_t s);
// part: the slab partials (lm_scratch_bytes), status: the sticky status word
hipError_t launch_lm(const rv_lm_args& a, void* part, int32_t* status, hipStream_t s);
// host checks of rv_lm_head_accept's arguments other than the workspace
rv_status lm_args_check(const rv_lm_args* a);
hipError_t launch_scatter(const rv_scatter_args& a, hipStream_t s);
hipError_t launch_calibration(const rv_calib_args& a, hipStream_t s);
hipError_t launch_estimate(const rv_estimate_args& a, hipStream_t s);
size_t estimator_state_bytes(int B, int gamma);
hipError_t launch_clear_status(void* ws, hipStream_t s);

// host-side sizing helpers shared by the API layer and the launchers
size_t attn_scratch_bytes(int B, int gamma, int Hq, int Hkv, int Dqk, int Dv, int dtype);
size_t lm_scratch_bytes(int B, int gamma, int V);
size_t lm_tiled_weight_bytes(int V, int H);
hipError_t launch_lm_tile_weight(const void* W, void* W_tiled, int V, int H, hipStream_t s);
bool attn_shape_supported(int Hq, int Hkv, int Dqk, int Dv, int dtype, bool latent);
int attn_max_pages_limit(int dtype, bool latent);

// ---- workgroup scans (one-workgroup metadata kernels) --------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

// Inclusive scan of N ints per lane within a wave.
template <int N>
__device__ inline void wave_incl_scan(int (&v)[N]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int u = __shfl_up(v[k], off);
      if (lane >= off) v[k] += u;
    }
  }
}

// Exclusive scan of N ints per thread (thread order) over a workgroup of
// kScanThreads threads: wave shuffles, then one pass over the wave totals
// (two barriers); tot gets the workgroup totals.  buf: kScanWaves * N ints
// of LDS.
template <int N>
__device__ inline void block_excl_scan(const int (&v)[N], int (&ex)[N], int (&tot)[N], int* buf) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc[N];
#pragma unroll
  for (int k = 0; k < N; ++k) inc[k] = v[k];
  wave_incl_scan<N>(inc);
  __syncthreads();   // buf is free
  if (lane == 63) {
#pragma unroll
    for (int k = 0; k < N; ++k) buf[wv * N + k] = inc[k];
  }
  __syncthreads();
  int before[N], all[N];
#pragma unroll
  for (int k = 0; k < N; ++k) before[k] = all[k] = 0;
#pragma unroll 1
  for (int u = 0; u < kScanWaves; ++u) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int x = buf[u * N + k];
      before[k] += u < wv ? x : 0;
      all[k] += x;
    }
  }
#pragma unroll
  for (int k = 0; k < N; ++k) {
    ex[k] = before[k] + inc[k] - v[k];
    tot[k] = all[k];
  }
}

}  // namespace rv
