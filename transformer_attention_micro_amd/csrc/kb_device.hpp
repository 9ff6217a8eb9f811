// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, MFMA wrappers, wave64 reductions and the launch-side
// interface each kernel file exports to the C ABI layer.
//
// The reductions are the "warp/block reductions, online softmax" helpers the
// kbench page ("Repository layout", device_softmax.cuh) puts beside its
// kernels, rebuilt for 64-lane wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kb {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// ---- MFMA -----------------------------------------------------------------
// 32x32 output tile, fp32 accumulate.  Operand layout (both A and B): lane l
// holds row/column (l % 32) and the contraction slots 8*(l/32) .. +7 (bf16)
// or slot l/32 (fp32).  Result: lane l holds column (l % 32) and the 16 rows
// 8*(v/4) + 4*(l/32) + v%4, v = 0..15.

__device__ __forceinline__ f32x16 mfma32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x2_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (M index) held in accumulator slot v by a lane in half h = lane / 32.
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// ---- cross-lane -------------------------------------------------------------
// Value of x in lane (l ^ 32), via the gfx950 half-swap permute.
__device__ __forceinline__ float xor32_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}
// Sum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int o = G / 2; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Block-wide max / sum for NW waves; `red` is NW floats of LDS.  Every
// thread of the block must call it; all get the result.
template <int NW>
__device__ __forceinline__ float block_max(float x, float *red) {
  x = wave_max(x);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}
template <int NW>
__device__ __forceinline__ float block_sum(float x, float *red) {
  x = wave_sum(x);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += red[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Four consecutive outputs at element `idx` of O (idx a multiple of 4): fp32,
// or rounded to bf16 (round to nearest even) when out_bf16.
__device__ __forceinline__ void store_out4(void *O, size_t idx, f32x4 v, int out_bf16) {
  if (out_bf16)
    *(bf16x4 *)((bf16_t *)O + idx) = bf16x4{(bf16_t)v[0], (bf16_t)v[1], (bf16_t)v[2], (bf16_t)v[3]};
  else
    *(f32x4 *)((float *)O + idx) = v;
}
__device__ __forceinline__ void store_out1(void *O, size_t idx, float v, int out_bf16) {
  if (out_bf16)
    ((bf16_t *)O)[idx] = (bf16_t)v;
  else
    ((float *)O)[idx] = v;
}

// bf16 pattern -> fp32 value (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace kb

// ---- launch-side interface (host code) --------------------------------------
// Problem description the C ABI layer hands to the kernel files after
// validation.  Sizes are already checked; pointers are device pointers.
struct kb_problem {
  int bh, S, D;
  int causal;
  int bf16;  // 1: Q/K/V are bf16 patterns, 0: fp32
  float scale;
  const void *Q, *K, *V;
  void *O;      // fp32, or bf16 patterns when out_bf16
  int out_bf16;
  float *work;  // naive only
  hipStream_t stream;
};

hipError_t kb_launch_flash(const kb_problem &p);
hipError_t kb_launch_naive(const kb_problem &p);
hipError_t kb_launch_fused(const kb_problem &p);
// LDS bytes the fused kernel needs for this problem.
size_t kb_fused_lds_bytes(const kb_problem &p);
hipError_t kb_launch_triad(float *a, const float *b, const float *c, float s, size_t n, int block,
                           hipStream_t stream);
// Copy (kind 1), read-only (2) and write-only (3) bandwidth kernels.
hipError_t kb_launch_stream(int kind, float *a, const float *b, float s, size_t n, int block,
                            hipStream_t stream);
// Ceiling probes (ceiling.hip): waves one launch runs on `cus` CUs,
// operations (or bytes) it performs, the work-buffer layout (clock counters,
// then one sink float per thread, then the data the cache probes read) and
// the launch itself (clk: 2 counters per wave).
int kb_ceiling_waves(int cus);
double kb_ceiling_ops(int kind, int cus, int iters);
size_t kb_ceiling_layout(int cus, size_t *sink_offset, size_t *data_offset);
hipError_t kb_launch_ceiling(int kind, int cus, int iters, unsigned long long *clk, float *sink,
                             const unsigned char *data, hipStream_t stream);
