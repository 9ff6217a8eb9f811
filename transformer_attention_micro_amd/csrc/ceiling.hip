// Compute ceilings: the sustained throughput of the instructions the
// attention kernels are built from, the compute analogue of the HBM triad.
//
// Method (the micro-benchmark log page, section on compute peaks, its B1
// and B2 tests): every thread runs several independent chains of one
// instruction, so no instruction waits for the one before it; the matrix
// products are dense with fp32 accumulation; and the clock the hardware
// actually ran at is recorded beside the result, because a datasheet peak
// assumes the nominal clock and a sustained load does not run there.
//
// Here one workgroup per CU (a 96 KiB LDS reservation keeps it alone) of
// eight waves, two per SIMD, loops over
//   KB_CEIL_MFMA_BF16  v_mfma_f32_32x32x16_bf16 on 8 independent accumulators
//   KB_CEIL_MFMA_F32   v_mfma_f32_32x32x2f32    on 8 independent accumulators
//   KB_CEIL_FMA_F32    v_fma_f32                on 8 independent chains
//   KB_CEIL_EXP_F32    v_exp_f32                on 8 independent chains
// and each wave records the shader clock counter (s_memtime) and the
// 100 MHz real-time counter (s_memrealtime) around its loop; their ratio is
// the clock the wave saw.
#include "kb_attention.h"
#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kCeilThreads = 512;
constexpr int kCeilWaves = kCeilThreads / kWave;
constexpr int kChains = 8;

template <int KIND>
__global__ __launch_bounds__(kCeilThreads) void ceiling_kernel(int iters, float seed,
                                                               unsigned long long *__restrict__ clk,
                                                               float *__restrict__ sink) {
  __shared__ float reserve[96 * 256];
  if (iters < 0) reserve[threadIdx.x] = seed;  // never taken; keeps the reservation
  const int lane = threadIdx.x & (kWave - 1);
  float r = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  if constexpr (KIND == KB_CEIL_MFMA_BF16) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (bf16_t)(seed * (lane + i));
      b[i] = (bf16_t)(seed * (i + 1));
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma32x16_bf16(a, b, acc[c]);
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][c];
  } else if constexpr (KIND == KB_CEIL_MFMA_F32) {
    const float a = seed * lane, b = seed;
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma32x2_f32(a, b, acc[c]);
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][c];
  } else if constexpr (KIND == KB_CEIL_FMA_F32) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = seed * (lane + c);
    const float m = 1.0f - 1e-7f * seed, s = 1e-7f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) x[c] = fmaf(x[c], m, s);
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += x[c];
  } else {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = -seed * (lane + c);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) x[c] = exp2_fast(x[c]);
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += x[c];
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  const size_t wave = (size_t)blockIdx.x * kCeilWaves + threadIdx.x / kWave;
  if (lane == 0) {
    clk[2 * wave] = t1 - t0;
    clk[2 * wave + 1] = r1 - r0;
  }
  sink[(size_t)blockIdx.x * kCeilThreads + threadIdx.x] = r;
}

}  // namespace

int kb_ceiling_waves(int cus) { return cus * kCeilWaves; }

double kb_ceiling_ops(int kind, int cus, int iters) {
  const double per_instr = kind == KB_CEIL_MFMA_BF16 ? 2.0 * 32 * 32 * 16
                           : kind == KB_CEIL_MFMA_F32 ? 2.0 * 32 * 32 * 2
                           : kind == KB_CEIL_FMA_F32  ? 2.0 * kWave
                                                      : 1.0 * kWave;
  return per_instr * kChains * (double)iters * kb_ceiling_waves(cus);
}

hipError_t kb_launch_ceiling(int kind, int cus, int iters, unsigned long long *clk, float *sink,
                             hipStream_t stream) {
  const dim3 grid((unsigned)cus), block(kCeilThreads);
  const float seed = 1e-3f;
  switch (kind) {
    case KB_CEIL_MFMA_BF16:
      hipLaunchKernelGGL(ceiling_kernel<KB_CEIL_MFMA_BF16>, grid, block, 0, stream, iters, seed, clk, sink);
      break;
    case KB_CEIL_MFMA_F32:
      hipLaunchKernelGGL(ceiling_kernel<KB_CEIL_MFMA_F32>, grid, block, 0, stream, iters, seed, clk, sink);
      break;
    case KB_CEIL_FMA_F32:
      hipLaunchKernelGGL(ceiling_kernel<KB_CEIL_FMA_F32>, grid, block, 0, stream, iters, seed, clk, sink);
      break;
    case KB_CEIL_EXP_F32:
      hipLaunchKernelGGL(ceiling_kernel<KB_CEIL_EXP_F32>, grid, block, 0, stream, iters, seed, clk, sink);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
