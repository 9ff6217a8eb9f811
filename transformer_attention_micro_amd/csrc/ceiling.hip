// Ceiling probes: the sustained throughput of the instructions the attention
// kernels are built from (the compute analogue of the HBM triad) and the
// read bandwidth of each on-chip memory level they stage data through.
//
// Method for the compute kinds (the micro-benchmark log page, section on
// compute peaks, its B1 and B2 tests): every thread runs several independent
// chains of one instruction, so no instruction waits for the one before it;
// the matrix products are dense with fp32 accumulation; and the clock the
// hardware actually ran at is recorded beside the result, because a
// datasheet peak assumes the nominal clock and a sustained load does not run
// there.  The memory kinds give the bandwidth ceilings of the hierarchical
// roofline (the GPU-Roofline-Python page, "Bandwidth Ceilings": measured
// bandwidths of each cache level beside the datasheet ones).
//
// Here one workgroup per CU (a 96 KiB LDS reservation keeps it alone) of
// eight waves, two per SIMD, loops over
//   KB_CEIL_MFMA_BF16  v_mfma_f32_32x32x16_bf16 on 8 independent accumulators
//   KB_CEIL_MFMA_F32   v_mfma_f32_32x32x2f32    on 8 independent accumulators
//   KB_CEIL_FMA_F32    v_fma_f32                on 8 independent chains
//   KB_CEIL_EXP_F32    v_exp_f32                on 8 independent chains
//   KB_CEIL_LDS_READ   8 ds_read_b128 per wave per iteration over a 64 KiB
//                      LDS window (1 KiB contiguous per wave instruction,
//                      free of bank conflicts)
//   KB_CEIL_L1_READ    8 global 16-byte-per-lane loads per wave per iteration
//                      over a 16 KiB slice private to the workgroup, which
//                      the CU's vector L1 cache holds after the first pass
//   KB_CEIL_L2_READ    the same loads over a 2 MiB region per XCD (workgroup
//                      g reads region g mod 8, the XCD it runs on): larger
//                      than the vector L1, well inside one XCD's 4 MiB L2,
//                      the workgroups of an XCD spread over the whole region
//   KB_CEIL_MFMA_BF16_DATA  v_mfma_f32_32x32x16_bf16 as KB_CEIL_MFMA_BF16,
//                      but on operands of random bits: 8 A and 8 B register
//                      sets of random bf16 values (random sign and mantissa,
//                      magnitudes 2^-4 .. 2^4), a different (A, B) pair for
//                      each product of 8 consecutive iterations, so the
//                      matrix core switches data like a real product does
//                      (the other MFMA kind repeats one constant pair)
//   KB_CEIL_MFMA_BF16_FMA3 / _EXP3 / _EXP4 / _LDS
//                      co-issue: the constant-operand products of
//                      KB_CEIL_MFMA_BF16, each followed (in the same wave, in
//                      a fixed order the compiler may not move) by 3
//                      independent v_fma_f32, 3 or 4 independent v_exp_f32,
//                      or LDS reads over the window, one ds_read_b128 after
//                      even products and a pair of ds_read_b64_tr_b16 after
//                      odd ones (1.5 per product, the mix of the flash
//                      step), whose fragment is the A operand of the product
//                      two later.  The rate counts the
//                      products only: how much of that other work a wave
//                      can issue in the products' shadow, two waves per
//                      SIMD as in the attention kernel, and at what clock.
// and each wave records the shader clock counter (s_memtime) and the
// 100 MHz real-time counter (s_memrealtime) around its loop; their ratio is
// the clock the wave saw.  Every loaded dword feeds an integer sum written
// to the sink, so no load can be dropped or narrowed.
#include "kb_attention.h"
#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kCeilThreads = 512;
constexpr int kCeilWaves = kCeilThreads / kWave;
constexpr int kChains = 8;
constexpr int kChunk = kWave * 16;                 // bytes one wave's 16-byte-per-lane load moves
constexpr int kLdsWindowChunks = 64;               // 64 KiB LDS window
constexpr size_t kL1Slice = 16 * 1024;             // per workgroup
constexpr size_t kL2Region = 2 * 1024 * 1024;      // per XCD
constexpr int kL2Groups = (int)(kL2Region / (kChains * kChunk));  // 8-chunk groups per region
constexpr int kXcdRegions = 8;

// Random bf16 bits for the data-driven MFMA probe: a 32-bit integer hash
// (multiply-xorshift rounds) of the lane, wave, workgroup and slot; random
// sign and 7-bit mantissa, exponent 123 .. 130.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ bf16x8 random_bf16x8(uint32_t key) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = mix32(key * 8u + (uint32_t)e);
    const unsigned short bits = (unsigned short)((h & 0x807Fu) | ((123u + ((h >> 8) & 7u)) << 7));
    r[e] = __builtin_bit_cast(bf16_t, bits);
  }
  return r;
}

__device__ __forceinline__ void consume(const u32x4 v, uint32_t &s0, uint32_t &s1) {
  s0 += v.x + v.y;
  s1 += v.z + v.w;
}

template <int KIND>
__global__ __launch_bounds__(kCeilThreads) void ceiling_kernel(int iters, float seed,
                                                               unsigned long long *__restrict__ clk,
                                                               float *__restrict__ sink,
                                                               const unsigned char *__restrict__ data) {
  __shared__ float reserve[96 * 256];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  if constexpr (KIND == KB_CEIL_LDS_READ || KIND == KB_CEIL_MFMA_BF16_LDS) {
    // Defined contents for the window the loop reads.
    for (int i = threadIdx.x; i < kLdsWindowChunks * kChunk / 4; i += kCeilThreads) reserve[i] = seed * i;
    __syncthreads();
  } else {
    if (iters < 0) reserve[threadIdx.x] = seed;  // never taken; keeps the reservation
  }
  float r = 0.f;
  uint32_t s0 = 0, s1 = 0;
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
  } else if constexpr (KIND == KB_CEIL_MFMA_BF16_DATA) {
    bf16x8 a[kChains], b[kChains];
    const uint32_t key = (((uint32_t)blockIdx.x * kCeilWaves + (uint32_t)wave) * kWave + (uint32_t)lane) * 16u +
                         (uint32_t)(seed * 1e3f);
#pragma unroll
    for (int i = 0; i < kChains; ++i) {
      a[i] = random_bf16x8(key + (uint32_t)i);
      b[i] = random_bf16x8(key + 8u + (uint32_t)i);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    // Iteration it uses pair (a[(c + it) % 8], b[(c + 3 it + 1) % 8]) for
    // chain c: blocks of 8 iterations, then the remainder.
    auto step = [&](int u) {
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = mfma32x16_bf16(a[(c + u) & 7], b[(c + 3 * u + 1) & 7], acc[c]);
    };
    int it = 0;
    for (; it + 8 <= iters; it += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) step(u);
    }
#pragma unroll
    for (int u = 0; u < 7; ++u)
      if (it + u < iters) step(u);
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][c];
  } else if constexpr (KIND == KB_CEIL_MFMA_BF16_FMA3 || KIND == KB_CEIL_MFMA_BF16_EXP3 ||
                       KIND == KB_CEIL_MFMA_BF16_EXP4 || KIND == KB_CEIL_MFMA_BF16_LDS) {
    constexpr bool kExp = KIND == KB_CEIL_MFMA_BF16_EXP3 || KIND == KB_CEIL_MFMA_BF16_EXP4;
    constexpr int kV = KIND == KB_CEIL_MFMA_BF16_EXP4 ? 4 : KIND == KB_CEIL_MFMA_BF16_LDS ? 0 : 3;
    constexpr int kRegs = 16;  // independent vector chains, each touched every 16 / kV products
    typedef __attribute__((address_space(3))) bf16x8 lds_frag;
    typedef __attribute__((address_space(3))) s16x4 lds_half;
    typedef __attribute__((address_space(3))) unsigned char lds_byte;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (bf16_t)(seed * (lane + i));
      b[i] = (bf16_t)(seed * (i + 1));
    }
    bf16x8 fr[4] = {a, a, a, a};
    float v[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) v[i] = kExp ? -seed * (lane + i) : seed * (lane + i);
    const float m = 1.0f - 1e-7f * seed, s = 1e-7f;
    const lds_byte *win = (const lds_byte *)(const __attribute__((address_space(3))) float *)reserve + lane * 16;
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) {
        acc[c] = mfma32x16_bf16(KIND == KB_CEIL_MFMA_BF16_LDS ? fr[c & 3] : a, b, acc[c]);
#pragma unroll
        for (int k = 0; k < kV; ++k) {
          float &x = v[(c * kV + k) % kRegs];
          x = kExp ? exp2_fast(x) : fmaf(x, m, s);
        }
        if constexpr (KIND == KB_CEIL_MFMA_BF16_LDS) {
          // Even products: one 16-byte read of 1 KiB chunk (it * 8 + c) mod
          // 32 of the window; odd ones: two 8-byte transposing reads of it.
          const lds_byte *p = win + (((unsigned)(it * kChains + c)) & 31u) * kChunk;
          if ((c & 1) == 0) {
            fr[(c + 2) & 3] = *(const lds_frag *)p;
          } else {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_half *)p);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_half *)(p + 512));
            fr[(c + 2) & 3] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][c];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) r += v[i];
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
  } else if constexpr (KIND == KB_CEIL_EXP_F32) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = -seed * (lane + c);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) x[c] = exp2_fast(x[c]);
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += x[c];
  } else if constexpr (KIND == KB_CEIL_LDS_READ) {
    const unsigned char *lds = (const unsigned char *)reserve + lane * 16;
    for (int it = 0; it < iters; ++it) {
      // First chunk of this wave's 8 (a multiple of 8, at most 56).
      const unsigned base = ((unsigned)(it + wave) * kChains) & (kLdsWindowChunks - 1);
      const unsigned char *p = lds + base * kChunk;
#pragma unroll
      for (int c = 0; c < kChains; ++c) consume(*(const u32x4 *)(p + c * kChunk), s0, s1);
    }
  } else if constexpr (KIND == KB_CEIL_L1_READ) {
    const unsigned char *g = data + (size_t)blockIdx.x * kL1Slice + lane * 16;
    for (int it = 0; it < iters; ++it) {
      const unsigned char *p = g + (size_t)(it & 1) * (kChains * kChunk);
#pragma unroll
      for (int c = 0; c < kChains; ++c) consume(*(const u32x4 *)(p + c * kChunk), s0, s1);
    }
  } else {
    const int xcd = blockIdx.x % kXcdRegions, jw = blockIdx.x / kXcdRegions;
    const unsigned char *g = data + (size_t)xcd * kL2Region + lane * 16;
    for (int it = 0; it < iters; ++it) {
      const unsigned group = ((unsigned)it * kCeilWaves + wave + jw * kChains) & (kL2Groups - 1);
      const unsigned char *p = g + (size_t)group * (kChains * kChunk);
#pragma unroll
      for (int c = 0; c < kChains; ++c) consume(*(const u32x4 *)(p + c * kChunk), s0, s1);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if constexpr (KIND == KB_CEIL_LDS_READ || KIND == KB_CEIL_L1_READ || KIND == KB_CEIL_L2_READ)
    r = __uint_as_float(s0 ^ s1);
  const size_t w = (size_t)blockIdx.x * kCeilWaves + wave;
  if (lane == 0) {
    clk[2 * w] = t1 - t0;
    clk[2 * w + 1] = r1 - r0;
  }
  sink[(size_t)blockIdx.x * kCeilThreads + threadIdx.x] = r;
}

static_assert((kL2Groups & (kL2Groups - 1)) == 0, "the L2 region is a power of two of 8-chunk groups");
static_assert(kLdsWindowChunks * kChunk <= 96 * 256 * 4, "the LDS window fits the reservation");
static_assert(2 * kChains * kChunk <= (int)kL1Slice, "two 8-chunk halves fit the L1 slice");

template <int KIND>
void launch_kind(int cus, int iters, unsigned long long *clk, float *sink, const unsigned char *data,
                 hipStream_t stream) {
  hipLaunchKernelGGL(ceiling_kernel<KIND>, dim3((unsigned)cus), dim3(kCeilThreads), 0, stream, iters, 1e-3f,
                     clk, sink, data);
}

}  // namespace

int kb_ceiling_waves(int cus) { return cus * kCeilWaves; }

double kb_ceiling_ops(int kind, int cus, int iters) {
  const bool bf16_mfma = kind == KB_CEIL_MFMA_BF16 || kind == KB_CEIL_MFMA_BF16_DATA || kind == KB_CEIL_MFMA_BF16_FMA3 ||
                         kind == KB_CEIL_MFMA_BF16_EXP3 || kind == KB_CEIL_MFMA_BF16_EXP4 ||
                         kind == KB_CEIL_MFMA_BF16_LDS;
  const double per_instr = bf16_mfma ? 2.0 * 32 * 32 * 16
                           : kind == KB_CEIL_MFMA_F32 ? 2.0 * 32 * 32 * 2
                           : kind == KB_CEIL_FMA_F32  ? 2.0 * kWave
                           : kind == KB_CEIL_EXP_F32  ? 1.0 * kWave
                                                      : (double)kChunk;
  return per_instr * kChains * (double)iters * kb_ceiling_waves(cus);
}

// Work buffer: per-wave clock counters, one sink float per thread, then the
// data the cache probes read (4 KiB aligned): an L2 region per XCD or an L1
// slice per workgroup, whichever is larger.
size_t kb_ceiling_layout(int cus, size_t *sink_offset, size_t *data_offset) {
  const size_t sink_off = (size_t)kb_ceiling_waves(cus) * 2 * sizeof(unsigned long long);
  const size_t data_off = (sink_off + (size_t)cus * kCeilThreads * sizeof(float) + 4095) & ~(size_t)4095;
  const size_t l2 = (size_t)kXcdRegions * kL2Region, l1 = (size_t)cus * kL1Slice;
  if (sink_offset) *sink_offset = sink_off;
  if (data_offset) *data_offset = data_off;
  return data_off + (l2 > l1 ? l2 : l1);
}

hipError_t kb_launch_ceiling(int kind, int cus, int iters, unsigned long long *clk, float *sink,
                             const unsigned char *data, hipStream_t stream) {
  switch (kind) {
    case KB_CEIL_MFMA_BF16: launch_kind<KB_CEIL_MFMA_BF16>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_MFMA_F32: launch_kind<KB_CEIL_MFMA_F32>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_FMA_F32: launch_kind<KB_CEIL_FMA_F32>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_EXP_F32: launch_kind<KB_CEIL_EXP_F32>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_LDS_READ: launch_kind<KB_CEIL_LDS_READ>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_L1_READ: launch_kind<KB_CEIL_L1_READ>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_L2_READ: launch_kind<KB_CEIL_L2_READ>(cus, iters, clk, sink, data, stream); break;
    case KB_CEIL_MFMA_BF16_DATA:
      launch_kind<KB_CEIL_MFMA_BF16_DATA>(cus, iters, clk, sink, data, stream);
      break;
    case KB_CEIL_MFMA_BF16_FMA3:
      launch_kind<KB_CEIL_MFMA_BF16_FMA3>(cus, iters, clk, sink, data, stream);
      break;
    case KB_CEIL_MFMA_BF16_EXP3:
      launch_kind<KB_CEIL_MFMA_BF16_EXP3>(cus, iters, clk, sink, data, stream);
      break;
    case KB_CEIL_MFMA_BF16_EXP4:
      launch_kind<KB_CEIL_MFMA_BF16_EXP4>(cus, iters, clk, sink, data, stream);
      break;
    case KB_CEIL_MFMA_BF16_LDS:
      launch_kind<KB_CEIL_MFMA_BF16_LDS>(cus, iters, clk, sink, data, stream);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
