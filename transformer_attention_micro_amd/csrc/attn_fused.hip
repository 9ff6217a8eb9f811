// attn_fused: one workgroup per query row, the row's scores kept in LDS.
//
// Method (kbench page, "The three GPU kernels", the fused kernel): a block
// handles one query row and holds its S-length score vector in on-chip
// memory, so the three passes collapse into one kernel with no score
// round-trip through DRAM.  The LDS footprint grows with S, which caps the
// sequence length the kernel supports (4 * S bytes of scores per workgroup).
//
// Per row (bh, i), 256 threads:
//  1. scores  s_j = scale * <q, k_j> for the visible keys, each written to
//     LDS by the leader of the 4 lanes that read key row j with 16-byte
//     loads, lane k taking the chunks k, k + 4, ... (so each load
//     instruction reads 64 contiguous bytes of 16 keys' rows): packed bf16
//     dot products with fp32 accumulation (v_dot2c_f32_bf16: products of
//     bf16 values are exact in fp32), or fp32 FMAs, and a sum over the 4
//     lanes;
//  2. m = max_j s_j (wave shuffles, then across the 4 waves through LDS);
//  3. p_j = 2^((s_j - m) log2 e) in place, l = sum_j p_j;
//  4. o = sum_j p_j v_j / l: thread (g, c) accumulates 16-byte column chunk c
//     over keys j = g mod G; the G partial rows are summed through LDS.
// Everything after the input loads is fp32.
#include <type_traits>

#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;  // elements per 16-byte chunk
  __device__ static void unpack(const u32x4 &u, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = __uint_as_float(u[e] << 16);
      f[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
  }
};
template <>
struct Elem<float> {
  static constexpr int kPerChunk = 4;
  __device__ static void unpack(const u32x4 &u, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(u[e]);
  }
};

template <int D, typename T>
__global__ __launch_bounds__(kThreads) void fused_kernel(const T *__restrict__ Q, const T *__restrict__ K,
                                                         const T *__restrict__ V, void *__restrict__ O,
                                                         int out_bf16, int S, int causal, float scale) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int CPR = D / EPC;            // 16-byte chunks per row
  constexpr int G = kThreads / CPR;       // key groups in the P V phase
  static_assert(CPR <= kWave && kWave % CPR == 0, "row chunking");

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float *sc = smem;                       // S scores / probabilities
  float *part = smem + ((S + 3) & ~3);    // G x D partial output rows
  __shared__ float red[kWaves];

  const size_t row = blockIdx.x;
  const int bh = (int)(row / (size_t)S), i = (int)(row % (size_t)S);
  const int nvis = causal ? i + 1 : S;
  const size_t base = (size_t)bh * S * D;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // 1. scores: 4 lanes per key row, lane k taking the row's 16-byte chunks
  // k, k + 4, ... (each load instruction reads 64 contiguous bytes of 16
  // keys' rows); bf16 by packed dot products (v_dot2c_f32_bf16, fp32
  // accumulation: products of bf16 values are exact in fp32), fp32 by FMAs;
  // then a shuffle sum over the 4 lanes.
  float mloc = -INFINITY;
  {
    constexpr int LPK = 4, CPL = CPR / LPK, KPS = kWave / LPK;  // lanes / chunks per key, keys per step
    static_assert(CPR % LPK == 0, "row chunking");
    const int k4 = lane % LPK, key = lane / LPK;
    u32x4 qc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) qc[c] = *(const u32x4 *)(Q + base + (size_t)i * D + (LPK * c + k4) * EPC);
    for (int j0 = 0; j0 < nvis; j0 += kWaves * KPS) {
      const int j = j0 + w * KPS + key;
      float dot = 0.f;
      if (j < nvis) {
        const T *kr = K + base + (size_t)j * D;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const u32x4 kv = *(const u32x4 *)(kr + (LPK * c + k4) * EPC);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // (through scalars: a bit_cast straight from a vector element
            // reads element 0)
            const uint32_t ke = kv[e], qe = qc[c][e];
            if constexpr (std::is_same<T, bf16_t>::value)
              dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ke), __builtin_bit_cast(bf16x2, qe),
                                                    dot, false);
            else
              dot = fmaf(__uint_as_float(qe), __uint_as_float(ke), dot);
          }
        }
      }
      dot = group_sum<LPK>(dot);
      if (j < nvis && k4 == 0) {
        const float s = dot * scale;
        sc[j] = s;
        mloc = fmaxf(mloc, s);
      }
    }
  }
  __syncthreads();
  // 2. max
  const float m = block_max<kWaves>(mloc, red);
  // 3. exponentials and their sum
  float lloc = 0.f;
  for (int j = tid; j < nvis; j += kThreads) {
    const float p = exp2_fast((sc[j] - m) * kLog2e);
    sc[j] = p;
    lloc += p;
  }
  const float l = block_sum<kWaves>(lloc, red);  // includes a barrier: sc[] complete
  // 4. P V
  {
    const int c = tid % CPR, g = tid / CPR;
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    for (int j = g; j < nvis; j += G) {
      float vv[EPC];
      Elem<T>::unpack(*(const u32x4 *)(V + base + (size_t)j * D + c * EPC), vv);
      const float p = sc[j];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = fmaf(p, vv[e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) part[g * D + c * EPC + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
    for (int g = 0; g < G; ++g) o += part[g * D + tid];
    store_out1(O, base + (size_t)i * D + tid, o / l, out_bf16);
  }
}

template <int D, typename T>
size_t lds_bytes(int S) {
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int G = kThreads / (D / EPC);
  return (size_t)((S + 3) & ~3) * sizeof(float) + (size_t)G * D * sizeof(float);
}

template <int D, typename T>
hipError_t launch_t(const kb_problem &p) {
  const size_t lds = lds_bytes<D, T>(p.S);
  auto fn = fused_kernel<D, T>;
  hipError_t e = hipFuncSetAttribute((const void *)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((size_t)p.bh * p.S));
  hipLaunchKernelGGL(fn, grid, dim3(kThreads), lds, p.stream, (const T *)p.Q, (const T *)p.K,
                     (const T *)p.V, p.O, p.out_bf16, p.S, p.causal, p.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const kb_problem &p) {
  return p.bf16 ? launch_t<D, bf16_t>(p) : launch_t<D, float>(p);
}

}  // namespace

size_t kb_fused_lds_bytes(const kb_problem &p) {
  // static part (red[]) is small; count it too
  size_t extra = kWaves * sizeof(float);
  switch (p.D) {
    case 32: return extra + (p.bf16 ? lds_bytes<32, bf16_t>(p.S) : lds_bytes<32, float>(p.S));
    case 64: return extra + (p.bf16 ? lds_bytes<64, bf16_t>(p.S) : lds_bytes<64, float>(p.S));
    case 128: return extra + (p.bf16 ? lds_bytes<128, bf16_t>(p.S) : lds_bytes<128, float>(p.S));
    default: return (size_t)-1;
  }
}

hipError_t kb_launch_fused(const kb_problem &p) {
  switch (p.D) {
    case 32: return launch_d<32>(p);
    case 64: return launch_d<64>(p);
    case 128: return launch_d<128>(p);
    default: return hipErrorInvalidValue;
  }
}
