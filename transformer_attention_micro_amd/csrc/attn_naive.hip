// attn_naive: the three-pass, bandwidth-bound baseline, for gfx950.
//
// Method (kbench page, "The three GPU kernels", the naive kernel): a GEMM
// writes the full S x S score matrix to DRAM, a row-wise softmax runs over
// it, and a second GEMM forms P V.  All O(S^2) scores stream through HBM, so
// the kernel is bound by HBM bandwidth (page section "Expected results").
//
// Pass 1  W[bh, i, j] = scale * <Q[bh, i], K[bh, j]>      all i, j < S (fp32)
// Pass 2  W[bh, i, :] <- softmax over the visible j, in place; masked
//         entries (causal, j > i) are written as exactly 0
// Pass 3  O[bh, i, :] = sum_j W[bh, i, j] V[bh, j, :]      fp32 out
// The full S x S block is computed even under the causal mask: the mask is
// applied by the softmax pass, as in the plain three-pass reading.
//
// bf16 inputs: bf16 MFMA with fp32 accumulate in both GEMMs; pass 3 rounds
// each fp32 probability to bf16 (round to nearest even) as it loads it, the
// same rounding the flash kernel applies.  fp32 inputs: fp32 MFMA.
#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kThreads = 256;
// Score matrices larger than the 256 MB Infinity Cache leave the caches
// before the next pass reads them: their stores (pass 1, pass 2) and the
// softmax pass's loads then carry the non-temporal hint, which keeps them
// from displacing lines that are still to be used.  Measured (same box,
// interleaved): B2 H32 S8192 causal -2.3 %, B1 H16 S32768 -2.5 %, B4 H16
// S2048 causal -11.8 %; at B1 H8 S512 (8 MiB of scores, served from the
// caches between passes) the hint cost 5.5 %, so small matrices keep plain
// accesses.  (Pass 3's probability loads take 32-byte pieces of a line per
// instruction, which the cached path merges: with the hint it was 17 %
// slower.)
constexpr size_t kStreamingScoreBytes = (size_t)256 << 20;

template <bool NT, typename T>
__device__ __forceinline__ void put(T *p, const T &v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}
template <bool NT, typename T>
__device__ __forceinline__ T get(const T *p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// ------------------------------------------------------------- pass 1 -----
// Workgroup tile: 128 keys j x 128 queries i, computed transposed,
// W^T block = K Q^T: the K tile (128 x D) is staged once in LDS (rows padded
// by 16 bytes) and read by all four waves; wave w keeps Q^T of its 32
// queries i0 .. i0 + 31 in registers.  Lane (l32, h) then holds, for each
// 32-key block jb, the scores of query i0 + l32 against keys
// 32 jb + 8 r + 4 h + {0, 1, 2, 3}.  The scores leave through LDS (the K
// tile's space, rows padded to 68 floats) in two halves of 64 keys, so each
// store instruction writes four whole 256-byte pieces of rows; the pass is
// bound by these HBM writes.
template <int D, bool VEC, bool NT>
__global__ __launch_bounds__(kThreads) void scores_bf16_kernel(const bf16_t *__restrict__ Q,
                                                               const bf16_t *__restrict__ K,
                                                               float *__restrict__ W, int S,
                                                               float scale) {
  constexpr int KC = D / 16;
  constexpr int STR = D + 8;
  constexpr int CPR = D / 8;
  constexpr int NCH = 128 * CPR / kThreads;
  // K tile (bf16, 128 x STR) or, after the MFMAs, four 32 x 68 fp32 blocks.
  constexpr int LDS_BYTES = 128 * STR * 2 > 4 * 32 * 68 * 4 ? 128 * STR * 2 : 4 * 32 * 68 * 4;
  __shared__ __attribute__((aligned(16))) float lds[LDS_BYTES / 4];
  bf16_t *Ks = (bf16_t *)lds;
  const int bh = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int i0 = blockIdx.y * 128 + 32 * w;
  const int j0 = blockIdx.x * 128;
  const size_t base = (size_t)bh * S * D;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int idx = tid + c * kThreads;
    const int row = idx / CPR, col = (idx % CPR) * 8;
    const int key = j0 + row;
    u32x4 val = u32x4{0, 0, 0, 0};
    if (key < S) val = *(const u32x4 *)(K + base + (size_t)key * D + col);
    *(u32x4 *)&Ks[row * STR + col] = val;
  }
  bf16x8 qf[KC];
  const bf16_t *qp = Q + base + (size_t)min(i0 + l32, S - 1) * D + 8 * h;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const bf16x8 *)(qp + 16 * kc);
  __syncthreads();
  f32x16 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      acc[jb] = mfma32x16_bf16(*(const bf16x8 *)&Ks[(32 * jb + l32) * STR + 16 * kc + 8 * h], qf[kc], acc[jb]);
  if (VEC) {
    float *T = lds + w * 32 * 68;
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      __syncthreads();
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jb = 2 * ph + jj;
          const f32x4 val = {acc[jb][4 * r] * scale, acc[jb][4 * r + 1] * scale, acc[jb][4 * r + 2] * scale,
                             acc[jb][4 * r + 3] * scale};
          *(f32x4 *)&T[l32 * 68 + 32 * jj + 8 * r + 4 * h] = val;
        }
      __syncthreads();
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int row = 4 * rr + (lane >> 4), col = 4 * (lane & 15);
        const int i = i0 + row, j = j0 + 64 * ph + col;
        const f32x4 val = *(const f32x4 *)&T[row * 68 + col];
        if (i < S && j + 4 <= S) put<NT>((f32x4 *)(W + ((size_t)bh * S + i) * (size_t)S + j), val);
        else if (i < S)
          for (int e = 0; e < 4; ++e)
            if (j + e < S) W[((size_t)bh * S + i) * (size_t)S + j + e] = val[e];
      }
    }
    return;
  }
  const int i = i0 + l32;
  if (i >= S) return;
  float *wp = W + ((size_t)bh * S + i) * (size_t)S + j0;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = 32 * jb + 8 * r + 4 * h;
      const f32x4 val = {acc[jb][4 * r] * scale, acc[jb][4 * r + 1] * scale, acc[jb][4 * r + 2] * scale,
                         acc[jb][4 * r + 3] * scale};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j0 + j + e < S) wp[j + e] = val[e];
    }
}

// fp32: contraction step (g, e) uses d-column 8g + 4h + e from lane half h.
template <int D, bool NT>
__global__ __launch_bounds__(kThreads) void scores_f32_kernel(const float *__restrict__ Q,
                                                              const float *__restrict__ K,
                                                              float *__restrict__ W, int S,
                                                              float scale) {
  const int bh = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int i0 = blockIdx.y * 128 + 32 * w;
  const int j0 = blockIdx.x * 128;
  const size_t base = (size_t)bh * S * D;
  const float *qp = Q + base + (size_t)min(i0 + l32, S - 1) * D + 4 * h;
  const float *kp[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) kp[jb] = K + base + (size_t)min(j0 + 32 * jb + l32, S - 1) * D + 4 * h;
  f32x16 acc[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) acc[jb] = f32x16{};
#pragma unroll
  for (int g = 0; g < D / 8; ++g) {
    const f32x4 a = *(const f32x4 *)(qp + 8 * g);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const f32x4 b = *(const f32x4 *)(kp[jb] + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[jb] = mfma32x2_f32(a[e], b[e], acc[jb]);
    }
  }
  float *wp = W + (size_t)bh * S * S;
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int j = j0 + 32 * jb + l32;
    if (j >= S) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + acc_row(v, h);
      if (i < S) put<NT>(&wp[(size_t)i * S + j], acc[jb][v] * scale);
    }
  }
}

// ------------------------------------------------------------- pass 2 -----
// One workgroup per row.  Vector path: the row (S % 4 == 0, S <= 1024 * NV)
// is held in registers as NV float4 per thread, so it is read once and
// written once.
template <int NV, bool NT>
__global__ __launch_bounds__(kThreads) void softmax_vec_kernel(float *__restrict__ W, int S,
                                                               int causal) {
  __shared__ float red[kThreads / kWave];
  const size_t row = blockIdx.x;
  const int i = (int)(row % (size_t)S);
  const int nvis = causal ? i + 1 : S;
  float4 *rp = (float4 *)(W + row * (size_t)S);
  float4 x[NV];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int e = 4 * (threadIdx.x + kThreads * k);
    if (e < S) {
      const f32x4 t = get<NT>((const f32x4 *)&rp[threadIdx.x + kThreads * k]);
      x[k] = make_float4(t[0], t[1], t[2], t[3]);
      if (e + 0 >= nvis) x[k].x = -INFINITY;
      if (e + 1 >= nvis) x[k].y = -INFINITY;
      if (e + 2 >= nvis) x[k].z = -INFINITY;
      if (e + 3 >= nvis) x[k].w = -INFINITY;
    } else {
      x[k] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    m = fmaxf(m, fmaxf(fmaxf(x[k].x, x[k].y), fmaxf(x[k].z, x[k].w)));
  }
  m = block_max<kThreads / kWave>(m, red);
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    x[k].x = exp2_fast((x[k].x - m) * kLog2e);
    x[k].y = exp2_fast((x[k].y - m) * kLog2e);
    x[k].z = exp2_fast((x[k].z - m) * kLog2e);
    x[k].w = exp2_fast((x[k].w - m) * kLog2e);
    l += (x[k].x + x[k].y) + (x[k].z + x[k].w);
  }
  l = block_sum<kThreads / kWave>(l, red);
  const float inv = 1.f / l;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int e = 4 * (threadIdx.x + kThreads * k);
    if (e < S)
      put<NT>((f32x4 *)&rp[threadIdx.x + kThreads * k], f32x4{x[k].x * inv, x[k].y * inv, x[k].z * inv, x[k].w * inv});
  }
}

// General path (any S): three sweeps over the row in global memory.
__global__ __launch_bounds__(kThreads) void softmax_any_kernel(float *__restrict__ W, int S, int causal) {
  __shared__ float red[kThreads / kWave];
  const size_t row = blockIdx.x;
  const int i = (int)(row % (size_t)S);
  const int nvis = causal ? i + 1 : S;
  float *rp = W + row * (size_t)S;
  float m = -INFINITY;
  for (int j = threadIdx.x; j < nvis; j += kThreads) m = fmaxf(m, rp[j]);
  m = block_max<kThreads / kWave>(m, red);
  float l = 0.f;
  for (int j = threadIdx.x; j < nvis; j += kThreads) l += exp2_fast((rp[j] - m) * kLog2e);
  l = block_sum<kThreads / kWave>(l, red);
  const float inv = 1.f / l;
  for (int j = threadIdx.x; j < S; j += kThreads)
    rp[j] = j < nvis ? exp2_fast((rp[j] - m) * kLog2e) * inv : 0.f;
}

// ------------------------------------------------------------- pass 3 -----
// O^T = V^T P^T per workgroup of 128 query rows (wave w: rows 32w..32w+31);
// 64-key V tiles staged in LDS and read transposed, P^T streamed from global
// memory.  The key order inside each 16-key chunk matches the transposing
// read: lane half h holds keys {4h..4h+3, 8+4h..8+4h+3}.  The global loads
// of tile t+1 (its V rows and this lane's 32 probabilities) are issued before
// tile t is computed, so their latency hides behind the MFMAs; the pass is
// bound by the HBM reads of P.
template <int D, bool VEC>
__global__ __launch_bounds__(kThreads) void pv_bf16_kernel(const float *__restrict__ W,
                                                           const bf16_t *__restrict__ V,
                                                           void *__restrict__ O, int out_bf16, int S) {
  constexpr int BC = 64;
  constexpr int STR = D + 8;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int CH = BC * CPR / kThreads;
  __shared__ __attribute__((aligned(16))) bf16_t Vs[BC * STR];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int q = blockIdx.x * 128 + 32 * w + l32;
  const size_t base = (size_t)bh * S * D;
  const float *prow = W + ((size_t)bh * S + min(q, S - 1)) * (size_t)S;
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  // This thread's share of a V tile and this lane's probabilities of a tile
  // (chunk c16: keys 16 c16 + 4h + {0..3} in slots 0-3, + 8 in slots 4-7).
  u32x4 vreg[CH];
  float pc[BC / 2], pn[BC / 2];
  auto load_v = [&](int kt0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 8;
      const int key = kt0 + row;
      vreg[c] = u32x4{0, 0, 0, 0};
      if (key < S) vreg[c] = *(const u32x4 *)(V + base + (size_t)key * D + col);
    }
  };
  auto load_p = [&](float *pv, int kt0) {
#pragma unroll
    for (int c16 = 0; c16 < BC / 16; ++c16) {
      const int k0 = kt0 + 16 * c16 + 4 * h;
      float *d = pv + 8 * c16;
      if (VEC && k0 + 12 <= S) {
        const float4 a = *(const float4 *)(prow + k0);
        const float4 b = *(const float4 *)(prow + k0 + 8);
        d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
        d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
      } else {
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
          const int key = k0 + (s8 < 4 ? s8 : 4 + s8);
          d[s8] = key < S ? prow[key] : 0.f;
        }
      }
    }
  };
  load_v(0);
  load_p(pc, 0);
  for (int kt0 = 0; kt0 < S; kt0 += BC) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 8;
      *(u32x4 *)&Vs[row * STR + col] = vreg[c];
    }
    __syncthreads();
    const bool more = kt0 + BC < S;
    if (more) {
      load_v(kt0 + BC);
      load_p(pn, kt0 + BC);
    }
#pragma unroll
    for (int c16 = 0; c16 < BC / 16; ++c16) {
      bf16x8 pb;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) pb[s8] = (bf16_t)pc[8 * c16 + s8];
      const bf16_t *vp = &Vs[(16 * c16 + tr_row) * STR + tr_col];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(vp + 32 * mb));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(vp + 8 * STR + 32 * mb));
        const auto a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[mb] = mfma32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, oacc[mb]);
      }
    }
    if (more) {
#pragma unroll
      for (int e = 0; e < BC / 2; ++e) pc[e] = pn[e];
    }
  }
  if (q < S) {
    const size_t op = base + (size_t)q * D + 4 * h;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store_out4(O, op + 32 * mb + 8 * r,
                   f32x4{oacc[mb][4 * r], oacc[mb][4 * r + 1], oacc[mb][4 * r + 2], oacc[mb][4 * r + 3]},
                   out_bf16);
  }
}

// fp32: 32-key V tiles; MFMA step c uses key acc_row(c, h) from lane half h,
// so a lane reads P[q, 8r + 4h .. 8r + 4h + 3] as one vector for steps 4r..4r+3.
template <int D, bool VEC>
__global__ __launch_bounds__(kThreads) void pv_f32_kernel(const float *__restrict__ W,
                                                          const float *__restrict__ V,
                                                          void *__restrict__ O, int out_bf16, int S) {
  constexpr int BC = 32;
  constexpr int STR = D + 4;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 4;
  constexpr int CH = BC * CPR / kThreads;
  __shared__ __attribute__((aligned(16))) float Vs[BC * STR];
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int q = blockIdx.x * 128 + 32 * w + l32;
  const size_t base = (size_t)bh * S * D;
  const float *prow = W + ((size_t)bh * S + min(q, S - 1)) * (size_t)S;
  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  for (int kt0 = 0; kt0 < S; kt0 += BC) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 4;
      const int key = kt0 + row;
      f32x4 val = f32x4{};
      if (key < S) val = *(const f32x4 *)(V + base + (size_t)key * D + col);
      *(f32x4 *)&Vs[row * STR + col] = val;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k0 = kt0 + 8 * r + 4 * h;
      float pv[4];
      if (VEC && k0 + 4 <= S) {
        const float4 a = *(const float4 *)(prow + k0);
        pv[0] = a.x; pv[1] = a.y; pv[2] = a.z; pv[3] = a.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = (k0 + e) < S ? prow[k0 + e] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float *vp = &Vs[(8 * r + 4 * h + e) * STR + l32];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] = mfma32x2_f32(vp[32 * mb], pv[e], oacc[mb]);
      }
    }
  }
  if (q < S) {
    const size_t op = base + (size_t)q * D + 4 * h;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store_out4(O, op + 32 * mb + 8 * r,
                   f32x4{oacc[mb][4 * r], oacc[mb][4 * r + 1], oacc[mb][4 * r + 2], oacc[mb][4 * r + 3]},
                   out_bf16);
  }
}

bool streaming_scores(const kb_problem &p) {
  return (size_t)4 * p.bh * (size_t)p.S * (size_t)p.S > kStreamingScoreBytes;
}

template <int D, bool NT>
hipError_t launch_scores_nt(const kb_problem &p) {
  const int nt = (p.S + 127) / 128;
  const dim3 grid(nt, nt, p.bh);
  if (p.bf16 && p.S % 4 == 0)
    hipLaunchKernelGGL((scores_bf16_kernel<D, true, NT>), grid, dim3(kThreads), 0, p.stream,
                       (const bf16_t *)p.Q, (const bf16_t *)p.K, p.work, p.S, p.scale);
  else if (p.bf16)
    hipLaunchKernelGGL((scores_bf16_kernel<D, false, NT>), grid, dim3(kThreads), 0, p.stream,
                       (const bf16_t *)p.Q, (const bf16_t *)p.K, p.work, p.S, p.scale);
  else
    hipLaunchKernelGGL((scores_f32_kernel<D, NT>), grid, dim3(kThreads), 0, p.stream,
                       (const float *)p.Q, (const float *)p.K, p.work, p.S, p.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_scores(const kb_problem &p) {
  return streaming_scores(p) ? launch_scores_nt<D, true>(p) : launch_scores_nt<D, false>(p);
}

template <bool NT>
hipError_t launch_softmax_nt(const kb_problem &p) {
  const size_t rows = (size_t)p.bh * p.S;
  const dim3 grid((unsigned)rows), block(kThreads);
  if (p.S % 4 == 0 && p.S <= 1024 * 32) {
    const int nv = (p.S + 1023) / 1024;
    if (nv <= 1) hipLaunchKernelGGL((softmax_vec_kernel<1, NT>), grid, block, 0, p.stream, p.work, p.S, p.causal);
    else if (nv <= 2) hipLaunchKernelGGL((softmax_vec_kernel<2, NT>), grid, block, 0, p.stream, p.work, p.S, p.causal);
    else if (nv <= 4) hipLaunchKernelGGL((softmax_vec_kernel<4, NT>), grid, block, 0, p.stream, p.work, p.S, p.causal);
    else if (nv <= 8) hipLaunchKernelGGL((softmax_vec_kernel<8, NT>), grid, block, 0, p.stream, p.work, p.S, p.causal);
    else if (nv <= 16)
      hipLaunchKernelGGL((softmax_vec_kernel<16, NT>), grid, block, 0, p.stream, p.work, p.S, p.causal);
    else hipLaunchKernelGGL((softmax_vec_kernel<32, NT>), grid, block, 0, p.stream, p.work, p.S, p.causal);
  } else {
    hipLaunchKernelGGL(softmax_any_kernel, grid, block, 0, p.stream, p.work, p.S, p.causal);
  }
  return hipGetLastError();
}

hipError_t launch_softmax(const kb_problem &p) {
  return streaming_scores(p) ? launch_softmax_nt<true>(p) : launch_softmax_nt<false>(p);
}

template <int D>
hipError_t launch_pv(const kb_problem &p) {
  const dim3 grid((p.S + 127) / 128, p.bh);
  const bool vec = p.S % 4 == 0;
  if (p.bf16) {
    if (vec)
      hipLaunchKernelGGL((pv_bf16_kernel<D, true>), grid, dim3(kThreads), 0, p.stream, p.work,
                         (const bf16_t *)p.V, p.O, p.out_bf16, p.S);
    else
      hipLaunchKernelGGL((pv_bf16_kernel<D, false>), grid, dim3(kThreads), 0, p.stream, p.work,
                         (const bf16_t *)p.V, p.O, p.out_bf16, p.S);
  } else {
    if (vec)
      hipLaunchKernelGGL((pv_f32_kernel<D, true>), grid, dim3(kThreads), 0, p.stream, p.work,
                         (const float *)p.V, p.O, p.out_bf16, p.S);
    else
      hipLaunchKernelGGL((pv_f32_kernel<D, false>), grid, dim3(kThreads), 0, p.stream, p.work,
                         (const float *)p.V, p.O, p.out_bf16, p.S);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_all(const kb_problem &p) {
  hipError_t e = launch_scores<D>(p);
  if (e != hipSuccess) return e;
  e = launch_softmax(p);
  if (e != hipSuccess) return e;
  return launch_pv<D>(p);
}

}  // namespace

hipError_t kb_launch_naive(const kb_problem &p) {
  switch (p.D) {
    case 32: return launch_all<32>(p);
    case 64: return launch_all<64>(p);
    case 128: return launch_all<128>(p);
    default: return hipErrorInvalidValue;
  }
}
