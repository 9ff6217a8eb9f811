// attn_flash: tiled attention forward with an online softmax, for gfx950.
//
// Method (kbench page, "The three GPU kernels", the flash kernel): keys and
// values are streamed in tiles; each query row keeps a running maximum m and
// a running denominator l, earlier partial sums are rescaled by
// 2^(m_old - m_new) whenever the maximum grows, and the S x S score matrix is
// never stored.  On-chip memory per workgroup is O(tile * d), independent of
// the sequence length.
//
// gfx950 design (not the page's scalar design):
//  * A workgroup is 4 waves; each wave owns 32 query rows, so a workgroup
//    covers 128 queries of one (batch, head) slice.
//  * Both contractions run on MFMA 32x32 tiles, computed transposed:
//      S^T = K Q^T   (A = K tile from LDS, B = Q^T kept in VGPRs)
//      O^T += V^T P^T (A = V^T read from LDS with the transposing ds_read,
//                      B = P^T straight from the S^T accumulator registers)
//    With this orientation every lane owns ONE query row (lane % 32) and
//    holds 16 keys of it per 32-key block, so the row max / row sum are
//    in-lane plus one exchange with lane ^ 32, and the rescale factor of
//    O^T is a per-lane scalar.
//  * bf16 inputs: bf16 MFMA (32x32x16), fp32 accumulate, the probabilities
//    rounded to bf16 (round to nearest even) for P V.  fp32 inputs: fp32
//    MFMA (32x32x2) and fp32 probabilities throughout.
//  * The logit scale is applied in fp32 to the fp32 dot products, folded
//    with log2(e) so that one v_exp_f32 (2^x) gives the exponential.
//  * K/V tiles are double-buffered in LDS: the global loads of tile t+1 are
//    issued before tile t is computed and written to the other buffer after.
//  * Causal: a workgroup stops at the last key tile its queries can see, a
//    wave skips the tiles entirely above its rows, and only tiles that cross
//    the diagonal (or the ragged end of the sequence) evaluate the mask.
//    Heavy (late) query tiles are dispatched first, and blockIdx.x is the
//    (batch, head) slice, so with round-robin dispatch over the 8 XCDs all
//    query tiles of a slice share one XCD's L2.
#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kThreads = 256;
constexpr int kBr = 128;  // queries per workgroup

// ------------------------------------------------------------------ bf16 ---
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_bf16_kernel(const bf16_t *__restrict__ Q,
                                                              const bf16_t *__restrict__ K,
                                                              const bf16_t *__restrict__ V,
                                                              float *__restrict__ O, int S,
                                                              int nqt, float sl2e) {
  constexpr int BC = 64;        // keys per tile
  constexpr int STR = D + 8;    // LDS row stride (elements): 16-byte pad per row
  constexpr int KC = D / 16;    // bf16 MFMA steps along d for S^T
  constexpr int MB = D / 32;    // 32-row blocks of O^T
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int CH = BC * CPR / kThreads;
  static_assert(CH >= 1 && BC * CPR % kThreads == 0, "tile staging shape");

  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][BC * STR];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][BC * STR];

  const int bh = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int q0 = qt * kBr;
  const int qw = q0 + 32 * w;
  const int q = qw + l32;
  const size_t base = (size_t)bh * S * D;

  bf16x8 qf[KC];
  {
    const bf16_t *qp = Q + base + (size_t)min(q, S - 1) * D + 8 * h;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const bf16x8 *)(qp + 16 * kc);
  }

  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = CAUSAL ? min(S, q0 + kBr) : S;
  const int ntiles = (kend + BC - 1) / BC;

  u32x4 kreg[CH], vreg[CH];
  auto gload = [&](int t) {
    const int kt0 = t * BC;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 8;
      const int key = kt0 + row;
      if (key < S) {
        const size_t off = base + (size_t)key * D + col;
        kreg[c] = *(const u32x4 *)(K + off);
        vreg[c] = *(const u32x4 *)(V + off);
      } else {
        kreg[c] = u32x4{0, 0, 0, 0};
        vreg[c] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 8;
      *(u32x4 *)&Ks[buf][row * STR + col] = kreg[c];
      *(u32x4 *)&Vs[buf][row * STR + col] = vreg[c];
    }
  };

  // Per-lane offsets of the transposing V reads: within each 16-lane group,
  // lane p fetches 4 consecutive d-columns of key row (p / 4); the hardware
  // hands lane i the 4 keys of column i.
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int kt0 = t * BC;
    if (!CAUSAL || kt0 <= qw + 31) {
      // S^T for the two 32-key halves of the tile.
      f32x16 sacc[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        sacc[sb] = f32x16{};
        const bf16_t *kp = &Ks[buf][(32 * sb + l32) * STR + 8 * h];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          sacc[sb] = mfma32x16_bf16(*(const bf16x8 *)(kp + 16 * kc), qf[kc], sacc[sb]);
      }
      const bool need_mask = (kt0 + BC > S) || (CAUSAL && kt0 + BC - 1 > qw);
      float mt = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[sb][v] * sl2e;
          if (need_mask) {
            const int key = kt0 + 32 * sb + acc_row(v, h);
            if (key >= S || (CAUSAL && key > q)) x = -INFINITY;
          }
          sacc[sb][v] = x;
          mt = fmaxf(mt, x);
        }
      mt = xor32_max(mt);
      // Every processed tile holds a visible key for every lane of an active
      // wave (tiles start at multiples of 64, waves at multiples of 32), so
      // m_new is finite and 2^(m_run - m_new) is 0 on the first tile.
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      float ls = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = exp2_fast(sacc[sb][v] - m_new);
          sacc[sb][v] = p;
          ls += p;
        }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;

      // O^T += V^T P^T, one 16-key chunk at a time.  Chunk c of half sb
      // is accumulator slots 8c..8c+7, i.e. keys 16c + {4h..4h+3, 8+4h..8+4h+3}.
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          bf16x8 pb;
#pragma unroll
          for (int s = 0; s < 8; ++s) pb[s] = (bf16_t)sacc[sb][8 * c + s];
          const bf16_t *vp = &Vs[buf][(32 * sb + 16 * c + tr_row) * STR + tr_col];
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
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.f / xor32_sum(l_run);
  if (q < S) {
    float *op = O + base + (size_t)q * D + 4 * h;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 o4 = {oacc[mb][4 * r] * inv, oacc[mb][4 * r + 1] * inv,
                          oacc[mb][4 * r + 2] * inv, oacc[mb][4 * r + 3] * inv};
        *(f32x4 *)(op + 32 * mb + 8 * r) = o4;
      }
  }
}

// ------------------------------------------------------------------- fp32 ---
// Same structure with 32-key tiles and the fp32 MFMA (contraction 2 per
// instruction).  The contraction index is permuted consistently on both
// operands: step (g, e) uses d-columns 8g + 4h + e from lane half h, so each
// lane reads 16-byte vectors.  P^T slot c of a lane is key acc_row(c, h).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void flash_f32_kernel(const float *__restrict__ Q,
                                                             const float *__restrict__ K,
                                                             const float *__restrict__ V,
                                                             float *__restrict__ O, int S, int nqt,
                                                             float sl2e) {
  constexpr int BC = 32;
  constexpr int STR = D + 4;  // 16-byte aligned rows, 4-bank shift per row
  constexpr int G = D / 8;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 4;
  constexpr int CH = BC * CPR / kThreads;
  static_assert(CH >= 1 && BC * CPR % kThreads == 0, "tile staging shape");

  __shared__ __attribute__((aligned(16))) float Ks[2][BC * STR];
  __shared__ __attribute__((aligned(16))) float Vs[2][BC * STR];

  const int bh = blockIdx.x;
  const int qt = CAUSAL ? (nqt - 1 - (int)blockIdx.y) : (int)blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int q0 = qt * kBr;
  const int qw = q0 + 32 * w;
  const int q = qw + l32;
  const size_t base = (size_t)bh * S * D;

  f32x4 qf[G];
  {
    const float *qp = Q + base + (size_t)min(q, S - 1) * D + 4 * h;
#pragma unroll
    for (int g = 0; g < G; ++g) qf[g] = *(const f32x4 *)(qp + 8 * g);
  }
  f32x16 oacc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int kend = CAUSAL ? min(S, q0 + kBr) : S;
  const int ntiles = (kend + BC - 1) / BC;

  f32x4 kreg[CH], vreg[CH];
  auto gload = [&](int t) {
    const int kt0 = t * BC;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 4;
      const int key = kt0 + row;
      if (key < S) {
        const size_t off = base + (size_t)key * D + col;
        kreg[c] = *(const f32x4 *)(K + off);
        vreg[c] = *(const f32x4 *)(V + off);
      } else {
        kreg[c] = f32x4{};
        vreg[c] = f32x4{};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int idx = tid + c * kThreads;
      const int row = idx / CPR, col = (idx % CPR) * 4;
      *(f32x4 *)&Ks[buf][row * STR + col] = kreg[c];
      *(f32x4 *)&Vs[buf][row * STR + col] = vreg[c];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int kt0 = t * BC;
    if (!CAUSAL || kt0 <= qw + 31) {
      f32x16 sacc = f32x16{};
      const float *kp = &Ks[buf][l32 * STR + 4 * h];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const f32x4 a = *(const f32x4 *)(kp + 8 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc = mfma32x2_f32(a[e], qf[g][e], sacc);
      }
      const bool need_mask = (kt0 + BC > S) || (CAUSAL && kt0 + BC - 1 > qw);
      float mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = sacc[v] * sl2e;
        if (need_mask) {
          const int key = kt0 + acc_row(v, h);
          if (key >= S || (CAUSAL && key > q)) x = -INFINITY;
        }
        sacc[v] = x;
        mt = fmaxf(mt, x);
      }
      mt = xor32_max(mt);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2_fast(m_run - m_new);
      m_run = m_new;
      float ls = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2_fast(sacc[v] - m_new);
        sacc[v] = p;
        ls += p;
      }
      l_run = l_run * alpha + ls;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float *vp = &Vs[buf][acc_row(c, h) * STR + l32];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] = mfma32x2_f32(vp[32 * mb], sacc[c], oacc[mb]);
      }
    }
    if (t + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.f / xor32_sum(l_run);
  if (q < S) {
    float *op = O + base + (size_t)q * D + 4 * h;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 o4 = {oacc[mb][4 * r] * inv, oacc[mb][4 * r + 1] * inv,
                          oacc[mb][4 * r + 2] * inv, oacc[mb][4 * r + 3] * inv};
        *(f32x4 *)(op + 32 * mb + 8 * r) = o4;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_d(const kb_problem &p) {
  const int nqt = (p.S + kBr - 1) / kBr;
  const dim3 grid(p.bh, nqt);
  const float sl2e = p.scale * kLog2e;
  if (p.bf16)
    hipLaunchKernelGGL((flash_bf16_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, p.stream,
                       (const bf16_t *)p.Q, (const bf16_t *)p.K, (const bf16_t *)p.V, p.O, p.S, nqt,
                       sl2e);
  else
    hipLaunchKernelGGL((flash_f32_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, p.stream,
                       (const float *)p.Q, (const float *)p.K, (const float *)p.V, p.O, p.S, nqt,
                       sl2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_c(const kb_problem &p) {
  return p.causal ? launch_d<D, true>(p) : launch_d<D, false>(p);
}

}  // namespace

hipError_t kb_launch_flash(const kb_problem &p) {
  switch (p.D) {
    case 32: return launch_c<32>(p);
    case 64: return launch_c<64>(p);
    case 128: return launch_c<128>(p);
    default: return hipErrorInvalidValue;
  }
}
