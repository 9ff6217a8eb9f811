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
#include <type_traits>

#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kThreads = 256;
constexpr int kBr = 128;  // queries per workgroup (fp32 kernel)
// Growth of a row maximum (log2 units) tolerated before rescaling.
constexpr float kRescaleLog2 = 8.0f;
constexpr int kXcds = 8;
// s_waitcnt immediate for "vmcnt(0)" with the other counters left alone
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm0 = 0x0F70;

#define KB_INLINE __attribute__((always_inline))
typedef __attribute__((address_space(3))) bf16_t lds_bf16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;  // MI355X: workgroups are dealt round-robin to 8 XCDs

// Workgroup -> (slice, query tile).  The 1-D grid is padded to a multiple of
// the XCD count; block L runs on XCD L % 8, so it is given item
// (L % 8) * per + L / 8 of the (slice-major, query-tile-minor) work list.
// Each XCD thus owns a contiguous run of slices and works through them one
// at a time, keeping that slice's K/V hot in its own L2.  Causal: inside a
// slice the heaviest (last) query tiles come first.  Returns false for the
// padding blocks.
__device__ __forceinline__ bool tile_of_block(int &bh, int &qt, int nbh, int nqt, bool causal) {
  const int total = nbh * nqt;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int item = (L % kXcds) * per + L / kXcds;
  if (item >= total) return false;
  bh = item / nqt;
  const int t = item % nqt;
  qt = causal ? nqt - 1 - t : t;
  return true;
}

// ------------------------------------------------------------------ bf16 ---
// LDS tile layout (bf16): BC rows of D elements, no padding, the 16-byte
// chunks of each row permuted by an XOR with a per-row value.  Tiles are
// filled by direct global->LDS loads, where lane l of a wave always writes
// bytes [16 l, 16 l + 16) of the wave's 1 KiB destination, so padding is not
// available; the XOR keeps both read patterns free of bank conflicts:
//   K (16 lanes read chunk c of 16 consecutive rows): chunk c ^ fk(row)
//   V (32 lanes read 4 rows x 4 chunks, transposing): chunk c ^ fv(row)
template <int D>
struct Swz {
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RP = 256 / (2 * D);     // rows per 256-byte bank span
  __device__ static int fk(int r) { return (r / RP) % CPR; }
  __device__ static int fv(int r) { return D == 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0; }
};

// Workgroup of the bf16 kernel: 4 waves x 32 query rows, two workgroups per
// CU (the two waves sharing a SIMD belong to different workgroups, so their
// matrix-core and vector phases drift apart and overlap).
constexpr int kBrB = 128;

// Pipeline per wave, per 64-key tile t.  LDS holds K(t+1) and V(t); the
// direct loads of K(t+2) and V(t+1) fill the other two buffers and are
// issued in small groups between the MFMAs instead of in one burst.
//   A: the MFMAs of S^T(t+1) = K(t+1) Q^T, interleaved with the VALU work
//      of tile t: row maxima, the rescaling decision and the exponentials;
//   B: O^T += V(t)^T P(t)^T.
// The loop is unrolled by two so every LDS buffer is a distinct object and
// the compiler never waits for loads in flight before an LDS read.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_bf16_kernel(
    const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ V,
    float *__restrict__ O, int S, int nbh, int nqt, float sl2e) {
  constexpr int BC = 64;        // keys per tile
  constexpr int KC = D / 16;    // bf16 MFMA steps along d for S^T
  constexpr int MB = D / 32;    // 32-row blocks of O^T
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int NCH = BC * CPR; // 16-byte chunks per tile
  constexpr int CH = NCH / kThreads;  // direct loads per thread per tile and tensor
  static_assert(CH >= 1 && NCH % kThreads == 0, "tile staging shape");
  using SW = Swz<D>;

  __shared__ __attribute__((aligned(1024))) bf16_t K0s[BC * D], K1s[BC * D];
  __shared__ __attribute__((aligned(1024))) bf16_t V0s[BC * D], V1s[BC * D];

  int bh, qt;
  if (!tile_of_block(bh, qt, nbh, nqt, CAUSAL)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int q0 = qt * kBrB;
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
  float m_run, l_run = 0.f;

  const int kend = CAUSAL ? min(S, q0 + kBrB) : S;
  const int ntiles = (kend + BC - 1) / BC;
  // Tiles this wave computes: causal waves stop after the tile holding
  // their last query (tiles start at multiples of 64, waves at multiples of
  // 32, so every computed tile has a visible key for every lane).
  const int tw = CAUSAL ? min(ntiles, (qw + 31) / BC + 1) : ntiles;
  auto needs_mask = [&](int t) KB_INLINE {
    const int kt0 = t * BC;
    return (kt0 + BC > S) || (CAUSAL && kt0 + BC - 1 > qw);
  };

  // Direct global->LDS loads.  Physical 16-byte slot P of a tile (P = c *
  // 256 + tid, so each wave instruction fills 1 KiB) holds logical chunk
  // (P % CPR) ^ f(row) of row P / CPR.  Rows past the end of the sequence
  // repeat the last row: their scores are masked and their probabilities
  // are exactly 0, so any finite content is harmless.  A tile index past
  // the last tile reloads the last tile into a buffer nobody reads, which
  // keeps the issue code free of branches.
  uint32_t krow[CH], vrow[CH], kcol[CH], vcol8[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int P = c * kThreads + tid, row = P / CPR;
    krow[c] = vrow[c] = (uint32_t)row;
    kcol[c] = (uint32_t)(((P % CPR) ^ SW::fk(row)) * 8);
    vcol8[c] = (uint32_t)(((P % CPR) ^ SW::fv(row)) * 8);
  }
  auto load_chunk = [&](const bf16_t *__restrict__ src, lds_bf16 *dst, int t, int c, bool is_v) KB_INLINE {
    const int kt0 = min(t, ntiles - 1) * BC;
    const int row = min((int)krow[c], S - 1 - kt0);
    const bf16_t *g = src + base + (size_t)kt0 * D + (uint32_t)(row * D) + (is_v ? vcol8[c] : kcol[c]);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)(dst + (c * kThreads + 64 * w) * 8),
                                     16, 0, 0);
  };

  // K fragment (A operand of S^T) of contraction step kc, key row r.
  const int fk0 = SW::fk(l32), fk1 = SW::fk(32 + l32);
  auto kfrag = [&](const lds_bf16 *kb, int half, int kc) KB_INLINE {
    const int lc = 2 * kc + h;
    return half ? *(const lds_bf16x8 *)(kb + (32 + l32) * D + ((lc ^ fk1) * 8))
                : *(const lds_bf16x8 *)(kb + l32 * D + ((lc ^ fk0) * 8));
  };
  // Transposing V reads: within each 16-lane group, lane p fetches 4
  // consecutive d-columns of key row (p / 4); the hardware hands lane i the
  // 4 keys of column i.  Rows read by this lane: 16 cc + tr_row (+8), all
  // congruent to tr_row mod 4, hence one swizzle value.
  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t vcol[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int col = 32 * mb + tr_col;
    vcol[mb] = (uint32_t)(tr_row * D + (((col >> 3) ^ SW::fv(tr_row)) * 8) + (col & 7));
  }
  auto vfrag = [&](const lds_bf16 *vb, int j) KB_INLINE {
    const int mb = j % MB, cc = j / MB;  // cc = 16-key chunk of the tile
    const lds_bf16 *vr = vb + 16 * cc * D + vcol[mb];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)vr);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vr + 8 * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // sc[sb]: S^T of the lane's query against the 32 keys of half sb.
  f32x16 sc[2];
  auto mask_scores = [&](f32x16 *sv, int t) KB_INLINE {
    // Key offsets beyond `lim` are invisible to this lane's query: past the
    // sequence end, or (causal) after the query itself.
    const int lim = (CAUSAL ? min(q, S - 1) : S - 1) - t * BC;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * sb + acc_row(v, h) > lim) sv[sb][v] = -INFINITY;
  };
  auto row_max = [&](const f32x16 *sv) KB_INLINE {
    // The scale is positive, so it commutes with max.
    float a = -INFINITY, b = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      a = fmaxf(a, fmaxf(sv[0][v], sv[0][v + 1]));
      b = fmaxf(b, fmaxf(sv[1][v], sv[1][v + 1]));
    }
    return xor32_max(fmaxf(a, b)) * sl2e;
  };

  // One pipeline step on tile t, with the direct loads of the next tiles
  // (kdst <- K(t+2), vdst <- V(t+1)) spread over it.  On entry sc holds
  // S^T(t), already masked.
  auto step = [&](int t, const lds_bf16 *knext, const lds_bf16 *vcur, lds_bf16 *kdst, lds_bf16 *vdst) KB_INLINE {
    // A: S^T(t+1) MFMAs (K fragments read one contraction step ahead),
    // interleaved with the row maxima, the rescaling decision and the
    // exponentials of tile t, and with the K(t+2) loads.
    f32x16 sn[2] = {f32x16{}, f32x16{}};
    bf16x8 a0 = kfrag(knext, 0, 0), a1 = kfrag(knext, 1, 0);
    auto qk_step = [&](int kc) KB_INLINE {
      bf16x8 n0 = a0, n1 = a1;
      if (kc + 1 < KC) {
        n0 = kfrag(knext, 0, kc + 1);
        n1 = kfrag(knext, 1, kc + 1);
      }
      sn[0] = mfma32x16_bf16(a0, qf[kc], sn[0]);
      sn[1] = mfma32x16_bf16(a1, qf[kc], sn[1]);
      a0 = n0;
      a1 = n1;
    };
    qk_step(0);
    const float mt = row_max(sc);
    // Lazy rescaling: the reference maximum only moves when some row of the
    // wave grows by more than 2^kRescaleLog2; otherwise the probabilities are
    // taken against the stale maximum and stay below that bound.  O and l use
    // the same reference, so O / l is unchanged in exact arithmetic.
    const bool grow = __builtin_amdgcn_ballot_w64(mt > m_run + kRescaleLog2) != 0;
    const float m_use = fmaxf(m_run, grow ? mt : m_run);
    const float alpha = exp2_fast(m_run - m_use);
    m_run = m_use;
    const float nm = -m_use;
    // Rescale before the straight-line block below, so the branch does not
    // split it.
    if (grow) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
    }
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int NST = KC - 1;
    constexpr int EPS = (32 + NST - 1) / NST;  // exponentials per later step
#pragma unroll
    for (int kc = 1; kc < KC; ++kc) {
      qk_step(kc);
      if (kc - 1 < CH) load_chunk(K, kdst, t + 2, kc - 1, false);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int i = (kc - 1) * EPS + e;
        if (i < 32) {
          const int sb = i >> 4, v = i & 15;
          const float p = exp2_fast(fmaf(sc[sb][v], sl2e, nm));
          sc[sb][v] = p;
          ls[i & 3] += p;
        }
      }
      if (kc + 1 < KC) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // next K reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                   // 2 MFMA
      if (kc - 1 < CH) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 direct load
      __builtin_amdgcn_sched_group_barrier(0x002, 3 * EPS, 0);             // fma, exp, add
    }
    // Loads that did not fit between the MFMAs above.
#pragma unroll
    for (int c = KC - 1; c < CH; ++c) load_chunk(K, kdst, t + 2, c, false);
    l_run = l_run * alpha + ((ls[0] + ls[1]) + (ls[2] + ls[3]));

    // B: O^T += V^T P^T per 16-key chunk cc (accumulator slots 8c..8c+7 of
    // key half sb = cc / 2, i.e. keys 16c + {4h..4h+3, 8+4h..8+4h+3}); the
    // V fragments are read one MFMA ahead, the V(t+1) loads spread between.
    bf16x8 pb[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int s = 0; s < 8; ++s) pb[cc][s] = (bf16_t)sc[cc >> 1][8 * (cc & 1) + s];
    bf16x8 va = vfrag(vcur, 0);
    constexpr int NJ = 4 * MB;
    constexpr int JPL = NJ / CH;  // MFMAs per direct load
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      bf16x8 vn = va;
      if (j + 1 < NJ) vn = vfrag(vcur, j + 1);
      oacc[j % MB] = mfma32x16_bf16(va, pb[j / MB], oacc[j % MB]);
      const bool ld = j % JPL == 0;
      if (ld) load_chunk(V, vdst, t + 1, j / JPL, true);
      if (j + 1 < NJ) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // next V reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);                  // MFMA
      if (ld) __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);          // direct load
      va = vn;
    }
    if (t + 1 < tw && needs_mask(t + 1)) mask_scores(sn, t + 1);
    sc[0] = sn[0];
    sc[1] = sn[1];
  };
  // A wave with no tile left to compute still carries its share of the loads.
  auto loads_only = [&](int t, lds_bf16 *kdst, lds_bf16 *vdst) KB_INLINE {
#pragma unroll
    for (int c = 0; c < CH; ++c) load_chunk(K, kdst, t + 2, c, false);
#pragma unroll
    for (int c = 0; c < CH; ++c) load_chunk(V, vdst, t + 1, c, true);
  };

  using T_ = std::integral_constant<bool, true>;
  using F_ = std::integral_constant<bool, false>;
  // Iteration t with buffer parity PH = t & 1: LDS holds K(t+1) in
  // K-buffer !PH and V(t) in V-buffer PH; K(t+2) goes to K-buffer PH (its
  // K(t) was consumed by the previous iteration) and V(t+1) to V-buffer !PH
  // (its V(t-1) likewise).
  auto iteration = [&](auto ph_tag, int t) KB_INLINE {
    constexpr bool PH = decltype(ph_tag)::value;
    lds_bf16 *kfree = (lds_bf16 *)(PH ? K1s : K0s);
    lds_bf16 *knext = (lds_bf16 *)(PH ? K0s : K1s);
    lds_bf16 *vcur = (lds_bf16 *)(PH ? V1s : V0s);
    lds_bf16 *vfree = (lds_bf16 *)(PH ? V0s : V1s);
    if (t < tw) step(t, knext, vcur, kfree, vfree);
    else loads_only(t, kfree, vfree);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };

  // Prologue: K(0), V(0), K(1); S^T(0) and its maxima, which initialise the
  // reference maxima.
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    load_chunk(K, (lds_bf16 *)K0s, 0, c, false);
    load_chunk(V, (lds_bf16 *)V0s, 0, c, true);
    load_chunk(K, (lds_bf16 *)K1s, 1, c, false);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  sc[0] = sc[1] = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const bf16x8 a0 = kfrag((lds_bf16 *)K0s, 0, kc), a1 = kfrag((lds_bf16 *)K0s, 1, kc);
    sc[0] = mfma32x16_bf16(a0, qf[kc], sc[0]);
    sc[1] = mfma32x16_bf16(a1, qf[kc], sc[1]);
  }
  if (needs_mask(0)) mask_scores(sc, 0);
  m_run = row_max(sc);
  // Iteration 0 refills K-buffer 0, which every wave has just read.
  __syncthreads();

  for (int t = 0; t < ntiles; t += 2) {
    iteration(F_{}, t);
    if (t + 1 < ntiles) iteration(T_{}, t + 1);
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
                                                             float *__restrict__ O, int S, int nbh,
                                                             int nqt, float sl2e) {
  constexpr int BC = 32;
  constexpr int STR = D + 4;  // 16-byte aligned rows, 4-bank shift per row
  constexpr int G = D / 8;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 4;
  constexpr int CH = BC * CPR / kThreads;
  static_assert(CH >= 1 && BC * CPR % kThreads == 0, "tile staging shape");

  __shared__ __attribute__((aligned(16))) float Ks[2][BC * STR];
  __shared__ __attribute__((aligned(16))) float Vs[2][BC * STR];

  int bh, qt;
  if (!tile_of_block(bh, qt, nbh, nqt, CAUSAL)) return;
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
  const int br = p.bf16 ? kBrB : kBr;
  const int nqt = (p.S + br - 1) / br;
  const long long total = (long long)p.bh * nqt;
  if (total > 0x7fffffffLL - kXcds) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + kXcds - 1) / kXcds * kXcds));
  const float sl2e = p.scale * kLog2e;
  if (p.bf16)
    hipLaunchKernelGGL((flash_bf16_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, p.stream,
                       (const bf16_t *)p.Q, (const bf16_t *)p.K, (const bf16_t *)p.V, p.O, p.S, p.bh,
                       nqt, sl2e);
  else
    hipLaunchKernelGGL((flash_f32_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, p.stream,
                       (const float *)p.Q, (const float *)p.K, (const float *)p.V, p.O, p.S, p.bh,
                       nqt, sl2e);
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
