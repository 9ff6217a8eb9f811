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
//  * bf16: each wave owns 32 query rows; a workgroup is 8 waves (256 queries
//    of one (batch, head) slice), two per SIMD, alone on its CU, or 4 waves
//    (128 queries) when 256-query items would leave CUs idle.  fp32: when
//    128-query workgroups would leave CUs idle, a workgroup is several waves
//    on one block of 16 queries, each wave taking a part of the keys, the
//    partial results merged through LDS (so even small problems fill the
//    chip); otherwise 4 waves of 32 queries share K/V tiles in LDS.
//  * Both contractions run on MFMA tiles (bf16 32x32, fp32 16x16 or 32x32),
//    computed transposed:
//      S^T = K Q^T   (A = K tile from LDS, B = Q^T kept in VGPRs)
//      O^T += V^T P^T (A = V^T read from LDS with the transposing ds_read,
//                      B = P^T straight from the S^T accumulator registers)
//    With this orientation every lane owns ONE query row (lane % 32) and
//    holds 16 keys of it per 32-key block, so the row max / row sum are
//    in-lane plus one exchange with lane ^ 32, and the rescale factor of
//    O^T is a per-lane scalar.
//  * bf16 inputs: bf16 MFMA (32x32x16), fp32 accumulate, the probabilities
//    rounded to bf16 (round to nearest even) for P V.  fp32 inputs: fp32
//    MFMA (16x16x4 or 32x32x2) and fp32 probabilities throughout.
//  * The logit scale is applied in fp32 to the fp32 dot products, folded
//    with log2(e) so that one v_exp_f32 (2^x) gives the exponential.  (It is
//    not folded into Q: rounding the scaled Q to bf16 errs in proportion to
//    the logits, several times the bf16 tolerance at large logits.)
//  * bf16: K/V tiles go global->LDS by direct loads into a 4-stage ring, and
//    a persistent grid walks an XCD-aware list of query tiles.  The row sums
//    are taken by sparse MFMAs from the bf16 probabilities, which keeps an
//    add per score off the vector ALU.
//    fp32, key-split: each wave reads its K/V blocks straight from global
//    memory into MFMA operand registers (no tile is shared between its
//    waves); fp32, tiles: K/V tiles double-buffered in LDS through
//    registers.  Both on a dispatched grid.
//  * O and l share a reference m that need not be the running maximum (O / l
//    does not depend on it in exact arithmetic).  bf16: the first tile
//    takes the exact row maximum (the reference starts a fixed margin above
//    it), and, non-causal, so does the last; the others
//    (a causal wave's diagonal tile among them, masked first) take none
//    and check the sum of their probabilities instead, correcting the tile
//    in place (or, if the exponentials overflowed, recomputing the query
//    tile exactly) when the reference proves stale.
//  * Causal: a workgroup stops at the last key tile its queries can see, a
//    wave skips the tiles entirely above its rows, and only tiles that cross
//    the diagonal (or the ragged end of the sequence) evaluate the mask.
//    The query tiles of a (batch, head) slice all run on one XCD, so they
//    share its L2; causal work is balanced by pairing heavy and light query
//    tiles (bf16) or by dispatching heavy tiles first (fp32).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kb_device.hpp"

using namespace kb;

namespace {

constexpr int kThreads = 256;
// Growth of a row maximum (log2 units) tolerated before rescaling.
constexpr float kRescaleLog2 = 8.0f;
// Largest per-lane sum of a steady tile's probabilities, taken against the
// current reference without a row maximum, accepted without redoing the
// tile exactly; every accepted probability is then at most this.
constexpr float kSpecLimit = 4096.0f;
// The fast pass starts each row's reference this many log2 units above the
// exact maximum of its first tile.  Every probability then carries a common
// factor 2^-64, which O and l share: O / l is unchanged, and bf16 and fp32
// keep the same relative precision at that scale.  Probabilities below
// 2^-62 of the row's largest fall under the fp32 normal range and come out
// as zero or denormal; at S = 32768 they sum to under 2^-47 of l, so O / l
// moves by less than 2^-46 of the largest |v|.  The margin leaves headroom for later tiles whose scores
// outgrow the first tile's: a steady tile fails its sum check only once a
// row's scores exceed the first tile's maximum by 71 log2 units or more (7
// without the margin), so rows of large logits (a standard deviation of 8,
// about 11.5 log2 units) take no in-place corrections.
constexpr float kRefMargin = 64.0f;
constexpr int kXcds = 8;
// s_waitcnt immediate for "vmcnt(0)" with the other counters left alone
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm0 = 0x0F70;

#define KB_INLINE __attribute__((always_inline))
typedef __attribute__((address_space(3))) bf16_t lds_bf16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Workgroup -> (slice, query tile).  Block L runs on XCD L % 8 (workgroups
// are dealt round-robin to the XCDs) as that XCD's k-th workgroup, k = L / 8.
// XCD x owns the slices [x HP, min(nbh, (x + 1) HP)), HP = ceil(nbh / 8),
// so every slice's K/V stays in one XCD's L2.  Non-causal: its k-th item
// is query tile k % nqt of its slice k / nqt (one slice at a time).  Causal:
// tiles cost work proportional to their index, so the XCD's list runs from
// the heaviest query tile of each of its slices down to the lightest
// (longest-processing-time-first order), and the CUs that finish early take
// the light tiles at the end instead of starting a heavy one late.  Returns
// false for the padding blocks.
__device__ __forceinline__ bool tile_of_block(int &bh, int &qt, int nbh, int nqt, bool causal) {
  const int hp = (nbh + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int x = L % kXcds, k = L / kXcds;
  const int h0 = x * hp;
  const int hx = min(nbh - h0, hp);  // slices of this XCD (may be <= 0)
  if (hx <= 0 || k >= hx * nqt) return false;
  if (causal) {
    bh = h0 + k % hx;
    qt = nqt - 1 - k / hx;
  } else {
    bh = h0 + k / nqt;
    qt = k % nqt;
  }
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

// Workgroup barrier without the memory fence of __syncthreads, which on
// gfx9 also waits for every outstanding global load, prefetches of later
// tiles included.  Ordering is explicit instead: LDS reads are drained here
// (lgkmcnt(0)), direct global->LDS loads are waited for with vmcnt before
// the call, and the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt / expcnt untouched
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Makes `x` depend on `dep` without emitting code: the compiler must
// produce `dep` first.  Used to keep a register set's new contents from
// being computed while its old contents are still being read (which would
// need a second set of registers).
template <typename T, typename U>
__device__ __forceinline__ void after(T &x, const U &dep) {
  asm volatile("" : "+v"(x) : "v"(dep));
}

// Pins a value in place in the instruction stream (no code): the compiler
// must compute it before this point and may not move its later uses above.
template <typename T>
__device__ __forceinline__ void pin(T &x) {
  asm volatile("" : "+v"(x));
}

// bf16 kernel.  A workgroup is NW = 8 waves, two per SIMD, each owning 32
// query rows, so it covers 256 queries of one head; its LDS ring (128 KiB at
// d = 128) keeps it alone on its CU, and every K/V tile staged there feeds
// 256 queries.  While one wave of a SIMD waits at a barrier or on an LDS
// read, the other keeps the matrix core busy.  Problems with fewer 256-query
// work units than CUs take NW = 4 (128 queries per item, twice the units):
// the same code, each K/V tile feeding half as many queries, on twice as
// many CUs (two such workgroups share a CU where their rings fit in LDS).
// Per 64-key tile step t a wave has three pieces of work:
//   O^T += V(t-1)^T P(t-1)^T    (MFMA, V from LDS, P from registers)
//   softmax of tile t           (vector ALU: exponentials, bf16 P; a row
//                                max only on the first tile and, non-causal,
//                                the last; the first step has no P V yet)
//   S^T(t+1) = K(t+1) Q^T       (MFMA, K from LDS)
// and its instruction stream interleaves them, so the vector ALU works in
// the shadow of the matrix core (a wave keeps issuing independent
// instructions while an MFMA runs).  At d = 128 scores live in one set of
// registers: the MFMAs of P(t-1) V(t-1) read each P block before the
// softmax overwrites it, and the score MFMAs of each 32-key half of t+1
// start once the softmax has consumed that half.  At d <= 64, where a step
// has half the products for the same vector work, consecutive tiles' scores
// alternate between two register sets and the softmax spreads over the
// whole step.  When the softmax of t moves the reference maximum, O is
// rescaled after P(t-1) V(t-1) is in.
//
// LDS: rings of kStages K tiles and kStages V tiles filled by direct
// global->LDS loads; step t issues K(t+4) and V(t+2), and waits (before its
// barrier) for the loads of step t-2, which hold K(t+2) and V(t).
constexpr int kStages = 4;

// s_waitcnt immediate for vmcnt(n), n < 64, other counters left alone.
constexpr int wait_vm_imm(int n) { return kWaitVm0 | (n & 15) | ((n >> 4) << 14); }
// ... and lgkmcnt(l), l < 16, as well.
constexpr int wait_vm_lgkm_imm(int n, int l) { return (wait_vm_imm(n) & ~0x0F00) | ((l & 15) << 8); }
// Operand fragments each wave reads ahead of its MFMAs.
constexpr int kPre = 4;

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_bf16_kernel(
    const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ V,
    void *__restrict__ O, int out_bf16, int S, int nbh, int nqt, float sl2e) {
  constexpr int BC = 64;                 // keys per tile
  constexpr int KC = D / 16;             // bf16 MFMA steps along d for S^T
  constexpr int MB = D / 32;             // 32-row blocks of O^T
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int BR = 32 * NW;            // queries per item (32 per wave)
  constexpr int NI = BC * CPR / 64;      // 1 KiB direct-load instructions per tile
  constexpr int CHW = (NI + NW - 1) / NW;  // of which each wave issues (or none)
  constexpr int NPV = 4 * MB;            // MFMAs of P V per tile
  constexpr int TB = 2 * BC * D;         // bytes per tile
  static_assert(CHW >= 1, "tile staging shape");
  using SW = Swz<D>;

  // The LDS ring: kStages K tiles, then kStages V tiles, each BC x D.
  __shared__ __attribute__((aligned(TB))) bf16_t ring[2 * kStages * BC * D];
  __shared__ int redo_flag;
  // d <= 64, 8 waves: each wave's 32 query rows staged in LDS (laid out like
  // the first 32 rows of a K tile), so that Q is read from memory in whole
  // rows rather than in the 16-byte pieces each lane's fragments take.
  constexpr bool kQLds = D <= 64 && NW == 8;
  __shared__ __attribute__((aligned(16))) bf16_t qring[kQLds ? NW * 32 * D : 8];
  auto kst = [&](int j) KB_INLINE { return (lds_bf16 *)(ring + j * BC * D); };
  auto vst = [&](int j) KB_INLINE { return (lds_bf16 *)(ring + (kStages + j) * BC * D); };

  // Persistent schedule: the grid holds kXcds * nw workgroups (one per CU;
  // 4-wave workgroups two per CU where both LDS rings fit).
  // Workgroup g runs on XCD x = g % 8 (workgroups are dealt round-robin to
  // the XCDs) as its j-th workgroup, j = g / 8.  XCD x owns the slices
  // [x hp, min(nbh, (x + 1) hp)), hp = ceil(nbh / 8), so each slice's K/V
  // stays in one XCD's L2, and its workgroups take the XCD's work units
  // j, j + nw, j + 2 nw, ... (slice-major, so the units in flight share few
  // slices).  Non-causal, a unit is one query tile.  Causal, query tile t
  // costs work in proportion to t + 1, so a unit is the pair of tiles
  // (nqt - 1 - u, u) of one slice (the single middle tile when nqt is odd):
  // every unit then costs the same and the CUs finish together.
  const int nw = gridDim.x / kXcds, xcd = blockIdx.x % kXcds, jw = blockIdx.x / kXcds;
  const int hp = (nbh + kXcds - 1) / kXcds, h0 = xcd * hp, hx = min(nbh - h0, hp);
  const int upd = CAUSAL ? (nqt + 1) / 2 : nqt;  // units per slice
  bool first_item = true;
  // One query tile of one slice; every wave of the workgroup calls it with
  // the same arguments.
  auto one_item = [&](const int bh, const int qt) KB_INLINE {
    // The LDS ring of the previous item must be drained by every wave.
    if (!first_item) wg_barrier();
    first_item = false;
    // The wave index is made visibly wave-uniform, so branches on the
    // wave's tile range stay scalar.
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int q0 = qt * BR;
    const int qw = q0 + 32 * w;
    const int q = qw + l32;
    const size_t base = (size_t)bh * S * D;

    bf16x8 qf[KC];
    if constexpr (kQLds) {
      // The wave's rows qw .. qw + 31 are one contiguous block; instruction
      // c, lane l fills 16-byte slot P = 64 c + l of the wave's LDS block
      // with chunk (P % CPR) ^ fk(row) of row P / CPR.  Rows past the
      // sequence end are outside the buffer descriptor and read as zeros.
      // Waited for (vmcnt) before the prologue's barrier.
      const uint64_t qa = (uint64_t)(uintptr_t)(Q + base + (size_t)min(qw, S) * D);
      u32x4 rq;
      rq.x = __builtin_amdgcn_readfirstlane((uint32_t)qa);
      rq.y = __builtin_amdgcn_readfirstlane((uint32_t)(qa >> 32) & 0xffffu);
      rq.z = __builtin_amdgcn_readfirstlane((uint32_t)(max(0, min(32, S - qw)) * 2 * D));
      rq.w = __builtin_amdgcn_readfirstlane(0x00020000u);
  #pragma clang diagnostic push
  #pragma clang diagnostic ignored "-Winline-asm"
  #pragma unroll
      for (int c = 0; c < 32 * CPR / 64; ++c) {
        const int P = 64 * c + lane, row = P / CPR;
        const uint32_t off = (uint32_t)(row * 2 * D + (((P % CPR) ^ SW::fk(row)) << 4));
        const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(
            (__attribute__((address_space(3))) bf16_t *)(qring + w * 32 * D + c * 512)));
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(m0), "v"(off), "s"(rq) : "memory", "m0");
      }
  #pragma clang diagnostic pop
    } else {
      const bf16_t *qp = Q + base + (size_t)min(q, S - 1) * D + 8 * h;
  #pragma unroll
      for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const bf16x8 *)(qp + 16 * kc);
    }

    f32x16 oacc[MB];
  #pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    bool inexact = false;  // a steady tile's reference was stale beyond repair
    int pv_lim = 0;        // tiles whose P V the general steps still do

    const int kend = CAUSAL ? min(S, q0 + BR) : S;
    const int ntiles = (kend + BC - 1) / BC;
    // Tiles this wave computes: causal waves stop after the tile holding
    // their last query.  Query blocks start at multiples of 32 and tiles at
    // multiples of 64, so every tile before that one is entirely visible to
    // all 32 queries, and every computed tile has a visible key for each.
    const int tw = CAUSAL ? min(ntiles, (qw + 31) / BC + 1) : ntiles;

    // Direct global->LDS loads (buffer loads with the LDS flag).  Instruction
    // c of a tile fills bytes [1 KiB c, 1 KiB (c + 1)) of the stage; its lane
    // l writes physical 16-byte slot P = 64 c + l, which holds logical chunk
    // (P % CPR) ^ f(row) of row P / CPR.  Wave w issues instructions w, w + NW,
    // ... (at d = 32 a tile is 4 instructions, and with 8 waves waves 4-7
    // issue none).  The
    // lane's byte offset within a tile is fixed (koff / voff) and the tile's
    // offset is a scalar, so a load costs no vector instructions.  The
    // buffer descriptors span this head's K and V exactly: rows past the end
    // of the sequence, and tiles past the last one, read as zeros (their
    // scores are masked and their probabilities are exactly 0).  The loads are
    // issued from inline asm, so their completion is tracked by the explicit
    // waits of the step loop alone.
    uint32_t koff[CHW], voff[CHW];
  #pragma unroll
    for (int i = 0; i < CHW; ++i) {
      const int P = 64 * min(w + NW * i, NI - 1) + lane, row = P / CPR;
      koff[i] = (uint32_t)(row * 2 * D + (((P % CPR) ^ SW::fk(row)) << 4));
      voff[i] = (uint32_t)(row * 2 * D + (((P % CPR) ^ SW::fv(row)) << 4));
    }
    const uint32_t head_bytes = (uint32_t)S * 2u * D;
    auto rsrc = [&](const bf16_t *p) KB_INLINE {
      const uint64_t a = (uint64_t)(uintptr_t)p;
      u32x4 r;
      r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
      r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
      r.z = __builtin_amdgcn_readfirstlane(head_bytes);
      r.w = __builtin_amdgcn_readfirstlane(0x00020000u);  // 32-bit data format, untyped
      return r;
    };
    const u32x4 rk = rsrc(K + base), rv = rsrc(V + base);
    // Scalar byte offset of tile t (past the last tile: out of range).
    auto tile_off = [&](int t) KB_INLINE {
      return (uint32_t)__builtin_amdgcn_readfirstlane(t < ntiles ? (uint32_t)t * BC * 2u * D : head_bytes);
    };
    // Load instruction i (0 <= i < CHW) of tile `t` of K (is_v false) or V.
    // The statements write m0 (the LDS destination of the load), so it is in
    // their clobber list; the compiler then knows m0 changed (it warns that a
    // reserved register is not preserved, which is what is meant here).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    auto dma = [&](bool is_v, int i, lds_bf16 *dst, uint32_t toff) KB_INLINE {
      // Wave w issues instruction w + NW i of the tile; when NI = NW CHW
      // (d >= 64) every wave issues all CHW of them, known at compile time,
      // so the loads of a step carry no branch.
      if (NI < NW * CHW && w + NW * i >= NI) return;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(dst + (w + NW * i) * 512));
      if (is_v)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(m0), "v"(voff[i]), "s"(rv), "s"(toff) : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :: "s"(m0), "v"(koff[i]), "s"(rk), "s"(toff) : "memory", "m0");
    };
#pragma clang diagnostic pop
    auto load_tile = [&](bool is_v, lds_bf16 *dst, int t) KB_INLINE {
      const uint32_t toff = tile_off(t);
  #pragma unroll
      for (int i = 0; i < CHW; ++i) dma(is_v, i, dst, toff);
    };


    // LDS operand offsets within a stage (each term stays below the tile
    // size, and the per-fragment parts are XORs of the swizzled chunk index).
    //  K fragment (A operand of S^T), contraction step kc, key half `half`:
    //    row 32 half + l32, logical chunk 2 kc + h, physical chunk
    //    (2 kc + h) ^ fk(row) (fk is the same for row and row + 32): byte
    //    offset kx[kc] + half * 64 D with kx[kc] = KL ^ (kc << 5).
    //  V^T fragment (A operand of O^T, transposing reads): within each 16-lane
    //    group, lane p fetches 4 consecutive d-columns of key row (p / 4) and
    //    the hardware hands lane i the 4 keys of column i.  This lane reads key
    //    rows 16 cc + tr_row (+8), all congruent to tr_row mod 4 (one swizzle
    //    value fv = 4 g), d-columns 32 mb + tr_col .. +3: byte offset
    //    vx[mb] + 32 D cc (+ 16 D for the upper 8 rows), vx[mb] = VL ^ (mb << 6).
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const uint32_t KL = (uint32_t)(l32 * 2 * D + ((h ^ SW::fk(l32)) << 4));
    const uint32_t VL = (uint32_t)(tr_row * 2 * D + ((SW::fv(tr_row) >> 2) << 6) + ((tr_col >> 3) << 4) +
                                   (tr_col & 7) * 2);
    // Per-lane LDS addresses of the fragments in stage 0 of each ring (kx,
    // vx), made opaque to the compiler: every fragment address is then one
    // of these plus a constant below 64 KiB (stage, key half or 16-key
    // chunk), which the LDS instruction takes as its immediate offset.
    typedef __attribute__((address_space(3))) char lds_char;
    const uint32_t k_ring = (uint32_t)(uintptr_t)(const lds_char *)kst(0);
    const uint32_t v_ring = (uint32_t)(uintptr_t)(const lds_char *)vst(0);
    uint32_t kx[KC], vx[MB];
  #pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      kx[kc] = k_ring + (KL ^ (uint32_t)(kc << 5));
      pin(kx[kc]);
    }
  #pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      vx[mb] = v_ring + (VL ^ (uint32_t)(mb << 6));
      pin(vx[mb]);
    }
    auto kfrag = [&](const lds_bf16 *kb, int half, int kc) KB_INLINE {
      const uint32_t so = (uint32_t)((const lds_char *)kb - (const lds_char *)kst(0));
      return *(const lds_bf16x8 *)((const lds_char *)(uintptr_t)kx[kc] + so + half * 64 * D);
    };
    // V^T fragment j of a tile: 32-row block mb = j % MB, 16-key chunk j / MB.
    auto vfrag = [&](const lds_bf16 *vb, int j) KB_INLINE {
      const int mb = j % MB, cc = j / MB;
      const uint32_t so = (uint32_t)((const lds_char *)vb - (const lds_char *)vst(0));
      const lds_char *a = (const lds_char *)(uintptr_t)vx[mb] + so + cc * 32 * D;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)a);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a + 16 * D));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    // First fragments of a steady step: V^T of the previous tile (kPre <= 4 MB).
    auto fetch_first = [&](const lds_bf16 *vb, const lds_bf16 *kb, int i) KB_INLINE {
      (void)kb;
      return vfrag(vb, i);
    };
    // Operand fragments read ahead of their MFMAs, carried across steps.
    bf16x8 buf[kPre];

    // Scores of a tile: sc[sb] = S^T of the lane's query against the 32 keys
    // of half sb (raw dot products).  Probabilities in bf16: pb[cc] =
    // accumulator slots 8(cc & 1) .. +7 of half cc / 2, i.e. keys
    // 16 cc + {4h..4h+3, 8+4h..8+4h+3} (the B operand layout of P^T).
    // At d <= 64 the fused steps keep the scores of consecutive tiles in two
    // register sets (tile t in scd[(t + 1) & 1]; sc is scd[1], the set the
    // other steps use), so the softmax of tile t and the score products of
    // tile t + 1 need not take turns.
    f32x16 scd[2][2];
    f32x16(&sc)[2] = scd[1];
    bf16x8 pb[4];
    // Row sums by sparse MFMA: v_smfmac_f32_16x16x64_bf16 computes
    // C[m][n] += sum_k A[m][k] B[k][n] over 64 contraction slots, A stored
    // 2:4-compressed (in every group of 4 slots, two values and their 2-bit
    // positions in the index register).  B = two blocks of P (16 values):
    // lane l holds column l % 16, slots 8 g .. 8 g + 7 and 32 + 8 g .. +7
    // (g = l / 16); A lane l holds row l % 16 over slots 16 (l / 16) .. +15
    // (8 stored values, groups of 4 in order, two per group); C lane l holds
    // rows 4 g .. 4 g + 3 of column l % 16 (layouts measured on gfx950).
    // The constant A below puts, in rows 4 g and 4 g + 1, ones on exactly
    // the slots that lane group g of B holds: row 4 g on positions 0 and 1
    // of each group, row 4 g + 1 on positions 2 and 3 (rows 4 g + 2 and
    // 4 g + 3 are zero).  C[0] + C[1] of lane l is then the fp32 sum of
    // the lane's own 16 probabilities; two such products per tile take all
    // 32, half the matrix-pipe time of the four dense 16x16x32 products
    // that would take them one block at a time.
    bf16x8 smf_a;
    int smf_idx;
    {
      const int m = lane & 15, j = lane >> 4, g = m >> 2, r = m & 3;
      const bool row_on = r < 2 && (j == (g >> 1) || j == 2 + (g >> 1));
  #pragma unroll
      for (int e = 0; e < 8; ++e) smf_a[e] = (bf16_t)((row_on && (e >> 2) == (g & 1)) ? 1.0f : 0.0f);
      const unsigned pat = r == 0 ? 0x4444u : 0xEEEEu;
      smf_idx = (int)(pat | (pat << 16));
    }
    auto smf = [&](const bf16x8 &x, const bf16x8 &y, f32x4 c) KB_INLINE {
      return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(
          smf_a, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15), c, smf_idx, 0, 0);
    };

    // Scores of the next tile into sc; each half starts once the
    // probabilities of the old contents (pb[2 half], pb[2 half + 1]) exist.
    auto qk = [&](const lds_bf16 *kb) KB_INLINE {
  #pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        bf16x8 a0 = kfrag(kb, 0, kc), a1 = kfrag(kb, 1, kc);
        if (kc == 0) {
          after(a0, pb[1]);
          after(a1, pb[3]);
        }
        sc[0] = mfma32x16_bf16(a0, qf[kc], kc == 0 ? f32x16{} : sc[0]);
        sc[1] = mfma32x16_bf16(a1, qf[kc], kc == 0 ? f32x16{} : sc[1]);
      }
    };
    auto pv = [&](const lds_bf16 *vb) KB_INLINE {
  #pragma unroll
      for (int j = 0; j < NPV; ++j) oacc[j % MB] = mfma32x16_bf16(vfrag(vb, j), pb[j / MB], oacc[j % MB]);
    };
    // Diagonal / ragged tiles: key offsets beyond `lim` are invisible to this
    // lane's query (past the sequence end, or after the query itself).
    auto mask = [&](int t) KB_INLINE {
      const int kt0 = t * BC;
      if ((kt0 + BC > S) || (CAUSAL && kt0 + BC - 1 > qw)) {
        // Key 32 sb + acc_row(v, h) is c(sb, v) + 4 h, c a constant of 0..63:
        // one per-lane limit, and each score a compare with an inline
        // constant and a select, both through VCC (written out, because the
        // compiler otherwise keeps all 32 compare results, or 32 per-lane
        // key offsets, live across the kernel and spills registers).
        const int lim = (CAUSAL ? min(q, S - 1) : S - 1) - kt0 - 4 * h;
        const float ninf = -INFINITY;
  #pragma unroll
        for (int sb = 0; sb < 2; ++sb)
  #pragma unroll
          for (int v = 0; v < 16; ++v) {
            float x = sc[sb][v];
            asm volatile("v_cmp_lt_i32 vcc, %1, %2\n\tv_cndmask_b32 %0, %0, %3, vcc"
                         : "+v"(x) : "v"(lim), "i"(32 * sb + 8 * (v >> 2) + (v & 3)), "v"(ninf) : "vcc");
            sc[sb][v] = x;
          }
      }
    };
    // Softmax, first part: row max and lazy rescaling.  The row max is taken
    // over the raw dot products (the scale is positive, so it commutes with
    // max), then in log2 units, with three-input max steps.  The reference
    // maximum only moves when some row of the wave grows by more than
    // 2^kRescaleLog2; otherwise the probabilities are taken against the stale
    // maximum and stay below that bound.  O and l use the same reference, so
    // O / l is unchanged in exact arithmetic.  The first tile always moves it
    // (m_run starts at -inf, every row sees a key).  Returns whether it moved;
    // `alpha` is then the factor for O.  `thr` is the tolerated growth
    // (kRescaleLog2, or 0 to move the reference to the maximum).
    auto row_max = [&](float &alpha, float thr) KB_INLINE {
      float a = -INFINITY, b = -INFINITY;
  #pragma unroll
      for (int v = 0; v < 16; v += 2) {
        a = fmaxf(fmaxf(a, sc[0][v]), sc[0][v + 1]);
        b = fmaxf(fmaxf(b, sc[1][v]), sc[1][v + 1]);
      }
      const float mt = xor32_max(fmaxf(a, b)) * sl2e;
      const bool grow = __builtin_amdgcn_ballot_w64(mt > m_run + thr) != 0;
      const float m_new = grow ? fmaxf(m_run, mt) : m_run;
      alpha = exp2_fast(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      return grow;
    };
    // Softmax, second part, for key half sb: exponentials and the bf16
    // probabilities (the P operand of P V).
    auto probs = [&](int sb) KB_INLINE {
      const float nm = -m_run;
  #pragma unroll
      for (int v = 0; v < 16; ++v) sc[sb][v] = exp2_fast(fmaf(sc[sb][v], sl2e, nm));
  #pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int cc = 2 * sb + c2;
  #pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) pb[cc][s2] = (bf16_t)sc[sb][8 * c2 + s2];
      }
    };
    // The lane's share of the row sum l for the current tile: the fp32 sum of
    // its 32 bf16 probabilities, the very weights P V multiplies (so O is
    // divided by exactly the total of the weights it summed), by the sparse
    // row-sum MFMAs described at smf_a.  Every tile takes l this way.
    auto pb_sum = [&]() KB_INLINE {
      f32x4 s4 = smf(pb[0], pb[1], f32x4{});
      s4 = smf(pb[2], pb[3], s4);
      return s4[0] + s4[1];
    };

    // Steady-state step: O += P(t-1) V(t-1), the softmax of t and S^T(t+1) as
    // one instruction stream of NS slots.  Slot i issues the LDS reads of slot
    // i + kPre, MFMA i and its share of the vector work, and the compiler may
    // not move instructions between slots, so the interleave is exactly this:
    //   MFMA slots  [0, NPV)        P V, probability block cc of t-1 in
    //                               slots [cc NPV/4, (cc+1) NPV/4)
    //               [NPV, NPV+KC)   scores of key half 0 of t+1 (kc = 0..KC-1)
    //               [NPV+KC, NS)    scores of key half 1
    //   vector work exponentials and bf16 P of key half 0 of t in slots
    //               [NPV/4, 3 NPV/4), of half 1 in [3 NPV/4, NPV+KC): each
    //               block of P is rewritten after the MFMAs that read its old
    //               contents, and each half of the scores is consumed before
    //               the MFMAs that overwrite it.
    // A steady tile takes no row maximum: its probabilities are taken against
    // the current reference m_run, and the per-lane sum of their bf16 values,
    // which bounds each of them, is returned.  It is taken by two sparse
    // row-sum MFMAs, each issued in the slot after its two probability blocks
    // are complete, so the vector ALU does no add per score.  If some lane's sum exceeds
    // kSpecLimit (or is not a number below it: a reference stale by more
    // than the fp32 exponential can take gives an infinite probability),
    // the caller corrects the tile or redoes the item exactly.
    // The exponentials go two values at a time (two fma, two exp) and the
    // conversion of each pair trails one op behind, so no vector instruction
    // waits on the one just before it.
    auto fused_step = [&](const lds_bf16 *vprev, const lds_bf16 *knext, const lds_bf16 *vnn,
                          const lds_bf16 *knn, auto &&ld, auto prev_tag, auto next_tag) KB_INLINE {
      constexpr bool PREV = decltype(prev_tag)::value, NEXT = decltype(next_tag)::value;
      constexpr int NS = NPV + 2 * KC;
      constexpr int A0 = NPV / 4, B0 = 3 * NPV / 4, E1 = NPV + KC;
      static_assert(NS % kPre == 0 && NPV >= kPre, "fragment ring");
      // Fragment i of this step (i < NS) or of the next one (i >= NS, read
      // from the next step's stages, resident since this step's barrier).
      // Without NEXT (a wave's last tile) the scores of the next tile and
      // the next step's fragments are not needed and not read.
      auto fetch = [&](int i) KB_INLINE {
        if (!NEXT && i >= NPV) return bf16x8{};
        if (!PREV && i < NPV) return bf16x8{};
        if (i >= NS) return fetch_first(vnn, knn, i - NS);
        return i < NPV ? vfrag(vprev, i) : kfrag(knext, (i - NPV) / KC, (i - NPV) % KC);
      };
      const float nm = -m_run;
      f32x4 lsv = f32x4{};
      // bf16 pair p (elements 2p, 2p+1) of half sb -> P.
      auto cvt_pair = [&](int sb, int p) KB_INLINE {
        bf16x2 pr = {(bf16_t)sc[sb][2 * p], (bf16_t)sc[sb][2 * p + 1]};
        pin(pr);
        const int cc = 2 * sb + p / 4, e = p % 4;
        pb[cc][2 * e] = pr[0];
        pb[cc][2 * e + 1] = pr[1];
      };
      // Exponential op p (0..8) of half sb: exponentials of pair p (p < 8),
      // then the conversion of pair p - 1.
      auto exp_op = [&](int sb, int p) KB_INLINE {
        if (p < 8) {
          float x0 = sc[sb][2 * p], x1 = sc[sb][2 * p + 1];
          pin(x0);
          pin(x1);
          x0 = fmaf(x0, sl2e, nm);
          x1 = fmaf(x1, sl2e, nm);
          x0 = exp2_fast(x0);
          x1 = exp2_fast(x1);
          pin(x0);
          pin(x1);
          sc[sb][2 * p] = x0;
          sc[sb][2 * p + 1] = x1;
        }
        if (p > 0) cvt_pair(sb, p - 1);
      };
      // Vector work of slot i: the 9 ops of half 0 spread evenly over
      // [A0, B0), those of half 1 over [B0, E1).
      auto slot_work = [&](int i) KB_INLINE {
        if (i >= A0 && i < B0) {
          const int g = i - A0, n = B0 - A0;
          for (int p = (9 * g) / n; p < (9 * (g + 1)) / n; ++p) exp_op(0, p);
        } else if (i >= B0 && i < E1) {
          const int g = i - B0, n = E1 - B0;
          for (int p = (9 * g) / n; p < (9 * (g + 1)) / n; ++p) exp_op(1, p);
        }
      };
      // Slot of exponential op p of half sb (as slot_work places it), and the
      // slot after the one completing probability block cc.
      constexpr auto op_slot = [](int sb, int p) {
        const int st = sb == 0 ? A0 : B0, n = sb == 0 ? B0 - A0 : E1 - B0;
        for (int g = 0; g < n; ++g)
          if ((9 * g) / n <= p && p < (9 * (g + 1)) / n) return st + g;
        return -1;
      };
      constexpr auto sum_slot = [op_slot](int cc) { return op_slot(cc / 2, 4 * (cc % 2) + 4) + 1; };
      static_assert(sum_slot(3) < NS, "row sums inside the step");
      bf16x8 pbo[4];
  #pragma unroll
      for (int cc = 0; cc < 4; ++cc) pbo[cc] = pb[cc];
  #pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bf16x8 op = buf[i % kPre];
        buf[i % kPre] = fetch(i + kPre);
        if (i < NPV) {
          if constexpr (PREV) oacc[i % MB] = mfma32x16_bf16(op, pbo[i / MB], oacc[i % MB]);
        } else if constexpr (NEXT) {
          const int half = (i - NPV) / KC, kc = (i - NPV) % KC;
          sc[half] = mfma32x16_bf16(op, qf[kc], kc == 0 ? f32x16{} : sc[half]);
        }
        slot_work(i);
        if (i == sum_slot(1)) lsv = smf(pb[0], pb[1], lsv);
        if (i == sum_slot(3)) lsv = smf(pb[2], pb[3], lsv);
        // This step's 2 CHW tile loads, spread evenly over the slots so the
        // CU's load pipeline never backs up into the instruction stream.
        constexpr int LDI = NS / (2 * CHW);
        if (i % LDI == 1 % LDI && i / LDI < 2 * CHW) ld(i / LDI);
        __builtin_amdgcn_sched_barrier(0);
      }
      return lsv[0] + lsv[1];
    };

    // d <= 64: the same step with the scores of tile t in `cur` and those of
    // tile t + 1 written to `nxt`.  The softmax of t no longer has to finish
    // before the score products of t + 1 start, so its 18 exponential ops
    // are dealt evenly over all NS slots (with one set they fit between the
    // P V products that read each old probability block and the score
    // products that overwrite each half, leaving slots with no vector work,
    // where the step is bound by the vector ALU).
    auto fused_step_db = [&](const lds_bf16 *vprev, const lds_bf16 *knext, const lds_bf16 *vnn,
                             const lds_bf16 *knn, auto &&ld, auto prev_tag, auto next_tag, f32x16(&cur)[2],
                             f32x16(&nxt)[2]) KB_INLINE {
      constexpr bool PREV = decltype(prev_tag)::value, NEXT = decltype(next_tag)::value;
      constexpr int NS = NPV + 2 * KC;
      constexpr int NOP = 18;
      static_assert(NS % kPre == 0 && NPV >= kPre, "fragment ring");
      auto fetch = [&](int i) KB_INLINE {
        if (!NEXT && i >= NPV) return bf16x8{};
        if (!PREV && i < NPV) return bf16x8{};
        if (i >= NS) return fetch_first(vnn, knn, i - NS);
        return i < NPV ? vfrag(vprev, i) : kfrag(knext, (i - NPV) / KC, (i - NPV) % KC);
      };
      const float nm = -m_run;
      f32x4 lsv = f32x4{};
      auto cvt_pair = [&](int sb, int p) KB_INLINE {
        bf16x2 pr = {(bf16_t)cur[sb][2 * p], (bf16_t)cur[sb][2 * p + 1]};
        pin(pr);
        const int cc = 2 * sb + p / 4, e = p % 4;
        pb[cc][2 * e] = pr[0];
        pb[cc][2 * e + 1] = pr[1];
      };
      // Op k (0..17) is op k % 9 of half k / 9: the exponentials of pair
      // k % 9 (if below 8), then the conversion of the pair before it.
      auto exp_op = [&](int k) KB_INLINE {
        const int sb = k / 9, p = k % 9;
        if (p < 8) {
          float x0 = cur[sb][2 * p], x1 = cur[sb][2 * p + 1];
          pin(x0);
          pin(x1);
          x0 = fmaf(x0, sl2e, nm);
          x1 = fmaf(x1, sl2e, nm);
          x0 = exp2_fast(x0);
          x1 = exp2_fast(x1);
          pin(x0);
          pin(x1);
          cur[sb][2 * p] = x0;
          cur[sb][2 * p + 1] = x1;
        }
        if (p > 0) cvt_pair(sb, p - 1);
      };
      // Slot i runs ops [NOP i / NS, NOP (i + 1) / NS); the row sum of blocks
      // 0 and 1 follows the slot of op 8, that of blocks 2 and 3 the last.
      constexpr auto op_slot = [](int k) {
        for (int i = 0; i < NS; ++i)
          if ((NOP * i) / NS <= k && k < (NOP * (i + 1)) / NS) return i;
        return -1;
      };
      static_assert(op_slot(NOP - 1) == NS - 1, "ops dealt over every slot");
      bf16x8 pbo[4];
  #pragma unroll
      for (int cc = 0; cc < 4; ++cc) pbo[cc] = pb[cc];
  #pragma unroll
      for (int i = 0; i < NS; ++i) {
        const bf16x8 op = buf[i % kPre];
        buf[i % kPre] = fetch(i + kPre);
        if (i < NPV) {
          if constexpr (PREV) oacc[i % MB] = mfma32x16_bf16(op, pbo[i / MB], oacc[i % MB]);
        } else if constexpr (NEXT) {
          const int half = (i - NPV) / KC, kc = (i - NPV) % KC;
          nxt[half] = mfma32x16_bf16(op, qf[kc], kc == 0 ? f32x16{} : nxt[half]);
        }
        for (int k = (NOP * i) / NS; k < (NOP * (i + 1)) / NS; ++k) exp_op(k);
        if (i == op_slot(8)) lsv = smf(pb[0], pb[1], lsv);
        if (i == NS - 1) lsv = smf(pb[2], pb[3], lsv);
        constexpr int LDI = NS / (2 * CHW);
        if (i % LDI == 1 % LDI && i / LDI < 2 * CHW) ld(i / LDI);
        __builtin_amdgcn_sched_barrier(0);
      }
      return lsv[0] + lsv[1];
    };

    // Correction of a steady tile whose sum check failed.  Every probability
    // of the tile is bf16(2^(x - m_run)); the row's largest one, pmax, shows
    // how far the reference is below the row's maximum.  If pmax is finite,
    // the reference moves up by the integer k with pmax 2^-k < 1, and O, l
    // and the tile's bf16 probabilities are multiplied by 2^-k: exactly, the
    // probabilities by subtracting k from their exponent field (with
    // unsigned saturation: the few whose exponent would drop to zero or
    // below become zero or a denormal, all under 2^-126 against the row's
    // largest, which the moved reference makes < 1).  The tile's sum is then
    // taken again from the corrected probabilities (scaling the old one
    // would keep an fp32 overflow of the sum of finite values).  The result
    // is what the tile would have given against the moved reference.  If
    // pmax is infinite (the reference is stale by more than the fp32
    // exponential can take) the probabilities hold no information; returns
    // false and the item is redone exactly.
    auto spec_fix = [&](float &ls) KB_INLINE {
      u16x2 mx = {0, 0};
  #pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const u32x4 wds = __builtin_bit_cast(u32x4, pb[cc]);
  #pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          // (a bit_cast straight from a vector element would read element 0)
          const uint32_t wv = wds[w4];
          mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, wv));
        }
      }
      const uint32_t m16 = mx.x > mx.y ? mx.x : mx.y;
      // Infinity or NaN (exponent field all ones), tested on the bits.
      if (__builtin_amdgcn_ballot_w64(m16 >= 0x7F80u) != 0) return false;
      const float pmax = xor32_max(__uint_as_float(m16 << 16));
      // pmax < 2^e; k = max(e, 0) <= 128.
      const int k = max((int)(__float_as_uint(pmax) >> 23) - 126, 0);
      const float alpha = __builtin_amdgcn_ldexpf(1.0f, -k);
      const u16x2 sub = {(unsigned short)(k << 7), (unsigned short)(k << 7)};
  #pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        u32x4 wds = __builtin_bit_cast(u32x4, pb[cc]);
  #pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const uint32_t wv = wds[w4];
          wds[w4] = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, wv), sub));
        }
        pb[cc] = __builtin_bit_cast(bf16x8, wds);
      }
      // The tile's sum from the corrected probabilities (each now below 1).
      ls = pb_sum();
      m_run += (float)k;
      l_run *= alpha;
  #pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      return true;
    };


    // Start of step t: wait for this wave's loads of step t-2 (K(t+2), V(t))
    // and earlier, and for its LDS reads except the last 2 kPre
    // instructions (the next step's first fragments, read ahead from stages
    // nobody refills in step t).  The barrier then makes everyone's loads
    // resident and ends step t-1's reads everywhere, freeing K(t) (stage
    // t % 4) and V(t-2) (stage (t + 2) % 4), which are refilled with K(t+4)
    // and V(t+2); K(t+2) and V(t) are now readable, so the end of step t
    // reads the first fragments of step t+1 from them.
    // `drain` (general steps and the first step): wait for every LDS read,
    // since a general step or the prologue before them ends with score
    // products that read the K stage step t refills.
    // `relax`: the wave issued its 4 MB output stores at the end of step
    // t-1 or t-2, after the loads this wait is for.  vmcnt counts loads and
    // stores together and retires them in issue order, so allowing those
    // stores to stay outstanding still leaves the wanted loads complete.
    auto begin_step = [&](int t, bool relax = false, bool drain = false) KB_INLINE {
      if (relax && drain)
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm_imm(2 * CHW + 4 * MB, 0));
      else if (relax)
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm_imm(2 * CHW + 4 * MB, 2 * kPre));
      else if (drain)
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm_imm(2 * CHW, 0));
      else
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm_imm(2 * CHW, 2 * kPre));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    auto rescale = [&](bool grow, float alpha) KB_INLINE {
      if (grow) {
  #pragma unroll
        for (int mb = 0; mb < MB; ++mb) oacc[mb] *= alpha;
      }
    };
    // Steady step (1 <= t < tw - 1) with ST = t % 4, so every LDS buffer it
    // touches is known at compile time.
    auto steady = [&](auto st_tag, int t) KB_INLINE {
      constexpr int ST = decltype(st_tag)::value;
      begin_step(t);
      const uint32_t tk = tile_off(t + 4), tv = tile_off(t + 2);
      auto ld = [&](int k) KB_INLINE {
        if (k < CHW) dma(false, k, kst(ST), tk);
        else dma(true, k - CHW, vst((ST + 2) % kStages), tv);
      };
      float ls;
      if constexpr (D <= 64)
        ls = fused_step_db(vst((ST + 3) % kStages), kst((ST + 1) % kStages), vst(ST), kst((ST + 2) % kStages), ld,
                           std::true_type{}, std::true_type{}, scd[(ST + 1) & 1], scd[ST & 1]);
      else
        ls = fused_step(vst((ST + 3) % kStages), kst((ST + 1) % kStages), vst(ST), kst((ST + 2) % kStages), ld,
                        std::true_type{}, std::true_type{});
      float lsum = ls;
      // The check compares bit patterns (the sum is never negative): it also
      // fails a NaN sum, which the row-sum MFMA gives the lanes that share a
      // column with an infinite probability (its zero weights times
      // infinity), and which a float comparison, compiled here without NaN
      // semantics, could let through.
      if (__builtin_amdgcn_ballot_w64(__float_as_uint(lsum) > __float_as_uint(kSpecLimit)) != 0 && !spec_fix(lsum))
        inexact = true;
      l_run += lsum;
    };
    // Causal: the wave's last tile (its diagonal one) as a fused step, the
    // same instruction stream as a steady step but with its ring stages
    // chosen at run time, the mask applied first and no score products for a
    // next tile; its probabilities are checked by their sum like a steady
    // tile's (every row has a visible key there).  A general step here took
    // twice as long, and every wave of the workgroup waited for it at the
    // next barrier.
    auto steady_last = [&](int t) KB_INLINE {
      const int st = t & 3;
      begin_step(t);
      mask(t);
      const uint32_t tk = tile_off(t + 4), tv = tile_off(t + 2);
      auto ld = [&](int k) KB_INLINE {
        if (k < CHW) dma(false, k, kst(st), tk);
        else dma(true, k - CHW, vst((st + 2) & 3), tv);
      };
      float lsum;
      if constexpr (D <= 64)
        lsum = fused_step_db(vst((st + 3) & 3), kst((st + 1) & 3), vst(st), kst((st + 2) & 3), ld, std::true_type{},
                             std::false_type{}, scd[1], scd[0]);
      else
        lsum = fused_step(vst((st + 3) & 3), kst((st + 1) & 3), vst(st), kst((st + 2) & 3), ld, std::true_type{},
                          std::false_type{});
      if (__builtin_amdgcn_ballot_w64(__float_as_uint(lsum) > __float_as_uint(kSpecLimit)) != 0 && !spec_fix(lsum))
        inexact = true;
      l_run += lsum;
    };
    // Any step, buffers chosen at run time: every step of the exact pass; in
    // the fast pass a non-causal item's last two and the steps of causal
    // waves after their last tile (each wave takes part in every step's
    // barrier and loads).
    auto general = [&](int t, bool relax = false) KB_INLINE {
      const int st = t & 3;
      begin_step(t, relax, true);
      load_tile(false, kst(st), t + 4);
      load_tile(true, vst((st + 2) & 3), t + 2);
      float alpha = 1.f;
      bool grow = false;
      if (t >= 1 && t - 1 < pv_lim) pv(vst((st + 3) & 3));
      if (t < tw) {
        mask(t);
        grow = row_max(alpha, kRescaleLog2);
        probs(0);
        probs(1);
        l_run += pb_sum();
      }
      if (t + 1 < tw) qk(kst((st + 1) & 3));
      rescale(grow, alpha);
    };

    // This wave's 32 output rows, normalised, skipping rows past the end.
    auto store_rows = [&]() KB_INLINE {
      const float inv = 1.f / xor32_sum(l_run);
      if (q < S) {
        const size_t op = base + (size_t)q * D + 4 * h;
  #pragma unroll
        for (int mb = 0; mb < MB; ++mb)
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            const f32x4 o4 = {oacc[mb][4 * r] * inv, oacc[mb][4 * r + 1] * inv,
                              oacc[mb][4 * r + 2] * inv, oacc[mb][4 * r + 3] * inv};
            store_out4(O, op + 32 * mb + 8 * r, o4, out_bf16);
          }
      }
    };
    // Causal: a wave whose last tile comes before the item's last step
    // stores its rows right after that tile's P V, during the steps in which
    // the waves with later tiles finish.  At d = 128 its next two barrier
    // waits let the 16 stores stay outstanding (`relax` of begin_step), and
    // the steps after the store are a loop of their own (with the store
    // inside the one loop the kernel spills); at d <= 64 the 8 stores are
    // waited for at the next barrier, which measured faster there.
    constexpr bool kEarlyStore = CAUSAL;

    // Fast pass, step 0: the exact row maximum of tile 0 plus kRefMargin
    // (the reference for the steady tiles), then the softmax of tile 0
    // interleaved with the score products of tile 1 in the fused instruction
    // stream (no P V yet).  The prologue's score products read stage 0, which
    // this step refills.
    auto step0 = [&]() KB_INLINE {
      begin_step(0, false, true);
      mask(0);
      float alpha;
      row_max(alpha, 0.f);
      m_run += kRefMargin;
      const uint32_t tk = tile_off(4), tv = tile_off(2);
      auto ld = [&](int k) KB_INLINE {
        if (k < CHW) dma(false, k, kst(0), tk);
        else dma(true, k - CHW, vst(2), tv);
      };
      float lsum;
      if constexpr (D <= 64)
        lsum = fused_step_db(vst(3), kst(1), vst(0), kst(2), ld, std::false_type{}, std::true_type{}, scd[1], scd[0]);
      else
        lsum = fused_step(vst(3), kst(1), vst(0), kst(2), ld, std::false_type{}, std::true_type{});
      l_run += lsum;
    };

    // One pass over the item's key tiles.  The exact pass takes every step
    // through `general` (a row maximum per tile); it runs only if the fast
    // pass met a tile whose reference was stale beyond repair.
    auto pass = [&](bool exact) KB_INLINE {
      pv_lim = tw;
      int st_step = -8;  // step at whose end this wave issued its output stores
      // Prologue: K(0..3), V(0..1); every wave computes S^T(0).
      load_tile(false, kst(0), 0);
      load_tile(false, kst(1), 1);
      load_tile(false, kst(2), 2);
      load_tile(false, kst(3), 3);
      load_tile(true, vst(0), 0);
      load_tile(true, vst(1), 1);
      __builtin_amdgcn_s_waitcnt(wait_vm_imm(0));
      wg_barrier();
      if constexpr (kQLds) {
        // The B operand fragments of S^T from the wave's staged rows (same
        // offsets as the K fragments of rows 0 .. 31 of a stage).
        const lds_char *qb = (const lds_char *)(const lds_bf16 *)(qring + w * 32 * D);
  #pragma unroll
        for (int kc = 0; kc < KC; ++kc) qf[kc] = *(const lds_bf16x8 *)(qb + (KL ^ (uint32_t)(kc << 5)));
      }
      qk(kst(0));

      if (exact)
        general(0);
      else
        step0();
      int t = 1;
      if (!exact) {
        // Steady steps 1 .. tw - 2: four per iteration, then up to three more;
        // then, causal, the wave's last tile.  (Step 0 read the first
        // fragments of step 1, V(0), ahead.)
        for (; t + 3 <= tw - 2; t += 4) {
          steady(std::integral_constant<int, 1>{}, t);
          steady(std::integral_constant<int, 2>{}, t + 1);
          steady(std::integral_constant<int, 3>{}, t + 2);
          steady(std::integral_constant<int, 0>{}, t + 3);
        }
        if (t <= tw - 2) steady(std::integral_constant<int, 1>{}, t++);
        if (t <= tw - 2) steady(std::integral_constant<int, 2>{}, t++);
        if (t <= tw - 2) steady(std::integral_constant<int, 3>{}, t++);
        // The scores of tile t are in scd[(t + 1) & 1]; the steps that follow
        // read sc.
        if constexpr (D <= 64) {
          if ((t & 1) == 1) {
            scd[1][0] = scd[0][0];
            scd[1][1] = scd[0][1];
          }
        }
        // A causal wave's last tile.  The item's last waves then take its
        // P V right away (V(t) is resident: every wave waited for it at this
        // step's barrier) and store their rows, so the item needs no step
        // after it.  (Earlier waves leave that P V to the next step, which
        // the others spend on steady work anyway: done here it held up the
        // next barrier.)
        if (CAUSAL && t == tw - 1) {
          steady_last(t);
          if (tw == ntiles) {
            pv(vst(t & 3));
            pv_lim = tw - 1;
            if (!inexact) {
              store_rows();
              st_step = t;
            }
          }
          ++t;
        }
      }
      // Once the P V of its last tile is in, a wave's O and l are final and
      // it stores its rows: the item's last waves (tw = ntiles) in the step
      // of their last tile, the others after the general step that takes
      // that P V (all their 32 rows then lie before the sequence end, so
      // they issue all 4 MB store instructions).  A wave whose fast pass
      // went inexact does not store (its item is redone and every wave
      // stores after the exact pass).  The fast causal pass ends with the
      // step of the last waves' last tile; otherwise a final step takes the
      // P V of every wave's last tile.
      const int last = (CAUSAL && !exact && ntiles >= 2) ? ntiles - 1 : ntiles;
      if constexpr (D > 64) {
        bool stored = st_step >= 0;
        if (!stored) {
          for (; t <= last; ++t) {
            general(t);
            if (kEarlyStore && !exact && t == tw && !inexact) {
              store_rows();
              stored = true;
              st_step = t;
              ++t;
              break;
            }
          }
        }
        for (; t <= last; ++t) general(t, stored && t <= st_step + 2);
      } else {
        for (; t <= last; ++t) {
          general(t);
          if (kEarlyStore && !exact && t == tw && st_step < 0 && !inexact) {
            store_rows();
            st_step = t;
          }
        }
      }
      // A store in the item's last step leaves the 4 MB store instructions
      // as the youngest memory operations (if the wave has a row before the
      // sequence end, all of them issue).
      const bool last_store = st_step == last && qw < S;
      // No tile load may still be writing this workgroup's LDS when it ends
      // (vmcnt retires in issue order: past the stores of the last step, the
      // loads are in; the next item's prologue waits for the stores).
      if (last_store)
        __builtin_amdgcn_s_waitcnt(wait_vm_imm(4 * MB));
      else
        __builtin_amdgcn_s_waitcnt(wait_vm_imm(0));
    };

    // Cleared before the prologue's barrier; set by any wave whose fast pass
    // went inexact; read by all after the barrier that ends the pass.
    if (tid == 0) redo_flag = 0;
    pass(false);
    if (inexact && lane == 0) redo_flag = 1;
    wg_barrier();
    const bool redone = redo_flag != 0;
    if (redone) {
  #pragma unroll
      for (int mb = 0; mb < MB; ++mb) oacc[mb] = f32x16{};
      m_run = -INFINITY;
      l_run = 0.f;
      inexact = false;
      pass(true);
    }
    if (!kEarlyStore || redone) store_rows();
  };
  for (int u = jw; u < hx * upd; u += nw) {
    const int bh = h0 + u / upd, r = u % upd;
    if (CAUSAL) {
      one_item(bh, nqt - 1 - r);
      if (r != nqt - 1 - r) one_item(bh, r);
    } else {
      one_item(bh, r);
    }
  }
}

// ------------------------------------------------------------------- fp32 ---
// fp32 inputs, small grids: 16-query blocks on the 16x16x4 fp32 MFMA, so
// that small problems still spread over every CU.  A workgroup is NW waves
// on one block of 16 queries; wave w takes the w-th of NW parts of the
// block's visible keys (in 16-key blocks), runs the online softmax over it,
// and the partial results (m_w, l_w, O_w) are merged through LDS by the same
// identity that merges the tiles of one wave: m = max m_w,
// l = sum 2^(m_w - m) l_w, O = sum 2^(m_w - m) O_w / l.
//   S^T = K Q^T:  A = K (row = key, lane % 16), B = Q^T (column = query,
//                 lane % 16), contraction step (c, e) on d-column
//                 16 c + 4 (lane / 16) + e, so each lane reads 16-byte
//                 vectors of K and Q.  Lane l then holds the scores of query
//                 l % 16 against keys 4 (l / 16) + i, i = 0..3, of the block.
//   O^T += V^T P^T: contraction step s on keys 4 g + s (g = lane / 16), so
//                 the B operand of step s is the lane's own probability i = s;
//                 A = V^T, lane l providing V[key 4 g + s][16 c + l % 16].
//                 Lane l accumulates O^T[d = 16 c + 4 (l / 16) + i][query l % 16].
// The next block's scores are computed before the current block's softmax,
// so the matrix core has independent work while the vector ALU runs.
constexpr int kQb = 16;  // queries per workgroup of the key-split kernel
// Waves (key parts) per workgroup of the key-split kernel: two per SIMD, so
// one wave's softmax overlaps the other's products (8 measured 12 % faster
// than 4 at B1 H8 S512 d64).
constexpr int kSplitWaves = 8;

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW) void flash_f32_split_kernel(const float *__restrict__ Q,
                                                                  const float *__restrict__ K,
                                                                  const float *__restrict__ V,
                                                                  void *__restrict__ O, int out_bf16, int S,
                                                                  int nbh, int nqt, float sl2e) {
  constexpr int G = D / 16;  // 16-wide column groups of d
  __shared__ float part_o[NW][G][16][kQb];  // [wave][column group][d % 16][query]
  __shared__ float part_m[NW][kQb], part_l[NW][kQb];

  int bh, qt;
  if (!tile_of_block(bh, qt, nbh, nqt, CAUSAL)) return;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int q0 = qt * kQb, q = q0 + n;
  const size_t base = (size_t)bh * S * D;

  f32x4 qf[G];
  {
    const float *qp = Q + base + (size_t)min(q, S - 1) * D + 4 * g;
#pragma unroll
    for (int c = 0; c < G; ++c) qf[c] = *(const f32x4 *)(qp + 16 * c);
  }
  // This wave's 16-key blocks [b0, b1) of the block's visible range.
  const int kend = CAUSAL ? min(S, q0 + kQb) : S;
  const int nblk = (kend + 15) / 16;
  const int per = (nblk + NW - 1) / NW;
  const int b0 = min(nblk, w * per), b1 = min(nblk, b0 + per);

  f32x4 oacc[G];
#pragma unroll
  for (int c = 0; c < G; ++c) oacc[c] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's share (its 4 keys per block)

  // Scores of block b (raw dot products): two accumulators for two
  // independent MFMA chains, added at the end.
  auto scores = [&](int b) KB_INLINE {
    const float *kp = K + base + (size_t)min(16 * b + n, S - 1) * D + 4 * g;
    f32x4 kf[G];
#pragma unroll
    for (int c = 0; c < G; ++c) kf[c] = *(const f32x4 *)(kp + 16 * c);
    f32x4 s0 = f32x4{}, s1 = f32x4{};
#pragma unroll
    for (int c = 0; c < G; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (((c * 4 + e) & 1) == 0) s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[c][e], qf[c][e], s0, 0, 0, 0);
        else s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[c][e], qf[c][e], s1, 0, 0, 0);
      }
    return s0 + s1;
  };

  f32x4 snext = b0 < b1 ? scores(b0) : f32x4{};
  for (int b = b0; b < b1; ++b) {
    const f32x4 sraw = snext;
    // V^T operands of this block (loaded before the next block's scores).
    float vf[4][G];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float *vp = V + base + (size_t)min(16 * b + 4 * g + s4, S - 1) * D + n;
#pragma unroll
      for (int c = 0; c < G; ++c) vf[s4][c] = vp[16 * c];
    }
    if (b + 1 < b1) snext = scores(b + 1);
    // Mask (ragged end of the sequence; causal: keys after the query), scale
    // to log2 units, row max over the lane's 4 keys and the 4 lane groups.
    const int kb = 16 * b + 4 * g;
    const bool need_mask = (16 * b + 16 > S) || (CAUSAL && 16 * b + 15 > q0);
    float x[4], mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = sraw[i] * sl2e;
      if (need_mask && (kb + i >= S || (CAUSAL && kb + i > q))) x[i] = -INFINITY;
      mt = fmaxf(mt, x[i]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2_fast(m_run - m_new);
    m_run = m_new;
    float p[4], ls = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2_fast(x[i] - m_new);
      ls += p[i];
    }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int c = 0; c < G; ++c) oacc[c] *= alpha;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int c = 0; c < G; ++c) oacc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[s4][c], p[s4], oacc[c], 0, 0, 0);
  }

  // Merge the waves' partial results.  The row sum over the 4 lane groups
  // first (every group holds the same reference m_run).
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (g == 0) {
    part_m[w][n] = m_run;
    part_l[w][n] = l_run;
  }
#pragma unroll
  for (int c = 0; c < G; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) part_o[w][c][4 * g + i][n] = oacc[c][i];
  __syncthreads();
  // Wave w finishes the column groups c = w, w + NW, ...: lane (g, n) the
  // four d-columns 16 c + 4 g .. + 3 of query n.
  float mw[NW], m_all = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    mw[v] = part_m[v][n];
    m_all = fmaxf(m_all, mw[v]);
  }
  float l_all = 0.f, sc[NW];
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    sc[v] = exp2_fast(mw[v] - m_all);  // 0 for a wave with no keys (m = -inf)
    l_all += sc[v] * part_l[v][n];
  }
  const float inv = 1.f / l_all;
  for (int c = w; c < G; c += NW) {
    f32x4 o4 = f32x4{};
#pragma unroll
    for (int v = 0; v < NW; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] += sc[v] * part_o[v][c][4 * g + i][n];
    if (q < S) store_out4(O, base + (size_t)q * D + 16 * c + 4 * g, o4 * inv, out_bf16);
  }
}

// fp32 inputs, large grids: 128 queries per workgroup (4 waves of 32), the
// K/V tiles (32 keys) staged in LDS once for all of them and double-
// buffered through registers (the loads of tile t+1 are issued before tile
// t is computed); 32x32x2 fp32 MFMAs.  The contraction index is permuted
// consistently on both operands: step (g, e) uses d-columns 8g + 4h + e
// from lane half h, so each lane reads 16-byte vectors.  P^T slot c of a
// lane is key acc_row(c, h).  Used when its grid already covers the CUs;
// smaller problems take the key-split kernel above.
constexpr int kBr = 128;  // queries per workgroup of the tile kernel

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void flash_f32_tile_kernel(const float *__restrict__ Q,
                                                             const float *__restrict__ K,
                                                             const float *__restrict__ V,
                                                             void *__restrict__ O, int out_bf16, int S, int nbh,
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
    const size_t op = base + (size_t)q * D + 4 * h;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 o4 = {oacc[mb][4 * r] * inv, oacc[mb][4 * r + 1] * inv,
                          oacc[mb][4 * r + 2] * inv, oacc[mb][4 * r + 3] * inv};
        store_out4(O, op + 32 * mb + 8 * r, o4, out_bf16);
      }
  }
}

// Work units per slice of the persistent bf16 schedule.
constexpr int causal_units(int nqt, bool causal) { return causal ? (nqt + 1) / 2 : nqt; }

// Compute units of the current device (queried once per device; callers on
// several host threads may race to fill the cache with the same value).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, bool CAUSAL>
hipError_t launch_d(const kb_problem &p) {
  // fp32: the tile kernel once its 128-query grid covers every CU, else the
  // key-split kernel on 16-query blocks.
  const bool split = !p.bf16 && (long long)p.bh * ((p.S + kBr - 1) / kBr) < cu_count();
  // bf16: persistent workgroups, one per CU at most, kXcds * nw in all (see
  // the kernel's schedule), never more than there are work units.  8 waves
  // on 256-query items unless that leaves CUs of an XCD without a unit, then
  // 4 waves on 128-query items (two per CU where both LDS rings fit).
  const int cus_x = std::max(1, cu_count() / kXcds);
  const long long slices_x = (p.bh + kXcds - 1) / kXcds;
  const bool narrow = p.bf16 && slices_x * causal_units((p.S + 255) / 256, CAUSAL) < cus_x;
  const int br = p.bf16 ? (narrow ? 128 : 256) : split ? kQb : kBr;
  const int nqt = (p.S + br - 1) / br;
  // kXcds workgroups per item of the longest per-XCD list (see tile_of_block).
  const long long per = (long long)((p.bh + kXcds - 1) / kXcds) * nqt;
  if (per * kXcds > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(per * kXcds));
  const long long units = slices_x * causal_units(nqt, CAUSAL);
  const int per_cu = narrow && D <= 64 ? 2 : 1;
  const int nw = (int)std::max(1LL, std::min<long long>(units, (long long)per_cu * cus_x));
  const dim3 grid_b((unsigned)(nw * kXcds));
  const float sl2e = p.scale * kLog2e;
  if (p.bf16 && narrow)
    hipLaunchKernelGGL((flash_bf16_kernel<D, CAUSAL, 4>), grid_b, dim3(256), 0, p.stream,
                       (const bf16_t *)p.Q, (const bf16_t *)p.K, (const bf16_t *)p.V, p.O, p.out_bf16, p.S, p.bh,
                       nqt, sl2e);
  else if (p.bf16)
    hipLaunchKernelGGL((flash_bf16_kernel<D, CAUSAL, 8>), grid_b, dim3(512), 0, p.stream,
                       (const bf16_t *)p.Q, (const bf16_t *)p.K, (const bf16_t *)p.V, p.O, p.out_bf16, p.S, p.bh,
                       nqt, sl2e);
  else if (split)
    hipLaunchKernelGGL((flash_f32_split_kernel<D, CAUSAL, kSplitWaves>), grid, dim3(64 * kSplitWaves), 0, p.stream,
                       (const float *)p.Q, (const float *)p.K, (const float *)p.V, p.O, p.out_bf16, p.S, p.bh,
                       nqt, sl2e);
  else
    hipLaunchKernelGGL((flash_f32_tile_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, p.stream,
                       (const float *)p.Q, (const float *)p.K, (const float *)p.V, p.O, p.out_bf16, p.S, p.bh,
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
