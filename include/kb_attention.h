/*
 * kb_attention.h: C ABI of the MI355X (gfx950) scaled dot-product attention
 * forward library (libkb.so).
 *
 * What the library computes is defined on the page "kbench — Transformer
 * Attention Micro-benchmark Harness", section "The three GPU kernels":
 *
 *     O = softmax(Q K^T / sqrt(d)) V
 *
 * over a flattened (batch * heads) axis, every tensor laid out
 * [head, seq, dim] row-major.  The problem parameters (seq, dim, heads and
 * the causal flag) are the fields the same page's harness sweeps (section
 * "Running") and sends in its RUN_ATTN request (section "Architecture",
 * sequence diagram).  "causal" is read as: key j is visible to query i iff
 * j <= i (0-based), masked keys get weight exactly 0.
 *
 * The three variants are the page's three kernels (same section):
 *   KB_NAIVE  three passes, the full S x S fp32 score matrix in HBM
 *             (caller-provided workspace), row softmax in place, then P V;
 *   KB_FUSED  one workgroup per query row, the row's scores held in LDS;
 *   KB_FLASH  key/value tiles streamed through LDS with an online softmax
 *             (running max m and denominator l), MFMA tiles for both
 *             contractions, the score matrix never materialised.
 * The HBM triad a[i] = b[i] + s * c[i] is the bandwidth calibration of the
 * page "TileOPs-Metax benchmarks/hardware", section "HBM Bandwidth".
 *
 * Conventions for every entry point:
 *   - Pointers named Q, K, V, O, a, b, c, workspace are DEVICE pointers
 *     (hipMalloc / torch CUDA tensors); everything else is host memory.
 *   - The caller owns every buffer.  The library allocates nothing that
 *     outlives a call (the benchmark helpers create and destroy their own
 *     hipEvents).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  kb_attention and kb_triad do not synchronise.
 *   - Arguments are validated before anything is launched.  Errors are
 *     returned as a kb_status; nothing aborts or exits.  After a non-KB_OK
 *     return, kb_last_error() gives a message for the calling thread.
 *   - The library is stateless and may be called from several host threads.
 */
#ifndef KB_ATTENTION_H
#define KB_ATTENTION_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  KB_BF16 data is passed as raw 16-bit bfloat16 patterns. */
typedef enum { KB_F32 = 0, KB_BF16 = 1 } kb_dtype;

/* Kernel selector (kbench page, "The three GPU kernels"). */
typedef enum { KB_NAIVE = 0, KB_FUSED = 1, KB_FLASH = 2 } kb_variant;

typedef enum {
  KB_OK = 0,
  KB_ERR_INVALID = 1,     /* null pointer, non-positive size, bad enum value */
  KB_ERR_UNSUPPORTED = 2, /* valid but not implemented (dim, dtype, LDS size) */
  KB_ERR_WORKSPACE = 3,   /* naive: workspace missing or too small */
  KB_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  KB_ERR_NO_DEVICE = 5    /* no usable gfx950 device */
} kb_status;

/*
 * One attention problem.  Q, K, V are [batch*heads, seq, dim] row-major of
 * type in_dtype; O is [batch*heads, seq, dim] row-major of type out_dtype.
 *   batch, heads >= 1, seq >= 1 (any length: tails are masked),
 *   dim in {32, 64, 128},
 *   causal 0 or 1,
 *   in_dtype KB_F32 or KB_BF16, out_dtype KB_F32 or KB_BF16 (bf16 output is the
 *   fp32 result rounded to nearest even, in the kernels' epilogue),
 *   scale: the logit scale; 0.0f means 1/sqrt(dim).  It is applied in fp32
 *          to the fp32 dot products, never folded into the inputs.
 *   workspace / workspace_bytes: device scratch, used by KB_NAIVE only
 *          (>= kb_attention_workspace_size bytes, 256-byte aligned, not
 *          overlapping Q, K, V or O: KB_ERR_INVALID otherwise);
 *          ignored by the other variants.
 * batch * heads * seq * dim must stay below 2^31 elements per tensor, and
 * batch * heads * seq * seq below 2^40 (naive workspace).
 */
typedef struct {
  int32_t batch, heads, seq, dim;
  int32_t causal;
  int32_t in_dtype;  /* kb_dtype */
  int32_t out_dtype; /* kb_dtype of O */
  float scale;
  void *workspace;
  size_t workspace_bytes;
} kb_attn_cfg;

/*
 * Enqueue one attention forward pass of `variant` on `stream`.
 * Returns KB_OK once the kernels are enqueued (not finished).
 * KB_ERR_INVALID / KB_ERR_UNSUPPORTED / KB_ERR_WORKSPACE are returned before
 * any launch; KB_ERR_HIP if a launch fails.  O may not alias Q, K or V.
 */
kb_status kb_attention(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V,
                       void *O, int32_t variant, void *stream);

/*
 * kb_attention(cfg, Q, K, V, O, KB_NAIVE, stream) without a caller-provided
 * workspace and without allocating: for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The naive variant's fp32 score matrix goes to a
 * static device array of KB_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on each GPU it runs on until the process ends (its device address
 * is looked up once per device, on the first call made with that device
 * current).  cfg->workspace and cfg->workspace_bytes are ignored.  Limit:
 * 4 * batch * heads * seq * seq <= KB_NOALLOC_SCRATCH_BYTES (e.g. 16 heads
 * at seq 1024), else KB_ERR_WORKSPACE before any launch.  Every call on one
 * GPU uses the same array, so calls that overlap on one GPU (other streams
 * or host threads) race and must be serialised by the caller.  Nothing in
 * the array needs to start at zero: the first pass writes every score the
 * later passes read.  Other errors as kb_attention; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 */
#define KB_NOALLOC_SCRATCH_BYTES (64u << 20)
kb_status kb_attention_naive_noalloc(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V,
                                     void *O, void *stream);

/*
 * Bytes of device workspace `variant` needs for `cfg`: 4 * B*H*S*S for
 * KB_NAIVE (the fp32 score / probability matrix that the naive kernel's
 * first pass writes to DRAM and its softmax and P V passes stream back:
 * kbench page, "The three GPU kernels", naive), 0 for the others, and
 * (size_t)-1 if cfg is invalid (the same checks as kb_attention's, made
 * without touching a device; kb_last_error() says which failed).
 */
size_t kb_attention_workspace_size(const kb_attn_cfg *cfg, int32_t variant);

/*
 * HBM triad, a[i] = b[i] + s * c[i] for i < n (fp32, 128-bit accesses where
 * alignment allows; the page "TileOPs-Metax benchmarks/hardware", "HBM
 * Bandwidth": the STREAM triad, two reads and one write per element, is the
 * calibration kernel).  block: threads per workgroup, a multiple of 64 in
 * [64, 1024].  a, b, c must not overlap.  Enqueued on `stream`.
 * KB_ERR_INVALID for NULL pointers, n == 0, a bad block or overlap.
 */
kb_status kb_triad(float *a, const float *b, const float *c, float s, size_t n, int32_t block,
                   void *stream);

/*
 * Timing helper: `warmup` untimed launches of kb_attention, then `iters`
 * timed ones, each bracketed by hipEvents recorded on `stream` (so the times
 * cover exactly the kernels of one call, nothing else).  ms_per_iter (host,
 * length iters) receives each call's GPU time; *ms_total the time from the
 * first to the last event.  With ms_per_iter NULL only those two outer
 * events are recorded and the timed calls follow each other with no event
 * between them: *ms_total / iters is then the batched mean, which for
 * kernels of a few microseconds leaves out the cost of the per-call events
 * (about 3 us per call on MI355X).  Synchronises `stream` before returning.
 * Protocol: kbench page, "The three GPU kernels", last paragraph (events
 * around the kernel only, no host-device copies in the window, configurable
 * warmup, per-launch times for mean / p50 / p99 / min); the warmup also
 * lets the clocks settle ("TileOPs-Metax benchmarks/hardware",
 * "Methodology").  Errors: those of kb_attention (before any launch), and
 * KB_ERR_INVALID for warmup < 0, iters < 1 or a NULL ms_total;
 * KB_ERR_HIP if an event call or launch fails (the stream is synchronised
 * first).
 */
kb_status kb_bench_attention(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V,
                             void *O, int32_t variant, void *stream, int32_t warmup,
                             int32_t iters, float *ms_per_iter, float *ms_total);

/*
 * The same protocol for kb_triad ("TileOPs-Metax benchmarks/hardware",
 * "Methodology": event timing on the GPU side, warmup iterations before the
 * timed ones; the caller repeats it per block size and keeps the best).
 * Errors: those of kb_triad and kb_bench_attention's result checks.
 */
kb_status kb_bench_triad(float *a, const float *b, const float *c, float s, size_t n,
                         int32_t block, void *stream, int32_t warmup, int32_t iters,
                         float *ms_per_iter, float *ms_total);

/*
 * The reference bandwidth kernels beside the triad (same page, "HBM
 * Bandwidth"), timed with the same protocol, 128-bit accesses:
 *   KB_STREAM_COPY   a[i] = b[i]           8 bytes per element
 *   KB_STREAM_READ   read b[i], no writes  4 bytes per element
 *   KB_STREAM_WRITE  a[i] = s              4 bytes per element
 * n: elements, a multiple of 4, >= 4; a and b: 16-byte aligned,
 * non-overlapping fp32 device buffers of n elements (b is not read by WRITE;
 * READ stores a thread's sum into a only if it equals s, so pass s = NaN to
 * write nothing).  block as for kb_triad.  KB_ERR_INVALID for a bad kind, n
 * or block, or NULL, misaligned or overlapping buffers.
 */
typedef enum { KB_STREAM_COPY = 1, KB_STREAM_READ = 2, KB_STREAM_WRITE = 3 } kb_stream_kind;
kb_status kb_bench_stream(int32_t kind, float *a, const float *b, float s, size_t n, int32_t block,
                          void *stream, int32_t warmup, int32_t iters, float *ms_per_iter,
                          float *ms_total);

/*
 * Ceiling probes.  Compute kinds (the compute analogue of the triad; method
 * of the micro-benchmark log page, section on compute peaks: independent
 * instruction chains per thread, dense matrix products with fp32
 * accumulation, the sustained clock recorded beside the result) and the
 * read bandwidth of each on-chip memory level (the measured bandwidth
 * ceilings of the hierarchical roofline, GPU-Roofline-Python page,
 * "Bandwidth Ceilings").  One workgroup per CU of eight waves, two per SIMD,
 * each running `iters` iterations of 8 independent instructions of one kind:
 */
typedef enum {
  KB_CEIL_MFMA_BF16 = 0, /* v_mfma_f32_32x32x16_bf16: 32768 flops each */
  KB_CEIL_MFMA_F32 = 1,  /* v_mfma_f32_32x32x2f32: 4096 flops each */
  KB_CEIL_FMA_F32 = 2,   /* v_fma_f32 (wave64): 128 flops each */
  KB_CEIL_EXP_F32 = 3,   /* v_exp_f32 (wave64): 64 exponentials each */
  KB_CEIL_LDS_READ = 4,  /* ds_read_b128 over a 64 KiB LDS window: 1024 bytes each */
  KB_CEIL_L1_READ = 5,   /* 16-byte-per-lane global loads over a 16 KiB slice per
                            workgroup (vector L1 hits): 1024 bytes each */
  KB_CEIL_L2_READ = 6,   /* the same loads over a 2 MiB region per XCD (L2 hits,
                            L1 misses): 1024 bytes each */
  KB_CEIL_MFMA_BF16_DATA = 7, /* v_mfma_f32_32x32x16_bf16 on random-bit operands
                                 (8 A and 8 B register sets, a new pair for every
                                 product): 32768 flops each */
  /* Co-issue beside the matrix core: v_mfma_f32_32x32x16_bf16 as in
     KB_CEIL_MFMA_BF16, each product followed by independent work of another
     kind from the same wave; the rate counts the products' flops only, so
     it falls below KB_CEIL_MFMA_BF16 once that work no longer fits in the
     products' shadow (or, for the LDS reads, once their power lowers the
     clock). */
  KB_CEIL_MFMA_BF16_FMA3 = 8, /* ... + 3 independent v_fma_f32 per product */
  KB_CEIL_MFMA_BF16_EXP3 = 9, /* ... + 3 independent v_exp_f32 per product */
  KB_CEIL_MFMA_BF16_EXP4 = 10, /* ... + 4 independent v_exp_f32 per product */
  KB_CEIL_MFMA_BF16_LDS = 11  /* ... + one ds_read_b128 after even products and
                                 two ds_read_b64_tr_b16 after odd ones (the flash
                                 kernel's LDS mix), each fragment the A operand
                                 of the product two later */
} kb_ceiling_kind;

/*
 * Bytes of device work buffer kb_bench_ceiling needs on the current device
 * (per-wave clock counters, one output float per thread and the 16 MiB the
 * cache probes read); 0 if there is no device.  Same passages as the
 * probes above: the micro-benchmark log page's compute-peak section records
 * the clock beside each peak, hence the per-wave clock counters.
 */
size_t kb_ceiling_work_size(void);

/*
 * Timing helper for a ceiling probe, same protocol as kb_bench_attention:
 * `warmup` untimed launches, then `reps` timed ones (ms_per_rep, host,
 * length reps).  *ops_per_launch receives the operations one launch
 * performs (flops for the MFMA and FMA kinds, exponentials for EXP, bytes
 * read for the LDS, L1 and L2 kinds).  The cache probes read whatever the
 * work buffer holds (no initialisation needed).  If
 * clock_mhz is non-NULL it receives the mean shader clock the waves of the
 * last launch ran at (s_memtime over the 100 MHz s_memrealtime).  `work`:
 * device buffer of >= kb_ceiling_work_size() bytes, owned by the caller
 * (KB_ERR_WORKSPACE if smaller).  Errors: KB_ERR_INVALID for a bad kind,
 * iters < 1, reps < 1, warmup < 0 or NULL result pointers; no device:
 * KB_ERR_NO_DEVICE; not gfx950: KB_ERR_UNSUPPORTED.  Synchronises `stream`.
 */
kb_status kb_bench_ceiling(int32_t kind, int32_t iters, void *work, size_t work_bytes, void *stream,
                           int32_t warmup, int32_t reps, float *ms_per_rep, double *ops_per_launch,
                           float *clock_mhz);

/*
 * Properties of the current device, filled by kb_device_info (the kbench
 * page lists a device_info source beside the kernel launcher, "Repository
 * layout"; the report needs the chip's name, unit count and clocks to
 * place each measurement against its ceilings).
 */
typedef struct {
  char arch[64];              /* e.g. "gfx950:sramecc+:xnack-" */
  int32_t compute_units;
  int32_t max_lds_per_block;  /* bytes of LDS one workgroup may use */
  int32_t clock_mhz;          /* peak engine clock the runtime reports */
  int32_t memory_clock_mhz;
  int64_t global_mem_bytes;
} kb_device_props;

/*
 * Query the current HIP device.  KB_ERR_INVALID if out is NULL;
 * KB_ERR_NO_DEVICE without a device (the caller then skips its GPU rows
 * instead of failing: kbench page, "Architecture", the GPU path is
 * optional and its rows are skipped without a GPU toolkit).
 */
kb_status kb_device_info(kb_device_props *out);

/*
 * Static text for a status code (never NULL; "unknown status" for a value
 * that is not a kb_status).  Errors are reported, never fatal, so a caller
 * can skip what the device cannot run (kbench page, "Architecture": GPU
 * rows are skipped, the run goes on).
 */
const char *kb_status_string(int32_t status);

/*
 * Message describing the last failure on the calling thread ("" if none;
 * the text lives in thread-local storage and stays valid until the next
 * failing call on the same thread).  Same reading as kb_status_string.
 */
const char *kb_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KB_ATTENTION_H */
