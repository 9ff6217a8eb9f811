// C ABI of libkb.so: argument validation, variant dispatch, event timing.
//
// The dispatch mirrors the kbench page's run_attention(kernel, cfg) entry
// ("Architecture" diagram: one shared problem definition, one dispatch call
// per kernel choice); the timing helpers follow its launch.cu description
// ("The three GPU kernels", last paragraph): events around the kernels only,
// no host-device copies inside the timed window, configurable warmup.
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kb_attention.h"
#include "kb_device.hpp"

// Device scratch of kb_attention_naive_noalloc: the naive variant's fp32
// score matrix lives here instead of in a caller-provided workspace.  Every
// GPU the library runs on holds its own copy from the code object's load
// until the process ends.  Host code never uses this name as an address
// (on the host it is only a stand-in for the symbol): the device address
// comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[KB_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

thread_local char g_err[512] = "";

void set_err(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
void set_err(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

kb_status hip_fail(hipError_t e, const char *what) {
  set_err("%s: %s", what, hipGetErrorString(e));
  return KB_ERR_HIP;
}

// Per-device facts, queried once: 1 = gfx950, 2 = other; LDS limit per block.
constexpr int kMaxDev = 64;
std::atomic<int> g_arch[kMaxDev];
std::atomic<long long> g_lds[kMaxDev];

kb_status device_check(int *lds_limit) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_err("hipGetDevice: %s", hipGetErrorString(e));
    return KB_ERR_NO_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDev) {
    set_err("device id %d out of range", dev);
    return KB_ERR_NO_DEVICE;
  }
  int a = g_arch[dev].load(std::memory_order_acquire);
  if (a == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      set_err("hipGetDeviceProperties: %s", hipGetErrorString(e));
      return KB_ERR_NO_DEVICE;
    }
    a = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    size_t lds = prop.sharedMemPerBlock;
    if (prop.sharedMemPerBlockOptin > lds) lds = prop.sharedMemPerBlockOptin;
    g_lds[dev].store((long long)lds, std::memory_order_relaxed);
    g_arch[dev].store(a, std::memory_order_release);
  }
  if (a != 1) {
    set_err("the current device is not gfx950");
    return KB_ERR_NO_DEVICE;
  }
  if (lds_limit) *lds_limit = (int)g_lds[dev].load(std::memory_order_relaxed);
  return KB_OK;
}

// Host-side validation; fills `p` (without pointers / stream).
kb_status validate(const kb_attn_cfg *cfg, int32_t variant, kb_problem *p) {
  if (!cfg) {
    set_err("cfg is NULL");
    return KB_ERR_INVALID;
  }
  if (cfg->batch < 1 || cfg->heads < 1 || cfg->seq < 1 || cfg->dim < 1) {
    set_err("batch, heads, seq, dim must be >= 1 (got %d, %d, %d, %d)", cfg->batch, cfg->heads,
            cfg->seq, cfg->dim);
    return KB_ERR_INVALID;
  }
  if (cfg->causal != 0 && cfg->causal != 1) {
    set_err("causal must be 0 or 1 (got %d)", cfg->causal);
    return KB_ERR_INVALID;
  }
  if (cfg->in_dtype != KB_F32 && cfg->in_dtype != KB_BF16) {
    set_err("in_dtype %d is not a kb_dtype", cfg->in_dtype);
    return KB_ERR_INVALID;
  }
  if (cfg->out_dtype != KB_F32 && cfg->out_dtype != KB_BF16) {
    set_err("out_dtype %d is not a kb_dtype", cfg->out_dtype);
    return KB_ERR_INVALID;
  }
  if (variant != KB_NAIVE && variant != KB_FUSED && variant != KB_FLASH) {
    set_err("variant %d is not a kb_variant", variant);
    return KB_ERR_INVALID;
  }
  if (!std::isfinite(cfg->scale) || cfg->scale < 0.f) {
    set_err("scale must be finite and >= 0 (0 selects 1/sqrt(dim))");
    return KB_ERR_INVALID;
  }
  if (cfg->dim != 32 && cfg->dim != 64 && cfg->dim != 128) {
    set_err("dim %d unsupported (32, 64 or 128)", cfg->dim);
    return KB_ERR_UNSUPPORTED;
  }
  const long long bh = (long long)cfg->batch * cfg->heads;
  const long long elems = bh * cfg->seq * cfg->dim;
  if (bh > 0x7fffffffLL || elems >= (1LL << 31)) {
    set_err("tensor of %lld elements exceeds the 2^31 element limit", elems);
    return KB_ERR_UNSUPPORTED;
  }
  if (variant == KB_NAIVE && (double)bh * cfg->seq * cfg->seq >= 1099511627776.0) {
    set_err("naive score matrix exceeds 2^40 elements");
    return KB_ERR_UNSUPPORTED;
  }
  // Dispatch limits, checked here so that no kernel of a multi-pass variant
  // is enqueued before a later one fails to launch: a dispatch holds fewer
  // than 2^32 work-items per grid dimension, and the y / z grid dimensions
  // (naive: one per slice) at most 65535 workgroups.  The naive softmax and
  // the fused kernel launch one 256-thread workgroup per query row.
  if (variant == KB_NAIVE || variant == KB_FUSED) {
    if (bh * cfg->seq * 256LL > 0xffffffffLL) {
      set_err("%lld query rows exceed the dispatch limit of the %s variant (2^24 rows)", bh * cfg->seq,
              variant == KB_NAIVE ? "naive" : "fused");
      return KB_ERR_UNSUPPORTED;
    }
    if (variant == KB_NAIVE && bh > 65535) {
      set_err("naive launches one grid row per slice: %lld slices exceed 65535", bh);
      return KB_ERR_UNSUPPORTED;
    }
  }
  p->bh = (int)bh;
  p->S = cfg->seq;
  p->D = cfg->dim;
  p->causal = cfg->causal;
  p->bf16 = cfg->in_dtype == KB_BF16;
  p->out_bf16 = cfg->out_dtype == KB_BF16;
  p->scale = cfg->scale > 0.f ? cfg->scale : (float)(1.0 / std::sqrt((double)cfg->dim));
  return KB_OK;
}

size_t naive_ws_bytes(const kb_problem &p) { return (size_t)4 * p.bh * (size_t)p.S * (size_t)p.S; }

kb_status prepare(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V, void *O,
                  int32_t variant, void *stream, kb_problem *p) {
  kb_status st = validate(cfg, variant, p);
  if (st != KB_OK) return st;
  if (!Q || !K || !V || !O) {
    set_err("Q, K, V and O must be non-NULL device pointers");
    return KB_ERR_INVALID;
  }
  const size_t esz = p->bf16 ? 2 : 4;
  const size_t in_bytes = (size_t)p->bh * p->S * p->D * esz;
  const size_t out_bytes = (size_t)p->bh * p->S * p->D * (p->out_bf16 ? 2 : 4);
  auto overlap = [](const void *a, size_t na, const void *b, size_t nb) {
    const char *x = (const char *)a, *y = (const char *)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(O, out_bytes, Q, in_bytes) || overlap(O, out_bytes, K, in_bytes) ||
      overlap(O, out_bytes, V, in_bytes)) {
    set_err("O overlaps an input");
    return KB_ERR_INVALID;
  }
  if (((uintptr_t)Q | (uintptr_t)K | (uintptr_t)V | (uintptr_t)O) % 16 != 0) {
    set_err("Q, K, V, O must be 16-byte aligned");
    return KB_ERR_INVALID;
  }
  p->Q = Q;
  p->K = K;
  p->V = V;
  p->O = O;
  p->work = nullptr;
  p->stream = (hipStream_t)stream;
  if (variant == KB_NAIVE) {
    if (!cfg->workspace || cfg->workspace_bytes < naive_ws_bytes(*p)) {
      set_err("naive needs a workspace of %zu bytes (got %zu)", naive_ws_bytes(*p),
              cfg->workspace ? cfg->workspace_bytes : (size_t)0);
      return KB_ERR_WORKSPACE;
    }
    if ((uintptr_t)cfg->workspace % 256 != 0) {
      set_err("workspace must be 256-byte aligned");
      return KB_ERR_WORKSPACE;
    }
    const size_t wb = naive_ws_bytes(*p);
    if (overlap(cfg->workspace, wb, Q, in_bytes) || overlap(cfg->workspace, wb, K, in_bytes) ||
        overlap(cfg->workspace, wb, V, in_bytes) || overlap(cfg->workspace, wb, O, out_bytes)) {
      set_err("the workspace overlaps Q, K, V or O");
      return KB_ERR_INVALID;
    }
    p->work = (float *)cfg->workspace;
  }
  int lds_limit = 0;
  st = device_check(&lds_limit);
  if (st != KB_OK) return st;
  if (variant == KB_FUSED && kb_fused_lds_bytes(*p) > (size_t)lds_limit) {
    set_err("fused needs %zu bytes of LDS per workgroup, the device allows %d",
            kb_fused_lds_bytes(*p), lds_limit);
    return KB_ERR_UNSUPPORTED;
  }
  return KB_OK;
}

kb_status launch(const kb_problem &p, int32_t variant) {
  hipError_t e;
  switch (variant) {
    case KB_NAIVE: e = kb_launch_naive(p); break;
    case KB_FUSED: e = kb_launch_fused(p); break;
    default: e = kb_launch_flash(p); break;
  }
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  return KB_OK;
}

kb_status triad_check(float *a, const float *b, const float *c, size_t n, int32_t block) {
  if (!a || !b || !c) {
    set_err("a, b, c must be non-NULL device pointers");
    return KB_ERR_INVALID;
  }
  if (n == 0) {
    set_err("n must be >= 1");
    return KB_ERR_INVALID;
  }
  if (block < 64 || block > 1024 || block % 64 != 0) {
    set_err("block must be a multiple of 64 in [64, 1024] (got %d)", block);
    return KB_ERR_INVALID;
  }
  const char *pa = (const char *)a, *pb = (const char *)b, *pc = (const char *)c;
  const size_t nb = n * sizeof(float);
  if ((pa < pb + nb && pb < pa + nb) || (pa < pc + nb && pc < pa + nb)) {
    set_err("a overlaps b or c");
    return KB_ERR_INVALID;
  }
  return device_check(nullptr);
}

// Shared event-timing loop: `fn` enqueues one call on `stream`.
template <typename F>
kb_status bench_loop(F fn, hipStream_t stream, int32_t warmup, int32_t iters, float *ms_per_iter,
                     float *ms_total) {
  if (warmup < 0 || iters < 1 || !ms_total) {
    set_err("warmup >= 0, iters >= 1 and a non-NULL ms_total are required");
    return KB_ERR_INVALID;
  }
  // Without ms_per_iter only the two outer events are recorded: the launches
  // then follow each other with no event between them (the batched mean).
  const bool each = ms_per_iter != nullptr;
  for (int i = 0; i < warmup; ++i) {
    kb_status st = fn();
    if (st != KB_OK) return st;
  }
  std::vector<hipEvent_t> ev((size_t)iters + 1, nullptr);
  kb_status st = KB_OK;
  hipError_t e = hipSuccess;
  for (int i = 0; i <= iters; ++i) {
    if (!each && i != 0 && i != iters) continue;
    e = hipEventCreate(&ev[(size_t)i]);
    if (e != hipSuccess) {
      st = hip_fail(e, "hipEventCreate");
      break;
    }
  }
  if (st == KB_OK) {
    e = hipEventRecord(ev[0], stream);
    if (e != hipSuccess) st = hip_fail(e, "hipEventRecord");
    for (int i = 0; i < iters && st == KB_OK; ++i) {
      st = fn();
      if (st != KB_OK) break;
      if (each || i + 1 == iters) {
        e = hipEventRecord(ev[i + 1], stream);
        if (e != hipSuccess) st = hip_fail(e, "hipEventRecord");
      }
    }
  }
  if (st == KB_OK) {
    e = hipEventSynchronize(ev[iters]);
    if (e != hipSuccess) st = hip_fail(e, "hipEventSynchronize");
  }
  if (st == KB_OK) {
    for (int i = 0; each && i < iters && st == KB_OK; ++i) {
      e = hipEventElapsedTime(&ms_per_iter[i], ev[i], ev[i + 1]);
      if (e != hipSuccess) st = hip_fail(e, "hipEventElapsedTime");
    }
    if (st == KB_OK) {
      e = hipEventElapsedTime(ms_total, ev[0], ev[iters]);
      if (e != hipSuccess) st = hip_fail(e, "hipEventElapsedTime");
    }
  } else {
    (void)hipStreamSynchronize(stream);
  }
  for (auto &x : ev)
    if (x) (void)hipEventDestroy(x);
  return st;
}

// Per-device address of `scratch`, looked up on the first call on each
// device (with that device current) and kept.
std::atomic<void *> g_scratch[kMaxDev];
std::mutex g_scratch_mu;

kb_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_err("hipGetDevice: %s", hipGetErrorString(e));
    return KB_ERR_NO_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDev) {
    set_err("device id %d out of range", dev);
    return KB_ERR_NO_DEVICE;
  }
  void *ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                   "hipGetSymbolAddress(scratch)");
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return KB_OK;
}

}  // namespace

extern "C" {

kb_status kb_attention_naive_noalloc(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V,
                                     void *O, void *stream) {
  kb_problem p;
  kb_status st = validate(cfg, KB_NAIVE, &p);
  if (st != KB_OK) return st;
  const size_t need = naive_ws_bytes(p);
  if (need > (size_t)KB_NOALLOC_SCRATCH_BYTES) {
    set_err("naive needs %zu bytes of scores (batch*heads*seq*seq*4); the static scratch holds %zu",
            need, (size_t)KB_NOALLOC_SCRATCH_BYTES);
    return KB_ERR_WORKSPACE;
  }
  st = device_check(nullptr);
  if (st != KB_OK) return st;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != KB_OK) return st;
  kb_attn_cfg c = *cfg;
  c.workspace = ws;
  c.workspace_bytes = KB_NOALLOC_SCRATCH_BYTES;
  st = prepare(&c, Q, K, V, O, KB_NAIVE, stream, &p);
  if (st != KB_OK) return st;
  return launch(p, KB_NAIVE);
}

kb_status kb_attention(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V, void *O,
                       int32_t variant, void *stream) {
  kb_problem p;
  kb_status st = prepare(cfg, Q, K, V, O, variant, stream, &p);
  if (st != KB_OK) return st;
  return launch(p, variant);
}

size_t kb_attention_workspace_size(const kb_attn_cfg *cfg, int32_t variant) {
  kb_problem p;
  if (validate(cfg, variant, &p) != KB_OK) return (size_t)-1;
  return variant == KB_NAIVE ? naive_ws_bytes(p) : 0;
}

kb_status kb_triad(float *a, const float *b, const float *c, float s, size_t n, int32_t block,
                   void *stream) {
  kb_status st = triad_check(a, b, c, n, block);
  if (st != KB_OK) return st;
  hipError_t e = kb_launch_triad(a, b, c, s, n, block, (hipStream_t)stream);
  return e == hipSuccess ? KB_OK : hip_fail(e, "triad launch");
}

kb_status kb_bench_attention(const kb_attn_cfg *cfg, const void *Q, const void *K, const void *V,
                             void *O, int32_t variant, void *stream, int32_t warmup, int32_t iters,
                             float *ms_per_iter, float *ms_total) {
  kb_problem p;
  kb_status st = prepare(cfg, Q, K, V, O, variant, stream, &p);
  if (st != KB_OK) return st;
  return bench_loop([&]() { return launch(p, variant); }, p.stream, warmup, iters, ms_per_iter,
                    ms_total);
}

kb_status kb_bench_triad(float *a, const float *b, const float *c, float s, size_t n, int32_t block,
                         void *stream, int32_t warmup, int32_t iters, float *ms_per_iter,
                         float *ms_total) {
  kb_status st = triad_check(a, b, c, n, block);
  if (st != KB_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  return bench_loop(
      [&]() {
        hipError_t e = kb_launch_triad(a, b, c, s, n, block, hs);
        return e == hipSuccess ? KB_OK : hip_fail(e, "triad launch");
      },
      hs, warmup, iters, ms_per_iter, ms_total);
}

kb_status kb_bench_stream(int32_t kind, float *a, const float *b, float s, size_t n, int32_t block,
                          void *stream, int32_t warmup, int32_t iters, float *ms_per_iter,
                          float *ms_total) {
  if (kind < KB_STREAM_COPY || kind > KB_STREAM_WRITE) {
    set_err("kind %d is not a kb_stream_kind", kind);
    return KB_ERR_INVALID;
  }
  if (n < 4 || n % 4 != 0) {
    set_err("n must be a positive multiple of 4 (got %zu)", n);
    return KB_ERR_INVALID;
  }
  if (((uintptr_t)a | (uintptr_t)b) % 16 != 0) {
    set_err("a and b must be 16-byte aligned");
    return KB_ERR_INVALID;
  }
  kb_status st = triad_check(a, b, b, n, block);
  if (st != KB_OK) return st;
  hipStream_t hs = (hipStream_t)stream;
  return bench_loop(
      [&]() {
        hipError_t e = kb_launch_stream(kind, a, b, s, n, block, hs);
        return e == hipSuccess ? KB_OK : hip_fail(e, "stream kernel launch");
      },
      hs, warmup, iters, ms_per_iter, ms_total);
}

size_t kb_ceiling_work_size(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  return kb_ceiling_layout(cus, nullptr, nullptr);
}

kb_status kb_bench_ceiling(int32_t kind, int32_t iters, void *work, size_t work_bytes, void *stream,
                           int32_t warmup, int32_t reps, float *ms_per_rep, double *ops_per_launch,
                           float *clock_mhz) {
  if (kind < KB_CEIL_MFMA_BF16 || kind > KB_CEIL_MFMA_BF16_LDS) {
    set_err("kind %d is not a kb_ceiling_kind", kind);
    return KB_ERR_INVALID;
  }
  if (iters < 1 || reps < 1 || warmup < 0 || !ms_per_rep || !ops_per_launch) {
    set_err("iters >= 1, reps >= 1, warmup >= 0 and non-NULL results are required");
    return KB_ERR_INVALID;
  }
  kb_status st = device_check(nullptr);
  if (st != KB_OK) return st;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "multiprocessor count");
  const size_t waves = (size_t)kb_ceiling_waves(cus);
  size_t sink_off = 0, data_off = 0;
  const size_t need = kb_ceiling_layout(cus, &sink_off, &data_off);
  if (!work || work_bytes < need) {
    set_err("work buffer of %zu bytes needed (got %zu)", need, work ? work_bytes : (size_t)0);
    return KB_ERR_WORKSPACE;
  }
  unsigned long long *clk = (unsigned long long *)work;
  float *sink = (float *)((unsigned char *)work + sink_off);
  const unsigned char *data = (const unsigned char *)work + data_off;
  hipStream_t hs = (hipStream_t)stream;
  float total = 0.f;
  st = bench_loop(
      [&]() {
        hipError_t le = kb_launch_ceiling(kind, cus, iters, clk, sink, data, hs);
        return le == hipSuccess ? KB_OK : hip_fail(le, "ceiling launch");
      },
      hs, warmup, reps, ms_per_rep, &total);
  if (st != KB_OK) return st;
  *ops_per_launch = kb_ceiling_ops(kind, cus, iters);
  if (clock_mhz) {
    std::vector<unsigned long long> h(2 * waves);
    e = hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "reading the clock counters");
    double sum = 0.0;
    size_t n = 0;
    for (size_t w = 0; w < waves; ++w)
      if (h[2 * w + 1] > 0) {
        sum += (double)h[2 * w] / ((double)h[2 * w + 1] / 100.0);
        ++n;
      }
    *clock_mhz = n ? (float)(sum / (double)n) : 0.f;
  }
  return KB_OK;
}

kb_status kb_device_info(kb_device_props *out) {
  if (!out) {
    set_err("out is NULL");
    return KB_ERR_INVALID;
  }
  memset(out, 0, sizeof *out);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_err("hipGetDevice: %s", hipGetErrorString(e));
    return KB_ERR_NO_DEVICE;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    set_err("hipGetDeviceProperties: %s", hipGetErrorString(e));
    return KB_ERR_NO_DEVICE;
  }
  snprintf(out->arch, sizeof out->arch, "%s", prop.gcnArchName);
  out->compute_units = prop.multiProcessorCount;
  size_t lds = prop.sharedMemPerBlock;
  if (prop.sharedMemPerBlockOptin > lds) lds = prop.sharedMemPerBlockOptin;
  out->max_lds_per_block = (int32_t)lds;
  out->clock_mhz = prop.clockRate / 1000;
  out->memory_clock_mhz = prop.memoryClockRate / 1000;
  out->global_mem_bytes = (int64_t)prop.totalGlobalMem;
  return KB_OK;
}

const char *kb_status_string(int32_t status) {
  switch (status) {
    case KB_OK: return "ok";
    case KB_ERR_INVALID: return "invalid argument";
    case KB_ERR_UNSUPPORTED: return "unsupported problem";
    case KB_ERR_WORKSPACE: return "workspace missing or too small";
    case KB_ERR_HIP: return "HIP runtime error";
    case KB_ERR_NO_DEVICE: return "no usable gfx950 device";
    default: return "unknown status";
  }
}

const char *kb_last_error(void) { return g_err; }

}  // extern "C"
