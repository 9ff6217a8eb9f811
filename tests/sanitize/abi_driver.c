/* Drives the host side of libkb's C ABI (include/kb_attention.h) on the CPU,
 * for a build of the library with AddressSanitizer and UndefinedBehavior-
 * Sanitizer on its host code: argument validation, size and overlap
 * arithmetic at the limits, error strings, the per-thread last error and,
 * without a GPU, the device query of valid calls.  Nothing is launched: the
 * pointers are aligned stand-ins that the library must reject (or stop at
 * the device query) before touching them.  With a GPU present, the calls
 * that would pass every argument check are skipped.  Exits non-zero on the
 * first unexpected status; the sanitizers abort on the first report. */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kb_attention.h"

static int failures = 0;

#define EXPECT(call, want)                                                           \
  do {                                                                               \
    int got_ = (int)(call);                                                          \
    if (got_ != (int)(want)) {                                                       \
      fprintf(stderr, "%s:%d: %s -> %d, want %d (%s)\n", __FILE__, __LINE__, #call, \
              got_, (int)(want), kb_last_error());                                   \
      ++failures;                                                                    \
    }                                                                                \
  } while (0)

/* Aligned, non-NULL stand-ins, never dereferenced on these paths. */
#define P(k) ((void *)((uintptr_t)(k) << 28))

static kb_attn_cfg cfg(int b, int h, int s, int d, int causal, int dt) {
  kb_attn_cfg c;
  memset(&c, 0, sizeof c);
  c.batch = b;
  c.heads = h;
  c.seq = s;
  c.dim = d;
  c.causal = causal;
  c.in_dtype = (kb_dtype)dt;
  c.out_dtype = KB_F32;
  return c;
}

static void *other_thread(void *arg) {
  (void)arg;
  kb_attn_cfg c = cfg(1, 1, 0, 64, 0, KB_BF16);
  EXPECT(kb_attention(&c, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  return (void *)(uintptr_t)(strstr(kb_last_error(), "seq") != NULL);
}

int main(void) {
  kb_device_props props;
  const int have_gpu = kb_device_info(&props) == KB_OK;

  /* status strings, including codes outside the enum */
  for (int st = -2; st <= 8; ++st) {
    const char *s = kb_status_string(st);
    if (!s || !*s) {
      fprintf(stderr, "empty status string for %d\n", st);
      ++failures;
    }
  }

  /* configuration checks */
  kb_attn_cfg c = cfg(2, 3, 100, 64, 0, KB_BF16);
  EXPECT(kb_attention(NULL, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  int bad[][6] = {{0, 3, 100, 64, 0, KB_BF16}, {2, -1, 100, 64, 0, KB_BF16}, {2, 3, 0, 64, 0, KB_BF16},
                  {2, 3, 100, 64, 2, KB_BF16},  {2, 3, 100, 64, 0, 7},        {2, 3, -5, 64, 1, KB_F32}};
  for (unsigned i = 0; i < sizeof bad / sizeof bad[0]; ++i) {
    kb_attn_cfg x = cfg(bad[i][0], bad[i][1], bad[i][2], bad[i][3], bad[i][4], bad[i][5]);
    EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
    EXPECT(kb_attention_workspace_size(&x, KB_NAIVE), (size_t)-1);
  }
  kb_attn_cfg x = c;
  x.out_dtype = (kb_dtype)9;
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  x = c;
  x.scale = -1.0f;
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  x = c;
  x.scale = 1.0f / 0.0f;
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  EXPECT(kb_attention(&c, P(1), P(2), P(3), P(4), 3, NULL), KB_ERR_INVALID);
  EXPECT(kb_attention(&c, P(1), P(2), P(3), P(4), -1, NULL), KB_ERR_INVALID);
  x = cfg(2, 3, 100, 96, 0, KB_BF16);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_UNSUPPORTED);

  /* size limits: products that overflow 32-bit (and, for naive, 2^40) */
  x = cfg(65536, 65536, 1, 32, 0, KB_BF16);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_UNSUPPORTED);
  x = cfg(1, 1, 0x7fffffff, 128, 1, KB_F32);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_UNSUPPORTED);
  x = cfg(1, 2, 1 << 20, 32, 0, KB_BF16);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_UNSUPPORTED);
  EXPECT(kb_attention_workspace_size(&x, KB_NAIVE), (size_t)-1);
  x = cfg(1, 16384, 1024, 32, 0, KB_BF16);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FUSED, NULL), KB_ERR_UNSUPPORTED);
  EXPECT(kb_attention_workspace_size(&c, KB_NAIVE), (size_t)4 * 6 * 100 * 100);
  EXPECT(kb_attention_workspace_size(&c, KB_FLASH), 0);

  /* pointers: NULL, misaligned, overlapping */
  EXPECT(kb_attention(&c, NULL, P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  EXPECT(kb_attention(&c, P(1), P(2), P(3), NULL, KB_FLASH, NULL), KB_ERR_INVALID);
  EXPECT(kb_attention(&c, (char *)P(1) + 8, P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_INVALID);
  EXPECT(kb_attention(&c, P(1), P(2), P(3), (char *)P(1) + 64, KB_FLASH, NULL), KB_ERR_INVALID);

  /* naive workspace: missing, short, misaligned, overlapping */
  const size_t nb = (size_t)4 * 6 * 100 * 100;
  EXPECT(kb_attention(&c, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_WORKSPACE);
  x = c;
  x.workspace = P(8);
  x.workspace_bytes = nb - 1;
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_WORKSPACE);
  x.workspace = (char *)P(8) + 16;
  x.workspace_bytes = nb;
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_WORKSPACE);
  x.workspace = P(2);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_INVALID);
  x.workspace = (char *)P(4) - 256;
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_INVALID);

  /* the allocation-free naive entry point */
  EXPECT(kb_attention_naive_noalloc(NULL, P(1), P(2), P(3), P(4), NULL), KB_ERR_INVALID);
  x = cfg(1, 64, 1024, 64, 0, KB_BF16); /* 256 MiB of scores: past the static scratch */
  EXPECT(kb_attention_naive_noalloc(&x, P(1), P(2), P(3), P(4), NULL), KB_ERR_WORKSPACE);

  /* bandwidth kernels and timing helpers: argument checks */
  float per[4], tot;
  double ops;
  EXPECT(kb_triad(NULL, P(2), P(3), 1.0f, 16, 256, NULL), KB_ERR_INVALID);
  EXPECT(kb_triad(P(1), P(2), P(3), 1.0f, 0, 256, NULL), KB_ERR_INVALID);
  EXPECT(kb_triad(P(1), P(2), P(3), 1.0f, 16, 100, NULL), KB_ERR_INVALID);
  EXPECT(kb_triad(P(1), (void *)((char *)P(1) + 8), P(3), 1.0f, 16, 256, NULL), KB_ERR_INVALID);
  EXPECT(kb_bench_triad(P(1), P(2), P(3), 1.0f, 16, 2048, NULL, 0, 4, per, &tot), KB_ERR_INVALID);
  EXPECT(kb_bench_stream(0, P(1), P(2), 1.0f, 1024, 256, NULL, 0, 4, per, &tot), KB_ERR_INVALID);
  EXPECT(kb_bench_stream(1, P(1), P(2), 1.0f, 1022, 256, NULL, 0, 4, per, &tot), KB_ERR_INVALID);
  EXPECT(kb_bench_stream(1, P(1), (void *)((char *)P(1) + 64), 1.0f, 1024, 256, NULL, 0, 4, per, &tot), KB_ERR_INVALID);
  EXPECT(kb_bench_ceiling(99, 10, P(1), 1u << 20, NULL, 0, 4, per, &ops, NULL), KB_ERR_INVALID);
  EXPECT(kb_bench_ceiling(0, 0, P(1), 1u << 20, NULL, 0, 4, per, &ops, NULL), KB_ERR_INVALID);
  EXPECT(kb_bench_ceiling(0, 10, P(1), 1u << 20, NULL, -1, 4, per, &ops, NULL), KB_ERR_INVALID);
  EXPECT(kb_bench_ceiling(0, 10, P(1), 1u << 20, NULL, 0, 4, NULL, &ops, NULL), KB_ERR_INVALID);
  x = cfg(2, 3, 0, 64, 0, KB_BF16);
  EXPECT(kb_bench_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL, 0, 4, per, &tot), KB_ERR_INVALID);

  /* the last error is kept per thread */
  x = cfg(2, 3, 100, 96, 0, KB_BF16);
  EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_UNSUPPORTED);
  pthread_t th;
  void *ok = NULL;
  pthread_create(&th, NULL, other_thread, NULL);
  pthread_join(th, &ok);
  if (!ok || !strstr(kb_last_error(), "dim")) {
    fprintf(stderr, "last error not per thread: '%s'\n", kb_last_error());
    ++failures;
  }

  /* without a GPU, calls that pass every argument check stop at the device query */
  if (!have_gpu) {
    EXPECT(kb_attention(&c, P(1), P(2), P(3), P(4), KB_FLASH, NULL), KB_ERR_NO_DEVICE);
    x = c;
    x.workspace = P(8);
    x.workspace_bytes = nb;
    EXPECT(kb_attention(&x, P(1), P(2), P(3), P(4), KB_NAIVE, NULL), KB_ERR_NO_DEVICE);
    EXPECT(kb_bench_attention(&c, P(1), P(2), P(3), P(4), KB_FLASH, NULL, 0, 4, NULL, &tot), KB_ERR_NO_DEVICE);
    EXPECT(kb_triad(P(1), P(2), P(3), 1.0f, 16, 256, NULL), KB_ERR_NO_DEVICE);
    EXPECT(kb_ceiling_work_size(), 0);
  }

  if (failures) {
    fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  printf("all checks passed (gpu %s)\n", have_gpu ? "present: device paths skipped" : "absent");
  return 0;
}
