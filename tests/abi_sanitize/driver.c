/* Drives the C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer
 * (host code only; no call here reaches a HIP runtime function or a kernel): every case
 * returns its documented status before anything is enqueued. Exit status 0 and "ok" when
 * every status matches. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sagebwd.h"

static int failures = 0;
#define EXPECT(expr, want)                                                                        \
  do {                                                                                            \
    int got_ = (int)(expr);                                                                       \
    if (got_ != (want)) {                                                                         \
      fprintf(stderr, "%s:%d: %s = %d, expected %d\n", __FILE__, __LINE__, #expr, got_, (want)); \
      ++failures;                                                                                 \
    }                                                                                             \
  } while (0)

static sagebwd_params P(void) {
  sagebwd_params p;
  memset(&p, 0, sizeof p);
  p.B = 1; p.H = 2; p.N = 256; p.d = 64; p.blk = 64; p.causal = 1; p.qk_norm = 1; p.k_smooth = 1;
  p.eps = 1e-6f; p.dtype = SAGEBWD_FP16;
  return p;
}

#define F ((void*)(uintptr_t)0x10000) /* aligned, never dereferenced */
#define M ((void*)(uintptr_t)0x10001) /* misaligned */

static int pro(const sagebwd_params* p, void* x, void* ws, size_t wsb) {
  return sagebwd_quant_prologue(p, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, ws, wsb, NULL);
}
static int pro_na(const sagebwd_params* p, void* x) {
  return sagebwd_quant_prologue_noalloc(p, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, NULL);
}
static int fwd(const sagebwd_params* p, void* x) {
  return sagebwd_forward(p, x, x, x, x, x, x, x, x, x, x, NULL);
}
static int bwd(const sagebwd_params* p, void* x, void* ws, size_t wsb) {
  return sagebwd_backward(p, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, ws, wsb, NULL);
}
static int bwd_part(const sagebwd_params* p, int part, void* x) {
  return sagebwd_backward_part(p, part, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, x, F,
                               (size_t)1 << 40, NULL);
}

int main(void) {
  sagebwd_params p;
  const size_t big = (size_t)1 << 40;
  /* invalid options, every entry point */
  for (int which = 0; which < 4; ++which) {
    int (*call)(const sagebwd_params*) = 0;
    (void)call;
#define ALL(mod, want)                                             \
    do {                                                           \
      p = P(); mod;                                                \
      if (which == 0) EXPECT(pro(&p, F, F, big), want);            \
      if (which == 1) EXPECT(pro_na(&p, F), want);                 \
      if (which == 2) EXPECT(fwd(&p, F), want);                    \
      if (which == 3) EXPECT(bwd(&p, F, F, big), want);            \
    } while (0)
    ALL(p.d = 96, SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.blk = 32, SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.dtype = 7, SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.eps = -1.0f, SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.dq_mode = 3, SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.layout = 2, SAGEBWD_ERR_UNSUPPORTED);
    ALL((p.qk_gain = 1, p.qk_norm = 0), SAGEBWD_ERR_UNSUPPORTED);
    ALL((p.normed_grads = 1, p.qk_gain = 1), SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.fmt = 2, SAGEBWD_ERR_UNSUPPORTED);
    ALL((p.fmt = SAGEBWD_FMT_FP8, p.q_smooth = 1), SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.split = 5, SAGEBWD_ERR_UNSUPPORTED);
    ALL((p.split = SAGEBWD_SPLIT_QATTN, p.q_smooth = 1), SAGEBWD_ERR_UNSUPPORTED);
    ALL(p.B = -1, SAGEBWD_ERR_SHAPE);
    ALL(p.N = (1 << 22) + 64, SAGEBWD_ERR_SHAPE);
    ALL(p.N = 0, SAGEBWD_OK);
    ALL(p.B = 0, SAGEBWD_OK);
#undef ALL
  }
  /* null and misaligned tensors, empty problems */
  p = P();
  EXPECT(pro(&p, NULL, F, big), SAGEBWD_ERR_NULL);
  EXPECT(pro(&p, M, F, big), SAGEBWD_ERR_ALIGN);
  EXPECT(pro_na(&p, NULL), SAGEBWD_ERR_NULL);
  EXPECT(fwd(&p, NULL), SAGEBWD_ERR_NULL);
  EXPECT(fwd(&p, M), SAGEBWD_ERR_ALIGN);
  EXPECT(bwd(&p, NULL, F, big), SAGEBWD_ERR_NULL);
  EXPECT(bwd(&p, M, F, big), SAGEBWD_ERR_ALIGN);
  EXPECT(sagebwd_forward(NULL, F, F, F, F, F, F, F, F, F, F, NULL), SAGEBWD_ERR_NULL);
  /* workspaces: sizes, nulls, too small */
  EXPECT(sagebwd_backward_workspace_bytes(NULL) == 0, 1);
  EXPECT(sagebwd_prologue_workspace_bytes(NULL) == 0, 1);
  const size_t need = sagebwd_backward_workspace_bytes(&p);
  EXPECT(need > 0, 1);
  EXPECT(bwd(&p, F, F, need - 1), SAGEBWD_ERR_WORKSPACE);
  EXPECT(bwd(&p, F, NULL, need), SAGEBWD_ERR_NULL);
  EXPECT(bwd(&p, F, M, need), SAGEBWD_ERR_ALIGN);
  const size_t pneed = sagebwd_prologue_workspace_bytes(&p);
  EXPECT(pneed > 0, 1);
  EXPECT(pro(&p, F, F, pneed - 1), SAGEBWD_ERR_WORKSPACE);
  EXPECT(pro(&p, F, NULL, pneed), SAGEBWD_ERR_NULL);
  EXPECT(bwd_part(&p, 3, F), SAGEBWD_ERR_UNSUPPORTED);
  EXPECT(bwd_part(&p, -1, F), SAGEBWD_ERR_UNSUPPORTED);
  /* every dq_mode / gain / split combination sizes its workspace without overflow */
  for (int dq = 0; dq < 3; ++dq)
    for (int g = 0; g < 2; ++g)
      for (int sp = 0; sp < 2; ++sp) {
        p = P(); p.dq_mode = dq; p.qk_gain = g; p.split = sp; p.N = 32768; p.d = 128; p.blk = 128; p.H = 8;
        EXPECT(sagebwd_backward_workspace_bytes(&p) > 0, 1);
      }
  /* the allocation-free prologue refuses a problem beyond its static scratch */
  p = P(); p.B = 64; p.H = 64; p.N = 32768; p.d = 128; p.blk = 128;
  EXPECT(pro_na(&p, F), SAGEBWD_ERR_SCRATCH);
  /* status strings and the error text */
  for (int s = -8; s <= 1; ++s) EXPECT(sagebwd_status_string((sagebwd_status)s) != NULL, 1);
  EXPECT(strlen(sagebwd_last_error()) == 0, 1);
  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
