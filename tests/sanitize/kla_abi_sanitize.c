/* A driver for the C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * tests/test_abi_sanitized.py compiles the library's sources with the sanitizers on the host
 * side, links them with this file and runs it on a machine without a GPU.  It is C, as the
 * ABI's callers are: an enum argument is an int here and may carry any value (7 for a
 * dtype, -77 for a status), which the library must reject without undefined behaviour.
 * Every call below is rejected (or is a no-op) during argument validation, which by the
 * header's contract happens before any HIP call; the workspace queries run their size
 * arithmetic, including shapes near the 32-bit limits.  A status other than the expected
 * one, or any sanitizer report, fails the test (the process exits non-zero). */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kla.h"

static int failures = 0;

static void expect(const char *what, long long got, long long want) {
  if (got != want) {
    printf("FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

/* never dereferenced: every call below stops in validation first */
#define FAKE_BASE ((uintptr_t)0x7F0000000000ull)
static void *fake(uintptr_t off) { return (void *)(FAKE_BASE + off); }
#define FAKE fake(0)

typedef struct {
  const void *q, *k, *v, *g, *eta;
  float eps;
  const float *s0;
  void *o;
  float *sf;
  const int32_t *cu, *cuh;
  int N, B, H, T, dk, dv, chunk, dtype;
  void *ws;
  size_t wsb;
  /* backward only */
  const void *dout;
  const float *dsf;
  void *dq, *dk_, *dv_;
  float *dg, *deta, *ds0;
} Args;

static Args base(void) {
  Args a;
  memset(&a, 0, sizeof a);
  a.q = a.k = a.v = a.g = a.eta = FAKE;
  a.eps = 1e-6f;
  a.o = FAKE;
  a.sf = (float *)FAKE;
  a.N = 2; a.B = 2; a.H = 4; a.T = 100; a.dk = 128; a.dv = 128; a.chunk = 64; a.dtype = 0;
  a.ws = FAKE;
  a.wsb = (size_t)1 << 40;
  a.dout = FAKE;
  a.dq = a.dk_ = a.dv_ = FAKE;
  a.dg = a.deta = (float *)FAKE;
  return a;
}

static kla_status_t fwd(Args a) {
  return kla_chunk_fwd(a.q, a.k, a.v, a.g, a.eta, a.eps, a.s0, a.o, a.sf, a.cu, a.cuh, a.N, a.B, a.H, a.T, a.dk,
                       a.dv, a.chunk, (kla_dtype_t)a.dtype, a.ws, a.wsb, NULL);
}
static kla_status_t noalloc(Args a) {
  return kla_chunk_fwd_noalloc(a.q, a.k, a.v, a.g, a.eta, a.eps, a.s0, a.o, a.sf, a.cu, a.cuh, a.N, a.B, a.H, a.T,
                               a.dk, a.dv, a.chunk, (kla_dtype_t)a.dtype, NULL);
}
static kla_status_t gdn(Args a) {
  return kla_gdn_chunk_fwd(a.q, a.k, a.v, a.g, a.eta, a.s0, a.o, a.sf, a.cu, a.cuh, a.N, a.B, a.H, a.T, a.dk, a.dv,
                           a.chunk, (kla_dtype_t)a.dtype, a.ws, a.wsb, NULL);
}
static size_t ws_bytes(Args a) {
  return kla_chunk_workspace_bytes(a.cu, a.cuh, a.N, a.B, a.H, a.T, a.dk, a.dv, a.chunk, (kla_dtype_t)a.dtype);
}
static kla_status_t bwd(Args a, int gdn_mode) {
  if (gdn_mode)
    return kla_gdn_chunk_bwd(a.q, a.k, a.v, a.g, a.eta, a.s0, a.dout, a.dsf, a.dq, a.dk_, a.dv_, a.dg, a.deta, a.ds0,
                             a.cu, a.cuh, a.N, a.B, a.H, a.T, a.dk, a.dv, a.chunk, (kla_dtype_t)a.dtype, a.ws, a.wsb,
                             NULL);
  return kla_chunk_bwd(a.q, a.k, a.v, a.g, a.eta, a.eps, a.s0, a.dout, a.dsf, a.dq, a.dk_, a.dv_, a.dg, a.deta,
                       a.ds0, a.cu, a.cuh, a.N, a.B, a.H, a.T, a.dk, a.dv, a.chunk, (kla_dtype_t)a.dtype, a.ws, a.wsb,
                       NULL);
}

static void status_strings(void) {
  static const int codes[] = {0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -77, 5, INT_MIN, INT_MAX};
  for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
    const char *txt = kla_status_str((kla_status_t)codes[i]);
    expect("status string present", txt != NULL && strlen(txt) > 0, 1);
  }
  expect("abi version", kla_abi_version(), KLA_ABI_VERSION);
}

static void chunk_fwd(void) {
  const float bad_eps[] = {-1.f, NAN, INFINITY};
  Args a;
  a = base(); a.dtype = 7; expect("fwd dtype 7", fwd(a), KLA_ERR_DTYPE);
  a = base(); a.dtype = -1; expect("fwd dtype -1", fwd(a), KLA_ERR_DTYPE);
  a = base(); a.dtype = INT_MIN; expect("fwd dtype min", fwd(a), KLA_ERR_DTYPE);
  a = base(); a.H = 0; expect("fwd H=0", fwd(a), KLA_ERR_SHAPE);
  a = base(); a.T = -1; expect("fwd T<0", fwd(a), KLA_ERR_SHAPE);
  a = base(); a.N = 3; expect("fwd N!=B", fwd(a), KLA_ERR_SHAPE);
  for (int i = 0; i < 3; ++i) { a = base(); a.eps = bad_eps[i]; expect("fwd eps", fwd(a), KLA_ERR_EPS); }
  a = base(); a.dk = 96; expect("fwd dk 96", fwd(a), KLA_ERR_UNSUPPORTED);
  a = base(); a.dk = 256; expect("fwd dk 256", fwd(a), KLA_ERR_UNSUPPORTED);
  a = base(); a.dv = 24; expect("fwd dv 24", fwd(a), KLA_ERR_UNSUPPORTED);
  a = base(); a.dv = 272; expect("fwd dv 272", fwd(a), KLA_ERR_UNSUPPORTED);
  a = base(); a.chunk = 32; expect("fwd chunk", fwd(a), KLA_ERR_UNSUPPORTED);
  a = base(); a.q = NULL; expect("fwd q null", fwd(a), KLA_ERR_NULL);
  a = base(); a.o = NULL; expect("fwd o null", fwd(a), KLA_ERR_NULL);
  a = base(); a.k = fake(8); expect("fwd k align", fwd(a), KLA_ERR_ALIGN);
  a = base(); a.sf = (float *)fake(4); expect("fwd sf align", fwd(a), KLA_ERR_ALIGN);
  a = base(); a.cu = (const int32_t *)FAKE; expect("fwd cu without host", fwd(a), KLA_ERR_NULL);
  a = base(); a.ws = NULL; expect("fwd ws null", fwd(a), KLA_ERR_WORKSPACE);
  a = base(); a.wsb = 1000; expect("fwd ws small", fwd(a), KLA_ERR_WORKSPACE);
  a = base(); a.wsb = ws_bytes(a) - 1; expect("fwd ws one short", fwd(a), KLA_ERR_WORKSPACE);
  a = base(); a.ws = fake(8); expect("fwd ws align", fwd(a), KLA_ERR_ALIGN);
  a = base(); a.N = 0; a.B = 0; expect("fwd nothing to do", fwd(a), KLA_OK);
  /* the contract's shape set passes the shape checks (and stops at the null q) */
  static const int Cs[] = {16, 64}, dks[] = {16, 32, 64, 128}, dvs[] = {16, 128, 256};
  for (int dt = 0; dt < 2; ++dt)
    for (int i = 0; i < 2; ++i)
      for (int j = 0; j < 4; ++j)
        for (int l = 0; l < 3; ++l) {
          a = base(); a.dtype = dt; a.chunk = Cs[i]; a.dk = dks[j]; a.dv = dvs[l]; a.q = NULL;
          expect("fwd supported shape", fwd(a), KLA_ERR_NULL);
        }
}

static void seqlens(void) {
  /* host mirrors of cu_seqlens (the device pointer is never read in validation) */
  static const int32_t dec[] = {0, 30, 20, 100}, short_end[] = {0, 30, 60, 90}, late_start[] = {5, 30, 60, 100};
  static const int32_t good[] = {0, 30, 60, 100};
  Args a = base();
  a.cu = (const int32_t *)FAKE; a.N = 3; a.B = 1;
  a.cuh = dec; expect("seqlens decreasing", fwd(a), KLA_ERR_SEQLENS);
  a.cuh = short_end; expect("seqlens end", fwd(a), KLA_ERR_SEQLENS);
  a.cuh = late_start; expect("seqlens start", fwd(a), KLA_ERR_SEQLENS);
  a.cuh = good; a.B = 2; expect("seqlens B", fwd(a), KLA_ERR_SHAPE);
  a.B = 1; a.cu = (const int32_t *)fake(2); expect("seqlens align", fwd(a), KLA_ERR_ALIGN);
  a.cu = (const int32_t *)FAKE;
  expect("seqlens ws > 0", ws_bytes(a) > 0, 1);
  /* many sequences, lengths 0 .. 9, in a heap array of exactly num_seqs + 1 entries (an
     over-read is caught) */
  const int n = 1000;
  int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (n + 1));
  cu[0] = 0;
  for (int i = 0; i < n; ++i) cu[i + 1] = cu[i] + (i % 10);
  Args m = base();
  m.cu = (const int32_t *)FAKE; m.cuh = cu; m.N = n; m.B = 1; m.T = cu[n];
  expect("many seqlens ws > 0", ws_bytes(m) > 0, 1);
  m.q = NULL; expect("many seqlens reach the pointer checks", fwd(m), KLA_ERR_NULL);
  m.cuh = cu; m.T = cu[n] + 1; expect("many seqlens wrong end", fwd(m), KLA_ERR_SEQLENS);
  free(cu);
}

static void workspace_queries(void) {
  Args a = base();
  expect("ws bf16 > 0", ws_bytes(a) > 0, 1);
  a.dtype = 1; a.chunk = 16; a.dk = 32; a.dv = 16; expect("ws fp32 > 0", ws_bytes(a) > 0, 1);
  a = base(); a.dk = 96; expect("ws unsupported", (long long)ws_bytes(a), 0);
  a = base(); a.T = 0; expect("ws no tokens", (long long)ws_bytes(a), 0);
  a = base(); a.dtype = 9; expect("ws bad dtype", (long long)ws_bytes(a), 0);
  a = base();
  expect("fwd bound >= exact", kla_chunk_fwd_workspace_bytes(2, 4, 100, 128, 128, 64, 2) >= ws_bytes(a), 1);
  expect("fwd bound bad", (long long)kla_chunk_fwd_workspace_bytes(2, 0, 100, 128, 128, 64, 2), 0);
  /* shapes near the limits: the size arithmetic must not overflow (a large size or 0) */
  a = base(); a.B = 1; a.N = 1; a.H = 64; a.T = 1 << 30;
  size_t big = ws_bytes(a);
  expect("ws huge is large or refused", big == 0 || big > ((size_t)1 << 32), 1);
  a.H = 1 << 20;
  (void)ws_bytes(a);
  (void)kla_chunk_fwd_workspace_bytes(1, 1 << 20, 1 << 30, 128, 256, 64, 1);
  (void)kla_chunk_fwd_workspace_bytes(INT_MAX, 2, 2, 128, 128, 64, INT_MAX);
  (void)kla_chunk_fwd_workspace_bytes(1, INT_MAX, INT_MAX - 1, 128, 256, 16, 1);
  (void)kla_chunk_bwd_workspace_bytes(NULL, NULL, 1, 1, 1 << 20, 1 << 30, 128, 256, 64, KLA_DT_BF16);
  (void)kla_pgdn_chunk_workspace_bytes(NULL, NULL, 1, 1, 1 << 20, 1 << 30, 128, 256, 64, KLA_DT_BF16);
}

static kla_status_t fwd_seg(Args a, int seg) {
  return kla_chunk_fwd_seg(a.q, a.k, a.v, a.g, a.eta, a.eps, a.s0, a.o, a.sf, a.cu, a.cuh, a.N, a.B, a.H, a.T,
                           a.dk, a.dv, a.chunk, (kla_dtype_t)a.dtype, seg, a.ws, a.wsb, NULL);
}
static size_t seg_bytes(Args a, int seg) {
  return kla_chunk_seg_workspace_bytes(a.cu, a.cuh, a.N, a.B, a.H, a.T, a.dk, a.dv, a.chunk,
                                       (kla_dtype_t)a.dtype, seg);
}

static void segmented(void) {
  Args a = base();
  expect("seg -1", fwd_seg(a, -1), KLA_ERR_SHAPE);
  expect("seg INT_MIN", fwd_seg(a, INT_MIN), KLA_ERR_SHAPE);
  a = base(); a.dtype = 7; expect("seg dtype", fwd_seg(a, 2), KLA_ERR_DTYPE);
  a = base(); a.dtype = 1; a.chunk = 64; a.dk = 128; expect("seg general shape", fwd_seg(a, 2), KLA_ERR_UNSUPPORTED);
  a = base(); a.q = NULL; expect("seg null", fwd_seg(a, 2), KLA_ERR_NULL);
  a = base(); a.wsb = seg_bytes(a, 2) - 1; expect("seg ws one short", fwd_seg(a, 2), KLA_ERR_WORKSPACE);
  a = base(); a.N = 0; a.B = 0; expect("seg nothing to do", fwd_seg(a, 2), KLA_OK);
  a = base();
  expect("seg 0 = plain", (long long)seg_bytes(a, 0), (long long)ws_bytes(a));
  expect("seg 1 > plain", seg_bytes(a, 1) > ws_bytes(a), 1);
  expect("seg bytes negative", (long long)seg_bytes(a, -3), 0);
  expect("seg huge length = one segment each", seg_bytes(a, INT_MAX) > ws_bytes(a), 1);
  /* the library's own choice on a long sequence */
  a = base(); a.N = 1; a.B = 1; a.H = 16; a.T = 65536; a.dv = 256;
  expect("auto segments", (long long)ws_bytes(a), (long long)seg_bytes(a, 342));
  /* packed, with a heap mirror of exactly num_seqs + 1 entries */
  const int n = 300;
  int32_t *cu = (int32_t *)malloc(sizeof(int32_t) * (n + 1));
  cu[0] = 0;
  for (int i = 0; i < n; ++i) cu[i + 1] = cu[i] + (i % 7 == 0 ? 5000 : i % 3);
  Args m = base();
  m.cu = (const int32_t *)FAKE; m.cuh = cu; m.N = n; m.B = 1; m.T = cu[n]; m.H = 1; m.dv = 64;
  expect("seg packed bytes", seg_bytes(m, 3) > ws_bytes(m), 1);
  m.q = NULL; expect("seg packed reaches the pointer checks", fwd_seg(m, 3), KLA_ERR_NULL);
  (void)ws_bytes(m);
  free(cu);
  /* sizes near the limits */
  a = base(); a.N = 1; a.B = 1; a.H = 1; a.T = 1 << 30; a.dv = 256;
  (void)ws_bytes(a);
  (void)seg_bytes(a, 1);
  (void)seg_bytes(a, 7);
  a.H = 1 << 20;
  (void)seg_bytes(a, 1);
}

static void noalloc_limits(void) {
  Args a = base();
  a.N = 4; a.B = 4; a.H = 64; a.T = 8192;
  expect("noalloc over the scratch", ws_bytes(a) > KLA_NOALLOC_SCRATCH_BYTES, 1);
  expect("noalloc refuses", noalloc(a), KLA_ERR_SCRATCH);
  a = base(); a.dtype = 7; expect("noalloc dtype", noalloc(a), KLA_ERR_DTYPE);
  a = base(); a.eps = -1.f; expect("noalloc eps", noalloc(a), KLA_ERR_EPS);
  a = base(); a.q = NULL; expect("noalloc null", noalloc(a), KLA_ERR_NULL);
  a = base(); a.N = 0; a.B = 0; expect("noalloc nothing to do", noalloc(a), KLA_OK);
}

static kla_status_t dec(int dtype, int N, int H, int dk, int dv, float eps, float *S, const void *v, int gdn_mode,
                        const void *eta) {
  if (gdn_mode) return kla_gdn_decode_step(FAKE, FAKE, v, FAKE, eta, S, FAKE, N, H, dk, dv, (kla_dtype_t)dtype, NULL);
  return kla_decode_step(FAKE, FAKE, v, FAKE, eta, eps, S, FAKE, N, H, dk, dv, (kla_dtype_t)dtype, NULL);
}

static void decode(void) {
  float *S = (float *)FAKE;
  expect("dec dtype", dec(2, 3, 2, 128, 128, 1e-6f, S, FAKE, 0, FAKE), KLA_ERR_DTYPE);
  expect("dec H", dec(0, 3, 0, 128, 128, 1e-6f, S, FAKE, 0, FAKE), KLA_ERR_SHAPE);
  expect("dec N", dec(0, -1, 2, 128, 128, 1e-6f, S, FAKE, 0, FAKE), KLA_ERR_SHAPE);
  expect("dec eps", dec(0, 3, 2, 128, 128, -0.5f, S, FAKE, 0, FAKE), KLA_ERR_EPS);
  expect("dec dk", dec(0, 3, 2, 48, 128, 1e-6f, S, FAKE, 0, FAKE), KLA_ERR_UNSUPPORTED);
  expect("dec dv", dec(0, 3, 2, 128, 512, 1e-6f, S, FAKE, 0, FAKE), KLA_ERR_UNSUPPORTED);
  expect("dec S null", dec(0, 3, 2, 128, 128, 1e-6f, NULL, FAKE, 0, FAKE), KLA_ERR_NULL);
  expect("dec v align", dec(0, 3, 2, 128, 128, 1e-6f, S, fake(2), 0, FAKE), KLA_ERR_ALIGN);
  expect("dec nothing", dec(0, 0, 2, 128, 128, 1e-6f, S, FAKE, 0, FAKE), KLA_OK);
  expect("gdn dec dv", dec(0, 3, 2, 128, 24, 0.f, S, FAKE, 1, FAKE), KLA_ERR_UNSUPPORTED);
  expect("gdn dec beta null", dec(0, 3, 2, 128, 128, 0.f, S, FAKE, 1, NULL), KLA_ERR_NULL);
  expect("gdn dec dtype", dec(5, 3, 2, 128, 128, 0.f, S, FAKE, 1, FAKE), KLA_ERR_DTYPE);
  expect("gdn dec nothing", dec(0, 0, 2, 128, 128, 0.f, S, FAKE, 1, FAKE), KLA_OK);
}

static void gdn_chunk(void) {
  Args a;
  a = base(); a.dtype = 5; expect("gdn dtype", gdn(a), KLA_ERR_DTYPE);
  a = base(); a.T = -3; expect("gdn T", gdn(a), KLA_ERR_SHAPE);
  a = base(); a.eta = NULL; expect("gdn beta null", gdn(a), KLA_ERR_NULL);
  a = base(); a.eta = fake(4); expect("gdn beta align", gdn(a), KLA_ERR_ALIGN);
  a = base(); a.ws = NULL; expect("gdn ws", gdn(a), KLA_ERR_WORKSPACE);
  a = base(); a.N = 0; a.B = 0; expect("gdn nothing", gdn(a), KLA_OK);
}

static void backward(void) {
  for (int m = 0; m < 2; ++m) {
    Args a;
    a = base(); a.chunk = 16; expect("bwd chunk 16", bwd(a, m), KLA_ERR_UNSUPPORTED);
    a = base(); a.dk = 16; expect("bwd dk 16", bwd(a, m), KLA_ERR_UNSUPPORTED);
    a = base(); a.dtype = 1; expect("bwd fp32 chunk 64 dk 128", bwd(a, m), KLA_ERR_UNSUPPORTED);
    a = base(); a.dtype = 7; expect("bwd dtype", bwd(a, m), KLA_ERR_DTYPE);
    a = base(); a.H = 0; expect("bwd H", bwd(a, m), KLA_ERR_SHAPE);
    a = base(); a.N = 3; expect("bwd N", bwd(a, m), KLA_ERR_SHAPE);
    a = base(); a.dout = NULL; expect("bwd dout", bwd(a, m), KLA_ERR_NULL);
    a = base(); a.dq = NULL; expect("bwd dq", bwd(a, m), KLA_ERR_NULL);
    a = base(); a.dg = NULL; expect("bwd dg", bwd(a, m), KLA_ERR_NULL);
    a = base(); a.deta = NULL; expect("bwd deta", bwd(a, m), KLA_ERR_NULL);
    a = base(); a.dk_ = fake(8); expect("bwd dk align", bwd(a, m), KLA_ERR_ALIGN);
    a = base(); a.ds0 = (float *)fake(4); expect("bwd ds0 align", bwd(a, m), KLA_ERR_ALIGN);
    a = base(); a.dsf = (const float *)fake(4); expect("bwd dsf align", bwd(a, m), KLA_ERR_ALIGN);
    a = base(); a.cu = (const int32_t *)FAKE; expect("bwd cu", bwd(a, m), KLA_ERR_NULL);
    a = base(); a.ws = NULL; expect("bwd ws", bwd(a, m), KLA_ERR_WORKSPACE);
    a = base(); a.wsb = 1000; expect("bwd ws small", bwd(a, m), KLA_ERR_WORKSPACE);
    a = base(); a.N = 0; a.B = 0; expect("bwd nothing", bwd(a, m), KLA_OK);
  }
  Args a = base();
  a.eps = -1.f; expect("bwd eps", bwd(a, 0), KLA_ERR_EPS);
  const size_t w = kla_chunk_bwd_workspace_bytes(NULL, NULL, 2, 2, 4, 100, 128, 128, 64, KLA_DT_BF16);
  expect("bwd ws > fwd ws", w > ws_bytes(base()), 1);
  a = base(); a.wsb = w - 1; expect("bwd ws one short", bwd(a, 0), KLA_ERR_WORKSPACE);
}

static kla_status_t pg(int gain, float band, float eps, int dtype, int dk, int chunk, int N, const void *c,
                       const float *a0, void *ws, size_t wsb) {
  return kla_pgdn_chunk_fwd(FAKE, FAKE, FAKE, FAKE, c, eps, (kla_gain_t)gain, band, NULL, a0, FAKE, NULL, NULL, NULL,
                            NULL, N, 2, 4, 100, dk, 128, chunk, (kla_dtype_t)dtype, ws, wsb, NULL);
}

static void pgdn(void) {
  expect("pgdn gain 2", pg(2, 1.5f, 1e-6f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_PARAM);
  expect("pgdn gain -1", pg(-1, 1.5f, 1e-6f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_PARAM);
  expect("pgdn band 0.9", pg(0, 0.9f, 1e-6f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_PARAM);
  expect("pgdn band nan", pg(0, NAN, 1e-6f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_PARAM);
  expect("pgdn band inf", pg(0, INFINITY, 1e-6f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_PARAM);
  expect("pgdn eps", pg(1, 1.5f, -1.f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_EPS);
  expect("pgdn dtype", pg(0, 1.5f, 1e-6f, 3, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_DTYPE);
  expect("pgdn dk", pg(0, 1.5f, 1e-6f, 0, 96, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_UNSUPPORTED);
  expect("pgdn chunk", pg(0, 1.5f, 1e-6f, 0, 128, 32, 2, FAKE, NULL, NULL, 0), KLA_ERR_UNSUPPORTED);
  expect("pgdn coef", pg(0, 1.5f, 1e-6f, 0, 128, 64, 2, NULL, NULL, NULL, 0), KLA_ERR_NULL);
  expect("pgdn a0 align", pg(0, 1.5f, 1e-6f, 0, 128, 64, 2, FAKE, (const float *)fake(4), NULL, 0), KLA_ERR_ALIGN);
  expect("pgdn N", pg(0, 1.5f, 1e-6f, 0, 128, 64, 3, FAKE, NULL, NULL, 0), KLA_ERR_SHAPE);
  expect("pgdn without workspace", pg(0, 1.5f, 1e-6f, 0, 128, 64, 2, FAKE, NULL, NULL, 0), KLA_ERR_WORKSPACE);
  const size_t w = kla_pgdn_chunk_workspace_bytes(NULL, NULL, 2, 2, 4, 100, 128, 128, 64, KLA_DT_BF16);
  expect("pgdn ws > 0", w > 0, 1);
  expect("pgdn ws one short", pg(0, 1.5f, 1e-6f, 0, 128, 64, 2, FAKE, NULL, FAKE, w - 1), KLA_ERR_WORKSPACE);
  float *S = (float *)FAKE, *A = (float *)FAKE;
  expect("pgdn dec gain", kla_pgdn_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6f, (kla_gain_t)5, 1.5f, S, A, FAKE, 3,
                                               2, 128, 128, KLA_DT_BF16, NULL), KLA_ERR_PARAM);
  expect("pgdn dec acc null", kla_pgdn_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6f, KLA_GAIN_KACZMARZ, 1.5f, S,
                                                   NULL, FAKE, 3, 2, 128, 128, KLA_DT_BF16, NULL), KLA_ERR_NULL);
  expect("pgdn dec dtype", kla_pgdn_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6f, KLA_GAIN_KACZMARZ, 1.5f, S, A,
                                                FAKE, 3, 2, 128, 128, (kla_dtype_t)9, NULL), KLA_ERR_DTYPE);
  expect("pgdn dec nothing", kla_pgdn_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6f, KLA_GAIN_KACZMARZ, 1.5f, S, A,
                                                  FAKE, 0, 2, 128, 128, KLA_DT_BF16, NULL), KLA_OK);
}

int main(void) {
  status_strings();
  chunk_fwd();
  seqlens();
  workspace_queries();
  noalloc_limits();
  segmented();
  decode();
  gdn_chunk();
  backward();
  pgdn();
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
