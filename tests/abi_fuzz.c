/*
 * Host-side check of the C ABI (include/qw.h), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer on the host code of libqw (see
 * tests/test_host_sanitizers.py, which builds and runs it on a machine
 * without a GPU).
 *
 * Part 1 calls every entry point with arguments whose status is known --
 * invalid bits, groups, shapes, counts, m, NULL pointers, sizes at and just
 * beyond the limits -- and checks each status.  Part 2 draws arguments from
 * edge-value sets (negative, zero, small, ragged, 2^31 - 1, 2^31, 2^40,
 * INT64_MAX, misaligned pointers, batches longer than one launch) with a
 * seeded generator and checks that every call returns one of the documented
 * statuses.  With no GPU, calls that pass validation run the dispatch code on
 * the host up to the kernel launch, which fails with QW_EHIP; the sanitizers
 * watch all of it (integer overflow, out-of-bounds host arrays, use of
 * uninitialized descriptors).  Pointers are fake device addresses that the
 * host code never dereferences; if a GPU is visible the driver runs only the
 * calls that fail validation.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qw.h"

/* from the HIP runtime (C linkage; hipError_t is an enum) */
int hipGetDeviceCount(int* count);

static int g_fail = 0;
static long g_calls = 0;
static long g_hist[16];

static void seen(int st) {
  ++g_calls;
  if (st > 0 || st < -10) {
    printf("FAIL: undocumented status %d\n", st);
    ++g_fail;
    return;
  }
  ++g_hist[-st];
}

#define EXPECT(call, want)                                                        \
  do {                                                                            \
    int st_ = (int)(call);                                                        \
    seen(st_ < 0 && st_ >= -10 ? st_ : 0);                                        \
    if (st_ != (want)) {                                                          \
      printf("FAIL line %d: %s returned %d, expected %d\n", __LINE__, #call, st_, \
             (int)(want));                                                        \
      ++g_fail;                                                                   \
    }                                                                             \
  } while (0)

#define EXPECT64(call, want)                                                            \
  do {                                                                                  \
    int64_t v_ = (call);                                                                \
    ++g_calls;                                                                          \
    if (v_ != (int64_t)(want)) {                                                        \
      printf("FAIL line %d: %s returned %lld, expected %lld\n", __LINE__, #call,        \
             (long long)v_, (long long)(want));                                         \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

/* fake device addresses: 256-aligned, 4-aligned, unaligned */
#define PA ((void*)(uintptr_t)0x7f0000000000ull)
#define P4 ((void*)(uintptr_t)0x7f0000000004ull)
#define P1 ((void*)(uintptr_t)0x7f0000000001ull)

static const int64_t MAXE = QW_MAX_ELEMENTS;

static void fixed_cases(int launches_ok) {
  /* sizes */
  EXPECT64(qw_payload_bytes(4, 11008, 4096), 11008ll * 4096 / 2);
  EXPECT64(qw_payload_bytes(8, 0, 5), 0);
  EXPECT64(qw_payload_bytes(4, 3, 3), -1);
  EXPECT64(qw_payload_bytes(6, 4, 4), -1);
  EXPECT64(qw_payload_bytes(8, -1, 4), -1);
  EXPECT64(qw_payload_bytes(8, MAXE, 1), MAXE);
  EXPECT64(qw_payload_bytes(8, MAXE, 2), -1);
  EXPECT64(qw_payload_bytes(8, INT64_MAX, INT64_MAX), -1);
  EXPECT64(qw_payload_bytes(4, 1ll << 40, 0), -1);
  EXPECT64(qw_num_scales(128, 11008, 4096), 11008ll * 32);
  EXPECT64(qw_num_scales(0, 4, 4), -1);
  EXPECT64(qw_num_scales(-5, 4, 4), -1);
  EXPECT64(qw_num_scales(3, 4, 4), -1);
  EXPECT64(qw_num_scales(INT64_MAX, 0, 0), 0);
  EXPECT64(qw_num_scales(1, INT64_MAX, 2), -1);
  EXPECT64(qw_matmul_work_bytes(-1, 8), -1);
  EXPECT64(qw_matmul_work_bytes(4, 8), 0);
  EXPECT64(qw_matmul_work_bytes(MAXE, 2), -1);
  EXPECT64(qw_gptq_factor_work_bytes(INT64_MAX), -1);
  EXPECT64(qw_gptq_factor_work_bytes(QW_GPTQ_MAX_K + 1), -1);
  EXPECT64(qw_gptq_hessian_work_bytes(INT64_MAX - 10, 1), -1);
  EXPECT64(qw_gptq_hessian_work_bytes(64, INT64_MAX), -1);
  EXPECT64(qw_gptq_quantize_work_bytes(1, INT64_MAX - 3), -1);
  EXPECT64(qw_gptq_quantize_work_bytes(QW_GPTQ_MAX_N + 1, 64), -1);
  for (int s = -20; s <= 5; ++s) {
    const char* t = qw_status_string(s);
    if (!t || !t[0]) {
      printf("FAIL: empty status string for %d\n", s);
      ++g_fail;
    }
  }
  if (!qw_last_error()) {
    printf("FAIL: qw_last_error returned NULL\n");
    ++g_fail;
  }

  /* validation failures (nothing is launched) */
  EXPECT(qw_quantize_pack(5, 32, 4, 32, PA, PA, PA, 0), QW_EBITS);
  EXPECT(qw_quantize_pack(4, 0, 4, 32, PA, PA, PA, 0), QW_EGROUP);
  EXPECT(qw_quantize_pack(4, 3, 4, 32, PA, PA, PA, 0), QW_EGROUP);
  EXPECT(qw_quantize_pack(4, 1, 3, 3, PA, PA, PA, 0), QW_ESHAPE);
  EXPECT(qw_quantize_pack(4, 32, -4, 32, PA, PA, PA, 0), QW_ESHAPE);
  EXPECT(qw_quantize_pack(8, 1, MAXE, 2, PA, PA, PA, 0), QW_ESHAPE);
  EXPECT(qw_quantize_pack(8, 1, INT64_MAX, INT64_MAX, PA, PA, PA, 0), QW_ESHAPE);
  EXPECT(qw_quantize_pack(8, 1, 1ll << 40, 0, PA, PA, PA, 0), QW_ESHAPE);
  EXPECT(qw_quantize_pack(4, 32, 4, 32, 0, PA, PA, 0), QW_ENULL);
  EXPECT(qw_quantize_pack(4, 32, 0, 32, 0, 0, 0, 0), QW_OK);
  EXPECT(qw_unpack(4, 32, 4, 32, PA, 0, PA, 0), QW_ENULL);
  EXPECT(qw_unpack(8, 7, 4, 32, PA, PA, PA, 0), QW_EGROUP);
  EXPECT(qw_gemv(4, 32, 4, 32, PA, PA, 9, PA, PA, 0), QW_EM);
  EXPECT(qw_gemv(4, 32, 4, 32, PA, PA, -1, PA, PA, 0), QW_EM);
  EXPECT(qw_gemv(4, 32, 4, 32, PA, PA, 0, 0, 0, 0), QW_OK);
  /* k == 0 with a huge n: n*k is 0, yet m*n outputs must stay in range */
  EXPECT(qw_gemv(4, 1, MAXE, 0, 0, 0, 8, 0, PA, 0), QW_EM);
  EXPECT(qw_gemv(4, 1, INT64_MAX, 0, 0, 0, 8, 0, PA, 0), QW_ESHAPE);
  EXPECT(qw_gemv(4, 32, 4, 32, PA, PA, 1, PA, 0, 0), QW_ENULL);
  EXPECT(qw_gemm(4, 128, 256, 256, PA, PA, -1, PA, PA, 0), QW_EM);
  EXPECT(qw_gemm(4, 128, 256, 256, PA, PA, MAXE, PA, PA, 0), QW_EM);
  EXPECT(qw_gemm(4, 128, 256, 256, PA, PA, INT64_MAX, PA, PA, 0), QW_EM);
  EXPECT(qw_matmul(4, 128, 256, 256, PA, PA, 300, PA, PA, 0, 0, 0), QW_EWORK);
  EXPECT(qw_matmul(4, 128, 256, 256, PA, PA, 300, PA, PA, PA, 1, 0), QW_EWORK);
  EXPECT(qw_matmul_noalloc(4, 128, 256, 1 << 20, PA, PA, 300, PA, PA, 0), QW_ESCRATCH);
  EXPECT(qw_matmul_noalloc(4, 128, 256, 256, PA, PA, 300, PA, 0, 0), QW_ENULL);
  EXPECT(qw_gptq_hessian(-1, 8, PA, PA, PA, 1 << 20, 0), QW_ESHAPE);
  EXPECT(qw_gptq_hessian(QW_GPTQ_MAX_K + 1, 8, PA, PA, PA, 1 << 20, 0), QW_ESHAPE);
  EXPECT(qw_gptq_hessian(64, 64, PA, PA, PA, 0, 0), QW_EWORK);
  EXPECT(qw_gptq_factor(64, PA, -1.0, PA, PA, PA, 1 << 20, 0), QW_EARG);
  EXPECT(qw_gptq_factor(INT64_MAX - 10, PA, 0.01, PA, PA, PA, 1 << 20, 0), QW_ESHAPE);
  EXPECT(qw_gptq_quantize_pack(4, 3, 4, 64, PA, PA, PA, PA, PA, 1 << 30, 0), QW_EGROUP);
  EXPECT(qw_gptq_quantize_pack(4, 32, 4, INT64_MAX - 3, PA, PA, PA, PA, PA, 1 << 30, 0),
         QW_ESHAPE);
  EXPECT(qw_gptq_quantize_pack(4, 32, 4, 64, PA, PA, PA, PA, PA, 0, 0), QW_EWORK);

  /* batched calls: validation of every descriptor before anything is launched */
  {
    qw_quant_desc qd[3];
    memset(qd, 0, sizeof(qd));
    for (int i = 0; i < 3; ++i) {
      qd[i].bits = 4; qd[i].group = 32; qd[i].n = 64; qd[i].k = 128;
      qd[i].w = PA; qd[i].payload = PA; qd[i].scales = PA;
    }
    EXPECT(qw_quantize_pack_batched(-1, qd, 0), QW_ECOUNT);
    EXPECT(qw_quantize_pack_batched(0, 0, 0), QW_OK);
    EXPECT(qw_quantize_pack_batched(3, 0, 0), QW_ENULL);
    qd[2].reserved = 1;
    EXPECT(qw_quantize_pack_batched(3, qd, 0), QW_ECOUNT);
    qd[2].reserved = 0;
    qd[1].group = 0;
    EXPECT(qw_quantize_pack_batched(3, qd, 0), QW_EGROUP);
    qd[1].group = 32;
    qd[2].w = 0;
    EXPECT(qw_quantize_pack_batched(3, qd, 0), QW_ENULL);
  }
  {
    qw_gemv_desc gd[2];
    int32_t stage[2] = {1, 0};
    memset(gd, 0, sizeof(gd));
    for (int i = 0; i < 2; ++i) {
      gd[i].bits = 4; gd[i].group = 32; gd[i].n = 64; gd[i].k = 128;
      gd[i].payload = PA; gd[i].scales = PA; gd[i].x = PA; gd[i].y = PA;
    }
    EXPECT(qw_gemv_batched(2, gd, 9, 0), QW_EM);
    EXPECT(qw_gemv_chain(2, gd, stage, 1, 0), QW_ECOUNT);
    EXPECT(qw_gemv_chain(2, gd, 0, 1, 0), QW_ECOUNT);
    gd[1].n = MAXE;
    gd[1].k = 0;
    EXPECT(qw_gemv_batched(2, gd, 8, 0), QW_EM);
    stage[0] = 0;
    EXPECT(qw_gemv_chain(2, gd, stage, 8, 0), QW_EM);
  }
  {
    qw_unpack_desc ud[1];
    memset(ud, 0, sizeof(ud));
    ud[0].bits = 8; ud[0].group = 4; ud[0].n = 4; ud[0].k = 4;
    ud[0].payload = PA; ud[0].scales = PA;
    EXPECT(qw_unpack_batched(1, ud, 0), QW_ENULL);
  }

  if (!launches_ok) return;
  /* valid calls: with no GPU the launch fails (QW_EHIP); the host dispatch
     up to it runs under the sanitizers, for every kernel family */
  EXPECT(qw_quantize_pack(4, 32, 4096, 4096, PA, PA, PA, 0), QW_EHIP);
  EXPECT(qw_quantize_pack(4, 12, 96, 96, PA, PA, PA, 0), QW_EHIP);      /* block path */
  EXPECT(qw_quantize_pack(4, 100, 10, 100, P1, PA, PA, 0), QW_EHIP);    /* generic */
  EXPECT(qw_quantize_pack(8, 4, MAXE / 4, 4, PA, PA, PA, 0), QW_EHIP);  /* at the limit */
  EXPECT(qw_quantize_pack(8, 12, MAXE / 16, 12, PA, PA, PA, 0), QW_EHIP);
  EXPECT(qw_quantize_pack(8, 65, MAXE / 65, 65, P1, PA, PA, 0), QW_EHIP);
  EXPECT(qw_quantize_pack(4, 32, MAXE / 32, 32, PA, PA, PA, 0), QW_EHIP); /* several launches */
  {
    qw_quant_desc big[2];
    memset(big, 0, sizeof(big));
    for (int i = 0; i < 2; ++i) {
      big[i].bits = 4; big[i].group = 32; big[i].w = PA; big[i].payload = PA; big[i].scales = PA;
    }
    big[0].n = MAXE / 64; big[0].k = 64;  /* too large to share a launch */
    big[1].n = 64; big[1].k = 64;
    EXPECT(qw_quantize_pack_batched(2, big, 0), QW_EHIP);
  }
  EXPECT(qw_unpack(4, 32, MAXE / 32, 32, PA, PA, PA, 0), QW_EHIP);
  EXPECT(qw_unpack(8, 7, MAXE / 7, 7, P1, PA, PA, 0), QW_EHIP);
  EXPECT(qw_gemv(4, 128, 11008, 4096, PA, PA, 4, PA, PA, 0), QW_EHIP);
  EXPECT(qw_gemv(4, 1, MAXE / 8, 0, 0, 0, 8, 0, PA, 0), QW_EHIP);       /* zero fill */
  EXPECT(qw_gemv(8, 3, MAXE / 3, 3, P1, PA, 1, PA, PA, 0), QW_EHIP);    /* generic */
  EXPECT(qw_gemv(8, 8, MAXE / 8, 8, PA, PA, 8, PA, PA, 0), QW_EHIP);   /* m*n at the limit */
  EXPECT(qw_gemv(8, 1, MAXE / 4, 1, PA, PA, 8, PA, PA, 0), QW_EM);     /* m*n over */
  EXPECT(qw_gemv(8, 8, MAXE / 64, 8, PA, PA, 8, PA, PA, 0), QW_EHIP);
  EXPECT(qw_gemm(4, 128, 28672, 8192, PA, PA, 2048, PA, PA, 0), QW_EHIP);
  EXPECT(qw_gemm(4, 128, 28672, 8192, PA, PA, 17, PA, PA, 0), QW_EHIP); /* small M */
  EXPECT(qw_gemm(8, 3, 99, 33, P1, PA, 5, PA, PA, 0), QW_EHIP);         /* generic */
  EXPECT(qw_gemm(8, 64, MAXE / 64, 64, PA, PA, 32, PA, PA, 0), QW_EHIP); /* small-M grid */
  EXPECT(qw_gemm(8, 8, MAXE / 16, 8, PA, PA, 32, PA, PA, 0), QW_EM);     /* m*n over */
  EXPECT(qw_gemm(8, 64, MAXE / 2048, 64, PA, PA, 32, PA, PA, 0), QW_EHIP);
  EXPECT(qw_matmul(4, 128, 4096, 4096, PA, PA, 300, PA, PA, PA, 1 << 30, 0), QW_EHIP);
  EXPECT(qw_matmul_noalloc(4, 128, 4096, 4096, PA, PA, 300, PA, PA, 0), QW_EHIP);
  EXPECT(qw_gptq_hessian(1368, 8192, PA, PA, PA, qw_gptq_hessian_work_bytes(1368, 8192), 0),
         QW_EHIP);
  EXPECT(qw_gptq_factor(1368, PA, 0.01, PA, PA, PA, qw_gptq_factor_work_bytes(1368), 0),
         QW_EHIP);
  EXPECT(qw_gptq_quantize_pack(4, 64, 1368, 512, PA, PA, PA, PA, PA,
                               qw_gptq_quantize_work_bytes(1368, 512), 0),
         QW_EHIP);
}

/* ------------------------------------------------------------ fuzz */

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void) { /* xorshift64* */
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return g_rng * 0x2545F4914F6CDD1Dull;
}
static int64_t pick(const int64_t* v, int n) { return v[rnd() % (uint64_t)n]; }

static const int64_t kDims[] = {-1, 0, 1, 2, 3, 7, 8, 31, 32, 33, 64, 100, 128, 255, 256,
                                4096, 11008, 28672, (1ll << 31) - 1, 1ll << 31, 1ll << 40,
                                INT64_MAX - 63, INT64_MAX};
static const int64_t kGroups[] = {-3, 0, 1, 2, 3, 4, 8, 12, 32, 64, 65, 96, 128, 256, 1024,
                                  4096, 1ll << 20, 1ll << 31, INT64_MAX};
static const int64_t kMs[] = {-1, 0, 1, 2, 4, 5, 8, 9, 17, 32, 33, 300, 2048, 1ll << 31,
                              INT64_MAX};

static void* ptr(int allow_null) {
  switch (rnd() % (allow_null ? 4 : 3)) {
    case 0: return PA;
    case 1: return P4;
    case 2: return P1;
    default: return 0;
  }
}

static void fuzz(long iters, int launches_ok) {
  static qw_quant_desc qd[300];
  static qw_unpack_desc ud[300];
  static qw_gemv_desc gd[300];
  static int32_t stage[300];
  for (long it = 0; it < iters; ++it) {
    const int bits = (int)(rnd() % 3 == 0 ? pick((const int64_t[]){-1, 0, 5, 16}, 4)
                                          : (rnd() & 1 ? 4 : 8));
    const int64_t group = pick(kGroups, (int)(sizeof(kGroups) / sizeof(kGroups[0])));
    const int64_t n = pick(kDims, (int)(sizeof(kDims) / sizeof(kDims[0])));
    const int64_t k = pick(kDims, (int)(sizeof(kDims) / sizeof(kDims[0])));
    const int64_t m = pick(kMs, (int)(sizeof(kMs) / sizeof(kMs[0])));
    const int op = (int)(rnd() % 14);
    int st = 0;
    /* without launches, keep only calls that must fail validation: a NULL
       output (or another required pointer) makes every valid call fail */
    void* out = launches_ok ? ptr(1) : 0;
    switch (op) {
      case 0: st = qw_quantize_pack(bits, group, n, k, ptr(1), out, ptr(1), 0); break;
      case 1: st = qw_unpack(bits, group, n, k, ptr(1), ptr(1), out, 0); break;
      case 2: st = qw_gemv(bits, group, n, k, ptr(1), ptr(1), m, ptr(1), out, 0); break;
      case 3: st = qw_gemm(bits, group, n, k, ptr(1), ptr(1), m, ptr(1), out, 0); break;
      case 4: st = qw_matmul(bits, group, n, k, ptr(1), ptr(1), m, ptr(1), out, ptr(1),
                             (int64_t)(rnd() % 3) << 28, 0); break;
      case 5: st = qw_matmul_noalloc(bits, group, n, k, ptr(1), ptr(1), m, ptr(1), out, 0);
        break;
      case 6: st = qw_gptq_hessian(k, m, ptr(1), out, ptr(1), (int64_t)(rnd() % 3) << 30, 0);
        break;
      case 7: st = qw_gptq_factor(k, ptr(1), (rnd() & 1) ? 0.01 : -1.0, out, ptr(1), ptr(1),
                                  (int64_t)(rnd() % 3) << 30, 0);
        break;
      case 8: st = qw_gptq_quantize_pack(bits, group, n, k, ptr(1), ptr(1), out, ptr(1), ptr(1),
                                         (int64_t)(rnd() % 3) << 30, 0);
        break;
      case 9:
      case 10:
      case 11:
      case 12: {
        const int count = (int)(rnd() % 4 == 0 ? pick((const int64_t[]){-1, 0, 257, 300}, 4)
                                               : 1 + (int64_t)(rnd() % 6));
        const int cnt = count > 0 ? count : 0;
        for (int i = 0; i < cnt; ++i) {
          const int b = rnd() % 5 == 0 ? 5 : (rnd() & 1 ? 4 : 8);
          /* mostly sane shapes, so that long batches reach the chunking */
          const int64_t dn = rnd() % 4 ? pick((const int64_t[]){0, 64, 100, 4096}, 4)
                                       : pick(kDims, (int)(sizeof(kDims) / sizeof(kDims[0])));
          const int64_t dk = rnd() % 4 ? pick((const int64_t[]){0, 128, 4096}, 3)
                                       : pick(kDims, (int)(sizeof(kDims) / sizeof(kDims[0])));
          const int64_t dg = rnd() % 4 ? 32 : pick(kGroups, (int)(sizeof(kGroups) / sizeof(kGroups[0])));
          const int64_t res = rnd() % 50 == 0 ? 1 : 0;
          void* o = launches_ok ? ptr(1) : 0;
          memset(&qd[i], 0, sizeof(qd[i]));
          qd[i].bits = b; qd[i].group = dg; qd[i].n = dn; qd[i].k = dk; qd[i].reserved = res;
          qd[i].w = ptr(1); qd[i].payload = o; qd[i].scales = ptr(1);
          memset(&ud[i], 0, sizeof(ud[i]));
          ud[i].bits = b; ud[i].group = dg; ud[i].n = dn; ud[i].k = dk; ud[i].reserved = res;
          ud[i].payload = ptr(1); ud[i].scales = ptr(1); ud[i].w_out = o;
          memset(&gd[i], 0, sizeof(gd[i]));
          gd[i].bits = b; gd[i].group = dg; gd[i].n = dn; gd[i].k = dk; gd[i].reserved = res;
          gd[i].payload = ptr(1); gd[i].scales = ptr(1); gd[i].x = ptr(1); gd[i].y = o;
          stage[i] = i / 3 - (rnd() % 40 == 0 ? 5 : 0);
        }
        if (!launches_ok && cnt > 0) {
          /* make sure one descriptor cannot pass: n * k > 0 with NULL outputs */
          qd[0].n = ud[0].n = gd[0].n = 64;
          qd[0].k = ud[0].k = gd[0].k = 128;
          qd[0].bits = ud[0].bits = gd[0].bits = 8;
          qd[0].group = ud[0].group = gd[0].group = 32;
          qd[0].reserved = ud[0].reserved = gd[0].reserved = 0;
        }
        const int mm = (int)(m > 8 ? 8 : (m < -1 ? -1 : m));
        if (op == 9) st = qw_quantize_pack_batched(count, qd, 0);
        else if (op == 10) st = qw_unpack_batched(count, ud, 0);
        else if (op == 11) st = qw_gemv_batched(count, gd, launches_ok ? m : (mm > 0 ? mm : 1), 0);
        else st = qw_gemv_chain(count, gd, stage, launches_ok ? m : (mm > 0 ? mm : 1), 0);
        break;
      }
      default: st = qw_debug_path((int)(rnd() % 7), bits, group, n, k, ptr(1), ptr(1)); break;
    }
    if (op == 13) {
      ++g_calls;
      if (st < -10 || st > 4) {
        printf("FAIL: qw_debug_path returned %d\n", st);
        ++g_fail;
      }
      continue;
    }
    seen(st);
    if (!launches_ok && st == QW_OK && op < 9 && out != 0) {
      printf("FAIL: op %d passed validation without a GPU\n", op);
      ++g_fail;
    }
  }
}

int main(int argc, char** argv) {
  long iters = argc > 1 ? atol(argv[1]) : 20000;
  int devices = 0;
  if (hipGetDeviceCount(&devices) != 0) devices = 0;
  const int launches_ok = devices == 0;
  if (!launches_ok) printf("a GPU is visible: only calls that fail validation are made\n");
  fixed_cases(launches_ok);
  fuzz(iters, launches_ok);
  printf("abi_fuzz: %ld calls, %d failures; statuses:", g_calls, g_fail);
  for (int i = 0; i <= 10; ++i) printf(" %d:%ld", -i, g_hist[i]);
  printf("\n");
  return g_fail ? 1 : 0;
}
