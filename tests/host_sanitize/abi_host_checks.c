/* Host-side checks of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer against a host-only build of the library (no
 * device code: no kernel can run).  Every call made here must be rejected by
 * the argument checks before the first HIP call, or be a pure host query
 * (workspace sizes, status strings, the kernel-choice setter).  Device
 * pointers are stand-in addresses that are never dereferenced.
 *
 * Exit status 0 when every expectation holds; the sanitizers abort on the
 * first finding (the build uses -fno-sanitize-recover).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "logra.h"
#include "logra_calib.h"

static int g_fail = 0;
static int g_checks = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    ++g_checks;                                                        \
    if (!(cond)) {                                                     \
      ++g_fail;                                                        \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
              __LINE__, #cond);                                        \
    }                                                                  \
  } while (0)

/* Stand-in device addresses: aligned as the entry points require unless a
 * case asks otherwise. */
static void* fake(uintptr_t a) { return (void*)a; }
#define X_PTR ((const uint16_t*)fake(0x100000))
#define DY_PTR ((const uint16_t*)fake(0x200000))
#define S_PTR ((float*)fake(0x300000))
#define WS_PTR (fake(0x400000))
#define W_PTR ((uint16_t*)fake(0x500000))

static const int64_t kDims[] = {1, 2, 7, 8, 31, 32, 33, 127, 128, 129, 255, 256, 257,
                                1536, 3584, 4096, 8960, 18944, 25600, 152064,
                                (int64_t)1 << 20, ((int64_t)1 << 31) - 1};
static const int32_t kRanks[] = {1, 3, 4, 15, 16, 17, 32, 63, 64, 65, 127, 128, 129,
                                 192, 255, 256};
#define N_OF(a) ((int)(sizeof(a) / sizeof((a)[0])))

static void check_status_strings(void) {
  const int codes[] = {LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE, LOGRA_EHIP, 7, -99};
  for (int i = 0; i < N_OF(codes); ++i) {
    const char* s = logra_status_str(codes[i]);
    EXPECT(s != NULL && strlen(s) > 0);
  }
  EXPECT(logra_abi_version() == LOGRA_ABI_VERSION);
}

/* Workspace queries over a sweep of shapes: zero exactly for invalid
 * arguments, otherwise a multiple of 256 bytes that does not shrink as T
 * grows; the shared query with one output equals the single-output one. */
static void check_sketch_ws(void) {
  const int64_t Ts[] = {1, 2, 31, 32, 33, 1000, 8192, 16384, 32768, 65536, (int64_t)1 << 24};
  for (int ik = 0; ik < N_OF(kDims); ik += 3) {
    for (int id = 0; id < N_OF(kDims); id += 2) {
      for (int ir = 0; ir < N_OF(kRanks); ++ir) {
        size_t prev = 0;
        for (int it = 0; it < N_OF(Ts); ++it) {
          const int64_t T = Ts[it], d = kDims[id], k = kDims[ik];
          const int32_t r = kRanks[ir];
          const size_t b = logra_sketch_ws_bytes(T, d, k, r);
          if (b != 0) {
            EXPECT(b % 256 == 0);
            EXPECT(b >= prev);
            prev = b;
          }
          const size_t bs = logra_sketch_shared_ws_bytes(T, k, r, 1, &d);
          EXPECT(bs == b);
        }
      }
    }
  }
  /* invalid sizes */
  EXPECT(logra_sketch_ws_bytes(0, 64, 64, 4) == 0 || logra_sketch_ws_bytes(0, 64, 64, 4) % 256 == 0);
  EXPECT(logra_sketch_ws_bytes(-1, 64, 64, 4) == 0);
  EXPECT(logra_sketch_ws_bytes(64, 0, 64, 4) == 0);
  EXPECT(logra_sketch_ws_bytes(64, 64, 0, 4) == 0);
  EXPECT(logra_sketch_ws_bytes(64, 64, 64, 0) == 0);
  EXPECT(logra_sketch_ws_bytes(64, 64, 64, LOGRA_MAX_RANK + 1) == 0);
  EXPECT(logra_sketch_ws_bytes(64, (int64_t)1 << 31, 64, 4) == 0);
  EXPECT(logra_sketch_ws_bytes(64, 64, (int64_t)1 << 31, 4) == 0);
  EXPECT(logra_sketch_ws_bytes((int64_t)1 << 31, 64, 64, 4) == 0);
  EXPECT(logra_sketch_ws_bytes(INT64_MAX, INT64_MAX, INT64_MAX, INT32_MAX) == 0);
  EXPECT(logra_sketch_ws_bytes(INT64_MIN, INT64_MIN, INT64_MIN, INT32_MIN) == 0);
  /* shared: output counts and d arrays */
  const int64_t ds[LOGRA_MAX_SHARED + 1] = {1536, 256, 256, 8960, 99};
  for (int n = -1; n <= LOGRA_MAX_SHARED + 1; ++n) {
    const size_t b = logra_sketch_shared_ws_bytes(16384, 1536, 64, n, ds);
    EXPECT((n >= 1 && n <= LOGRA_MAX_SHARED) == (b != 0));
  }
  EXPECT(logra_sketch_shared_ws_bytes(16384, 1536, 64, 2, NULL) == 0);
  const int64_t bad[2] = {1536, 0};
  EXPECT(logra_sketch_shared_ws_bytes(16384, 1536, 64, 2, bad) == 0);
  /* KL workspaces */
  EXPECT(logra_kl_ws_bytes(65536, 152064) >= 65536 * 4);
  EXPECT(logra_kl_ws_bytes(0, 152064) == 0);
  EXPECT(logra_kl_ws_bytes(65536, 0) == 0);
  EXPECT(logra_kl_ws_bytes(INT64_MAX, INT64_MAX) == 0);
  for (int a = -1; a <= LOGRA_MAX_SWEEP + 1; ++a) {
    const size_t b = logra_kl_sweep_ws_bytes(65536, a);
    EXPECT((a >= 1 && a <= LOGRA_MAX_SWEEP) == (b != 0));
    if (b) EXPECT(b >= (size_t)65536 * 4 * (size_t)a);
  }
  EXPECT(logra_kl_sweep_ws_bytes(INT64_MAX, 4) == 0);
}

static void check_sketch_rejects(void) {
  const int64_t T = 8192, d = 4096, k = 4096;
  const int32_t r = 64;
  const size_t ws = logra_sketch_ws_bytes(T, d, k, r);
  EXPECT(ws > 0);
  /* one bad argument at a time; every other argument valid */
  EXPECT(logra_sketch_accumulate(NULL, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, NULL, d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, NULL, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate((const uint16_t*)fake(0x100008), k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, (const uint16_t*)fake(0x200002), d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, (float*)fake(0x300002), WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k - 8, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k + 4, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d - 8, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, (int64_t)1 << 26, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, -1, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, (int64_t)1 << 31, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, 0, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, 0, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, 0, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, 257, 1, 0, 0, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 2, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, -1, 0, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  /* flags: unknown bits, DEFER with OVERWRITE, deferral on T == 0 */
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 8, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, LOGRA_SKETCH_DEFER | LOGRA_SKETCH_OVERWRITE, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, 0, d, k, r, 1, 0, 0, LOGRA_SKETCH_DEFER, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, 0, d, k, r, 1, 0, 0, LOGRA_SKETCH_PENDING, S_PTR, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  /* T == 0 without the overwrite flag: nothing to do, no HIP call */
  EXPECT(logra_sketch_accumulate(NULL, 0, NULL, 0, 0, d, k, r, 1, 0, 0, 0, NULL, NULL, 0, NULL) == LOGRA_OK);
  /* workspace: missing, too small, misaligned */
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, NULL, ws, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, WS_PTR, ws - 1, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_sketch_accumulate(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, fake(0x400080), ws, NULL) == LOGRA_EWORKSPACE);
  /* the entry point that allocates nothing: no deferral, size limit */
  EXPECT(logra_sketch_accumulate_noalloc(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, LOGRA_SKETCH_DEFER, S_PTR, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_noalloc(X_PTR, k, DY_PTR, d, T, d, k, r, 1, 0, 0, LOGRA_SKETCH_PENDING, S_PTR, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_noalloc(NULL, k, DY_PTR, d, T, d, k, r, 1, 0, 0, 0, S_PTR, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_noalloc(X_PTR, k, DY_PTR, d, 0, d, k, r, 1, 0, 0, 0, S_PTR, NULL) == LOGRA_OK);
  {
    /* a shape whose workspace exceeds the scratch */
    const int64_t dd = 1 << 20, kk = 4096, TT = 65536;
    EXPECT(logra_sketch_ws_bytes(TT, dd, kk, 256) > LOGRA_NOALLOC_SCRATCH_BYTES);
    EXPECT(logra_sketch_accumulate_noalloc(X_PTR, kk, DY_PTR, dd, TT, dd, kk, 256, 1, 0, 0, 0, S_PTR, NULL) == LOGRA_EWORKSPACE);
  }
  /* shared outputs */
  {
    const uint16_t* dys[4] = {DY_PTR, (const uint16_t*)fake(0x210000), (const uint16_t*)fake(0x220000), (const uint16_t*)fake(0x230000)};
    const int64_t ldd[4] = {1536, 256, 256, 256};
    const int64_t dd[4] = {1536, 256, 256, 256};
    /* S arrays 1 MiB apart: no two d x r ranges overlap */
    float* Ss[4] = {(float*)fake(0x3000000), (float*)fake(0x3100000), (float*)fake(0x3200000),
                    (float*)fake(0x3300000)};
    const size_t wsb = logra_sketch_shared_ws_bytes(16384, 1536, 64, 3, dd);
    EXPECT(wsb > 0);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 0, dys, ldd, dd, Ss, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 5, dys, ldd, dd, Ss, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, NULL, ldd, dd, Ss, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, NULL, dd, Ss, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, ldd, NULL, Ss, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, ldd, dd, NULL, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    float* dup[3] = {Ss[0], Ss[1], Ss[0]};
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, ldd, dd, dup, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    float* part[3] = {Ss[0], Ss[1], (float*)fake(0x3000000 + 4096)};   /* partial overlap */
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, ldd, dd, part, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, ldd, dd, dup, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, ldd, dd, Ss, WS_PTR, wsb - 256, NULL) == LOGRA_EWORKSPACE);
    const int64_t bad_ld[3] = {1536, 255, 256};
    EXPECT(logra_sketch_accumulate_shared(X_PTR, 1536, 16384, 1536, 64, 1, 0, 0, 0, 3, dys, bad_ld, dd, Ss, WS_PTR, wsb, NULL) == LOGRA_EINVAL);
  }
}

static void check_other_rejects(void) {
  /* projection */
  EXPECT(logra_regen_A(1, 0, 0, 64, 4096, NULL, NULL) == LOGRA_EINVAL);
  EXPECT(logra_regen_A(1, 0, 0, 64, 4096, (float*)fake(0x300002), NULL) == LOGRA_EINVAL);
  EXPECT(logra_regen_A(1, 0, 0, 0, 4096, S_PTR, NULL) == LOGRA_EINVAL);
  EXPECT(logra_regen_A(1, 0, 0, 64, 0, S_PTR, NULL) == LOGRA_EINVAL);
  EXPECT(logra_regen_A(1, 0, 5, 64, 4096, S_PTR, NULL) == LOGRA_EINVAL);
  /* merge */
  EXPECT(logra_merge(NULL, 4096, S_PTR, 4096, 4096, 64, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge(W_PTR, 4096, NULL, 4096, 4096, 64, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge((uint16_t*)fake(0x500008), 4096, S_PTR, 4096, 4096, 64, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge(W_PTR, 4092, S_PTR, 4096, 4096, 64, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge(W_PTR, 4096, S_PTR, 4096, 4096, 64, 1, 0, 0, NAN, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge(W_PTR, 4096, S_PTR, 4096, 4096, 64, 1, 0, 0, 1.0f, INFINITY, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge(W_PTR, 4096, S_PTR, 0, 4096, 64, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge(W_PTR, 4096, S_PTR, 4096, 4096, 300, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  /* a grid of more than 2^31 tiles */
  EXPECT(logra_merge(W_PTR, ((int64_t)1 << 31) - 8, S_PTR, ((int64_t)1 << 31) - 1, ((int64_t)1 << 31) - 8, 64, 1, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  /* sketch-space update: bad rule, missing state, bad betas, overlaps */
  float* S = S_PTR;
  float* m = (float*)fake(0x600000);
  float* v = (float*)fake(0x700000);
  float* U = (float*)fake(0x800000);
  EXPECT(logra_sketch_update(3, S, m, v, U, 4096, 64, 0.9f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_MOMENTUM, S, NULL, v, U, 4096, 64, 0.9f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, NULL, U, 4096, 64, 0.9f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, v, U, 4096, 64, 1.0f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, v, U, 4096, 64, 0.9f, NAN, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, v, U, 4096, 64, 0.9f, 0.999f, -1.0f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, v, U, 4096, 64, 0.9f, 0.999f, 1e-8f, 0, NULL) == LOGRA_EINVAL);
  /* d r floats each: 4096 * 64 * 4 = 1 MiB; a partial overlap of m and v */
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, (float*)fake(0x600000 + 4096), U, 4096, 64, 0.9f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  /* U == v is not an allowed alias */
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, v, v, 4096, 64, 0.9f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  /* U == m is allowed only for momentum */
  EXPECT(logra_sketch_update(LOGRA_UPDATE_ADAM, S, m, v, m, 4096, 64, 0.9f, 0.999f, 1e-8f, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_SGD, S, NULL, NULL, NULL, 4096, 64, 0, 0, 0, 1, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_update(LOGRA_UPDATE_SGD, (float*)fake(0x300002), NULL, NULL, U, 4096, 64, 0, 0, 0, 1, NULL) == LOGRA_EINVAL);
  /* predicted KL */
  const int64_t n = 65536, V = 152064;
  const size_t kws = logra_kl_ws_bytes(n, V);
  float* qa = (float*)fake(0x900000);
  EXPECT(logra_predicted_kl(NULL, X_PTR, n, V, V, 1.0f, 2e-4f, 4.0f, qa, NULL, WS_PTR, kws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl(X_PTR, X_PTR, n, V, V - 8, 1.0f, 2e-4f, 4.0f, qa, NULL, WS_PTR, kws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl(X_PTR, DY_PTR, n, V, V, 0.0f, 2e-4f, 4.0f, qa, NULL, WS_PTR, kws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl(X_PTR, DY_PTR, n, V, V, 1.0f, 0.0f, 4.0f, qa, NULL, WS_PTR, kws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl(X_PTR, DY_PTR, n, V, V, 1.0f, 2e-4f, -1.0f, qa, NULL, WS_PTR, kws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl(X_PTR, DY_PTR, n, V, V, 1.0f, 2e-4f, 4.0f, (float*)fake(0x900002), NULL, WS_PTR, kws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl(X_PTR, DY_PTR, n, V, V, 1.0f, 2e-4f, 4.0f, qa, NULL, NULL, kws, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_predicted_kl(X_PTR, DY_PTR, n, V, V, 1.0f, 2e-4f, 4.0f, qa, NULL, WS_PTR, kws - 4, NULL) == LOGRA_EWORKSPACE);
  /* sweep: the multipliers are read on the host */
  float alphas[LOGRA_MAX_SWEEP] = {0.25f, 0.5f, 1.0f, 2.0f, 0, 0, 0, 0};
  const size_t sws = logra_kl_sweep_ws_bytes(n, 4);
  EXPECT(logra_predicted_kl_sweep(X_PTR, DY_PTR, n, V, V, NULL, 4, 1.0f, NULL, qa, NULL, WS_PTR, sws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl_sweep(X_PTR, DY_PTR, n, V, V, alphas, 0, 1.0f, NULL, qa, NULL, WS_PTR, sws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_predicted_kl_sweep(X_PTR, DY_PTR, n, V, V, alphas, LOGRA_MAX_SWEEP + 1, 1.0f, NULL, qa, NULL, WS_PTR, sws, NULL) == LOGRA_EINVAL);
  alphas[2] = NAN;
  EXPECT(logra_predicted_kl_sweep(X_PTR, DY_PTR, n, V, V, alphas, 4, 1.0f, NULL, qa, NULL, WS_PTR, sws, NULL) == LOGRA_EINVAL);
  alphas[2] = 1.0f;
  EXPECT(logra_predicted_kl_sweep(X_PTR, DY_PTR, n, V, V, alphas, 4, 1.0f, NULL, qa, NULL, WS_PTR, sws - 4, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_predicted_kl_sweep(X_PTR, DY_PTR, ((int64_t)1 << 29), V, V, alphas, 4, 1.0f, NULL, qa, NULL, WS_PTR, sws, NULL) == LOGRA_EINVAL);
  /* copy calibration helper */
  EXPECT(logra_calib_copy(NULL, X_PTR, 4096, NULL) != 0);
  EXPECT(logra_calib_copy(S_PTR, X_PTR, 4095, NULL) != 0);
  EXPECT(logra_calib_copy((void*)fake(0x300004), X_PTR, 4096, NULL) != 0);
  EXPECT(logra_calib_copy(S_PTR, X_PTR, 0, NULL) == 0);
  EXPECT(logra_calib_read(NULL, 4096, 0, S_PTR, NULL) != 0);
  EXPECT(logra_calib_read(X_PTR, 4096, 0, NULL, NULL) != 0);
  EXPECT(logra_calib_read(X_PTR, 4095, 1, S_PTR, NULL) != 0);
  EXPECT(logra_calib_read((const void*)fake(0x100008), 4096, 0, S_PTR, NULL) != 0);
  EXPECT(logra_calib_read(X_PTR, 4096, 0, (void*)fake(0x300002), NULL) != 0);
  EXPECT(logra_calib_read(X_PTR, 0, 0, S_PTR, NULL) == 0);
}

/* The layer sketch and the grouped merge: workspace queries over group
 * structures, and rejected calls. */
static void check_layer_and_merge_many(void) {
  logra_sketch_group g[LOGRA_MAX_GROUPS + 1];
  memset(g, 0, sizeof(g));
  const int64_t ks[4] = {1536, 1536, 1536, 8960};
  const int nouts[4] = {3, 1, 2, 1};
  const int64_t ds[4][4] = {{1536, 256, 256, 0}, {1536, 0, 0, 0}, {8960, 8960, 0, 0}, {1536, 0, 0, 0}};
  uintptr_t s_next = 0x10000000;
  for (int i = 0; i < 4; ++i) {
    g[i].X = X_PTR;
    g[i].ldx = ks[i];
    g[i].k = ks[i];
    g[i].seed = 1234;
    g[i].n_out = nouts[i];
    for (int o = 0; o < nouts[i]; ++o) {
      g[i].dY[o] = DY_PTR;
      g[i].ldd[o] = ds[i][o];
      g[i].d[o] = ds[i][o];
      g[i].S[o] = (float*)fake(s_next);
      s_next += (uintptr_t)ds[i][o] * 256 * 4 + 4096;
    }
  }
  for (int n = 1; n <= 4; ++n) {
    for (int ir = 0; ir < N_OF(kRanks); ++ir) {
      const size_t b = logra_sketch_layer_ws_bytes(16384, kRanks[ir], n, g);
      EXPECT(b > 0 && b % 256 == 0);
      if (n == 1)
        EXPECT(b == logra_sketch_shared_ws_bytes(16384, 1536, kRanks[ir], 3, g[0].d));
    }
  }
  EXPECT(logra_sketch_layer_ws_bytes(16384, 64, 0, g) == 0);
  EXPECT(logra_sketch_layer_ws_bytes(16384, 64, 5, g) == 0);
  EXPECT(logra_sketch_layer_ws_bytes(16384, 64, 4, NULL) == 0);
  EXPECT(logra_sketch_layer_ws_bytes(-1, 64, 4, g) == 0);
  EXPECT(logra_sketch_layer_ws_bytes(INT64_MAX, INT32_MAX, 4, g) == 0);
  const size_t ws = logra_sketch_layer_ws_bytes(16384, 64, 4, g);
  /* bad call-level arguments */
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 0, g, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 5, g, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, NULL, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_layer(16384, 0, 0, 0, 4, g, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 16, 4, g, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 3, 4, g, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, g, WS_PTR, ws - 256, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, g, NULL, ws, NULL) == LOGRA_EWORKSPACE);
  /* T == 0 without overwrite: nothing to do */
  EXPECT(logra_sketch_accumulate_layer(0, 64, 0, 0, 4, g, NULL, 0, NULL) == LOGRA_OK);
  /* one bad group field at a time */
  logra_sketch_group bad[4];
  memcpy(bad, g, sizeof(bad));
  bad[2].X = NULL;
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  memcpy(bad, g, sizeof(bad));
  bad[3].ldx = 8952;
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  memcpy(bad, g, sizeof(bad));
  bad[1].n_out = 0;
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  memcpy(bad, g, sizeof(bad));
  bad[0].n_out = 4;   /* nine outputs in all (and a fourth d of zero) */
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  memcpy(bad, g, sizeof(bad));
  bad[2].S[1] = bad[0].S[2];   /* one accumulator for two outputs */
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  memcpy(bad, g, sizeof(bad));
  bad[2].S[1] = (float*)((char*)bad[2].S[0] + 64);   /* partial overlap */
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  memcpy(bad, g, sizeof(bad));
  bad[1].ldd[0] = (int64_t)1 << 26;
  EXPECT(logra_sketch_accumulate_layer(16384, 64, 0, 0, 4, bad, WS_PTR, ws, NULL) == LOGRA_EINVAL);
  /* the grouped merge */
  logra_merge_item m[LOGRA_MAX_MERGE + 1];
  memset(m, 0, sizeof(m));
  for (int i = 0; i <= LOGRA_MAX_MERGE; ++i) {
    m[i].W = (uint16_t*)fake(0x20000000 + (uintptr_t)i * 0x1000000);
    m[i].ldw = 1536;
    m[i].S = (const float*)fake(0x80000000u + (uintptr_t)i * 0x100000);
    m[i].d = 1536;
    m[i].k = 1536;
  }
  EXPECT(logra_merge_many(0, m, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge_many(LOGRA_MAX_MERGE + 1, m, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge_many(2, NULL, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge_many(2, m, 0, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge_many(2, m, 64, 4, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  EXPECT(logra_merge_many(2, m, 64, 0, NAN, 2e-4f, NULL) == LOGRA_EINVAL);
  logra_merge_item mb[3];
  memcpy(mb, m, sizeof(mb));
  mb[1].W = mb[0].W + 1536 * 100;   /* rows inside the first weight */
  EXPECT(logra_merge_many(3, mb, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  memcpy(mb, m, sizeof(mb));
  mb[2].S = (const float*)(mb[1].W + 64);   /* an S inside a W */
  EXPECT(logra_merge_many(3, mb, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  memcpy(mb, m, sizeof(mb));
  mb[1].ldw = 1000;
  EXPECT(logra_merge_many(3, mb, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
  memcpy(mb, m, sizeof(mb));
  mb[2].d = ((int64_t)1 << 31) - 1;
  mb[2].k = ((int64_t)1 << 31) - 8;
  mb[2].ldw = ((int64_t)1 << 31) - 8;
  EXPECT(logra_merge_many(3, mb, 64, 0, 1.0f, 2e-4f, NULL) == LOGRA_EINVAL);
}

static void check_kernel_choice(void) {
  EXPECT(logra_set_kernel_choice(2, 0) == LOGRA_EINVAL);
  EXPECT(logra_set_kernel_choice(-1, 0) == LOGRA_EINVAL);
  EXPECT(logra_set_kernel_choice(LOGRA_CHOICE_PROJECT_TILE, 3) == LOGRA_EINVAL);
  EXPECT(logra_set_kernel_choice(LOGRA_CHOICE_ACC_WIDE, 2) == LOGRA_EINVAL);
  EXPECT(logra_set_kernel_choice(LOGRA_CHOICE_PROJECT_TILE, 2) == LOGRA_OK);
  for (int which = 0; which < 2; ++which)
    for (int mode = -1; mode <= 1; ++mode)
      EXPECT(logra_set_kernel_choice(which, mode) == LOGRA_OK);
  EXPECT(logra_set_kernel_choice(LOGRA_CHOICE_PROJECT_TILE, LOGRA_CHOICE_AUTO) == LOGRA_OK);
  EXPECT(logra_set_kernel_choice(LOGRA_CHOICE_ACC_WIDE, LOGRA_CHOICE_AUTO) == LOGRA_OK);
}

/* The one path that reaches HIP here: T == 0 with the overwrite flag zero
 * fills exactly the call's outputs.  Only without a visible device (every
 * launch then fails with a HIP error and nothing runs); the sanitizers check
 * that the output list is not read past its end. */
static void check_zero_fill_without_device(void) {
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) == hipSuccess && n_dev > 0) {
    printf("a device is visible: zero-fill checks skipped\n");
    return;
  }
  const int st1 = logra_sketch_accumulate(NULL, 0, NULL, 0, 0, 64, 64, 4, 1, 0, 0,
                                          LOGRA_SKETCH_OVERWRITE, S_PTR, NULL, 0, NULL);
  EXPECT(st1 == LOGRA_EHIP);
  const uint16_t* dys[2] = {NULL, NULL};
  const int64_t ldd[2] = {0, 0}, dd[2] = {64, 32};
  float* Ss[2] = {S_PTR, (float*)fake(0x3400000)};
  const int st2 = logra_sketch_accumulate_shared(NULL, 0, 0, 64, 4, 1, 0, 0, LOGRA_SKETCH_OVERWRITE,
                                                 2, dys, ldd, dd, Ss, NULL, 0, NULL);
  EXPECT(st2 == LOGRA_EHIP);
  logra_sketch_group g[2];
  memset(g, 0, sizeof(g));
  g[0].k = 64;
  g[0].n_out = 1;
  g[0].d[0] = 64;
  g[0].S[0] = S_PTR;
  g[1].k = 128;
  g[1].n_out = 2;
  g[1].d[0] = 32;
  g[1].d[1] = 16;
  g[1].S[0] = (float*)fake(0x3400000);
  g[1].S[1] = (float*)fake(0x3500000);
  const int st3 = logra_sketch_accumulate_layer(0, 4, 0, LOGRA_SKETCH_OVERWRITE, 2, g, NULL, 0, NULL);
  EXPECT(st3 == LOGRA_EHIP);
  const int st4 = logra_sketch_accumulate_noalloc(NULL, 0, NULL, 0, 0, 64, 64, 4, 1, 0, 0,
                                                  LOGRA_SKETCH_OVERWRITE, S_PTR, NULL);
  EXPECT(st4 == LOGRA_EHIP);
  const int st5 = logra_sketch_accumulate_p(NULL, 0, 0, 4, LOGRA_SKETCH_OVERWRITE, 2, dys, ldd, dd,
                                            Ss, NULL, 0, NULL);
  EXPECT(st5 == LOGRA_EHIP);
}

/* The two-call sketch: sizes that add up to the one-call workspace over a
 * sweep of shapes, and one bad argument at a time for both halves. */
static void check_split_sketch(void) {
  const int64_t Ts[] = {1, 31, 33, 1000, 8192, 16384, 65536};
  for (int it = 0; it < N_OF(Ts); ++it)
    for (int id = 0; id < N_OF(kDims); id += 3)
      for (int ir = 0; ir < N_OF(kRanks); ir += 2) {
        const int64_t T = Ts[it], d = kDims[id], k = 4096;
        const int32_t r = kRanks[ir];
        const size_t full = logra_sketch_ws_bytes(T, d, k, r);
        const size_t pb = logra_sketch_p_bytes(T, r);
        const size_t gb = logra_sketch_project_ws_bytes(k, r);
        const size_t ab = logra_sketch_accumulate_p_ws_bytes(T, r, 1, &d);
        EXPECT((full != 0) == (ab != 0));
        if (full == 0) continue;
        EXPECT(pb % 256 == 0 && gb % 256 == 0 && ab % 256 == 0);
        EXPECT(pb + gb + ab == full);
      }
  EXPECT(logra_sketch_p_bytes(64, 0) == 0);
  EXPECT(logra_sketch_p_bytes(-1, 4) == 0);
  EXPECT(logra_sketch_p_bytes(INT64_MAX, INT32_MAX) == 0);
  EXPECT(logra_sketch_project_ws_bytes(0, 4) == 0);
  EXPECT(logra_sketch_project_ws_bytes(INT64_MIN, 4) == 0);
  EXPECT(logra_sketch_accumulate_p_ws_bytes(64, 4, 1, NULL) == 0);
  EXPECT(logra_sketch_accumulate_p_ws_bytes(64, 4, LOGRA_MAX_SHARED + 1, kDims) == 0);

  const int64_t T = 8192, d = 4096, k = 4096;
  const int32_t r = 64;
  uint16_t* Pp = (uint16_t*)fake(0x600000);
  const size_t pb = logra_sketch_p_bytes(T, r), gb = logra_sketch_project_ws_bytes(k, r);
  EXPECT(logra_sketch_project(NULL, k, T, k, r, 1, 0, 0, Pp, pb, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k - 8, T, k, r, 1, 0, 0, Pp, pb, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, 0, 1, 0, 0, Pp, pb, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, r, 1, 0, 3, Pp, pb, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, r, 1, 0, 0, NULL, pb, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, r, 1, 0, 0, Pp + 4, pb, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, r, 1, 0, 0, Pp, pb - 1, NULL, 0, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, r, 1, 0, 1, Pp, pb, NULL, 0, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_sketch_project(X_PTR, k, T, k, r, 1, 0, 1, Pp, pb, WS_PTR, gb - 1, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_sketch_project(NULL, 0, 0, k, r, 1, 0, 0, NULL, 0, NULL, 0, NULL) == LOGRA_OK);

  const uint16_t* dys[2] = {DY_PTR, DY_PTR};
  const int64_t ldd[2] = {d, d}, dd[2] = {d, d};
  float* Ss[2] = {S_PTR, (float*)fake(0x3400000)};
  const size_t ab = logra_sketch_accumulate_p_ws_bytes(T, r, 2, dd);
  EXPECT(ab > 0);
  EXPECT(logra_sketch_accumulate_p(NULL, pb, T, r, 0, 2, dys, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb - 1, T, r, 0, 2, dys, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, 0, dys, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, LOGRA_MAX_SHARED + 1, dys, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, 2, NULL, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, 2, dys, ldd, dd, NULL, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, 0, 0, 2, dys, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 3, 2, dys, ldd, dd, Ss, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, 2, dys, ldd, dd, Ss, NULL, ab, NULL) == LOGRA_EWORKSPACE);
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, 2, dys, ldd, dd, Ss, WS_PTR, ab - 1, NULL) == LOGRA_EWORKSPACE);
  float* same[2] = {S_PTR, S_PTR};
  EXPECT(logra_sketch_accumulate_p(Pp, pb, T, r, 0, 2, dys, ldd, dd, same, WS_PTR, ab, NULL) == LOGRA_EINVAL);
  EXPECT(logra_sketch_accumulate_p(NULL, 0, 0, r, 0, 2, dys, ldd, dd, Ss, NULL, 0, NULL) == LOGRA_OK);
}

int main(void) {
  check_status_strings();
  check_sketch_ws();
  check_sketch_rejects();
  check_other_rejects();
  check_layer_and_merge_many();
  check_kernel_choice();
  check_zero_fill_without_device();
  check_split_sketch();
  printf("host ABI checks: %d expectations, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
