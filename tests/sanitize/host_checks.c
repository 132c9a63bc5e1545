/* Host-side checks of libkvx under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built against a host-only build of the library (no device code objects), so
 * no call here can launch a kernel: every call either is pure host logic (the
 * layer map, status strings, workspace and map sizes) or is rejected by the
 * argument checks before the first HIP runtime call.  Arrays the library reads
 * on the host (tap tables, sequence offsets, per-problem pointer arrays) are
 * heap blocks of exactly the documented length, so a read past them is an
 * ASan report; integer overflow in the size arithmetic is a UBSan report.
 * Exits 0 and prints "host checks passed" when every expectation holds. */
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvx.h"

static int failures = 0;

#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

#define EXPECT_EQ(got, want)                                                \
  do {                                                                      \
    long long g_ = (long long)(got), w_ = (long long)(want);                \
    if (g_ != w_) {                                                         \
      fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #got, g_, w_); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

/* A device-looking address that is never dereferenced on the host. */
#define FAKE ((void*)(uintptr_t)0x1000)

static kvx_cache_desc desc(int32_t layers, int32_t tokens, int32_t heads, int32_t dim, int32_t dtype, double rope) {
  kvx_cache_desc d;
  memset(&d, 0, sizeof d);
  d.layers = layers;
  d.tokens = tokens;
  d.kv_heads = heads;
  d.head_dim = dim;
  d.dtype = dtype;
  d.rope_base = rope;
  d.k_norm = NULL;
  d.k_norm_eps = 0.0;
  return d;
}

/* Heap copy of n int32 values: the library may read exactly n of them. */
static int32_t* exact_i32(const int32_t* v, size_t n) {
  int32_t* p = (int32_t*)malloc(n * sizeof(int32_t));
  memcpy(p, v, n * sizeof(int32_t));
  return p;
}

static void check_status_strings(void) {
  const char* unknown = kvx_status_string(-1);
  EXPECT(unknown && strcmp(unknown, "unknown status") == 0);
  for (int s = 0; s <= KVX_ERR_NOT_CONVERGED; ++s) {
    const char* t = kvx_status_string(s);
    EXPECT(t && t[0] && strcmp(t, "unknown status") != 0);
  }
  EXPECT(strcmp(kvx_status_string(KVX_ERR_NOT_CONVERGED + 1), "unknown status") == 0);
  EXPECT(strcmp(kvx_status_string(INT_MIN), "unknown status") == 0);
  EXPECT(strcmp(kvx_status_string(INT_MAX), "unknown status") == 0);
}

static void check_layer_map(void) {
  /* 36 -> 32 layers, taps -4/0/+4: every tap inside the sender, the middle
     tap non-decreasing, the first and last receiver layers as documented. */
  int32_t* t = (int32_t*)malloc(32 * 3 * sizeof(int32_t));
  EXPECT_EQ(kvx_layer_map(36, 32, 3, 4, t), KVX_OK);
  for (int l = 0; l < 32; ++l)
    for (int k = 0; k < 3; ++k) EXPECT(t[l * 3 + k] >= 0 && t[l * 3 + k] <= 35);
  for (int l = 1; l < 32; ++l) EXPECT(t[l * 3 + 1] >= t[(l - 1) * 3 + 1]);
  EXPECT(t[0] == 0 && t[1] == 0 && t[2] == 4);
  EXPECT(t[93] == 31 && t[94] == 35 && t[95] == 35);
  free(t);

  int32_t* one = (int32_t*)malloc(sizeof(int32_t));
  EXPECT_EQ(kvx_layer_map(10, 1, 1, 4, one), KVX_OK);
  EXPECT_EQ(one[0], 0);
  free(one);

  /* extremes: the largest layer counts and strides stay in range */
  int32_t* big = (int32_t*)malloc(2 * 7 * sizeof(int32_t));
  EXPECT_EQ(kvx_layer_map(INT32_MAX, 2, 7, INT32_MAX, big), KVX_OK);
  for (int i = 0; i < 14; ++i) EXPECT(big[i] >= 0 && big[i] <= INT32_MAX - 1);
  EXPECT_EQ(big[3], 0);                 /* receiver layer 0, middle tap */
  EXPECT_EQ(big[7 + 3], INT32_MAX - 1); /* last receiver layer, middle tap */
  free(big);
  int32_t* wide = (int32_t*)malloc(255 * 7 * sizeof(int32_t));
  EXPECT_EQ(kvx_layer_map(2, 255, 7, 1, wide), KVX_OK);
  for (int i = 0; i < 255 * 7; ++i) EXPECT(wide[i] == 0 || wide[i] == 1);
  free(wide);

  int32_t out[64];
  EXPECT_EQ(kvx_layer_map(36, 32, 2, 4, out), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_layer_map(0, 32, 3, 4, out), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_layer_map(36, 0, 3, 4, out), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_layer_map(36, 32, 9, 4, out), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_layer_map(36, 32, 3, -1, out), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_layer_map(36, 32, 3, 4, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_layer_map(INT32_MIN, 32, 3, 4, out), KVX_ERR_INVALID);
}

static void check_alignment(void) {
  EXPECT(kvx_align_workspace_size(INT32_MAX) > kvx_align_workspace_size(1 << 20));
  EXPECT(kvx_align_workspace_size(1 << 20) > kvx_align_workspace_size(1000));
  EXPECT(kvx_align_workspace_size(0) > 0);
  EXPECT_EQ(kvx_align_tokens(FAKE, 5, FAKE, 0, FAKE, NULL, 0, NULL), KVX_OK);
  EXPECT_EQ(kvx_align_tokens(FAKE, 0, FAKE, 5, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_SHAPE);
  EXPECT_EQ(kvx_align_tokens(FAKE, 5, FAKE, 5, FAKE, NULL, 0, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_align_tokens(FAKE, 5, FAKE, INT32_MAX, FAKE, FAKE, 64, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_align_tokens(NULL, 5, FAKE, 5, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_align_tokens(FAKE, -1, FAKE, 5, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_align_tokens(FAKE, 5, FAKE, INT32_MIN, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_INVALID);

  EXPECT_EQ(kvx_align_tokens_async(FAKE, 5, FAKE, 5, FAKE, NULL, FAKE, (size_t)1 << 30, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_align_tokens_async(FAKE, 5, FAKE, 5, FAKE, FAKE, NULL, 0, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_align_tokens_async(FAKE, 5, FAKE, 0, FAKE, NULL, NULL, 0, NULL), KVX_OK);

  EXPECT_EQ(kvx_align_tokens_noalloc(FAKE, 5, FAKE, KVX_NOALLOC_MAX_RECV + 1, FAKE, FAKE, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_align_tokens_noalloc(FAKE, 5, FAKE, INT32_MAX, FAKE, FAKE, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_align_tokens_noalloc(FAKE, 5, FAKE, 0, FAKE, FAKE, NULL), KVX_OK);
  EXPECT_EQ(kvx_align_tokens_noalloc(FAKE, 0, FAKE, 5, FAKE, FAKE, NULL), KVX_ERR_SHAPE);
  EXPECT_EQ(kvx_align_tokens_noalloc(FAKE, 5, FAKE, 5, FAKE, NULL, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_align_tokens_noalloc(FAKE, -3, FAKE, 5, FAKE, FAKE, NULL), KVX_ERR_INVALID);

  /* several sequences: offsets arrays of exactly n_seq + 1 entries */
  const int32_t so[4] = {0, 10, 10, 25}, ro[4] = {0, 12, 12, 30};
  int32_t* s_off = exact_i32(so, 4);
  int32_t* r_off = exact_i32(ro, 4);
  EXPECT(kvx_align_batched_workspace_size(r_off, 3) > 0);
  EXPECT_EQ(kvx_align_batched_workspace_size(NULL, 3), 0);
  EXPECT_EQ(kvx_align_batched_workspace_size(r_off, 0), 0);
  EXPECT_EQ(kvx_align_tokens_batched(FAKE, s_off, FAKE, r_off, 3, FAKE, NULL, 0, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_align_tokens_batched(NULL, s_off, FAKE, r_off, 3, FAKE, FAKE, (size_t)1 << 30, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_align_tokens_batched(FAKE, s_off, FAKE, r_off, 0, FAKE, FAKE, (size_t)1 << 30, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_align_tokens_batched(FAKE, NULL, FAKE, r_off, 3, FAKE, FAKE, (size_t)1 << 30, NULL),
            KVX_ERR_INVALID);
  free(s_off);
  free(r_off);
  const int32_t so_bad0[3] = {1, 5, 9}, ro_ok[3] = {0, 4, 8};
  const int32_t so_dec[3] = {0, 5, 4}, so_empty[3] = {0, 5, 5}, ro_zero[3] = {0, 0, 0};
  const int32_t ro_wild[3] = {0, INT32_MAX, INT32_MIN}, ro_start[3] = {3, 4, 8};
  int32_t* w3 = exact_i32(ro_wild, 3);
  EXPECT_EQ(kvx_align_batched_workspace_size(w3, 2), 0); /* decreasing offsets: no size */
  free(w3);
  w3 = exact_i32(ro_start, 3);
  EXPECT_EQ(kvx_align_batched_workspace_size(w3, 2), 0); /* offsets must start at 0 */
  free(w3);
  int32_t* a = exact_i32(so_bad0, 3);
  int32_t* b = exact_i32(ro_ok, 3);
  EXPECT_EQ(kvx_align_tokens_batched(FAKE, a, FAKE, b, 2, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_INVALID);
  free(a);
  a = exact_i32(so_dec, 3);
  EXPECT_EQ(kvx_align_tokens_batched(FAKE, a, FAKE, b, 2, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_INVALID);
  free(a);
  a = exact_i32(so_empty, 3); /* the second sequence has receiver tokens but no sender tokens */
  EXPECT_EQ(kvx_align_tokens_batched(FAKE, a, FAKE, b, 2, FAKE, FAKE, (size_t)1 << 30, NULL), KVX_ERR_SHAPE);
  free(b);
  b = exact_i32(ro_zero, 3); /* no receiver tokens at all */
  EXPECT_EQ(kvx_align_tokens_batched(NULL, a, NULL, b, 2, NULL, NULL, 0, NULL), KVX_OK);
  free(a);
  free(b);
}

/* Descriptors that every translation entry point must refuse. */
static void check_descriptors(const int32_t* taps36) {
  kvx_cache_desc r = desc(32, 120, 8, 128, KVX_BF16, 0.0);
  kvx_cache_desc bad[9];
  bad[0] = desc(0, 100, 8, 128, KVX_BF16, 0.0);
  bad[1] = desc(256, 100, 8, 128, KVX_BF16, 0.0);
  bad[2] = desc(36, -1, 8, 128, KVX_BF16, 0.0);
  bad[3] = desc(36, 100, 0, 128, KVX_BF16, 0.0);
  bad[4] = desc(36, 100, 8, 0, KVX_BF16, 0.0);
  bad[5] = desc(36, 100, 8, 128, 2, 0.0);
  bad[6] = desc(36, 100, 8, 128, KVX_BF16, NAN);
  bad[7] = desc(36, 100, 8, 127, KVX_BF16, 1e4); /* odd head_dim with rotation */
  bad[8] = desc(36, 100, 8, 128, KVX_BF16, -1.0);
  for (int i = 0; i < 9; ++i) {
    EXPECT_EQ(kvx_translate(&bad[i], FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                            NULL, FAKE, (size_t)1 << 40, NULL),
              KVX_ERR_INVALID);
    EXPECT_EQ(kvx_translate_workspace_size(&bad[i], &r, 3, 0), 0);
    EXPECT_EQ(kvx_prepared_maps_size(&bad[i], &r, 3, 0, 0, KVX_BF16), 0);
  }
  EXPECT_EQ(kvx_translate_workspace_size(NULL, &r, 3, 0), 0);
  kvx_cache_desc kn = desc(32, 120, 8, 128, KVX_BF16, 0.0);
  kn.k_norm = (const float*)FAKE;
  kn.k_norm_eps = NAN;
  kvx_cache_desc s = desc(36, 100, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(kvx_translate(&s, FAKE, FAKE, &kn, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL, NULL,
                          FAKE, (size_t)1 << 40, NULL),
            KVX_ERR_INVALID);
}

/* Sizes at the edges of what a descriptor allows: positive, monotone, and no
   integer overflow on the way (UBSan reports one). */
static void check_sizes(void) {
  kvx_cache_desc s = desc(255, INT32_MAX, 8, 128, KVX_BF16, 5e5);
  kvx_cache_desc r = desc(255, INT32_MAX, 8, 128, KVX_BF16, 1e6);
  kvx_cache_desc s1 = desc(255, 1 << 20, 8, 128, KVX_BF16, 5e5);
  kvx_cache_desc r1 = desc(255, 1 << 20, 8, 128, KVX_BF16, 1e6);
  EXPECT(kvx_translate_workspace_size(&s, &r, 7, 0) > kvx_translate_workspace_size(&s1, &r1, 7, 0));
  EXPECT(kvx_translate_workspace_size(&s1, &r1, 7, 0) > 0);
  EXPECT(kvx_translate_workspace_size(&s, &r, 1, 1) > 0);
  EXPECT(kvx_translate_prepared_workspace_size(&s, &r, 7, 0, INT32_MAX) > 0);
  EXPECT(kvx_translate_placed_workspace_size(&s, &r, 7, 0, INT32_MAX) > 0);
  EXPECT_EQ(kvx_translate_placed_workspace_size(&s, &r, 7, 0, -1), 0);
  EXPECT(kvx_prepared_maps_size(&s, &r, 7, 0, 0, KVX_F32) ==
         (size_t)255 * (7 * 8 * 128) * (8 * 128) * 4);
  EXPECT(kvx_prepared_maps_size(&s, &r, 1, 1, 1, KVX_BF16) == (size_t)255 * 8 * 128 * 128 * 2);
  /* the largest feature counts a descriptor allows */
  kvx_cache_desc wide_s = desc(255, 1000, 4096, 16, KVX_F32, 0.0);
  kvx_cache_desc wide_r = desc(255, 1000, 4096, 16, KVX_F32, 0.0);
  EXPECT(kvx_prepared_maps_size(&wide_s, &wide_r, 7, 0, 1, KVX_F32) ==
         (size_t)255 * (7 * 65536) * (size_t)65536 * 4);
  EXPECT(kvx_translate_workspace_size(&wide_s, &wide_r, 7, 0) > 0);
  /* past that limit the descriptor is refused */
  kvx_cache_desc huge = desc(255, 1000, 1 << 20, 1 << 12, KVX_F32, 0.0);
  EXPECT_EQ(kvx_translate_workspace_size(&huge, &wide_r, 7, 0), 0);
  EXPECT_EQ(kvx_prepared_maps_size(&wide_s, &huge, 7, 0, 0, KVX_F32), 0);
  kvx_cache_desc huge2 = desc(255, 1000, INT32_MAX, INT32_MAX, KVX_BF16, 0.0);
  EXPECT_EQ(kvx_translate_workspace_size(&huge2, &wide_r, 1, 0), 0);
  EXPECT_EQ(kvx_gather_features(&huge2, FAKE, 0, FAKE, 3, (const int32_t*)FAKE, 1, FAKE, NULL), KVX_ERR_INVALID);

  EXPECT(kvx_fit_ridge_workspace_size(3072, 1024) > (size_t)3072 * 3072 * 8);
  EXPECT_EQ(kvx_fit_ridge_workspace_size(0, 1024), 0);
  EXPECT(kvx_fit_ridge_batched_workspace_size(65535, 3072, 1024) > kvx_fit_ridge_batched_workspace_size(64, 3072, 1024));
  EXPECT(kvx_fit_ridge_batched_workspace_size(1, KVX_MAX_FIT_FEATURES, KVX_MAX_FIT_FEATURES) > 0);
  EXPECT_EQ(kvx_fit_ridge_batched_workspace_size(1, 1 << 16, 1 << 16), 0);
  EXPECT(kvx_fit_ridge_batched_workspace_size(KVX_MAX_PROBLEMS, KVX_MAX_FIT_FEATURES, KVX_MAX_FIT_FEATURES) >
         (size_t)KVX_MAX_PROBLEMS * KVX_MAX_FIT_FEATURES * KVX_MAX_FIT_FEATURES * 8);
  EXPECT_EQ(kvx_fit_ridge_batched_workspace_size(KVX_MAX_PROBLEMS + 1, 64, 64), 0);
  EXPECT_EQ(kvx_fit_ridge_batched_workspace_size(INT32_MAX, 1 << 16, 1 << 16), 0);
  EXPECT_EQ(kvx_fit_ridge_batched_workspace_size(1, KVX_MAX_FIT_FEATURES + 1, 64), 0);
  EXPECT_EQ(kvx_fit_ridge_batched_workspace_size(1, INT32_MAX, 1024), 0);
  EXPECT_EQ(kvx_fit_ridge_batched_workspace_size(-1, 64, 64), 0);
  EXPECT(kvx_fit_recolor_workspace_size(64, 3072, 1024) > (size_t)64 * 8 * (3072 * 3072 + 2 * 3072 * 1024));
  EXPECT(kvx_fit_recolor_workspace_size(KVX_MAX_PROBLEMS, KVX_MAX_FIT_FEATURES, KVX_MAX_FIT_FEATURES) > 0);
  EXPECT_EQ(kvx_fit_recolor_workspace_size(INT32_MAX, 1 << 16, 1 << 16), 0);
  EXPECT_EQ(kvx_fit_recolor_workspace_size(1, 1024, INT32_MAX), 0);
  EXPECT_EQ(kvx_fit_recolor_workspace_size(0, 3072, 1024), 0);
  EXPECT(kvx_probe_scratch_words() > 0);
}

static void check_translate(const int32_t* taps36) {
  kvx_cache_desc s = desc(36, 100, 8, 128, KVX_BF16, 0.0), r = desc(32, 120, 8, 128, KVX_BF16, 0.0);
  const size_t huge_ws = (size_t)1 << 40;
#define TR(sd, rd, ks, vs, kr, vr, map, taps, nt, ph, wd, wk, wv, ws, wsb) \
  kvx_translate(sd, ks, vs, rd, kr, vr, map, taps, nt, ph, wd, wk, wv, NULL, NULL, ws, wsb, NULL)
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, 7, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 0, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 8, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, NULL, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, NULL, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, NULL, taps36, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 1, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_SHAPE);
  kvx_cache_desc rf = desc(32, 120, 8, 128, KVX_F32, 0.0);
  EXPECT_EQ(TR(&s, &rf, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws),
            KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL, huge_ws), KVX_ERR_WORKSPACE);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, 16), KVX_ERR_WORKSPACE);
  kvx_cache_desc r0 = desc(32, 0, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(TR(&s, &r0, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL, 0), KVX_OK);
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, NULL, NULL, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL, 0), KVX_OK);
  kvx_cache_desc s0 = desc(36, 0, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(TR(&s0, &r, FAKE, FAKE, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_SHAPE);

  /* a tap past the last sender layer, in a table of exactly 32 x 3 entries */
  int32_t* bad = exact_i32(taps36, 96);
  bad[95] = 36;
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, bad, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  bad[95] = -1;
  EXPECT_EQ(TR(&s, &r, FAKE, FAKE, FAKE, FAKE, FAKE, bad, 3, 0, KVX_BF16, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_INVALID);
  free(bad);

  /* per head: one tap per receiver layer (a table of exactly 80 entries) */
  kvx_cache_desc ps = desc(32, 100, 8, 128, KVX_BF16, 0.0), pr = desc(80, 120, 8, 128, KVX_BF16, 0.0);
  int32_t* t80 = (int32_t*)malloc(80 * sizeof(int32_t));
  EXPECT_EQ(kvx_layer_map(32, 80, 1, 4, t80), KVX_OK);
  EXPECT_EQ(TR(&ps, &pr, FAKE, FAKE, FAKE, FAKE, FAKE, t80, 1, 1, KVX_F32, FAKE, FAKE, FAKE, 16), KVX_ERR_WORKSPACE);
  kvx_cache_desc pr_h = desc(80, 120, 4, 128, KVX_BF16, 0.0);
  EXPECT_EQ(TR(&ps, &pr_h, FAKE, FAKE, FAKE, FAKE, FAKE, t80, 1, 1, KVX_F32, FAKE, FAKE, FAKE, huge_ws), KVX_ERR_SHAPE);
  kvx_cache_desc pkn = desc(80, 120, 8, 128, KVX_BF16, 0.0);
  pkn.k_norm = (const float*)FAKE;
  pkn.k_norm_eps = 1e-6;
  EXPECT_EQ(TR(&ps, &pkn, FAKE, FAKE, FAKE, FAKE, FAKE, t80, 1, 1, KVX_F32, FAKE, FAKE, FAKE, huge_ws),
            KVX_ERR_UNSUPPORTED);
  free(t80);
#undef TR

  float ms[2];
  EXPECT_EQ(kvx_translate_timed(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL, NULL,
                                FAKE, huge_ws, NULL, NULL),
            KVX_ERR_INVALID);
  (void)ms;
  void* ev_bad[3] = {FAKE, NULL, FAKE};
  EXPECT_EQ(kvx_translate_recorded(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                   NULL, FAKE, huge_ws, NULL, ev_bad),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_translate_recorded(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                   NULL, FAKE, huge_ws, NULL, NULL),
            KVX_ERR_INVALID);

  /* placements */
  kvx_placement pl;
  memset(&pl, 0, sizeof pl);
  pl.pool_rows = -1;
  EXPECT_EQ(kvx_translate_placed(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                 NULL, FAKE, huge_ws, NULL, &pl),
            KVX_ERR_INVALID);
  pl.pool_rows = 0;
  pl.slot = (const int64_t*)FAKE;
  EXPECT_EQ(kvx_translate_placed(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                 NULL, FAKE, huge_ws, NULL, &pl),
            KVX_ERR_INVALID);
  pl.slot = NULL;
  pl.pool_rows = 119; /* fewer rows than receiver tokens, no slots */
  EXPECT_EQ(kvx_translate_placed(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                 NULL, FAKE, huge_ws, NULL, &pl),
            KVX_ERR_SHAPE);
  pl.pool_rows = 0;
  pl.recv_pos = (const int32_t*)FAKE;
  pl.pos_limit = 0;
  EXPECT_EQ(kvx_translate_placed(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                 NULL, FAKE, huge_ws, NULL, &pl),
            KVX_ERR_INVALID);
  pl.pos_limit = 4096;
  EXPECT_EQ(kvx_translate_placed(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                 NULL, FAKE, 16, NULL, &pl),
            KVX_ERR_WORKSPACE);
  kvx_cache_desc fs = desc(36, 100, 8, 128, KVX_F32, 0.0);
  EXPECT_EQ(kvx_translate_placed(&fs, FAKE, FAKE, &rf, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_F32, FAKE, FAKE, NULL,
                                 NULL, FAKE, huge_ws, NULL, &pl),
            KVX_ERR_UNSUPPORTED);

  /* prepared maps */
  kvx_cache_desc rs = desc(36, 25000, 8, 128, KVX_BF16, 5e5), rr = desc(32, 32768, 8, 128, KVX_BF16, 1e6);
  const size_t n = (size_t)32 * 3072 * 1024;
  EXPECT(kvx_prepared_maps_size(&rs, &rr, 3, 0, 0, KVX_BF16) == 2 * n);
  EXPECT(kvx_prepared_maps_size(&rs, &rr, 3, 0, 0, KVX_F32) == 4 * n);
  EXPECT_EQ(kvx_prepared_maps_size(&rs, &rr, 3, 0, 2, KVX_BF16), 0);
  EXPECT_EQ(kvx_prepared_maps_size(&rs, &rr, 3, 0, 0, 5), 0);
  EXPECT_EQ(kvx_prepare_maps(&rs, &rr, 3, 0, 0, KVX_BF16, FAKE, FAKE, 16, NULL), KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_prepare_maps(&rs, &rr, 3, 0, 0, KVX_BF16, NULL, FAKE, huge_ws, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_prepare_maps(&rs, &rr, 3, 1, 0, KVX_BF16, FAKE, FAKE, huge_ws, NULL), KVX_ERR_SHAPE);
  EXPECT_EQ(kvx_prepare_maps(&rs, &rr, 3, 0, 3, KVX_BF16, FAKE, FAKE, huge_ws, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_prepare_maps(&rs, &rr, 0, 0, 0, KVX_BF16, FAKE, FAKE, huge_ws, NULL), KVX_ERR_INVALID);
  EXPECT(kvx_translate_prepared_workspace_size(&rs, &rr, 3, 0, 0) < kvx_translate_workspace_size(&rs, &rr, 3, 0));
  EXPECT_EQ(kvx_translate_prepared(&rs, FAKE, FAKE, &rr, FAKE, FAKE, FAKE, taps36, 3, 0, 2, FAKE, FAKE, NULL, NULL,
                                   FAKE, huge_ws, NULL, NULL, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_translate_prepared(&rs, FAKE, FAKE, &rr, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                   NULL, FAKE, 16, NULL, NULL, NULL),
            KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_translate_prepared(&rs, FAKE, FAKE, &rr, FAKE, FAKE, FAKE, taps36, 3, 0, KVX_BF16, FAKE, FAKE, NULL,
                                   NULL, FAKE, huge_ws, NULL, NULL, ev_bad),
            KVX_ERR_INVALID);

  /* fp8 maps */
  const uint8_t* q = (const uint8_t*)FAKE;
  const float* sc = (const float*)FAKE;
  EXPECT_EQ(kvx_translate_fp8(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, q, q, NULL, sc, NULL, NULL, FAKE,
                              huge_ws, NULL, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_translate_fp8(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, q, q, sc, NULL, NULL, NULL, FAKE,
                              huge_ws, NULL, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_translate_fp8(&fs, FAKE, FAKE, &rf, FAKE, FAKE, FAKE, taps36, 3, q, q, sc, sc, NULL, NULL, FAKE,
                              huge_ws, NULL, NULL),
            KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(kvx_translate_fp8(&s, FAKE, FAKE, &r, FAKE, FAKE, FAKE, taps36, 3, q, q, sc, sc, NULL, NULL, FAKE, 16,
                              NULL, NULL),
            KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_translate_fp8(&s, FAKE, FAKE, &r0, FAKE, FAKE, FAKE, taps36, 3, q, q, sc, sc, NULL, NULL, NULL, 0,
                              NULL, NULL),
            KVX_OK);
}

static void check_gather(void) {
  kvx_cache_desc s = desc(4, 10, 2, 8, KVX_BF16, 0.0);
  const int32_t tv[2] = {0, 1}, bv[2] = {0, 4};
  int32_t* tp = exact_i32(tv, 2);
  int32_t* bad = exact_i32(bv, 2);
  EXPECT_EQ(kvx_gather_features(&s, FAKE, 1, FAKE, 3, tp, 2, FAKE, NULL), KVX_ERR_INVALID); /* no rotation */
  EXPECT_EQ(kvx_gather_features(&s, FAKE, 0, FAKE, 3, bad, 2, FAKE, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_gather_features(&s, FAKE, 0, FAKE, 0, tp, 2, FAKE, NULL), KVX_OK);
  EXPECT_EQ(kvx_gather_features(&s, FAKE, 0, FAKE, -1, tp, 2, FAKE, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_gather_features(&s, NULL, 0, FAKE, 3, tp, 2, FAKE, NULL), KVX_ERR_INVALID);
  kvx_cache_desc s0 = desc(4, 0, 2, 8, KVX_BF16, 0.0);
  EXPECT_EQ(kvx_gather_features(&s0, FAKE, 0, FAKE, 3, tp, 2, FAKE, NULL), KVX_ERR_SHAPE);
  kvx_cache_desc odd = desc(4, 10, 1, 7, KVX_BF16, 0.0);
  EXPECT_EQ(kvx_gather_features(&odd, FAKE, 0, FAKE, 3, tp, 2, FAKE, NULL), KVX_ERR_UNSUPPORTED);
  free(tp);
  free(bad);
}

static void check_fits(void) {
  const size_t huge_ws = (size_t)1 << 40;
  EXPECT_EQ(kvx_fit_ridge(FAKE, 64, FAKE, 64, KVX_BF16, 10, 64, 64, -1.0, 0.0, 0, (float*)FAKE, NULL, FAKE,
                          huge_ws, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fit_ridge(FAKE, 64, FAKE, 64, KVX_BF16, 10, 64, 64, NAN, 0.0, 0, (float*)FAKE, NULL, FAKE, huge_ws,
                          NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fit_ridge(FAKE, 32, FAKE, 64, KVX_BF16, 10, 64, 64, 0.0, 0.0, 0, (float*)FAKE, NULL, FAKE, huge_ws,
                          NULL),
            KVX_ERR_SHAPE);
  EXPECT_EQ(kvx_fit_ridge(FAKE, 64, FAKE, 64, KVX_BF16, 10, 60, 64, 0.0, 0.0, 0, (float*)FAKE, NULL, FAKE, huge_ws,
                          NULL),
            KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(kvx_fit_ridge((void*)(uintptr_t)0x1008, 64, FAKE, 64, KVX_BF16, 10, 64, 64, 0.0, 0.0, 0, (float*)FAKE,
                          NULL, FAKE, huge_ws, NULL),
            KVX_ERR_UNSUPPORTED); /* bf16 rows must start on 16 bytes */
  EXPECT_EQ(kvx_fit_ridge(FAKE, 64, FAKE, 64, KVX_BF16, 10, 64, 64, 0.0, 0.0, 1, (float*)FAKE, NULL, FAKE, huge_ws,
                          NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fit_ridge(FAKE, 64, FAKE, 64, KVX_BF16, 10, 64, 64, 0.0, 0.0, 0, (float*)FAKE, NULL, FAKE, 16, NULL),
            KVX_ERR_WORKSPACE);
  EXPECT_EQ(kvx_fit_ridge(FAKE, 64, FAKE, 64, 3, 10, 64, 64, 0.0, 0.0, 0, (float*)FAKE, NULL, FAKE, huge_ws, NULL),
            KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fit_ridge(FAKE, 1 << 20, FAKE, 64, KVX_BF16, 10, KVX_MAX_FIT_FEATURES + 8, 64, 0.0, 0.0, 0,
                          (float*)FAKE, NULL, FAKE, huge_ws, NULL),
            KVX_ERR_UNSUPPORTED);

  /* several problems: pointer arrays of exactly `count` entries */
  const int count = 3;
  const void** xs = (const void**)malloc(count * sizeof(void*));
  const void** ys = (const void**)malloc(count * sizeof(void*));
  float** ws = (float**)malloc(count * sizeof(float*));
  float** bs = (float**)malloc(count * sizeof(float*));
  for (int i = 0; i < count; ++i) {
    xs[i] = ys[i] = FAKE;
    ws[i] = bs[i] = (float*)FAKE;
  }
  int32_t* status = (int32_t*)malloc(count * sizeof(int32_t));
  EXPECT_EQ(kvx_fit_ridge_batched(count, xs, 64, ys, 64, KVX_BF16, 10, 64, 64, 0.0, 1e-3, 1, ws, bs, status, FAKE,
                                  16, NULL),
            KVX_ERR_WORKSPACE);
  ws[2] = NULL;
  EXPECT_EQ(kvx_fit_ridge_batched(count, xs, 64, ys, 64, KVX_BF16, 10, 64, 64, 0.0, 1e-3, 1, ws, bs, status, FAKE,
                                  huge_ws, NULL),
            KVX_ERR_INVALID);
  ws[2] = (float*)FAKE;
  ys[1] = NULL;
  EXPECT_EQ(kvx_fit_ridge_batched(count, xs, 64, ys, 64, KVX_BF16, 10, 64, 64, 0.0, 1e-3, 1, ws, bs, status, FAKE,
                                  huge_ws, NULL),
            KVX_ERR_INVALID);
  ys[1] = FAKE;
  EXPECT_EQ(kvx_fit_ridge_batched(0, NULL, 64, NULL, 64, KVX_BF16, 10, 64, 64, 0.0, 1e-3, 1, NULL, NULL, NULL, NULL,
                                  0, NULL),
            KVX_OK);
  EXPECT_EQ(kvx_fit_ridge_batched(-1, xs, 64, ys, 64, KVX_BF16, 10, 64, 64, 0.0, 1e-3, 1, ws, bs, status, FAKE,
                                  huge_ws, NULL),
            KVX_ERR_INVALID);
  /* more problems than one call takes: refused before the pointer arrays are read */
  EXPECT_EQ(kvx_fit_ridge_batched(KVX_MAX_PROBLEMS + 1, xs, 64, ys, 64, KVX_BF16, 10, 64, 64, 0.0, 1e-3, 1, ws, bs,
                                  status, FAKE, huge_ws, NULL),
            KVX_ERR_UNSUPPORTED);

#define RC(cnt, ldx, fi, fo, dt, rx, ry, w, b, wsb) \
  kvx_fit_recolor(cnt, xs, ldx, ys, 64, dt, 10, fi, fo, rx, ry, w, b, status, NULL, FAKE, wsb, NULL)
  EXPECT_EQ(RC(0, 64, 64, 64, KVX_BF16, 1e-3, 0.0, ws, bs, huge_ws), KVX_OK);
  EXPECT_EQ(RC(count, 64, 64, 64, KVX_BF16, -1.0, 0.0, ws, bs, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(count, 64, 64, 64, KVX_BF16, 1e-3, 0.0, ws, NULL, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(count, 32, 64, 64, KVX_BF16, 1e-3, 0.0, ws, bs, huge_ws), KVX_ERR_SHAPE);
  EXPECT_EQ(RC(count, 64, 32, 64, KVX_BF16, 1e-3, 0.0, ws, bs, huge_ws), KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(RC(count, 64, 60, 56, KVX_BF16, 1e-3, 0.0, ws, bs, huge_ws), KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(RC(count, 64, 64, 64, KVX_BF16, 1e-3, 0.0, ws, bs, 16), KVX_ERR_WORKSPACE);
  EXPECT_EQ(RC(KVX_MAX_PROBLEMS + 1, 64, 64, 64, KVX_BF16, 1e-3, 0.0, ws, bs, huge_ws), KVX_ERR_UNSUPPORTED);
  bs[0] = NULL;
  EXPECT_EQ(RC(count, 64, 64, 64, KVX_BF16, 1e-3, 0.0, ws, bs, huge_ws), KVX_ERR_INVALID);
#undef RC
  free(xs);
  free(ys);
  free(ws);
  free(bs);
  free(status);
}

static void check_fit_from_caches(const int32_t* taps36) {
  const size_t huge_ws = (size_t)1 << 40;
  kvx_cache_desc s = desc(36, 50000, 8, 128, KVX_BF16, 0.0), r = desc(32, 65536, 8, 128, KVX_BF16, 0.0);
  EXPECT(kvx_fit_ridge_caches_workspace_size(&s, &r, 3) > (size_t)64 * 8 * (3072 * 3072 + 3072 * 1024));
  kvx_cache_desc rmax = desc(255, INT32_MAX, 8, 128, KVX_BF16, 0.0), smax = desc(255, INT32_MAX, 8, 128, KVX_BF16, 0.0);
  EXPECT(kvx_fit_ridge_caches_workspace_size(&smax, &rmax, 7) > 0);
  kvx_cache_desc r0 = desc(32, 0, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(kvx_fit_ridge_caches_workspace_size(&s, &r0, 3), 0);
  float* w = (float*)FAKE;
#define FC(sd, rd, ks, kr, map, taps, nt, lam, wk, wv, wsb) \
  kvx_fit_ridge_caches(sd, ks, FAKE, rd, kr, FAKE, map, taps, nt, 0.0, lam, wk, wv, NULL, FAKE, wsb, NULL)
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, FAKE, taps36, 3, 1e-3, NULL, NULL, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, FAKE, taps36, 3, NAN, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(FC(&s, &r, NULL, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, NULL, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, FAKE, NULL, 3, 1e-3, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, FAKE, taps36, 0, 1e-3, w, w, huge_ws), KVX_ERR_INVALID);
  int32_t* bad = exact_i32(taps36, 96);
  bad[95] = 36;
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, FAKE, bad, 3, 1e-3, w, w, huge_ws), KVX_ERR_INVALID);
  free(bad);
  /* rotated keys are turned back 8 pairs at a time: head_dim a multiple of 16 */
  kvx_cache_desc srot = desc(36, 50000, 32, 8, KVX_BF16, 1e4), rrot = desc(32, 65536, 32, 8, KVX_BF16, 1e6);
  EXPECT_EQ(FC(&srot, &r, FAKE, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(FC(&s, &rrot, FAKE, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
  /* workspace sizes grow by the (cos, sin) tables of rotated keys */
  kvx_cache_desc s_rope = desc(36, 50000, 8, 128, KVX_BF16, 1e4);
  EXPECT(kvx_fit_ridge_caches_workspace_size(&s_rope, &r, 3) >= kvx_fit_ridge_caches_workspace_size(&s, &r, 3) +
                                                                    (size_t)50000 * 64 * 8);
  kvx_cache_desc snarrow = desc(36, 50000, 3, 64, KVX_BF16, 0.0);
  EXPECT_EQ(FC(&snarrow, &r, FAKE, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(FC(&s, &r, (void*)(uintptr_t)0x1008, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(FC(&s, &r0, FAKE, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_SHAPE);
  EXPECT_EQ(FC(&s, &r, FAKE, FAKE, FAKE, taps36, 3, 1e-3, w, w, 16), KVX_ERR_WORKSPACE);
  /* the Gram's 32-bit offsets: too many calibration tokens for one call */
  kvx_cache_desc rbig = desc(32, 1 << 26, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(FC(&s, &rbig, FAKE, FAKE, FAKE, taps36, 3, 1e-3, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
#undef FC
}

static void check_recolor_from_caches(const int32_t* taps36) {
  const size_t huge_ws = (size_t)1 << 40;
  kvx_cache_desc s = desc(36, 50000, 8, 128, KVX_BF16, 0.0), r = desc(32, 65536, 8, 128, KVX_BF16, 0.0);
  EXPECT(kvx_fit_recolor_caches_workspace_size(&s, &r, 3) > kvx_fit_ridge_caches_workspace_size(&s, &r, 3));
  kvx_cache_desc rmax = desc(255, INT32_MAX, 8, 128, KVX_BF16, 0.0), smax = desc(255, INT32_MAX, 8, 128, KVX_BF16, 0.0);
  EXPECT(kvx_fit_recolor_caches_workspace_size(&smax, &rmax, 7) > 0);
  kvx_cache_desc r0 = desc(32, 0, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(kvx_fit_recolor_caches_workspace_size(&s, &r0, 3), 0);
  float* w = (float*)FAKE;
  int32_t status[64], iters = 0;
#define RC(sd, rd, ks, map, taps, nt, rho, wk, wv, bk, bv, wsb)                                              \
  kvx_fit_recolor_caches(sd, ks, FAKE, rd, FAKE, FAKE, map, taps, nt, rho, 0.0, wk, wv, bk, bv, status, &iters, \
                         FAKE, wsb, NULL)
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, taps36, 3, 1e-3, NULL, NULL, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, taps36, 3, NAN, w, w, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, taps36, 3, 1e-3, w, w, NULL, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, taps36, 3, 1e-3, w, w, w, NULL, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(&s, &r, NULL, FAKE, taps36, 3, 1e-3, w, w, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(&s, &r, FAKE, NULL, taps36, 3, 1e-3, w, w, w, w, huge_ws), KVX_ERR_INVALID);
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, NULL, 3, 1e-3, w, w, w, w, huge_ws), KVX_ERR_INVALID);
  int32_t* bad = exact_i32(taps36, 96);
  bad[0] = -1;
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, bad, 3, 1e-3, w, w, w, w, huge_ws), KVX_ERR_INVALID);
  free(bad);
  /* F_in < F_out: one tap of a 2 x 128 sender row, 8 x 128 targets */
  kvx_cache_desc s2 = desc(36, 50000, 2, 128, KVX_BF16, 0.0);
  int32_t* one = exact_i32(taps36, 32);
  for (int i = 0; i < 32; ++i) one[i] = i;
  EXPECT_EQ(RC(&s2, &r, FAKE, FAKE, one, 1, 1e-3, w, w, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
  free(one);
  EXPECT_EQ(RC(&s, &r0, FAKE, FAKE, taps36, 3, 1e-3, w, w, w, w, huge_ws), KVX_ERR_SHAPE);
  EXPECT_EQ(RC(&s, &r, FAKE, FAKE, taps36, 3, 1e-3, w, w, w, w, 16), KVX_ERR_WORKSPACE);
  kvx_cache_desc rbig = desc(32, 1 << 26, 8, 128, KVX_BF16, 0.0);
  EXPECT_EQ(RC(&s, &rbig, FAKE, FAKE, taps36, 3, 1e-3, w, w, w, w, huge_ws), KVX_ERR_UNSUPPORTED);
#undef RC
}

static void check_maps_and_probes(void) {
  const float* w = (const float*)FAKE;
  EXPECT_EQ(kvx_quantize_fp8(w, 0, 16, 16, (uint8_t*)FAKE, (float*)FAKE, NULL), KVX_OK);
  EXPECT_EQ(kvx_quantize_fp8(w, 4, 0, 16, (uint8_t*)FAKE, (float*)FAKE, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_quantize_fp8(w, 4, 16, 0, (uint8_t*)FAKE, (float*)FAKE, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_quantize_fp8(w, 4, 16, 16, NULL, (float*)FAKE, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_quantize_fp8(w, 65536, 16, 16, (uint8_t*)FAKE, (float*)FAKE, NULL), KVX_ERR_UNSUPPORTED);
  EXPECT_EQ(kvx_fold_lowrank(w, w, w, 0, 8, 8, 2, FAKE, KVX_BF16, NULL), KVX_OK);
  EXPECT_EQ(kvx_fold_lowrank(w, NULL, w, 1, 8, 8, 2, FAKE, KVX_BF16, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fold_lowrank(w, w, w, 1, 8, 8, 2, FAKE, 5, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fold_lowrank(w, w, w, 1, 8, 8, -1, FAKE, KVX_BF16, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_fold_lowrank(NULL, w, w, 1, 8, 8, 2, FAKE, KVX_BF16, NULL), KVX_ERR_INVALID);
  float ms = 0.0f;
  double fl = 0.0;
  EXPECT_EQ(kvx_probe_hbm(3, FAKE, FAKE, 1024, 1, &ms, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_probe_hbm(0, FAKE, NULL, 1024, 1, &ms, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_probe_hbm(2, FAKE, NULL, 1000, 1, &ms, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_probe_hbm(2, FAKE, NULL, 1024, 0, &ms, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_probe_hbm(2, FAKE, NULL, INT64_MIN, 1, &ms, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_probe_mfma((float*)FAKE, 0, 1, &ms, &fl, NULL), KVX_ERR_INVALID);
  EXPECT_EQ(kvx_probe_mfma((float*)FAKE, 1, 1, NULL, &fl, NULL), KVX_ERR_INVALID);
}

int main(void) {
  int32_t* taps36 = (int32_t*)malloc(32 * 3 * sizeof(int32_t));
  if (kvx_layer_map(36, 32, 3, 4, taps36) != KVX_OK) return 2;
  check_status_strings();
  check_layer_map();
  check_alignment();
  check_descriptors(taps36);
  check_sizes();
  check_translate(taps36);
  check_gather();
  check_fits();
  check_fit_from_caches(taps36);
  check_recolor_from_caches(taps36);
  check_maps_and_probes();
  free(taps36);
  if (failures) {
    fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
