/* Host-side driver for the sanitizer test (tests/test_host_sanitizers.py):
 * walks the C ABI's argument validation and size arithmetic, which run on
 * the host before any device work, and checks the status codes.  Built with
 * AddressSanitizer and UndefinedBehaviorSanitizer around salr_api.cpp; no
 * GPU is needed (no call here reaches the device).  Prints "ok" and exits 0
 * when every expectation holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "salr.h"

static int failures = 0;

#define EXPECT(cond)                                          \
  do {                                                        \
    if (!(cond)) {                                            \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                             \
    }                                                         \
  } while (0)

/* A layer record with fake, 256-byte-aligned device addresses (never
 * dereferenced by the validation paths exercised here). */
static salr_layer_t fake_layer(int64_t N, int64_t K, int32_t n_keep, int32_t r_cat) {
  salr_layer_t L;
  memset(&L, 0, sizeof L);
  L.N = N;
  L.K = K;
  L.n_keep = n_keep;
  L.r_cat = r_cat;
  L.masks = (uint64_t*)(uintptr_t)0x100000;
  L.values = (uint16_t*)(uintptr_t)0x200000;
  L.offsets = (uint32_t*)(uintptr_t)0x300000;
  L.a_cat = (uint16_t*)(uintptr_t)0x400000;
  L.b_cat = (uint16_t*)(uintptr_t)0x500000;
  return L;
}

static void sizes(void) {
  salr_sizes_t s;
  /* valid shapes, including large ones (size arithmetic in 64 bits) */
  const int64_t shapes[][6] = {
      {4096, 4096, 2048, 64, 80, 16},     {28672, 8192, 4096, 128, 160, 8192},
      {8192, 28672, 14336, 128, 160, 8192}, {512, 512, 256, 16, 24, 16},
      {17, 104, 1, 0, 0, 1},              {1, 64, 64, 0, 8, 0},
  };
  for (size_t k = 0; k < sizeof shapes / sizeof shapes[0]; ++k) {
    const int64_t* v = shapes[k];
    memset(&s, 0xA5, sizeof s);
    EXPECT(salr_query_sizes(v[0], v[1], (int32_t)v[2], (int32_t)v[3], (int32_t)v[4], v[5], &s) == SALR_OK);
    EXPECT(s.masks_bytes == (size_t)(v[0] * ((v[1] + 63) / 64) * 8));
    EXPECT(s.values_bytes >= (size_t)(v[0] * v[2] * 2));
    EXPECT(s.a_cat_bytes == (size_t)(v[4] * v[1] * 2));
    EXPECT(s.b_cat_bytes >= (size_t)(v[0] * v[4] * 2));
  }
  /* invalid: null output, non-positive or oversized dimensions, ranks */
  EXPECT(salr_query_sizes(64, 64, 32, 0, 8, 16, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(0, 64, 32, 0, 8, 16, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(64, -1, 32, 0, 8, 16, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(64, 100, 32, 0, 8, 16, &s) == SALR_ERR_INVALID_ARG); /* K % 8 */
  EXPECT(salr_query_sizes(64, 64, 65, 0, 8, 16, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(64, 64, -1, 0, 8, 16, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(64, 64, 32, 9, 8, 16, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(64, 64, 32, -1, 8, 16, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(64, 64, 32, 0, 8, -5, &s) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_query_sizes(INT64_MAX / 2, INT64_MAX / 2, 32, 0, 8, 16, &s) != SALR_OK);
  EXPECT(salr_query_sizes(64, 64, 32, 0, 1 << 20, 16, &s) != SALR_OK);

  size_t t = 0;
  EXPECT(salr_transpose_ws_bytes(4096, 4096, &t) == SALR_OK && t > 0);
  EXPECT(salr_transpose_ws_bytes(4096, 4096, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_transpose_ws_bytes(-4, 4096, &t) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_backward_ws_bytes(4096, 4096, 2100, 80, 2048, &t) == SALR_OK && t > 0);
  EXPECT(salr_backward_ws_bytes(4096, 4096, 2100, 80, 2048, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_backward_ws_bytes(4096, 4096, -1, 80, 2048, &t) != SALR_OK);

  salr_moe_sizes_t ms;
  EXPECT(salr_moe_query_sizes(8, 14336, 4096, 2048, 80, 32, &ms) == SALR_OK);
  EXPECT(salr_moe_query_sizes(0, 14336, 4096, 2048, 80, 32, &ms) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_moe_query_sizes(8, 14336, 4096, 2048, 80, 32, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_moe_query_sizes(1 << 30, 14336, 4096, 2048, 80, 32, &ms) != SALR_OK);

  float lv[16];
  EXPECT(salr_nf4_levels(lv) == SALR_OK && lv[0] == -1.0f && lv[15] == 1.0f && lv[7] == 0.0f);
  EXPECT(salr_nf4_levels(NULL) == SALR_ERR_INVALID_ARG);
}

static void calls(void) {
  salr_layer_t L = fake_layer(256, 1024, 512, 16);
  const uint16_t* X = (const uint16_t*)(uintptr_t)0x600000;
  uint16_t* Y = (uint16_t*)(uintptr_t)0x700000;
  void* ws = (void*)(uintptr_t)0x800000;
  salr_sizes_t s;
  EXPECT(salr_query_sizes(256, 1024, 512, 0, 16, 64, &s) == SALR_OK);

  /* forward: nulls, negative M, a workspace that is too small, a bad part
   * record, misaligned pointers */
  EXPECT(salr_linear_forward(NULL, X, 16, Y, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_linear_forward(&L, NULL, 16, Y, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_linear_forward(&L, X, 16, NULL, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_linear_forward(&L, X, -1, Y, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_linear_forward(&L, X, 16, Y, NULL, s.forward_ws_bytes, NULL) == SALR_ERR_WORKSPACE);
  EXPECT(salr_linear_forward(&L, X, 16, Y, ws, 16, NULL) == SALR_ERR_WORKSPACE);
  salr_layer_t bad = L;
  bad.n_parts = 9;
  EXPECT(salr_linear_forward(&bad, X, 16, Y, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  bad = L;
  bad.n_parts = 2;
  bad.part_rows[0] = 128;
  bad.part_rows[1] = 64; /* rows do not sum to N */
  bad.part_ranks[0] = 8;
  bad.part_ranks[1] = 8;
  EXPECT(salr_linear_forward(&bad, X, 16, Y, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  bad = L;
  bad.values = (uint16_t*)(uintptr_t)0x200001;
  EXPECT(salr_linear_forward(&bad, X, 16, Y, ws, s.forward_ws_bytes, NULL) == SALR_ERR_INVALID_ARG);
  bad = L;
  bad.value_format = 7;
  EXPECT(salr_linear_forward(&bad, X, 16, Y, ws, s.forward_ws_bytes, NULL) != SALR_OK);
  EXPECT(salr_linear_forward_noalloc(NULL, X, 16, Y, NULL, NULL) == SALR_ERR_INVALID_ARG);

  /* encode: shapes, nulls, r_cat that disagrees with the ranks */
  const uint16_t* W = (const uint16_t*)(uintptr_t)0x900000;
  salr_layer_t E = fake_layer(256, 1024, 512, 16);
  EXPECT(salr_encode(NULL, 256, 1024, 512, 16, 0, NULL, NULL, NULL, NULL, &E, NULL, ws, s.encode_ws_bytes, NULL) ==
         SALR_ERR_INVALID_ARG);
  EXPECT(salr_encode(W, 256, 1024, 512, 16, 0, NULL, NULL, NULL, NULL, NULL, NULL, ws, s.encode_ws_bytes, NULL) ==
         SALR_ERR_INVALID_ARG);
  E.r_cat = 17;
  EXPECT(salr_encode(W, 256, 1024, 512, 16, 0, NULL, NULL, NULL, NULL, &E, NULL, ws, s.encode_ws_bytes, NULL) ==
         SALR_ERR_INVALID_ARG);
  E.r_cat = 16;
  EXPECT(salr_encode(W, 256, 1024, 512, 16, 1, NULL, NULL, NULL, NULL, &E, NULL, ws, s.encode_ws_bytes, NULL) ==
         SALR_ERR_INVALID_ARG);
  EXPECT(salr_encode(W, 256, 1024, 512, 16, 0, NULL, NULL, NULL, NULL, &E, NULL, ws, 8, NULL) == SALR_ERR_WORKSPACE);
  salr_encode_opts_t o = {100, 24, 0};
  EXPECT(salr_encode(W, 256, 1024, 512, 16, 0, NULL, NULL, NULL, &o, &E, NULL, ws, s.encode_ws_bytes, NULL) ==
         SALR_ERR_INVALID_ARG);

  /* fusion: part counts and mismatched shapes */
  salr_layer_t P0 = fake_layer(128, 1024, 512, 8), P1 = fake_layer(128, 512, 512, 8);
  const salr_layer_t* parts[2] = {&P0, &P1};
  salr_layer_t F = fake_layer(256, 1024, 512, 16);
  EXPECT(salr_fuse_layers(parts, 0, &F, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_fuse_layers(parts, 9, &F, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_fuse_layers(parts, 2, &F, NULL) == SALR_ERR_INVALID_ARG); /* K differs */
  EXPECT(salr_fuse_layers(NULL, 2, &F, NULL) == SALR_ERR_INVALID_ARG);

  /* NF4, transpose, backward, MoE: nulls and records that do not fit */
  EXPECT(salr_quantize_nf4(NULL, NULL) == SALR_ERR_INVALID_ARG);
  int32_t nkt = 0;
  EXPECT(salr_transpose_count(NULL, &nkt, ws, 1 << 20, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_transpose_layer(&L, NULL, ws, 1 << 20, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_linear_backward(NULL, NULL, X, X, 16, NULL, NULL, NULL, ws, 1 << 20, NULL) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_linear_backward(&L, &L, X, X, -3, Y, NULL, NULL, ws, 1 << 20, NULL) == SALR_ERR_INVALID_ARG);
  salr_moe_layer_t G;
  memset(&G, 0, sizeof G);
  salr_layer_t one;
  EXPECT(salr_moe_expert(NULL, 0, &one) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_moe_expert(&G, -1, &one) == SALR_ERR_INVALID_ARG);
  EXPECT(salr_moe_forward(NULL, X, 16, NULL, 0, Y, ws, 1 << 20, NULL) == SALR_ERR_INVALID_ARG);

  /* status strings */
  for (int c = -8; c <= 1; ++c) EXPECT(salr_status_string(c) != NULL && strlen(salr_status_string(c)) > 0);
  EXPECT(salr_version() > 0);
}

int main(void) {
  sizes();
  calls();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
