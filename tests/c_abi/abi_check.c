/*
 * The C ABI used from plain C, with no Python in between.
 *
 *   abi_check host   argument checks, sizes and messages (no device needed)
 *   abi_check gpu    device buffers from the HIP runtime and two calls whose results the
 *                    pages fix exactly: a greedy call against the target argmax, and a
 *                    sampling call whose draft equals its target (every draft accepted)
 *
 * Prints one line per check and exits 0 only if all pass.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_verify.h"

static int failures = 0;

#define CHECK(cond, ...)                 \
  do {                                   \
    if (cond) {                          \
      printf("ok    ");                  \
    } else {                             \
      printf("FAIL  ");                  \
      ++failures;                        \
    }                                    \
    printf(__VA_ARGS__);                 \
    printf("\n");                        \
  } while (0)

static int host_checks(void) {
  const size_t ws = spec_verify_workspace_size(8, 4, 32000, SPEC_BF16);
  CHECK(ws > 0, "workspace size for B=8 gamma=4 V=32000 bf16: %zu bytes", ws);
  CHECK(spec_verify_workspace_size(8, SPEC_MAX_GAMMA + 1, 32000, SPEC_BF16) == 0,
        "gamma above SPEC_MAX_GAMMA has no workspace size");
  CHECK(strlen(spec_verify_strerror(SPEC_ERR_WORKSPACE)) > 0, "strerror: %s",
        spec_verify_strerror(SPEC_ERR_WORKSPACE));
  int rc = spec_verify_sample(NULL, NULL, SPEC_BF16, NULL, NULL, NULL, 8, 4, NULL, 32000, NULL,
                              NULL, NULL, 0, NULL, NULL);
  CHECK(rc == SPEC_ERR_NULL, "NULL buffers: %d", rc);
  rc = spec_verify_greedy(NULL, SPEC_BF16, NULL, 0, 4, NULL, 32000, NULL, NULL, NULL, 0, NULL,
                          NULL);
  CHECK(rc == SPEC_OK, "an empty batch is a no-op: %d", rc);
  rc = spec_verify_sample(NULL, NULL, 7, NULL, NULL, NULL, 8, 4, NULL, 32000, NULL, NULL, NULL,
                          0, NULL, NULL);
  CHECK(rc == SPEC_ERR_DTYPE, "unknown dtype: %d", rc);
  return failures;
}

/* ---- device part: the HIP runtime's C API, declared here to keep the build plain C ---- */
typedef int hipError_t;
extern hipError_t hipMalloc(void **ptr, size_t size);
extern hipError_t hipFree(void *ptr);
extern hipError_t hipMemcpy(void *dst, const void *src, size_t bytes, int kind);
extern hipError_t hipMemset(void *dst, int value, size_t bytes);
extern hipError_t hipDeviceSynchronize(void);
enum { kH2D = 1, kD2H = 2 };

static void *dev_copy(const void *src, size_t bytes) {
  void *p = NULL;
  if (hipMalloc(&p, bytes) != 0) {
    printf("FAIL  hipMalloc of %zu bytes\n", bytes);
    exit(2);
  }
  if (src) hipMemcpy(p, src, bytes, kH2D);
  return p;
}

/* a small reproducible pseudo-random sequence for the logits (not part of the method) */
static uint32_t lcg = 12345u;
static float next_logit(void) {
  lcg = lcg * 1664525u + 1013904223u;
  return (float)((lcg >> 8) & 0xffff) / 4096.0f - 8.0f;  /* in [-8, 8) */
}

static int gpu_checks(void) {
  enum { B = 4, G = 3, V = 5000 };
  const int rows_t = B * (G + 1), rows_d = B * G;
  float *target = malloc(sizeof(float) * rows_t * V);
  float *draft = malloc(sizeof(float) * rows_d * V);
  int32_t tokens[B * G], argmax[B * (G + 1)];
  float uniforms[B * (G + 1) * 2], temps[B];
  for (int r = 0; r < rows_t; ++r) {
    for (int k = 0; k < V; ++k) target[(size_t)r * V + k] = next_logit();
    argmax[r] = (r * 811 + 17) % V;  /* one clear maximum per row */
    target[(size_t)r * V + argmax[r]] = 20.0f;
  }
  /* greedy: request b's drafts follow the argmax up to position b % (G + 1), then differ */
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < G; ++i) {
      const int r = b * (G + 1) + i;
      tokens[b * G + i] = i < b % (G + 1) ? argmax[r] : (argmax[r] + 1) % V;
    }
  const size_t ws_bytes = spec_verify_workspace_size(B, G, V, SPEC_F32);
  void *ws = dev_copy(NULL, ws_bytes);
  hipMemset(ws, 0, ws_bytes);
  float *d_t = dev_copy(target, sizeof(float) * rows_t * V);
  int32_t *d_tok = dev_copy(tokens, sizeof tokens);
  int32_t *d_out = dev_copy(NULL, sizeof(int32_t) * rows_t);
  int32_t *d_n = dev_copy(NULL, sizeof(int32_t) * B);
  int rc = spec_verify_greedy(d_t, SPEC_F32, d_tok, B, G, NULL, V, d_out, d_n, ws, ws_bytes,
                              NULL, NULL);
  hipDeviceSynchronize();
  CHECK(rc == SPEC_OK, "greedy call: %d", rc);
  int32_t out[B * (G + 1)], n[B];
  hipMemcpy(out, d_out, sizeof out, kD2H);
  hipMemcpy(n, d_n, sizeof n, kD2H);
  for (int b = 0; b < B; ++b) {
    const int want = b % (G + 1);
    int ok = n[b] == want;
    for (int i = 0; i <= G; ++i) {
      const int r = b * (G + 1) + i;
      const int32_t expect = i < want ? tokens[b * G + i] : (i == want ? argmax[r] : -1);
      ok = ok && out[r] == expect;
    }
    CHECK(ok, "greedy request %d: %d accepted, the target argmax emitted at the mismatch", b,
          n[b]);
  }
  /* sampling with the draft equal to the target: min(1, p/q) = 1, every draft is accepted */
  for (int b = 0; b < B; ++b) {
    temps[b] = 0.5f + 0.25f * (float)b;
    for (int i = 0; i < G; ++i)
      memcpy(draft + (size_t)(b * G + i) * V, target + (size_t)(b * (G + 1) + i) * V,
             sizeof(float) * V);
  }
  for (int i = 0; i < B * (G + 1) * 2; ++i) uniforms[i] = (float)((i * 37) % 100) / 100.0f;
  float *d_d = dev_copy(draft, sizeof(float) * rows_d * V);
  float *d_u = dev_copy(uniforms, sizeof uniforms);
  float *d_temps = dev_copy(temps, sizeof temps);
  hipMemset(ws, 0, ws_bytes);
  rc = spec_verify_sample(d_t, d_d, SPEC_F32, d_tok, d_u, d_temps, B, G, NULL, V, d_out, d_n, ws,
                          ws_bytes, NULL, NULL);
  hipDeviceSynchronize();
  CHECK(rc == SPEC_OK, "sampling call: %d", rc);
  hipMemcpy(out, d_out, sizeof out, kD2H);
  hipMemcpy(n, d_n, sizeof n, kD2H);
  for (int b = 0; b < B; ++b) {
    int ok = n[b] == G;
    for (int i = 0; i < G; ++i) ok = ok && out[b * (G + 1) + i] == tokens[b * G + i];
    ok = ok && out[b * (G + 1) + G] >= 0 && out[b * (G + 1) + G] < V;
    CHECK(ok, "p = q, request %d: all %d drafts accepted, bonus token %d", b, n[b],
          out[b * (G + 1) + G]);
  }
  hipFree(ws);
  hipFree(d_t);
  hipFree(d_d);
  hipFree(d_tok);
  hipFree(d_u);
  hipFree(d_temps);
  hipFree(d_out);
  hipFree(d_n);
  free(target);
  free(draft);
  return failures;
}

int main(int argc, char **argv) {
  if (argc < 2 || (strcmp(argv[1], "host") != 0 && strcmp(argv[1], "gpu") != 0)) {
    fprintf(stderr, "usage: %s host|gpu\n", argv[0]);
    return 2;
  }
  host_checks();
  if (strcmp(argv[1], "gpu") == 0) gpu_checks();
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
  return failures ? 1 : 0;
}
