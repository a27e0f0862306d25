/*
 * Drives the C oracle (oracle/kda_oracle.c) through every input mode under
 * AddressSanitizer and UndefinedBehaviorSanitizer (built and run by
 * tests/test_oracle_sanitized.py, CPU only): bf16, fp32 and fp64 inputs; zero and
 * nonzero initial states; all pairs and a listed subset; outputs per token,
 * packed per pair, and not stored; empty sequences; and every argument error.
 * Exit status 0 when every call returns what it should; the sanitizers abort on any
 * invalid access or undefined operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_kda_forward(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, int in_dtype, const void* s0, int s0_dtype,
                    const int64_t* seq_start, const int64_t* seq_len, int N, int H,
                    int dk, int dv, double scale, const int32_t* pairs, int npairs,
                    double* out, int out_mode, double* sT, int nthreads);

static uint32_t rng = 12345u;
static double urand(void) {   /* uniform in [-1, 1) */
  rng = rng * 1664525u + 1013904223u;
  return (double)(rng >> 8) / (double)(1u << 23) - 1.0;
}

static void fill(void* p, int dtype, size_t n, double lo, double hi) {
  for (size_t i = 0; i < n; ++i) {
    const double x = lo + (hi - lo) * 0.5 * (urand() + 1.0);
    if (dtype == 0) {
      const float f = (float)x;
      uint32_t b;
      memcpy(&b, &f, 4);
      ((uint16_t*)p)[i] = (uint16_t)(b >> 16);
    } else if (dtype == 1) {
      ((float*)p)[i] = (float)x;
    } else {
      ((double*)p)[i] = x;
    }
  }
}

int main(void) {
  const int H = 3, dk = 8, dv = 4, N = 4;
  const int64_t start[4] = {0, 5, 5, 17};
  const int64_t len[4] = {5, 0, 12, 3};
  const int total = 20;
  const size_t esz[3] = {2, 4, 8};
  int failures = 0;
  for (int dt = 0; dt < 3; ++dt) {
    void* q = malloc(esz[dt] * total * H * dk);
    void* k = malloc(esz[dt] * total * H * dk);
    void* g = malloc(esz[dt] * total * H * dk);
    void* v = malloc(esz[dt] * total * H * dv);
    void* b = malloc(esz[dt] * total * H);
    float* s0 = malloc(sizeof(float) * N * H * dk * dv);
    fill(q, dt, (size_t)total * H * dk, -1, 1);
    fill(k, dt, (size_t)total * H * dk, -0.3, 0.3);
    fill(g, dt, (size_t)total * H * dk, -5, 0);
    fill(v, dt, (size_t)total * H * dv, -1, 1);
    fill(b, dt, (size_t)total * H, 0, 1);
    fill(s0, 1, (size_t)N * H * dk * dv, -0.1, 0.1);
    double* out = calloc((size_t)total * H * dv, sizeof(double));
    double* packed = calloc((size_t)total * H * dv, sizeof(double));
    double* sT = calloc((size_t)N * H * dk * dv, sizeof(double));
    const int32_t pairs[6] = {2, 1, 0, 0, 3, 2};
    for (int with_s0 = 0; with_s0 < 2; ++with_s0) {
      failures += orc_kda_forward(q, k, v, g, b, dt, with_s0 ? s0 : NULL, 1, start, len, N, H,
                                  dk, dv, 0.5, NULL, 0, out, 0, sT, 2) != 0;
      failures += orc_kda_forward(q, k, v, g, b, dt, with_s0 ? s0 : NULL, 1, start, len, N, H,
                                  dk, dv, 0.5, pairs, 3, packed, 1, sT, 1) != 0;
      failures += orc_kda_forward(q, k, v, g, b, dt, with_s0 ? s0 : NULL, 1, start, len, N, H,
                                  dk, dv, 0.5, pairs, 3, NULL, 0, sT, 0) != 0;
    }
    for (size_t i = 0; i < (size_t)total * H * dv; ++i) failures += !isfinite(out[i]);
    /* argument errors */
    failures += orc_kda_forward(NULL, k, v, g, b, dt, NULL, 1, start, len, N, H, dk, dv, 1, NULL, 0,
                                out, 0, sT, 1) != -1;
    failures += orc_kda_forward(q, k, v, g, b, dt, NULL, 1, start, len, 0, H, dk, dv, 1, NULL, 0,
                                out, 0, sT, 1) != -2;
    failures += orc_kda_forward(q, k, v, g, b, 7, NULL, 1, start, len, N, H, dk, dv, 1, NULL, 0,
                                out, 0, sT, 1) != -3;
    failures += orc_kda_forward(q, k, v, g, b, dt, NULL, 1, start, len, N, H, dk, dv, 1, pairs, 0,
                                out, 0, sT, 1) != -4;
    const int32_t bad[2] = {9, 0};
    failures += orc_kda_forward(q, k, v, g, b, dt, NULL, 1, start, len, N, H, dk, dv, 1, bad, 1,
                                out, 0, sT, 1) != -6;
    free(q); free(k); free(g); free(v); free(b); free(s0); free(out); free(packed); free(sT);
  }
  printf("oracle sanitizer driver: %d failures\n", failures);
  return failures != 0;
}
