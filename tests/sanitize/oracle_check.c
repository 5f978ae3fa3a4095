/* Drives the C oracle (oracle/ssd_ref.c) on small dense and packed cases, its
 * argument checks and its backward pass, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer: any out-of-bounds access, use after free, leak,
 * signed overflow or misaligned access fails the run.  Exit status 0 when
 * every call returned what it should and every output is finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int ssd_ref_fwd(int64_t batch, int64_t seqlen, int64_t H, int64_t P, int64_t N, int64_t G,
                int64_t Gc, int64_t nseqs, const int32_t* cu_seqlens, const float* x,
                const float* dt, const float* A, const float* B, const float* C, const float* D,
                const float* dt_bias, const float* init, unsigned flags, double dt_min,
                double dt_max, int64_t n_pairs, const int64_t* pairs, double* y,
                double* final_states);
int ssd_ref_bwd(int64_t batch, int64_t seqlen, int64_t H, int64_t P, int64_t N, int64_t G,
                int64_t Gc, int64_t nseqs, const int32_t* cu_seqlens, const float* x,
                const float* dt, const float* A, const float* B, const float* C, const float* D,
                const float* dt_bias, const float* init, unsigned flags, double dt_min,
                double dt_max, const float* dy, const float* dfinal, double* dx, double* ddt,
                double* dA, double* dB, double* dC, double* dD, double* ddt_bias,
                double* dinit);

static uint64_t rng = 88172645463325252ull;
static float uniform(void) { /* xorshift64, in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (float)((double)(rng >> 11) / 4503599627370496.0 - 1.0);
}
static float* fill(size_t n, float lo, float hi) {
  float* v = malloc(n * sizeof(float) + 1);
  for (size_t i = 0; i < n; ++i) v[i] = lo + (hi - lo) * 0.5f * (uniform() + 1.0f);
  return v;
}
static double* dbl(size_t n) { return calloc(n + 1, sizeof(double)); }
static int finite(const double* v, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(v[i])) return 0;
  return 1;
}

static int failures = 0;
#define CHECK(cond, what)                            \
  do {                                               \
    if (!(cond)) {                                   \
      fprintf(stderr, "oracle check failed: %s\n", what); \
      ++failures;                                    \
    }                                                \
  } while (0)

static void run(int64_t b, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Gc,
                int64_t nseqs, const int32_t* cu, int with_init, unsigned flags) {
  const int64_t S = cu ? nseqs : b;
  float* x = fill((size_t)(b * L * H * P), -1, 1);
  float* dt = fill((size_t)(b * L * H), -3, 1);
  float* A = fill((size_t)H, -4, -0.5f);
  float* B = fill((size_t)(b * L * G * N), -1, 1);
  float* C = fill((size_t)(b * L * Gc * N), -1, 1);
  float* D = fill((size_t)H, -1, 1);
  float* bias = fill((size_t)H, -0.5f, 0.5f);
  float* init = with_init ? fill((size_t)(S * H * N * P), -1, 1) : NULL;
  float* dy = fill((size_t)(b * L * H * P), -1, 1);
  float* dfin = fill((size_t)(S * H * N * P), -1, 1);
  double* y = dbl((size_t)(b * L * H * P));
  double* fin = dbl((size_t)(S * H * N * P));
  CHECK(ssd_ref_fwd(b, L, H, P, N, G, Gc, nseqs, cu, x, dt, A, B, C, D, bias, init, flags, 1e-3,
                    0.5, 0, NULL, y, fin) == 0, "forward");
  CHECK(finite(y, (size_t)(b * L * H * P)) && finite(fin, (size_t)(S * H * N * P)), "finite forward");
  /* two (sequence, head) streams only */
  const int64_t pairs[4] = {S - 1, H - 1, 0, 0};
  CHECK(ssd_ref_fwd(b, L, H, P, N, G, Gc, nseqs, cu, x, dt, A, B, C, NULL, NULL, init, flags, 0.0,
                    1e30, 2, pairs, y, NULL) == 0, "forward on pairs");
  double* dx = dbl((size_t)(b * L * H * P));
  double* ddt = dbl((size_t)(b * L * H));
  double* dA = dbl((size_t)H);
  double* dB = dbl((size_t)(b * L * G * N));
  double* dC = dbl((size_t)(b * L * Gc * N));
  double* dD = dbl((size_t)H);
  double* dbias = dbl((size_t)H);
  double* dinit = dbl((size_t)(S * H * N * P));
  CHECK(ssd_ref_bwd(b, L, H, P, N, G, Gc, nseqs, cu, x, dt, A, B, C, D, bias, init, flags, 1e-3,
                    0.5, dy, dfin, dx, ddt, dA, dB, dC, dD, dbias, with_init ? dinit : NULL) == 0,
        "backward");
  CHECK(finite(dx, (size_t)(b * L * H * P)) && finite(dB, (size_t)(b * L * G * N)) &&
            finite(dC, (size_t)(b * L * Gc * N)) && finite(ddt, (size_t)(b * L * H)),
        "finite backward");
  free(x), free(dt), free(A), free(B), free(C), free(D), free(bias), free(init), free(dy);
  free(dfin), free(y), free(fin), free(dx), free(ddt), free(dA), free(dB), free(dC), free(dD);
  free(dbias), free(dinit);
}

int main(void) {
  /* dense rows: groups for B and C, initial states, softplus and input scaling */
  run(2, 37, 4, 3, 5, 2, 1, 0, NULL, 1, 1u);
  run(3, 1, 2, 1, 1, 1, 2, 0, NULL, 0, 3u);
  run(1, 0, 2, 4, 4, 1, 1, 0, NULL, 1, 1u); /* no tokens */
  /* packed sequences with empty ones and a one-token one */
  const int32_t cu[6] = {0, 0, 5, 6, 20, 20};
  run(1, 20, 4, 2, 3, 2, 4, 5, cu, 1, 1u);
  run(1, 20, 2, 2, 3, 1, 1, 5, cu, 0, 2u);
  /* inconsistent arguments are refused */
  float one = 1.0f;
  double out[64];
  const int32_t bad_end[3] = {0, 3, 7};
  const int32_t bad_order[3] = {0, 5, 3};
  const int64_t bad_pair[2] = {4, 0};
  CHECK(ssd_ref_fwd(1, 8, 3, 1, 1, 2, 1, 0, NULL, &one, &one, &one, &one, &one, NULL, NULL, NULL,
                    0, 0.0, 1.0, 0, NULL, out, NULL) == -1, "H % G refused");
  CHECK(ssd_ref_fwd(1, 8, 1, 1, 1, 1, 1, 2, bad_end, &one, &one, &one, &one, &one, NULL, NULL,
                    NULL, 0, 0.0, 1.0, 0, NULL, out, NULL) == -1, "cu_seqlens end refused");
  CHECK(ssd_ref_fwd(1, 3, 1, 1, 1, 1, 1, 2, bad_order, &one, &one, &one, &one, &one, NULL, NULL,
                    NULL, 0, 0.0, 1.0, 0, NULL, out, NULL) == -1, "decreasing cu_seqlens refused");
  CHECK(ssd_ref_fwd(2, 1, 1, 1, 1, 1, 1, 0, NULL, &one, &one, &one, &one, &one, NULL, NULL, NULL,
                    0, 0.0, 1.0, 1, bad_pair, out, NULL) == -1, "pair out of range refused");
  CHECK(ssd_ref_fwd(-1, 1, 1, 1, 1, 1, 1, 0, NULL, &one, &one, &one, &one, &one, NULL, NULL, NULL,
                    0, 0.0, 1.0, 0, NULL, out, NULL) == -1, "negative batch refused");
  if (failures == 0) printf("oracle checks passed\n");
  return failures != 0;
}
