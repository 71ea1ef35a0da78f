/* Host-side driver for the sanitizer build of the C oracle (kda_oracle.c built
 * with AddressSanitizer and UndefinedBehaviorSanitizer): kdao_prefill on small
 * fp32 and bf16 inputs, both decay forms, dk != dv, head subsets, T = 0 and a
 * ragged length, one and two threads, and its argument checks.  Exit status 0
 * when every run succeeds with finite outputs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* uniform in (-1, 1), xorshift64* */
  g_state ^= g_state >> 12; g_state ^= g_state << 25; g_state ^= g_state >> 27;
  return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static uint16_t to_bf16(float x) { uint32_t u; memcpy(&u, &x, 4); return (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16); }

static void* fill(size_t n, int bf16, double lo, double hi) {
  if (bf16) {
    uint16_t* p = (uint16_t*)malloc(n * 2 + 2);
    for (size_t i = 0; i < n; ++i) p[i] = to_bf16((float)(lo + (hi - lo) * 0.5 * (urand() + 1.0)));
    return p;
  }
  float* p = (float*)malloc(n * 4 + 4);
  for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * 0.5 * (urand() + 1.0));
  return p;
}

static int run(int B, int T, int H, int dk, int dv, int bf16, int k3, int nsel, int nthreads) {
  const size_t BT = (size_t)B * (T > 0 ? T : 1) * H;
  kdao_inputs in;
  memset(&in, 0, sizeof in);
  in.B = B; in.T = T; in.H = H; in.dk = dk; in.dv = dv; in.in_dtype = bf16 ? KDAO_BF16 : KDAO_F32;
  in.q = fill(BT * dk, bf16, -2, 2);
  in.k = fill(BT * dk, bf16, -2, 2);
  in.v = fill(BT * dv, bf16, -2, 2);
  in.conv_w = (const float*)fill((size_t)H * (2 * dk + dv) * 4, 0, -0.5, 0.5);
  in.g = fill(BT * dk, bf16, k3 ? -4 : -0.5, k3 ? 6 : 0);
  in.beta = fill(BT, bf16, k3 ? -2 : 0, k3 ? 2 : 1);
  in.gate = fill(BT * dv, bf16, -2, 2);
  in.decay_form = k3 ? KDAO_DECAY_K3 : KDAO_DECAY_DIRECT;
  in.A = k3 ? (const float*)fill((size_t)H * dk, 0, -0.2, 0.2) : NULL;
  int32_t bh[64];
  for (int i = 0; i < nsel; ++i) bh[i] = (i * 7) % (B * H);
  const int nc = 2 * dk + dv;
  double* S = (double*)calloc((size_t)nsel * dk * dv, sizeof(double));
  double* hist = (double*)calloc((size_t)nsel * 3 * nc, sizeof(double));
  double* o = (double*)calloc((size_t)nsel * (T > 0 ? T : 1) * dv, sizeof(double));
  double* prep = (double*)calloc((size_t)nsel * (T > 0 ? T : 1) * nc, sizeof(double));
  for (size_t i = 0; i < (size_t)nsel * dk * dv; ++i) S[i] = 0.05 * urand();
  for (size_t i = 0; i < (size_t)nsel * 3 * nc; ++i) hist[i] = urand();
  int rc = kdao_prefill(&in, bh, nsel, S, hist, o, prep, nthreads);
  int bad = rc != 0;
  for (size_t i = 0; i < (size_t)nsel * T * dv && !bad; ++i) bad = !isfinite(o[i]);
  for (size_t i = 0; i < (size_t)nsel * dk * dv && !bad; ++i) bad = !isfinite(S[i]);
  /* argument checks: a pair index out of range and a bad dtype are refused */
  int32_t bad_bh = B * H;
  if (kdao_prefill(&in, &bad_bh, 1, S, hist, o, prep, 1) != -1) bad = 1;
  in.in_dtype = 9;
  if (kdao_prefill(&in, bh, nsel, S, hist, o, prep, 1) != -1) bad = 1;
  free((void*)in.q); free((void*)in.k); free((void*)in.v); free((void*)in.conv_w); free((void*)in.g);
  free((void*)in.beta); free((void*)in.gate); free((void*)in.A);
  free(S); free(hist); free(o); free(prep);
  if (bad) fprintf(stderr, "case B%d T%d H%d dk%d dv%d bf16=%d k3=%d: failed (rc %d)\n", B, T, H, dk, dv, bf16, k3, rc);
  return bad;
}

int main(void) {
  int fails = 0;
  fails += run(1, 37, 2, 16, 16, 0, 0, 2, 1);
  fails += run(2, 70, 3, 16, 24, 1, 0, 4, 2);   /* dk != dv, subset of heads */
  fails += run(1, 20, 2, 32, 32, 1, 1, 2, 1);   /* K3 logits */
  fails += run(1, 0, 2, 16, 16, 0, 0, 2, 1);    /* empty sequence */
  fails += run(1, 2, 1, 16, 16, 1, 0, 1, 1);    /* fewer tokens than the conv history */
  if (fails == 0) printf("oracle driver: all runs passed\n");
  return fails ? 1 : 0;
}
