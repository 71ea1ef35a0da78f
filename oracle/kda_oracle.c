/*
 * kda_oracle.c -- plain fp64 token-by-token KDA recurrence (test infrastructure).
 *
 * Definition followed (pages: "Kimi K3, previewed", section "Kimi Delta
 * Attention - the workhorse"; "Kimi K3.1 Pro vs gpt-oss-120b" and
 * "Gemma 4 31B vs Kimi K3", component tables, row "Gated DeltaNet / KDA";
 * "Gemma 4 31B vs Kimi K3", row "Output gate + sink"; the RMSNorm epsilon is
 * the model's rms_norm_eps from the "Kimi K3" model card's config table):
 * see kda_oracle.h for the seven steps.  This file restates them as loops in
 * the order of the definition; nothing is blocked, fused or reordered.
 *
 * Decode is the same routine with T = 1 and the state / history carried by
 * the caller.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static const double L2_EPS = 1e-6;   /* L2 normalisation epsilon */
static const double RMS_EPS = 1e-5;  /* rms_norm_eps of the model config */

static double bf16_to_f64(uint16_t u) {
  uint32_t w = (uint32_t)u << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* element i of an input tensor stored as f32 or bf16 bits */
static double load(const void* p, int dtype, size_t i) {
  if (dtype == KDAO_BF16) return bf16_to_f64(((const uint16_t*)p)[i]);
  return (double)((const float*)p)[i];
}

static double silu(double x) { return x / (1.0 + exp(-x)); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* K3's bounded log-decay of a decay logit z in a channel with parameter A */
static double k3_log_decay(double z, double A) { return -5.0 * sigmoid(exp(A) * z); }

/* One (b,h) pair over all T tokens.  S: dk*dv (row = key channel),
 * hist: 3 rows of nc = 2dk+dv raw values (row 0 oldest). */
static void run_head(const kdao_inputs* in, int b, int h, double* S, double* hist,
                     double* o, double* prep, double* work) {
  const int T = in->T, H = in->H, dk = in->dk, dv = in->dv;
  const int nc = 2 * dk + dv;
  double* x = work;           /* raw current token, nc        */
  double* xt = x + nc;        /* conv + SiLU, nc              */
  double* y = xt + nc;        /* S^T k, dv                    */
  double* oc = y + dv;        /* o_core, dv                   */
  double* qh = xt;            /* views into xt after normalising */
  double* kh = xt + dk;
  double* vh = xt + 2 * dk;

  for (int t = 0; t < T; ++t) {
    const size_t tok = (size_t)b * T + t;         /* row of [B,T,...] */
    const size_t base_qk = (tok * H + h) * (size_t)dk;
    const size_t base_v = (tok * H + h) * (size_t)dv;
    for (int c = 0; c < dk; ++c) x[c] = load(in->q, in->in_dtype, base_qk + c);
    for (int c = 0; c < dk; ++c) x[dk + c] = load(in->k, in->in_dtype, base_qk + c);
    for (int c = 0; c < dv; ++c) x[2 * dk + c] = load(in->v, in->in_dtype, base_v + c);

    /* 1-2: causal depthwise conv (kernel 4) then SiLU */
    for (int c = 0; c < nc; ++c) {
      size_t ch;
      if (c < dk) ch = (size_t)h * dk + c;
      else if (c < 2 * dk) ch = (size_t)H * dk + (size_t)h * dk + (c - dk);
      else ch = (size_t)2 * H * dk + (size_t)h * dv + (c - 2 * dk);
      const float* w = in->conv_w + ch * 4;
      double acc = (double)w[0] * hist[0 * nc + c] + (double)w[1] * hist[1 * nc + c] +
                   (double)w[2] * hist[2 * nc + c] + (double)w[3] * x[c];
      xt[c] = silu(acc);
    }
    /* shift the raw history: oldest drops out, current token enters */
    for (int c = 0; c < nc; ++c) {
      hist[0 * nc + c] = hist[1 * nc + c];
      hist[1 * nc + c] = hist[2 * nc + c];
      hist[2 * nc + c] = x[c];
    }

    /* 3: L2 normalisation of q and k, 1/sqrt(dk) on q */
    double sq = 0.0, sk = 0.0;
    for (int c = 0; c < dk; ++c) { sq += qh[c] * qh[c]; sk += kh[c] * kh[c]; }
    const double rq = 1.0 / sqrt(sq + L2_EPS) / sqrt((double)dk);
    const double rk = 1.0 / sqrt(sk + L2_EPS);
    for (int c = 0; c < dk; ++c) { qh[c] *= rq; kh[c] *= rk; }
    if (prep) memcpy(prep + (size_t)t * nc, xt, sizeof(double) * nc);

    /* 4: per-channel decay of the state rows */
    const size_t base_g = base_qk;
    for (int i = 0; i < dk; ++i) {
      double gi = load(in->g, in->in_dtype, base_g + i);
      if (in->decay_form == KDAO_DECAY_K3) gi = k3_log_decay(gi, (double)in->A[(size_t)h * dk + i]);
      const double a = exp(gi);
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
    }
    /* 5: delta rule  y = S^T k ; S += beta k (v - y)^T */
    double beta = load(in->beta, in->in_dtype, tok * H + h);
    if (in->decay_form == KDAO_DECAY_K3) beta = sigmoid(beta);
    for (int j = 0; j < dv; ++j) y[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) y[j] += S[(size_t)i * dv + j] * kh[i];
    for (int i = 0; i < dk; ++i) {
      const double bk = beta * kh[i];
      for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += bk * (vh[j] - y[j]);
    }
    /* 6: read-out with the updated state */
    for (int j = 0; j < dv; ++j) oc[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) oc[j] += S[(size_t)i * dv + j] * qh[i];
    /* 7: head-wise RMSNorm (no gain) times sigmoid(gate) */
    if (o) {
      double ms = 0.0;
      for (int j = 0; j < dv; ++j) ms += oc[j] * oc[j];
      ms /= (double)dv;
      const double r = 1.0 / sqrt(ms + RMS_EPS);
      for (int j = 0; j < dv; ++j)
        o[(size_t)t * dv + j] = oc[j] * r * sigmoid(load(in->gate, in->in_dtype, base_v + j));
    }
  }
}

int kdao_prefill(const kdao_inputs* in, const int32_t* bh, int n_bh, double* S_inout,
                 double* hist, double* o, double* prep, int nthreads) {
  if (!in || !bh || n_bh < 0 || !S_inout || !hist) return -1;
  if (in->B < 1 || in->T < 0 || in->H < 1 || in->dk < 1 || in->dv < 1) return -1;
  if (!in->q || !in->k || !in->v || !in->conv_w || !in->g || !in->beta || !in->gate) return -1;
  if (in->in_dtype != KDAO_F32 && in->in_dtype != KDAO_BF16) return -1;
  if (in->decay_form != KDAO_DECAY_DIRECT && in->decay_form != KDAO_DECAY_K3) return -1;
  if (in->decay_form == KDAO_DECAY_K3 && !in->A) return -1;
  for (int i = 0; i < n_bh; ++i)
    if (bh[i] < 0 || bh[i] >= in->B * in->H) return -1;
  const int dk = in->dk, dv = in->dv, nc = 2 * dk + dv, T = in->T;
  int err = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (int i = 0; i < n_bh; ++i) {
    double* work = (double*)malloc(sizeof(double) * (2 * nc + 2 * dv));
    if (!work) { err = 1; continue; }
    run_head(in, bh[i] / in->H, bh[i] % in->H, S_inout + (size_t)i * dk * dv,
             hist + (size_t)i * 3 * nc, o ? o + (size_t)i * T * dv : NULL,
             prep ? prep + (size_t)i * T * nc : NULL, work);
    free(work);
  }
  (void)nthreads;
  return err ? -1 : 0;
}

/* number of OpenMP threads a parallel region would use (for reporting) */
int kdao_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
