/*
 * kda_oracle.h -- plain fp64 CPU oracle for Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may call this.  The GPU library never
 * includes this header and this code never includes the GPU library's.
 *
 * What is computed, per (batch b, head h), token by token (the pages outline
 * KDA as short convolutions, L2-normalised q/k and gated delta-rule state
 * updates -- "Kimi K3, previewed", section "Kimi Delta Attention - the
 * workhorse"; "Gemma 4 31B vs Kimi K3", component table, rows
 * "Gated DeltaNet / KDA" and "Output gate + sink"):
 *
 *   1. causal depthwise conv, kernel 4, over the raw q, k, v channels,
 *      tap 3 on the current token, history from conv_in (zeros if absent)
 *   2. SiLU  x / (1 + e^-x)
 *   3. q^ = q~ (sum q~^2 + 1e-6)^-1/2 dk^-1/2 ;  k^ = k~ (sum k~^2 + 1e-6)^-1/2
 *   4. S <- diag(exp g_t) S                       (per-channel decay, g <= 0)
 *      With decay_form KDAO_DECAY_K3 the inputs g and beta hold logits z and
 *      b instead: g = -5 sigmoid(e^A z) (K3's bounded log-decay, "Kimi K3.1
 *      Pro vs gpt-oss-120b" and "Gemma 4 31B vs Kimi K3", component tables,
 *      row "Gated DeltaNet / KDA"; A per head and key channel) and
 *      beta = sigmoid(b).
 *   5. y = S^T k^ ;  S <- S + beta_t k^ (v^ - y)^T   (delta rule)
 *   6. o_core = S^T q^                             (post-update state)
 *   7. o = o_core / sqrt(mean(o_core^2) + 1e-5) * sigmoid(gate)
 *
 * Everything is fp64 from the exact input values (bf16 and f32 convert to
 * fp64 exactly).  No chunking, no cumulative sums, no reordering.
 *
 * Channel packing of conv_w / conv history (Cch = H(2dk+dv) channels):
 *   q channel c of head h : h*dk + c
 *   k channel c of head h : H*dk + h*dk + c
 *   v channel c of head h : 2*H*dk + h*dv + c
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { KDAO_F32 = 0, KDAO_BF16 = 1 };
enum { KDAO_DECAY_DIRECT = 0, KDAO_DECAY_K3 = 1 };

typedef struct {
  int B, T, H, dk, dv;
  int in_dtype;          /* KDAO_F32 or KDAO_BF16 (bf16 passed as raw uint16 bits) */
  const void* q;         /* [B,T,H,dk] */
  const void* k;         /* [B,T,H,dk] */
  const void* v;         /* [B,T,H,dv] */
  const float* conv_w;   /* [H(2dk+dv), 4] fp32, tap 3 = current token */
  const void* g;         /* [B,T,H,dk] log-decay, g <= 0 */
  const void* beta;      /* [B,T,H] */
  const void* gate;      /* [B,T,H,dv] */
  int decay_form;        /* KDAO_DECAY_DIRECT: g, beta as given; KDAO_DECAY_K3: logits (step 4) */
  const float* A;        /* [H,dk] fp32, KDAO_DECAY_K3 only */
} kdao_inputs;

/*
 * Prefill over the (b,h) pairs listed in bh[0..n_bh) (bh[i] = b*H + h).
 * Per listed pair i (all arrays fp64, compact per pair):
 *   S_inout  [n_bh, dk, dv]   in: initial state, out: final state
 *   hist     [n_bh, 3, 2dk+dv] in: raw conv history (row 0 oldest), out: last 3 raw tokens
 *   o        [n_bh, T, dv]    output (NULL allowed)
 *   prep     [n_bh, T, 2dk+dv] the normalised q^, k^, v^ (NULL allowed)
 * Returns 0, or -1 on bad arguments.
 */
int kdao_prefill(const kdao_inputs* in, const int32_t* bh, int n_bh,
                 double* S_inout, double* hist, double* o, double* prep,
                 int nthreads);

/* Threads an OpenMP region would use by default (1 without OpenMP). */
int kdao_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
