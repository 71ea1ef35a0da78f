/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library, libkda.so.
 *
 * KDA is the gated delta-rule linear attention of Kimi K3 ("Kimi K3,
 * previewed", section "Kimi Delta Attention - the workhorse"; component tables
 * of "Kimi K3.1 Pro vs gpt-oss-120b" and "Gemma 4 31B vs Kimi K3", row
 * "Gated DeltaNet / KDA"; output gate from "Gemma 4 31B vs Kimi K3", row
 * "Output gate + sink").  Per (batch b, head h), per token t:
 *
 *   x~ = SiLU(causal depthwise conv, kernel 4, of the raw q, k, v channels)
 *   q  = q~ (|q~|^2 + 1e-6)^-1/2 dk^-1/2 ;  k = k~ (|k~|^2 + 1e-6)^-1/2 ;  v = v~
 *   S_t = (I - beta_t k k^T) Diag(exp g_t) S_{t-1} + beta_t k v^T     (S: dk x dv)
 *   o_t = RMSNorm(S_t^T q) * sigmoid(gate_t),  RMSNorm(x) = x / sqrt(mean(x^2) + 1e-5)
 *
 * Layouts (all row-major, contiguous, no padding):
 *   q, k, g      [B, T, H, dk]        v, gate, o  [B, T, H, dv]      beta [B, T, H]
 *   S0, S_T      [B, H, dk, dv] fp32  (row index = key channel)
 *   conv_w       [H*(2dk+dv), 4] fp32, tap 3 multiplies the current token
 *   conv_in/out  [B, 3, H*(2dk+dv)]   raw (pre-conv) tokens, row 0 the oldest
 *   Conv channel order: q channels (head-major), then k, then v:
 *     q ch c of head h -> h*dk + c;  k -> H*dk + h*dk + c;  v -> 2*H*dk + h*dv + c
 *
 * Dtypes: activations (q, k, v, g, beta, gate, conv history) are all KDA_F32 or
 * all KDA_BF16 (in_dtype); o is KDA_F32 or KDA_BF16 (out_dtype); state and
 * conv_w are always fp32.
 *
 * Ownership: the caller owns every buffer (device memory).  The library keeps
 * no device allocations; inputs are never written.  Long prefill and backward
 * calls fork onto compute-unit-restricted streams (default priority) that the
 * library creates on first use, keeps for later calls, and destroys in
 * kda_release() or, failing that, at process exit, before the HIP runtime
 * tears itself down.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream);
 * execution faults surface at the caller's next synchronisation.  A call that
 * fails validation returns a negative code and launches nothing.  The library
 * is reentrant; kda_last_error() is per calling thread.
 *
 * Decay and beta inputs (decay_form):
 *   KDA_DECAY_DIRECT  g is the log-decay (g <= 0) and beta is beta in [0, 1].
 *   KDA_DECAY_K3      g holds the decay logits z and beta the beta logits b:
 *                     g = -5 sigmoid(e^A z) with A [H, dk] fp32 (one value per
 *                     head and key channel), beta = sigmoid(b).  K3's bounded
 *                     log-decay ("Kimi K3.1 Pro vs gpt-oss-120b" and "Gemma 4
 *                     31B vs Kimi K3", component tables, row "Gated DeltaNet /
 *                     KDA"; the pages give A's shape nowhere, and beta's form
 *                     only as a value in (0, 1)), computed in the kernels where
 *                     they load g and beta.
 *
 * Preconditions not checked (for cost): g <= 0 and 0 <= beta <= 1 in the
 * direct form; inputs finite; on the single-kernel path (no workspace, or
 * sizes without the two-kernel path) |v~| and the state below 6e4 (fp16
 * operand range) -- the two-kernel path scales each 32-column group of V, the
 * state and the outputs by a power of two chosen per chunk from the raw v
 * values and S0, so any finite bf16 v and fp32 S0 stay in range there; the
 * summed log-decay of any 16 consecutive tokens of a chunk at
 * least -80 per channel (g >= -5 per token suffices, which K3's bounded decay
 * g = -5 sigmoid(.) guarantees: the pages' 16-token tile bound), so that the
 * in-tile decay factors stay finite in fp32.
 * Precision: the prefill's matrix-core operands are fp16 with fp32
 * accumulation and an fp32 state.  Decay factors inside a 16-token tile are
 * formed relative to a per-tile reference.  A chunk in which some tile's
 * summed log-decay in some channel is below -8 ("wide") computes its in-tile
 * blocks with fp32 operands and passes U to its state and output products as
 * a pair of fp16 parts (about 22 significant bits).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 8

/* element types */
enum { KDA_F32 = 0, KDA_BF16 = 1 };

/* how g and beta are given (see above) */
enum { KDA_DECAY_DIRECT = 0, KDA_DECAY_K3 = 1 };

/* status codes */
enum {
  KDA_OK = 0,
  KDA_E_NULL = -1,        /* a required pointer is NULL                          */
  KDA_E_SHAPE = -2,       /* a size is out of range (negative, zero, too large)  */
  KDA_E_DTYPE = -3,       /* in_dtype / out_dtype not one of the enum values     */
  KDA_E_ALIGN = -4,       /* a pointer is not 16-byte aligned                    */
  KDA_E_UNSUPPORTED = -5, /* dk != dv, dk not in {16,32,64,128}, chunk not in {16,32,64},
                             or decay_form not one of the enum values */
  KDA_E_WORKSPACE = -6,   /* workspace given but smaller than kda_prefill_workspace_min_bytes */
  KDA_E_HIP = -7          /* a HIP runtime call failed (text in kda_last_error)  */
};

/*
 * Chunkwise prefill (the definition above over t = 0..T-1 for every (b, h)).
 * Starts from S0 (NULL = zeros) and the raw conv history conv_in (NULL =
 * zeros); writes o for every token, the final state S_T and the last three raw
 * tokens conv_out (taken from conv_in where T < 3).  S_T may alias S0 and
 * conv_out may alias conv_in, so a long sequence can be processed as
 * consecutive segments carrying both in place.  T = 0 is allowed (copies the
 * carry).  T need not be a multiple of `chunk`.
 *
 * Two execution paths, same results within the stated tolerance:
 *  - workspace != NULL (kda_prefill_workspace_bytes, or at least
 *    kda_prefill_workspace_min_bytes): for bf16 inputs
 *    with chunk 64 and dk = dv = 128 the work runs as two kernels, one over
 *    all chunks of all heads at once (prep and intra-chunk products) and one
 *    per (b, h) walking the chunks (state recurrence and output), which meet
 *    in the workspace.  For other sizes the workspace is unused.
 *  - workspace == NULL: one kernel per (b, h) walks the chunks and keeps every
 *    intermediate on chip (no device memory beyond the arguments).
 * With a workspace, a sequence of more than 64 chunks with 2*B*H at most the
 * device's compute units runs as a pipeline of slabs of up to 64 chunks: the
 * per-(b, h) kernel runs on a stream restricted to B*H (rounded up to 8)
 * compute units while the all-chunks kernels of the slabs run on two streams
 * restricted to the others.  When every slab has a workspace region of its
 * own (the size kda_prefill_workspace_bytes returns), S_T is given and
 * `stream` is not capturing a graph, the per-(b, h) kernel is one launch over
 * all slabs that waits on a device flag per slab, set by a one-wave kernel
 * queued after the slab's all-chunks kernel.  A wait is bounded (20 ms): a
 * workgroup whose wait expires (the all-chunks kernels could not run beside
 * it, e.g. kernels serialised by a profiler collecting counters) stops, leaves
 * its state in S_T, and a second launch queued after every slab finishes its
 * chunks, so the results do not depend on the timing (kda_wait_timeouts
 * counts such stops).  Otherwise the per-(b, h) kernel is launched once per
 * slab, after a stream event, and the slabs go through up to three buffers in
 * turn.  While `stream` is capturing a graph, nothing is forked: the slabs run
 * one after the other on `stream` (as in kda_prefill_noalloc).
 * The library creates these three streams (default priority) and their
 * events once per host thread, device and B*H, keeps them for the life of
 * the thread, starts them after the work already queued on `stream` and
 * makes `stream` wait for all three before any later work.
 * The library owns no device memory: the caller allocates the workspace and
 * may reuse it once the call's work on `stream` has finished.
 */
typedef struct kda_prefill_args {
  int B, T, H, dk, dv;
  int chunk;              /* tokens per chunk: 16, 32 or 64 */
  int in_dtype;           /* KDA_F32 or KDA_BF16 */
  int out_dtype;          /* KDA_F32 or KDA_BF16 */
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  const float* S0;        /* may be NULL */
  const void* conv_in;    /* may be NULL */
  void* o;
  float* S_T;             /* may be NULL */
  void* conv_out;         /* may be NULL */
  void* workspace;        /* NULL, or >= kda_prefill_workspace_min_bytes bytes, 16-byte aligned */
  size_t workspace_bytes;
  int decay_form;         /* KDA_DECAY_DIRECT (0) or KDA_DECAY_K3 */
  const float* A;         /* [H, dk] fp32 for KDA_DECAY_K3 (required, 16-byte aligned); else unused */
} kda_prefill_args;

int kda_prefill(const kda_prefill_args* args, void* stream);

/* Device workspace the two-kernel path prefers for these sizes: 64 KiB per
 * (b, h, chunk of 64 tokens) of one slab; for a pipelined sequence (more than
 * 64 chunks, 2*B*H <= 256) one region of 64 chunks per slab while all of them
 * fit 16 GiB (6.4 GB at K3 width for 65,536 tokens), else three such buffers
 * used in turn, plus B*H*dk*dv*4 bytes to carry the state; otherwise all chunks in one slab,
 * capped near 16 GiB (plus the carry) by running longer sequences in slabs
 * one after the other.  0 when the sizes have no two-kernel path or the
 * arguments are invalid.  The fields B, T, H, dk, dv, chunk, in_dtype and
 * out_dtype are read; pointers are not. */
size_t kda_prefill_workspace_bytes(const kda_prefill_args* args);

/* Smallest workspace the two-kernel path accepts (one chunk per slab): any size
 * from this up to kda_prefill_workspace_bytes works, a smaller one in more
 * slabs.  A non-NULL workspace below it is rejected with KDA_E_WORKSPACE. */
size_t kda_prefill_workspace_min_bytes(const kda_prefill_args* args);

/*
 * One decode step for N sequences of one new token each: the definition above
 * with T = 1, updating the state S [N,H,dk,dv] (fp32) and the raw conv history
 * conv_state [N,3,Cch] (in_dtype) in place, and writing o [N,H,dv].
 * Inputs q, k, g [N,H,dk]; v, gate [N,H,dv]; beta [N,H].
 */
typedef struct kda_decode_args {
  int N, H, dk, dv;
  int in_dtype;
  int out_dtype;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  float* S;               /* in/out */
  void* conv_state;       /* in/out */
  void* o;
  int decay_form;         /* as in kda_prefill_args */
  const float* A;         /* as in kda_prefill_args */
} kda_decode_args;

int kda_decode_step(const kda_decode_args* args, void* stream);

/*
 * M consecutive tokens per sequence in one call (1 <= M <= KDA_MAX_DECODE_TOKENS),
 * for speculative decoding: drafted tokens are verified in one pass (the pages
 * name MTP self-drafting and an EAGLE-3 drafter for K3: "Kimi K3.1 Pro vs
 * gpt-oss-120b" and "Gemma 4 31B vs Kimi K3", component tables, rows "Speculative
 * decoding" and "MTP layer turned EAGLE-3 drafter").
 *
 * Inputs are [N, M, H, .] (token t of sequence n at row n*M + t): q, k [N,M,H,dk],
 * v, gate, o [N,M,H,dv], g [N,M,H,dk], beta [N,M,H].  o is written for all M
 * tokens, each from the state after the tokens before it -- exactly a prefill
 * of the M tokens from (S, conv_state).  S and conv_state are then replaced by
 * the state and raw history after the first accept[n] tokens of sequence n
 * (accept: int32 [N] in device memory, values clamped to [0, M]; NULL means M;
 * 0 leaves both unchanged).  Typical use: one call with accept[n] = 0 to verify
 * (outputs only), then one with the accepted counts to commit.
 * The state is read and written once per call, whatever M is.
 * Errors as kda_decode_step; M outside [1, KDA_MAX_DECODE_TOKENS] is
 * KDA_E_SHAPE; accept must be 4-byte aligned (KDA_E_ALIGN).
 */
#define KDA_MAX_DECODE_TOKENS 16
typedef struct kda_decode_multi_args {
  int N, M, H, dk, dv;
  int in_dtype;
  int out_dtype;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  float* S;               /* in/out */
  void* conv_state;       /* in/out */
  void* o;
  const int32_t* accept;  /* [N] device, or NULL (all M tokens) */
  int decay_form;         /* as in kda_prefill_args */
  const float* A;         /* as in kda_prefill_args */
} kda_decode_multi_args;

int kda_decode_multi(const kda_decode_multi_args* args, void* stream);

/*
 * The first stage of the prefill on its own: conv + SiLU + L2 normalisation
 * (q scaled by dk^-1/2) and the chunk-local inclusive cumulative sum of g.
 * Writes fp32 q^, k^ [B,T,H,dk], v^ [B,T,H,dv] and G [B,T,H,dk], where
 * G restarts at every multiple of `chunk`.  Same inputs and validation as
 * kda_prefill (o, S0, S_T, conv_out, gate, beta unused and may be NULL).
 */
typedef struct kda_prep_args {
  int B, T, H, dk, dv;
  int chunk;
  int in_dtype;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* conv_in;    /* may be NULL */
  float* q_out;
  float* k_out;
  float* v_out;
  float* G_out;
  int decay_form;         /* as in kda_prefill_args (G sums the g it implies) */
  const float* A;
} kda_prep_args;

int kda_prep(const kda_prep_args* args, void* stream);

/*
 * Context-parallel prefill.  The long-context training row of "Gemma 4 31B vs
 * Kimi K3" (component table) says that ranks exchange only fixed-size state
 * fragments.  The update above is affine in the state, so a segment of tokens
 * maps the state S entering it to M S + N (M: dk x dk, N: dk x dv), whatever S
 * is.  With dk = dv, two prefills
 * of a segment give both: from S = 0 its final state is N, from S = I it is
 * P = M + N.  Each rank forms (N, P) for its segment, the ranks exchange them
 * (dk*(dk+dv)*4 bytes per head each), each composes the state entering its own
 * segment, and runs its segment again from that state for the outputs.
 *
 * kda_cp_compose: the composition, for every (b, h):
 *   S_start[b*R]         = S0[b]                          (zeros if S0 is NULL)
 *   S_start[b*R + r + 1] = (P[b*R + r] - N[b*R + r]) S_start[b*R + r] + N[b*R + r]
 *   S_T[b]               = the same map applied after the last segment r = R - 1
 * N, P, S_start: [B*R, H, d, d] fp32 (the R segments of sequence b consecutive,
 * as in a prefill batch of B*R segments); S0, S_T: [B, H, d, d] fp32, may be
 * NULL; S_T may alias S0.  S_start must not overlap N, P or S0.  d in {16, 32,
 * 64, 128}; all pointers 16-byte aligned.  Errors: KDA_E_NULL (N, P or
 * S_start NULL), KDA_E_SHAPE (B, R or H < 1, or too large), KDA_E_UNSUPPORTED
 * (d), KDA_E_ALIGN.
 */
typedef struct kda_cp_compose_args {
  int B, R, H, d;
  const float* N;         /* [B*R, H, d, d] final states from S = 0 */
  const float* P;         /* [B*R, H, d, d] final states from S = I */
  const float* S0;        /* [B, H, d, d] state entering segment 0, or NULL */
  float* S_start;         /* [B*R, H, d, d] out: state entering each segment */
  float* S_T;             /* [B, H, d, d] out: state after the last segment, or NULL */
} kda_cp_compose_args;

int kda_cp_compose(const kda_cp_compose_args* args, void* stream);

/*
 * kda_prefill_cp: the whole context-parallel prefill on one device, the R
 * segments of each sequence standing in for R ranks.  Same arguments and
 * results as kda_prefill (o, S_T, conv_out; S_T may alias S0 and conv_out
 * conv_in), computed as
 *   1. the raw conv history of every segment: the three raw tokens before it
 *      (from conv_in, or zeros, before the first);
 *   2. all B*R segments as one prefill batch from S = 0, then from S = I
 *      (their outputs o are overwritten by step 4);
 *   3. kda_cp_compose of the two final-state batches, from S0;
 *   4. all B*R segments again from their entering states: o, and the last
 *      segment's final state as S_T; conv_out from the last three raw tokens.
 * Requires T a multiple of `segments` with at least 3 tokens per segment (T = 0
 * is passed to kda_prefill), dk = dv.  Every step runs on `stream` in the
 * caller's workspace (kda_prefill_cp_workspace_bytes, 16-byte aligned): the
 * segment histories, the N / P / entering-state batches and the segment
 * prefills' own workspace.  The workspace fields inside `prefill` are ignored.
 * Errors: those of kda_prefill, KDA_E_SHAPE (segments < 1, T not a multiple,
 * fewer than 3 tokens per segment), KDA_E_NULL (no workspace),
 * KDA_E_WORKSPACE (workspace too small).
 */
typedef struct kda_prefill_cp_args {
  kda_prefill_args prefill;  /* the whole sequences, as for kda_prefill */
  int segments;              /* R >= 1 segments per sequence */
  void* workspace;
  size_t workspace_bytes;
} kda_prefill_cp_args;

int kda_prefill_cp(const kda_prefill_cp_args* args, void* stream);

/* Workspace kda_prefill_cp needs for these sizes (fields B, T, H, dk, dv,
 * chunk, in_dtype, out_dtype and segments are read); 0 if they are invalid. */
size_t kda_prefill_cp_workspace_bytes(const kda_prefill_cp_args* args);

/*
 * One rank's share of context-parallel prefill, in two calls around the
 * exchange of fragments (the long-context training row of "Gemma 4 31B vs
 * Kimi K3", component table: ranks exchange only fixed-size state fragments).
 * `args` describes the rank's own segment as a kda_prefill call: its tokens,
 * conv_in = the three raw tokens before the segment (the previous rank's last
 * ones; NULL = zeros at the sequence start), and a workspace of at least
 * kda_cp_rank_workspace_bytes bytes (16-byte aligned, required) that the
 * caller leaves untouched between the two calls.
 *   kda_cp_fragments(args, N, P): N = the segment's final state from S = 0,
 *     P = from S = I ([B, H, dk, dv] fp32 each, caller-owned, 16-byte
 *     aligned); args->S0, S_T and conv_out are ignored.  With bf16 inputs,
 *     chunk 64 and dk = dv = 128 the intra-chunk work of every chunk runs once
 *     into the workspace and the two recurrences run side by side without
 *     forming outputs; other sizes run two plain prefills (args->o is then
 *     used as scratch).
 *   (exchange the fragments; kda_cp_compose gives the entering state)
 *   kda_cp_finish(args): the segment from the entering state args->S0 with
 *     the same inputs and workspace: o, S_T and conv_out as kda_prefill.  On
 *     the two-kernel path it reruns only the recurrence over the kept chunk
 *     blocks.
 * Calls are asynchronous on `stream`; both must be ordered on one stream (or
 * synchronised) with the workspace untouched between them.  Errors as
 * kda_prefill; KDA_E_NULL (N, P or the workspace NULL), KDA_E_WORKSPACE.
 */
int kda_cp_fragments(const kda_prefill_args* args, float* N, float* P, void* stream);
int kda_cp_finish(const kda_prefill_args* args, void* stream);

/* Workspace of kda_cp_fragments / kda_cp_finish for these sizes: with the
 * two-kernel path (bf16, chunk 64, dk = dv = 128) 64 KiB per (b, h, chunk of
 * 64 tokens), B*H*ceil(T/64)*65536 bytes; otherwise B*H*dk*dv*4 bytes rounded
 * up to 256.  0 when the sizes are invalid.  Pointers are not read. */
size_t kda_cp_rank_workspace_bytes(const kda_prefill_args* args);

/*
 * kda_prefill_backward: gradients of the prefill for training (the long
 * contexts of "Gemma 4 31B vs Kimi K3", component table, long-context training
 * row), for the loss <grad_o, o> + <grad_S_T, S_T> + <grad_conv_out, conv_out>
 * of kda_prefill with the same inputs: grad_q, grad_k, grad_v, grad_g,
 * grad_beta, grad_gate (fp32, the layouts of q, k, v, g, beta, gate), grad_S0
 * [B,H,dk,dv] and grad_conv_in [B,3,Cch] (fp32, each may be NULL).  A long
 * sequence run as carried segments is differentiated segment by segment, the
 * last first: a segment's grad_S0 and grad_conv_in are the grad_S_T and
 * grad_conv_out of the segment before it (its S0 and conv_in being that
 * segment's S_T and conv_out from the forward pass).
 * Gradients are with respect to the input values (bf16 inputs: their bf16
 * values).  Direct decay form only (decay_form KDA_DECAY_DIRECT), dk = dv.
 * Computed in fp32: the forward again, chunkwise with fp32 matrix-core
 * operands (one workgroup per (b, h)), with the state stored every 32 tokens
 * in the workspace; then, for slabs of up to 32 such stretches (1,024 tokens)
 * from the last to the first, every stretch of the slab recomputed at once,
 * and the slab walked back token by token (one
 * workgroup per (b, h)); the next slab's recompute runs on the other compute
 * units meanwhile (streams of the library's own, ordered after the work
 * already on `stream`, which in turn waits for them; while `stream` is
 * capturing a graph, everything runs on `stream`).  Workspace
 * (kda_prefill_backward_workspace_bytes, 16-byte aligned, required), with
 * n = ceil(T/32):
 * B*H*(n*dk*dv + dk*dv + 9*dk + 2*min(n, 32)*32*(dk*dv + 13*dk + 8))*4 bytes.
 * Errors as kda_prefill; KDA_E_NULL (grad_o, a required gradient output or the
 * workspace NULL), KDA_E_UNSUPPORTED (KDA_DECAY_K3), KDA_E_WORKSPACE.
 */
typedef struct kda_prefill_backward_args {
  int B, T, H, dk, dv;
  int in_dtype;           /* KDA_F32 or KDA_BF16 (q, k, v, g, beta, gate, conv_in) */
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  const float* S0;        /* may be NULL */
  const void* conv_in;    /* may be NULL */
  const float* grad_o;    /* dL/do [B,T,H,dv] fp32 */
  const float* grad_S_T;  /* dL/dS_T [B,H,dk,dv] fp32, or NULL (no loss on S_T) */
  const float* grad_conv_out;  /* dL/dconv_out [B,3,Cch] fp32 (conv_out: the last three raw
                                  tokens, as kda_prefill writes them), or NULL */
  float* grad_q;
  float* grad_k;
  float* grad_v;
  float* grad_g;
  float* grad_beta;
  float* grad_gate;
  float* grad_S0;         /* may be NULL */
  float* grad_conv_in;    /* may be NULL */
  void* workspace;
  size_t workspace_bytes;
  int decay_form;         /* KDA_DECAY_DIRECT */
  const float* A;         /* unused */
} kda_prefill_backward_args;

int kda_prefill_backward(const kda_prefill_backward_args* args, void* stream);

/* Workspace kda_prefill_backward needs (fields B, T, H, dk, dv, in_dtype read);
 * 0 if they are invalid. */
size_t kda_prefill_backward_workspace_bytes(const kda_prefill_backward_args* args);

/* Static text of a status code. */
const char* kda_status_string(int code);

/* Detail of the last failure on the calling thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

/* Bounded in-kernel waits that expired on the current device since the
 * library was loaded: the per-slab flags of a pipelined kda_prefill (see
 * there) whose producer had not run within the bound.  Each one stopped a
 * workgroup whose remaining chunks the call's second launch then ran (slower,
 * same results).  Waits for the device's work to finish.  Returns KDA_OK,
 * KDA_E_NULL or KDA_E_HIP. */
int kda_wait_timeouts(unsigned* count);

/* Test aid for that stop-and-resume path, for later kda_prefill calls from any
 * thread: wait_limit_us replaces the 20 ms bound (0 restores it), and
 * withhold_slab >= 0 makes the calls skip setting that slab's flag, so every
 * workgroup's wait for it expires and the second launch finishes the work
 * (-1: none).  (0, -1) restores normal operation.  Returns KDA_OK, or
 * KDA_E_SHAPE for withhold_slab < -1. */
int kda_debug_pipeline(unsigned wait_limit_us, int withhold_slab);

/* kda_prefill for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments and results as kda_prefill; args->workspace and workspace_bytes
 * are ignored.  Where kda_prefill would take its two-kernel path (bf16
 * inputs, chunk 64, dk = dv = 128) the workspace is instead a device array of
 * KDA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; its slabs run one after the other on `stream` (no
 * streams are created).  Other shapes take the single-kernel path, which
 * needs no workspace.  The call makes no hipMalloc / hipFree or other
 * allocating call.  Limit: B*H * (64 KiB + 64 KiB) must fit the scratch, i.e.
 * at most 1024 heads (B*H) for sequences longer than one chunk; beyond that it
 * returns KDA_E_WORKSPACE and launches nothing.  Every call on one GPU uses
 * the same scratch: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int kda_prefill_noalloc(const kda_prefill_args* args, void* stream);

/* Destroy the streams and events the library keeps between calls (the
 * compute-unit-restricted streams of pipelined prefill and backward calls),
 * on every device and for every host thread; later calls create them again.
 * Call it with no library call in flight (it waits for those streams first).
 * The library also does this at process exit, before the HIP runtime's own
 * teardown (streams still alive then have crashed profiled runs at exit).
 * Returns KDA_OK, or KDA_E_HIP (text in kda_last_error) if a destroy failed. */
int kda_release(void);

#ifdef __cplusplus
}
#endif
#endif
