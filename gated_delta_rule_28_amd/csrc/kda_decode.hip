// kda_decode.hip -- batched one-token KDA decode step for gfx950.
//
// One workgroup per (sequence n, head h).  The step is the recurrence of the
// KDA definition at T = 1 (pages: "Kimi K3, previewed", section "Kimi Delta
// Attention - the workhorse"; "Gemma 4 31B vs Kimi K3", component table, rows
// "Gated DeltaNet / KDA" and "Output gate + sink"):
//   conv step over the 3-token raw history, SiLU, L2 norms (q also dk^-1/2),
//   S' = diag(e^g) S,  y = S'^T k,  u = beta (v - y),  S <- S' + k u^T,
//   o = RMSNorm(S'^T q + (k.q) u) * sigmoid(gate).
// The state is the only large operand (dk*dv fp32 per head, 64 KiB at 128x128),
// so the kernel reads it once and writes it once: each thread keeps its rows
// of S in registers between the read-out reduction and the update, and
// S'^T k and S'^T q are formed in the same pass.  Loads and stores of S are
// 16-byte, nontemporal and coalesced along dv.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

struct DecodeParams {
  int H;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  float* S;
  void* conv_state;
  void* o;
  const float* A;  // [H, dk]: g and beta are K3's logits (see k3_decay); null: given directly
};

constexpr int kDecodeThreads = 256;

template <int DK, int DV, bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeParams p) {
  constexpr int NC = 2 * DK + DV;          // q | k | v channels of one head
  constexpr int CG = DV / 4;               // float4 column groups of the state
  constexpr int RG0 = kDecodeThreads / CG;
  constexpr int RG = RG0 < DK ? RG0 : DK;  // row groups
  constexpr int RPT = DK / RG;             // state rows per thread

  const int tid = threadIdx.x;
  const int nh = blockIdx.x;               // n * H + h
  const int H = p.H;
  const int n = nh / H;
  const int h = nh - n * H;
  const size_t cch = (size_t)H * NC;

  __shared__ float xs[NC];                 // conv + SiLU of q | k | v
  __shared__ float aq[DK];                 // e^g * q^
  __shared__ float ak[DK];                 // e^g * k^
  __shared__ float kn[DK];                 // k^
  __shared__ float alpha[DK];              // e^g
  __shared__ float red[2][RG][DV];         // partial S'^T k and S'^T q
  __shared__ float us[DV];                 // u
  __shared__ float ocs[DV];                // o_core
  __shared__ float scal[4];

  // This thread's conv channels (c = tid, tid + 256) are requested first, then
  // the state block, which is the step's traffic: the state's loads are in
  // flight while the conv step and the norms run, and the conv inputs, being
  // older, are waited for without waiting for the state.  Every load here is
  // unconditional from a clamped, in-bounds address (a load under a branch
  // makes the wait after the branch a wait for everything in flight); which
  // values are real is decided at use.
  constexpr int NCH = (NC + kDecodeThreads - 1) / kDecodeThreads;
  float xr[NCH], hr[NCH][3];
  float4 wr[NCH];
  size_t chr[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = min(tid + kDecodeThreads * j, NC - 1);
    size_t ch;
    const void* src;
    size_t idx;
    if (c < DK) {
      ch = (size_t)h * DK + c;
      src = p.q;
      idx = (size_t)nh * DK + c;
    } else if (c < 2 * DK) {
      ch = (size_t)H * DK + (size_t)h * DK + (c - DK);
      src = p.k;
      idx = (size_t)nh * DK + (c - DK);
    } else {
      ch = (size_t)2 * H * DK + (size_t)h * DV + (c - 2 * DK);
      src = p.v;
      idx = (size_t)nh * DV + (c - 2 * DK);
    }
    xr[j] = load1<IN_BF16>(src, idx);
    chr[j] = ch;
    const size_t r0 = (size_t)n * 3 * cch + ch;
#pragma unroll
    for (int r = 0; r < 3; ++r) hr[j][r] = load1<IN_BF16>(p.conv_state, r0 + r * cch);
    wr[j] = *reinterpret_cast<const float4*>(p.conv_w + ch * 4);
  }
  // the per-channel decay (and K3's A), beta and gate: also requested before the state
  const int tk = min(tid, DK - 1), tv = min(tid, DV - 1);
  const float g_raw = load1<IN_BF16>(p.g, (size_t)nh * DK + tk);
  const float a_log = (p.A != nullptr ? p.A : p.conv_w)[(size_t)h * DK + tk];  // used only with p.A
  const float beta_raw = load1<IN_BF16>(p.beta, (size_t)nh);
  const float gate_raw = load1<IN_BF16>(p.gate, (size_t)nh * DV + tv);
  const int cg = tid % CG;
  const int rg = tid / CG;
  // every thread holds state rows when the row groups fit (no branch around
  // the loads then, so the conv inputs can be waited for on their own)
  constexpr bool kAllActive = kDecodeThreads / CG <= DK;
  const bool active = kAllActive || rg < RG;
  f4* Sp = reinterpret_cast<f4*>(p.S + (size_t)nh * DK * DV);
  f4 s[RPT];
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      s[i] = __builtin_nontemporal_load(Sp + (size_t)(rg + RG * i) * CG + cg);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the conv work after the state requests

  // 1. conv step on the raw history + SiLU; shift the history in place.
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = tid + kDecodeThreads * j;
    if (c < NC) {
      const float4 w = wr[j];
      const float acc = w.x * hr[j][0] + w.y * hr[j][1] + w.z * hr[j][2] + w.w * xr[j];
      xs[c] = siluf_(acc);
    }
  }
  __syncthreads();

  // 2. |q~|^2, |k~|^2 and q~.k~ in wave 0.
  if (tid < 64) {
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    for (int c = tid; c < DK; c += 64) {
      const float a = xs[c], b = xs[DK + c];
      sq += a * a;
      sk += b * b;
      sqk += a * b;
    }
    sq = group_sum<64>(sq);
    sk = group_sum<64>(sk);
    sqk = group_sum<64>(sqk);
    if (tid == 0) {
      const float rq = fast_rsq(sq + kL2Eps) * fast_rsq((float)DK);
      const float rk = fast_rsq(sk + kL2Eps);
      scal[0] = rq;
      scal[1] = rk;
      scal[2] = sqk * rq * rk;  // k^ . q^
    }
  }
  __syncthreads();
  if (tid < DK) {
    float gv = g_raw;
    if (p.A != nullptr) gv = k3_decay(gv, fast_exp(a_log));
    const float a = fast_exp(gv);
    const float kq = xs[DK + tid] * scal[1];
    alpha[tid] = a;
    kn[tid] = kq;
    ak[tid] = a * kq;
    aq[tid] = a * xs[tid] * scal[0];
  }
  __syncthreads();

  // 3. one pass over S (requested at the start): keep this thread's rows,
  // accumulate S'^T k and S'^T q.
  if (active) {
    f4 y = f4{0.f, 0.f, 0.f, 0.f}, z = y;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      y += s[i] * ak[r];
      z += s[i] * aq[r];
    }
    *reinterpret_cast<f4*>(&red[0][rg][4 * cg]) = y;
    *reinterpret_cast<f4*>(&red[1][rg][4 * cg]) = z;
  }
  __syncthreads();

  // 4. u = beta (v - y); o_core = z + (k.q) u; mean square of o_core.
  if (tid < DV) {
    float y = 0.f, z = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      y += red[0][r][tid];
      z += red[1][r][tid];
    }
    float beta = beta_raw;
    if (p.A != nullptr) beta = sigmoidf_(beta);
    const float u = beta * (xs[2 * DK + tid] - y);
    us[tid] = u;
    ocs[tid] = z + scal[2] * u;
  }
  __syncthreads();
  if (tid < 64) {
    float ss = 0.f;
    for (int j = tid; j < DV; j += 64) ss += ocs[j] * ocs[j];
    ss = group_sum<64>(ss);
    if (tid == 0) scal[3] = fast_rsq(ss * (1.0f / DV) + kRmsEps);
  }
  __syncthreads();

  // 5. S <- S' + k u^T, written once.
  if (active) {
    const f4 u = *reinterpret_cast<const f4*>(&us[4 * cg]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      const f4 t = s[i] * alpha[r] + u * kn[r];
      __builtin_nontemporal_store(t, Sp + (size_t)r * CG + cg);
    }
  }
  if (tid < DV) store1<OUT_BF16>(p.o, (size_t)nh * DV + tid, ocs[tid] * scal[3] * sigmoidf_(gate_raw));
  // The conv history shifted by one token, stored last: a store issued earlier
  // would make the state's loads be waited for at once (loads and stores share
  // one counter).  The shifted values are exact in the history dtype (they came
  // from it or from the input, which has the same dtype).
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    if (tid + kDecodeThreads * j < NC) {
      const size_t r0 = (size_t)n * 3 * cch + chr[j];
      store1<IN_BF16>(p.conv_state, r0, hr[j][1]);
      store1<IN_BF16>(p.conv_state, r0 + cch, hr[j][2]);
      store1<IN_BF16>(p.conv_state, r0 + 2 * cch, xr[j]);
    }
  }
}

// ---------------------------------------------------------------------------
// decode_multi_kernel: M consecutive tokens per sequence (speculative decoding:
// verify M drafted tokens in one pass), one workgroup per (n, h).  The same
// recurrence as M calls of decode_kernel, but the state is read once, kept in
// registers for the M tokens and written once, after token accept[n] - 1 (not
// at all when accept[n] = 0): its traffic is that of one step.  The conv
// history is replaced by the last three raw tokens of the accepted prefix.
// ---------------------------------------------------------------------------
struct DecodeMultiParams {
  int H, M;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  float* S;
  void* conv_state;
  void* o;
  const int32_t* accept;  // [N] tokens whose updates are kept, or null (all M)
  const float* A;         // [H, dk]: g and beta are K3's logits; null: given directly
};

// MT: tokens the LDS arrays hold (M <= MT); a smaller MT for short drafts
// leaves room for more workgroups per compute unit.
// LANE_SUM: how the threads share the state in the token loop.
//   false  thread (cg = tid % CG, rg = tid / CG) holds rows rg + RG i of column
//          group cg.  A wave's state accesses are 512-byte row pieces; the
//          read-outs S'^T k^ and S'^T q^ are summed over row groups through
//          LDS, three barriers per token.
//   true   thread (rg = tid % RG, cg = tid / RG): the RG threads of a column
//          group are consecutive lanes of one wave, so the read-outs are lane
//          sums and the token loop has no barrier; the state accesses become
//          128-byte row pieces, and the outputs are normalised after the loop.
//          Fewer instructions per token, worse memory access: the better
//          choice for long drafts.
template <int DK, int DV, bool IN_BF16, bool OUT_BF16, int MT, bool LANE_SUM>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(LANE_SUM ? 4 : 1)))
void decode_multi_kernel(DecodeMultiParams p) {
  constexpr int NC = 2 * DK + DV;
  constexpr int CG = DV / 4;
  constexpr int RG0 = kDecodeThreads / CG;
  constexpr int RG = RG0 < DK ? RG0 : DK;
  constexpr int RPT = DK / RG;
  // LDS of the row-group reduction and of one token's u and o_core; unused
  // with LANE_SUM, where o_core replaces v^ in xs
  constexpr int RED = LANE_SUM ? 1 : RG;
  constexpr int RDV = LANE_SUM ? 1 : DV;

  const int tid = threadIdx.x;
  const int nh = blockIdx.x;
  const int H = p.H, M = p.M;
  const int n = nh / H;
  const int h = nh - n * H;
  const size_t cch = (size_t)H * NC;
  const int acc_n = p.accept != nullptr ? min(max(p.accept[n], 0), M) : M;

  __shared__ float xs[MT][NC];             // conv + SiLU, then q^ | k^ | v^
  __shared__ float alpha[MT][DK];          // e^g
  __shared__ float betas[MT];
  __shared__ float scal[MT][3];            // q scale, k scale, k^ . q^
  __shared__ float red[2][RED][RDV];
  __shared__ float us[RDV];
  __shared__ float ocs[RDV];
  __shared__ float rs_s;

  // row of token t of this (n, h) in the [N, M, H, .] inputs
  auto tok = [&](int t) { return ((size_t)n * M + t) * H + h; };

  // 1. conv + SiLU of every token; the new raw history is the accepted
  //    prefix's last three tokens (from the old history where it is shorter)
  for (int c = tid; c < NC; c += kDecodeThreads) {
    size_t ch;
    const void* src;
    int D, cc;
    if (c < DK) {
      ch = (size_t)h * DK + c; src = p.q; D = DK; cc = c;
    } else if (c < 2 * DK) {
      ch = (size_t)H * DK + (size_t)h * DK + (c - DK); src = p.k; D = DK; cc = c - DK;
    } else {
      ch = (size_t)2 * H * DK + (size_t)h * DV + (c - 2 * DK); src = p.v; D = DV; cc = c - 2 * DK;
    }
    const size_t r0 = ((size_t)n * 3 + 0) * cch + ch;
    const float h0 = load1<IN_BF16>(p.conv_state, r0);
    const float h1 = load1<IN_BF16>(p.conv_state, r0 + cch);
    const float h2 = load1<IN_BF16>(p.conv_state, r0 + 2 * cch);
    const float4 w = *reinterpret_cast<const float4*>(p.conv_w + ch * 4);
    // new history rows R(a-3), R(a-2), R(a-1), with R(i) = history row 3 + i for i < 0
    float n0 = acc_n == 0 ? h0 : acc_n == 1 ? h1 : h2;
    float n1 = acc_n == 0 ? h1 : h2;
    float n2 = h2;
    float xm3 = h0, xm2 = h1, xm1 = h2;
    for (int t = 0; t < M; ++t) {
      const float x = load1<IN_BF16>(src, tok(t) * D + cc);
      xs[t][c] = siluf_(w.x * xm3 + w.y * xm2 + w.z * xm1 + w.w * x);
      xm3 = xm2; xm2 = xm1; xm1 = x;
      if (t == acc_n - 3) n0 = x;
      if (t == acc_n - 2) n1 = x;
      if (t == acc_n - 1) n2 = x;
    }
    // exact in the history dtype: every value came from it or from the input
    if (acc_n > 0) {
      store1<IN_BF16>(p.conv_state, r0, n0);
      store1<IN_BF16>(p.conv_state, r0 + cch, n1);
      store1<IN_BF16>(p.conv_state, r0 + 2 * cch, n2);
    }
  }
  // decay factors and beta of every token
  for (int idx = tid; idx < M * DK; idx += kDecodeThreads) {
    const int t = idx / DK, c = idx - t * DK;
    float gv = load1<IN_BF16>(p.g, tok(t) * DK + c);
    if (p.A != nullptr) gv = k3_decay(gv, fast_exp(p.A[(size_t)h * DK + c]));
    alpha[t][c] = fast_exp(gv);
  }
  if (tid < M) {
    float b = load1<IN_BF16>(p.beta, tok(tid));
    if (p.A != nullptr) b = sigmoidf_(b);
    betas[tid] = b;
  }
  __syncthreads();

  // 2. L2 norms of q and k per token, one wave per token
  {
    const int wv = tid >> 6, ln = tid & 63;
    for (int t = wv; t < M; t += kDecodeThreads / 64) {
      float sq = 0.f, sk = 0.f, sqk = 0.f;
      for (int c = ln; c < DK; c += 64) {
        const float a = xs[t][c], b = xs[t][DK + c];
        sq += a * a;
        sk += b * b;
        sqk += a * b;
      }
      sq = group_sum<64>(sq);
      sk = group_sum<64>(sk);
      sqk = group_sum<64>(sqk);
      if (ln == 0) {
        const float rq = fast_rsq(sq + kL2Eps) * fast_rsq((float)DK);
        const float rk = fast_rsq(sk + kL2Eps);
        scal[t][0] = rq;
        scal[t][1] = rk;
        scal[t][2] = sqk * rq * rk;
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < M * 2 * DK; idx += kDecodeThreads) {
    const int t = idx / (2 * DK), c = idx - t * 2 * DK;
    xs[t][c] *= c < DK ? scal[t][0] : scal[t][1];
  }
  __syncthreads();

  // 3. the tokens in order, the state in registers
  const int cg = LANE_SUM ? tid / RG : tid % CG;
  const int rg = LANE_SUM ? tid % RG : tid / CG;
  const bool active = LANE_SUM ? cg < CG : rg < RG;
  f4* Sp = reinterpret_cast<f4*>(p.S + (size_t)nh * DK * DV);
  f4 s[RPT];
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(Sp + (size_t)(rg + RG * i) * CG + cg);
  }
  if constexpr (LANE_SUM) {
    if (active) {
      auto step = [&](int t) {
        // S' = diag(e^g) S;  S'^T k^ and S'^T q^ as sums over the RG lanes
        f4 y = f4{0.f, 0.f, 0.f, 0.f}, z = y;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + RG * i;
          s[i] *= alpha[t][r];
          y += s[i] * xs[t][DK + r];
          z += s[i] * xs[t][r];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = group_sum<RG>(y[e]);
          z[e] = group_sum<RG>(z[e]);
        }
        // u = beta (v^ - y);  S <- S' + k^ u^T;  o_core = S'^T q^ + (k^ . q^) u
        const f4 u = betas[t] * (*reinterpret_cast<const f4*>(&xs[t][2 * DK + 4 * cg]) - y);
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] += u * xs[t][DK + rg + RG * i];
        // o_core over v^ of this column group: only this wave's lanes read it,
        // and they have (LDS accesses of a wave complete in order)
        if (rg == 0) *reinterpret_cast<f4*>(&xs[t][2 * DK + 4 * cg]) = z + scal[t][2] * u;
      };
      // the accepted prefix, its state to memory, then the rest of the tokens
      // (their outputs only).  Storing between the two loops keeps the store
      // addresses out of the registers the loops hold.
      for (int t = 0; t < acc_n; ++t) step(t);
      if (acc_n > 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(s[i], Sp + (size_t)(rg + RG * i) * CG + cg);
      }
      for (int t = acc_n; t < M; ++t) step(t);
    }
    __syncthreads();
    // RMSNorm * sigmoid(gate) of every token, one wave per token
    const int wv = tid >> 6, ln = tid & 63;
    for (int t = wv; t < M; t += kDecodeThreads / 64) {
      float ss = 0.f;
      const float* oc = &xs[t][2 * DK];
      for (int j = ln; j < DV; j += 64) ss += oc[j] * oc[j];
      const float rs = fast_rsq(group_sum<64>(ss) * (1.0f / DV) + kRmsEps);
      for (int j = ln; j < DV; j += 64) {
        const float gt = load1<IN_BF16>(p.gate, tok(t) * DV + j);
        store1<OUT_BF16>(p.o, tok(t) * DV + j, oc[j] * rs * sigmoidf_(gt));
      }
    }
  } else {
    auto step = [&](int t, bool store) {
      // S' = diag(e^g) S;  S'^T k^ and S'^T q^
      if (active) {
        f4 y = f4{0.f, 0.f, 0.f, 0.f}, z = y;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + RG * i;
          s[i] *= alpha[t][r];
          y += s[i] * xs[t][DK + r];
          z += s[i] * xs[t][r];
        }
        *reinterpret_cast<f4*>(&red[0][rg][4 * cg]) = y;
        *reinterpret_cast<f4*>(&red[1][rg][4 * cg]) = z;
      }
      __syncthreads();
      // u = beta (v^ - y);  o_core = S'^T q^ + (k^ . q^) u
      if (tid < DV) {
        float y = 0.f, z = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          y += red[0][r][tid];
          z += red[1][r][tid];
        }
        const float u = betas[t] * (xs[t][2 * DK + tid] - y);
        us[tid] = u;
        ocs[tid] = z + scal[t][2] * u;
      }
      __syncthreads();
      // S <- S' + k^ u^T; after the accepted prefix, the state goes to memory
      if (active) {
        const f4 u = *reinterpret_cast<const f4*>(&us[4 * cg]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] += u * xs[t][DK + rg + RG * i];
        if (store) {
#pragma unroll
          for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(s[i], Sp + (size_t)(rg + RG * i) * CG + cg);
        }
      }
      if (tid < 64) {
        float ss = 0.f;
        for (int j = tid; j < DV; j += 64) ss += ocs[j] * ocs[j];
        ss = group_sum<64>(ss);
        if (tid == 0) rs_s = fast_rsq(ss * (1.0f / DV) + kRmsEps);
      }
      __syncthreads();
      if (tid < DV) {
        const float gt = load1<IN_BF16>(p.gate, tok(t) * DV + tid);
        store1<OUT_BF16>(p.o, tok(t) * DV + tid, ocs[tid] * rs_s * sigmoidf_(gt));
      }
    };
    if constexpr (MT <= 2) {
      // one or two tokens: one loop, the store under a condition (faster here,
      // measured, though it holds the store addresses through the loop)
      for (int t = 0; t < M; ++t) step(t, t == acc_n - 1);
    } else {
      // as above, with the last accepted token's step on its own: its state
      // stores are issued before its output is normalised
      for (int t = 0; t < acc_n - 1; ++t) step(t, false);
      if (acc_n > 0) step(acc_n - 1, true);
      for (int t = acc_n; t < M; ++t) step(t, false);
    }
  }
}

template <int DK, int DV, bool IB, bool OB>
int run_multi(const kda_decode_multi_args& a, hipStream_t s) {
  DecodeMultiParams p{a.H, a.M, a.q, a.k, a.v, a.conv_w, a.g, a.beta, a.gate, a.S, a.conv_state, a.o,
                      a.accept, a.decay_form == KDA_DECAY_K3 ? a.A : nullptr};
  const unsigned grid = (unsigned)((size_t)a.N * a.H);
  if (a.M <= 2)
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, IB, OB, 2, false>), dim3(grid), dim3(kDecodeThreads), 0, s, p);
  else if (a.M <= 4)
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, IB, OB, 4, false>), dim3(grid), dim3(kDecodeThreads), 0, s, p);
  else if (a.M <= 8)
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, IB, OB, 8, false>), dim3(grid), dim3(kDecodeThreads), 0, s, p);
  else
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, IB, OB, KDA_MAX_DECODE_TOKENS, true>), dim3(grid),
                       dim3(kDecodeThreads), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("multi-token decode launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

template <int DK, int DV>
int run_multi_dt(const kda_decode_multi_args& a, hipStream_t s) {
  const bool ib = a.in_dtype == KDA_BF16, ob = a.out_dtype == KDA_BF16;
  if (ib && ob) return run_multi<DK, DV, true, true>(a, s);
  if (ib) return run_multi<DK, DV, true, false>(a, s);
  if (ob) return run_multi<DK, DV, false, true>(a, s);
  return run_multi<DK, DV, false, false>(a, s);
}

template <int DK, int DV, bool IB, bool OB>
int run(const kda_decode_args& a, hipStream_t s) {
  DecodeParams p{a.H, a.q, a.k, a.v, a.conv_w, a.g, a.beta, a.gate, a.S, a.conv_state, a.o,
                 a.decay_form == KDA_DECAY_K3 ? a.A : nullptr};
  const unsigned grid = (unsigned)((size_t)a.N * a.H);
  hipLaunchKernelGGL((decode_kernel<DK, DV, IB, OB>), dim3(grid), dim3(kDecodeThreads), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("decode launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

template <int DK, int DV>
int run_dt(const kda_decode_args& a, hipStream_t s) {
  const bool ib = a.in_dtype == KDA_BF16, ob = a.out_dtype == KDA_BF16;
  if (ib && ob) return run<DK, DV, true, true>(a, s);
  if (ib) return run<DK, DV, true, false>(a, s);
  if (ob) return run<DK, DV, false, true>(a, s);
  return run<DK, DV, false, false>(a, s);
}

}  // namespace

int launch_decode_multi(const kda_decode_multi_args& a, hipStream_t s) {
  switch (a.dk) {
    case 16: return run_multi_dt<16, 16>(a, s);
    case 32: return run_multi_dt<32, 32>(a, s);
    case 64: return run_multi_dt<64, 64>(a, s);
    case 128: return run_multi_dt<128, 128>(a, s);
    default:
      set_error("multi-token decode: head dim %d not in {16,32,64,128}", a.dk);
      return KDA_E_UNSUPPORTED;
  }
}

int launch_decode(const kda_decode_args& a, hipStream_t s) {
  if (a.dk != a.dv) {
    set_error("decode: dk (%d) != dv (%d) is not instantiated", a.dk, a.dv);
    return KDA_E_UNSUPPORTED;
  }
  switch (a.dk) {
    case 16: return run_dt<16, 16>(a, s);
    case 32: return run_dt<32, 32>(a, s);
    case 64: return run_dt<64, 64>(a, s);
    case 128: return run_dt<128, 128>(a, s);
    default:
      set_error("decode: head dim %d not in {16,32,64,128}", a.dk);
      return KDA_E_UNSUPPORTED;
  }
}

}  // namespace kda
