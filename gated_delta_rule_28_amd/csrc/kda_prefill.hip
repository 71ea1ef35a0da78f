// kda_prefill.hip -- chunkwise KDA prefill for gfx950 (CDNA4).
//
// What is computed is the KDA recurrence (pages: "Kimi K3, previewed", section
// "Kimi Delta Attention - the workhorse"; "Kimi K3.1 Pro vs gpt-oss-120b" and
// "Gemma 4 31B vs Kimi K3", component tables, row "Gated DeltaNet / KDA"; the
// output gate from "Gemma 4 31B vs Kimi K3", row "Output gate + sink").  The
// kernels reach it through the exact chunkwise (WY / UT) rewrite.  Per chunk of
// C tokens entering with state S (dk x dv), G = inclusive cumsum of g in the
// chunk:
//   A_rj = beta_r sum_c k_rc k_jc e^{G_rc - G_jc} (j < r)     T = (I + A)^-1
//   W = T diag(beta) (K * e^G)          U~ = T diag(beta) V
//   U = U~ - W S                        P_rj = sum_c q_rc k_jc e^{G_rc - G_jc} (j <= r)
//   O = (Q * e^G) S + P U               S <- diag(e^{G_C}) S + (K * e^{G_C - G})^T U
//   o = O / sqrt(mean_dv(O^2) + 1e-5) * sigmoid(gate)
//
// Decay-weighted products on the matrix cores use 16-token tiles, as the
// pages describe for K3 ("Gemma 4 31B vs Kimi K3", row "Gated DeltaNet / KDA":
// 16-token-tile rescaling so every intra-chunk tile is a matrix-core product).
// Row tile a takes the reference rho_a = G at the token before the tile
// (0 for the first tile): row factors e^{G_r - rho_a} <= 1, column factors
// e^{rho_a - G_j} <= 1 for earlier tiles and <= e^{span} inside the tile,
// where span is the tile's total decay.  Masked entries are discarded with a
// select, never multiplied by zero.
//
// Precision: matrix-core operands are fp16 (bf16 would put the max error at
// several 1e-2 of RMS; fp16 has the same rate and three more mantissa bits),
// accumulation fp32, state fp32, output fp32 by default.  When some tile's
// span exceeds what fp16 holds at full precision (e^8), that chunk's
// decay-weighted operands are bf16 instead (finite up to e^88, but with
// bf16's 8-bit precision on those products).  fp32 inputs use fp32
// operands on the fp32 matrix-core instruction throughout.
//
// Work decomposition: one workgroup (8 waves) per (b, h) walks the chunks in
// order; the fp32 state stays in VGPRs as matrix-core accumulators, each wave
// owning 16 of the dv columns, and is fed straight back in as a B operand (the
// contraction index is permuted so the accumulator layout is the operand
// layout).  The chunk's prepared operands live in LDS.
//
// Stage 1 (prep) of a chunk is a block-level device function shared with the
// standalone kda_prep kernel: causal depthwise conv (kernel 4, history from
// the previous chunk's raw tokens or conv_in), SiLU, L2 normalisation of q and
// k (q scaled by dk^-1/2), and the chunk-local cumulative sum of g.
#include <type_traits>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kThreads = 512;  // 8 waves
constexpr int kWaves = kThreads / 64;
// Largest decay span of a 16-token tile (per channel, in nats) for which the
// decay-weighted operands stay fp16: column factors reach e^span and row
// factors e^-span, and both must stay in fp16's normal range (6e-5 .. 6.5e4)
// after multiplying a normalised key component.
constexpr float kF16SpanMax = 8.0f;

struct PrefillParams {
  int B, T, H;
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  const float* S0;
  const void* conv_in;
  void* o;
  float* S_T;
  void* conv_out;
  // prep-only outputs
  float* q_out;
  float* k_out;
  float* v_out;
  float* G_out;
};

// ---------------------------------------------------------------------------
// matrix-core fragments: 8 contraction elements per lane (see kda_device.h)
// ---------------------------------------------------------------------------
template <bool F32> struct Frag;
template <> struct Frag<false> { half8 v; };        // fp16 or bf16 bits
template <> struct Frag<true> { float v[8]; };

template <bool F32>
using OpT = typename std::conditional<F32, float, uint16_t>::type;

__device__ __forceinline__ uint16_t to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t to_op16(float x, bool bf) {
  return bf ? f_to_bf16(x) : to_f16_bits(x);
}

template <bool F32>
__device__ __forceinline__ void frag_zero(Frag<F32>& f) {
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = 0.f;
  } else {
    f.v = half8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// Eight fp32 values (k order) -> fragment (fp16 rounding for the fp16 path).
template <bool F32>
__device__ __forceinline__ void frag_from_f(Frag<F32>& f, const float* x) {
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (_Float16)x[e];
  }
}

// Fragment of 8 consecutive contraction elements buf[row*ld + k0 .. k0+7].
template <bool F32>
__device__ __forceinline__ void frag_std(Frag<F32>& f, const OpT<F32>* buf, int row, int ld, int k0,
                                         bool valid) {
  if (!valid) { frag_zero(f); return; }
  const OpT<F32>* p = buf + row * ld + k0;
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  } else {
    f.v = *reinterpret_cast<const half8*>(p);
  }
}

// Fragment in the permuted contraction order used with register-resident B
// operands: elements buf[row*ld + kb + 4g + 0..3] and buf[row*ld + kb + 16 + 4g + 0..3].
template <bool F32>
__device__ __forceinline__ void frag_perm(Frag<F32>& f, const OpT<F32>* buf, int row, int ld, int kb,
                                          int g, bool lo_valid, bool hi_valid) {
  const OpT<F32>* p = buf + row * ld + kb + 4 * g;
  if constexpr (F32) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (lo_valid) a = *reinterpret_cast<const float4*>(p);
    if (hi_valid) b = *reinterpret_cast<const float4*>(p + 16);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  } else {
    half4 a = half4{0, 0, 0, 0}, b = a;
    if (lo_valid) a = *reinterpret_cast<const half4*>(p);
    if (hi_valid) b = *reinterpret_cast<const half4*>(p + 16);
    f.v = half8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
}

// c += A(16x32) * B(32x16) with the lane layout of kda_device.h.
template <bool F32>
__device__ __forceinline__ f4 mma(const Frag<F32>& a, const Frag<F32>& b, f4 c, bool bf = false) {
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
  } else {
    if (bf) return mma_bf16(__builtin_bit_cast(bf16x8, a.v), __builtin_bit_cast(bf16x8, b.v), c);
    return mma_f16(a.v, b.v, c);
  }
}

template <bool F32>
__device__ __forceinline__ void st_op(OpT<F32>* p, float x, bool bf) {
  if constexpr (F32) *p = x;
  else *p = to_op16(x, bf);
}

// 8 consecutive operand elements from 8 fp32 values.
template <bool F32>
__device__ __forceinline__ void st_op8(OpT<F32>* p, const float* x, bool bf) {
  if constexpr (F32) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  } else {
    uint4 u;
    u.x = (uint32_t)to_op16(x[0], bf) | ((uint32_t)to_op16(x[1], bf) << 16);
    u.y = (uint32_t)to_op16(x[2], bf) | ((uint32_t)to_op16(x[3], bf) << 16);
    u.z = (uint32_t)to_op16(x[4], bf) | ((uint32_t)to_op16(x[5], bf) << 16);
    u.w = (uint32_t)to_op16(x[6], bf) | ((uint32_t)to_op16(x[7], bf) << 16);
    *reinterpret_cast<uint4*>(p) = u;
  }
}

// ---------------------------------------------------------------------------
// LDS layout of the fused kernel (byte offsets)
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool F32>
struct Smem {
  static constexpr int E = F32 ? 4 : 2;              // operand element bytes
  static constexpr int NT = C / 16;                  // 16-token tiles per chunk
  static constexpr int NKV = NT * (NT + 1) / 2;      // lower tile pairs
  // region X, phase 1: decay-weighted A/P operands
  static constexpr int QR = 0;                              // [C][DK]
  static constexpr int KR = QR + C * DK * E;                // [C][DK]
  static constexpr int KC = KR + C * DK * E;                // [16*NKV][DK]
  static constexpr int X1 = KC + 16 * NKV * DK * E;
  // region X, phase 2 (after the A/P products)
  static constexpr int AS = 0;                              // [C][C] fp32
  static constexpr int TS = AS + C * C * 4;                 // [C][C] fp32
  static constexpr int TB = TS + C * C * 4;                 // [C][C] op
  static constexpr int PS = TB + C * C * E;                 // [C][C] op
  static constexpr int WS = PS + C * C * E;                 // [C][DK] op
  static constexpr int X2 = WS + C * DK * E;
  static constexpr int XE = X1 > X2 ? X1 : X2;
  // region Y: operands of the W / U~ / inter-chunk products
  static constexpr int QG = (XE + 15) / 16 * 16;            // [C][DK]  q^ e^G
  static constexpr int KGT = QG + C * DK * E;               // [DK][C]  (k^ e^G)^T
  static constexpr int KBT = KGT + DK * C * E;              // [DK][C]  (k^ e^{G_C-G})^T
  static constexpr int VT = KBT + DK * C * E;               // [DV][C]  v^T
  // small fp32 arrays
  static constexpr int BETA = VT + DV * C * E;              // [C]
  static constexpr int GAM = BETA + C * 4;                  // [DK]  e^{G_C}
  static constexpr int GC = GAM + DK * 4;                   // [DK]  G_C
  static constexpr int RHO = GC + DK * 4;                   // [NT][DK]
  static constexpr int ERHO = RHO + NT * DK * 4;            // [NT][DK] e^{rho}
  static constexpr int BTOT = ERHO + NT * DK * 4;           // [8][DK] token-block sums of g
  static constexpr int SSQ = BTOT + 8 * DK * 4;             // [8 waves][C]
  static constexpr int FLAG = SSQ + kWaves * C * 4;         // [4] ints
  static constexpr int BYTES = FLAG + 16;
};

template <int C, int DK, int DV>
struct SmemPrep {  // standalone prep kernel
  static constexpr int BTOT = 0;
  static constexpr int BYTES = 8 * DK * 4;
};

// ---------------------------------------------------------------------------
// Stage 1: conv + SiLU + L2 norm + chunk-local cumsum of g (block-level).
// Thread roles (NC = 2dk + dv items, one per thread):
//   item i <  dk        : q, channel octet i % (dk/8), token block i / (dk/8)
//   dk <= i < 2dk        : k, same mapping
//   2dk <= i < NC        : v, octet (i-2dk) % (dv/8), token block (i-2dk) / (dv/8)
// A token block is C/8 consecutive tokens.  q and k items also hold the
// chunk-local cumsum G for their octet and tokens.  Tokens past n_valid are
// zero (and have g = 0, beta = 0), which makes a ragged last chunk exact.
// Must be called by all threads of the block.
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool IN_BF16>
struct PrepItem {
  static constexpr int TBS = C / 8;
  int role;          // 0 q, 1 k, 2 v, -1 idle
  int oct;           // channel octet within the tensor
  int tb;            // token block
  float x[TBS][8];   // normalised q^ / k^ or v^
  float G[TBS][8];   // chunk-local cumsum (q, k items)
};

template <int C, int DK, int DV, bool IN_BF16>
__device__ __forceinline__ void prep_stage(const PrefillParams& p, int b, int h, int c0, int n_valid,
                                           float* btot, PrepItem<C, DK, DV, IN_BF16>& it) {
  constexpr int TBS = C / 8;
  constexpr int NC = 2 * DK + DV;
  const int tid = threadIdx.x;
  const int T = p.T, H = p.H;
  const size_t cch = (size_t)H * NC;

  int D = DK, base = 0;
  const void* src = p.q;
  size_t chb = 0;
  it.role = -1;
  if (tid < DK) {
    it.role = 0; D = DK; base = 0; src = p.q;
  } else if (tid < 2 * DK) {
    it.role = 1; D = DK; base = DK; src = p.k;
  } else if (tid < NC) {
    it.role = 2; D = DV; base = 2 * DK; src = p.v;
  }
  if (it.role >= 0) {
    const int j = tid - base;
    it.oct = j % (D / 8);
    it.tb = j / (D / 8);
    const int c8 = 8 * it.oct;
    if (it.role == 0) chb = (size_t)h * DK + c8;
    else if (it.role == 1) chb = (size_t)H * DK + (size_t)h * DK + c8;
    else chb = (size_t)2 * H * DK + (size_t)h * DV + c8;

    // conv taps of the octet
    float w[8][4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 t = *reinterpret_cast<const float4*>(p.conv_w + (chb + e) * 4);
      w[e][0] = t.x; w[e][1] = t.y; w[e][2] = t.z; w[e][3] = t.w;
    }
    // sliding window over the raw tokens tau0-3 .. tau0+TBS-1 (chunk-relative)
    const int tau0 = it.tb * TBS;
    float win[4][8];
#pragma unroll
    for (int u = 0; u < TBS + 3; ++u) {
      const int t = c0 + tau0 - 3 + u;  // absolute token
      float* cur = win[u & 3];
      if (t >= 0 && t < T) {
        load8<IN_BF16>(src, ((size_t)b * T + t) * H * D + (size_t)h * D + c8, cur);
      } else if (t < 0 && p.conv_in != nullptr) {
        load8<IN_BF16>(p.conv_in, ((size_t)b * 3 + (3 + t)) * cch + chb, cur);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) cur[e] = 0.f;
      }
      if (u >= 3) {
        const int tt = u - 3;
        const bool ok = tau0 + tt < n_valid;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = w[e][0] * win[(u - 3) & 3][e] + w[e][1] * win[(u - 2) & 3][e] +
                          w[e][2] * win[(u - 1) & 3][e] + w[e][3] * win[u & 3][e];
          it.x[tt][e] = ok ? siluf_(a) : 0.f;
        }
      }
    }
    if (it.role < 2) {
      // L2 normalisation over the dk channels of each token (dk/8 lanes)
      const float extra = it.role == 0 ? fast_rsq((float)DK) : 1.0f;
#pragma unroll
      for (int tt = 0; tt < TBS; ++tt) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += it.x[tt][e] * it.x[tt][e];
        ss = group_sum<DK / 8>(ss);
        const float r = fast_rsq(ss + kL2Eps) * extra;
#pragma unroll
        for (int e = 0; e < 8; ++e) it.x[tt][e] *= r;
      }
      // local cumsum of g over the token block
      float run[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
      for (int tt = 0; tt < TBS; ++tt) {
        const int t = c0 + tau0 + tt;
        float gv[8];
        if (tau0 + tt < n_valid) {
          load8<IN_BF16>(p.g, ((size_t)b * T + t) * H * DK + (size_t)h * DK + c8, gv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gv[e] = 0.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          run[e] += gv[e];
          it.G[tt][e] = run[e];
        }
      }
      if (it.role == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) btot[it.tb * DK + c8 + e] = run[e];
      }
    }
  }
  __syncthreads();
  if (it.role == 0 || it.role == 1) {
    const int c8 = 8 * it.oct;
    float pre[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pre[e] = 0.f;
    for (int q = 0; q < it.tb; ++q) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pre[e] += btot[q * DK + c8 + e];
    }
#pragma unroll
    for (int tt = 0; tt < TBS; ++tt)
#pragma unroll
      for (int e = 0; e < 8; ++e) it.G[tt][e] += pre[e];
  }
}

// ---------------------------------------------------------------------------
// standalone stage-1 kernel: one block per (b, h, chunk)
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrefillParams p) {
  constexpr int TBS = C / 8;
  __shared__ float btot[8 * DK];
  const int nchunks = (p.T + C - 1) / C;
  const int bh = blockIdx.x / nchunks;
  const int ci = blockIdx.x - bh * nchunks;
  const int b = bh / p.H, h = bh - b * p.H;
  const int c0 = ci * C;
  const int n_valid = min(C, p.T - c0);
  PrepItem<C, DK, DV, IN_BF16> it;
  prep_stage<C, DK, DV, IN_BF16>(p, b, h, c0, n_valid, btot, it);
  if (it.role < 0) return;
  const int D = it.role == 2 ? DV : DK;
  float* dst = it.role == 0 ? p.q_out : it.role == 1 ? p.k_out : p.v_out;
  const int c8 = 8 * it.oct;
  for (int tt = 0; tt < TBS; ++tt) {
    const int tau = it.tb * TBS + tt;
    if (tau >= n_valid) break;
    const size_t row = ((size_t)b * p.T + c0 + tau) * p.H + h;
    float* o = dst + row * D + c8;
    *reinterpret_cast<float4*>(o) = make_float4(it.x[tt][0], it.x[tt][1], it.x[tt][2], it.x[tt][3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(it.x[tt][4], it.x[tt][5], it.x[tt][6], it.x[tt][7]);
    if (it.role == 0) {
      float* go = p.G_out + row * DK + c8;
      *reinterpret_cast<float4*>(go) = make_float4(it.G[tt][0], it.G[tt][1], it.G[tt][2], it.G[tt][3]);
      *reinterpret_cast<float4*>(go + 4) = make_float4(it.G[tt][4], it.G[tt][5], it.G[tt][6], it.G[tt][7]);
    }
  }
}

// ---------------------------------------------------------------------------
// fused chunkwise prefill: one block per (b, h)
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool IN_BF16, bool OUT_BF16, bool F32>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  using L = Smem<C, DK, DV, F32>;
  using Op = OpT<F32>;
  constexpr int NT = C / 16;
  constexpr int NKV = L::NKV;
  constexpr int TBS = C / 8;
  constexpr int NC = 2 * DK + DV;
  constexpr int KSD = (DK + 31) / 32;   // 32-wide contraction steps over dk
  constexpr int KSC = (C + 31) / 32;    // ... over the tokens of a chunk
  constexpr int RTK = DK / 16;          // 16-row tiles of the state
  constexpr int CTV = DV / 16;          // 16-column tiles of dv (one per wave)
  static_assert(CTV <= kWaves && DK / 16 <= kWaves, "head dim too large for 8 waves");
  static_assert(TBS <= 16 && 16 % TBS == 0, "token blocks must tile the 16-token tiles");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Op* sQR = reinterpret_cast<Op*>(smem + L::QR);
  Op* sKR = reinterpret_cast<Op*>(smem + L::KR);
  Op* sKC = reinterpret_cast<Op*>(smem + L::KC);
  float* sA = reinterpret_cast<float*>(smem + L::AS);
  float* sT = reinterpret_cast<float*>(smem + L::TS);
  Op* sTB = reinterpret_cast<Op*>(smem + L::TB);
  Op* sP = reinterpret_cast<Op*>(smem + L::PS);
  Op* sW = reinterpret_cast<Op*>(smem + L::WS);
  Op* sQG = reinterpret_cast<Op*>(smem + L::QG);
  Op* sKGT = reinterpret_cast<Op*>(smem + L::KGT);
  Op* sKBT = reinterpret_cast<Op*>(smem + L::KBT);
  Op* sVT = reinterpret_cast<Op*>(smem + L::VT);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sGam = reinterpret_cast<float*>(smem + L::GAM);
  float* sGC = reinterpret_cast<float*>(smem + L::GC);
  float* sRho = reinterpret_cast<float*>(smem + L::RHO);
  float* sERho = reinterpret_cast<float*>(smem + L::ERHO);
  float* sBtot = reinterpret_cast<float*>(smem + L::BTOT);
  float* sSsq = reinterpret_cast<float*>(smem + L::SSQ);
  int* sFlag = reinterpret_cast<int*>(smem + L::FLAG);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int gq = lane >> 4;   // lane group (0..3)
  const int li = lane & 15;   // index within the group
  const int bh = blockIdx.x;
  const int H = p.H, T = p.T;
  const int b = bh / H, h = bh - b * H;
  const bool owns_cols = wave < CTV;
  const int col0 = 16 * wave;  // first dv column of this wave

  // state columns [col0, col0+16) of S, as RTK accumulator tiles (C/D layout:
  // element r of tile t is S[16t + 4gq + r][col0 + li])
  f4 S[RTK];
#pragma unroll
  for (int t = 0; t < RTK; ++t) S[t] = f4{0.f, 0.f, 0.f, 0.f};
  if (owns_cols && p.S0 != nullptr) {
    const float* s0 = p.S0 + (size_t)bh * DK * DV;
#pragma unroll
    for (int t = 0; t < RTK; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[t][r] = s0[(16 * t + 4 * gq + r) * DV + col0 + li];
  }

  const int nchunks = (T + C - 1) / C;
  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = ci * C;
    const int n_valid = min(C, T - c0);

    // ---- stage 1: prep ----------------------------------------------------
    if (tid < 4) sFlag[tid] = 0;
    PrepItem<C, DK, DV, IN_BF16> it;
    prep_stage<C, DK, DV, IN_BF16>(p, b, h, c0, n_valid, sBtot, it);
    if (tid < C) {
      const int t = c0 + tid;
      sBeta[tid] = tid < n_valid ? load1<IN_BF16>(p.beta, ((size_t)b * T + t) * H + h) : 0.f;
    }
    // tile references rho_a = G(16a - 1), G_C, and the fp16-range check
    if (it.role == 0) {
      const int c8 = 8 * it.oct;
      const int last = it.tb * TBS + TBS - 1;  // chunk-relative last token of the block
      if (((last + 1) & 15) == 0) {
        const int a = (last + 1) >> 4;         // tile that starts after this block
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gv = it.G[TBS - 1][e];
          if (a < NT) {
            sRho[a * DK + c8 + e] = gv;
            sERho[a * DK + c8 + e] = fast_exp(gv);
          } else {
            sGC[c8 + e] = gv;
            sGam[c8 + e] = fast_exp(gv);
          }
        }
      }
      if (it.tb == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sRho[c8 + e] = 0.f;
          sERho[c8 + e] = 1.f;
        }
      }
      if constexpr (!F32) {
        // span of every tile for this octet: -(sum of g over the tile)
        float mx = 0.f;
        for (int a = 0; a < NT; ++a) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float s = 0.f;
            for (int q = a * (16 / TBS); q < (a + 1) * (16 / TBS); ++q) s -= sBtot[q * DK + c8 + e];
            mx = fmaxf(mx, s);
          }
        }
        if (mx > kF16SpanMax) atomicOr(&sFlag[0], 1);
      }
    }
    // v items write v^T now (no G needed)
    if (it.role == 2) {
      const int c8 = 8 * it.oct;
      const int tau0 = it.tb * TBS;
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int tt = 0; tt < TBS; ++tt) st_op<F32>(sVT + (c8 + e) * C + tau0 + tt, it.x[tt][e], false);
    }
    __syncthreads();
    const bool bfAP = sFlag[0] != 0;  // decay-weighted operands in bf16 for this chunk

    // q / k items: decay-scaled operands
    if (it.role == 0 || it.role == 1) {
      const int c8 = 8 * it.oct;
      const int tau0 = it.tb * TBS;
      const int bt = tau0 >> 4;  // 16-token tile of this block
      float rho[8], erho[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rho[e] = sRho[bt * DK + c8 + e];
        erho[e] = sERho[bt * DK + c8 + e];
      }
#pragma unroll
      for (int tt = 0; tt < TBS; ++tt) {
        const int tau = tau0 + tt;
        float er[8], rowv[8], gv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          er[e] = fast_exp(it.G[tt][e] - rho[e]);  // e^{G - rho_bt} <= 1
          rowv[e] = it.x[tt][e] * er[e];
          gv[e] = rowv[e] * erho[e];                // x e^{G}
        }
        if (it.role == 0) {
          st_op8<F32>(sQR + tau * DK + c8, rowv, bfAP);
          st_op8<F32>(sQG + tau * DK + c8, gv, false);
        } else {
          st_op8<F32>(sKR + tau * DK + c8, rowv, bfAP);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            st_op<F32>(sKGT + (c8 + e) * C + tau, gv[e], false);
            st_op<F32>(sKBT + (c8 + e) * C + tau, it.x[tt][e] * fast_exp(sGC[c8 + e] - it.G[tt][e]), false);
          }
          // column operands for row tiles a >= bt: k e^{rho_a - G}
          float ec[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ec[e] = it.x[tt][e] * fast_rcp(er[e]);
          for (int a = bt; a < NT; ++a) {
            float cv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              cv[e] = a == bt ? ec[e] : ec[e] * fast_exp(sRho[a * DK + c8 + e] - rho[e]);
            const int vrow = 16 * (a * (a + 1) / 2) + tau;  // rows of variant a start at 16*a(a+1)/2
            st_op8<F32>(sKC + vrow * DK + c8, cv, bfAP);
          }
        }
      }
    }
    __syncthreads();

    // ---- stage 2: A and P tiles on the matrix cores --------------------------
    // jobs: A(a,b) for b <= a (NKV), then P(a,b) (NKV); wave w takes w, w+8, ...
    constexpr int NJ = 2 * NKV;
    constexpr int JPW = (NJ + kWaves - 1) / kWaves;
    f4 acc[JPW];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      acc[jj] = f4{0.f, 0.f, 0.f, 0.f};
      const int job = wave + kWaves * jj;
      if (job < NJ) {
        const bool isP = job >= NKV;
        const int pj = isP ? job - NKV : job;
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= pj) ++a;
        const int bcol = pj - a * (a + 1) / 2;
        const Op* rowb = isP ? sQR : sKR;
        const int vrow = 16 * (a * (a + 1) / 2) + 16 * bcol + li;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int k0 = 32 * ks + 8 * gq;
          Frag<F32> fa, fb;
          frag_std<F32>(fa, rowb, 16 * a + li, DK, k0, k0 < DK);
          frag_std<F32>(fb, sKC, vrow, DK, k0, k0 < DK);
          acc[jj] = mma<F32>(fa, fb, acc[jj], bfAP);
        }
      }
    }
    __syncthreads();  // region X (A/P operands) is dead from here on
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int job = wave + kWaves * jj;
      if (job < NJ) {
        const bool isP = job >= NKV;
        const int pj = isP ? job - NKV : job;
        int a = 0;
        while ((a + 1) * (a + 2) / 2 <= pj) ++a;
        const int bcol = pj - a * (a + 1) / 2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * a + 4 * gq + r;
          const int col = 16 * bcol + li;
          if (isP) st_op<F32>(sP + row * C + col, row >= col ? acc[jj][r] : 0.f, false);
          else sA[row * C + col] = row > col ? sBeta[row] * acc[jj][r] : 0.f;
        }
      }
    }
    // upper tiles of P are zero (P.U runs over whole 32-token steps)
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int row = idx / C, col = idx - row * C;
      if ((col >> 4) > (row >> 4)) st_op<F32>(sP + idx, 0.f, false);
    }
    __syncthreads();

    // ---- stage 3: T = (I + A)^-1 ------------------------------------------------
    // diagonal 16x16 blocks by forward substitution: wave 0, lane = (block, column)
    if (wave == 0) {
      const int a = gq;   // block
      const int j = li;   // column
      if (a < NT) {
        float col[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = 0.f;
#pragma unroll
          for (int m = 0; m < i; ++m) s += sA[(16 * a + i) * C + 16 * a + m] * col[m];
          col[i] = i == j ? 1.f : (i > j ? -s : 0.f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(16 * a + i) * C + 16 * a + j] = col[i];
      }
    }
    // zero the upper blocks of T
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int row = idx / C, col = idx - row * C;
      if ((col >> 4) > (row >> 4)) sT[idx] = 0.f;
    }
    __syncthreads();
    // off-diagonal blocks by block diagonals d = a - b:
    //   T_ab = -T_aa * sum_{m=b}^{a-1} A_am T_mb
    float* scratch = reinterpret_cast<float*>(smem + L::TB);  // TB is free until stage 3 ends
    for (int d = 1; d < NT; ++d) {
      const int nb = NT - d;
      if (wave < nb) {
        const int bb = wave, a = wave + d;
        float* X = scratch + wave * 256;
        const int j = li;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int i = gq + 4 * s4;
          float x = 0.f;
          for (int m = bb; m < a; ++m)
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
              x += sA[(16 * a + i) * C + 16 * m + kk] * sT[(16 * m + kk) * C + 16 * bb + j];
          X[i * 16 + j] = x;
        }
      }
      __syncthreads();
      if (wave < nb) {
        const int bb = wave, a = wave + d;
        const float* X = scratch + wave * 256;
        const int j = li;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int i = gq + 4 * s4;
          float x = 0.f;
#pragma unroll
          for (int kk = 0; kk < 16; ++kk) x += sT[(16 * a + i) * C + 16 * a + kk] * X[kk * 16 + j];
          sT[(16 * a + i) * C + 16 * bb + j] = -x;
        }
      }
      __syncthreads();
    }
    // Tb = T diag(beta)
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int col = idx % C;
      st_op<F32>(sTB + idx, sT[idx] * sBeta[col], false);
    }
    __syncthreads();

    // ---- stage 4: W = Tb (K e^G)  (all dk columns) and U~ = Tb V (own columns)
    if (wave < DK / 16) {
      const int ct = wave;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        f4 w = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KSC; ++kt) {
          const int k0 = 32 * kt + 8 * gq;
          Frag<F32> fa, fb;
          frag_std<F32>(fa, sTB, 16 * rt + li, C, k0, k0 < C);
          frag_std<F32>(fb, sKGT, 16 * ct + li, C, k0, k0 < C);
          w = mma<F32>(fa, fb, w);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) st_op<F32>(sW + (16 * rt + 4 * gq + r) * DK + 16 * ct + li, w[r], false);
      }
    }
    f4 U[NT];
    if (owns_cols) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        U[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KSC; ++kt) {
          const int k0 = 32 * kt + 8 * gq;
          Frag<F32> fa, fb;
          frag_std<F32>(fa, sTB, 16 * rt + li, C, k0, k0 < C);
          frag_std<F32>(fb, sVT, col0 + li, C, k0, k0 < C);
          U[rt] = mma<F32>(fa, fb, U[rt]);
        }
      }
    }
    __syncthreads();

    // ---- stage 5: inter-chunk products and state update (own dv columns) -----
    f4 O[NT];
    if (owns_cols) {
      // S as B operand, contraction rows {32ks + 4gq + r} u {32ks + 16 + 4gq + r}
      Frag<F32> Sb[KSD];
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = S[2 * ks][r];
          x[4 + r] = (2 * ks + 1 < RTK) ? S[2 * ks + 1][r] : 0.f;
        }
        frag_from_f<F32>(Sb[ks], x);
      }
      // U = U~ - W S
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        f4 ws = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          Frag<F32> fa;
          frag_perm<F32>(fa, sW, 16 * rt + li, DK, 32 * ks, gq, true, 32 * ks + 16 < DK);
          ws = mma<F32>(fa, Sb[ks], ws);
        }
        U[rt] = U[rt] - ws;
      }
      // U as B operand over tokens, same permutation
      Frag<F32> Ub[KSC];
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt) {
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = U[2 * kt][r];
          x[4 + r] = (2 * kt + 1 < NT) ? U[2 * kt + 1][r] : 0.f;
        }
        frag_from_f<F32>(Ub[kt], x);
      }
      // O = (Q e^G) S + P U
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        f4 o = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          Frag<F32> fa;
          frag_perm<F32>(fa, sQG, 16 * rt + li, DK, 32 * ks, gq, true, 32 * ks + 16 < DK);
          o = mma<F32>(fa, Sb[ks], o);
        }
#pragma unroll
        for (int kt = 0; kt < KSC; ++kt) {
          if (32 * kt <= 16 * rt + 15) {
            Frag<F32> fa;
            frag_perm<F32>(fa, sP, 16 * rt + li, C, 32 * kt, gq, true, 32 * kt + 16 < C);
            o = mma<F32>(fa, Ub[kt], o);
          }
        }
        O[rt] = o;
      }
      // S <- e^{G_C} S + (K e^{G_C - G})^T U
#pragma unroll
      for (int t = 0; t < RTK; ++t) {
        f4 s = S[t];
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] *= sGam[16 * t + 4 * gq + r];
#pragma unroll
        for (int kt = 0; kt < KSC; ++kt) {
          Frag<F32> fa;
          frag_perm<F32>(fa, sKBT, 16 * t + li, C, 32 * kt, gq, true, 32 * kt + 16 < C);
          s = mma<F32>(fa, Ub[kt], s);
        }
        S[t] = s;
      }
      // partial sums of squares of each output row over this wave's 16 columns
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ss = group_sum<16>(O[rt][r] * O[rt][r]);
          if (li == 0) sSsq[wave * C + 16 * rt + 4 * gq + r] = ss;
        }
    }
    __syncthreads();

    // ---- epilogue: head-wise RMSNorm * sigmoid(gate) ----------------------------
    if (owns_cols) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * gq + r;
          if (row < n_valid) {
            float ss = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < CTV; ++w2) ss += sSsq[w2 * C + row];
            const float rs = fast_rsq(ss * (1.0f / DV) + kRmsEps);
            const size_t oi = (((size_t)b * T + c0 + row) * H + h) * DV + col0 + li;
            const float gt = load1<IN_BF16>(p.gate, oi);
            store1<OUT_BF16>(p.o, oi, O[rt][r] * rs * sigmoidf_(gt));
          }
        }
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  // ---- final state and conv history ------------------------------------------
  if (owns_cols && p.S_T != nullptr) {
    float* st = p.S_T + (size_t)bh * DK * DV;
#pragma unroll
    for (int t = 0; t < RTK; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(16 * t + 4 * gq + r) * DV + col0 + li] = S[t][r];
  }
  if (p.conv_out != nullptr && tid < NC) {
    const size_t cch = (size_t)H * NC;
    const void* src;
    size_t chb, D, c;
    if (tid < DK) { src = p.q; c = tid; D = DK; chb = (size_t)h * DK + c; }
    else if (tid < 2 * DK) { src = p.k; c = tid - DK; D = DK; chb = (size_t)H * DK + (size_t)h * DK + c; }
    else { src = p.v; c = tid - 2 * DK; D = DV; chb = (size_t)2 * H * DK + (size_t)h * DV + c; }
    float v3[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int t = T - 3 + r;
      if (t >= 0) v3[r] = load1<IN_BF16>(src, (((size_t)b * T + t) * H + h) * D + c);
      else if (p.conv_in != nullptr) v3[r] = load1<IN_BF16>(p.conv_in, ((size_t)b * 3 + (3 + t)) * cch + chb);
      else v3[r] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) store1<IN_BF16>(p.conv_out, ((size_t)b * 3 + r) * cch + chb, v3[r]);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
PrefillParams make_params(const kda_prefill_args& a) {
  PrefillParams p{};
  p.B = a.B; p.T = a.T; p.H = a.H;
  p.q = a.q; p.k = a.k; p.v = a.v; p.conv_w = a.conv_w;
  p.g = a.g; p.beta = a.beta; p.gate = a.gate;
  p.S0 = a.S0; p.conv_in = a.conv_in;
  p.o = a.o; p.S_T = a.S_T; p.conv_out = a.conv_out;
  return p;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s launch failed: %s", what, hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

template <int C, int D, bool IB, bool OB, bool F32>
int run_prefill(const kda_prefill_args& a, hipStream_t s) {
  using L = Smem<C, D, D, F32>;
  if (L::BYTES > 160 * 1024) {
    set_error("prefill: chunk %d x head dim %d needs %d bytes of LDS with %s operands", C, D, L::BYTES,
              F32 ? "fp32" : "16-bit");
    return KDA_E_UNSUPPORTED;
  }
  auto kern = prefill_kernel<C, D, D, IB, OB, F32>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
  if (e != hipSuccess) {
    set_error("prefill: hipFuncSetAttribute failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  PrefillParams p = make_params(a);
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.B * a.H)), dim3(kThreads), L::BYTES, s, p);
  return check_launch("prefill");
}

template <int C, int D>
int prefill_dt(const kda_prefill_args& a, hipStream_t s) {
  const bool ib = a.in_dtype == KDA_BF16, ob = a.out_dtype == KDA_BF16;
  if (ib) {
    if (ob) return run_prefill<C, D, true, true, false>(a, s);
    return run_prefill<C, D, true, false, false>(a, s);
  }
  if (ob) return run_prefill<C, D, false, true, true>(a, s);
  return run_prefill<C, D, false, false, true>(a, s);
}

template <int C>
int prefill_d(const kda_prefill_args& a, hipStream_t s) {
  switch (a.dk) {
    case 16: return prefill_dt<C, 16>(a, s);
    case 32: return prefill_dt<C, 32>(a, s);
    case 64: return prefill_dt<C, 64>(a, s);
    case 128: return prefill_dt<C, 128>(a, s);
  }
  set_error("prefill: head dim %d not instantiated", a.dk);
  return KDA_E_UNSUPPORTED;
}

template <int C, int D, bool IB>
int run_prep(const kda_prep_args& a, hipStream_t s) {
  PrefillParams p{};
  p.B = a.B; p.T = a.T; p.H = a.H;
  p.q = a.q; p.k = a.k; p.v = a.v; p.conv_w = a.conv_w; p.g = a.g; p.conv_in = a.conv_in;
  p.q_out = a.q_out; p.k_out = a.k_out; p.v_out = a.v_out; p.G_out = a.G_out;
  const int nchunks = (a.T + C - 1) / C;
  const size_t grid = (size_t)a.B * a.H * nchunks;
  hipLaunchKernelGGL((prep_kernel<C, D, D, IB>), dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return check_launch("prep");
}

template <int C>
int prep_d(const kda_prep_args& a, hipStream_t s) {
  const bool ib = a.in_dtype == KDA_BF16;
  switch (a.dk) {
    case 16: return ib ? run_prep<C, 16, true>(a, s) : run_prep<C, 16, false>(a, s);
    case 32: return ib ? run_prep<C, 32, true>(a, s) : run_prep<C, 32, false>(a, s);
    case 64: return ib ? run_prep<C, 64, true>(a, s) : run_prep<C, 64, false>(a, s);
    case 128: return ib ? run_prep<C, 128, true>(a, s) : run_prep<C, 128, false>(a, s);
  }
  set_error("prep: head dim %d not instantiated", a.dk);
  return KDA_E_UNSUPPORTED;
}

}  // namespace

int launch_prefill(const kda_prefill_args& a, hipStream_t s) {
  if (a.dk != a.dv) {
    set_error("prefill: dk (%d) != dv (%d) is not instantiated", a.dk, a.dv);
    return KDA_E_UNSUPPORTED;
  }
  switch (a.chunk) {
    case 16: return prefill_d<16>(a, s);
    case 32: return prefill_d<32>(a, s);
    case 64: return prefill_d<64>(a, s);
  }
  set_error("prefill: chunk %d not in {16,32,64}", a.chunk);
  return KDA_E_UNSUPPORTED;
}

int launch_prep(const kda_prep_args& a, hipStream_t s) {
  if (a.dk != a.dv) {
    set_error("prep: dk (%d) != dv (%d) is not instantiated", a.dk, a.dv);
    return KDA_E_UNSUPPORTED;
  }
  switch (a.chunk) {
    case 16: return prep_d<16>(a, s);
    case 32: return prep_d<32>(a, s);
    case 64: return prep_d<64>(a, s);
  }
  set_error("prep: chunk %d not in {16,32,64}", a.chunk);
  return KDA_E_UNSUPPORTED;
}

}  // namespace kda
