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
// accumulation fp32, state fp32, output fp32 by default.  The exceptions are
// where a factor can leave fp16's range or a single rounding shows:
//   * the column operand of the A and P tiles, k e^{rho_b - G} (up to e^80 at
//     K3's bound of -5 per token), is kept in fp32 and those products run on
//     the fp32 matrix-core instruction, with the fp16 row operands widened;
//   * in a chunk where some 16-token tile decays by more than e^8 ("wide":
//     the state then forgets nearly everything per token, so S_T and o are
//     dominated by the last tokens' U), U enters the P U and
//     (K e^{G_C-G})^T U products as an fp16 pair hi + lo (about 22 bits).
// fp32 inputs use fp32 operands on the fp32 matrix-core instruction throughout.
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
// Largest decay span of a 16-token tile (per channel, in nats) below which a
// chunk is not "wide" (see the precision notes above).
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
  const float* A;  // [H, dk]: g and beta are K3's logits (see k3_decay); null: given directly
  // [B*H][chunks][dk][dv]: the state entering every chunk, or null (the
  // backward's checkpoints); o may be null when only these are wanted
  float* S_chunks;
};

// ---------------------------------------------------------------------------
// matrix-core fragments: 8 contraction elements per lane (see kda_device.h)
// ---------------------------------------------------------------------------
template <bool F32> struct Frag;
template <> struct Frag<false> { half8 v; };        // fp16 or bf16 bits
template <> struct Frag<true> { float v[8]; };

template <bool F32>
using OpT = typename std::conditional<F32, float, uint16_t>::type;

// A value the compiler must treat as unknown at this point: per-lane indices
// derived from it inside a loop are recomputed each iteration instead of being
// hoisted out of the loop and kept live (or spilled) across it.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// 8 consecutive activations kept packed in registers until used.
template <bool BF16> struct Raw8;
template <> struct Raw8<true> { uint4 u; };
template <> struct Raw8<false> { float4 a, b; };

template <bool BF16>
__device__ __forceinline__ void raw_load(Raw8<BF16>& r, const void* base, size_t idx) {
  if constexpr (BF16) r.u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
  else {
    r.a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    r.b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx + 4);
  }
}
template <bool BF16>
__device__ __forceinline__ void raw_zero(Raw8<BF16>& r) {
  if constexpr (BF16) r.u = make_uint4(0, 0, 0, 0);
  else { r.a = make_float4(0.f, 0.f, 0.f, 0.f); r.b = r.a; }
}
// Unpack, giving zeros when `ok` is false (the mask is applied at use so that
// the load it guards never has to be waited for early).
template <bool BF16>
__device__ __forceinline__ void raw_unpack_if(const Raw8<BF16>& r, bool ok, float* o);

template <bool BF16>
__device__ __forceinline__ void raw_unpack(const Raw8<BF16>& r, float* o) {
  if constexpr (BF16) {
    o[0] = bf16lo(r.u.x); o[1] = bf16hi(r.u.x); o[2] = bf16lo(r.u.y); o[3] = bf16hi(r.u.y);
    o[4] = bf16lo(r.u.z); o[5] = bf16hi(r.u.z); o[6] = bf16lo(r.u.w); o[7] = bf16hi(r.u.w);
  } else {
    o[0] = r.a.x; o[1] = r.a.y; o[2] = r.a.z; o[3] = r.a.w;
    o[4] = r.b.x; o[5] = r.b.y; o[6] = r.b.z; o[7] = r.b.w;
  }
}

// Element e (0..7, a compile-time constant after unrolling) of a packed Raw8.
template <bool BF16>
__device__ __forceinline__ float raw_elem(const Raw8<BF16>& r, int e) {
  if constexpr (BF16) {
    const uint32_t w = e < 2 ? r.u.x : e < 4 ? r.u.y : e < 6 ? r.u.z : r.u.w;
    return (e & 1) ? bf16hi(w) : bf16lo(w);
  } else {
    return e == 0 ? r.a.x : e == 1 ? r.a.y : e == 2 ? r.a.z : e == 3 ? r.a.w
         : e == 4 ? r.b.x : e == 5 ? r.b.y : e == 6 ? r.b.z : r.b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void raw_unpack_if(const Raw8<BF16>& r, bool ok, float* o) {
  raw_unpack<BF16>(r, o);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = ok ? o[e] : 0.f;
}

__device__ __forceinline__ uint16_t to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t to_op16(float x) { return to_f16_bits(x); }

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
__device__ __forceinline__ f4 mma(const Frag<F32>& a, const Frag<F32>& b, f4 c) {
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
  } else {
    return mma_f16(a.v, b.v, c);
  }
}

template <bool F32>
__device__ __forceinline__ void st_op(OpT<F32>* p, float x) {
  if constexpr (F32) *p = x;
  else *p = to_op16(x);
}

// 8 consecutive operand elements from 8 fp32 values.
template <bool F32>
__device__ __forceinline__ void st_op8(OpT<F32>* p, const float* x) {
  if constexpr (F32) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  } else {
    uint4 u;
    u.x = (uint32_t)to_op16(x[0]) | ((uint32_t)to_op16(x[1]) << 16);
    u.y = (uint32_t)to_op16(x[2]) | ((uint32_t)to_op16(x[3]) << 16);
    u.z = (uint32_t)to_op16(x[4]) | ((uint32_t)to_op16(x[5]) << 16);
    u.w = (uint32_t)to_op16(x[6]) | ((uint32_t)to_op16(x[7]) << 16);
    *reinterpret_cast<uint4*>(p) = u;
  }
}

// Scale the 8 elements of a fragment by f[0..7] (fp32, 16-byte aligned),
// rounding back to the operand type.
template <bool F32>
__device__ __forceinline__ void frag_scale(Frag<F32>& fr, const float* f) {
  const float4 a = *reinterpret_cast<const float4*>(f);
  const float4 c = *reinterpret_cast<const float4*>(f + 4);
  const float s[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) fr.v[e] *= s[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) fr.v[e] = (_Float16)((float)fr.v[e] * s[e]);
  }
}

// 8 consecutive outputs (fp32 or bf16) to global memory.
template <bool BF16>
__device__ __forceinline__ void store8(void* base, size_t idx, const float* x) {
  if constexpr (BF16) {
    uint4 u;
    u.x = (uint32_t)f_to_bf16(x[0]) | ((uint32_t)f_to_bf16(x[1]) << 16);
    u.y = (uint32_t)f_to_bf16(x[2]) | ((uint32_t)f_to_bf16(x[3]) << 16);
    u.z = (uint32_t)f_to_bf16(x[4]) | ((uint32_t)f_to_bf16(x[5]) << 16);
    u.w = (uint32_t)f_to_bf16(x[6]) | ((uint32_t)f_to_bf16(x[7]) << 16);
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + idx) = u;
  } else {
    float* o = reinterpret_cast<float*>(base) + idx;
    *reinterpret_cast<float4*>(o) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// ---------------------------------------------------------------------------
// LDS layout of the fused kernel (byte offsets).  Operand rows are padded by
// 16 bytes so 16 lanes reading 16 consecutive rows hit distinct banks; arrays
// stored transposed ([channel][token]) also XOR-swizzle their 16-byte granules
// by (row / 16) so the per-token transposed stores spread over banks.
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool F32>
struct Smem {
  static constexpr int E = F32 ? 4 : 2;              // operand element bytes
  static constexpr int PAD = 16 / E;                 // 16 bytes of padding, in elements
  static constexpr int NT = C / 16;                  // 16-token tiles per chunk
  static constexpr int NOFF = NT * (NT - 1) / 2;     // strictly-lower tile pairs
  static constexpr int LDR = DK + PAD;               // rows of dk-wide operands
  static constexpr int LDC = C + PAD;                // rows of chunk-wide operands
  static constexpr int LDT = C + PAD;                // rows of transposed operands
  static constexpr int LDA = C + 4;                  // fp32 A and T
  // region X, phase 0 (stage 1a/1b only): sums of g per 4-token k block
  static constexpr int BTOT = 0;                            // [16][DK] fp32
  static constexpr int BTOT_BYTES = 16 * DK * 4;
  // region X, phase 1: decay-weighted A/P operands
  static constexpr int LDRF = DK + 4;                       // rows of the fp32 column operand
  static constexpr int QR = 0;                              // [C][LDR]  q^ e^{G - rho_tile}
  static constexpr int KR = QR + C * LDR * E;               // [C][LDR]  k^ e^{G - rho_tile}
  static constexpr int KC = KR + C * LDR * E;               // [C][LDRF] k^ e^{rho_tile - G}, fp32
  static constexpr int X1 = KC + C * LDRF * 4;
  // wide chunks (16-bit operands): the A/P rows in fp32 instead, q's over QR
  // and KR, k's over QG and KGT (rebuilt from these rows after the products)
  static constexpr int QRF = QR;                            // [C][LDRF] fp32
  // region X, phase 2 (after the A/P products)
  static constexpr int AS = 0;                              // [C][LDA] fp32
  static constexpr int TS = AS + C * LDA * 4;               // [C][LDA] fp32
  static constexpr int TB = TS + C * LDA * 4;               // [C][LDC] T diag(beta)
  static constexpr int PS = TB + C * LDC * E;               // [C][LDC] P
  static constexpr int X2 = PS + C * LDC * E;
  static constexpr int XE0 = X1 > X2 ? X1 : X2;
  static constexpr int XE = XE0 > BTOT_BYTES ? XE0 : BTOT_BYTES;
  // region Y: operands of the W / U~ / inter-chunk products
  static constexpr int QG = (XE + 15) / 16 * 16;            // [C][LDR]   q^ e^G
  static constexpr int KGT = QG + C * LDR * E;              // [DK][LDT]  (k^ e^G)^T, later W [C][LDR]
  static constexpr int KGT_BYTES = (DK * LDT > C * LDR ? DK * LDT : C * LDR) * E;
  static constexpr int KBT = KGT + KGT_BYTES;               // [DK][LDT]  (k^ e^{G_C-G})^T
  static constexpr int KRF = QG;                            // [C][LDRF] fp32, wide chunks
  static constexpr int VT = KBT + DK * LDT * E;             // [DV][LDT]  v^T
  // small fp32 arrays
  static constexpr int BETA = VT + DV * LDT * E;            // [C]
  static constexpr int GAM = BETA + C * 4;                  // [DK]  e^{G_C}
  static constexpr int GC = GAM + DK * 4;                   // [DK]  G_C
  static constexpr int RHO = GC + DK * 4;                   // [NT][DK]  rho_a
  static constexpr int ERHO = RHO + NT * DK * 4;            // [NT][DK]  e^{rho_a}
  static constexpr int FAB = ERHO + NT * DK * 4;            // [NOFF][DK] e^{rho_a - rho_b}, b < a
  static constexpr int CW = FAB + (NOFF > 0 ? NOFF : 1) * DK * 4;  // [2dk+dv][4] conv taps of the head
  static constexpr int FLAG = CW + (2 * DK + DV) * 16;      // [4] ints
  // O of a chunk, staged for the epilogue: [C][DV+4] fp32, in A / T's space
  // (dead by then) when it fits, else after everything else
  static constexpr int LDO = DV + 4;
  static constexpr int OS_BYTES = C * LDO * 4;
  static constexpr int OS = OS_BYTES <= TB ? 0 : FLAG + 16;
  static constexpr int BYTES = OS_BYTES <= TB ? FLAG + 16 : FLAG + 16 + OS_BYTES;
  static_assert(F32 || QRF + C * LDRF * 4 <= KC, "wide-chunk q rows overlap the column operand");
  static_assert(F32 || KRF + C * LDRF * 4 <= KBT, "wide-chunk k rows overlap (k e^{G_C-G})^T");
};

// index of the pair (a, b), b < a, among the strictly-lower tile pairs
__device__ __forceinline__ int off_pair(int a, int b) { return a * (a - 1) / 2 + b; }

// element (row, k) of a transposed operand array with LDT columns and
// 8-element granules swizzled by row / 16
template <int C, int LDT>
__device__ __forceinline__ int tidx(int row, int k) {
  constexpr int NG = C / 8;
  return row * LDT + ((((k >> 3) ^ (row >> 4)) & (NG - 1)) << 3) + (k & 7);
}

// Fragment of 8 consecutive tokens k0..k0+7 (k0 % 8 == 0) of row `row` of a
// transposed operand array.
template <bool F32, int C, int LDT>
__device__ __forceinline__ void frag_std_t(Frag<F32>& f, const OpT<F32>* buf, int row, int k0, bool valid) {
  if (!valid) { frag_zero(f); return; }
  frag_std<F32>(f, buf + tidx<C, LDT>(row, k0), 0, 0, 0, true);
}

// Permuted-order fragment (tokens kb + 4g + 0..3 and kb + 16 + 4g + 0..3) of a
// transposed operand array.
template <bool F32, int C, int LDT>
__device__ __forceinline__ void frag_perm_t(Frag<F32>& f, const OpT<F32>* buf, int row, int kb, int g,
                                            bool hi_valid) {
  const OpT<F32>* p1 = buf + tidx<C, LDT>(row, kb + 4 * g);
  if constexpr (F32) {
    const float4 a = *reinterpret_cast<const float4*>(p1);
    float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
    if (hi_valid) c = *reinterpret_cast<const float4*>(buf + tidx<C, LDT>(row, kb + 16 + 4 * g));
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = c.x; f.v[5] = c.y; f.v[6] = c.z; f.v[7] = c.w;
  } else {
    const half4 a = *reinterpret_cast<const half4*>(p1);
    half4 c = half4{0, 0, 0, 0};
    if (hi_valid) c = *reinterpret_cast<const half4*>(buf + tidx<C, LDT>(row, kb + 16 + 4 * g));
    f.v = half8{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  }
}

// ---------------------------------------------------------------------------
// Stage 1 pieces (shared by the fused kernel and the standalone kda_prep).
// Thread roles (NC = 2dk + dv items, one per thread):
//   item i <  dk        : q, channel octet i % (dk/8), token block i / (dk/8)
//   dk <= i < 2dk        : k, same mapping
//   2dk <= i < NC        : v, octet (i-2dk) % (dv/8), token block (i-2dk) / (dv/8)
// A token block is C/8 consecutive tokens; a thread walks its block token by
// token with a 4-token window of raw values, so it never holds the block.
// Tokens past n_valid are zero (with g = 0 and beta = 0), which makes a
// ragged last chunk exact.
// ---------------------------------------------------------------------------
struct Item {
  int role;   // 0 q, 1 k, 2 v, -1 idle
  int oct;    // channel octet within its tensor
  int tb;     // token block
  int D;      // channels of the tensor
  size_t chb; // first conv channel of the octet
  const void* src;
};

template <int DK, int DV>
__device__ __forceinline__ Item make_item(const PrefillParams& p, int h, int tid) {
  constexpr int NC = 2 * DK + DV;
  Item it;
  it.role = -1; it.oct = 0; it.tb = 0; it.D = DK; it.chb = 0; it.src = p.q;
  const int H = p.H;
  if (tid < DK) {
    it.role = 0; it.D = DK; it.src = p.q;
    it.oct = tid % (DK / 8); it.tb = tid / (DK / 8);
    it.chb = (size_t)h * DK + 8 * it.oct;
  } else if (tid < 2 * DK) {
    it.role = 1; it.D = DK; it.src = p.k;
    it.oct = (tid - DK) % (DK / 8); it.tb = (tid - DK) / (DK / 8);
    it.chb = (size_t)H * DK + (size_t)h * DK + 8 * it.oct;
  } else if (tid < NC) {
    it.role = 2; it.D = DV; it.src = p.v;
    it.oct = (tid - 2 * DK) % (DV / 8); it.tb = (tid - 2 * DK) / (DV / 8);
    it.chb = (size_t)2 * H * DK + (size_t)h * DV + 8 * it.oct;
  }
  return it;
}

// Conv + SiLU state of one item for one chunk: taps and the three previous raw
// tokens (h0 oldest).  The window shifts by assignment, so a rolled token loop
// never indexes a register array dynamically.
struct ConvState {
  float w[8][4];
  float h0[8], h1[8], h2[8];
};

template <bool IN_BF16, int NC>
__device__ __forceinline__ void conv_begin(const PrefillParams& p, const Item& it, int b, int h, int t0,
                                           ConvState& cs) {
  const size_t cch = (size_t)p.H * NC;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float4 t = *reinterpret_cast<const float4*>(p.conv_w + (it.chb + e) * 4);
    cs.w[e][0] = t.x; cs.w[e][1] = t.y; cs.w[e][2] = t.z; cs.w[e][3] = t.w;
  }
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int t = t0 - 3 + u;
    float* dst = u == 0 ? cs.h0 : u == 1 ? cs.h1 : cs.h2;
    if (t >= 0 && t < p.T) {
      load8<IN_BF16>(it.src, ((size_t)b * p.T + t) * p.H * it.D + (size_t)h * it.D + 8 * it.oct, dst);
    } else if (t < 0 && p.conv_in != nullptr) {
      load8<IN_BF16>(p.conv_in, ((size_t)b * 3 + (3 + t)) * cch + it.chb, dst);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = 0.f;
    }
  }
}

// Next token t: SiLU(conv) into x (0 if !valid), then shift the window.
template <bool IN_BF16>
__device__ __forceinline__ void conv_step(const PrefillParams& p, const Item& it, int b, int h, int t,
                                          bool valid, ConvState& cs, float* x) {
  float cur[8];
  if (t < p.T) {
    load8<IN_BF16>(it.src, ((size_t)b * p.T + t) * p.H * it.D + (size_t)h * it.D + 8 * it.oct, cur);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) cur[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float a = cs.w[e][0] * cs.h0[e] + cs.w[e][1] * cs.h1[e] + cs.w[e][2] * cs.h2[e] + cs.w[e][3] * cur[e];
    x[e] = valid ? siluf_(a) : 0.f;
    cs.h0[e] = cs.h1[e];
    cs.h1[e] = cs.h2[e];
    cs.h2[e] = cur[e];
  }
}

// L2 normalisation of one token over dk channels held by DK/8 consecutive lanes.
template <int DK>
__device__ __forceinline__ void l2norm(float* x, float extra) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  ss = group_sum<DK / 8>(ss);
  const float r = fast_rsq(ss + kL2Eps) * extra;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= r;
}

// g of channels c8 .. c8+7 of head h from the loaded input: the input itself,
// or K3's bounded log-decay of the logits in it (tokens that are not loaded
// keep g = 0)
__device__ __forceinline__ void g_from_input(const float* A, int h, int DK, int c8, bool loaded, float* gv) {
  if (A != nullptr && loaded) {
    const float4 a0 = *reinterpret_cast<const float4*>(A + (size_t)h * DK + c8);
    const float4 a1 = *reinterpret_cast<const float4*>(A + (size_t)h * DK + c8 + 4);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = k3_decay(gv[e], fast_exp(av[e]));
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void load_g(const PrefillParams& p, int b, int h, int t, int c8, int DK, bool valid,
                                       float* gv) {
  if (valid) {
    load8<IN_BF16>(p.g, ((size_t)b * p.T + t) * p.H * DK + (size_t)h * DK + c8, gv);
    g_from_input(p.A, h, DK, c8, true, gv);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) gv[e] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// standalone stage-1 kernel: one block per (b, h, chunk)
// ---------------------------------------------------------------------------
template <int C, int DK, int DV, bool IN_BF16>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrefillParams p) {
  constexpr int TBS = C / 8;
  constexpr int NC = 2 * DK + DV;
  __shared__ float btot[8 * DK];
  const int nchunks = (p.T + C - 1) / C;
  const int bh = blockIdx.x / nchunks;
  const int ci = blockIdx.x - bh * nchunks;
  const int b = bh / p.H, h = bh - b * p.H;
  const int c0 = ci * C;
  const int n_valid = min(C, p.T - c0);
  const Item it = make_item<DK, DV>(p, h, threadIdx.x);
  const int c8 = 8 * it.oct;
  const int tau0 = it.tb * TBS;
  // block sums of g, then each thread's prefix
  if (it.role == 0) {
    float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int tt = 0; tt < TBS; ++tt) {
      float gv[8];
      load_g<IN_BF16>(p, b, h, c0 + tau0 + tt, c8, DK, tau0 + tt < n_valid, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += gv[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) btot[it.tb * DK + c8 + e] = s[e];
  }
  __syncthreads();
  if (it.role < 0) return;
  float G[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (it.role == 0) {
    for (int q = 0; q < it.tb; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) G[e] += btot[q * DK + c8 + e];
  }
  ConvState cs;
  conv_begin<IN_BF16, NC>(p, it, b, h, c0 + tau0, cs);
  float* dst = it.role == 0 ? p.q_out : it.role == 1 ? p.k_out : p.v_out;
#pragma unroll 1
  for (int tt = 0; tt < TBS; ++tt) {
    const int tau = tau0 + tt;
    const bool valid = tau < n_valid;
    float x[8];
    conv_step<IN_BF16>(p, it, b, h, c0 + tau, valid, cs, x);
    if (it.role < 2) l2norm<DK>(x, it.role == 0 ? fast_rsq((float)DK) : 1.0f);
    if (!valid) continue;
    const size_t row = ((size_t)b * p.T + c0 + tau) * p.H + h;
    float* o = dst + row * it.D + c8;
    *reinterpret_cast<float4*>(o) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(x[4], x[5], x[6], x[7]);
    if (it.role == 0) {
      float gv[8];
      load_g<IN_BF16>(p, b, h, c0 + tau, c8, DK, true, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) G[e] += gv[e];
      float* go = p.G_out + row * DK + c8;
      *reinterpret_cast<float4*>(go) = make_float4(G[0], G[1], G[2], G[3]);
      *reinterpret_cast<float4*>(go + 4) = make_float4(G[4], G[5], G[6], G[7]);
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
  constexpr int NKV = NT * (NT + 1) / 2;
  constexpr int NC = 2 * DK + DV;
  constexpr int KSD = (DK + 31) / 32;   // 32-wide contraction steps over dk
  constexpr int KSC = (C + 31) / 32;    // ... over the tokens of a chunk
  constexpr int RTK = DK / 16;          // 16-row tiles of the state
  constexpr int CTV = DV / 16;          // 16-column tiles of dv (one per wave)
  constexpr int LDR = L::LDR, LDC = L::LDC, LDT = L::LDT, LDA = L::LDA;
  static_assert(CTV <= kWaves && DK / 16 <= kWaves, "head dim too large for 8 waves");
  static_assert(C >= 16 && 256 % C == 0, "k blocks must tile the 16-token tiles");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Op* sQR = reinterpret_cast<Op*>(smem + L::QR);
  Op* sKR = reinterpret_cast<Op*>(smem + L::KR);
  float* sKC = reinterpret_cast<float*>(smem + L::KC);
  float* sA = reinterpret_cast<float*>(smem + L::AS);
  float* sT = reinterpret_cast<float*>(smem + L::TS);
  Op* sTB = reinterpret_cast<Op*>(smem + L::TB);
  Op* sP = reinterpret_cast<Op*>(smem + L::PS);
  Op* sQG = reinterpret_cast<Op*>(smem + L::QG);
  float* sQRf = reinterpret_cast<float*>(smem + L::QRF);  // wide chunks (16-bit operands)
  float* sKRf = reinterpret_cast<float*>(smem + L::KRF);
  Op* sKGT = reinterpret_cast<Op*>(smem + L::KGT);
  Op* sW = reinterpret_cast<Op*>(smem + L::KGT);   // W replaces (k e^G)^T after stage 4
  Op* sKBT = reinterpret_cast<Op*>(smem + L::KBT);
  Op* sVT = reinterpret_cast<Op*>(smem + L::VT);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  float* sGam = reinterpret_cast<float*>(smem + L::GAM);
  float* sGC = reinterpret_cast<float*>(smem + L::GC);
  float* sRho = reinterpret_cast<float*>(smem + L::RHO);
  float* sERho = reinterpret_cast<float*>(smem + L::ERHO);
  float* sFab = reinterpret_cast<float*>(smem + L::FAB);
  float* sBtot = reinterpret_cast<float*>(smem + L::BTOT);
  float* sO = reinterpret_cast<float*>(smem + L::OS);
  int* sFlag = reinterpret_cast<int*>(smem + L::FLAG);
  float4* sCW = reinterpret_cast<float4*>(smem + L::CW);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = blockIdx.x;
  const int H = p.H, T = p.T;
  const int b = bh / H, h = bh - b * H;
  const bool owns_cols = wave < CTV;
  const int col0 = 16 * wave;  // first dv column of this wave

  // state columns [col0, col0+16) of S as RTK accumulator tiles: element r of
  // tile t is S[16t + 4gq + r][col0 + li]
  f4 S[RTK];
#pragma unroll
  for (int t = 0; t < RTK; ++t) S[t] = f4{0.f, 0.f, 0.f, 0.f};
  if (owns_cols && p.S0 != nullptr) {
    const int gq = (threadIdx.x & 63) >> 4, li = threadIdx.x & 15;
    const float* s0 = p.S0 + (size_t)bh * DK * DV;
#pragma unroll
    for (int t = 0; t < RTK; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[t][r] = s0[(16 * t + 4 * gq + r) * DV + col0 + li];
  }

  // conv taps of this head's q | k | v channels, in the head-local channel order
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    size_t ch;
    if (c < DK) ch = (size_t)h * DK + c;
    else if (c < 2 * DK) ch = (size_t)H * DK + (size_t)h * DK + (c - DK);
    else ch = (size_t)2 * H * DK + (size_t)h * DV + (c - 2 * DK);
    sCW[c] = *reinterpret_cast<const float4*>(p.conv_w + ch * 4);
  }

  // Stage-1 roles (one per wave, so every role branch is wave-uniform):
  //   q items: threads [0, DK)         octet i % (DK/8), block i / (DK/8) of C/8 tokens
  //   k items: threads [DK, 3DK)       octet j % (DK/8), block j / (DK/8) of C/16 tokens
  //   v items: threads [3DK, 3DK + DV) octet j % (DV/8), block j / (DV/8) of C/8 tokens
  // Keys get twice the threads: their per-token work (row, column and two
  // transposed operands, two exponentials) is the heaviest.
  constexpr int TBQ = C / 8;            // tokens per q / v block
  constexpr int TBK = C / 16;           // tokens per k block
  constexpr int BPT = 16 / TBK;         // k blocks per 16-token tile
  constexpr int NE = C * DV / 8;        // epilogue items: (token, dv octet)
  constexpr int EPT = (NE + kThreads - 1) / kThreads;
  static_assert(3 * DK + DV <= kThreads, "stage-1 roles need 3dk + dv threads");

  const int nchunks = (T + C - 1) / C;
  const size_t cch = (size_t)H * NC;
  const bool has_hist = p.conv_in != nullptr;

  // per-thread role, recomputed from an opaque thread id wherever needed
  struct Role { int role, oct, blk, tau0, D; size_t chb; const void* src; };
  auto make_role = [&](int t) {
    Role r;
    if (t < DK) {
      r.role = 0; r.D = DK; r.src = p.q; r.oct = t % (DK / 8); r.blk = t / (DK / 8); r.tau0 = r.blk * TBQ;
      r.chb = (size_t)h * DK + 8 * r.oct;
    } else if (t < 3 * DK) {
      const int j = t - DK;
      r.role = 1; r.D = DK; r.src = p.k; r.oct = j % (DK / 8); r.blk = j / (DK / 8); r.tau0 = r.blk * TBK;
      r.chb = (size_t)H * DK + (size_t)h * DK + 8 * r.oct;
    } else if (t < 3 * DK + DV) {
      const int j = t - 3 * DK;
      r.role = 2; r.D = DV; r.src = p.v; r.oct = j % (DV / 8); r.blk = j / (DV / 8); r.tau0 = r.blk * TBQ;
      r.chb = (size_t)2 * H * DK + (size_t)h * DV + 8 * r.oct;
    } else {
      r.role = -1; r.D = DK; r.src = p.q; r.oct = 0; r.blk = 0; r.tau0 = 0; r.chb = 0;
    }
    return r;
  };

  // Loads of one chunk: raw tokens tau0-3 .. tau0+ntok-1 of the item's octet,
  // g for q / k items, beta.  Unconditional from clamped, in-bounds addresses;
  // which values are real is kept in bit masks applied at use.  (A load under
  // a per-load branch, or a register overwritten after a load, makes the
  // compiler wait for it on the spot and serialises the loads.)
  Raw8<IN_BF16> rw[TBQ + 3];
  Raw8<IN_BF16> gr[TBQ];
  uint32_t rw_ok = 0, gr_ok = 0;
  float beta_v = 0.f;
  auto issue_loads = [&](int ci_load) {
    const int tl = opaque((int)threadIdx.x);
    const Role r = make_role(tl);
    const int cl = ci_load * C;
    const int nv = min(C, T - cl);
    const int c8 = 8 * r.oct;
    rw_ok = 0;
    gr_ok = 0;
    auto load_raw = [&](int u) {
      const int t = cl + r.tau0 - 3 + u;
      const bool hist = t < 0 && has_hist;
      const int tc = min(max(t, 0), T - 1);
      const void* base = hist ? p.conv_in : r.src;
      const size_t idx = hist ? ((size_t)b * 3 + (3 + t)) * cch + r.chb
                              : ((size_t)b * T + tc) * H * r.D + (size_t)h * r.D + c8;
      raw_load<IN_BF16>(rw[u], base, idx);
      rw_ok |= (hist || (t >= 0 && t < T)) ? (1u << u) : 0u;
    };
    auto load_g = [&](int tt) {
      const int t = min(cl + r.tau0 + tt, T - 1);
      raw_load<IN_BF16>(gr[tt], p.g, ((size_t)b * T + t) * H * DK + (size_t)h * DK + c8);
      gr_ok |= (r.tau0 + tt < nv) ? (1u << tt) : 0u;
    };
    if (r.role == 1) {
#pragma unroll
      for (int u = 0; u < TBK + 3; ++u) load_raw(u);
#pragma unroll
      for (int tt = 0; tt < TBK; ++tt) load_g(tt);
    } else if (r.role >= 0) {
#pragma unroll
      for (int u = 0; u < TBQ + 3; ++u) load_raw(u);
      if (r.role == 0) {
#pragma unroll
        for (int tt = 0; tt < TBQ; ++tt) load_g(tt);
      }
    }
    if (tl < C) {
      beta_v = load1<IN_BF16>(p.beta, ((size_t)b * T + cl + min(tl, nv - 1)) * H + h);
      if (p.A != nullptr) beta_v = sigmoidf_(beta_v);
    }
  };

  if (nchunks > 0) issue_loads(0);

  for (int ci = 0; ci < nchunks; ++ci) {
    const int c0 = ci * C;
    const int n_valid = min(C, T - c0);
    if (p.S_chunks != nullptr && owns_cols) {
      float* sc = p.S_chunks + ((size_t)bh * nchunks + ci) * DK * DV;
      const int sg = (threadIdx.x & 63) >> 4, sl = threadIdx.x & 15;
#pragma unroll
      for (int t = 0; t < RTK; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[(16 * t + 4 * sg + r) * DV + col0 + sl] = S[t][r];
    }
    // per-lane indices, recomputed every chunk (see opaque())
    const int tid = opaque((int)threadIdx.x);
    const int lane = tid & 63;
    const int gq = lane >> 4;   // lane group (0..3)
    const int li = lane & 15;   // index within the group
    const Role it = make_role(tid);
    const int c8 = 8 * it.oct;
    const int tau0 = it.tau0;

    // ---- stage 1a: beta, sums of g over the k blocks --------------------------
    if (tid < 4) sFlag[tid] = 0;
    if (tid < C) sBeta[tid] = tid < n_valid ? beta_v : 0.f;
    if (it.role == 1) {
      float s8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int tt = 0; tt < TBK; ++tt) {
        float gv[8];
        raw_unpack_if<IN_BF16>(gr[tt], (gr_ok >> tt) & 1u, gv);
        g_from_input(p.A, h, DK, c8, (gr_ok >> tt) & 1u, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) s8[e] += gv[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sBtot[it.blk * DK + c8 + e] = s8[e];
    }
    lds_barrier();

    // ---- stage 1b: per-tile decay scalars (k-item threads, one job per block) -
    //   blk <  NT : rho_blk = G before tile blk, e^{rho_blk}, e^{rho_blk - rho_b} (b < blk)
    //   blk == NT : G_C and e^{G_C}
    //   blk == NT+1 : fp16 range check of the tile spans
    if (it.role == 1 && it.blk < NT + 2) {
      float rho[NT + 1][8];  // rho[a] = sum of the blocks before tile a; rho[NT] = G_C
#pragma unroll
      for (int e = 0; e < 8; ++e) rho[0][e] = 0.f;
#pragma unroll
      for (int a = 0; a < NT; ++a) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float sa = rho[a][e];
#pragma unroll
          for (int q = a * BPT; q < (a + 1) * BPT; ++q) sa += sBtot[q * DK + c8 + e];
          rho[a + 1][e] = sa;
        }
      }
      if (it.blk < NT) {
#pragma unroll
        for (int a = 0; a < NT; ++a) {
          if (a != it.blk) continue;  // static indices into rho[][]
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            sRho[a * DK + c8 + e] = rho[a][e];
            sERho[a * DK + c8 + e] = fast_exp(rho[a][e]);
          }
#pragma unroll
          for (int bb = 0; bb < a; ++bb)
#pragma unroll
            for (int e = 0; e < 8; ++e) sFab[off_pair(a, bb) * DK + c8 + e] = fast_exp(rho[a][e] - rho[bb][e]);
        }
      } else if (it.blk == NT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sGC[c8 + e] = rho[NT][e];
          sGam[c8 + e] = fast_exp(rho[NT][e]);
        }
      } else {
        float mx = 0.f;
#pragma unroll
        for (int a = 0; a < NT; ++a)
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = fmaxf(mx, rho[a][e] - rho[a + 1][e]);
        if (mx > kF16SpanMax) atomicOr(&sFlag[0], 1);
      }
    }
    // each q / k thread: G just before its first token
    float G[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (it.role == 0 || it.role == 1) {
      const int nb = tau0 / TBK;  // k blocks before tau0
      for (int q = 0; q < nb; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) G[e] += sBtot[q * DK + c8 + e];
    }
    lds_barrier();
    const bool wide = __builtin_amdgcn_readfirstlane(sFlag[0]) != 0;  // U split in two fp16 parts

    // ---- stage 1c: conv + SiLU + L2, then the decay-scaled operands -----------
    auto token_work = [&](int tt, bool is_k) {
      const int tau = tau0 + tt;
      const bool valid = tau < n_valid;
      float x[8];
      {
        // raw tokens tau-3 .. tau, unpacked per channel; taps from LDS
        const bool ok0 = (rw_ok >> tt) & 1u, ok1 = (rw_ok >> (tt + 1)) & 1u;
        const bool ok2 = (rw_ok >> (tt + 2)) & 1u, ok3 = (rw_ok >> (tt + 3)) & 1u;
        const float4* cw = sCW + (it.role == 0 ? 0 : it.role == 1 ? DK : 2 * DK) + c8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float4 wv = cw[e];
          const float a = wv.x * (ok0 ? raw_elem<IN_BF16>(rw[tt], e) : 0.f) +
                          wv.y * (ok1 ? raw_elem<IN_BF16>(rw[tt + 1], e) : 0.f) +
                          wv.z * (ok2 ? raw_elem<IN_BF16>(rw[tt + 2], e) : 0.f) +
                          wv.w * (ok3 ? raw_elem<IN_BF16>(rw[tt + 3], e) : 0.f);
          x[e] = valid ? siluf_(a) : 0.f;
        }
      }
      if (it.role == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) st_op<F32>(sVT + tidx<C, LDT>(c8 + e, tau), x[e]);
        return;
      }
      l2norm<DK>(x, is_k ? 1.0f : fast_rsq((float)DK));
      const int bt = tau >> 4;  // 16-token tile
      const float* rho = sRho + bt * DK + c8;
      const float* erho = sERho + bt * DK + c8;
      float gv[8];
      raw_unpack_if<IN_BF16>(gr[tt], (gr_ok >> tt) & 1u, gv);
      g_from_input(p.A, h, DK, c8, (gr_ok >> tt) & 1u, gv);
      float er[8], rowv[8], xg[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        G[e] += gv[e];
        er[e] = fast_exp(G[e] - rho[e]);  // e^{G - rho_bt} <= 1
        rowv[e] = x[e] * er[e];
        xg[e] = rowv[e] * erho[e];         // x e^{G}
      }
      // A wide chunk keeps the rows in fp32 (the in-tile column factor can make
      // up for a row factor below fp16's range); q e^G and (k e^G)^T are then
      // rebuilt from those rows after the A / P products.
      const bool rows32 = !F32 && wide;
      if (!is_k) {
        if (rows32) {
          st_op8<true>(sQRf + tau * L::LDRF + c8, rowv);
        } else {
          st_op8<F32>(sQR + tau * LDR + c8, rowv);
          st_op8<F32>(sQG + tau * LDR + c8, xg);
        }
      } else {
        if (rows32) st_op8<true>(sKRf + tau * L::LDRF + c8, rowv);
        else st_op8<F32>(sKR + tau * LDR + c8, rowv);
        float cv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          cv[e] = x[e] * fast_rcp(er[e]);  // k e^{rho_bt - G}
          if (!rows32) st_op<F32>(sKGT + tidx<C, LDT>(c8 + e, tau), xg[e]);
          st_op<F32>(sKBT + tidx<C, LDT>(c8 + e, tau), x[e] * fast_exp(sGC[c8 + e] - G[e]));
        }
        st_op8<true>(sKC + tau * L::LDRF + c8, cv);
      }
    };
    if (it.role == 1) {
#pragma unroll
      for (int tt = 0; tt < TBK; ++tt) token_work(tt, true);
    } else if (it.role >= 0) {
#pragma unroll
      for (int tt = 0; tt < TBQ; ++tt) token_work(tt, false);
    }
    lds_barrier();

    // ---- stage 2: A and P tiles on the matrix cores --------------------------
    // jobs: A(a,b) for b <= a (NKV), then P(a,b) (NKV); wave w takes w, w+8, ...
    // The column operand of tile b is k e^{rho_b - G}; for b < a it is scaled
    // by e^{rho_a - rho_b} <= 1 while loading, giving the reference rho_a.
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
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const int k0 = 32 * ks + 8 * gq;
          Frag<true> fa, fb;  // fp32 instruction: the column factor needs fp32's range
          if constexpr (F32) {
            frag_std<true>(fa, rowb, 16 * a + li, LDR, k0, k0 < DK);
          } else if (wide) {
            frag_std<true>(fa, isP ? sQRf : sKRf, 16 * a + li, L::LDRF, k0, k0 < DK);
          } else {
            Frag<false> f16;
            frag_std<false>(f16, rowb, 16 * a + li, LDR, k0, k0 < DK);
#pragma unroll
            for (int e = 0; e < 8; ++e) fa.v[e] = (float)f16.v[e];
          }
          frag_std<true>(fb, sKC, 16 * bcol + li, L::LDRF, k0, k0 < DK);
          if (bcol < a && k0 < DK) frag_scale<true>(fb, sFab + off_pair(a, bcol) * DK + k0);
          acc[jj] = mma<true>(fa, fb, acc[jj]);
        }
      }
    }
    // wide chunks: q e^G and k e^G from the fp32 rows (x e^{G - rho_tile} times
    // e^{rho_tile}, the same products the plain path stores), read before the
    // barrier since the k rows sit where they go
    constexpr int NRB = (C * DK + kThreads - 1) / kThreads;
    float qgv[NRB], kgv[NRB];
    if (!F32 && wide) {
#pragma unroll
      for (int j = 0; j < NRB; ++j) {
        const int idx = tid + kThreads * j;
        const int r = min(idx / DK, C - 1), c = idx % DK;
        const float er = sERho[(r >> 4) * DK + c];
        qgv[j] = sQRf[r * L::LDRF + c] * er;
        kgv[j] = sKRf[r * L::LDRF + c] * er;
      }
    }
    lds_barrier();  // region X (A/P operands) is dead from here on
    if (!F32 && wide) {
#pragma unroll
      for (int j = 0; j < NRB; ++j) {
        const int idx = tid + kThreads * j;
        if (idx < C * DK) {
          const int r = idx / DK, c = idx % DK;
          st_op<F32>(sQG + r * LDR + c, qgv[j]);
          st_op<F32>(sKGT + tidx<C, LDT>(c, r), kgv[j]);
        }
      }
    }
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
          if (isP) st_op<F32>(sP + row * LDC + col, row >= col ? acc[jj][r] : 0.f);
          else sA[row * LDA + col] = row > col ? sBeta[row] * acc[jj][r] : 0.f;
        }
      }
    }
    // upper tiles of P are zero (P.U runs over whole 32-token steps)
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int row = idx / C, col = idx - row * C;
      if ((col >> 4) > (row >> 4)) st_op<F32>(sP + row * LDC + col, 0.f);
    }
    lds_barrier();

    // ---- stage 3: T = (I + A)^-1 ------------------------------------------------
    // diagonal 16x16 blocks by forward substitution: wave 0, lane = (block, column)
    if (wave == 0) {
      const int a = gq;   // block
      const int j = li;   // column
      if (a < NT) {
        float col[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s0 = 0.f, s1 = 0.f;  // two partial sums shorten the dependency chain
#pragma unroll
          for (int m = 0; m < i; ++m) {
            const float t = sA[(16 * a + i) * LDA + 16 * a + m] * col[m];
            if (m & 1) s1 += t; else s0 += t;
          }
          col[i] = i == j ? 1.f : (i > j ? -(s0 + s1) : 0.f);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(16 * a + i) * LDA + 16 * a + j] = col[i];
      }
    }
    lds_barrier();
    // off-diagonal blocks, one wave per block column b (fp32 matrix cores):
    //   T_ab = -T_aa * sum_{m=b}^{a-1} A_am T_mb,  a = b+1 .. NT-1 in order.
    // The blocks of column b stay in registers (C layout: element e of lane
    // (g, i) is row 4g+e, column i) and feed the next products as B operands,
    // with the contraction index k = 4g + s in sub-step s.
    if (wave < NT - 1) {
      const int bb = wave;
      f4 Tcol[NT];
#pragma unroll
      for (int e = 0; e < 4; ++e) Tcol[0][e] = sT[(16 * bb + 4 * gq + e) * LDA + 16 * bb + li];
#pragma unroll
      for (int d = 1; d < NT; ++d) {
        const int a = bb + d;
        if (a < NT) {
          f4 X = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int md = 0; md < d; ++md) {  // m = bb + md
            const int m = bb + md;
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
              X = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * a + li) * LDA + 16 * m + 4 * gq + s4],
                                                       Tcol[md][s4], X, 0, 0, 0);
          }
          f4 Y = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            Y = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * a + li) * LDA + 16 * a + 4 * gq + s4], X[s4], Y,
                                                     0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            Tcol[d][e] = -Y[e];
            sT[(16 * a + 4 * gq + e) * LDA + 16 * bb + li] = -Y[e];
          }
        }
      }
    }
    lds_barrier();
    // Tb = T diag(beta), zero above the block diagonal
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int row = idx / C, col = idx - row * C;
      const float v = (col >> 4) > (row >> 4) ? 0.f : sT[row * LDA + col] * sBeta[col];
      st_op<F32>(sTB + row * LDC + col, v);
    }
    lds_barrier();

    // ---- stage 4: W = Tb (K e^G)  (all dk columns) and U~ = Tb V (own columns)
    f4 Wt[NT];
    if (wave < DK / 16) {
      const int ct = wave;
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        Wt[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < KSC; ++kt) {
          const int k0 = 32 * kt + 8 * gq;
          Frag<F32> fa, fb;
          frag_std<F32>(fa, sTB, 16 * rt + li, LDC, k0, k0 < C);
          frag_std_t<F32, C, LDT>(fb, sKGT, 16 * ct + li, k0, k0 < C);
          Wt[rt] = mma<F32>(fa, fb, Wt[rt]);
        }
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
          frag_std<F32>(fa, sTB, 16 * rt + li, LDC, k0, k0 < C);
          frag_std_t<F32, C, LDT>(fb, sVT, col0 + li, k0, k0 < C);
          U[rt] = mma<F32>(fa, fb, U[rt]);
        }
      }
    }
    lds_barrier();  // (k e^G)^T is dead: W goes in its place
    if (wave < DK / 16) {
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st_op<F32>(sW + (16 * rt + 4 * gq + r) * LDR + 16 * wave + li, Wt[rt][r]);
    }
    lds_barrier();

    // ---- stage 5: inter-chunk products and state update (own dv columns) -----
    // gate octets of this thread's epilogue items, loaded now so their latency
    // hides behind the products below
    Raw8<IN_BF16> gt[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + kThreads * j;
      const int tok = min(e / (DV / 8), n_valid - 1);
      raw_load<IN_BF16>(gt[j], p.gate, (((size_t)b * T + c0 + tok) * H + h) * DV + 8 * (e % (DV / 8)));
    }
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
          frag_perm<F32>(fa, sW, 16 * rt + li, LDR, 32 * ks, gq, true, 32 * ks + 16 < DK);
          ws = mma<F32>(fa, Sb[ks], ws);
        }
        U[rt] = U[rt] - ws;
      }
      // U as B operand over tokens, same permutation
      // (wide chunks, 16-bit operands: also the remainder U - Ub in fp16)
      const bool split = !F32 && wide;
      Frag<F32> Ub[KSC], Ul[KSC];
#pragma unroll
      for (int kt = 0; kt < KSC; ++kt) {
        float x[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = U[2 * kt][r];
          x[4 + r] = (2 * kt + 1 < NT) ? U[2 * kt + 1][r] : 0.f;
        }
        frag_from_f<F32>(Ub[kt], x);
        if constexpr (!F32) {
          if (split) {
#pragma unroll
            for (int e = 0; e < 8; ++e) Ul[kt].v[e] = (_Float16)(x[e] - (float)Ub[kt].v[e]);
          }
        }
      }
      // O = (Q e^G) S + P U
#pragma unroll
      for (int rt = 0; rt < NT; ++rt) {
        f4 o = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          Frag<F32> fa;
          frag_perm<F32>(fa, sQG, 16 * rt + li, LDR, 32 * ks, gq, true, 32 * ks + 16 < DK);
          o = mma<F32>(fa, Sb[ks], o);
        }
#pragma unroll
        for (int kt = 0; kt < KSC; ++kt) {
          if (32 * kt <= 16 * rt + 15) {
            Frag<F32> fa;
            frag_perm<F32>(fa, sP, 16 * rt + li, LDC, 32 * kt, gq, true, 32 * kt + 16 < C);
            o = mma<F32>(fa, Ub[kt], o);
            if (split) o = mma<F32>(fa, Ul[kt], o);
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
          frag_perm_t<F32, C, LDT>(fa, sKBT, 16 * t + li, 32 * kt, gq, 32 * kt + 16 < C);
          s = mma<F32>(fa, Ub[kt], s);
          if (split) s = mma<F32>(fa, Ul[kt], s);
        }
        S[t] = s;
      }
      // stage O for the epilogue (A / T space is dead by now)
#pragma unroll
      for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sO[(16 * rt + 4 * gq + r) * L::LDO + col0 + li] = O[rt][r];
    }
    // the next chunk's loads fly while the epilogue runs
    if (ci + 1 < nchunks) issue_loads(ci + 1);
    lds_barrier();

    // ---- epilogue: head-wise RMSNorm * sigmoid(gate) ----------------------------
    // item (token, dv octet): DV/8 consecutive lanes hold one token's row
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int e = tid + kThreads * j;
      if (e < NE) {
        const int tok = e / (DV / 8), oc = e % (DV / 8);
        const float4 a4 = *reinterpret_cast<const float4*>(sO + tok * L::LDO + 8 * oc);
        const float4 b4 = *reinterpret_cast<const float4*>(sO + tok * L::LDO + 8 * oc + 4);
        float x[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) ss += x[q] * x[q];
        ss = group_sum<DV / 8>(ss);
        const float rs = fast_rsq(ss * (1.0f / DV) + kRmsEps);
        float gv[8];
        raw_unpack<IN_BF16>(gt[j], gv);
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = x[q] * rs * sigmoidf_(gv[q]);
        if (tok < n_valid && p.o != nullptr) store8<OUT_BF16>(p.o, (((size_t)b * T + c0 + tok) * H + h) * DV + 8 * oc, x);
      }
    }
    lds_barrier();  // LDS is rewritten by the next chunk
  }

  // ---- final state and conv history ------------------------------------------
  const int tid = threadIdx.x;
  const int gq = (tid & 63) >> 4, li = tid & 15;
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
  p.A = a.decay_form == KDA_DECAY_K3 ? a.A : nullptr;
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

// The state entering every C-token chunk, fp32 operands throughout, no outputs.
template <int C, int D, bool IB>
int run_states(const kda_prefill_args& a, float* S_chunks, hipStream_t s) {
  using L = Smem<C, D, D, true>;
  static_assert(L::BYTES <= 160 * 1024, "fp32-operand chunk exceeds LDS");
  auto kern = prefill_kernel<C, D, D, IB, false, true>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, L::BYTES);
  if (e != hipSuccess) {
    set_error("chunk states: hipFuncSetAttribute failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  PrefillParams p = make_params(a);
  p.o = nullptr;
  p.S_T = nullptr;
  p.conv_out = nullptr;
  p.S_chunks = S_chunks;
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.B * a.H)), dim3(kThreads), L::BYTES, s, p);
  return check_launch("chunk states");
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
  p.A = a.decay_form == KDA_DECAY_K3 ? a.A : nullptr;
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
  if (a.workspace != nullptr && prefill_split_eligible(a)) return launch_prefill_split(a, s);
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

int launch_prefill_states(const kda_prefill_args& a, int chunk, float* S_chunks, hipStream_t s) {
  const bool ib = a.in_dtype == KDA_BF16;
  if (chunk != kStateChunk) {
    set_error("chunk states: chunk %d is not %d", chunk, kStateChunk);
    return KDA_E_UNSUPPORTED;
  }
  switch (a.dk) {
    case 16: return ib ? run_states<kStateChunk, 16, true>(a, S_chunks, s) : run_states<kStateChunk, 16, false>(a, S_chunks, s);
    case 32: return ib ? run_states<kStateChunk, 32, true>(a, S_chunks, s) : run_states<kStateChunk, 32, false>(a, S_chunks, s);
    case 64: return ib ? run_states<kStateChunk, 64, true>(a, S_chunks, s) : run_states<kStateChunk, 64, false>(a, S_chunks, s);
    case 128: return ib ? run_states<kStateChunk, 128, true>(a, S_chunks, s) : run_states<kStateChunk, 128, false>(a, S_chunks, s);
  }
  set_error("chunk states: head dim %d not instantiated", a.dk);
  return KDA_E_UNSUPPORTED;
}

}  // namespace kda
