// kda_prefill_split.hip -- two-kernel chunkwise KDA prefill for bf16 inputs,
// chunk 64, dk = dv = 128 (the K3 head shape: "Kimi K3.1 Pro vs gpt-oss-120b"
// and "Gemma 4 31B vs Kimi K3", component tables, row "Gated DeltaNet / KDA").
//
// Same algebra as the single-kernel path in kda_prefill.hip (the chunkwise
// WY / UT form of the KDA recurrence, 16-token decay tiles), split where the
// work stops being parallel:
//
//   intra_chunk_kernel  one workgroup (4 waves) per (b, h, chunk); every chunk
//     of every head at once.  Conv + SiLU + L2 normalisation of q and k,
//     chunk-local cumulative sum of g, then A, P and T = (I + A)^-1 on the
//     matrix cores.
//   inter_chunk_kernel  one workgroup (8 waves) per (b, h) walks the chunks in
//     order with the fp32 state in registers: v's conv + SiLU, then
//       U = T diag(beta) (V - (K e^G) S)        (= U~ - W S of the WY form)
//       O = (Q e^G) S + P U,   S <- e^{G_C} S + (K e^{G_C-G})^T U,
//     then RMSNorm * sigmoid(gate).
//   Taking V - (K e^G) S first keeps the cancellation between the new values
//   and the state's prediction in fp32 accumulators, and hands over K e^G in
//   fp16 instead of W and an fp32 U~.  V itself is not handed over: the
//   second kernel reads raw v (as many bytes as fp16 V) and convolves it, so
//   the first kernel never touches v.
//
// The first kernel hands the second its operands in a workspace laid out as
// matrix-core fragments (64 lanes x 16 bytes, lane order), so every operand
// moves with one coalesced 16-byte access per lane and reaches the matrix
// cores with no conversion or transpose.
//
// Lane layout in intra_chunk_kernel: wave a owns the 16-token tile a; lane
// (g = lane / 16, i = lane % 16) holds token 16a + i and channels
// 32k + 8g + 0..7 of each 32-channel step k.  That is the operand layout of
// the 16x16x32 matrix-core instruction for products contracting over channels
// (A, P), the causal conv reads the previous tokens from lanes i-1 .. i-3
// (DPP row shifts), and the cumulative sum of g is a DPP scan over the row.
//
// State row order: the state lives in registers as accumulator tiles whose
// row 4g + e of tile m is used directly as the contraction index of the next
// products.  Register row R = 16m + r holds channel perm_row(R), chosen so the
// eight contraction values of lane group g in step k are channels
// 32k + 8g + 0..7: W and Q e^G fragments are then plain row-major pieces.
// S0 and S_T stay in natural order in memory.
//
// Precision: fp16 matrix-core operands, fp32 accumulation, fp32 state and
// output.  A chunk in which some 16-token tile decays by more than e^8 in some
// channel ("wide" chunk: the in-tile column factors e^{rho_a - G} leave fp16's
// range, reaching e^80 at K3's bound of -5 per token) takes two extra steps:
//   * the diagonal 16x16 blocks of A and P run on the fp32 matrix-core
//     instruction with fp32 column factors (fp32 holds e^{+-80});
//   * U enters the P U and (K e^{G_C-G})^T U products as an fp16 pair
//     hi + lo (about 22 significant bits): when the state forgets nearly
//     everything per token, S_T and o are dominated by the last tokens' U
//     and a single fp16 rounding of U is visible at the 2e-2 x RMS bound.
// Every other operand keeps fp16: all other decay factors are <= 1, so their
// rounding is relative to entries of at most unit size.
#include "kda_device.h"
#include "kda_internal.h"

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

namespace kda {

namespace {

constexpr int kC = 64;          // chunk
constexpr int kD = 128;         // dk = dv
constexpr int kNCh = 3 * kD;    // conv channels of one head (q | k | v)
constexpr float kSpanF16 = 8.0f;

// ---- workspace block of one (b, h, chunk), bytes ------------------------------
constexpr int kFrag = 1024;                  // 64 lanes x 16 bytes
constexpr int WS_KG = 0;                     // -(K e^G) fragments (rt, k)      16
constexpr int WS_QG = WS_KG + 16 * kFrag;    // Q e^G    fragments (rt, k)      16
constexpr int WS_KB = WS_QG + 16 * kFrag;    // (K e^{G_C-G})^T fragments (m, k') 16
constexpr int WS_P = WS_KB + 16 * kFrag;     // P        fragments (rt, k'), k' <= rt/2: 6
constexpr int WS_TB = WS_P + 6 * kFrag;      // T diag(beta) fragments, as P: 6
constexpr int WS_GAM = WS_TB + 6 * kFrag;    // e^{G_C} in state row order, 128 fp32; int "wide" flag at +512
constexpr int WS_WIDE = WS_GAM + 512;        // int: the chunk is wide (see the file header)
constexpr int WS_STAGE = WS_GAM + 4 * kFrag; // bytes the second kernel stages through LDS (64 KiB)
constexpr int WS_CHUNK = WS_STAGE;           // 64 KiB per chunk
constexpr size_t kSlabBytesMax = (size_t)16 << 30;  // workspace cap for the chunk blocks

__device__ __forceinline__ int p_frag(int rt, int kp) { return rt < 2 ? rt : 2 * rt - 2 + kp; }

// channel held by register row R of the state
__device__ __forceinline__ int perm_row(int R) {
  const int m = R >> 4, r = R & 15;
  return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3);
}

struct SplitParams {
  int B, T, H;
  int c_begin, n_chunks;  // chunks [c_begin, c_begin + n_chunks) of this launch
  const void* q;
  const void* k;
  const void* v;
  const float* conv_w;
  const void* g;
  const void* beta;
  const void* gate;
  const float* S_in;      // state entering chunk c_begin, or null (zeros)
  const void* conv_in;
  void* o;
  float* S_out;           // state after the last chunk, or null
  void* conv_out;         // raw conv history after the last token, or null
  unsigned char* ws;      // n_chunks * B * H chunk blocks
  const float* A;         // [H, dk]: g and beta are K3's logits (see k3_decay); null: given directly
  // A second copy of the recurrence over the same chunk blocks (inter-chunk
  // grid 2 * B * H, copy 1 in blocks B*H ..): it starts from the identity and
  // writes only its final state to S_out2.  o may be null (no outputs).
  float* S_out2;
  // Workspace addressing: the block of chunk c of head bh is block
  // bh * ws_stride + (c - ws_first) (0, 0: ws_stride = n_chunks, ws_first =
  // c_begin, the blocks of this launch alone).
  int ws_stride, ws_first;
  // One recurrence launch over every slab (see run_split): before copying the
  // first chunk of slab s the copying waves wait for slab_ready[s] (set after
  // that slab's intra-chunk kernel), a sync block laid out as kSync* says;
  // slabs are laid out as slab_range does (ramp leading slabs of kFirstChunks
  // << s chunks, then slab_per each).  A workgroup whose wait expires stops
  // before that chunk: it leaves its state after the chunks it finished in
  // S_out (required; S_in, which S_out may alias, is no longer needed then), or
  // nothing if it finished none, writes no conv_out, and records the chunks it
  // finished in the block's progress entry.
  const unsigned* slab_ready;
  int slab_ramp, slab_per;
  // Second launch after every slab is done: workgroup bh continues from chunk
  // c_begin + resume[bh] (from the state left in S_out, or from S_in when
  // resume[bh] == 0), or exits at once when resume[bh] == n_chunks.
  const int* resume;
};

// Slab lengths of the pipeline (see plan_slabs).
constexpr int kPipeChunks = 64;
constexpr int kFirstChunks = 32;

// Sync block of a one-launch recurrence (32-bit words): a flag per slab, the
// bound of each wait (100 MHz real-time counter ticks), the chunks each (b, h)
// finished.  Only pointers the kernel holds anyway lead to it.
constexpr int kMaxSlabs = 4096;
constexpr int kSyncBound = kMaxSlabs;
constexpr int kSyncProgress = kMaxSlabs + 64;
constexpr size_t sync_bytes(int nbh) { return ((size_t)kSyncProgress + nbh) * 4; }

// Bounded waits on slab_ready (default 20 ms).  The intra-chunk kernels are
// queued before the recurrence launch, on streams of their own, and normally
// run ahead of it; a wait this long means they cannot run beside it (kernels
// serialised, e.g. by a profiler collecting counters, or other work holding
// their compute units).  The workgroup then stops, counts the miss in
// g_wait_timeouts, and the resume launch finishes its work.
constexpr unsigned kReadyWaitUs = 20000;
__device__ unsigned g_wait_timeouts;

// DPP move inside rows of 16 lanes; lanes with no source or outside the bank
// mask read 0.
template <int CTRL, int BANK>
__device__ __forceinline__ float dppf(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, BANK, false));
}

__device__ __forceinline__ float bf16_at(const uint4& u, int e) {
  const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
  return (e & 1) ? bf16hi(w) : bf16lo(w);
}

__device__ __forceinline__ half8 to_half8(const float* x) {
  half8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
  return h;
}

// a + w1 * t_{-1} + w2 * t_{-2} + w3 * t_{-3} for a causal conv along the
// 16 lanes of a row: t_{-j} at lane i is z_j of lane (i - j) mod 16 (row
// rotation by j), where z_j is the lane's halo value y in lanes 16 - j .. 15
// and its own value x elsewhere.  The three selects come first so that each
// rotated read is two instructions after the write of its source (the DPP
// read-after-write wait), and each rotation is folded into its multiply-add,
// so no rotated copy occupies a register.
__device__ __forceinline__ float conv3_dpp(float a, float x, float y, float w1, float w2, float w3) {
  float z1, z2, z3;
  asm("v_cndmask_b32_e64 %0, %4, %5, %6\n\t"
      "v_cndmask_b32_e64 %1, %4, %5, %7\n\t"
      "v_cndmask_b32_e64 %2, %4, %5, %8\n\t"
      "v_fmac_f32_dpp %3, %0, %9 row_ror:1 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %1, %10 row_ror:2 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %2, %11 row_ror:3 row_mask:0xf bank_mask:0xf"
      : "=&v"(z1), "=&v"(z2), "=&v"(z3), "+v"(a)
      : "v"(x), "v"(y), "s"(0x8000800080008000ull), "s"(0xC000C000C000C000ull), "s"(0xE000E000E000E000ull),
        "v"(w1), "v"(w2), "v"(w3));
  return a;
}

// Causal depthwise conv (kernel 4) + SiLU of one tensor for this lane's token
// and 32 channels.  `cur` are the raw token's channels, `hal` the raw values of
// the token 16 positions earlier (used in lanes 13..15 only: the three tokens
// before the tile; zero when there are none), `cw` this lane's taps (32k + e
// indexing).  Token t - j is lane i - j of the row, or for i < j the halo of
// lane 16 + i - j: a rotation by j of the row in which lanes 16 - j .. 15
// offer their halo instead of their own token.
// `sink(kp, x8)` takes the 8 outputs of channel group kp.
// LOG2E: the taps are pre-multiplied by log2(e), so the conv gives
// t = log2(e) a and SiLU(a) = a / (1 + 2^-t) is returned as log2(e) SiLU(a)
// = t / (1 + 2^-t), one multiply fewer; the L2 normalisation that follows for
// q and k removes the constant factor (its epsilon is scaled to match).
template <bool LOG2E, typename Sink>
__device__ __forceinline__ void conv_silu(const uint4 (&cur)[4], const uint4 (&hal)[4], const float4* cw,
                                          Sink&& sink) {
#pragma unroll
  for (int kp = 0; kp < 4; ++kp) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xc = bf16_at(cur[kp], e);
      const float y = bf16_at(hal[kp], e);
      const float4 w = cw[32 * kp + e];
      const float a = conv3_dpp(w.w * xc, xc, y, w.z, w.y, w.x);
      if constexpr (LOG2E) x[e] = a * fast_rcp(1.0f + __builtin_amdgcn_exp2f(-a));
      else x[e] = siluf_(a);
    }
    sink(kp, x);
  }
}

// Scale x[32] to unit L2 norm over the token's 128 channels (held by lanes
// i, i+16, i+32, i+48), times `extra`; x holds log2(e) times the SiLU outputs
// (see conv_silu), so the epsilon is log2(e)^2 times the definition's.
__device__ __forceinline__ void l2norm128(float (&x)[32], float extra) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < 32; ++c) ss += x[c] * x[c];
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  const float r = fast_rsq(ss + kL2Eps * kLog2e * kLog2e) * extra;
#pragma unroll
  for (int c = 0; c < 32; ++c) x[c] *= r;
}

__device__ __forceinline__ void ld8f(const float* p, float* x) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// transposed [channel][token] fp16 arrays: 64 tokens + 8 pad per row, 8-token
// granules XOR-swizzled by row / 16 to spread the per-token stores over banks
constexpr int kLDT = kC + 8;
__device__ __forceinline__ int tix(int row, int tok) {
  return row * kLDT + ((((tok >> 3) ^ (row >> 4)) & 7) << 3) + (tok & 7);
}

// ---- LDS of intra_chunk_kernel (bytes) ----------------------------------------
struct ALds {
  static constexpr int LDA = kC + 4;                  // fp32 A / T rows
  static constexpr int LDB = kC + 8;                  // fp16 T diag(beta) rows
  static constexpr int TOT = 0;                       // [4][128] fp32: sum of g over each tile
  static constexpr int BETA = TOT + 4 * kD * 4;       // [64] fp32
  static constexpr int FLAG = BETA + kC * 4;          // int
  static constexpr int R1 = FLAG + 16;
  // R1, until the A / P products: column operands of tiles 0..2 and (K e^{G_C-G})^T
  static constexpr int CC = R1;                       // [3 tiles][4 k] fragments
  static constexpr int KBT = CC + 3 * 4 * kFrag;      // [128][kLDT] fp16
  static constexpr int R1_A = KBT + kD * kLDT * 2;
  // R1, afterwards: A (then T on its diagonal blocks) and T diag(beta)
  static constexpr int AM = R1;                       // [64][LDA] fp32
  static constexpr int TB = AM + kC * LDA * 4;        // [64][LDB] fp16
  static constexpr int R1_B = TB + kC * LDB * 2;
  static constexpr int R2 = ((R1_A > R1_B ? R1_A : R1_B) + 15) / 16 * 16;
  // R2: conv taps of q and k and per-channel decay factors
  static constexpr int CW = R2;                       // [256] float4
  static constexpr int ERHO = CW + 2 * kD * 16;       // [4][128] e^{rho_a}
  static constexpr int ETOT = ERHO + 4 * kD * 4;      // [4][128] e^{tot_a}
  static constexpr int EKB = ETOT + 4 * kD * 4;       // [4][128] e^{G_C - rho_a - tot_a}
  static constexpr int FOFF = EKB + 4 * kD * 4;       // [3][128] e^{rho_a - rho_{b+1}}: (2,0) (3,0) (3,1)
  static constexpr int BYTES = FOFF + 3 * kD * 4;
};

// ---------------------------------------------------------------------------
// intra_chunk_kernel: grid n_chunks * B * H, block 256
// ---------------------------------------------------------------------------
// K3: g and beta are K3's logits (p.A holds A), see k3_decay
template <bool K3>
__global__ __launch_bounds__(256, 3) void intra_chunk_kernel(SplitParams p) {
  using L = ALds;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sTot = reinterpret_cast<float*>(smem + L::TOT);
  float* sBeta = reinterpret_cast<float*>(smem + L::BETA);
  int* sFlag = reinterpret_cast<int*>(smem + L::FLAG);
  float4* sCW = reinterpret_cast<float4*>(smem + L::CW);
  float* sERho = reinterpret_cast<float*>(smem + L::ERHO);
  float* sETot = reinterpret_cast<float*>(smem + L::ETOT);
  float* sEKb = reinterpret_cast<float*>(smem + L::EKB);
  float* sFoff = reinterpret_cast<float*>(smem + L::FOFF);
  half8* sCC = reinterpret_cast<half8*>(smem + L::CC);
  _Float16* sKBT = reinterpret_cast<_Float16*>(smem + L::KBT);
  float* sAM = reinterpret_cast<float*>(smem + L::AM);
  _Float16* sTB = reinterpret_cast<_Float16*>(smem + L::TB);
  constexpr int LDA = L::LDA, LDB = L::LDB;

  const int H = p.H, T = p.T;
  const int nc = p.n_chunks;
  const int bh = blockIdx.x / nc;
  const int c = p.c_begin + (blockIdx.x - bh * nc);
  const int b = bh / H, h = bh - b * H;
  const int c0 = c * kC;
  const int n_valid = min(kC, T - c0);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // token tile
  const int lane = tid & 63, g = lane >> 4, i = lane & 15;
  const int tok = 16 * wave + i;
  const bool valid = tok < n_valid;
  const int wstride = p.ws_stride > 0 ? p.ws_stride : nc;
  const int wfirst = p.ws_stride > 0 ? p.ws_first : p.c_begin;
  unsigned char* wsb = p.ws + ((size_t)bh * wstride + (c - wfirst)) * WS_CHUNK;

  // ---- loads: this lane's token (clamped) and the tile's halo ------------------
  const size_t cch = (size_t)H * kNCh;
  const size_t row = ((size_t)b * T + c0 + min(tok, n_valid - 1)) * H + h;
  const int th = c0 + 16 * wave - 16 + max(i, 13);  // lanes 13..15: tokens before the tile
  const bool h_in = th >= 0;
  // the tile has earlier tokens (the same for lanes 13..15: c0 + 16 wave is a
  // multiple of 16), in the sequence or in the conv history
  const bool hok = c0 + 16 * wave > 0 || p.conv_in != nullptr;
  const size_t hrow = ((size_t)b * T + min(max(th, 0), T - 1)) * H + h;
  const size_t hist = ((size_t)b * 3 + (3 + max(th, -3))) * cch;  // conv_in row when th < 0
  const bool from_hist = !h_in && p.conv_in != nullptr;
  // Raw q / k (this token and the halo) of one tensor; k's are loaded while q
  // is processed.
  const uint16_t* ci16 = reinterpret_cast<const uint16_t*>(p.conv_in);
  auto load_raw = [&](const void* src, int part, uint4 (&r)[4], uint4 (&hr)[4]) {
    const uint16_t* x16 = reinterpret_cast<const uint16_t*>(src);
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      const int cl = 32 * kp + 8 * g;
      r[kp] = ld_nt(x16 + row * kD + cl);
      const uint16_t* ph =
          from_hist ? ci16 + hist + (size_t)part * H * kD + (size_t)h * kD + cl : x16 + hrow * kD + cl;
      hr[kp] = *reinterpret_cast<const uint4*>(ph);
    }
  };
  // no earlier tokens (a wave-uniform case): the halo is zero
  auto mask_halo = [&](uint4 (&hr)[4]) {
    if (!hok) {
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) hr[kp] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 rg[4], ra[4], ha[4], rb[4], hb[4];
  {
    const uint16_t* g16 = reinterpret_cast<const uint16_t*>(p.g);
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) rg[kp] = ld_nt(g16 + row * kD + 32 * kp + 8 * g);
  }
  load_raw(p.q, 0, rb, hb);  // q's raw values land during the decay-factor phase
  float beta_v = valid ? bf16_to_f(reinterpret_cast<const uint16_t*>(p.beta)[row]) : 0.f;
  if constexpr (K3) beta_v = valid ? sigmoidf_(beta_v) : 0.f;

  // conv taps of this head's q and k (times log2(e), see conv_silu), per-token
  // beta, fp16-range flag
  {
    const int ch = tid;  // 256 threads: q channels, then k channels
    const size_t gch = ch < kD ? (size_t)h * kD + ch : (size_t)H * kD + (size_t)h * kD + (ch - kD);
    const float4 w = *reinterpret_cast<const float4*>(p.conv_w + gch * 4);
    sCW[ch] = make_float4(w.x * kLog2e, w.y * kLog2e, w.z * kLog2e, w.w * kLog2e);
  }
  if (g == 0) sBeta[tok] = beta_v;
  if (tid == 0) *sFlag = 0;

  // ---- chunk-local cumulative sum of g: DPP scan over the tile, tile sums -----
  float s[32];
#pragma unroll
  for (int kp = 0; kp < 4; ++kp) {
    float av[8];  // K3's decay: A of this lane's channels 32kp + 8g + 0..7
    if constexpr (K3) ld8f(p.A + (size_t)h * kD + 32 * kp + 8 * g, av);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = valid ? bf16_at(rg[kp], e) : 0.f;
      if constexpr (K3) x = valid ? k3_decay(x, fast_exp(av[e])) : 0.f;
      x += dppf<0x111, 0xF>(x);
      x += dppf<0x112, 0xF>(x);
      x += dppf<0x114, 0xF>(x);
      x += dppf<0x118, 0xF>(x);
      s[8 * kp + e] = x;   // G - rho_a at this token
    }
  }
  if (i == 15) {
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      float* d = sTot + wave * kD + 32 * kp + 8 * g;
      *reinterpret_cast<float4*>(d) = make_float4(s[8 * kp], s[8 * kp + 1], s[8 * kp + 2], s[8 * kp + 3]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(s[8 * kp + 4], s[8 * kp + 5], s[8 * kp + 6], s[8 * kp + 7]);
    }
  }
  lds_barrier();

  // ---- per-channel decay factors of the chunk -----------------------------------
  {
    bool span_big = false;
    for (int idx = tid; idx < 4 * kD; idx += 256) {
      const int a = idx >> 7, ch = idx & (kD - 1);
      const float t0 = sTot[ch], t1 = sTot[kD + ch], t2 = sTot[2 * kD + ch], t3 = sTot[3 * kD + ch];
      const float ta = a == 0 ? t0 : a == 1 ? t1 : a == 2 ? t2 : t3;
      const float rho = (a > 0 ? t0 : 0.f) + (a > 1 ? t1 : 0.f) + (a > 2 ? t2 : 0.f);
      const float gc = t0 + t1 + t2 + t3;
      sERho[idx] = fast_exp(rho);
      sETot[idx] = fast_exp(ta);
      sEKb[idx] = fast_exp(gc - rho - ta);
      span_big |= -ta > kSpanF16;
    }
    for (int idx = tid; idx < 3 * kD; idx += 256) {
      const int pr = idx >> 7, ch = idx & (kD - 1);
      const float t1 = sTot[kD + ch], t2 = sTot[2 * kD + ch];
      sFoff[idx] = fast_exp(pr == 0 ? t1 : pr == 1 ? t1 + t2 : t2);
    }
    if (tid < kD) {
      const int ch = perm_row(tid);
      const float gc = sTot[ch] + sTot[kD + ch] + sTot[2 * kD + ch] + sTot[3 * kD + ch];
      reinterpret_cast<float*>(wsb + WS_GAM)[tid] = fast_exp(gc);
    }
    if (__any(span_big) && lane == 0) atomicOr(sFlag, 1);
  }
  lds_barrier();
  // wide chunk: fp32 diagonal blocks of A and P here, split U in the recurrence
  const bool wide = __builtin_amdgcn_readfirstlane(*sFlag) != 0;
  if (tid == 0) *reinterpret_cast<int*>(wsb + WS_WIDE) = wide ? 1 : 0;

  // e^{G - rho_a} of this lane's channels
  float E[32];
#pragma unroll
  for (int c2 = 0; c2 < 32; ++c2) E[c2] = fast_exp(s[c2]);

  // ---- q: rows of P and Q e^G -----------------------------------------------------
  half8 QrowF[4];
  {
    float x[32];
    mask_halo(hb);
    conv_silu<true>(rb, hb, sCW + 8 * g, [&](int kp, const float* x8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * kp + e] = x8[e];
    });
    load_raw(p.k, 1, ra, ha);  // k's raw values land during the rest of q's work
    __builtin_amdgcn_sched_barrier(0);
    l2norm128(x, fast_rsq((float)kD));
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      float er[8], qr[8], qg[8];
      ld8f(sERho + wave * kD + 32 * kp + 8 * g, er);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qr[e] = x[8 * kp + e] * E[8 * kp + e];
        qg[e] = qr[e] * er[e];
      }
      // a wide chunk keeps q's normalised value here: the k phase applies the
      // factor in fp32 for the diagonal blocks (it may underflow fp16 while the
      // in-tile column factor makes up for it), then forms the fp16 operand
      if (wide) {
        QrowF[kp] = to_half8(&x[8 * kp]);
      } else {
        QrowF[kp] = to_half8(qr);
      }
      st_nt(wsb + WS_QG + ((wave * 4 + kp) * 64 + lane) * 16, to_half8(qg));
    }
  }
  // ---- k: rows and columns of A / P, K e^G, K e^{G_C - G} ---------------------------
  // Wide chunks form the diagonal blocks (D[j][r], j, r in this wave's tile) here
  // on the fp32 instruction: column k e^{rho_a - G}, rows k e^{G - rho_a} and
  // q e^{G - rho_a} in fp32 (q from its fp16 normalised value).  Instruction
  // (kp, e) contracts over channels 32kp + 8g + e, g = 0..3.
  // Other chunks form them here too, on the fp16 instruction, so the column
  // operand k e^{rho_a - G} is never held.
  half8 KrowF[4];
  f4 diagA = f4{0.f, 0.f, 0.f, 0.f}, diagP = f4{0.f, 0.f, 0.f, 0.f};
  {
    float x[32];
    mask_halo(ha);
    conv_silu<true>(ra, ha, sCW + kD + 8 * g, [&](int kp, const float* x8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * kp + e] = x8[e];
    });
    __builtin_amdgcn_sched_barrier(0);
    l2norm128(x, 1.0f);
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
      float er[8], et[8], ek[8], kr[8], cd[8], cc[8], kb[8], kg[8];
      ld8f(sERho + wave * kD + 32 * kp + 8 * g, er);
      ld8f(sETot + wave * kD + 32 * kp + 8 * g, et);
      ld8f(sEKb + wave * kD + 32 * kp + 8 * g, ek);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xe = x[8 * kp + e], ee = E[8 * kp + e];
        kr[e] = xe * ee;                 // k e^{G - rho_a}
        cd[e] = xe * fast_rcp(ee);       // k e^{rho_a - G}
        cc[e] = cd[e] * et[e];           // k e^{rho_{a+1} - G}
        kb[e] = cc[e] * ek[e];           // k e^{G_C - G}
        kg[e] = -kr[e] * er[e];          // -k e^{G}
      }
      KrowF[kp] = to_half8(kr);
      if (wide) {
        float qr[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[e] = (float)QrowF[kp][e] * E[8 * kp + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          diagA = __builtin_amdgcn_mfma_f32_16x16x4f32(cd[e], kr[e], diagA, 0, 0, 0);
          diagP = __builtin_amdgcn_mfma_f32_16x16x4f32(cd[e], qr[e], diagP, 0, 0, 0);
        }
        QrowF[kp] = to_half8(qr);
      } else {
        const half8 cdf = to_half8(cd);
        diagA = mma_f16(cdf, KrowF[kp], diagA);
        diagP = mma_f16(cdf, QrowF[kp], diagP);
      }
      st_nt(wsb + WS_KG + ((wave * 4 + kp) * 64 + lane) * 16, to_half8(kg));
      if (wave < 3) sCC[(wave * 4 + kp) * 64 + lane] = to_half8(cc);
#pragma unroll
      for (int e = 0; e < 8; ++e) sKBT[tix(32 * kp + 8 * g + e, tok)] = (_Float16)kb[e];
    }
  }
  lds_barrier();

  // ---- A^T and P^T blocks (b, a), b <= a: D[j][r] = sum_c col_b[j][c] row_a[r][c] --
  // The column operand of an earlier tile b is scaled by e^{rho_a - rho_{b+1}} <= 1
  // (exact 1 for b = a - 1).
  f4 accA[4], accP[4];
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    accA[bb] = f4{0.f, 0.f, 0.f, 0.f};
    accP[bb] = f4{0.f, 0.f, 0.f, 0.f};
    if (bb == wave) {
      accA[bb] = diagA;
      accP[bb] = diagP;
    } else if (bb < wave) {
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) {
        half8 fa = sCC[(bb * 4 + kp) * 64 + lane];
        if (bb < wave - 1) {
          const int pr = wave == 2 ? 0 : 1 + bb;
          float fv[8];
          ld8f(sFoff + pr * kD + 32 * kp + 8 * g, fv);
#pragma unroll
          for (int e = 0; e < 8; ++e) fa[e] = (_Float16)((float)fa[e] * fv[e]);
        }
        accA[bb] = mma_f16(fa, KrowF[kp], accA[bb]);
        accP[bb] = mma_f16(fa, QrowF[kp], accP[bb]);
      }
    }
  }
  // (K e^{G_C - G})^T fragments (m, k'): wave w takes m = 2w, 2w + 1
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int m = 2 * wave + mm;
    const int rw = perm_row(16 * m + i);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      const half4 lo = *reinterpret_cast<const half4*>(sKBT + tix(rw, 32 * kp + 4 * g));
      const half4 hi = *reinterpret_cast<const half4*>(sKBT + tix(rw, 32 * kp + 16 + 4 * g));
      st_nt(wsb + WS_KB + ((m * 2 + kp) * 64 + lane) * 16, half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
  }
  lds_barrier();  // R1 is rewritten from here on

  // A (beta_r scaled, strictly lower) into AM; P fragments to the workspace
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    if (bb <= wave) {
      float4 w4;
      w4.x = 16 * bb + 4 * g + 0 < tok ? beta_v * accA[bb][0] : 0.f;
      w4.y = 16 * bb + 4 * g + 1 < tok ? beta_v * accA[bb][1] : 0.f;
      w4.z = 16 * bb + 4 * g + 2 < tok ? beta_v * accA[bb][2] : 0.f;
      w4.w = 16 * bb + 4 * g + 3 < tok ? beta_v * accA[bb][3] : 0.f;
      *reinterpret_cast<float4*>(sAM + tok * LDA + 16 * bb + 4 * g) = w4;
    }
  }
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    if (2 * kp <= wave) {
      float pv[8];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh) {
        const int bb = 2 * kp + sh;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = bb == 0 ? accP[0][e] : bb == 1 ? accP[1][e] : bb == 2 ? accP[2][e] : accP[3][e];
          pv[4 * sh + e] = (bb <= wave && 16 * bb + 4 * g + e <= tok) ? v : 0.f;
        }
      }
      st_nt(wsb + WS_P + (p_frag(wave, kp) * 64 + lane) * 16, to_half8(pv));
    }
  }
  lds_barrier();

  // ---- T = (I + A)^-1: diagonal 16x16 blocks by forward substitution --------------
  // wave 0, lane = (block g, column i); T_aa replaces A_aa in AM
  if (wave == 0) {
    const int a = g, j = i;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) {
        const float t = sAM[(16 * a + r) * LDA + 16 * a + m] * col[m];
        if (m & 1) s1 += t; else s0 += t;
      }
      col[r] = r == j ? 1.f : (r > j ? -(s0 + s1) : 0.f);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sAM[(16 * a + r) * LDA + 16 * a + j] = col[r];
  }
  lds_barrier();
  // off-diagonal blocks, wave bb = block column (fp32 matrix cores):
  //   T_ab = -T_aa sum_{m=b}^{a-1} A_am T_mb, a = b+1 .. 3; stored as T diag(beta) in fp16.
  // Wave 3 writes the diagonal blocks of T diag(beta) and the zero blocks the
  // W / U~ products read.
  if (wave < 3) {
    const int bb = wave;
    const float bcol = sBeta[16 * bb + i];
    f4 Tcol[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) Tcol[0][e] = sAM[(16 * bb + 4 * g + e) * LDA + 16 * bb + i];
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      const int a = bb + d;
      if (a < 4) {
        f4 X = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int md = 0; md < d; ++md) {
          const int m = bb + md;
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            X = __builtin_amdgcn_mfma_f32_16x16x4f32(sAM[(16 * a + i) * LDA + 16 * m + 4 * g + s4], Tcol[md][s4], X,
                                                     0, 0, 0);
        }
        f4 Y = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          Y = __builtin_amdgcn_mfma_f32_16x16x4f32(sAM[(16 * a + i) * LDA + 16 * a + 4 * g + s4], X[s4], Y, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Tcol[d][e] = -Y[e];
          sTB[(16 * a + 4 * g + e) * LDB + 16 * bb + i] = (_Float16)(-Y[e] * bcol);
        }
      }
    }
  } else {
    for (int idx = lane; idx < 4 * 256; idx += 64) {
      const int a = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
      sTB[(16 * a + r) * LDB + 16 * a + cc] =
          (_Float16)(sAM[(16 * a + r) * LDA + 16 * a + cc] * sBeta[16 * a + cc]);
    }
    for (int idx = lane; idx < 2 * 256; idx += 64) {
      const int a = 2 * (idx >> 8), r = (idx >> 4) & 15, cc = idx & 15;  // blocks (0,1), (2,3)
      sTB[(16 * a + r) * LDB + 16 * (a + 1) + cc] = (_Float16)0.f;
    }
  }
  lds_barrier();

  // ---- hand-over: T diag(beta) as row-operand fragments ------------------------------
  // T diag(beta) fragment (rt, k'), like P: lane (g, i) holds row 16rt + i at
  // tokens 32k' + 4g + 0..3 and 32k' + 16 + 4g + 0..3; wave w writes fragments w, w + 4
#pragma unroll
  for (int f = wave; f < 6; f += 4) {
    const int rt = f < 2 ? f : (f - 2) / 2 + 2, kp = f < 2 ? 0 : (f - 2) & 1;
    const half4 lo = *reinterpret_cast<const half4*>(sTB + (16 * rt + i) * LDB + 32 * kp + 4 * g);
    const half4 hi = *reinterpret_cast<const half4*>(sTB + (16 * rt + i) * LDB + 32 * kp + 16 + 4 * g);
    st_nt(wsb + WS_TB + (f * 64 + lane) * 16, half8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  }
}

// ---------------------------------------------------------------------------
// inter_chunk_kernel: grid B * H, block 512 (8 waves), one workgroup per (b, h)
//
//   waves 0..3 ("math"): wave w owns dv columns 32w .. 32w+31 and the state
//     columns with them; per chunk it forms V = SiLU(conv(v)) of its columns,
//     runs U = T diag(beta) (V - (K e^G) S), O = (Q e^G) S + P U and
//     S <- e^{G_C} S + (K e^{G_C-G})^T U on the matrix cores and leaves O in
//     LDS.  Its only memory accesses are LDS reads and the raw v of the next
//     chunk, so it never waits behind other traffic.
//   waves 4..7 ("epilogue"): wave 4 + r copies a quarter of the next chunk's
//     operands into LDS and takes token tile r of the previous chunk's O:
//     RMSNorm over its rows * sigmoid(gate), stores (16-byte pieces; the gate
//     is loaded a chunk ahead).  O passes through LDS in fp16: it is only
//     normalised and gated afterwards, so its rounding (2^-11 relative) stays
//     far below the tolerance.
// The epilogue of chunk j-1 runs beside the products of chunk j.  Two barriers
// per chunk: B1 (chunk j's operands have landed; O(j-1) is complete) and B2
// (the epilogue waves have read O(j-1), so the math waves may overwrite it).
// ---------------------------------------------------------------------------
constexpr int kStageQ = WS_STAGE / kFrag / 4;  // fragment slots of each copying wave per chunk
static_assert(WS_STAGE % (4 * kFrag) == 0, "staged part must split evenly over four waves");
constexpr int kStageFrags = WS_GAM / kFrag + 1;  // fragments holding data: up to e^{G_C}, not its padding

// LDS of inter_chunk_kernel as three separate objects: the compiler then knows
// that the direct-to-LDS copy into one staging buffer never aliases reads of
// the other or of O, and waits for the copies only where the kernel says so.
__shared__ __attribute__((aligned(16))) unsigned char g_stage0[WS_STAGE];  // operands of even chunks
__shared__ __attribute__((aligned(16))) unsigned char g_stage1[WS_STAGE];  // operands of odd chunks
// O of a chunk, fp16: block (rt, w) holds math wave w's accumulator tile rt in
// C layout, lane (g, i) at g * kOGrp + i * 16 + (i / 8) * 16.  The padding makes
// the epilogue's transposing 4-byte reads hit 64 different banks.
constexpr int kOGrp = 288;
constexpr int kOBlk = 4 * kOGrp;
__shared__ __attribute__((aligned(16))) unsigned char g_O[16 * kOBlk];
// conv taps of the head's v channels
__shared__ float4 g_vw[kD];
// scale of each math wave's columns of the O in g_O (see kRangeLimit)
__shared__ float g_Osig[4];
// the chunk before which the first copying wave stopped (-1: none)
__shared__ int g_dec;
// In place of a chunk's wide flag (WS_WIDE) in a staging buffer: the chunk was
// not copied, the workgroup stops before it.
constexpr int kStopFlag = 2;

// Range of the fp16 operands.  Each math wave keeps its columns of V, S, X, U
// and O divided by a power of two sigma (1 unless the values demand more):
// before a chunk, |V| <= sum_j |w_j| max|raw v| + 0.3 (SiLU's negative lobe) is
// bounded from the raw bf16 values, and sigma grows so that |V| / sigma and
// |S| / sigma stay below kRangeLimit, which leaves fp16 (max 65504) a factor
// 64 for X, U and O.  The recurrence is linear in (V, S), so the scaled state
// follows the same update; RMSNorm is applied to O = sigma * O~ in fp32, and
// S_T is written unscaled.  Sigma never shrinks within a launch.
constexpr float kRangeLimit = 1024.0f;

// Smallest power of two p with x / p <= kRangeLimit, at least `cur`.
__device__ __forceinline__ float grow_scale(float cur, float x) {
  if (!(x > kRangeLimit * cur)) return cur;
  int e;
  (void)__builtin_frexpf(x / kRangeLimit, &e);  // x / limit < 2^e
  return __builtin_ldexpf(1.0f, e);
}
static_assert(2 * WS_STAGE + 16 * kOBlk + kD * 16 <= 160 * 1024, "inter-chunk LDS exceeds 160 KiB");

// B operand of the 16x16x32 instruction that moves columns 16ct .. 16ct + 15
// of a row-operand tile into the C layout: lane (g, i) holds rows 8g .. 8g + 7
// of column i of the 32 x 16 matrix [k == i + 16 ct].
__device__ __forceinline__ half8 ident_frag(int g, int i, int ct) {
  half8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = 8 * g + e == i + 16 * ct ? (_Float16)1.0f : (_Float16)0.0f;
  return f;
}

template <int P>
__device__ __forceinline__ unsigned char* stage_buf() {
  if constexpr (P == 0) return g_stage0;
  else return g_stage1;
}

typedef __attribute__((address_space(3))) void lds_void;

// Copy one chunk's staged operands (61 fragments of 1 KiB) from the workspace
// into staging buffer P with direct-to-LDS loads (no registers): wave w moves
// fragments w, w + 4, ...; lane l's 16 bytes land at offset 16 l of the
// fragment.  Completion is tracked by the vector memory counter only, so the
// consumer waits with s_waitcnt vmcnt(0) and a barrier.
template <int P>
__device__ __forceinline__ void stage_dma(const unsigned char* chunk, int w, int lane) {
#pragma unroll
  for (int q = 0; q < kStageQ; ++q) {
    const int f = w + 4 * q;
    if (f < kStageFrags)
      __builtin_amdgcn_global_load_lds(chunk + f * kFrag + lane * 16, (lds_void*)(stage_buf<P>() + f * kFrag), 16,
                                       0, 2);
  }
}

// WANT_O = false: no outputs (O is not formed, o not written), the final state
// only.
template <bool OUT_BF16, bool WANT_O>
__global__ __launch_bounds__(512, 1) void inter_chunk_kernel(SplitParams p) {
  const int H = p.H, T = p.T;
  const int nbh = p.B * H;
  const bool copy2 = (int)blockIdx.x >= nbh;  // the copy from the identity (see SplitParams)
  const int bh = copy2 ? blockIdx.x - nbh : blockIdx.x;
  float* const S_out = copy2 ? p.S_out2 : p.S_out;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool math = wave < 4;
  const int w = wave & 3;
  const int lane = tid & 63, g = lane >> 4, i = lane & 15;
  // chunks [cb, cb + nc) of the sequence; a resume launch starts where the
  // first launch stopped
  int cb = p.c_begin, nc = p.n_chunks, done = 0;
  if (p.resume != nullptr) {
    done = p.resume[bh];
    if (done >= nc) return;  // the first launch finished this (b, h)
    cb += done;
    nc -= done;
  }
  const int wstride = p.ws_stride > 0 ? p.ws_stride : p.n_chunks;
  const int wfirst = p.ws_stride > 0 ? p.ws_first : p.c_begin;
  const unsigned char* wsh = p.ws + ((size_t)bh * wstride + (cb - wfirst)) * WS_CHUNK;
  // One launch over every slab (it starts at chunk 0): the copying waves wait
  // before copying chunk next_jc, the first of slab next_sl; slab s is
  // kFirstChunks << s chunks long while s < slab_ramp, then slab_per.
  int next_sl = 0, next_jc = p.slab_ready != nullptr ? 0 : 0x7fffffff;
  auto advance_slab = [&]() {
    next_jc += next_sl < p.slab_ramp ? kFirstChunks << next_sl : p.slab_per;
    ++next_sl;
  };
  // Each copying wave waits for slab sl's flag on its own (bounded); false: the
  // wait expired.  The first copying wave's wait decides: the others wait 5 ms
  // longer, so theirs expires only if the first wave's did (they start within
  // microseconds of each other, after the same barrier).
  auto wait_for_slab = [&](int sl) -> bool {
    const unsigned* f = p.slab_ready + sl;
    const unsigned ticks = p.slab_ready[kSyncBound];
    const unsigned bound = w == 0 ? ticks : ticks + 500000u;
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(8);
        if ((unsigned)(__builtin_amdgcn_s_memrealtime() - t0) > bound) {
          if (w == 0 && lane == 0) atomicAdd(&g_wait_timeouts, 1u);
          return false;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return true;
  };
  const int col0 = 32 * w;

  // math waves: S[m][ct] element e = S[channel perm_row(16m + 4g + e)][col0 + 16ct + i]
  f4 S[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) S[m][ct] = f4{0.f, 0.f, 0.f, 0.f};
  // math waves: the scale of this wave's columns (kRangeLimit) and the largest
  // sum of |taps| over its v channels
  float sig = 1.0f, tapsum = 0.0f;
  if (math) {
    if (tid < kD) g_vw[tid] = *reinterpret_cast<const float4*>(p.conv_w + ((size_t)2 * H * kD + (size_t)h * kD + tid) * 4);
    {
      float ts = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 t4 =
            *reinterpret_cast<const float4*>(p.conv_w + ((size_t)2 * H * kD + (size_t)h * kD + col0 + 8 * g + e) * 4);
        ts = fmaxf(ts, fabsf(t4.x) + fabsf(t4.y) + fabsf(t4.z) + fabsf(t4.w));
      }
      tapsum = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wave_max(ts))));
    }
    if (copy2) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[m][ct][e] = perm_row(16 * m + 4 * g + e) == col0 + 16 * ct + i ? 1.f : 0.f;
    } else if (p.S_in != nullptr || done > 0) {
      // a resumed (b, h) finds its state where the first launch left it
      const float* src = (done > 0 ? S_out : p.S_in) + (size_t)bh * kD * kD;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[m][ct][e] = src[(size_t)perm_row(16 * m + 4 * g + e) * kD + col0 + 16 * ct + i];
      float sm = 0.0f;
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e) sm = fmaxf(sm, fabsf(S[m][ct][e]));
      sm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wave_max(sm))));
      sig = grow_scale(1.0f, sm);
      if (sig != 1.0f) {
        const float r = 1.0f / sig;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) S[m][ct] *= r;
      }
    }
  }
  // Chunks this workgroup completes: nc, unless the first copying wave's wait
  // for a slab expires.  It then puts kStopFlag in place of that chunk's wide
  // flag (its own copy holds that flag) and posts the chunk in g_dec: the
  // copying waves read it after the next barrier, the math waves see the flag
  // in the step of that chunk, and all stop after that step.
  int nce = nc;
  if (!math && nc > 0) {
    bool ok = true;
    if (next_jc == 0) {
      if (w == 0) ok = wait_for_slab(0);
      advance_slab();
    }
    if (w == 0) {  // chunk 0: the first copying wave copies all of it
      if (ok) {
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) stage_dma<0>(wsh, ww, lane);
      } else if (lane == 0) {
        *reinterpret_cast<int*>(g_stage0 + WS_WIDE) = kStopFlag;
      }
      if (lane == 0) g_dec = ok ? -1 : 0;  // read by the others after the first B1
    }
    if (!ok) nce = 0;
    __builtin_amdgcn_s_waitcnt(0);  // chunk 0's operands land before the first B1
  }

  // Two loops with the same barriers, one per role, so that the state is live
  // only in the math waves' loop.
  // B1 (top of each iteration): chunk j's operands are in LDS (the copying
  // waves waited for their copies), O(j-1) is complete, and nobody reads the
  // buffer copied next.
  if (math) {
    // Raw v of this wave's columns in the row-operand layout: register rt of
    // lane (g, i) holds token 16 rt + i (clamped to the sequence) and channels
    // col0 + 8g .. col0 + 8g + 7, loaded one chunk ahead into the register set
    // of the chunk's parity.
    const uint16_t* v16 = reinterpret_cast<const uint16_t*>(p.v);
    auto load_v = [&](int jc, uint4 (&r)[4]) {
      const int c0 = (cb + jc) * kC;
      const int last = min(kC, T - c0) - 1;
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        r[rt] = ld_nt(v16 + (((size_t)b * T + c0 + min(16 * rt + i, last)) * H + h) * kD + col0 + 8 * g);
    };
    uint4 rv[2][4];
    if (nc > 0) {
      load_v(0, rv[0]);
      // The conv's halo of the first chunk goes where the previous chunk's last
      // tile would be: lanes 13..15 take the three raw tokens before the chunk,
      // from the sequence, the conv history, or zeros at the sequence start.
      const int c0 = cb * kC;
      const int th = c0 - 16 + max(i, 13);
      if (c0 > 0) {
        rv[1][3] = *reinterpret_cast<const uint4*>(v16 + (((size_t)b * T + th) * H + h) * kD + col0 + 8 * g);
      } else if (p.conv_in != nullptr) {
        const size_t cch = (size_t)H * kNCh;
        rv[1][3] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.conv_in) +
                                                   ((size_t)b * 3 + (3 + th)) * cch + (size_t)2 * H * kD +
                                                   (size_t)h * kD + col0 + 8 * g);
      } else {
        rv[1][3] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    // one chunk; P = j & 1 picks the staging buffer and the raw v registers
    auto step = [&](auto parity, int j) {
      constexpr int P = decltype(parity)::value;
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();  // B1
      f4 O[4][2], X[4][2];
      const unsigned char* sb = stage_buf<P>();
      if (j < nce) {
        // V = SiLU(conv(v)) in fp16 (the causal conv along the tokens of each
        // 16-lane row, the previous tile's raw values as the halo: for tile 0
        // the previous chunk's tile 3), moved into the C layout of X by a
        // product with the identity
        // the chunk's bound on |V| from its raw values (and the halo's): the
        // scale grows first if V or the state would leave fp16's range
        {
          // |bf16| as 16-bit integers (sign cleared), two per dword: packed maxima
          typedef unsigned short us2 __attribute__((ext_vector_type(2)));
          us2 mb = us2{0, 0};
#pragma unroll
          for (int rt = 0; rt < 5; ++rt) {
            const uint4 u = rt < 4 ? rv[P][rt] : rv[1 - P][3];
            mb = __builtin_elementwise_max(mb, __builtin_bit_cast(us2, u.x & 0x7fff7fffu));
            mb = __builtin_elementwise_max(mb, __builtin_bit_cast(us2, u.y & 0x7fff7fffu));
            mb = __builtin_elementwise_max(mb, __builtin_bit_cast(us2, u.z & 0x7fff7fffu));
            mb = __builtin_elementwise_max(mb, __builtin_bit_cast(us2, u.w & 0x7fff7fffu));
          }
          const uint32_t m1 = mb[0] > mb[1] ? mb[0] : mb[1];
          const float mv = wave_max(__builtin_bit_cast(float, m1 << 16));
          const float ns = grow_scale(sig, __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                                       __builtin_bit_cast(int, mv))) * tapsum + 0.3f);
          if (ns != sig) {
            const float r = sig / ns;
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) S[m][ct] *= r;
            sig = ns;
          }
        }
        half8 vh[4];
        auto conv_v = [&](auto scaled) {
          const float isig = 1.0f / sig;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float4 wv = g_vw[col0 + 8 * g + e];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
              const float xc = bf16_at(rv[P][rt], e);
              const float y = bf16_at(rt == 0 ? rv[1 - P][3] : rv[P][rt - 1], e);
              const float a = siluf_(conv3_dpp(wv.w * xc, xc, y, wv.z, wv.y, wv.x));
              vh[rt][e] = (_Float16)(decltype(scaled)::value ? a * isig : a);
            }
          }
        };
        if (sig == 1.0f) conv_v(std::false_type{});
        else conv_v(std::true_type{});
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            X[rt][ct] = mma_f16(vh[rt], ident_frag(g, i, ct), f4{0.f, 0.f, 0.f, 0.f});
            if constexpr (WANT_O) O[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
          }
        if (j + 1 < nce) load_v(j + 1, rv[1 - P]);
        // X = V + (-(K e^G)) S and (Q e^G) S, one 32-row step of S at a time:
        // its B operands are rows 16(2k + s) + 4g + e, s = 0, 1
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
          half8 Sb[2];
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const float x[8] = {S[2 * kp][ct][0], S[2 * kp][ct][1], S[2 * kp][ct][2], S[2 * kp][ct][3],
                                S[2 * kp + 1][ct][0], S[2 * kp + 1][ct][1], S[2 * kp + 1][ct][2], S[2 * kp + 1][ct][3]};
            Sb[ct] = to_half8(x);
          }
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const half8 wf = *reinterpret_cast<const half8*>(sb + WS_KG + ((rt * 4 + kp) * 64 + lane) * 16);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) X[rt][ct] = mma_f16(wf, Sb[ct], X[rt][ct]);
            if constexpr (WANT_O) {
              const half8 qf = *reinterpret_cast<const half8*>(sb + WS_QG + ((rt * 4 + kp) * 64 + lane) * 16);
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) O[rt][ct] = mma_f16(qf, Sb[ct], O[rt][ct]);
            }
          }
        }
      }
      lds_barrier();  // B2
      if (j < nce) {
        // U = T diag(beta) X, with X as B operands over tokens 32k' + 16s + 4g + e
        half8 Xb[2][2];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const float x[8] = {X[2 * kp][ct][0], X[2 * kp][ct][1], X[2 * kp][ct][2], X[2 * kp][ct][3],
                                X[2 * kp + 1][ct][0], X[2 * kp + 1][ct][1], X[2 * kp + 1][ct][2], X[2 * kp + 1][ct][3]};
            Xb[kp][ct] = to_half8(x);
          }
        f4 U[4][2];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) U[rt][ct] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kp = 0; kp < 2; ++kp)
            if (2 * kp <= rt) {
              const half8 tf = *reinterpret_cast<const half8*>(sb + WS_TB + (p_frag(rt, kp) * 64 + lane) * 16);
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) U[rt][ct] = mma_f16(tf, Xb[kp][ct], U[rt][ct]);
            }
        }
        // U as B operands over tokens 32k' + 16s + 4g + e; in a wide chunk also
        // the fp16 remainder U - Ub, so the two products below see U to about
        // 22 bits
        const int wflag = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(sb + WS_WIDE));
        if (wflag == kStopFlag) {  // chunk j was not copied: stop before it
          nce = j;
          return;
        }
        const bool wide = wflag != 0;
        half8 Ub[2][2], Ul[2][2];
#pragma unroll
        for (int kp = 0; kp < 2; ++kp)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const float x[8] = {U[2 * kp][ct][0], U[2 * kp][ct][1], U[2 * kp][ct][2], U[2 * kp][ct][3],
                                U[2 * kp + 1][ct][0], U[2 * kp + 1][ct][1], U[2 * kp + 1][ct][2], U[2 * kp + 1][ct][3]};
            Ub[kp][ct] = to_half8(x);
            if (wide) {
#pragma unroll
              for (int e = 0; e < 8; ++e) Ul[kp][ct][e] = (_Float16)(x[e] - (float)Ub[kp][ct][e]);
            }
          }
        // O += P U, then O to LDS for the epilogue waves
#pragma unroll
        for (int rt = 0; rt < 4 && WANT_O; ++rt) {
#pragma unroll
          for (int kp = 0; kp < 2; ++kp)
            if (2 * kp <= rt) {
              const half8 pf = *reinterpret_cast<const half8*>(sb + WS_P + (p_frag(rt, kp) * 64 + lane) * 16);
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) O[rt][ct] = mma_f16(pf, Ub[kp][ct], O[rt][ct]);
              if (wide) {
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) O[rt][ct] = mma_f16(pf, Ul[kp][ct], O[rt][ct]);
              }
            }
          const float ox[8] = {O[rt][0][0], O[rt][0][1], O[rt][0][2], O[rt][0][3],
                               O[rt][1][0], O[rt][1][1], O[rt][1][2], O[rt][1][3]};
          *reinterpret_cast<half8*>(g_O + (rt * 4 + w) * kOBlk + g * kOGrp + i * 16 + (i >> 3) * 16) = to_half8(ox);
        }
        if (WANT_O && lane == 0) g_Osig[w] = sig;
        // S <- e^{G_C} S + (K e^{G_C - G})^T U
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float4 gm = *reinterpret_cast<const float4*>(sb + WS_GAM + (16 * m + 4 * g) * 4);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            S[m][ct][0] *= gm.x;
            S[m][ct][1] *= gm.y;
            S[m][ct][2] *= gm.z;
            S[m][ct][3] *= gm.w;
          }
#pragma unroll
          for (int kp = 0; kp < 2; ++kp) {
            const half8 kf = *reinterpret_cast<const half8*>(sb + WS_KB + ((m * 2 + kp) * 64 + lane) * 16);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) S[m][ct] = mma_f16(kf, Ub[kp][ct], S[m][ct]);
            if (wide) {
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) S[m][ct] = mma_f16(kf, Ul[kp][ct], S[m][ct]);
            }
          }
        }
      }
    };
    // both roles skip the loop (and its barriers) in a launch without chunks
    if (nc > 0) {
      for (int j = 0; j <= nce; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        if (j + 1 <= nce) step(std::integral_constant<int, 1>{}, j + 1);
      }
    }
  } else {
    // lane (u, q) = (lane / 8, lane % 8) of epilogue wave r = w: tokens
    // 16r + 2u + tt (tt = 0, 1) of the previous chunk, columns 64s + 8q + c
    // (s = 0, 1; c = 0..7), so that gate and output move in 16-byte pieces.
    const int u = lane >> 3, q = lane & 7;
    const int tk0 = 16 * w + 2 * u;
    // In g_O: block (w, 2s + q / 4); C-layout lane (u / 2, 8 (q % 2) + c),
    // element 4 ((q / 2) % 2) + 2 (u % 2) + tt; one 4-byte read gives both tokens.
    const int obase = (u >> 1) * kOGrp + (q & 1) * 144 + ((q >> 1) & 1) * 8 + (u & 1) * 4;
    // gate of the chunk normalised next, loaded one chunk ahead: [tt][s], 8 bf16
    uint4 gt[2][2];
    auto load_gate = [&](int jc) {
      const int c0 = (cb + jc) * kC;
      const int nv = min(kC, T - c0);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tk = min(tk0 + tt, nv - 1);
        const uint16_t* gr =
            reinterpret_cast<const uint16_t*>(p.gate) + (((size_t)b * T + c0 + tk) * H + h) * kD + 8 * q;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) gt[tt][s2] = ld_nt(gr + 64 * s2);
      }
    };
    if (WANT_O && nc > 0) load_gate(0);
    // one chunk; P = j & 1 picks the staging buffer the next chunk goes to
    auto step = [&](auto parity, int j) {
      constexpr int P = decltype(parity)::value;
      // No memory wait before B1: this wave's copy of chunk j was waited for
      // after B2 of the previous chunk, and its stores need no wait.
      lds_barrier();  // B1
      if (j == 0 && w != 0 && __builtin_amdgcn_readfirstlane(g_dec) == 0) nce = 0;  // chunk 0 was not copied
      if (j + 1 < nce) {
        bool ok = true;
        if (j + 1 == next_jc) {
          ok = wait_for_slab(next_sl);
          advance_slab();
        }
        if (ok) {
          stage_dma<1 - P>(wsh + (size_t)(j + 1) * WS_CHUNK, w, lane);
        } else if (w == 0 && lane == 0) {
          *reinterpret_cast<int*>(stage_buf<1 - P>() + WS_WIDE) = kStopFlag;
          g_dec = j + 1;
        }
      }
      // ---- epilogue of chunk j-1 ----------------------------------------------------
      float ov[2][2][8], osig[2];
      if (WANT_O && j >= 1) {
        // the scales of the two math waves whose columns this lane normalises
        osig[0] = g_Osig[q >> 2];
        osig[1] = g_Osig[2 + (q >> 2)];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const hf2 o2 = *reinterpret_cast<const hf2*>(g_O + (w * 4 + 2 * s2 + (q >> 2)) * kOBlk + obase + 16 * c);
            ov[0][s2][c] = (float)o2[0];
            ov[1][s2][c] = (float)o2[1];
          }
      }
      lds_barrier();  // B2: O(j-1) is in registers
      if (__builtin_amdgcn_readfirstlane(g_dec) == j + 1) nce = j + 1;  // the first copying wave stopped there
      // The copy of chunk j + 1 (it must land before B1 of chunk j + 1), the
      // gate loaded a chunk ago and the previous chunk's stores: one wait here,
      // before this chunk's stores, so that those are never waited on.
      __builtin_amdgcn_s_waitcnt(0);
      if (WANT_O && j >= 1) {
        const int c0 = (cb + j - 1) * kC;
        const int nv = min(kC, T - c0);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float ss = 0.f;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            float sp = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) sp += ov[tt][s2][c] * ov[tt][s2][c];
            ss += sp * osig[s2] * osig[s2];
          }
          ss = group_sum<8>(ss);
          const float rs = fast_rsq(ss * (1.0f / kD) + kRmsEps);
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int c = 0; c < 8; ++c) ov[tt][s2][c] *= osig[s2] * rs * sigmoidf_(bf16_at(gt[tt][s2], c));
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int tk = tk0 + tt;
          if (tk < nv) {
            const size_t ob = (((size_t)b * T + c0 + tk) * H + h) * kD + 8 * q;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) store8_nt<OUT_BF16>(p.o, ob + 64 * s2, ov[tt][s2]);
          }
        }
      }
      if (WANT_O && j >= 1 && j < nce) load_gate(j);
    };
    // both roles skip the loop (and its barriers) in a launch without chunks
    if (nc > 0) {
      for (int j = 0; j <= nce; j += 2) {
        step(std::integral_constant<int, 0>{}, j);
        if (j + 1 <= nce) step(std::integral_constant<int, 1>{}, j + 1);
      }
    }
  }

  // ---- state and conv history out -------------------------------------------------
  // A workgroup that stopped early (nce < nc) leaves its state after chunk
  // nce - 1 in S_out for the resume launch (none if it finished no chunk).
  const bool stopped = nce < nc;
  if (math && S_out != nullptr && (!stopped || nce > 0)) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          S_out[(size_t)bh * kD * kD + (size_t)perm_row(16 * m + 4 * g + e) * kD + col0 + 16 * ct + i] =
              S[m][ct][e] * sig;
  }
  if (p.slab_ready != nullptr && wave == 4 && lane == 0)  // a first launch (done = 0)
    reinterpret_cast<int*>(const_cast<unsigned*>(p.slab_ready))[kSyncProgress + bh] = nce;
  if (!copy2 && !stopped && p.conv_out != nullptr) {
    const size_t cch = (size_t)H * kNCh;
    for (int cl = tid; cl < kNCh; cl += 512) {
      const void* src = cl < kD ? p.q : cl < 2 * kD ? p.k : p.v;
      const int cc = cl & (kD - 1);
      const size_t chb = cl < kD ? (size_t)h * kD + cc
                       : cl < 2 * kD ? (size_t)H * kD + (size_t)h * kD + cc
                                     : (size_t)2 * H * kD + (size_t)h * kD + cc;
      float v3[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int t = T - 3 + r;
        if (t >= 0) v3[r] = load1<true>(src, (((size_t)b * T + t) * H + h) * kD + cc);
        else if (p.conv_in != nullptr) v3[r] = load1<true>(p.conv_in, ((size_t)b * 3 + (3 + t)) * cch + chb);
        else v3[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 3; ++r) store1<true>(p.conv_out, ((size_t)b * 3 + r) * cch + chb, v3[r]);
    }
  }
}

// How the chunks of one call are split into launches ("slabs").
//
// Pipelined (a sequence of more than kPipeChunks chunks and B*H at most half
// the compute units): slabs of at most kPipeChunks chunks, each in its own
// workspace region when all fit under kSlabBytesMax, else in kPipeBufs
// buffers used in turn.  From 2 * kPipeChunks chunks on, the slabs ramp up from
// kFirstChunks, each twice as long as the one before, so the inter-chunk kernel
// (the slower stage) starts soon and later launches are few.  The inter-chunk kernel (one workgroup per (b, h), the state carried
// between slabs in a buffer) runs on a stream restricted to B*H compute units,
// the intra-chunk kernel of the next slab on a stream restricted to the others,
// so the two overlap without competing for compute units.
// Otherwise: one slab when all chunk blocks fit the workspace (and stay under
// the cap), else as many chunks per slab as fit next to the state carry, one
// slab after the other on the caller's stream.
constexpr int kPipeBufs = 3;  // the intra-chunk kernel runs up to two slabs ahead
constexpr int kPlanCUs = 256;  // compute units the preferred workspace is planned for

struct SlabPlan {
  int nchunks, per_slab, nslabs, nbuf;
  int ramp;  // leading slabs of kFirstChunks, 2 kFirstChunks, ... chunks (0: none)
  size_t region_bytes, carry_bytes;
};

// Chunks [c0, c0 + n) of slab sl.
void slab_range(const SlabPlan& pl, int sl, int& c0, int& n) {
  int len;
  if (sl < pl.ramp) {
    c0 = kFirstChunks * ((1 << sl) - 1);
    len = kFirstChunks << sl;
  } else {
    c0 = kFirstChunks * ((1 << pl.ramp) - 1) + (sl - pl.ramp) * pl.per_slab;
    len = pl.per_slab;
  }
  n = pl.nchunks - c0 < len ? pl.nchunks - c0 : len;
  if (n < 0) n = 0;
}

size_t per_chunk_bytes(const kda_prefill_args& a) { return (size_t)a.B * a.H * WS_CHUNK; }
size_t carry_bytes(const kda_prefill_args& a) { return (size_t)a.B * a.H * kD * kD * 4; }
bool pipe_shape(const kda_prefill_args& a, int ncu) { return 2L * a.B * a.H <= ncu; }

// pipe_ok = false plans the slabs one after the other on the caller's stream.
SlabPlan plan_slabs(const kda_prefill_args& a, size_t avail, bool pipe_ok = true) {
  SlabPlan s{};
  s.nchunks = (a.T + kC - 1) / kC;
  s.nbuf = 1;
  const size_t pc = per_chunk_bytes(a);
  const size_t cb = carry_bytes(a);
  if (pipe_ok && s.nchunks > kPipeChunks && pipe_shape(a, kPlanCUs) && avail >= cb + kPipeBufs * pc) {
    const size_t fit = (avail - cb) / (kPipeBufs * pc);
    const int most = (int)(fit < (size_t)kPipeChunks ? fit : (size_t)kPipeChunks);
    if (most == kPipeChunks && s.nchunks >= 2 * kPipeChunks) {
      int done = 0;
      while ((kFirstChunks << s.ramp) < kPipeChunks) done += kFirstChunks << s.ramp++;
      const int rest = s.nchunks - done;
      const int k = (rest + most - 1) / most;
      s.per_slab = (rest + k - 1) / k;  // balanced slabs after the ramp
      s.nslabs = s.ramp + k;
    } else {
      s.nslabs = (s.nchunks + most - 1) / most;
      s.per_slab = (s.nchunks + s.nslabs - 1) / s.nslabs;  // balanced slabs, no small tail
    }
    s.nbuf = s.nslabs < kPipeBufs ? s.nslabs : kPipeBufs;
    // Every slab its own region when they all fit (under the cap): the
    // intra-chunk kernel then never waits for the inter-chunk kernel to free a
    // buffer, and the inter-chunk stream records no per-slab event (measured
    // 5.74 against 5.88 ms at K3 width).
    const size_t all = (size_t)s.nslabs * kPipeChunks * pc;
    if (all <= kSlabBytesMax && avail >= cb + all) s.nbuf = s.nslabs;
    s.carry_bytes = cb;
  } else {
    const size_t room = avail < kSlabBytesMax ? avail : kSlabBytesMax;
    if ((size_t)s.nchunks * pc <= room) {
      s.per_slab = s.nchunks > 0 ? s.nchunks : 1;
      s.nslabs = 1;
      s.carry_bytes = 0;
    } else {
      const size_t room2 = avail < kSlabBytesMax + cb ? avail : kSlabBytesMax + cb;
      const size_t per = room2 > cb + pc ? (room2 - cb) / pc : 1;
      const int most = (int)(per < (size_t)s.nchunks ? per : (size_t)s.nchunks);
      s.nslabs = (s.nchunks + most - 1) / most;
      s.per_slab = (s.nchunks + s.nslabs - 1) / s.nslabs;
      s.carry_bytes = s.nslabs > 1 ? cb : 0;
    }
  }
  s.region_bytes = (size_t)s.per_slab * pc;
  if (s.ramp > 0) s.region_bytes = (size_t)kPipeChunks * pc;  // the same preferred size for any length
  return s;
}

// The compute-unit-restricted streams of the pipeline (default priority) and
// the events that order them, per host thread and device, for one inter-chunk
// width (B*H rounded up to a multiple of 8, so each of the eight accelerator
// dies gets the same share: mask bits interleave over the dies).  Slabs
// alternate between two intra-chunk streams, so the event recorded after one
// slab's intra-chunk kernel never holds back the next one's start.  Created on
// first use and kept until kda_release() or process exit.
struct Pipe {
  int n_inter = 0;
  unsigned gen = 0;  // release_generation() when created
  hipStream_t intra[2] = {nullptr, nullptr}, inter = nullptr;
  hipEvent_t fork = nullptr, a_done[2] = {nullptr, nullptr}, b_done[kPipeBufs] = {};
  hipEvent_t join[3] = {nullptr, nullptr, nullptr};
};

// 0 and pp = nullptr when the device has too few compute units to split.
int get_pipe(const kda_prefill_args& a, Pipe*& pp) {
  constexpr int kMaxDev = 64, kPerDev = 4;
  static thread_local Pipe pipes[kMaxDev][kPerDev];
  static thread_local int ncus[kMaxDev];
  pp = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    set_error("prefill: hipGetDevice failed or device %d out of range", dev);
    return KDA_E_HIP;
  }
  if (ncus[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0) {
      set_error("prefill: compute unit count query failed: %s", hipGetErrorString(e));
      return KDA_E_HIP;
    }
    ncus[dev] = n;
  }
  const int ncu = ncus[dev];
  if (!pipe_shape(a, ncu)) return KDA_OK;
  const int n_inter = (int)((a.B * a.H + 7) / 8 * 8);
  if (n_inter >= ncu) return KDA_OK;
  // slots made before the last kda_release() hold destroyed handles
  const unsigned gen = release_generation();
  for (int k = 0; k < kPerDev; ++k)
    if (pipes[dev][k].n_inter != 0 && pipes[dev][k].gen != gen) pipes[dev][k] = Pipe{};
  Pipe* slot = nullptr;
  for (int k = 0; k < kPerDev && slot == nullptr; ++k)
    if (pipes[dev][k].n_inter == n_inter) slot = &pipes[dev][k];
  for (int k = 0; k < kPerDev && slot == nullptr; ++k)
    if (pipes[dev][k].n_inter == 0) slot = &pipes[dev][k];
  if (slot == nullptr) return KDA_OK;  // every slot holds another width: run unpipelined
  if (slot->n_inter == 0) {
    uint32_t m_inter[32] = {0}, m_intra[32] = {0};
    const int nb = ncu < 32 * 32 ? ncu : 32 * 32;
    for (int c = 0; c < nb; ++c) (c < n_inter ? m_inter : m_intra)[c / 32] |= 1u << (c % 32);
    const uint32_t words = (uint32_t)((nb + 31) / 32);
    e = hipExtStreamCreateWithCUMask(&slot->inter, words, m_inter);
    for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipExtStreamCreateWithCUMask(&slot->intra[k], words, m_intra);
    hipEvent_t* evs[6 + kPipeBufs] = {&slot->fork, &slot->a_done[0], &slot->a_done[1],
                                      &slot->join[0], &slot->join[1], &slot->join[2]};
    for (int k = 0; k < kPipeBufs; ++k) evs[6 + k] = &slot->b_done[k];
    for (int k = 0; k < 6 + kPipeBufs && e == hipSuccess; ++k) e = hipEventCreateWithFlags(evs[k], hipEventDisableTiming);
    // everything created is registered, so kda_release() (or process exit) frees it
    if (slot->inter != nullptr) keep(slot->inter);
    for (int k = 0; k < 2; ++k)
      if (slot->intra[k] != nullptr) keep(slot->intra[k]);
    for (int k = 0; k < 6 + kPipeBufs; ++k)
      if (*evs[k] != nullptr) keep(*evs[k]);
    if (e != hipSuccess) {
      *slot = Pipe{};
      set_error("prefill: stream / event creation failed: %s", hipGetErrorString(e));
      return KDA_E_HIP;
    }
    slot->n_inter = n_inter;
    slot->gen = gen;
  }
  pp = slot;
  return KDA_OK;
}

// Test settings of the one-launch recurrence (kda_debug_pipeline): the bound
// of its waits (0: kReadyWaitUs) and a slab whose flag is never set (-1: none).
std::atomic<unsigned> g_dbg_wait_us{0};
std::atomic<int> g_dbg_withhold{-1};

// The flags of a one-launch recurrence: cleared on the caller's stream before
// the pipeline forks, set one by one after each slab's intra-chunk kernel.
__global__ void clear_flags_kernel(unsigned* f, int n, unsigned bound) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) f[i] = 0u;
  if (threadIdx.x == 0) f[kSyncBound] = bound;
}
__global__ void set_flag_kernel(unsigned* f) {
  if (threadIdx.x == 0) __hip_atomic_store(f, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

template <bool OB, bool K3>
int run_split(const kda_prefill_args& a, hipStream_t st, bool pipe_ok) {
  // Under stream capture the slabs run one after the other on the caller's
  // stream: no other streams, no events, no waits between kernels (a capture
  // that forked onto the compute-unit-restricted streams crashed in the
  // runtime's end of capture).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusActive;
  const bool capturing = hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone;
  const SlabPlan pl = plan_slabs(a, a.workspace_bytes, pipe_ok && !capturing);
  const hipError_t e1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&intra_chunk_kernel<K3>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, ALds::BYTES);
  if (e1 != hipSuccess) {
    set_error("prefill: hipFuncSetAttribute failed: %s", hipGetErrorString(e1));
    return KDA_E_HIP;
  }
  Pipe* pp = nullptr;
  if (pl.nbuf > 1) {
    const int rc = get_pipe(a, pp);
    if (rc != KDA_OK) return rc;
  }
  const bool piped = pp != nullptr;
  hipStream_t sb = piped ? pp->inter : st;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  float* carry = pl.carry_bytes ? reinterpret_cast<float*>(ws + pl.nbuf * pl.region_bytes) : nullptr;
  hipError_t e = hipSuccess;
  const char* what = "event";
  // Every slab resident at once: the chunk blocks of all slabs share one
  // head-major layout, and a single recurrence launch walks them all, waiting
  // on a flag per slab instead of a stream event before each slab's launch.
  // The flags and each (b, h)'s count of finished chunks are kept where the
  // state carry would be, which this mode does not use.  A resume launch after
  // all slabs finishes what a workgroup left when its wait expired (at once
  // when none did).
  // S_T is where a stopped workgroup leaves its state for the resume launch.
  const bool one_inter = piped && pl.nbuf == pl.nslabs && pl.nslabs > 1 && pl.nslabs <= kMaxSlabs &&
                         a.S_T != nullptr && pl.carry_bytes >= sync_bytes(a.B * a.H);
  unsigned* flags = one_inter ? reinterpret_cast<unsigned*>(carry) : nullptr;
  SplitParams resume{};
  if (one_inter) {
    const unsigned us = g_dbg_wait_us.load(std::memory_order_relaxed);
    // the counter runs at 100 MHz; at most about 40 s
    const unsigned ticks = 100u * std::min(us != 0 ? us : kReadyWaitUs, 40000000u);
    hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, st, flags, pl.nslabs, ticks);
    e = hipGetLastError();
    what = "flag clear launch";
  }
  if (e == hipSuccess && piped) {
    // both streams start after everything already queued on the caller's
    e = hipEventRecord(pp->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(pp->intra[0], pp->fork, 0);
    if (e == hipSuccess) e = hipStreamWaitEvent(pp->intra[1], pp->fork, 0);
    if (e == hipSuccess) e = hipStreamWaitEvent(sb, pp->fork, 0);
  }
  for (int sl = 0; sl < pl.nslabs && e == hipSuccess; ++sl) {
    SplitParams p{};
    p.B = a.B; p.T = a.T; p.H = a.H;
    slab_range(pl, sl, p.c_begin, p.n_chunks);
    p.q = a.q; p.k = a.k; p.v = a.v; p.conv_w = a.conv_w; p.g = a.g; p.beta = a.beta; p.gate = a.gate;
    p.A = a.decay_form == KDA_DECAY_K3 ? a.A : nullptr;
    const bool first = sl == 0, last = sl == pl.nslabs - 1;
    p.S_in = first ? a.S0 : carry;
    p.conv_in = a.conv_in;
    p.o = a.o;
    p.S_out = last ? a.S_T : carry;
    p.conv_out = last ? a.conv_out : nullptr;
    const int buf = sl % pl.nbuf;
    p.ws = ws + (size_t)buf * pl.region_bytes;
    if (one_inter) {
      p.ws = ws;
      p.ws_stride = pl.nchunks;
      p.ws_first = 0;
    }
    hipStream_t sa = piped ? pp->intra[sl & 1] : st;
    // the buffer is free once the inter-chunk kernel of slab sl - nbuf is done
    if (piped && sl >= pl.nbuf) e = hipStreamWaitEvent(sa, pp->b_done[buf], 0);
    if (e == hipSuccess && p.n_chunks > 0) {
      const size_t grid = (size_t)p.n_chunks * a.B * a.H;
      hipLaunchKernelGGL(intra_chunk_kernel<K3>, dim3((unsigned)grid), dim3(256), ALds::BYTES, sa, p);
      e = hipGetLastError();
      what = "intra-chunk launch";
    }
    if (one_inter) {
      if (e == hipSuccess && sl != g_dbg_withhold.load(std::memory_order_relaxed)) {
        hipLaunchKernelGGL(set_flag_kernel, dim3(1), dim3(64), 0, sa, flags + sl);
        e = hipGetLastError();
        what = "flag launch";
      }
      if (e != hipSuccess || !last) continue;
      // every slab is queued: the one recurrence launch over all chunks
      p.c_begin = 0;
      p.n_chunks = pl.nchunks;
      p.S_in = a.S0;
      resume = p;
      p.slab_ready = flags;
      p.slab_ramp = pl.ramp;
      p.slab_per = pl.per_slab;
      resume.resume = reinterpret_cast<const int*>(flags + kSyncProgress);
    } else if (e == hipSuccess && piped) {
      what = "event";
      e = hipEventRecord(pp->a_done[sl & 1], sa);
      if (e == hipSuccess) e = hipStreamWaitEvent(sb, pp->a_done[sl & 1], 0);
    }
    if (e == hipSuccess) {
      hipLaunchKernelGGL((inter_chunk_kernel<OB, true>), dim3((unsigned)(a.B * a.H)), dim3(512), 0, sb, p);
      e = hipGetLastError();
      what = "inter-chunk launch";
    }
    if (e == hipSuccess && piped && sl + pl.nbuf < pl.nslabs) {  // a later slab reuses the buffer
      what = "event";
      e = hipEventRecord(pp->b_done[buf], sb);
    }
  }
  if (piped) {
    // the caller's stream resumes after the three streams' work (also on an error
    // above, so that nothing of this call is left unordered)
    hipStream_t all[3] = {pp->intra[0], pp->intra[1], sb};
    hipError_t j = hipSuccess;
    for (int k = 0; k < 3 && j == hipSuccess; ++k) j = hipEventRecord(pp->join[k], all[k]);
    for (int k = 0; k < 3 && j == hipSuccess; ++k) j = hipStreamWaitEvent(st, pp->join[k], 0);
    if (e == hipSuccess && j != hipSuccess) {
      e = j;
      what = "event";
    }
  }
  if (e == hipSuccess && one_inter) {
    // after every slab: whatever a stopped workgroup left (nothing, normally)
    hipLaunchKernelGGL((inter_chunk_kernel<OB, true>), dim3((unsigned)(a.B * a.H)), dim3(512), 0, st, resume);
    e = hipGetLastError();
    what = "resume launch";
  }
  if (e != hipSuccess) {
    set_error("prefill: %s failed: %s", what, hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

}  // namespace

void debug_pipeline(unsigned wait_us, int withhold_slab) {
  g_dbg_wait_us.store(wait_us, std::memory_order_relaxed);
  g_dbg_withhold.store(withhold_slab, std::memory_order_relaxed);
}

int wait_timeouts(unsigned* count) {
  const hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(g_wait_timeouts), sizeof(unsigned), 0,
                                           hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    set_error("wait_timeouts: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

bool prefill_split_eligible(const kda_prefill_args& a) {
  return a.in_dtype == KDA_BF16 && a.chunk == kC && a.dk == kD && a.dv == kD;
}

size_t prefill_split_workspace_bytes(const kda_prefill_args& a) {
  if (!prefill_split_eligible(a)) return 0;
  const SlabPlan pl = plan_slabs(a, ~(size_t)0);
  return pl.nbuf * pl.region_bytes + pl.carry_bytes;
}

size_t prefill_split_workspace_min_bytes(const kda_prefill_args& a) {
  if (!prefill_split_eligible(a)) return 0;
  const int nchunks = (a.T + kC - 1) / kC;
  if (nchunks <= 1) return (size_t)nchunks * per_chunk_bytes(a);
  return per_chunk_bytes(a) + carry_bytes(a);
}

int launch_split(const kda_prefill_args& a, hipStream_t s, bool pipe_ok) {
  const bool k3 = a.decay_form == KDA_DECAY_K3;
  if (a.out_dtype == KDA_BF16) return k3 ? run_split<true, true>(a, s, pipe_ok) : run_split<true, false>(a, s, pipe_ok);
  return k3 ? run_split<false, true>(a, s, pipe_ok) : run_split<false, false>(a, s, pipe_ok);
}

int launch_prefill_split(const kda_prefill_args& a, hipStream_t s) { return launch_split(a, s, true); }

// ---- one rank's share of context-parallel prefill in two calls ------------------
// Fragments: the intra-chunk kernel over every chunk once (all blocks kept in
// the workspace), then two copies of the recurrence side by side, from S = 0
// (final state N) and from S = I (final state P), without outputs.  Finish:
// the recurrence again over the kept blocks from the entering state S0, with
// outputs.  The inter-chunk kernel reads raw v and gate itself, so the kept
// blocks are all that carries over between the calls.
size_t cp_rank_split_bytes(const kda_prefill_args& a) {
  if (!prefill_split_eligible(a)) return 0;
  return (size_t)((a.T + kC - 1) / kC) * per_chunk_bytes(a);
}

namespace {
SplitParams rank_params(const kda_prefill_args& a) {
  SplitParams p{};
  p.B = a.B; p.T = a.T; p.H = a.H;
  p.c_begin = 0;
  p.n_chunks = (a.T + kC - 1) / kC;
  p.q = a.q; p.k = a.k; p.v = a.v; p.conv_w = a.conv_w; p.g = a.g; p.beta = a.beta; p.gate = a.gate;
  p.A = a.decay_form == KDA_DECAY_K3 ? a.A : nullptr;
  p.conv_in = a.conv_in;
  p.ws = static_cast<unsigned char*>(a.workspace);
  return p;
}

template <bool K3>
int launch_intra_all(const SplitParams& p, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&intra_chunk_kernel<K3>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, ALds::BYTES);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(intra_chunk_kernel<K3>, dim3((unsigned)((size_t)p.n_chunks * p.B * p.H)), dim3(256),
                       ALds::BYTES, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    set_error("context-parallel fragments: intra-chunk launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}
}  // namespace

int launch_cp_fragments_split(const kda_prefill_args& a, float* N, float* P, hipStream_t s) {
  SplitParams p = rank_params(a);
  p.S_in = nullptr;
  p.S_out = N;
  p.S_out2 = P;
  const int rc = a.decay_form == KDA_DECAY_K3 ? launch_intra_all<true>(p, s) : launch_intra_all<false>(p, s);
  if (rc != KDA_OK) return rc;
  hipLaunchKernelGGL((inter_chunk_kernel<false, false>), dim3((unsigned)(2 * a.B * a.H)), dim3(512), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("context-parallel fragments: inter-chunk launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

int launch_cp_finish_split(const kda_prefill_args& a, hipStream_t s) {
  SplitParams p = rank_params(a);
  p.S_in = a.S0;
  p.S_out = a.S_T;
  p.o = a.o;
  p.conv_out = a.conv_out;
  if (a.out_dtype == KDA_BF16)
    hipLaunchKernelGGL((inter_chunk_kernel<true, true>), dim3((unsigned)(a.B * a.H)), dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((inter_chunk_kernel<false, true>), dim3((unsigned)(a.B * a.H)), dim3(512), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("context-parallel finish: inter-chunk launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

// ---- allocation-free prefill (kda_prefill_noalloc) ---------------------------------
// For callers that cannot allocate, the two-kernel path's workspace is this
// file-scope device array instead of a caller buffer.  Each GPU the library
// runs on holds its own copy until the process ends; its address differs per
// device and is looked up once per device.  In host code `scratch` names only
// a host-side stand-in: every host use goes through the looked-up address.
// Nothing in it has to start at zero (each slab's blocks and the state carry
// are written before they are read).  Calls that overlap on one GPU share it
// and race.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
// Device address of `scratch` on the current device (looked up on first use).
int scratch_address(unsigned char*& ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static unsigned char* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    set_error("prefill (no allocation): hipGetDevice failed or device %d out of range", dev);
    return KDA_E_HIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      set_error("prefill (no allocation): hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return KDA_E_HIP;
    }
    addr[dev] = static_cast<unsigned char*>(p);
  }
  ptr = addr[dev];
  return KDA_OK;
}
}  // namespace

int launch_prefill_noalloc(const kda_prefill_args& a, hipStream_t s) {
  kda_prefill_args b = a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (!prefill_split_eligible(a)) return launch_prefill(b, s);  // the single-kernel path: no workspace
  const size_t need = prefill_split_workspace_min_bytes(a);
  if (need > KDA_NOALLOC_SCRATCH_BYTES) {
    set_error("prefill (no allocation): B*H = %lld heads need %zu bytes of workspace, more than the %zu-byte "
              "scratch (at most %zu bytes per head)", (long long)a.B * a.H, need, (size_t)KDA_NOALLOC_SCRATCH_BYTES,
              (size_t)(WS_CHUNK + kD * kD * 4));
    return KDA_E_WORKSPACE;
  }
  unsigned char* ws = nullptr;
  const int rc = scratch_address(ws);
  if (rc != KDA_OK) return rc;
  b.workspace = ws;
  b.workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
  return launch_split(b, s, false);  // slabs in turn on the caller's stream: no streams created
}

}  // namespace kda
