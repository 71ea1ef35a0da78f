// kda_backward.hip -- gradients of the KDA prefill (training: the 1M-token
// context of "Gemma 4 31B vs Kimi K3", component table, long-context training
// row), for the definition of "Kimi K3, previewed", section "Kimi Delta
// Attention - the workhorse" and the KDA rows of the component tables.
//
// All in fp32, three launch kinds:
//   1. forward, one workgroup per (b, h): the chunkwise prefill kernel with
//      fp32 operands (kda_prefill.hip, launch_prefill_states), storing the
//      state at every stretch start (kBwdChunk tokens, one chunk);
//   then token by token (256 or 512 threads by head dim):
//   2. recompute, one workgroup per (b, h, stretch) of a slab of stretches:
//      from the stretch's stored state, the state entering every token and
//      the token's vectors go to the slab buffer (all stretches at once, on
//      every compute unit);
//   3. reverse, one workgroup per (b, h): the slab's tokens walked back with
//      the state gradient dS in registers; dS and the conv ring are carried
//      to the next (earlier) slab through the workspace.
// Slabs run from the last to the first, recompute then reverse.
// Reverse step of token t (dS = dL/dS_t, do = dL/do_t; s = sigmoid(gate)):
//   dgate = do n s (1 - s);  dz = (do s - n mean(do s n)) / r
//   dq^ = S_t dz;  dS += q^ dz^T;  du = dS^T k^;  dk^ = dS u
//   dbeta = du . (v^ - y);  dv^ = beta du;  dy = -beta du
//   dS' = dS + k^ dy^T;  dk^ += S' dy;  dg = rowsum(dS' * S');  dS <- Diag(alpha) dS'
// then the L2-norm, SiLU and conv backward (conv transpose over a 3-token ring
// of the pre-SiLU gradients).  The state uses the decode kernel's layout:
// thread (cg = tid % CG, rg = tid / CG) holds rows rg + RG i of the 4 columns
// 4cg..4cg+3 (the reverse's dS: rows RPT rg + i, consecutive), so row sums are
// lane sums over the CG lanes of a row group and column sums go through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

// Tokens between stored states: the chunk of the chunkwise forward that
// stores them (kda_prefill.hip, fp32 operands).
constexpr int kBwdChunk = kStateChunk;
constexpr int kBwdSlab = 1024 / kBwdChunk;  // stretches recomputed per launch (1,024 tokens)

enum : int { kModeRecompute = 2, kModeReverse = 3 };

// Threads per workgroup: eight state rows per thread at d = 128 (512 threads,
// 8 waves), so each SIMD has two waves to hide latency with (1024 threads
// would need more than the 128 registers four waves allow).
template <int D>
constexpr int bwd_threads() {
  return D >= 64 ? 512 : 256;
}

struct BwdParams {
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
  const float* dO;
  const float* dS_T;
  const float* dconv_out;  // gradient of the last three raw rows, or null
  float* dq;
  float* dk;
  float* dv;
  float* dg;
  float* dbeta;
  float* dgate;
  float* dS0;
  float* dconv_in;
  float* ws;
  int ch_lo, ch_hi;  // the slab's stretches (recompute, reverse)
  int buf;           // the slab buffer (0 or 1) they go through
};

// One token's record in the workspace (floats): a, x~ (3d each), q^, k^, y,
// u, dz = dL/dz, alpha = e^g, dq^ = S_t dz (d each), then scalars nq, nk, rq,
// rk, -, beta, q~ . dq^ (and a slot the reverse uses for k~ . dk^).  dz, dq^
// and q~ . dq^ need only forward values and dL/do, so the recompute computes
// them (and dgate) off the reverse's serial path.  The
// same layout serves as the token's LDS image.
template <int D>
struct Rec {
  static constexpr int A = 0, X = 3 * D, QN = 6 * D, KN = 7 * D, Y = 8 * D, U = 9 * D, DZ = 10 * D;
  static constexpr int AL = 11 * D, DQ = 12 * D, SC = 13 * D;
  static constexpr int SIZE = 13 * D + 8;
};

// Workspace, in floats: the stored states [BH][nch][D][D], the carry
// [BH][D*D + 9D] (dS, then the conv ring [3][3D]), and two slab buffers
// [2][BH][slab stretches][kBwdChunk][D*D] states + [kBwdChunk][Rec SIZE]
// records (one is recomputed into while the other is walked back).
template <int D>
struct BwdLayout {
  static constexpr size_t CARRY = (size_t)D * D + 9 * D;
  static constexpr size_t STRETCH = (size_t)kBwdChunk * ((size_t)D * D + Rec<D>::SIZE);
  __host__ __device__ static int nch(int T) { return (T + kBwdChunk - 1) / kBwdChunk; }
  __host__ __device__ static int slab(int T) { return nch(T) < kBwdSlab ? nch(T) : kBwdSlab; }
  __host__ __device__ static size_t ckpt(int T) { return (size_t)nch(T) * D * D; }
  // per (b, h)
  __host__ __device__ static size_t head_floats(int T) { return ckpt(T) + CARRY + 2 * (size_t)slab(T) * STRETCH; }
};

// Barriers are LDS-only (lds_barrier) wherever threads exchange data through
// LDS only, so global loads issued ahead (the next token's raw inputs and
// record) stay in flight across them.  The one exchange through the workspace
// (each token's record, written by the threads that hold each value and read
// back in another mapping) is ordered by a full barrier after each stretch's
// recompute.
template <int D, bool IB, int MODE>
__global__ __launch_bounds__(bwd_threads<D>()) void backward_kernel(BwdParams p) {
  constexpr int NT = bwd_threads<D>();
  constexpr int NC = 3 * D;
  constexpr int NCT = (NC + NT - 1) / NT;  // conv channels per thread
  constexpr int CG = D / 4;
  constexpr int RG0 = NT / CG;
  constexpr int RG = RG0 < D ? RG0 : D;
  constexpr int RPT = D / RG;
  using V = Rec<D>;
  constexpr int NPRE = (V::SIZE + NT - 1) / NT;  // record floats per thread
  // the wave that reduces dbeta: the last one when it holds no conv channel
  constexpr int kDbetaWave = NC <= NT - 64 ? NT / 64 - 1 : (NT > 64 ? 1 : 0);

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int H = p.H, T = p.T;
  const int b = bh / H, h = bh - b * H;
  const int cch = H * NC;
  const int cg = tid % CG, rg = tid / CG;
  const bool active = rg < RG;
  using L = BwdLayout<D>;
  const int nch = L::nch(T);
  const size_t BH = (size_t)p.B * H;

  float* ckpt = p.ws + (size_t)bh * L::ckpt(T);                           // [nch][D][D]
  float* carry = p.ws + BH * L::ckpt(T) + (size_t)bh * L::CARRY;          // dS, ring
  float* slab = p.ws + BH * (L::ckpt(T) + L::CARRY) + ((size_t)p.buf * BH + bh) * L::slab(T) * L::STRETCH;
  // stretch l of the slab: states [kBwdChunk][D][D], then records [kBwdChunk][V::SIZE]
  auto slot_st = [&](int l) { return slab + (size_t)l * L::STRETCH; };
  auto slot_rec = [&](int l) { return slab + (size_t)l * L::STRETCH + (size_t)kBwdChunk * D * D; };

  // Reverse: token t's record in R[t % 3] (fields a, x~, q^, k^, y, u, dz,
  // alpha, dq^ and the scalars nq, nk, rq, rk, -, beta, q~ . dq^), its du and
  // dk^ in dus[t & 1] and dkn[t & 1]; red holds the row-group partials of du.
  __shared__ __attribute__((aligned(16))) float R[3][V::SIZE];
  __shared__ __attribute__((aligned(16))) float dus[2][D];
  __shared__ float dkn[2][D];
  __shared__ __attribute__((aligned(16))) float red[RG][D];

  auto rowidx = [&](int t) { return ((size_t)b * T + t) * H + h; };
  // global conv channel of head-local channel c (q | k | v)
  auto gch = [&](int c) { return c < D ? h * D + c : c < 2 * D ? H * D + h * D + (c - D) : 2 * H * D + h * D + (c - 2 * D); };
  auto raw = [&](int t, int c) -> float {
    if (t >= T) return 0.f;
    if (t < 0) return p.conv_in != nullptr ? load1<IB>(p.conv_in, ((size_t)b * 3 + (size_t)(3 + t)) * cch + gch(c)) : 0.f;
    const void* src = c < D ? p.q : c < 2 * D ? p.k : p.v;
    return load1<IB>(src, rowidx(t) * D + (c % D));
  };

  // this thread's conv channels c = tid + NT j: taps, the raw window t-3..t-1,
  // and a FIFO of the raw values, g (channel tid) and beta of tokens t..t+PF-1,
  // requested PF tokens before they are used (deeper measured slower)
  constexpr int PF = 1;
  float4 wch[NCT];
  float win[NCT][3], rq[PF][NCT], gq[PF], bq[PF];
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int c = tid + NT * j;
    wch[j] = c < NC ? *reinterpret_cast<const float4*>(p.conv_w + (size_t)gch(c) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  auto request = [&](int t, int k) {  // FIFO slot k <- token t
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int c = tid + NT * j;
      if (c < NC) rq[k][j] = raw(t, c);
    }
    gq[k] = tid < D && t < T ? load1<IB>(p.g, rowidx(t) * D + tid) : 0.f;
    bq[k] = t < T ? load1<IB>(p.beta, rowidx(t)) : 0.f;
  };
  auto start_window = [&](int t) {  // the raw window and the FIFO for token t
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int c = tid + NT * j;
      if (c < NC) {
        win[j][0] = raw(t - 3, c);
        win[j][1] = raw(t - 2, c);
        win[j][2] = raw(t - 1, c);
      }
    }
#pragma unroll
    for (int k = 0; k < PF; ++k) request(t + k, k);
  };


  // Forward-pass exchange buffers, double-buffered by token parity: a token
  // has at least two barriers, so token t + 2 rewrites a buffer only after
  // every thread has passed token t + 1's first barrier, i.e. has finished
  // reading token t's.
  __shared__ float fx[2][NC];                                   // x~
  __shared__ float fal[2][D];                                   // alpha = e^g
  __shared__ float fn[2][NT / 64][2];                  // per-wave |q~|^2, |k~|^2
  __shared__ __attribute__((aligned(16))) float fy[2][RG][D];   // row-group partials of y
  __shared__ __attribute__((aligned(16))) float fz[2][RG][D];   // row-group partials of z
  __shared__ __attribute__((aligned(16))) float fdz[D];         // dz of the token (recompute)
  __shared__ float fqa[RG];                                     // row-group partials of q~ . dq^

  // One forward token t on the register state s[]: conv + SiLU, the L2 norms,
  // S' = Diag(alpha) S, y = S'^T k^, u = beta (v^ - y), S_t = S' + k^ u^T.
  // Every thread derives the norms from the per-wave partials and sums y (and
  // z) for its own columns, so a token needs two barriers (three with z).
  // With vt, the token's record is written straight from the threads that
  // hold each value, and the output side of the reverse step is taken here
  // (gate4, do4: the gate and dL/do of this thread's 4 columns, row group 0):
  //   r = rms(z), n = z / r, dgate = do n s (1 - s), dz = (do s - n mean(do s n)) / r,
  //   dq^ = S_t dz  (s = sigmoid(gate)).
  f4 s[RPT];
  auto forward_step = [&](int t, float* vt, const f4& gate4, const f4& do4) {
    const int u = t & 1;
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int c = tid + NT * j;
      if (c < NC) {
        const float4 w = wch[j];
        const float a = w.x * win[j][0] + w.y * win[j][1] + w.z * win[j][2] + w.w * rq[0][j];
        const float x = a * sigmoidf_(a);
        fx[u][c] = x;
        if (vt != nullptr) {
          vt[V::A + c] = a;
          vt[V::X + c] = x;
        }
        if (c < D) pq += x * x;
        else if (c < 2 * D) pk += x * x;
        win[j][0] = win[j][1];
        win[j][1] = win[j][2];
        win[j][2] = rq[0][j];
      }
    }
    if (tid < D) fal[u][tid] = __expf(gq[0]);
    const float beta_t = bq[0];
#pragma unroll
    for (int k = 0; k + 1 < PF; ++k) {
#pragma unroll
      for (int j = 0; j < NCT; ++j) rq[k][j] = rq[k + 1][j];
      gq[k] = gq[k + 1];
      bq[k] = bq[k + 1];
    }
    request(t + PF, PF - 1);
    pq = group_sum<64>(pq);
    pk = group_sum<64>(pk);
    if ((tid & 63) == 0) {
      fn[u][tid >> 6][0] = pq;
      fn[u][tid >> 6][1] = pk;
    }
    lds_barrier();
    float nq = kL2Eps, nk = kL2Eps;
#pragma unroll
    for (int wv = 0; wv < NT / 64; ++wv) {
      nq += fn[u][wv][0];
      nk += fn[u][wv][1];
    }
    const float rq = rsqrtf(nq) * rsqrtf((float)D), rk = rsqrtf(nk);
    f4 yp = f4{0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        s[i] *= fal[u][r];
        yp += s[i] * (fx[u][D + r] * rk);
      }
      *reinterpret_cast<f4*>(&fy[u][rg][4 * cg]) = yp;
    }
    lds_barrier();
    if (active) {
      f4 y = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int r = 0; r < RG; ++r) y += *reinterpret_cast<const f4*>(&fy[u][r][4 * cg]);
      const f4 v4 = f4{fx[u][2 * D + 4 * cg], fx[u][2 * D + 4 * cg + 1], fx[u][2 * D + 4 * cg + 2],
                       fx[u][2 * D + 4 * cg + 3]};
      const f4 uu = beta_t * (v4 - y);
      f4 zp = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        s[i] += uu * (fx[u][D + r] * rk);
        zp += s[i] * (fx[u][r] * rq);
      }
      if (vt != nullptr) {
        *reinterpret_cast<f4*>(&fz[u][rg][4 * cg]) = zp;
        if (rg == 0) {
          *reinterpret_cast<f4*>(vt + V::Y + 4 * cg) = y;
          *reinterpret_cast<f4*>(vt + V::U + 4 * cg) = uu;
        }
        if (cg == 0) {
#pragma unroll
          for (int i = 0; i < RPT; ++i) {
            const int r = rg + RG * i;
            vt[V::QN + r] = fx[u][r] * rq;
            vt[V::KN + r] = fx[u][D + r] * rk;
            vt[V::AL + r] = fal[u][r];
          }
        }
      }
    }
    if (vt != nullptr) {
      if (tid == 0) {
        vt[V::SC + 0] = nq;
        vt[V::SC + 1] = nk;
        vt[V::SC + 2] = rq;
        vt[V::SC + 3] = rk;
        vt[V::SC + 5] = beta_t;
      }
      lds_barrier();
      const bool lead = active && rg == 0;  // the CG lanes of row group 0 hold z, 4 columns each
      f4 z = f4{0.f, 0.f, 0.f, 0.f};
      if (lead) {
#pragma unroll 4
        for (int r = 0; r < RG; ++r) z += *reinterpret_cast<const f4*>(&fz[u][r][4 * cg]);
      }
      const float zz = group_sum<CG>(lead ? z.x * z.x + z.y * z.y + z.z * z.z + z.w * z.w : 0.f);
      const float rr = sqrtf(zz * (1.0f / D) + kRmsEps);
      const f4 n = z * (1.0f / rr);
      const f4 sg = f4{sigmoidf_(gate4.x), sigmoidf_(gate4.y), sigmoidf_(gate4.z), sigmoidf_(gate4.w)};
      const f4 dos = do4 * sg;
      const float dd =
          group_sum<CG>(lead ? dos.x * n.x + dos.y * n.y + dos.z * n.z + dos.w * n.w : 0.f) * (1.0f / D);
      if (lead) {
        *reinterpret_cast<f4*>(p.dgate + rowidx(t) * D + 4 * cg) = dos * n * (1.f - sg);
        const f4 dz = (dos - n * dd) * (1.0f / rr);
        *reinterpret_cast<f4*>(vt + V::DZ + 4 * cg) = dz;
        *reinterpret_cast<f4*>(&fdz[4 * cg]) = dz;
      }
      lds_barrier();
      const f4 dz = *reinterpret_cast<const f4*>(&fdz[4 * cg]);
      float qa = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float part = active ? s[i].x * dz.x + s[i].y * dz.y + s[i].z * dz.z + s[i].w * dz.w : 0.f;
        const float v = group_sum<CG>(part);  // (S_t dz)_r
        if (active && cg == 0) {
          const int r = rg + RG * i;
          vt[V::DQ + r] = v;
          qa += fx[u][r] * v;
        }
      }
      if (active && cg == 0) fqa[rg] = qa;
      lds_barrier();
      if (tid == 0) {
        float a = 0.f;
        for (int r = 0; r < RG; ++r) a += fqa[r];
        vt[V::SC + 6] = a;  // q~ . dq^
      }
    }
  };

  // ---- 2. recompute one stretch: the state entering each token, each token's record
  if constexpr (MODE == kModeRecompute) {
    const int l = blockIdx.y;
    const int ch = p.ch_lo + l;
    const int t0 = ch * kBwdChunk, t1 = min(T, t0 + kBwdChunk);
    float* st = slot_st(l);
    float* rec = slot_rec(l);
    if (active) {
      const float* src = ckpt + (size_t)ch * D * D;
#pragma unroll
      for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const f4*>(src + (size_t)(rg + RG * i) * D + 4 * cg);
    }
    start_window(t0);
    // gate and dL/do (4 columns per lane of row group 0) are requested a token
    // ahead: loads and stores share one in-order counter, so a load waited for
    // right after stores waits for them
    auto gate4_of = [&](int t) {
      const size_t i = rowidx(t) * D + 4 * cg;
      return f4{load1<IB>(p.gate, i), load1<IB>(p.gate, i + 1), load1<IB>(p.gate, i + 2), load1<IB>(p.gate, i + 3)};
    };
    auto do4_of = [&](int t) { return *reinterpret_cast<const f4*>(p.dO + rowidx(t) * D + 4 * cg); };
    const bool lead = tid < CG;
    f4 gate_n = lead ? gate4_of(t0) : f4{0.f, 0.f, 0.f, 0.f};
    f4 do_n = lead ? do4_of(t0) : f4{0.f, 0.f, 0.f, 0.f};
    for (int t = t0; t < t1; ++t) {
      float* vt = rec + (size_t)(t - t0) * V::SIZE;
      const f4 gate_t = gate_n, do_t = do_n;
      if (lead && t + 1 < t1) {
        gate_n = gate4_of(t + 1);
        do_n = do4_of(t + 1);
      }
      if (active) {
        float* dst = st + (size_t)(t - t0) * D * D;
#pragma unroll
        for (int i = 0; i < RPT; ++i) *reinterpret_cast<f4*>(dst + (size_t)(rg + RG * i) * D + 4 * cg) = s[i];
      }
      forward_step(t, vt, gate_t, do_t);
    }
    return;
  }

  // ---- 3. reverse over the slab's stretches (the records come from the recompute launch)
  // Token t's step has a state side and a channel side.  The state side carries
  // dS from token to token: dS += q^ dz^T, du = dS^T k^, dk^ = dS u + S' dy,
  // dS' = dS + k^ dy^T, dg = rowsum(dS' * S'), dS <- Diag(alpha) dS'.  The
  // channel side (the L2-norm, SiLU and conv-transpose backward of the token's
  // q, k and v channels, and dbeta) needs only the token's record, du and dk^,
  // and the conv ring, which it walks in token order.  So the loop runs the
  // state side of token t and then the channel side of token t + 1: two
  // barriers per token.  The buffers make that safe: R[t % 3] is rewritten
  // two tokens after its channel side read it, dus / dkn[t & 1] one token
  // after, each time with both barriers of a token in between.
  f4 dS[RPT];
  float ring[NCT][3];  // da of tokens t+1, t+2, t+3 for this thread's channels
  const bool first_slab = p.ch_hi >= nch;  // the slab holding the last token
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = RPT * rg + i;
      const float* src = first_slab ? p.dS_T + (size_t)bh * D * D : carry;
      dS[i] = first_slab && p.dS_T == nullptr ? f4{0.f, 0.f, 0.f, 0.f}
                                              : *reinterpret_cast<const f4*>(src + (size_t)r * D + 4 * cg);
    }
  }
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int c = tid + NT * j;
#pragma unroll
    for (int k = 0; k < 3; ++k) ring[j][k] = !first_slab && c < NC ? carry[(size_t)D * D + (size_t)k * NC + c] : 0.f;
  }

  // Gradients are stored one token late, after the next token's loads are
  // issued (the counter is in order), so the store latency stays off the chain:
  // dg of the token whose state side ran last (t_sd), and dq, dk, dv and dbeta
  // of the token whose channel side ran last (t_cd).
  int t_sd = -1, t_cd = -1;
  float dbeta_def = 0.f, dg_def[RPT], dx_def[NCT];
  // d = 128: the row sums of dk^ and dg are reduced together (see the state
  // side), and lane cg ends with row RPT rg + bfly_row of one of them
  constexpr bool kButterfly = CG == 32 && RPT == 8;
  const int bfly_row = 4 * ((cg >> 3) & 1) + 2 * ((cg >> 2) & 1) + ((cg >> 1) & 1);
  // Each thread's gradient array, chosen once: chosen per store, the choice
  // between the three kernel-argument pointers became a per-lane load of the
  // argument block whose use waited for every memory operation in flight,
  // the state loads just issued included.
  float* dx_dst[NCT];
#pragma unroll
  for (int j = 0; j < NCT; ++j) {
    const int c = tid + NT * j;
    dx_dst[j] = c < D ? p.dq + c : c < 2 * D ? p.dk + (c - D) : p.dv + (c - 2 * D);
  }
  auto flush = [&]() {
    if (t_sd >= 0 && active) {
      const size_t rw = rowidx(t_sd);
      if constexpr (kButterfly) {
        if ((cg & 17) == 16) p.dg[rw * D + RPT * rg + bfly_row] = dg_def[0];
      } else if (cg == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) p.dg[rw * D + RPT * rg + i] = dg_def[i];
      }
    }
    if (t_cd >= 0) {
      const size_t rw = rowidx(t_cd);
      if (tid == kDbetaWave * 64) p.dbeta[rw] = dbeta_def;
#pragma unroll
      for (int j = 0; j < NCT; ++j) {
        const int c = tid + NT * j;
        if (c < NC) dx_dst[j][rw * D] = dx_def[j];
      }
    }
    t_sd = t_cd = -1;
  };
  const int wv = tid >> 6, ln = tid & 63;
  // the wave holds k channels (channel c = tid + NT j)
  bool kwave = false;
#pragma unroll
  for (int j = 0; j < NCT; ++j) kwave |= 64 * wv + NT * j < 2 * D && 64 * wv + NT * j + 64 > D;
  // channel side of token tc (its state side has run and a barrier followed)
  auto channel_side = [&](int tc) {
    const float* Rc = R[tc % 3];
    const float* dknc = dkn[tc & 1];
    const float* dusc = dus[tc & 1];
    const float* sc = Rc + V::SC;  // nq, nk, rq, rk, -, beta, q~ . dq^
    // k~ . dk^, summed by each wave that holds k channels, for itself
    float bb = 0.f;
    if (kwave) {
      for (int c = ln; c < D; c += 64) bb += Rc[V::X + D + c] * dknc[c];
      bb = group_sum<64>(bb);
    }
    if (wv == kDbetaWave) {
      float db = 0.f;
      for (int c = ln; c < D; c += 64) db += dusc[c] * (Rc[V::X + 2 * D + c] - Rc[V::Y + c]);
      dbeta_def = group_sum<64>(db);
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int c = tid + NT * j;
      if (c < NC) {
        const float xc = Rc[V::X + c];
        float dx;
        if (c < D) dx = sc[2] * (Rc[V::DQ + c] - xc * sc[6] / sc[0]);
        else if (c < 2 * D) dx = sc[3] * (dknc[c - D] - xc * bb / sc[1]);
        else dx = sc[5] * dusc[c - 2 * D];
        const float a = Rc[V::A + c];
        const float sa = sigmoidf_(a);
        const float da = dx * sa * (1.f + a * (1.f - sa));
        const float4 w = wch[j];
        float dr = w.w * da + w.z * ring[j][0] + w.y * ring[j][1] + w.x * ring[j][2];
        // the last three tokens are also conv_out's rows
        if (p.dconv_out != nullptr && tc >= T - 3) dr += p.dconv_out[((size_t)b * 3 + (tc - (T - 3))) * cch + gch(c)];
        dx_def[j] = dr;
        ring[j][2] = ring[j][1];
        ring[j][1] = ring[j][0];
        ring[j][0] = da;
      }
    }
    t_cd = tc;
  };

  // The reverse holds rows RPT rg .. RPT rg + RPT - 1 of dS (consecutive, so
  // the per-row values of a token come in 16-byte LDS reads).
  auto rows_of = [&](const float* base, float (&out)[RPT]) {
    if constexpr (RPT % 4 == 0) {
#pragma unroll
      for (int q4 = 0; q4 < RPT / 4; ++q4) {
        const f4 v = *reinterpret_cast<const f4*>(base + RPT * rg + 4 * q4);
        out[4 * q4] = v.x; out[4 * q4 + 1] = v.y; out[4 * q4 + 2] = v.z; out[4 * q4 + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) out[i] = base[RPT * rg + i];
    }
  };
  int t_pend = -1;  // the token whose channel side comes next
  // the state entering token t (stored by the recompute), requested a token
  // ahead into prev_n
  const int t_lo = p.ch_lo * kBwdChunk;
  auto state_at = [&](int t) { return slot_st(t / kBwdChunk - p.ch_lo) + (size_t)(t % kBwdChunk) * D * D; };
  f4 prev_n[RPT];
  if (active && p.ch_hi > p.ch_lo) {
    const float* src = state_at(min(T, p.ch_hi * kBwdChunk) - 1);
#pragma unroll
    for (int i = 0; i < RPT; ++i) prev_n[i] = *reinterpret_cast<const f4*>(src + (size_t)(RPT * rg + i) * D + 4 * cg);
  }
  for (int ch = p.ch_hi - 1; ch >= p.ch_lo; --ch) {
    const int t0 = ch * kBwdChunk, t1 = min(T, t0 + kBwdChunk);
    const float* rec = slot_rec(ch - p.ch_lo);
    // the next token's record requested one token ahead
    float pre[NPRE];
    {
      const float* vt = rec + (size_t)(t1 - 1 - t0) * V::SIZE;
#pragma unroll
      for (int j = 0; j < NPRE; ++j) {
        const int i = tid + NT * j;
        pre[j] = i < V::SIZE ? vt[i] : 0.f;
      }
    }
    for (int t = t1 - 1; t >= t0; --t) {
      float* const Rt = R[t % 3];
#pragma unroll
      for (int j = 0; j < NPRE; ++j) {
        const int i = tid + NT * j;
        if (i < V::SIZE) Rt[i] = pre[j];
      }
      f4 prev[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) prev[i] = prev_n[i];
      if (active && t - 1 >= t_lo) {
        const float* src = state_at(t - 1);
#pragma unroll
        for (int i = 0; i < RPT; ++i) prev_n[i] = *reinterpret_cast<const f4*>(src + (size_t)(RPT * rg + i) * D + 4 * cg);
      }
      if (t > t0) {
        const float* vt = rec + (size_t)(t - 1 - t0) * V::SIZE;
#pragma unroll
        for (int j = 0; j < NPRE; ++j) {
          const int i = tid + NT * j;
          pre[j] = i < V::SIZE ? vt[i] : 0.f;
        }
      }
      flush();  // dg of token t + 1, the channel gradients of token t + 2
      lds_barrier();
      // state side; alpha, q^ and k^ of this thread's RPT consecutive rows
      float qn[RPT], kn[RPT], al[RPT];
      rows_of(Rt + V::QN, qn);
      rows_of(Rt + V::KN, kn);
      rows_of(Rt + V::AL, al);
      f4 sp[RPT];
      f4 dup = f4{0.f, 0.f, 0.f, 0.f};
      if (active) {
        const f4 dz = *reinterpret_cast<const f4*>(&Rt[V::DZ + 4 * cg]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          sp[i] = prev[i] * al[i];
          dS[i] += dz * qn[i];
          dup += dS[i] * kn[i];
        }
      }
      // du = dS^T k^: every thread sums the row groups' partials of its own
      // columns; row group 0 keeps du for the channel side.  With 32 column
      // groups a wave holds two row groups of the same columns (lanes l and
      // l + 32): they are added in the wave first, so half as many partials go
      // through LDS.
      constexpr int NRED = CG == 32 ? RG / 2 : RG;
      if constexpr (CG == 32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dup[e] += __shfl_xor(dup[e], 32, 64);
        if (active && (rg & 1) == 0) *reinterpret_cast<f4*>(&red[rg >> 1][4 * cg]) = dup;
      } else {
        if (active) *reinterpret_cast<f4*>(&red[rg][4 * cg]) = dup;
      }
      lds_barrier();
      if (active) {
        f4 du = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int r = 0; r < NRED; ++r) du += *reinterpret_cast<const f4*>(&red[r][4 * cg]);
        if (rg == 0) *reinterpret_cast<f4*>(&dus[t & 1][4 * cg]) = du;
        const f4 u = *reinterpret_cast<const f4*>(&Rt[V::U + 4 * cg]);
        const f4 dy = -Rt[V::SC + 5] * du;
        // this thread's 4-column parts of dk^ and of rowsum(dS' * S') (alpha is
        // inside S') for its rows, summed over the CG threads of the row group
        float kps[RPT], gps[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          // dk^ = dS u + S' dy, with dS before the dy term
          float kp = dS[i].x * u.x + dS[i].y * u.y + dS[i].z * u.z + dS[i].w * u.w;
          kp += sp[i].x * dy.x + sp[i].y * dy.y + sp[i].z * dy.z + sp[i].w * dy.w;
          dS[i] += dy * kn[i];  // dS'
          kps[i] = kp;
          gps[i] = dS[i].x * sp[i].x + dS[i].y * sp[i].y + dS[i].z * sp[i].z + dS[i].w * sp[i].w;
          dS[i] *= al[i];  // dS_{t-1}
        }
        if constexpr (kButterfly) {
          // 16 sums over 32 lanes by recursive halving: at each exchange a lane
          // keeps half of its values and adds its partner's copy of that half
          // (partners lane ^ 16, ^ 15, ^ 7, ^ 2, then ^ 1 for the last value).
          // Lane cg ends with the sum of value 8 b4 + bfly_row (bits b4..b1 of
          // cg; value k < 8 is row k's dk^ part, k >= 8 row k - 8's dg part).
          const bool b4 = cg & 16, b3 = cg & 8, b2 = cg & 4, b1 = cg & 2;
          float a8[8], a4[4], a2[2];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            a8[k] = (b4 ? gps[k] : kps[k]) + __shfl_xor(b4 ? kps[k] : gps[k], 16, 64);
#pragma unroll
          for (int k = 0; k < 4; ++k) a4[k] = (b3 ? a8[k + 4] : a8[k]) + dpp_mov<0x140>(b3 ? a8[k] : a8[k + 4]);
#pragma unroll
          for (int k = 0; k < 2; ++k) a2[k] = (b2 ? a4[k + 2] : a4[k]) + dpp_mov<0x141>(b2 ? a4[k] : a4[k + 2]);
          float e = (b1 ? a2[1] : a2[0]) + dpp_mov<0x4E>(b1 ? a2[0] : a2[1]);
          e += dpp_mov<0xB1>(e);
          if (!b4 && !(cg & 1)) dkn[t & 1][RPT * rg + bfly_row] = e;
          dg_def[0] = e;
        } else {
#pragma unroll
          for (int i = 0; i < RPT; ++i) {
            const float kp = group_sum<CG>(kps[i]);
            dg_def[i] = group_sum<CG>(gps[i]);
            if (cg == 0) dkn[t & 1][RPT * rg + i] = kp;
          }
        }
      }
      t_sd = t;
      // channel side of the later token (its du and dk^ were written before
      // this token's first barrier)
      if (t_pend >= 0) channel_side(t_pend);
      t_pend = t;
    }
  }
  // the channel side of the launch's last token, after the stores of the
  // gradients still held (the channel side overwrites them)
  if (t_pend >= 0) {
    flush();
    lds_barrier();
    channel_side(t_pend);
  }
  flush();
  if (p.ch_lo > 0) {  // carry dS and the ring to the earlier slab
    if (active) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        *reinterpret_cast<f4*>(carry + (size_t)(RPT * rg + i) * D + 4 * cg) = dS[i];
    }
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int c = tid + NT * j;
      if (c < NC) {
#pragma unroll
        for (int k = 0; k < 3; ++k) carry[(size_t)D * D + (size_t)k * NC + c] = ring[j][k];
      }
    }
    return;
  }

  // ---- 4. state and history gradients (after the first stretch) ----------------------
  if (p.dS0 != nullptr && active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<f4*>(p.dS0 + (size_t)bh * D * D + (size_t)(RPT * rg + i) * D + 4 * cg) = dS[i];
  }
  if (p.dconv_in != nullptr) {
    // history row s + 3 (token s = -3..-1): sum over t = 0 .. s + 3 of w_{s-t+3} da_t
#pragma unroll
    for (int j = 0; j < NCT; ++j) {
      const int c = tid + NT * j;
      if (c < NC) {
        const float4 w = wch[j];
        const float wj[4] = {w.x, w.y, w.z, w.w};
        for (int s3 = 0; s3 < 3; ++s3) {  // s = s3 - 3
          float acc = 0.f;
          for (int t = 0; t <= s3 && t < 3; ++t) acc += wj[s3 - t] * ring[j][t];
          // with fewer than three tokens, conv_out row s3 - T is this history row
          if (p.dconv_out != nullptr && s3 - T >= 0) acc += p.dconv_out[((size_t)b * 3 + (s3 - T)) * cch + gch(c)];
          p.dconv_in[((size_t)b * 3 + (size_t)s3) * cch + gch(c)] = acc;
        }
      }
    }
  }
}

// The streams of the slab pipeline (default priority) and the events that
// order them, per host thread and device, for one reverse width (B*H rounded
// up to a multiple of 8, so each of the eight accelerator dies gets the same
// share: mask bits interleave over the dies).  The reverse launches run on
// that many compute units, the recompute launches on the others, alternating
// between two streams.  Created on first use and kept until kda_release() or
// process exit.
struct BwdPipe {
  int n_rev = 0;
  unsigned gen = 0;  // release_generation() when created
  hipStream_t rev = nullptr, rec[2] = {nullptr, nullptr};
  hipEvent_t fork = nullptr, rec_done[2] = {nullptr, nullptr}, rev_done[2] = {nullptr, nullptr};
  hipEvent_t join[3] = {nullptr, nullptr, nullptr};
};

// pp = nullptr (and KDA_OK) when the device is too small to split for this width.
int get_bwd_pipe(int heads, BwdPipe*& pp) {
  constexpr int kMaxDev = 64, kPerDev = 4;
  static thread_local BwdPipe pipes[kMaxDev][kPerDev];
  static thread_local int ncus[kMaxDev];
  pp = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    set_error("backward: hipGetDevice failed or device %d out of range", dev);
    return KDA_E_HIP;
  }
  if (ncus[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n <= 0) {
      set_error("backward: compute unit count query failed: %s", hipGetErrorString(e));
      return KDA_E_HIP;
    }
    ncus[dev] = n;
  }
  const int ncu = ncus[dev];
  const int n_rev = (heads + 7) / 8 * 8;
  if (n_rev + 32 > ncu) return KDA_OK;  // too few compute units left for the recompute
  // slots made before the last kda_release() hold destroyed handles
  const unsigned gen = release_generation();
  for (int k = 0; k < kPerDev; ++k)
    if (pipes[dev][k].n_rev != 0 && pipes[dev][k].gen != gen) pipes[dev][k] = BwdPipe{};
  BwdPipe* slot = nullptr;
  for (int k = 0; k < kPerDev && slot == nullptr; ++k)
    if (pipes[dev][k].n_rev == n_rev) slot = &pipes[dev][k];
  for (int k = 0; k < kPerDev && slot == nullptr; ++k)
    if (pipes[dev][k].n_rev == 0) slot = &pipes[dev][k];
  if (slot == nullptr) return KDA_OK;  // every slot holds another width: run on one stream
  if (slot->n_rev == 0) {
    uint32_t m_rev[32] = {0}, m_rec[32] = {0};
    const int nb = ncu < 32 * 32 ? ncu : 32 * 32;
    for (int c = 0; c < nb; ++c) (c < n_rev ? m_rev : m_rec)[c / 32] |= 1u << (c % 32);
    const uint32_t words = (uint32_t)((nb + 31) / 32);
    e = hipExtStreamCreateWithCUMask(&slot->rev, words, m_rev);
    for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipExtStreamCreateWithCUMask(&slot->rec[k], words, m_rec);
    hipEvent_t* evs[8] = {&slot->fork, &slot->rec_done[0], &slot->rec_done[1], &slot->rev_done[0],
                          &slot->rev_done[1], &slot->join[0], &slot->join[1], &slot->join[2]};
    for (int k = 0; k < 8 && e == hipSuccess; ++k) e = hipEventCreateWithFlags(evs[k], hipEventDisableTiming);
    // everything created is registered, so kda_release() (or process exit) frees it
    if (slot->rev != nullptr) keep(slot->rev);
    for (int k = 0; k < 2; ++k)
      if (slot->rec[k] != nullptr) keep(slot->rec[k]);
    for (int k = 0; k < 8; ++k)
      if (*evs[k] != nullptr) keep(*evs[k]);
    if (e != hipSuccess) {
      *slot = BwdPipe{};
      set_error("backward: stream / event creation failed: %s", hipGetErrorString(e));
      return KDA_E_HIP;
    }
    slot->n_rev = n_rev;
    slot->gen = gen;
  }
  pp = slot;
  return KDA_OK;
}

template <int D, bool IB>
int run_backward_typed(const kda_prefill_backward_args& a, hipStream_t st) {
  BwdParams p{a.B, a.T, a.H, a.q, a.k, a.v, a.conv_w, a.g, a.beta, a.gate, a.S0, a.conv_in, a.grad_o,
              a.grad_S_T, a.grad_conv_out, a.grad_q, a.grad_k, a.grad_v, a.grad_g, a.grad_beta, a.grad_gate, a.grad_S0,
              a.grad_conv_in, static_cast<float*>(a.workspace), 0, 0, 0};
  using L = BwdLayout<D>;
  const unsigned heads = (unsigned)((size_t)a.B * a.H);
  const int nch = L::nch(a.T), sl = L::slab(a.T);
  const dim3 block(bwd_threads<D>());
  // slabs from the last to the first; with no tokens, one reverse launch writes dS0 and dconv_in
  const int nslab = nch > 0 ? (nch + sl - 1) / sl : 1;
  BwdPipe* pp = nullptr;
  // under stream capture the slabs run on the caller's stream only (as for
  // the prefill: no forks onto the compute-unit-restricted streams)
  hipStreamCaptureStatus cap = hipStreamCaptureStatusActive;
  const bool capturing = hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone;
  if (nslab > 1 && !capturing) {
    const int rc = get_bwd_pipe((int)heads, pp);
    if (rc != KDA_OK) return rc;
  }
  const bool piped = pp != nullptr;
  // the state at every stretch start, from the chunkwise forward (fp32 operands)
  {
    kda_prefill_args f{};
    f.B = a.B; f.T = a.T; f.H = a.H; f.dk = a.dk; f.dv = a.dv; f.chunk = kBwdChunk;
    f.in_dtype = a.in_dtype; f.out_dtype = KDA_F32;
    f.q = a.q; f.k = a.k; f.v = a.v; f.conv_w = a.conv_w; f.g = a.g; f.beta = a.beta; f.gate = a.gate;
    f.S0 = a.S0; f.conv_in = a.conv_in;
    f.decay_form = KDA_DECAY_DIRECT;
    if (a.T > 0) {
      const int rc = launch_prefill_states(f, kBwdChunk, static_cast<float*>(a.workspace), st);
      if (rc != KDA_OK) return rc;
    }
  }
  hipError_t e = hipSuccess;
  const char* what = "forward launch";
  if (e == hipSuccess && piped) {
    // the pipeline's streams start after the forward launch
    what = "event";
    e = hipEventRecord(pp->fork, st);
    for (int k = 0; k < 2 && e == hipSuccess; ++k) e = hipStreamWaitEvent(pp->rec[k], pp->fork, 0);
    if (e == hipSuccess) e = hipStreamWaitEvent(pp->rev, pp->fork, 0);
  }
  for (int i = 0; i < nslab && e == hipSuccess; ++i) {
    const int k = nslab - 1 - i;
    p.ch_lo = k * sl;
    p.ch_hi = nch < p.ch_lo + sl ? nch : p.ch_lo + sl;
    p.buf = i & 1;
    hipStream_t sa = piped ? pp->rec[i & 1] : st, sb = piped ? pp->rev : st;
    // the buffer is free once the reverse launch of slab i - 2 is done
    if (piped && i >= 2) e = hipStreamWaitEvent(sa, pp->rev_done[p.buf], 0);
    if (e == hipSuccess && p.ch_hi > p.ch_lo) {
      hipLaunchKernelGGL((backward_kernel<D, IB, kModeRecompute>), dim3(heads, (unsigned)(p.ch_hi - p.ch_lo)), block,
                         0, sa, p);
      e = hipGetLastError();
      what = "recompute launch";
    }
    if (e == hipSuccess && piped) {
      what = "event";
      e = hipEventRecord(pp->rec_done[i & 1], sa);
      if (e == hipSuccess) e = hipStreamWaitEvent(sb, pp->rec_done[i & 1], 0);
    }
    if (e == hipSuccess) {
      hipLaunchKernelGGL((backward_kernel<D, IB, kModeReverse>), dim3(heads), block, 0, sb, p);
      e = hipGetLastError();
      what = "reverse launch";
    }
    if (e == hipSuccess && piped) {
      what = "event";
      e = hipEventRecord(pp->rev_done[p.buf], sb);
    }
  }
  if (piped) {
    // the caller's stream resumes after the pipeline's work (also on an error above)
    hipStream_t all[3] = {pp->rec[0], pp->rec[1], pp->rev};
    hipError_t j = hipSuccess;
    for (int k = 0; k < 3 && j == hipSuccess; ++k) j = hipEventRecord(pp->join[k], all[k]);
    for (int k = 0; k < 3 && j == hipSuccess; ++k) j = hipStreamWaitEvent(st, pp->join[k], 0);
    if (e == hipSuccess && j != hipSuccess) {
      e = j;
      what = "event";
    }
  }
  if (e != hipSuccess) {
    set_error("backward: %s failed: %s", what, hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

template <int D>
int run_backward(const kda_prefill_backward_args& a, hipStream_t s) {
  return a.in_dtype == KDA_BF16 ? run_backward_typed<D, true>(a, s) : run_backward_typed<D, false>(a, s);
}

}  // namespace

size_t prefill_backward_workspace_bytes(const kda_prefill_backward_args& a) {
  size_t per = 0;
  switch (a.dk) {
    case 16: per = BwdLayout<16>::head_floats(a.T); break;
    case 32: per = BwdLayout<32>::head_floats(a.T); break;
    case 64: per = BwdLayout<64>::head_floats(a.T); break;
    case 128: per = BwdLayout<128>::head_floats(a.T); break;
    default: return 0;
  }
  return per * sizeof(float) * (size_t)a.B * a.H;
}

int launch_prefill_backward(const kda_prefill_backward_args& a, hipStream_t s) {
  switch (a.dk) {
    case 16: return run_backward<16>(a, s);
    case 32: return run_backward<32>(a, s);
    case 64: return run_backward<64>(a, s);
    case 128: return run_backward<128>(a, s);
    default:
      set_error("backward: head dim %d not in {16,32,64,128}", a.dk);
      return KDA_E_UNSUPPORTED;
  }
}

}  // namespace kda
