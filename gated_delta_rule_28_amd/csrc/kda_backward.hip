// kda_backward.hip -- gradients of the KDA prefill (training: the 1M-token
// context of "Gemma 4 31B vs Kimi K3", component table, long-context training
// row), for the definition of "Kimi K3, previewed", section "Kimi Delta
// Attention - the workhorse" and the KDA rows of the component tables.
//
// One workgroup per (b, h), token by token, all in fp32:
//   1. forward: the recurrence over the whole sequence, storing the state at
//      every chunk start (kBwdChunk tokens) in the workspace;
//   2. the chunks in reverse: each is recomputed from its stored state (the
//      state entering every token and the token's vectors go to the
//      workspace), then walked back token by token with the state gradient dS
//      in registers.
// Reverse step of token t (dS = dL/dS_t, do = dL/do_t; s = sigmoid(gate)):
//   dgate = do n s (1 - s);  dz = (do s - n mean(do s n)) / r
//   dq^ = S_t dz;  dS += q^ dz^T;  du = dS^T k^;  dk^ = dS u
//   dbeta = du . (v^ - y);  dv^ = beta du;  dy = -beta du
//   dS' = dS + k^ dy^T;  dk^ += S' dy;  dg = rowsum(dS' * S');  dS <- Diag(alpha) dS'
// then the L2-norm, SiLU and conv backward (conv transpose over a 3-token ring
// of the pre-SiLU gradients).  The state uses the decode kernel's layout:
// thread (cg = tid % CG, rg = tid / CG) holds rows rg + RG i of the 4 columns
// 4cg..4cg+3, so row sums are lane sums over the CG lanes of a row group and
// column sums go through LDS.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int kBwdThreads = 256;
constexpr int kBwdChunk = 64;  // tokens between stored states

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
  float* dq;
  float* dk;
  float* dv;
  float* dg;
  float* dbeta;
  float* dgate;
  float* dS0;
  float* dconv_in;
  float* ws;
};

// floats of one token's vectors in the workspace: a, x~ (3d each), q^, k^, y,
// u, z (d each), then scalars nq, nk, rq, rk, r, beta (8 slots)
template <int D>
struct Vec {
  static constexpr int A = 0, X = 3 * D, QN = 6 * D, KN = 7 * D, Y = 8 * D, U = 9 * D, Z = 10 * D;
  static constexpr int SC = 11 * D;
  static constexpr int SIZE = 11 * D + 8;
};

template <int D>
__host__ __device__ constexpr size_t bwd_head_floats(int T) {
  const size_t nch = (size_t)(T + kBwdChunk - 1) / kBwdChunk;
  return (nch + kBwdChunk) * D * D + (size_t)kBwdChunk * Vec<D>::SIZE;
}

template <int D, bool IB>
__global__ __launch_bounds__(kBwdThreads) void backward_kernel(BwdParams p) {
  constexpr int NC = 3 * D;
  constexpr int CG = D / 4;
  constexpr int RG0 = kBwdThreads / CG;
  constexpr int RG = RG0 < D ? RG0 : D;
  constexpr int RPT = D / RG;
  using V = Vec<D>;

  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int H = p.H, T = p.T;
  const int b = bh / H, h = bh - b * H;
  const int cch = H * NC;
  const int cg = tid % CG, rg = tid / CG;
  const bool active = rg < RG;
  const int nch = (T + kBwdChunk - 1) / kBwdChunk;

  float* ckpt = p.ws + (size_t)bh * bwd_head_floats<D>(T);     // [nch][D][D]
  float* st = ckpt + (size_t)nch * D * D;                      // [kBwdChunk][D][D]
  float* vec = st + (size_t)kBwdChunk * D * D;                 // [kBwdChunk][V::SIZE]

  // (16-byte aligned: rows of these are read as float4)
  __shared__ float xa[NC], xs[NC];                 // pre-SiLU a, x~ of the current token
  __shared__ float al[D], qn[D], kn[D], yv[D], zv[D];
  __shared__ __attribute__((aligned(16))) float uv[D];
  __shared__ __attribute__((aligned(16))) float dzs[D];
  __shared__ __attribute__((aligned(16))) float dus[D];
  __shared__ __attribute__((aligned(16))) float dys[D];
  __shared__ float dqn[D], dkn[D];
  __shared__ __attribute__((aligned(16))) float red[2][RG][D];
  __shared__ float ring[3][NC];                    // da of tokens t+1, t+2, t+3
  __shared__ float sc[16];  // nq, nk, rq, rk, -, beta, -, -, q~.dq^, k~.dk^

  auto rowidx = [&](int t) { return ((size_t)b * T + t) * H + h; };
  // global conv channel of head-local channel c (q | k | v)
  auto gch = [&](int c) { return c < D ? h * D + c : c < 2 * D ? H * D + h * D + (c - D) : 2 * H * D + h * D + (c - 2 * D); };
  auto raw = [&](int t, int c) -> float {
    if (t < 0) return p.conv_in != nullptr ? load1<IB>(p.conv_in, ((size_t)b * 3 + (size_t)(3 + t)) * cch + gch(c)) : 0.f;
    const void* src = c < D ? p.q : c < 2 * D ? p.k : p.v;
    return load1<IB>(src, rowidx(t) * D + (c % D));
  };

  // per-token vectors of token t into LDS (xa, xs, al, qn, kn, sc[0..5])
  auto token_vectors = [&](int t) {
    for (int c = tid; c < NC; c += kBwdThreads) {
      const float4 w = *reinterpret_cast<const float4*>(p.conv_w + (size_t)gch(c) * 4);
      const float a = w.x * raw(t - 3, c) + w.y * raw(t - 2, c) + w.z * raw(t - 1, c) + w.w * raw(t, c);
      xa[c] = a;
      xs[c] = a * sigmoidf_(a);
    }
    for (int c = tid; c < D; c += kBwdThreads) al[c] = __expf(load1<IB>(p.g, rowidx(t) * D + c));
    __syncthreads();
    if (tid < 64) {
      float sq = 0.f, sk = 0.f;
      for (int c = tid; c < D; c += 64) {
        sq += xs[c] * xs[c];
        sk += xs[D + c] * xs[D + c];
      }
      sq = group_sum<64>(sq);
      sk = group_sum<64>(sk);
      if (tid == 0) {
        const float nq = sq + kL2Eps, nk = sk + kL2Eps;
        sc[0] = nq;
        sc[1] = nk;
        sc[2] = rsqrtf(nq) * rsqrtf((float)D);
        sc[3] = rsqrtf(nk);
        sc[5] = load1<IB>(p.beta, rowidx(t));
      }
    }
    __syncthreads();
    for (int c = tid; c < D; c += kBwdThreads) {
      qn[c] = xs[c] * sc[2];
      kn[c] = xs[D + c] * sc[3];
    }
    __syncthreads();
  };

  // column sums over the rows: partial[4] of this thread's column group -> out[D]
  auto colsum2 = [&](const f4& pa, const f4& pb, float* outa, float* outb) {
    if (active) {
      *reinterpret_cast<f4*>(&red[0][rg][4 * cg]) = pa;
      *reinterpret_cast<f4*>(&red[1][rg][4 * cg]) = pb;
    }
    __syncthreads();
    for (int c = tid; c < D; c += kBwdThreads) {
      float sa = 0.f, sb = 0.f;
      for (int r = 0; r < RG; ++r) {
        sa += red[0][r][c];
        sb += red[1][r][c];
      }
      outa[c] = sa;
      if (outb != nullptr) outb[c] = sb;
    }
    __syncthreads();
  };

  // one forward token on the register state s[]: S' = Diag(al) S, y, u, S_t
  // (and z when want_z); leaves yv, uv (and zv) in LDS
  f4 s[RPT];
  auto forward_token = [&](bool want_z) {
    f4 yp = f4{0.f, 0.f, 0.f, 0.f};
    if (active) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        s[i] *= al[r];
        yp += s[i] * kn[r];
      }
    }
    colsum2(yp, yp, yv, nullptr);
    for (int c = tid; c < D; c += kBwdThreads) uv[c] = sc[5] * (xs[2 * D + c] - yv[c]);
    __syncthreads();
    f4 zp = f4{0.f, 0.f, 0.f, 0.f};
    if (active) {
      const f4 u = *reinterpret_cast<const f4*>(&uv[4 * cg]);
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        s[i] += u * kn[r];
        zp += s[i] * qn[r];
      }
    }
    if (want_z) colsum2(zp, zp, zv, nullptr);
  };

  // ---- 1. forward over the sequence, the state at every chunk start ----------
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      s[i] = p.S0 != nullptr ? *reinterpret_cast<const f4*>(p.S0 + (size_t)bh * D * D + (size_t)r * D + 4 * cg)
                             : f4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int t = 0; t < T; ++t) {
    if (t % kBwdChunk == 0 && active) {
      float* dst = ckpt + (size_t)(t / kBwdChunk) * D * D;
#pragma unroll
      for (int i = 0; i < RPT; ++i) *reinterpret_cast<f4*>(dst + (size_t)(rg + RG * i) * D + 4 * cg) = s[i];
    }
    token_vectors(t);
    forward_token(false);
  }

  // ---- 2. the chunks in reverse ---------------------------------------------------
  f4 dS[RPT];
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      dS[i] = p.dS_T != nullptr ? *reinterpret_cast<const f4*>(p.dS_T + (size_t)bh * D * D + (size_t)r * D + 4 * cg)
                                : f4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int c = tid; c < 3 * NC; c += kBwdThreads) (&ring[0][0])[c] = 0.f;
  __syncthreads();

  for (int ch = nch - 1; ch >= 0; --ch) {
    const int t0 = ch * kBwdChunk, t1 = min(T, t0 + kBwdChunk);
    // recompute: the state entering each token and the token's vectors
    if (active) {
      const float* src = ckpt + (size_t)ch * D * D;
#pragma unroll
      for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const f4*>(src + (size_t)(rg + RG * i) * D + 4 * cg);
    }
    for (int t = t0; t < t1; ++t) {
      if (active) {
        float* dst = st + (size_t)(t - t0) * D * D;
#pragma unroll
        for (int i = 0; i < RPT; ++i) *reinterpret_cast<f4*>(dst + (size_t)(rg + RG * i) * D + 4 * cg) = s[i];
      }
      token_vectors(t);
      forward_token(true);
      float* vt = vec + (size_t)(t - t0) * V::SIZE;
      for (int c = tid; c < NC; c += kBwdThreads) {
        vt[V::A + c] = xa[c];
        vt[V::X + c] = xs[c];
      }
      for (int c = tid; c < D; c += kBwdThreads) {
        vt[V::QN + c] = qn[c];
        vt[V::KN + c] = kn[c];
        vt[V::Y + c] = yv[c];
        vt[V::U + c] = uv[c];
        vt[V::Z + c] = zv[c];
      }
      if (tid < 6) vt[V::SC + tid] = sc[tid];
      __syncthreads();
    }
    // reverse
    for (int t = t1 - 1; t >= t0; --t) {
      const float* vt = vec + (size_t)(t - t0) * V::SIZE;
      for (int c = tid; c < NC; c += kBwdThreads) {
        xa[c] = vt[V::A + c];
        xs[c] = vt[V::X + c];
      }
      for (int c = tid; c < D; c += kBwdThreads) {
        qn[c] = vt[V::QN + c];
        kn[c] = vt[V::KN + c];
        yv[c] = vt[V::Y + c];
        uv[c] = vt[V::U + c];
        zv[c] = vt[V::Z + c];
        al[c] = __expf(load1<IB>(p.g, rowidx(t) * D + c));
      }
      if (tid < 6) sc[tid] = vt[V::SC + tid];
      __syncthreads();
      // output side: r, dgate, dz
      if (tid < 64) {
        float zz = 0.f;
        for (int c = tid; c < D; c += 64) zz += zv[c] * zv[c];
        zz = group_sum<64>(zz);
        const float r = sqrtf(zz * (1.0f / D) + kRmsEps);
        float dd = 0.f;
        for (int c = tid; c < D; c += 64) {
          const float n = zv[c] / r;
          const float sg = sigmoidf_(load1<IB>(p.gate, rowidx(t) * D + c));
          const float dov = p.dO[rowidx(t) * D + c];
          p.dgate[rowidx(t) * D + c] = dov * n * sg * (1.f - sg);
          dd += dov * sg * n;
        }
        dd = group_sum<64>(dd) * (1.0f / D);
        for (int c = tid; c < D; c += 64) {
          const float n = zv[c] / r;
          const float sg = sigmoidf_(load1<IB>(p.gate, rowidx(t) * D + c));
          dzs[c] = (p.dO[rowidx(t) * D + c] * sg - n * dd) / r;
        }
      }
      __syncthreads();
      // state side
      f4 sp[RPT];
      float rq_part[RPT];
      f4 dup = f4{0.f, 0.f, 0.f, 0.f};
      if (active) {
        const f4 dz = *reinterpret_cast<const f4*>(&dzs[4 * cg]);
        const f4 u = *reinterpret_cast<const f4*>(&uv[4 * cg]);
        const float* src = st + (size_t)(t - t0) * D * D;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + RG * i;
          const f4 prev = *reinterpret_cast<const f4*>(src + (size_t)r * D + 4 * cg);
          sp[i] = prev * al[r];
          const f4 stt = sp[i] + u * kn[r];
          rq_part[i] = stt.x * dz.x + stt.y * dz.y + stt.z * dz.z + stt.w * dz.w;  // (S_t dz)_r partial
          dS[i] += dz * qn[r];
          dup += dS[i] * kn[r];
        }
      }
      // dq^ = S_t dz: row sums over the CG lanes of a row group
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float v = group_sum<CG>(active ? rq_part[i] : 0.f);
        if (active && cg == 0) dqn[rg + RG * i] = v;
      }
      colsum2(dup, dup, dus, nullptr);  // du = dS^T k^
      // dbeta, dv^, dy
      if (tid < 64) {
        float db = 0.f;
        for (int c = tid; c < D; c += 64) db += dus[c] * (xs[2 * D + c] - yv[c]);
        db = group_sum<64>(db);
        if (tid == 0) p.dbeta[rowidx(t)] = db;
      }
      for (int c = tid; c < D; c += kBwdThreads) dys[c] = -sc[5] * dus[c];
      __syncthreads();
      if (active) {
        const f4 u = *reinterpret_cast<const f4*>(&uv[4 * cg]);
        const f4 dy = *reinterpret_cast<const f4*>(&dys[4 * cg]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const int r = rg + RG * i;
          // dk^ = dS u + S' dy, with dS before the dy term
          float kp = dS[i].x * u.x + dS[i].y * u.y + dS[i].z * u.z + dS[i].w * u.w;
          kp += sp[i].x * dy.x + sp[i].y * dy.y + sp[i].z * dy.z + sp[i].w * dy.w;
          dS[i] += dy * kn[r];  // dS'
          float gp = dS[i].x * sp[i].x + dS[i].y * sp[i].y + dS[i].z * sp[i].z + dS[i].w * sp[i].w;
          kp = group_sum<CG>(kp);
          gp = group_sum<CG>(gp);
          if (cg == 0) {
            dkn[r] = kp;
            p.dg[rowidx(t) * D + r] = gp;  // rowsum(dS' * S'): alpha is inside S'
          }
          dS[i] *= al[r];  // dS_{t-1}
        }
      }
      __syncthreads();
      // L2 norms, SiLU, conv transpose
      if (tid < 64) {
        float a = 0.f, bb = 0.f;
        for (int c = tid; c < D; c += 64) {
          a += xs[c] * dqn[c];
          bb += xs[D + c] * dkn[c];
        }
        a = group_sum<64>(a);
        bb = group_sum<64>(bb);
        if (tid == 0) {
          sc[8] = a;
          sc[9] = bb;
        }
      }
      __syncthreads();
      for (int c = tid; c < NC; c += kBwdThreads) {
        float dx;
        if (c < D) dx = sc[2] * (dqn[c] - xs[c] * sc[8] / sc[0]);
        else if (c < 2 * D) dx = sc[3] * (dkn[c - D] - xs[c] * sc[9] / sc[1]);
        else dx = sc[5] * dus[c - 2 * D];
        const float a = xa[c];
        const float sa = sigmoidf_(a);
        const float da = dx * sa * (1.f + a * (1.f - sa));
        const float4 w = *reinterpret_cast<const float4*>(p.conv_w + (size_t)gch(c) * 4);
        const float dr = w.w * da + w.z * ring[0][c] + w.y * ring[1][c] + w.x * ring[2][c];
        float* dst = c < D ? p.dq : c < 2 * D ? p.dk : p.dv;
        dst[rowidx(t) * D + (c % D)] = dr;
        ring[2][c] = ring[1][c];
        ring[1][c] = ring[0][c];
        ring[0][c] = da;
      }
      __syncthreads();
    }
  }

  // ---- 3. state and history gradients ------------------------------------------------
  if (p.dS0 != nullptr && active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<f4*>(p.dS0 + (size_t)bh * D * D + (size_t)(rg + RG * i) * D + 4 * cg) = dS[i];
  }
  if (p.dconv_in != nullptr) {
    // history row s + 3 (token s = -3..-1): sum over t = 0 .. s + 3 of w_{s-t+3} da_t
    for (int c = tid; c < NC; c += kBwdThreads) {
      const float4 w = *reinterpret_cast<const float4*>(p.conv_w + (size_t)gch(c) * 4);
      const float wj[4] = {w.x, w.y, w.z, w.w};
      for (int s = -3; s < 0; ++s) {
        float acc = 0.f;
        for (int t = 0; t <= s + 3 && t < 3; ++t) acc += wj[s - t + 3] * ring[t][c];
        p.dconv_in[((size_t)b * 3 + (size_t)(s + 3)) * cch + gch(c)] = acc;
      }
    }
  }
}

template <int D>
int run_backward(const kda_prefill_backward_args& a, hipStream_t s) {
  BwdParams p{a.B, a.T, a.H, a.q, a.k, a.v, a.conv_w, a.g, a.beta, a.gate, a.S0, a.conv_in, a.grad_o,
              a.grad_S_T, a.grad_q, a.grad_k, a.grad_v, a.grad_g, a.grad_beta, a.grad_gate, a.grad_S0,
              a.grad_conv_in, static_cast<float*>(a.workspace)};
  const unsigned grid = (unsigned)((size_t)a.B * a.H);
  if (a.in_dtype == KDA_BF16)
    hipLaunchKernelGGL((backward_kernel<D, true>), dim3(grid), dim3(kBwdThreads), 0, s, p);
  else
    hipLaunchKernelGGL((backward_kernel<D, false>), dim3(grid), dim3(kBwdThreads), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("backward launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

}  // namespace

size_t prefill_backward_workspace_bytes(const kda_prefill_backward_args& a) {
  size_t per = 0;
  switch (a.dk) {
    case 16: per = bwd_head_floats<16>(a.T); break;
    case 32: per = bwd_head_floats<32>(a.T); break;
    case 64: per = bwd_head_floats<64>(a.T); break;
    case 128: per = bwd_head_floats<128>(a.T); break;
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
