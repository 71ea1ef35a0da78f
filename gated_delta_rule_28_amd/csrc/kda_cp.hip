// kda_cp.hip -- context-parallel prefill helpers: the prefix composition of
// segment state maps, each segment's raw conv history, and the identity
// states the fragments are formed from.
//
// The long-context training row of "Gemma 4 31B vs Kimi K3" (component table)
// says that ranks exchange only fixed-size state fragments.  The state update is affine in the state, so a
// segment of tokens maps the state S entering it to M S + N (M dk x dk, N
// dk x dv).  With dk = dv, two prefills of the segment give both: from S = 0
// the final state is N, from S = I it is M + N.  Composing the segments in
// order gives each segment its entering state:
//   S_0 = S0,   S_{r+1} = (P_r - N_r) S_r + N_r,   P_r = M_r + N_r.
#include "kda_internal.h"

#include <cstdint>

namespace kda {

namespace {

constexpr int kThreads = 256;

struct ComposeParams {
  int B, R, H;
  const float* N;
  const float* P;
  const float* S0;
  float* S_start;
  float* S_T;
};

// Workgroup (b, h, column half) walks the R segments: the columns of the state
// are independent under X' = (P - N) X + N, so each of two workgroups per
// (b, h) takes D/2 of them.  The segment's map P - N (all of it) and the
// workgroup's columns of X sit in LDS; thread (ty, tx) of a GY x GX grid
// computes a TB x TB block of its columns of X' in fp32.  Global accesses are
// 16-byte pieces.
template <int D>
struct ComposeShape {
  static constexpr int W = D / 2;                 // columns per workgroup
  static constexpr int THREADS = D == 16 ? 128 : D == 32 ? 256 : 1024;
  static constexpr int GX = D >= 64 ? 16 : 8;     // thread grid over the W columns
  static constexpr int GY = THREADS / GX;         // ... and over the D rows
  static constexpr int TB = W / GX;               // columns per thread
  static constexpr int TR = D / GY;               // rows per thread
  static constexpr int LDM = D + 1;               // map rows: row groups of a wave in different banks
  static constexpr int LDX = W + 4;               // state rows: 16-byte aligned
  static constexpr size_t LDS = ((size_t)D * LDM + (size_t)D * LDX) * sizeof(float);
  static_assert(TB >= 1 && TR >= 1 && GX * TB == W && GY * TR == D, "thread grid");
};

template <int D>
__global__ __launch_bounds__(ComposeShape<D>::THREADS) void cp_compose_kernel(ComposeParams p) {
  using Sh = ComposeShape<D>;
  constexpr int W = Sh::W, NT = Sh::THREADS, TB = Sh::TB, TR = Sh::TR, LDM = Sh::LDM, LDX = Sh::LDX;
  extern __shared__ float sm[];
  float* sM = sm;
  float* sX = sm + D * LDM;
  const int bh = blockIdx.x >> 1, half = blockIdx.x & 1;
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, ty = tid / Sh::GX, tx = tid % Sh::GX;
  const int c0 = half * W;  // first column of this workgroup
  constexpr size_t DD = (size_t)D * D;
  constexpr int Q = W / 4;  // float4 pieces per row of the workgroup's columns

  for (int idx = tid; idx < D * Q; idx += NT) {
    const int i = idx / Q, j = 4 * (idx - i * Q);
    const float4 x = p.S0 != nullptr ? *reinterpret_cast<const float4*>(p.S0 + (size_t)bh * DD + (size_t)i * D + c0 + j)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(sX + i * LDX + j) = x;
  }
  // P and N of segment r + 1 are requested while segment r's product runs
  constexpr int NQ = (D * D / 4 + NT - 1) / NT;  // float4 pieces per thread
  float4 pv[NQ], nv[NQ];
  auto request = [&](int r) {
    const size_t seg = ((size_t)(b * p.R + r) * p.H + h) * DD;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int idx = tid + NT * q;
      if (idx < D * D / 4) {
        pv[q] = *reinterpret_cast<const float4*>(p.P + seg + 4 * (size_t)idx);
        nv[q] = *reinterpret_cast<const float4*>(p.N + seg + 4 * (size_t)idx);
      }
    }
  };
  request(0);
  for (int r = 0; r < p.R; ++r) {
    const size_t seg = ((size_t)(b * p.R + r) * p.H + h) * DD;
    __syncthreads();  // X complete
    for (int idx = tid; idx < D * Q; idx += NT) {
      const int i = idx / Q, j = 4 * (idx - i * Q);
      *reinterpret_cast<float4*>(p.S_start + seg + (size_t)i * D + c0 + j) =
          *reinterpret_cast<const float4*>(sX + i * LDX + j);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int idx = tid + NT * q;
      if (idx < D * D / 4) {
        const int i = (4 * idx) / D, j = 4 * idx - i * D;
        float* m = sM + i * LDM + j;
        m[0] = pv[q].x - nv[q].x; m[1] = pv[q].y - nv[q].y; m[2] = pv[q].z - nv[q].z; m[3] = pv[q].w - nv[q].w;
      }
    }
    __syncthreads();  // map complete
    if (r + 1 < p.R) request(r + 1);
    float acc[TR][TB];
#pragma unroll
    for (int u = 0; u < TR; ++u)
#pragma unroll
      for (int v = 0; v < TB; ++v) acc[u][v] = p.N[seg + (size_t)(ty * TR + u) * D + c0 + tx * TB + v];
#pragma unroll 4
    for (int k = 0; k < D; ++k) {
      float a[TR], x[TB];
#pragma unroll
      for (int u = 0; u < TR; ++u) a[u] = sM[(ty * TR + u) * LDM + k];
#pragma unroll
      for (int v = 0; v < TB; ++v) x[v] = sX[k * LDX + tx * TB + v];
#pragma unroll
      for (int u = 0; u < TR; ++u)
#pragma unroll
        for (int v = 0; v < TB; ++v) acc[u][v] += a[u] * x[v];
    }
    __syncthreads();  // every thread has read X
#pragma unroll
    for (int u = 0; u < TR; ++u)
#pragma unroll
      for (int v = 0; v < TB; ++v) sX[(ty * TR + u) * LDX + tx * TB + v] = acc[u][v];
  }
  if (p.S_T != nullptr) {
    __syncthreads();
    for (int idx = tid; idx < D * Q; idx += NT) {
      const int i = idx / Q, j = 4 * (idx - i * Q);
      *reinterpret_cast<float4*>(p.S_T + (size_t)bh * DD + (size_t)i * D + c0 + j) =
          *reinterpret_cast<const float4*>(sX + i * LDX + j);
    }
  }
}

template <int D>
int run_compose(const ComposeParams& p, hipStream_t s) {
  using Sh = ComposeShape<D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&cp_compose_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)Sh::LDS);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(cp_compose_kernel<D>, dim3((unsigned)(2 * p.B * p.H)), dim3(Sh::THREADS), Sh::LDS, s, p);
    e = hipGetLastError();
  }
  if (e != hipSuccess) {
    set_error("context-parallel composition launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

// Raw conv history rows: block j of `nblk` per sequence b takes the three raw
// tokens before token (first + j) * L of q, k and v, in the packed channel
// order of conv_in; tokens before 0 come from conv_in (zeros if NULL).
// Elements are copied bit for bit (E: element type of in_dtype).  Grid:
// x over b * nblk + j, y over pieces of kHistPiece elements of the 3 x Cch rows.
constexpr int kHistPiece = 4 * kThreads;

template <typename E>
__global__ __launch_bounds__(kThreads) void cp_history_kernel(const E* q, const E* k, const E* v, const E* conv_in,
                                                              E* dst, int nblk, int first, int L, int T, int H,
                                                              int d) {
  const int blk = blockIdx.x;  // b * nblk + j
  const int b = blk / nblk, j = blk - b * nblk;
  const int hd = H * d;
  const int cch = 3 * hd;
  const long long t0 = (long long)(first + j) * L - 3;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int idx = blockIdx.y * kHistPiece + e * kThreads + threadIdx.x;
    if (idx >= 3 * cch) break;
    const int row = idx / cch, c = idx - row * cch;
    const long long t = t0 + row;
    E val;
    if (t < 0) {
      val = conv_in != nullptr ? conv_in[((size_t)b * 3 + (size_t)(3 + t)) * cch + c] : E(0);
    } else {
      const E* src = c < hd ? q : c < 2 * hd ? k : v;
      const int cc = c < hd ? c : c < 2 * hd ? c - hd : c - 2 * hd;
      val = src[((size_t)b * T + (size_t)t) * hd + cc];
    }
    dst[(size_t)blk * 3 * cch + idx] = val;
  }
}

__global__ __launch_bounds__(kThreads) void cp_identity_kernel(float* S, int d) {
  const size_t base = (size_t)blockIdx.x * d * d;
  for (int idx = threadIdx.x; idx < d * d; idx += kThreads) {
    const int i = idx / d, j = idx - i * d;
    S[base + idx] = i == j ? 1.f : 0.f;
  }
}

}  // namespace

int launch_cp_compose(const kda_cp_compose_args& a, hipStream_t s) {
  const ComposeParams p{a.B, a.R, a.H, a.N, a.P, a.S0, a.S_start, a.S_T};
  switch (a.d) {
    case 16: return run_compose<16>(p, s);
    case 32: return run_compose<32>(p, s);
    case 64: return run_compose<64>(p, s);
    case 128: return run_compose<128>(p, s);
    default:
      set_error("context-parallel composition: d=%d not in {16,32,64,128}", a.d);
      return KDA_E_UNSUPPORTED;
  }
}

int launch_cp_history(const kda_prefill_args& a, int nblk, int first, int L, void* dst, hipStream_t s) {
  const size_t rows = 3 * (size_t)a.H * (2 * a.dk + a.dv);
  const size_t pieces = (rows + kHistPiece - 1) / kHistPiece;
  if (pieces > 65535) {
    set_error("context-parallel history: %zu channels too many", rows / 3);
    return KDA_E_SHAPE;
  }
  const dim3 grid((unsigned)((size_t)a.B * nblk), (unsigned)pieces);
  if (a.in_dtype == KDA_BF16)
    hipLaunchKernelGGL(cp_history_kernel<uint16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.conv_in),
                       static_cast<uint16_t*>(dst), nblk, first, L, a.T, a.H, a.dk);
  else
    hipLaunchKernelGGL(cp_history_kernel<uint32_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const uint32_t*>(a.q), static_cast<const uint32_t*>(a.k),
                       static_cast<const uint32_t*>(a.v), static_cast<const uint32_t*>(a.conv_in),
                       static_cast<uint32_t*>(dst), nblk, first, L, a.T, a.H, a.dk);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("context-parallel history launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

int launch_cp_identity(float* S, size_t count, int d, hipStream_t s) {
  hipLaunchKernelGGL(cp_identity_kernel, dim3((unsigned)count), dim3(kThreads), 0, s, S, d);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("identity fill launch failed: %s", hipGetErrorString(e));
    return KDA_E_HIP;
  }
  return KDA_OK;
}

}  // namespace kda
