// kda_peaks.hip -- measured peaks of this GPU, for reporting kernel rates against
// what the hardware delivers beside the vendor figures (libkda_peaks.so).
//
//   peak_fmw_kernel   fetch-modify-write of fp32 blocks with the decode step's
//                     access pattern: one 256-thread workgroup per 64 KiB block,
//                     every thread requests its sixteen 16-byte pieces first
//                     (non-temporal), scales them, and writes them back in place.
//                     Bytes moved = 2 x block bytes per block.
//   peak_read_kernel / peak_write_kernel  the same blocks read only (summed,
//                     no store) or written only: each direction's ceiling.
//   peak_rw_kernel    the same 64 KiB blocks with 256, 512 or 1024 threads per
//                     block (16, 8 or 4 pieces per thread), either in place
//                     (fetch-modify-write) or copied to a second buffer: the
//                     read + write ceiling, swept over workgroup size.
//   peak_mfma_kernel  back-to-back v_mfma_f32_16x16x32_f16 on register operands,
//                     4 or 8 independent accumulators per wave, no memory
//                     traffic inside the loop.  FLOP = blocks x 4 waves x iters
//                     x chains x 16 x 16 x 32 x 2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda_peaks.h"

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kFmwThreads = 256;
constexpr int kFmwPieces = 16;  // 16-byte pieces per thread: 64 KiB per workgroup

// Dynamic LDS (unused) caps the workgroups per compute unit: the sweep finds
// the occupancy at which this pattern moves the most bytes.
__global__ __launch_bounds__(kFmwThreads) void peak_fmw_kernel(float* buf, float a, float b) {
  f4* p = reinterpret_cast<f4*>(buf) + (size_t)blockIdx.x * kFmwThreads * kFmwPieces;
  f4 s[kFmwPieces];
#pragma unroll
  for (int i = 0; i < kFmwPieces; ++i) s[i] = __builtin_nontemporal_load(p + i * kFmwThreads + threadIdx.x);
#pragma unroll
  for (int i = 0; i < kFmwPieces; ++i) __builtin_nontemporal_store(s[i] * a + b, p + i * kFmwThreads + threadIdx.x);
}

// Read-only and write-only streams of the same blocks: the two directions'
// ceilings, which bound any read + write mix.
__global__ __launch_bounds__(kFmwThreads) void peak_read_kernel(const float* buf, float* out) {
  const f4* p = reinterpret_cast<const f4*>(buf) + (size_t)blockIdx.x * kFmwThreads * kFmwPieces;
  f4 s[kFmwPieces];
#pragma unroll
  for (int i = 0; i < kFmwPieces; ++i) s[i] = __builtin_nontemporal_load(p + i * kFmwThreads + threadIdx.x);
  f4 t = s[0];
#pragma unroll
  for (int i = 1; i < kFmwPieces; ++i) t += s[i];
  const float v = t[0] + t[1] + t[2] + t[3];
  if (v == 12345.678f) out[blockIdx.x] = v;  // keeps the loads; never true for the zeroed buffers used
}

__global__ __launch_bounds__(kFmwThreads) void peak_write_kernel(float* buf, float a) {
  f4* p = reinterpret_cast<f4*>(buf) + (size_t)blockIdx.x * kFmwThreads * kFmwPieces;
  const f4 v = f4{a, a, a, a};
#pragma unroll
  for (int i = 0; i < kFmwPieces; ++i) __builtin_nontemporal_store(v, p + i * kFmwThreads + threadIdx.x);
}

// One 64 KiB block per workgroup of NT threads: every thread requests its
// 65536 / 16 / NT pieces first (non-temporal), then stores them, scaled in
// place (src == dst) or unchanged into dst.
template <int NT>
__global__ __launch_bounds__(NT) void peak_rw_kernel(const float* src, float* dst, float a, float b) {
  constexpr int NP = 65536 / 16 / NT;
  const f4* p = reinterpret_cast<const f4*>(src) + (size_t)blockIdx.x * NT * NP;
  f4* q = reinterpret_cast<f4*>(dst) + (size_t)blockIdx.x * NT * NP;
  f4 s[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) s[i] = __builtin_nontemporal_load(p + i * NT + threadIdx.x);
#pragma unroll
  for (int i = 0; i < NP; ++i) __builtin_nontemporal_store(s[i] * a + b, q + i * NT + threadIdx.x);
}

constexpr int kMfmaThreads = 256;

// NC independent accumulation chains per wave, each instruction reading
// register operands only.
template <int NC>
__global__ __launch_bounds__(kMfmaThreads) void peak_mfma_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  half8 x, y;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = (_Float16)(0.001f * (lane + e));
    y[e] = (_Float16)(0.002f * (lane - e));
  }
  f4 c[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) c[j] = f4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NC; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16((j & 1) ? x : y, (j & 2) ? x : y, c[j], 0, 0, 0);
  }
  f4 s = c[0];
#pragma unroll
  for (int j = 1; j < NC; ++j) s += c[j];
  out[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

extern "C" {

int kda_peak_fmw(float* buf, size_t bytes, int lds_bytes, void* stream) {
  const size_t block = (size_t)kFmwThreads * kFmwPieces * sizeof(f4);
  if (buf == nullptr) return -1;
  if (bytes == 0 || bytes % block != 0 || bytes / block > 0x7fffffffu) return -2;
  if (lds_bytes < 0 || lds_bytes > 160 * 1024) return -2;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -3;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(&peak_fmw_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          lds_bytes) != hipSuccess)
    return -7;
  hipLaunchKernelGGL(peak_fmw_kernel, dim3((unsigned)(bytes / block)), dim3(kFmwThreads), (unsigned)lds_bytes,
                     reinterpret_cast<hipStream_t>(stream), buf, 1.0000001f, 1e-7f);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int kda_peak_stream(float* buf, size_t bytes, int direction, void* stream) {
  const size_t block = (size_t)kFmwThreads * kFmwPieces * sizeof(f4);
  if (buf == nullptr) return -1;
  if (bytes == 0 || bytes % block != 0 || bytes / block > 0x7fffffffu || (direction != 0 && direction != 1)) return -2;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return -3;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(bytes / block));
  if (direction == 0) hipLaunchKernelGGL(peak_read_kernel, grid, dim3(kFmwThreads), 0, s, buf, buf);
  else hipLaunchKernelGGL(peak_write_kernel, grid, dim3(kFmwThreads), 0, s, buf, 0.f);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int kda_peak_rw(const float* src, float* dst, size_t bytes, int threads, void* stream) {
  const size_t block = 65536;
  if (src == nullptr || dst == nullptr) return -1;
  if (bytes == 0 || bytes % block != 0 || bytes / block > 0x7fffffffu) return -2;
  if (threads != 256 && threads != 512 && threads != 1024) return -2;
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) != 0) return -3;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 != d0 && s0 < d0 + bytes && d0 < s0 + bytes) return -2;  // partial overlap
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)(bytes / block));
  // in place: the fetch-modify-write scale; copy: unchanged values
  const float a = s0 == d0 ? 1.0000001f : 1.0f, b = s0 == d0 ? 1e-7f : 0.0f;
  if (threads == 256) hipLaunchKernelGGL(peak_rw_kernel<256>, grid, dim3(256), 0, s, src, dst, a, b);
  else if (threads == 512) hipLaunchKernelGGL(peak_rw_kernel<512>, grid, dim3(512), 0, s, src, dst, a, b);
  else hipLaunchKernelGGL(peak_rw_kernel<1024>, grid, dim3(1024), 0, s, src, dst, a, b);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

int kda_peak_mfma(float* out, int blocks, int iters, int chains, void* stream) {
  if (out == nullptr) return -1;
  if (blocks < 1 || iters < 1 || (chains != 4 && chains != 8)) return -2;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (chains == 4) hipLaunchKernelGGL(peak_mfma_kernel<4>, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, s, out, iters);
  else hipLaunchKernelGGL(peak_mfma_kernel<8>, dim3((unsigned)blocks), dim3(kMfmaThreads), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
