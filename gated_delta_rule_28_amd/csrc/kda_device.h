// kda_device.h -- gfx950 device helpers shared by the KDA kernels.
//
// Vector types, bf16/fp16 conversion, fast transcendental wrappers (single
// hardware instructions: v_exp_f32, v_rcp_f32, v_rsq_f32), wave/block
// reductions and the 16x16x32 matrix-core wrappers.
//
// Matrix-core lane layout (v_mfma_f32_16x16x32_{f16,bf16}, wave of 64 lanes,
// lane l, group g = l / 16, i = l % 16):
//   A operand (16 x 32): lane holds A[i][8g .. 8g+7]
//   B operand (32 x 16): lane holds B[8g .. 8g+7][i]
//   C/D       (16 x 16): lane holds D[4g .. 4g+3][i]
// Only the contraction index has to agree between A and B, so a kernel may
// permute it; the kernels use that to feed an accumulator straight back in as
// a B operand (see kda_prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kL2Eps = 1e-6f;   // L2 normalisation epsilon of q and k
constexpr float kRmsEps = 1e-5f;  // head-wise RMSNorm epsilon (model rms_norm_eps)

// ---- scalar math (one hardware instruction each, ~1 ulp) ----------------------
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_rsq(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float sigmoidf_(float x) { return fast_rcp(1.0f + fast_exp(-x)); }
__device__ __forceinline__ float siluf_(float x) { return x * fast_rcp(1.0f + fast_exp(-x)); }
// K3's bounded log-decay from its logit z, given e^A of the channel
// ("Kimi K3.1 Pro vs gpt-oss-120b", component table, row "Gated DeltaNet / KDA")
__device__ __forceinline__ float k3_decay(float z, float eA) { return -5.0f * sigmoidf_(eA * z); }

// ---- bf16 / fp16 ---------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ uint16_t f_to_bf16(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

// Load 8 consecutive activations (fp32 or bf16) as fp32.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, size_t idx, float* out) {
  if constexpr (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    out[0] = bf16lo(u.x); out[1] = bf16hi(u.x); out[2] = bf16lo(u.y); out[3] = bf16hi(u.y);
    out[4] = bf16lo(u.z); out[5] = bf16hi(u.z); out[6] = bf16lo(u.w); out[7] = bf16hi(u.w);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* base, size_t idx) {
  if constexpr (BF16) return bf16_to_f(reinterpret_cast<const uint16_t*>(base)[idx]);
  else return reinterpret_cast<const float*>(base)[idx];
}

template <bool BF16>
__device__ __forceinline__ void store1(void* base, size_t idx, float x) {
  if constexpr (BF16) reinterpret_cast<uint16_t*>(base)[idx] = f_to_bf16(x);
  else reinterpret_cast<float*>(base)[idx] = x;
}

// Store 4 consecutive outputs (fp32 or bf16).
template <bool BF16>
__device__ __forceinline__ void store4(void* base, size_t idx, float a, float b, float c, float d) {
  if constexpr (BF16) {
    uint2 u;
    u.x = (uint32_t)f_to_bf16(a) | ((uint32_t)f_to_bf16(b) << 16);
    u.y = (uint32_t)f_to_bf16(c) | ((uint32_t)f_to_bf16(d) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + idx) = u;
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + idx) = make_float4(a, b, c, d);
  }
}

// Non-temporal 16-byte accesses (data used once: the memory system keeps it
// out of its caches, which measured up to 18% more bandwidth per CU on
// streams that every CU runs at once).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename V16>
__device__ __forceinline__ void st_nt(void* p, const V16& v) {
  static_assert(sizeof(V16) == 16, "16-byte value");
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
}

// Store 8 consecutive outputs (fp32 or bf16) with 16-byte non-temporal stores.
template <bool BF16>
__device__ __forceinline__ void store8_nt(void* base, size_t idx, const float* x) {
  if constexpr (BF16) {
    uint4 u;
    u.x = (uint32_t)f_to_bf16(x[0]) | ((uint32_t)f_to_bf16(x[1]) << 16);
    u.y = (uint32_t)f_to_bf16(x[2]) | ((uint32_t)f_to_bf16(x[3]) << 16);
    u.z = (uint32_t)f_to_bf16(x[4]) | ((uint32_t)f_to_bf16(x[5]) << 16);
    u.w = (uint32_t)f_to_bf16(x[6]) | ((uint32_t)f_to_bf16(x[7]) << 16);
    st_nt(reinterpret_cast<uint16_t*>(base) + idx, u);
  } else {
    float* f = reinterpret_cast<float*>(base) + idx;
    st_nt(f, make_float4(x[0], x[1], x[2], x[3]));
    st_nt(f + 4, make_float4(x[4], x[5], x[6], x[7]));
  }
}

// Store 8 consecutive outputs (fp32 or bf16) with 16-byte stores.
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
    float* f = reinterpret_cast<float*>(base) + idx;
    *reinterpret_cast<float4*>(f) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(f + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

// ---- reductions ------------------------------------------------------------------
// DPP lane moves inside a row of 16 lanes: quad_perm xor 1 and xor 2, then
// half-row and row mirrors.  Each step pairs every lane with a lane of the
// other half of its current group, so after log2(W) steps every lane of an
// aligned group of W lanes holds the group's sum (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of the group gets the sum.  All lanes of a group must be active.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W >= 1 && W <= 64 && (W & (W - 1)) == 0, "W must be a power of two <= 64");
  if constexpr (W >= 2) x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (W >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (W >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror: other quad of the half-row
  if constexpr (W >= 16) x += dpp_mov<0x140>(x);  // row_mirror: other half of the row
  if constexpr (W >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (W >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// Maximum over the 64 lanes of a wave (every lane gets it); all lanes active.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  x = fmaxf(x, dpp_mov<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

// Workgroup barrier that waits only for this wave's LDS operations, not for its
// outstanding global loads (which __syncthreads' release fence would drain):
// loads issued for later stages stay in flight across it.  The memory clobber
// keeps the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- matrix core -----------------------------------------------------------------
__device__ __forceinline__ f4 mma_f16(const half8& a, const half8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma_bf16(const bf16x8& a, const bf16x8& b, const f4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace kda
