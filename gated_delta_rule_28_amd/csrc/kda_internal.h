// kda_internal.h -- launcher interface between the C ABI (kda_api.cpp) and the
// kernels.  Launchers assume validated arguments; they return KDA_OK or
// KDA_E_UNSUPPORTED (no instantiation for the sizes) or KDA_E_HIP.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/kda.h"

namespace kda {

int launch_decode(const kda_decode_args& a, hipStream_t s);
int launch_decode_multi(const kda_decode_multi_args& a, hipStream_t s);
int launch_prefill(const kda_prefill_args& a, hipStream_t s);
int launch_prep(const kda_prep_args& a, hipStream_t s);

// Two-kernel prefill (bf16 inputs, chunk 64, dk = dv = 128) through a workspace.
bool prefill_split_eligible(const kda_prefill_args& a);
size_t prefill_split_workspace_bytes(const kda_prefill_args& a);
size_t prefill_split_workspace_min_bytes(const kda_prefill_args& a);
int launch_prefill_split(const kda_prefill_args& a, hipStream_t s);

// Context-parallel helpers: the prefix composition; the raw conv history of
// `nblk` blocks per sequence (the three raw tokens before token (first + j) * L
// of block j, from conv_in before token 0) into dst [B * nblk, 3, Cch]; the
// identity in `count` d x d fp32 matrices.
int launch_cp_compose(const kda_cp_compose_args& a, hipStream_t s);
int launch_cp_history(const kda_prefill_args& a, int nblk, int first, int L, void* dst, hipStream_t s);
int launch_cp_identity(float* S, size_t count, int d, hipStream_t s);

// Prefill gradients (fp32, one workgroup per (b, h)) and their workspace.
size_t prefill_backward_workspace_bytes(const kda_prefill_backward_args& a);
int launch_prefill_backward(const kda_prefill_backward_args& a, hipStream_t s);

// Set the calling thread's last-error text (printf-style).
void set_error(const char* fmt, ...);

}  // namespace kda
