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

// Set the calling thread's last-error text (printf-style).
void set_error(const char* fmt, ...);

}  // namespace kda
