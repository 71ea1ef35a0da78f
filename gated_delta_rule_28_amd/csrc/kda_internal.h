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
// Expired bounded waits of the one-launch recurrence on the current device.
int wait_timeouts(unsigned* count);
// Test settings of the one-launch recurrence (see kda_debug_pipeline).
void debug_pipeline(unsigned wait_us, int withhold_slab);
bool prefill_split_eligible(const kda_prefill_args& a);
size_t prefill_split_workspace_bytes(const kda_prefill_args& a);
size_t prefill_split_workspace_min_bytes(const kda_prefill_args& a);
int launch_prefill_split(const kda_prefill_args& a, hipStream_t s);
// kda_prefill without a caller workspace or any allocation: the two-kernel
// path's workspace is a file-scope device array (kda_prefill_split.hip).
int launch_prefill_noalloc(const kda_prefill_args& a, hipStream_t s);

// One rank's share of context-parallel prefill on the two-kernel path: the
// workspace that keeps every chunk block between the two calls (0 when the
// sizes have no two-kernel path), the fragments N (from S = 0) and P (from
// S = I), and the finishing pass from the entering state a.S0.
size_t cp_rank_split_bytes(const kda_prefill_args& a);
int launch_cp_fragments_split(const kda_prefill_args& a, float* N, float* P, hipStream_t s);
int launch_cp_finish_split(const kda_prefill_args& a, hipStream_t s);

// Context-parallel helpers: the prefix composition; the raw conv history of
// `nblk` blocks per sequence (the three raw tokens before token (first + j) * L
// of block j, from conv_in before token 0) into dst [B * nblk, 3, Cch]; the
// identity in `count` d x d fp32 matrices.
int launch_cp_compose(const kda_cp_compose_args& a, hipStream_t s);
int launch_cp_history(const kda_prefill_args& a, int nblk, int first, int L, void* dst, hipStream_t s);
int launch_cp_identity(float* S, size_t count, int d, hipStream_t s);

// The state entering every kStateChunk-token chunk of a prefill ([B*H][chunks]
// [dk][dv] fp32, natural order), computed chunkwise with fp32 operands and no
// outputs (kda_prefill.hip): the backward's checkpoints.
constexpr int kStateChunk = 32;
int launch_prefill_states(const kda_prefill_args& a, int chunk, float* S_chunks, hipStream_t s);

// Prefill gradients (fp32, one workgroup per (b, h)) and their workspace.
size_t prefill_backward_workspace_bytes(const kda_prefill_backward_args& a);
int launch_prefill_backward(const kda_prefill_backward_args& a, hipStream_t s);

// Set the calling thread's last-error text (printf-style).
void set_error(const char* fmt, ...);

// Streams and events kept between calls (kda_api.cpp).  keep() registers one
// for kda_release(); the first registration also arranges the release at
// process exit.  A cached handle is valid while release_generation() still
// returns the value read when it was created.
void keep(hipStream_t s);
void keep(hipEvent_t e);
unsigned release_generation();

}  // namespace kda
