/*
 * kda_peaks.h -- C ABI of libkda_peaks.so: microbenchmarks that measure this
 * GPU's own peaks, so kernel rates can be reported against the measured
 * figures beside the vendor ones (MI355X: 8 TB/s HBM3E, 2.5 PFLOP/s dense
 * fp16/bf16 matrix cores).  They are not part of the KDA computation.
 *
 * Launches are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream); time them with events on that stream.  Return codes: 0 on success,
 * -1 NULL pointer, -2 bad size, -3 misaligned pointer, -7 launch failure.
 */
#ifndef KDA_PEAKS_H
#define KDA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fetch-modify-write of `bytes` of fp32 in place with the decode step's access
 * pattern (one 256-thread workgroup per 64 KiB block, sixteen 16-byte
 * non-temporal loads per thread issued before any store):
 * buf[i] = buf[i] * 1.0000001f + 1e-7f.  `buf` is device memory owned by the
 * caller, 16-byte aligned; bytes is a positive multiple of 65536.  lds_bytes
 * (0 .. 160 KiB) of unused dynamic LDS per workgroup caps how many workgroups
 * share a compute unit.  HBM bytes moved: 2 * bytes. */
int kda_peak_fmw(float* buf, size_t bytes, int lds_bytes, void* stream);

/* Read-only (direction 0: every 16-byte piece loaded non-temporally and
 * summed, nothing stored while the buffer holds zeros) or write-only
 * (direction 1: zeros stored non-temporally) stream over `bytes` of the same
 * 64 KiB blocks, with the same constraints as kda_peak_fmw.  HBM bytes moved:
 * bytes.  The two directions' rates bound any mix of reads and writes. */
int kda_peak_stream(float* buf, size_t bytes, int direction, void* stream);

/* Read + write ceiling: every 64 KiB block of `src` is read (sixteen 16-byte
 * non-temporal loads per 256 threads) and written to the same offset of `dst`
 * before its workgroup ends, by workgroups of `threads` threads (256, 512 or
 * 1024).  src == dst: in place, dst[i] = src[i] * 1.0000001f + 1e-7f
 * (fetch-modify-write); otherwise dst[i] = src[i] (copy), and the two buffers
 * must not overlap.  Both device memory owned by the caller, 16-byte aligned;
 * bytes a positive multiple of 65536.  HBM bytes moved: 2 * bytes. */
int kda_peak_rw(const float* src, float* dst, size_t bytes, int threads, void* stream);

/* `blocks` workgroups of four waves, each wave issuing chains * iters
 * v_mfma_f32_16x16x32_f16 in `chains` (4 or 8) independent accumulation chains
 * on register operands (no memory traffic in the loop); one fp32 per thread is
 * written to out[blocks * 256] so the work is not removed.
 * FLOP = blocks * 4 * chains * iters * 16 * 16 * 32 * 2. */
int kda_peak_mfma(float* out, int blocks, int iters, int chains, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_PEAKS_H */
