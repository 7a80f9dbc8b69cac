/*
 * cosa_calib.h -- measurement-only microbenchmarks for MI355X (gfx950).
 *
 * Not part of the attention method: these kernels measure the attainable
 * bf16 MFMA rate and the attainable HBM streaming-read rate on the device at
 * hand, so that the prefill kernel's rate can be stated as a fraction of what the
 * chip delivers as well as of its published peaks.  Library: libcosa_calib.so.
 *
 * Both calls only enqueue work on `stream` (asynchronous); the caller times them
 * with events.  Pointers are device pointers owned by the caller.  Errors:
 * COSA_CALIB_ERR_ARG for a bad argument, COSA_CALIB_ERR_LAUNCH when the launch
 * fails; nothing is enqueued then.
 */
#ifndef COSA_CALIB_H
#define COSA_CALIB_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COSA_CALIB_OK 0
#define COSA_CALIB_ERR_ARG -1
#define COSA_CALIB_ERR_LAUNCH -2

/* Independent chains of v_mfma_f32_32x32x16_bf16: num_workgroups workgroups of
 * 256 threads, each wave running `iters` rounds of 8 MFMAs on 8 accumulators.
 * out: fp32 [num_workgroups * 4] (one checksum per wave, keeps the work live).
 * num_workgroups >= 1, iters >= 1. */
int32_t cosa_calib_mfma_bf16(float* out, int32_t num_workgroups, int32_t iters, hipStream_t stream);

/* The same chains on data-like operands: bf16 values with random signs and mantissas and
 * exponents over about 2^-8 .. 2^8 (a hash of seed, lane and element), two operand sets taken
 * in turn, so the MFMA datapath toggles as on real data; for rates sustained over long runs,
 * where power sets the clock.  `iters` counts rounds of 8 MFMAs as above and must be even
 * (>= 2); the flop count is cosa_calib_mfma_bf16_flop(num_workgroups, iters). */
int32_t cosa_calib_mfma_bf16_data(float* out, int32_t num_workgroups, int32_t iters, uint32_t seed,
                                  hipStream_t stream);

/* Floating-point operations one cosa_calib_mfma_bf16 (or _data) call performs (2 per multiply-add). */
double cosa_calib_mfma_bf16_flop(int32_t num_workgroups, int32_t iters);

/* Streaming read of `bytes` bytes at src (16-byte aligned, bytes a multiple of 16)
 * with 16-byte loads, grid-stride over num_workgroups workgroups of 256 threads.
 * out: uint32 [num_workgroups] (one XOR checksum per workgroup). */
int32_t cosa_calib_read(const void* src, size_t bytes, uint32_t* out, int32_t num_workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* COSA_CALIB_H */
