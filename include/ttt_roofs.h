/*
 * ttt_roofs.h -- measured roofs of the current device, exported by libttt.so
 * beside the TTT entry points of ttt.h.  The roofline fractions of the TTT
 * kernels are reported against the vendor's peak figures and against what
 * these plain kernels reach on the same GPU:
 *   - a streaming device-to-device copy (every byte read once and written
 *     once, 16-byte non-temporal accesses, four loads in flight per thread):
 *     achievable HBM bandwidth = 2 * bytes / time;
 *   - a dense MFMA loop (each wave issues independent accumulation chains of
 *     one MFMA shape, no memory traffic): achievable matrix-core throughput
 *     = flops / time;
 *   - an empty kernel: the floor of one launch, for steps as small as the
 *     single-token decode step (timed per launch in a HIP graph of many).
 * Each enqueues one kernel on `stream` and returns without synchronising; the
 * caller times them (e.g. with HIP events).  Errors: TTT_ERR_INVALID_ARG
 * (null pointer, negative or unaligned size, bad dtype, iters < 1, fewer
 * than one workgroup),
 * TTT_ERR_HIP (launch failed).
 */
#ifndef TTT_ROOFS_H
#define TTT_ROOFS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copies `bytes` bytes (a multiple of 16; src and dst 16-byte aligned, not
 * overlapping) from src to dst, both device memory owned by the caller.
 */
int ttt_roof_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * Runs `iters` iterations of 8 independent MFMA accumulations per wave on
 * `waves` waves (a multiple of 4: 4 per workgroup) and writes one float per
 * thread to out[waves * 64] (device memory) so the products are kept.
 * dtype 1: v_mfma_f32_16x16x32_bf16 (16384 flops each); dtype 0:
 * v_mfma_f32_16x16x4_f32 (2048 flops each).  Total flops =
 * waves * iters * 8 * (flops of one MFMA); returns that count through
 * *flops when flops is not NULL (host memory).
 */
int ttt_roof_mfma(float* out, int dtype, int64_t waves, int64_t iters, double* flops, void* stream);

/*
 * Launches an empty kernel of `workgroups` workgroups of 64 threads (1 to
 * 2^31 - 1).  It reads and writes nothing.
 */
int ttt_roof_launch(int64_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TTT_ROOFS_H */
