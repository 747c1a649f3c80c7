/*
 * qgceil.h -- C ABI of libqgceil.so, the measurement companion of
 * libqgemm.so. It is not part of the GEMM path: it holds the reference
 * kernels and host loops a benchmark needs to place a GEMM kernel's time
 * against what the chip delivers in the same process, on the same stream:
 *
 *   - an MFMA-only loop at the GEMM kernels' occupancy (the sustained matrix
 *     rate, and the shader clock it ran at);
 *   - a streaming read (the sustained HBM read rate);
 *   - how far vector work overlaps matrix work on one SIMD;
 *   - empty kernels (the runtime's launch cost, without and with a kernel
 *     argument block);
 *   - a host loop that times calls of a qg_run-shaped function.
 *
 * The DeepGEMM write-up (section 5.2) bases tuning on profiler evidence of
 * how busy the matrix units are and how much memory bandwidth is used; these
 * ceilings are the denominators of such fractions measured on this machine,
 * next to the published peaks.
 *
 * All pointers are device pointers unless stated otherwise. Every call
 * returns 0 on success or -1 when an argument is out of range, -6 when a
 * HIP call fails (the numbering of qgemm.h's QG_ERR_INVALID_ARG and
 * QG_ERR_HIP). Kernel launches are asynchronous on `stream`.
 */
#ifndef QGCEIL_H
#define QGCEIL_H

#include <stddef.h>
#include <stdint.h>

#include "qgemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA-only loop: `grid` workgroups of 8 waves (512 threads) that each hold
 * 96 KiB of LDS, so at most one workgroup runs per compute unit, as with the
 * 256 x 256 GEMM tile kernel. Every wave issues `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 on register operands (4 * 32768
 * flops per round), with no memory traffic in the loop.
 *   sink: grid floats (device), one accumulator value per workgroup so that
 *         nothing is optimised away;
 *   clk:  2 * grid uint64 (device): for each workgroup, shader-clock cycles
 *         (s_memtime) and 100 MHz reference ticks (s_memrealtime) spent in
 *         the loop; their ratio times 100 MHz is the clock the loop ran at.
 * Flops per launch: grid * 8 * iters * 4 * 32768. 1 <= grid <= 65535,
 * 1 <= iters <= 1 << 20. */
int qgc_mfma_loop(int grid, int iters, float* sink, uint64_t* clk, hipStream_t stream);

/* Streaming read of `bytes` (a multiple of 16, 0 < bytes < 2^31) at `src`
 * (16-byte aligned): `grid` workgroups of 256 threads, each thread with
 * eight 16-byte loads in flight, the workgroups walking the buffer in
 * grid-strided 32 KiB blocks. Each thread writes the XOR of every dword it
 * read to sink[thread] (grid * 256 dwords), so the XOR of the whole sink is
 * the XOR of the buffer's dwords. 1 <= grid <= 65535. */
int qgc_stream_read(const void* src, size_t bytes, int grid, uint32_t* sink, hipStream_t stream);

/* Issue overlap of matrix and vector work on one SIMD: `grid` workgroups
 * shaped like qgc_mfma_loop's (8 waves, 96 KiB of LDS, so two waves share
 * each SIMD). Every wave runs `iters` rounds; a round holds, interleaved one
 * MFMA to four VALU instructions,
 *   mode 1: four v_mfma_f32_16x16x32_bf16 on independent accumulators,
 *   mode 2: sixteen VALU instructions of one kind on eight independent
 *           chains,
 *   mode 3: both;
 * the VALU kind is 0: fp32 fused multiply-add (v_fma_f32); 1: the int4
 * unpack's bitwise pair (a byte permute and an and-or, eight pairs);
 * 2: fp32 fused multiply-add with an fp16 operand (v_fma_mix_f32).
 *   sink: grid floats (device), one value per workgroup so that nothing is
 *         optimised away;
 *   clk:  grid uint64 (device): for each workgroup, shader-clock cycles
 *         from the start of the rounds until all its waves have finished
 *         them (a workgroup barrier; per SIMD that is two waves' rounds).
 * 1 <= grid <= 65535, 1 <= iters <= 1 << 20, 1 <= mode <= 3, 0 <= kind <= 2
 * (kind is ignored for mode 1). */
int qgc_issue_mix(int mode, int kind, int grid, int iters, float* sink, uint64_t* clk, hipStream_t stream);

/* One launch of an empty kernel (one workgroup of 64 threads). */
int qgc_empty(hipStream_t stream);

/* A function with qg_run's signature. */
typedef int (*qgc_run_fn)(qg_handle*, const qg_operation*, float, const void*, const qg_layout*, const void*,
                          const qg_layout*, const void*, const qg_layout*, const void*, const qg_layout*, float,
                          const void*, const qg_layout*, void*, const qg_layout*, const qg_workspace*, hipStream_t);

/* Host time of `n` back-to-back calls fn(h, op, ...) with the same
 * arguments, in microseconds per call (steady clock, no synchronisation
 * inside the loop; the caller synchronises afterwards). `n` >= 1. Writes the
 * figure to *us_per_call (host pointer); a call that does not return 0 stops
 * the loop and its status is returned. */
int qgc_host_us_per_call(qgc_run_fn fn, int n, qg_handle* h, const qg_operation* op, float alpha, const void* A,
                         const qg_layout* Adesc, const void* U, const qg_layout* Udesc, const void* B,
                         const qg_layout* Bdesc, const void* V, const qg_layout* Vdesc, float beta, const void* C,
                         const qg_layout* Cdesc, void* D, const qg_layout* Ddesc, const qg_workspace* ws,
                         hipStream_t stream, double* us_per_call);

/* Host time of `n` back-to-back launches of an empty kernel (one workgroup
 * of 64 threads), microseconds per launch. arg_bytes 0: a kernel without
 * arguments; 256: one with a 256-byte argument block, which the runtime
 * copies on every launch (the GEMM kernels take one block of about that
 * size). Other values are rejected. */
int qgc_host_us_per_empty(int n, int arg_bytes, hipStream_t stream, double* us_per_call);

#ifdef __cplusplus
}
#endif

#endif /* QGCEIL_H */
