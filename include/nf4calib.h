/*
 * nf4calib.h -- C ABI of the measurement kernels that calibrate the roofline
 * of the NF4 QLoRA library on one MI355X (gfx950).  They compute nothing of
 * the layer; they give the achievable ceilings that the layer's kernels are
 * quoted against beside the published peaks (8 TB/s HBM, 2.5 PFLOP/s dense
 * bf16 MFMA): a plain streaming read of device memory, a loop of bf16
 * matrix-core instructions on register operands, and that loop fed like the
 * fused GEMM's inner loop (LDS fragments, with or without the dequantizing
 * lookups).
 *
 * Conventions as in nf4qlora.h: device pointers, caller-owned memory, work
 * enqueued on `stream` (a hipStream_t, NULL = the null stream), no
 * allocation or synchronization, status 0 on success.
 */
#ifndef NF4CALIB_H
#define NF4CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of device memory at `buf` (16-byte aligned, bytes a multiple
 * of 16) once, with 16-byte loads from `workgroups` workgroups of 256
 * threads (0: the number that are resident on the device at once); the XOR
 * of what each workgroup read is written to sink[workgroup] (uint32, device,
 * one entry per workgroup launched), so no load can be dropped.  Returns 1 for a bad argument, 5 for a failed launch. */
int nf4calib_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups, void* stream);

/* Run `iters` iterations of 8 independent v_mfma_f32_32x32x16_bf16 per wave
 * (operands in registers: bf16 values with random mantissa bits that change
 * every iteration, as a GEMM's operands do; fp32 accumulators) on
 * `workgroups` workgroups of
 * `waves` waves (64 threads each; 0 workgroups: 4 per compute unit).  Each
 * instruction is 32*32*16 multiply-adds, i.e. 32768 flops; the total is
 * workgroups * waves * iters * 8 * 32768.  The accumulators' sum goes to
 * sink[workgroup] (fp32, device; `workgroups` entries).  Returns 1 for a
 * bad argument, 5 for a failed launch. */
int nf4calib_mfma(int iters, int workgroups, int waves, float* sink, void* stream);

/* The fused forward GEMM's inner loop without its memory traffic: one
 * workgroup of 8 waves per compute unit, each wave a 256 x 32 slab of eight
 * 32x32 fp32 accumulators; per iteration it issues 8
 * v_mfma_f32_32x32x16_bf16, each followed by the 16-byte LDS read of its A
 * fragment for the next iteration (one LDS fragment per instruction, as in
 * the GEMM's 256-token tiles), and with `dequant` = 1 also the byte-plane
 * lookup that turns one dword of eight 4-bit codes into the next B operand
 * (the GEMM's per-slice dequantization).  Flops: workgroups * 8 waves *
 * iters * 8 * 32768.  `workgroups` 0: one per compute unit.  sink: fp32,
 * device, 8 entries per workgroup.  Returns 1 for a bad argument (dequant
 * not 0 or 1 included), 5 for a failed launch. */
int nf4calib_mfma_tile(int iters, int workgroups, int dequant, float* sink, void* stream);

/* Workgroups the read and MFMA-loop calls launch when passed 0 (device 0
 * query). */
int nf4calib_default_workgroups(int which /* 0 read, 1 mfma */);

#ifdef __cplusplus
}
#endif

#endif /* NF4CALIB_H */
