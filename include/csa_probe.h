/* csa_probe.h -- achievable-peak probes of the device (libcsa_probe.so).
 *
 * Measurement kernels that give the ceilings the hot-path kernels are read
 * against, next to the vendor's published peaks: a matrix-core loop (bf16
 * v_mfma_f32_32x32x16_bf16 on register operands, no memory traffic), a
 * streaming read of a large device buffer, and LDS reads in the two widths the
 * attention's operand paths use.  They are not part of the
 * attention path and share no code with libcsa.so.  The caller times a launch
 * (events on the same stream) and divides the work below by the time.
 *
 * Conventions: every pointer is a device pointer owned by the caller; calls
 * enqueue on `stream` and return without synchronizing; the return value is
 * 0 on success, otherwise a hipError_t (invalid arguments: hipErrorInvalidValue,
 * nothing enqueued).
 */
#ifndef CSA_PROBE_H
#define CSA_PROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix-core loop: n_wg workgroups of 256 threads (four waves); every wave
 * runs `iters` rounds of eight independent accumulation chains of
 * v_mfma_f32_32x32x16_bf16 on fixed register operands (bf16 values in (-1, 1)
 * from a hash of the lane), then thread i writes the sum of its accumulators
 * to sink[i] (sink: n_wg * 256 floats).  Work: csa_probe_mfma_flops(n_wg,
 * iters) flop.  n_wg >= 1, iters >= 1. */
int csa_probe_mfma_bf16(float *sink, int32_t n_wg, int32_t iters, hipStream_t stream);
double csa_probe_mfma_flops(int32_t n_wg, int32_t iters);

/* Streaming read: n_wg workgroups of 256 threads read `bytes` bytes at `buf`
 * once, 16 bytes per lane per non-temporal load with eight loads in flight per
 * thread (grid-stride order, so each load instruction of a wave covers 1 KiB
 * contiguous), and thread i writes the xor of the words it read to sink[i]
 * (sink: n_wg * 256 uint32).  bytes is a multiple of 16 and buf 16-byte
 * aligned. */
int csa_probe_read(const void *buf, size_t bytes, uint32_t *sink, int32_t n_wg,
                   hipStream_t stream);

/* LDS read rate: n_wg workgroups of 512 threads (eight waves), each over its
 * own 64 KiB LDS array; every wave issues `iters` rounds of eight independent
 * reads.  mode 0: 16-byte reads (a wave reads 1 KiB contiguous); mode 1: the
 * transposing 8-byte reads used for matrix-core operands (512 bytes per wave
 * instruction).  sink (2 * n_wg * 512 uint32): sink[2 i] is the sum of what
 * thread i read; sink[2 i + 1] holds, for the first thread of each workgroup,
 * the shader-clock cycles of its read loop (0 elsewhere).  Work:
 * csa_probe_lds_bytes(n_wg, iters, mode) bytes.  n_wg, iters >= 1. */
int csa_probe_lds(uint32_t *sink, int32_t n_wg, int32_t iters, int32_t mode,
                  hipStream_t stream);
double csa_probe_lds_bytes(int32_t n_wg, int32_t iters, int32_t mode);

#ifdef __cplusplus
}
#endif

#endif /* CSA_PROBE_H */
