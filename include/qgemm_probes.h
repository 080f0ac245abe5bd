/*
 * Measurement probes for MI355X (gfx950), built into libqgemm_probes.so beside
 * the GEMM library. They measure what the hardware sustains on the two units
 * that bound the GEMM kernels, so that their roofline fractions can be read
 * against achievable as well as published peaks:
 *   - a plain streaming read of device memory (the HBM bound of the
 *     memory-bound end of the batch range);
 *   - back-to-back matrix-core instructions on register operands (the bound of
 *     the compute-bound end).
 * They compute no GEMM and are not part of the qgemm_* interface.
 *
 * Conventions as in qgemm.h: `stream` is a hipStream_t (NULL = the default
 * stream), every call only enqueues work and returns 0 on success or a
 * negative QGEMM_ERR_* status (-1 bad argument, -6 HIP error).
 */
#ifndef QGEMM_PROBES_H
#define QGEMM_PROBES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device pointer `src` (16-byte aligned, bytes a
 * multiple of 16, at most 3 GiB) with 16-byte vector loads, eight in flight
 * per lane, from `workgroups` workgroups of 256 threads striding over the
 * buffer: with chunked = 0 a wave's eight 1 KB loads of a round lie one grid
 * width apart, with chunked = 1 they are 8 consecutive KB. Each wave writes
 * the sum of the 32-bit words it read, modulo 2^32, to its own uint32 of
 * `sink` (4 * workgroups words, given as `sink_words`; wave w of the grid at
 * sink[w]), so that the sum of the slots proves every byte was read. */
int qgemm_probe_stream_read(const void* src, int64_t bytes, void* sink, int64_t sink_words, int workgroups,
                            int chunked, void* stream);

/* Issues `iters` x 8 matrix-core instructions per wave (x 16 for kind 4),
 * four independent accumulators per wave, from `workgroups` workgroups of 256
 * threads. kind 0: v_mfma_f32_32x32x16_f16 (32768 flops each); kind 1:
 * v_mfma_f32_16x16x32_f16 (16384); kind 2: v_mfma_i32_16x16x64_i8 (32768
 * integer ops); kinds 3 and 4: v_mfma_f32_32x32x16_f16 whose A operand is
 * read from LDS, one 1 KB wave read (ds_read_b128) per instruction (kind 3)
 * or per two instructions (kind 4), with 16 KB of LDS per workgroup; kinds 5
 * and 6: kinds 0 and 2 on pseudo-random operands (fp16 uniform in [-1, 1),
 * int8 uniform over its range; kinds 0-4 feed small constants, and the rate
 * the chip sustains depends on the operand data). Each
 * wave writes one 32-bit word of its accumulators to
 * `sink` (at least 4 * workgroups 32-bit words, given as `sink_words`) so no
 * instruction is dead. */
int qgemm_probe_mfma(void* sink, int64_t sink_words, int workgroups, int iters, int kind, void* stream);

/* Floating-point or integer operations of one instruction of `kind`, 0 for an
 * unknown kind (kind 4 issues two instructions per iteration step: 16 per
 * iteration and wave). */
int64_t qgemm_probe_mfma_ops(int kind);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_PROBES_H */
