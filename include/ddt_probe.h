/* Roofline probes for libddt.so: the achievable bf16 MFMA rate and HBM
 * bandwidth of the device the library runs on, measured by the library's
 * own kernels.
 *
 * The verify-attention kernels are judged against the MI355X datasheet
 * peaks (dense bf16 MFMA 2.5 PFLOP/s at 2.4 GHz, HBM3E 8 TB/s).  These
 * probes measure what the device sustains on the same run:
 *
 *   - an MFMA loop (v_mfma_f32_32x32x16_bf16, four independent accumulator
 *     chains per wavefront) whose operands come from a caller buffer, so
 *     the same loop can run on random data and on zeros (the sustained
 *     rate under the board power limit depends on the operands);
 *   - a streaming read (every 16-byte word of a buffer, XOR-folded) and a
 *     streaming copy.
 *
 * They are measurement helpers, not steps of the verify path.  Every call
 * is asynchronous on `stream`; time it with events on that stream.  The
 * return value is 0 or a negative ddt_status (DDT_EINVAL for null pointers,
 * non-positive sizes or misaligned buffers, DDT_EHIP when the launch fails).
 * Nothing here allocates.
 */
#ifndef DDT_PROBE_H
#define DDT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per probe workgroup (four wavefronts). */
#define DDT_PROBE_THREADS 256
/* Operand buffer of ddt_probe_mfma_bf16: 2 * 4 * 64 * 8 bf16 values. */
#define DDT_PROBE_MFMA_OPERANDS 4096
/* Floating-point operations per wavefront per loop iteration:
 * 16 products of 32x32x16 (2 * 32 * 32 * 16 flop each). */
#define DDT_PROBE_MFMA_FLOP_PER_WAVE_ITER 524288

/* bf16 MFMA loop.
 *   ops    device, DDT_PROBE_MFMA_OPERANDS bf16 values (the bit patterns, as
 *          uint16), 16-byte aligned: lane l of every wavefront takes its
 *          eight A and eight B fragments from it and rotates through them.
 *   sink   device, blocks * DDT_PROBE_THREADS floats: one folded
 *          accumulator value per thread (keeps the products live).
 *   clk    device, nullable, 2 * blocks uint64: per workgroup, the
 *          s_memtime (core clock) and s_memrealtime (100 MHz) ticks its
 *          first wavefront spent in the loop; their ratio times 100 MHz is
 *          the core clock during the loop.
 *   blocks workgroups (> 0), iters loop iterations (> 0).
 * Work per call: blocks * 4 * iters * DDT_PROBE_MFMA_FLOP_PER_WAVE_ITER flop.
 */
int ddt_probe_mfma_bf16(const void* ops, float* sink, uint64_t* clk, int blocks, int iters,
                        hipStream_t stream);

/* Streaming read of `bytes` (a positive multiple of 16) at `src` (16-byte
 * aligned, device): every word is loaded once and XOR-folded; each thread
 * writes its fold to sink[blocks * DDT_PROBE_THREADS] (device). */
int ddt_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream);

/* Streaming copy of `bytes` (a positive multiple of 16) from `src` to
 * `dst` (both 16-byte aligned device buffers that do not overlap). */
int ddt_probe_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DDT_PROBE_H */
