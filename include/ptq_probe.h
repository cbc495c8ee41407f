/* ptq_probe.h -- matrix-core clock probe, VALU probe and HBM stream probe exported by libptq.so.
 *
 * Measurement aids for the rooflines, not steps of the quantization method.
 * The published dense int8 peak of the chip assumes its 2.4 GHz top shader
 * clock; under the board's power limit the clock that int8 MFMAs on varied
 * operands allow is lower.  ptq_probe_mfma measures that clock and the
 * throughput that goes with it, on the GEMM kernel's own instruction mix.
 * The published HBM bandwidth (8 TB/s) is likewise a ceiling no access
 * pattern reaches; ptq_probe_stream measures what plain streaming reads, or a
 * copy, of a buffer much larger than the last-level cache achieve, as the
 * measured peak of the memory-bound kernels.  The weight quantizer's search is bound by the vector ALUs, whose
 * issue rate depends on the instruction mix (fp32 and fp64 operations take different numbers of cycles);
 * ptq_probe_valu measures the rate of the search's own pass loop without its reductions and decisions, and of
 * plain fp32 and fp64 multiply-adds.
 */
#ifndef PTQ_PROBE_H
#define PTQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PTQ_PROBE_API __attribute__((visibility("default")))
#else
#define PTQ_PROBE_API
#endif

#define PTQ_PROBE_ERR_ARG 5 /* same code as PTQ_ERR_ARG */
#define PTQ_PROBE_ERR_HIP 7 /* same code as PTQ_ERR_HIP */

/* Multiply-adds per block and iteration, for every kind: 8 waves x 64 instructions of 16x16x64 (or 32 of
 * 32x32x32) = 8 * 64 * 16 * 16 * 64; operations are twice that. */
#define PTQ_PROBE_MACS_PER_BLOCK_ITER (8LL * 64 * 16 * 16 * 64)

/* Launch the probe on `stream` (a hipStream_t, or NULL for the default stream).
 *   kind    0: v_mfma_i32_16x16x64_i8 on pseudo-random operands
 *           1: v_mfma_i32_32x32x32_i8 on pseudo-random operands
 *           2: kind 0 plus the GEMM kernel's LDS operand reads (24 ds_read_b128 per 64 MFMAs per wave)
 *           3: kind 0 with zero operands
 *   blocks  1..65536 blocks of 512 threads (one block per CU fills the chip: 256 on MI355X)
 *   iters   1..1000000 loop iterations
 *   seed    operand hash seed
 *   out     device buffer of 3*blocks uint64, 8-byte aligned, written by the kernel: per block, the shader-clock
 *           cycles and the 100 MHz real-time ticks wave 0 spent in the loop, then a meaningless sink value.
 *           The shader clock is cycles / (ticks * 10 ns).  Owned by the caller.
 * Returns 0, PTQ_PROBE_ERR_ARG (nothing launched; ptq_probe_last_error() says why) or PTQ_PROBE_ERR_HIP. */
PTQ_PROBE_API int ptq_probe_mfma(int kind, int blocks, int iters, uint32_t seed, uint64_t* out, void* stream);

/* Element-passes per lane and iteration of kinds 0 and 1 (the SSZ search's loop over 64 values). */
#define PTQ_PROBE_VALU_ELEMS_PER_ITER 64
/* Multiply-adds per lane and iteration of kinds 2 and 3: 16 x 8 independent chains. */
#define PTQ_PROBE_VALU_FMAS_PER_ITER 128

/* Launch the VALU probe on `stream` (a hipStream_t, or NULL for the default stream): `blocks` blocks of one wave
 * (64 threads) each, so blocks / (4 * number of CUs) waves per SIMD (2048 blocks: two per SIMD on MI355X).
 *   kind    0: the SSZ search's pass loop alone: per lane 64 fp32 values held in fp64 and, per iteration, the fp64
 *              reciprocal of a scale, then per value the fp64 product rounded to fp32, round, clamp to [-127, 127],
 *              widening of the code, the fp64 multiply-add of sum w q and the fp32 one of sum q^2
 *           1: kind 0 plus the per-iteration 64-lane butterflies of both sums (fp64 and integer)
 *           2: fp32 multiply-adds only, 8 independent chains per lane
 *           3: fp64 multiply-adds only, 8 independent chains per lane
 *   blocks  1..65536;  iters 1..1000000;  seed: operand hash seed
 *   out     device buffer of 3*blocks uint64, 8-byte aligned, written by the kernel as for ptq_probe_mfma: per block
 *           the shader-clock cycles and 100 MHz ticks wave 0 spent in the loop, then a meaningless sink value.
 * Returns 0, PTQ_PROBE_ERR_ARG (nothing launched; ptq_probe_last_error() says why) or PTQ_PROBE_ERR_HIP. */
PTQ_PROBE_API int ptq_probe_valu(int kind, int blocks, int iters, uint32_t seed, uint64_t* out, void* stream);

/* Launch the HBM stream probe on `stream` (a hipStream_t, or NULL for the default stream).
 *   kind    0: read every byte of src once (16-byte loads, 1 KB of consecutive bytes per wave instruction,
 *              16 loads in flight per lane); out[b] receives block b's xor of the words read (meaningless,
 *              it keeps the loads live)
 *           1: copy src to dst (the same loads, then 16-byte stores)
 *   src     device buffer of `bytes` bytes, 16-byte aligned; read only
 *   bytes   a non-zero multiple of 16; larger than twice the 256 MB last-level cache for an HBM figure
 *   dst     kind 1: device buffer of `bytes` bytes, 16-byte aligned, not overlapping src; else ignored (may be NULL)
 *   blocks  1..65536 blocks of 256 threads (4 per CU: 1024 on MI355X)
 *   out     kind 0: device buffer of `blocks` uint32, 4-byte aligned; else ignored (may be NULL)
 * Buffers are owned by the caller.  Time the launch with events around it; the bytes moved are `bytes` (read)
 * or 2 * `bytes` (copy).  Returns 0, PTQ_PROBE_ERR_ARG (nothing launched; ptq_probe_last_error() says why) or
 * PTQ_PROBE_ERR_HIP. */
PTQ_PROBE_API int ptq_probe_stream(int kind, const void* src, uint64_t bytes, void* dst, int blocks, uint32_t* out,
                                   void* stream);

/* Message of the last failed ptq_probe_mfma, ptq_probe_valu or ptq_probe_stream call on this thread. */
PTQ_PROBE_API const char* ptq_probe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PTQ_PROBE_H */
