/*
 * spt_probe.h -- measurement probe of libspt.so (not part of the GEMM path).
 *
 * The dense MFMA peak of MI355X (2516.6 TFLOP/s fp16/bf16, 5033.2 TOPS int8)
 * assumes the 2.4 GHz engine clock.  Under the board power limit a long run
 * of MFMAs settles at a lower clock, and how low depends on the operand bits.
 * This call measures the rate MFMAs alone sustain with the caller's operand
 * data, so a kernel's roofline fraction can also be read against what the
 * part can do for that data ("Kernel-Engpass analysieren", Schritt 1: the
 * roofline's compute roof is the attainable peak).
 */
#ifndef SPT_PROBE_H
#define SPT_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launch one grid of 256 workgroups x 256 threads (one wave per SIMD on every
 * CU); each lane takes 8 sixteen-byte fragments from `operands` (wrapping
 * inside `operand_bytes`) and each wave issues `iters` rounds of 64
 * independent 16x16 MFMAs (v_mfma_f32_16x16x32_f16 / _bf16 for SPT_F16 /
 * SPT_BF16, v_mfma_i32_16x16x64_i8 for SPT_I8): 256 * 4 * 64 * iters MFMAs of
 * 16384 (fp16/bf16) or 32768 (int8) operations.  `sink` receives 65536
 * floats of checksum.  Device pointers owned by the caller; `operands`
 * 16-byte aligned; asynchronous on `stream`.  Errors: SPT_ERR_INVALID
 * (dtype other than f16/bf16/i8, null pointer, fewer than 16 bytes,
 * negative iters), SPT_ERR_MISALIGNED, SPT_ERR_LAUNCH.
 */
int spt_probe_mfma(int dtype, const void* operands, int64_t operand_bytes, int64_t iters, void* sink,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPT_PROBE_H */
