/* Peak probes for gfx950 (libkq_peaks.so): sustained matrix-core rates and
 * device copy bandwidth measured on the machine. Context for the rooflines of
 * the quantization path, whose kernels are priced against the published MI355X
 * peaks; not part of the path itself. Used by `bench.py --peaks`.
 *
 * All pointers are device pointers owned by the caller; `stream` is a
 * hipStream_t (NULL: the null stream). The calls enqueue and return. */
#ifndef KQ_PEAKS_H
#define KQ_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of one MFMA probe launch (4 per CU on 256 CUs, 256 threads each). */
int kqp_mfma_blocks(void);

/* Flops of one wave-round of probe `kind` (16 MFMAs; kinds as kqp_mfma). */
double kqp_flops_per_round(int kind);

/* One launch of MFMA probe `kind`: 0 bf16 random operands, 1 bf16 constant,
 * 2 float32 random, 3 float32 constant, 4 float64 random, 5 float64 constant
 * (v_mfma_f32_32x32x16_bf16, v_mfma_f32_32x32x2f32, v_mfma_f64_16x16x4f64).
 * Every wave runs `iters` rounds (float64: rounded down to a multiple of 8).
 *   out  [kqp_mfma_blocks() * 256] float, receives one sum per lane
 *   clk  [4] int64: shader-clock and 100 MHz real-time counters before and
 *        after workgroup 0's loop (clock in MHz = 100 (clk[2]-clk[0]) / (clk[3]-clk[1]))
 * Returns 0; -1 for an unknown kind, iters <= 0, NULL pointers or a failed launch. */
int kqp_mfma(int kind, int iters, float* out, long long* clk, void* stream);

/* Copies `bytes` from src to dst (bytes a multiple of 16 KiB, both pointers
 * 16-byte aligned, no overlap). Returns 0; -1 for bad arguments or a failed launch. */
int kqp_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_PEAKS_H */
