/*
 * jetprobe.h -- roofline probes for gfx950 (libjetprobe.so).  Not part of the
 * FP8 linear layer's ABI (jetfp8.h): these kernels measure the ceilings the
 * layer's kernels are compared with -- streaming bandwidth for the
 * quantizers' read/write mixes, the FP8 MFMA rate with and without the
 * per-step FP32 fold of the GEMMs, and the shader clock under that load.
 * All pointers are device pointers owned by the caller; every call only
 * enqueues on `stream` (a hipStream_t) and returns 0, or non-zero for a bad
 * argument (nothing launched) or a failed launch.
 */
#ifndef JETPROBE_H
#define JETPROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `units` units, each reading load_bytes (16 or 32) from `in` (16-byte
 * aligned, units*load_bytes bytes) and writing store_bytes (16, 8, or 0 for a
 * read-only pass) to `out` (units*store_bytes bytes); grid of `blocks`
 * workgroups of 256 threads, non-temporal accesses. */
int jet_probe_stream(const void* in, void* out, int64_t units, int load_bytes, int store_bytes, int blocks,
                     void* stream);

/* `blocks` workgroups of 8 wavefronts (one per CU: each holds 96 KB of LDS),
 * each wavefront issuing iters x 32 v_mfma_scale_f32_16x16x128_f8f6f4 on
 * register operands (8 A x 4 B fragments; 2*16*16*128 FLOP each).  fold != 0: each MFMA starts
 * from zero and its result is folded into an FP32 accumulator with one FMA
 * per element.  in: int32[1025] (operand bytes, then one word for the fold
 * factor); out: float[blocks*512]; clocks: int64[2] receives the core cycles
 * and wall-counter ticks wavefront 0 of block 0 spent in its loop. */
int jet_probe_mfma(const int* in, float* out, long long* clocks, int iters, int fold, int blocks, void* stream);

/* The GEMMs' K-step on synthetic bytes (8 wavefronts of 128 x 64, 256 x 256
 * block tile, two 64 KiB LDS stages, 32 MFMAs per wavefront and step), built
 * up from parts: parts = 0 MFMA only; +1 the step's LDS fragment reads; +2 the
 * pipeline (the next stage's direct global->LDS loads, the wait for them and
 * one barrier per step; needs +1); +4 the per-step FP32 fold; +8 the loads
 * miss L2 (each block cycles a 256 KiB window of its own; needs +2); +16 only
 * the 8 A fragments of the step are read from LDS (with +1); parts in
 * {0, 1, 17, 3, 4, 7, 11, 15}.  src: device bytes, at least blocks * 262144 (with
 * +8) or 32 * 131072; out: float[blocks * 512]; `steps` K steps per block. */
int jet_probe_gemm_step(const void* src, float* out, int steps, int parts, int blocks, void* stream);

/* Rate of the wall counter read by jet_probe_mfma, kHz (0 on failure). */
int jet_probe_wall_clock_khz(void);

/* Compute units of the current device (0 on failure). */
int jet_probe_cu_count(void);

#ifdef __cplusplus
}
#endif

#endif
