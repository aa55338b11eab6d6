// Roofline probes for gfx950: the measured ceilings the library's kernels are
// compared with, next to the published MI355X peaks.  Not part of the layer's
// C ABI (include/jetfp8.h); declared in include/jetprobe.h and used only by
// the benchmark.
//
//  * k_stream<LB, SB>: streams `units` units through the memory system, each
//    unit one LB-byte read and one SB-byte write (SB = 0: read only), with
//    non-temporal 16-byte accesses from a grid-stride loop.  The mixes match
//    the quantizers': BF16 in / E4M3 out is 16:8, the one-read quantizer
//    (BF16 in, two E4M3 outputs) and a plain copy 16:16, SwiGLU (gate and up
//    in, codes out) 32:8.
//  * k_mfma_rate<FOLD>: every wavefront runs the GEMMs' wave tile -- 8 A and
//    4 B fragments in registers, 32 v_mfma_scale_f32_16x16x128_f8f6f4 per
//    iteration on distinct operand pairs.  FOLD = false accumulates inside
//    the MFMA (the pure matrix rate); FOLD = true starts each MFMA from zero
//    and folds its result into an FP32 accumulator with one FMA per element,
//    the per-128-K-step scale fold of the FP32-scale GEMMs.  Wavefront 0 of
//    block 0 records the core cycle counter and the constant-rate wall
//    counter over its loop; the fold's VALU work lowers the clock the chip
//    sustains, so the host reports the clock of each pass.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/jetprobe.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int LB, int SB>
__global__ __launch_bounds__(256) void k_stream(const u32x4* __restrict__ in, uint8_t* __restrict__ out,
                                                int64_t units) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t keep = 0;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += stride) {
    u32x4 a = __builtin_nontemporal_load(in + u * (LB / 16));
    if (LB == 32) a ^= __builtin_nontemporal_load(in + u * 2 + 1);
    if (SB == 16) {
      __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(out) + u);
    } else if (SB == 8) {
      const u32x2 v = {a.x ^ a.z, a.y ^ a.w};
      __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(out) + u);
    } else {
      keep ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  }
  if (SB == 0 && keep == 0x9E3779B9u) out[0] = 1;   // keeps the loads of the read-only pass
}

template <bool FOLD>
__global__ __launch_bounds__(512) void k_mfma_rate(const int* __restrict__ in, float* __restrict__ out,
                                                   long long* __restrict__ clocks, int iters) {
  // 96 KB of LDS, more than half of a CU's 160 KB: one block per CU, so the
  // grid's 8-wavefront blocks put two wavefronts on each SIMD
  __shared__ uint8_t lds_hold[96 * 1024];
  constexpr int TM = 8, TN = 4;   // the GEMM's wave tile: 8 A and 4 B fragments, 32 MFMAs a step
  const int lane = threadIdx.x & 63;
  v8i a[TM], b[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a[i][e] = in[(lane * 8 + e + 7 * i) & 1023];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) b[j][e] = in[(lane * 8 + e + 13 * j + 512) & 1023];
  const float s = __int_as_float(0x3f800000 | (in[1024] & 0xff));   // about 1.0, unknown to the compiler
  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  lds_hold[threadIdx.x] = (uint8_t)in[1024];
  __syncthreads();
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  long long c0 = 0, w0 = 0;
  if (timer) {
    c0 = clock64();
    w0 = wall_clock64();
  }
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(a[0]), "+v"(b[0]));   // operands are not loop-invariant to the compiler
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (FOLD) {
          const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                         0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(p[r], s, acc[i][j][r]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
      }
  }
  if (timer) {
    clocks[0] = clock64() - c0;
    clocks[1] = wall_clock64() - w0;
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) t += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[(int64_t)blockIdx.x * 512 + threadIdx.x] = t + (float)lds_hold[(threadIdx.x + 1) & 511];
}

}  // namespace

extern "C" {

int jet_probe_stream(const void* in, void* out, int64_t units, int load_bytes, int store_bytes, int blocks,
                     void* stream) {
  if (!in || (store_bytes && !out) || units < 0 || blocks < 1) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* src = static_cast<const u32x4*>(in);
  uint8_t* dst = static_cast<uint8_t*>(out);
  const dim3 g((unsigned)blocks), b(256);
  if (load_bytes == 16 && store_bytes == 16) hipLaunchKernelGGL((k_stream<16, 16>), g, b, 0, st, src, dst, units);
  else if (load_bytes == 16 && store_bytes == 8) hipLaunchKernelGGL((k_stream<16, 8>), g, b, 0, st, src, dst, units);
  else if (load_bytes == 32 && store_bytes == 8) hipLaunchKernelGGL((k_stream<32, 8>), g, b, 0, st, src, dst, units);
  else if (load_bytes == 16 && store_bytes == 0) hipLaunchKernelGGL((k_stream<16, 0>), g, b, 0, st, src, dst, units);
  else return 2;
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int jet_probe_mfma(const int* in, float* out, long long* clocks, int iters, int fold, int blocks, void* stream) {
  if (!in || !out || !clocks || iters < 1 || blocks < 1) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (fold)
    hipLaunchKernelGGL((k_mfma_rate<true>), dim3((unsigned)blocks), dim3(512), 0, st, in, out, clocks, iters);
  else
    hipLaunchKernelGGL((k_mfma_rate<false>), dim3((unsigned)blocks), dim3(512), 0, st, in, out, clocks, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int jet_probe_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
  return khz;
}

int jet_probe_cu_count(void) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // extern "C"
