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
//  * k_gemm_step<PARTS>: the GEMMs' K-step on synthetic bytes, built up from
//    its parts.  A block is the GEMM's 8 wavefronts (2 x 4, wave tile 128 x
//    64 of a 256 x 256 tile) with two 64 KiB LDS stages (A and B, 256 rows x
//    128 bytes each, the GEMM's row swizzle); a step is 32 MFMAs per
//    wavefront on fragments held in registers, plus, by flag: the step's 12
//    fragment reads from LDS (24 ds_read_b128; or only the 8 A fragments), the next stage's direct
//    global->LDS loads (8 per wavefront, 64 KiB per block) waited for at the
//    next step's start and followed by one barrier, and the per-step FP32 fold
//    (each MFMA from zero, folded three MFMAs later with one FMA per
//    element).  The source is either a 128 KiB window shared by every 32nd
//    block (the loads hit L2) or a 256 KiB window of the block's own that the
//    steps cycle through (with 32 blocks per XCD, 8 MiB per XCD: every load
//    misses L2 and comes from the MALL).
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

enum { kStepLds = 1, kStepPipe = 2, kStepFold = 4, kStepMall = 8, kStepAOnly = 16 };

__device__ __forceinline__ uint32_t rfl(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// 64 lanes x 16 bytes from base + voff (per lane) to LDS [lds_addr, +1024).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void probe_dma16(uint32_t lds_addr, const uint8_t* base, uint32_t voff) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t bs = (uint64_t)rfl((uint32_t)b) | ((uint64_t)rfl((uint32_t)(b >> 32)) << 32);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(rfl(lds_addr)), "v"(voff), "s"(reinterpret_cast<const void*>(bs)) : "memory", "m0");
}
#pragma clang diagnostic pop

typedef __attribute__((address_space(3))) uint8_t lds_byte;

template <int PARTS>
__global__ __launch_bounds__(512) void k_gemm_step(const uint8_t* __restrict__ src, float* __restrict__ out,
                                                   int steps) {
  constexpr int kStage = 65536;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % 2, wn = wave / 2;
  const int lrow = lane & 15, kg = lane >> 4;
  for (int i = tid; i < 2 * kStage / 4; i += 512) reinterpret_cast<uint32_t*>(lds)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  v8i af[8], bf[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) af[i][e] = lane * 8 + e + i;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) bf[j][e] = lane * 8 + e + 3 * j;
  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t lds0 = (uint32_t)(uintptr_t)(const lds_byte*)lds;
  const uint8_t* base = src + ((PARTS & kStepMall) ? (int64_t)blockIdx.x * 262144 : (int64_t)(blockIdx.x % 32) * 131072);
  const uint32_t voff = (uint32_t)((lane >> 3) * 128 + (lane & 7) * 16);
  for (int kb = 0; kb < steps; ++kb) {
    const int st = kb & 1;
    if (PARTS & kStepPipe) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // this wavefront's 8 KiB of the next stage
      const int64_t off = (PARTS & kStepMall) ? (int64_t)((kb + 1) & 3) * kStage : (int64_t)((kb + 1) & 1) * kStage;
      const uint32_t dst = lds0 + (uint32_t)((st ^ 1) * kStage + wave * 8192);
#pragma unroll
      for (int t = 0; t < 8; ++t) probe_dma16(dst + t * 1024, base + off + wave * 8192 + t * 1024, voff);
    }
    const uint8_t* As = lds + st * kStage;
    const uint8_t* Bs = As + kStage / 2;
    v4f part[3];
    const float c = (float)(lane + kb) * 1e-3f;
#pragma unroll
    for (int n = 0; n < 32 + 3; ++n) {
      if ((PARTS & kStepFold) && n >= 3) {
        const int ii = (n - 3) / 4, jj = (n - 3) % 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[ii][jj][r] = fmaf(part[(n - 3) % 3][r], c, acc[ii][jj][r]);
      }
      if (n >= 32) continue;
      const int i = n / 4, j = n % 4;
      if (j == 0) {
        if (PARTS & kStepLds) {
          // rows i (and i + 1 ahead), all B fragments at the step's start
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int ia = (i == 0) ? q : (q == 0 ? -1 : i + 1);
            if (ia < 0 || ia >= 8) continue;
            const int row = (wm * 8 + ia) * 16 + lrow, f = (row & 7) ^ ((row >> 3) & 1);
            const uint4 lo = *reinterpret_cast<const uint4*>(As + row * 128 + (((2 * kg) ^ f) << 4));
            const uint4 hi = *reinterpret_cast<const uint4*>(As + row * 128 + (((2 * kg + 1) ^ f) << 4));
            af[ia] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          }
          if (i == 0 && !(PARTS & kStepAOnly)) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
              const int row = (wn * 4 + jb) * 16 + lrow, f = (row & 7) ^ ((row >> 3) & 1);
              const uint4 lo = *reinterpret_cast<const uint4*>(Bs + row * 128 + (((2 * kg) ^ f) << 4));
              const uint4 hi = *reinterpret_cast<const uint4*>(Bs + row * 128 + (((2 * kg + 1) ^ f) << 4));
              bf[jb] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
          }
        } else {
          asm volatile("" : "+v"(af[i]));   // operands are not loop-invariant to the compiler
        }
      }
      if (PARTS & kStepFold)
        part[n % 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                       0, 0, 0, 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) t += acc[i][j][0] + acc[i][j][3];
  // an LDS read keeps the 128 KiB allocation in every variant: one block per CU
  out[(int64_t)blockIdx.x * 512 + tid] = t + (float)lds[(tid * 257) & (2 * kStage - 1)];
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

int jet_probe_gemm_step(const void* src, float* out, int steps, int parts, int blocks, void* stream) {
  if (!src || !out || steps < 1 || blocks < 1 || parts < 0 || parts > 31) return 1;
  if ((parts & kStepMall) && !(parts & kStepPipe)) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* s8 = static_cast<const uint8_t*>(src);
  const dim3 g((unsigned)blocks), b(512);
  switch (parts) {
#define JET_STEP(P) \
  case P: hipLaunchKernelGGL((k_gemm_step<P>), g, b, 0, st, s8, out, steps); break;
    JET_STEP(0) JET_STEP(1) JET_STEP(17) JET_STEP(3) JET_STEP(4) JET_STEP(7) JET_STEP(11) JET_STEP(15)
#undef JET_STEP
    default: return 2;
  }
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
