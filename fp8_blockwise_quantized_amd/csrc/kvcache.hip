// FP8 (E4M3) KV cache with per-tensor FP32 scales recalibrated after a weight
// update (66260.cn FP8-RL item, KV-cache paragraph: scale factors calibrated
// dynamically and re-adjusted after each model update; nmedialink NeMo-RL
// repost: FP8 in the rollout's KV cache).  Bandwidth-bound; no MFMA.
//
//  * Calibration: amax over the K (and V) rows of a calibration batch, then the
//    scale pair of the quantizers: s = amax_c / 448, r = 448 / amax_c with
//    amax_c = max(amax, 2^-96).  Three launches on the stream: clear the two
//    amax words (a kernel, not a memset, so the call can be captured in a
//    graph), a grid-stride maximum with one atomicMax per workgroup (BF16
//    magnitudes compared as integers are exact), and the scale pair.
//  * Append: token t's K (V) row, 8 values per lane, codes = E4M3 of
//    clamp(x * r, +-448) (saturating, round to nearest even), written to cache
//    row slots[t]; a slot outside [0, rows) writes nothing.
#include <algorithm>

#include "jet_device.hpp"
#include "jet_launch.hpp"

namespace jet {

namespace {

__global__ void k_kv_clear(uint32_t* __restrict__ amax_bits) {
  if (threadIdx.x < 2) amax_bits[threadIdx.x] = 0u;
}

// blockIdx.y: 0 = K, 1 = V.  Each thread takes 16-byte chunks (8 BF16 values),
// kAmaxUnroll independent loads per iteration; at most kAmaxBlocks workgroups
// per tensor, so few atomics meet on the two amax words.
constexpr int kAmaxUnroll = 8;
constexpr int64_t kAmaxBlocks = 256;

__global__ __launch_bounds__(256) void k_kv_amax(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                  int64_t T, int64_t D, int64_t ldk, int64_t ldv,
                                                  uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t red[4];
  const uint16_t* x = blockIdx.y == 0 ? k : v;
  const int64_t ld = blockIdx.y == 0 ? ldk : ldv;
  const int64_t cpr = D / 8;                         // chunks per row
  const int64_t chunks = T * cpr;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t am = 0u;                                  // two packed BF16 magnitudes
  for (int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x; c0 < chunks; c0 += stride * kAmaxUnroll) {
    uint4 w[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      const int64_t c = c0 + stride * u;
      w[u] = make_uint4(0u, 0u, 0u, 0u);
      if (c < chunks) {
        const int64_t t = c / cpr, j = c - t * cpr;
        w[u] = load_stream16(x + t * ld + 8 * j);
      }
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      am = max_abs_bf16x2(am, w[u].x);
      am = max_abs_bf16x2(am, w[u].y);
      am = max_abs_bf16x2(am, w[u].z);
      am = max_abs_bf16x2(am, w[u].w);
    }
  }
  am = row16_max_u16x2(am);
  uint32_t f = __float_as_uint(fold_bf16x2(am));     // BF16 magnitude as FP32 bits
  f = max(f, (uint32_t)__shfl_xor((int)f, 16, 64));
  f = max(f, (uint32_t)__shfl_xor((int)f, 32, 64));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = f;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t b = max(max(red[0], red[1]), max(red[2], red[3]));
    if (b) atomicMax(amax_bits + blockIdx.y, b);
  }
}

__global__ void k_kv_scales(const uint32_t* __restrict__ amax_bits, float* __restrict__ scales) {
  if (threadIdx.x < 2) {
    const ScalePair sp = scale_pair(__uint_as_float(amax_bits[threadIdx.x]));
    scales[2 * threadIdx.x] = sp.s;
    scales[2 * threadIdx.x + 1] = sp.r;
  }
}

__device__ __forceinline__ float sat448(float p) { return fminf(fmaxf(p, -kE4M3Max), kE4M3Max); }

// blockIdx.y: 0 = K, 1 = V.  One thread per 16-byte chunk of a token row.
__global__ __launch_bounds__(256) void k_kv_append(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                    int64_t T, int64_t D, int64_t ldk, int64_t ldv,
                                                    const int64_t* __restrict__ slots,
                                                    const float* __restrict__ scales,
                                                    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                    int64_t ldc, int64_t rows) {
  const bool isv = blockIdx.y != 0;
  const uint16_t* x = isv ? v : k;
  const int64_t ld = isv ? ldv : ldk;
  uint8_t* cache = isv ? vc : kc;
  const float r = scales[isv ? 3 : 1];
  const int64_t cpr = D / 8;
  const int64_t chunks = T * cpr;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
    const int64_t t = c / cpr, j = c - t * cpr;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= rows) continue;
    const uint4 w = load_stream16(x + t * ld + 8 * j);
    const uint32_t c0 = e4m3x4(sat448(bf16_lo(w.x) * r), sat448(bf16_hi(w.x) * r),
                               sat448(bf16_lo(w.y) * r), sat448(bf16_hi(w.y) * r));
    const uint32_t c1 = e4m3x4(sat448(bf16_lo(w.z) * r), sat448(bf16_hi(w.z) * r),
                               sat448(bf16_lo(w.w) * r), sat448(bf16_hi(w.w) * r));
    *reinterpret_cast<uint2*>(cache + slot * ldc + 8 * j) = make_uint2(c0, c1);
  }
}

int64_t kv_blocks(int64_t chunks) {
  constexpr int64_t kMaxBlocks = 2048;
  return std::max<int64_t>(1, std::min<int64_t>((chunks + 255) / 256, kMaxBlocks));
}

}  // namespace

hipError_t launch_kv_calibrate(const uint16_t* k, const uint16_t* v, int64_t T, int64_t D, int64_t ldk,
                               int64_t ldv, float* scales, hipStream_t st) {
  uint32_t* amax_bits = reinterpret_cast<uint32_t*>(scales + 4);
  hipLaunchKernelGGL(k_kv_clear, dim3(1), dim3(64), 0, st, amax_bits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (T > 0 && D > 0) {
    const int64_t blocks = std::max<int64_t>(
        1, std::min<int64_t>((T * (D / 8) + 256 * kAmaxUnroll - 1) / (256 * kAmaxUnroll), kAmaxBlocks));
    hipLaunchKernelGGL(k_kv_amax, dim3((unsigned)blocks, 2), dim3(256), 0, st, k, v, T, D, ldk, ldv, amax_bits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_kv_scales, dim3(1), dim3(64), 0, st, amax_bits, scales);
  return hipGetLastError();
}

hipError_t launch_kv_append(const uint16_t* k, const uint16_t* v, int64_t T, int64_t D, int64_t ldk,
                            int64_t ldv, const int64_t* slots, const float* scales, uint8_t* kc, uint8_t* vc,
                            int64_t ldc, int64_t rows, hipStream_t st) {
  if (T == 0 || D == 0 || rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_append, dim3((unsigned)kv_blocks(T * (D / 8)), 2), dim3(256), 0, st, k, v, T, D, ldk,
                     ldv, slots, scales, kc, vc, ldc, rows);
  return hipGetLastError();
}

}  // namespace jet
