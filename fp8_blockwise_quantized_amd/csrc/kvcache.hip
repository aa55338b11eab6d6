// FP8 (E4M3) KV cache with per-tensor FP32 scales recalibrated after a weight
// update (66260.cn FP8-RL item, KV-cache paragraph: scale factors calibrated
// dynamically and re-adjusted after each model update; nmedialink NeMo-RL
// repost: FP8 in the rollout's KV cache).  Bandwidth-bound; no MFMA.
//
//  * Calibration: amax over the K (and V) rows of a calibration batch, then the
//    scale pair of the quantizers: s = amax_c / 448, r = 448 / amax_c with
//    amax_c = max(amax, 2^-96).  Two launches on the stream: clear the two
//    amax words and an arrival counter (a kernel, not a memset, so the call
//    can be captured in a graph), then a grid-stride maximum with one
//    atomicMax per workgroup (BF16 magnitudes compared as integers are
//    exact) whose last workgroup to arrive writes the scale pairs.
//  * Append: token t's K (V) row, 8 values per lane, codes = E4M3 of
//    clamp(x * r, +-448) (saturating, round to nearest even), written to cache
//    row slots[t]; a slot outside [0, rows) writes nothing.
#include <algorithm>

#include "jet_device.hpp"
#include "jet_launch.hpp"

namespace jet {

namespace {

// Zero the two amax words and the arrival counter (the bits of scales[0],
// which the last workgroup of k_kv_amax overwrites with s_k).
__global__ void k_kv_clear(uint32_t* __restrict__ amax_bits, uint32_t* __restrict__ arrivals) {
  if (threadIdx.x < 2) amax_bits[threadIdx.x] = 0u;
  if (threadIdx.x == 2) *arrivals = 0u;
}

// A thread's chunks c, c + stride, c + 2*stride, ... of a [T, D] tensor, as
// (row t, chunk j of the row), advanced by additions: no division in the
// loops, so every load of an unrolled batch is issued before the first one is
// waited for.
struct ChunkWalk {
  int64_t t, j, dt, dj, cpr;
  __device__ ChunkWalk(int64_t c, int64_t stride, int64_t cpr_) : cpr(cpr_) {
    t = c / cpr;
    j = c - t * cpr;
    dt = stride / cpr;
    dj = stride - dt * cpr;
  }
  __device__ __forceinline__ void next() {
    j += dj;
    t += dt;
    const bool wrap = j >= cpr;
    j = wrap ? j - cpr : j;
    t = wrap ? t + 1 : t;
  }
};

// blockIdx.y: 0 = K, 1 = V.  Each thread takes kAmaxUnroll 16-byte chunks (8
// BF16 values each) per pass, all loads in flight together (a chunk past the
// last row reloads a chunk of the last row, which leaves the maximum as it
// is).  At most kAmaxBlocks workgroups per tensor: the atomics of the
// workgroups' ends meet on three words and take their turns there (kernel
// time on Llama-8B K and V at 8192 tokens, 16.8 MB each: 256 / 128 / 64 / 32
// workgroups per tensor 17.0 / 12.4 / 12.3 / 17.1 us).
constexpr int kAmaxUnroll = 16;
constexpr int64_t kAmaxBlocks = 128;

__global__ __launch_bounds__(256) void k_kv_amax(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                  int64_t T, int64_t D, int64_t ldk, int64_t ldv,
                                                  uint32_t* __restrict__ amax_bits, float* __restrict__ scales) {
  __shared__ uint32_t red[4];
  const uint16_t* x = blockIdx.y == 0 ? k : v;
  const int64_t ld = blockIdx.y == 0 ? ldk : ldv;
  const int64_t stride = (int64_t)gridDim.x * 256;
  ChunkWalk w((int64_t)blockIdx.x * 256 + threadIdx.x, stride, D / 8);
  uint32_t am = 0u;                                  // two packed BF16 magnitudes
  while (w.t < T) {
    uint4 q[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      q[u] = load_stream16(x + min(w.t, T - 1) * ld + 8 * w.j);
      w.next();
    }
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) {
      am = max_abs_bf16x2(am, q[u].x);
      am = max_abs_bf16x2(am, q[u].y);
      am = max_abs_bf16x2(am, q[u].z);
      am = max_abs_bf16x2(am, q[u].w);
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
    // Contribute this workgroup's maximum, wait until the atomic has been
    // performed (its returned value is consumed), then count the arrival;
    // the last workgroup to arrive reads both maxima, whose every
    // contribution has then been performed, and writes the scale pairs.
    const uint32_t b = max(max(red[0], red[1]), max(red[2], red[3]));
    const uint32_t old = atomicMax(amax_bits + blockIdx.y, b);
    asm volatile("" :: "v"(old));
    uint32_t* arrivals = reinterpret_cast<uint32_t*>(scales);
    const uint32_t n = atomicAdd(arrivals, 1u);
    if (n + 1 == gridDim.x * gridDim.y) {
      const ScalePair pk = scale_pair(__uint_as_float(atomicOr(amax_bits, 0u)));
      const ScalePair pv = scale_pair(__uint_as_float(atomicOr(amax_bits + 1, 0u)));
      uint32_t* out = reinterpret_cast<uint32_t*>(scales);
      atomicExch(out + 1, __float_as_uint(pk.r));
      atomicExch(out + 2, __float_as_uint(pv.s));
      atomicExch(out + 3, __float_as_uint(pv.r));
      atomicExch(out, __float_as_uint(pk.s));
    }
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
  hipLaunchKernelGGL(k_kv_clear, dim3(1), dim3(64), 0, st, amax_bits, reinterpret_cast<uint32_t*>(scales));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // T == 0 still runs one workgroup per tensor: no rows, amax 0, the floor scale
  const int64_t blocks = std::max<int64_t>(
      1, std::min<int64_t>((T * (D / 8) + 256 * kAmaxUnroll - 1) / (256 * kAmaxUnroll), kAmaxBlocks));
  hipLaunchKernelGGL(k_kv_amax, dim3((unsigned)blocks, 2), dim3(256), 0, st, k, v, T, D, ldk, ldv, amax_bits,
                     scales);
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
