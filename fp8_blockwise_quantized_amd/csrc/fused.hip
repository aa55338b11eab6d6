// Fused producers of the 1x128-quantized linear input (bandwidth-bound; no
// MFMA): the operator before a linear layer writes the layer's FP8 input
// directly, so the BF16 activation is never written and re-read just to be
// quantized.  gist.science explainer "Jet-RL ...", section "Implementierung"
// (own kernels for fused activation/RMSNorm operations) and section
// "Quantisierungsschema" (activations kept in FP8, quantized together with the
// operator that produces them); 163.com write-up, section 五 (every
// quantization runs fused with the computation before it).
//
//  * RMSNorm (inputs of the QKV and gate+up projections):
//      y = bf16((x * r) * gamma),  r = 1 / sqrt(mean(x^2) + eps)  per row,
//    then the 1x128 quantization of y.
//  * SwiGLU (input of the down projection), from the fused gate+up output
//    gu = [gate | up] (columns 0..I-1 and I..2I-1):
//      h = bf16(gate * sigmoid(gate) * up), then the 1x128 quantization of h.
//
// The arithmetic is FP32 (RMSNorm: IEEE division and square root; SwiGLU: the
// hardware exp2 and reciprocal, see swiglu1) and the BF16 tensor is rounded
// once; its 1x128 codes and scales are computed exactly as
// jet_quant_act_1x128 would compute them from that BF16 tensor, and the BF16
// tensor itself is written too when the caller asks for it.
#include <algorithm>

#include "jet_device.hpp"
#include "jet_launch.hpp"

namespace jet {

namespace {

// Sum over the 64 lanes of a wavefront; every lane ends with the same bits
// (each butterfly step adds the same two operands on both partner lanes).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace

// ---------------------------------------------------------------------------
// RMSNorm + 1x128.  One wavefront per row; lane l holds columns 512c + 8l ..
// +7 of every 512-column chunk c (16-byte loads, each instruction a whole
// 1 KiB of the row), so the 16 lanes of a DPP row hold one 128-column group.
// Each wavefront issues its row's loads first; the block then stages gamma
// in LDS once (one 16-byte load per thread and chunk) for all its rows,
// instead of every wavefront loading and holding its own copy.  A block of
// kRmsRowsPerBlock wavefronts takes as many consecutive rows; its scales are
// staged in LDS and written as runs of consecutive rows per group.
// ---------------------------------------------------------------------------
constexpr int kRmsMaxChunks = 16;                  // H <= 8192
constexpr int kRmsRowsPerBlock = 8;                // = wavefronts per block

// CH: 512-column chunks held in registers (H <= 512*CH)
template <int CH, bool P2>
__global__ __launch_bounds__(64 * kRmsRowsPerBlock) void k_rmsnorm_quant_1x128(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, int64_t M, int64_t H,
    int64_t ldx, float eps, uint16_t* __restrict__ y, int64_t ldy, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ s) {
  __shared__ float stg[CH * 4][kRmsRowsPerBlock];
  __shared__ uint4 gsh[CH * 64];                  // gamma, 8 BF16 per entry
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = (int)gridDim.x, b = (int)blockIdx.x;
  // consecutive blocks on one XCD (blocks are dealt round-robin to the 8 XCDs),
  // so the partial lines of a scale row meet in one L2
  const int blk = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  const int64_t m0 = (int64_t)blk * kRmsRowsPerBlock;
  const int chunks = (int)((H + 511) / 512);
  const int G = (int)(H / kGroup);
  const float inv_h = 1.0f / (float)H;

  const int rr = wave;
  const int64_t m = m0 + rr;
  uint4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    v[c] = make_uint4(0u, 0u, 0u, 0u);
    const int64_t col = 512 * c + 8 * lane;
    if (m < M && c < chunks && col < H) v[c] = load_stream16(x + m * ldx + col);
  }
  for (int i = threadIdx.x; i < (int)(H / 8); i += 64 * kRmsRowsPerBlock)
    gsh[i] = *reinterpret_cast<const uint4*>(gamma + 8 * (int64_t)i);
  __syncthreads();
  if (m < M) {
    float ss = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = bf16_lo(w[k]), bb = bf16_hi(w[k]);
        ss = fmaf(a, a, ss);
        ss = fmaf(bb, bb, ss);
      }
    }
    const float ms = wave_sum(ss) * inv_h;
    const float r = 1.0f / sqrtf(ms + eps);
    uint4 yv[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t col = 512 * c + 8 * lane;
      const bool ok = c < chunks && col < H;       // uniform per DPP row (H % 128 == 0)
      const uint32_t xw[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
      const uint4 g4 = gsh[ok ? 64 * c + lane : 0];
      const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
      uint32_t yw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        yw[k] = bf16x2_rne((bf16_lo(xw[k]) * r) * bf16_lo(gw[k]), (bf16_hi(xw[k]) * r) * bf16_hi(gw[k]));
      }
      yv[c] = make_uint4(yw[0], yw[1], yw[2], yw[3]);
    }
    // 1x128 codes of every chunk (a DPP row holds one group per chunk), one
    // scale computation for the row's 4*CH groups
    uint2 qc[CH];
    const float sc = quant_1x128_passes<CH, P2>(yv, qc);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t col = 512 * c + 8 * lane;
      if (c < chunks && col < H) {
        store_stream8(q + m * ldq + col, qc[c].x, qc[c].y);
        if (y) store_stream16(y + m * ldy + col, yv[c]);
      }
    }
    {
      // lane L holds the scale of chunk L/4, DPP row L%4
      const int c = lane >> 2, g = 4 * c + (lane & 3);
      if (c < CH && c < chunks && 128 * (int64_t)g < H) stg[g][rr] = sc;
    }
  }
  __syncthreads();
  // scales: group j of rows m0 .. m0 + kRmsRowsPerBlock - 1 at s[j*M + m]
  for (int i = threadIdx.x; i < G * kRmsRowsPerBlock; i += 64 * kRmsRowsPerBlock) {
    const int j = i / kRmsRowsPerBlock, r2 = i % kRmsRowsPerBlock;
    const int64_t m2 = m0 + r2;
    if (m2 < M) s[(int64_t)j * M + m2] = stg[j][r2];
  }
}

hipError_t launch_rmsnorm_quant_1x128(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t H,
                                      int64_t ldx, float eps, uint16_t* y, int64_t ldy, uint8_t* q,
                                      int64_t ldq, float* s, hipStream_t st, bool p2) {
  if (M == 0) return hipSuccess;
  if (H <= 0 || H % kGroup || H > 512 * kRmsMaxChunks) return hipErrorInvalidValue;
  const int64_t blocks = (M + kRmsRowsPerBlock - 1) / kRmsRowsPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * kRmsRowsPerBlock);
#define JET_RMS(ch_)                                                                                  \
  do {                                                                                                \
    if (p2)                                                                                           \
      hipLaunchKernelGGL((k_rmsnorm_quant_1x128<ch_, true>), grid, block, 0, st, x, gamma, M, H, ldx, \
                         eps, y, ldy, q, ldq, s);                                                     \
    else                                                                                              \
      hipLaunchKernelGGL((k_rmsnorm_quant_1x128<ch_, false>), grid, block, 0, st, x, gamma, M, H, ldx, \
                         eps, y, ldy, q, ldq, s);                                                     \
  } while (0)
  if (H <= 2048) JET_RMS(4);
  else if (H <= 4096) JET_RMS(8);
  else JET_RMS(16);
#undef JET_RMS
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SwiGLU + 1x128.  The layout of the 1x128 quantizer (k_quant_1x128): units of
// 32 rows x 4 consecutive groups of h; in each of a block's 8 passes the 4
// DPP rows of a wavefront take 4 rows of one group, each lane 8 columns of
// gate and the same 8 columns of up (all loads issued before any compute).
// sigmoid(g) = 1/(1 + e) for g >= 0 and e/(1 + e) for g < 0 with
// e = exp(-|g|), which never overflows.  exp(-|g|) = 2^(-|g| * log2(e)) on the
// hardware base-2 exponential and 1/(1 + e) on the hardware reciprocal (each
// within about 1 ulp): the element stays within a few 2^-24 relative of the
// exact value for the gate values that matter (|g| up to a few tens), far
// inside half a BF16 step, at a fraction of the instructions of a libm exp and
// an IEEE division (this kernel is otherwise bound by VALU issue).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float swiglu1(float g, float u) {
  constexpr float kLog2e = 1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(-fabsf(g) * kLog2e);
  const float inv = __builtin_amdgcn_rcpf(1.0f + e);
  const float sg = g >= 0.0f ? inv : e * inv;
  return (g * sg) * u;
}

template <bool P2>
__global__ __launch_bounds__(256) void k_swiglu_quant_1x128(
    const uint16_t* __restrict__ gu, int64_t M, int64_t I, int64_t ldgu, uint16_t* __restrict__ h,
    int64_t ldh, uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s) {
  __shared__ float stg[2][4][32];
  const int64_t G = I / kGroup;
  const int64_t ugc = (G + 3) / 4;
  const int64_t units = ((M + 31) / 32) * ugc;
  const int dr = threadIdx.x >> 4, lane16 = threadIdx.x & 15;
  int buf = 0;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x, buf ^= 1) {
    const int64_t m0 = (u / ugc) * 32, j0 = (u % ugc) * 4;
    uint4 vg[8], vu[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t m = m0 + 16 * (p & 1) + dr, j = j0 + (p >> 1);
      vg[p] = make_uint4(0u, 0u, 0u, 0u);
      vu[p] = vg[p];
      if (m < M && j < G) {
        const uint16_t* row = gu + m * ldgu + j * kGroup + lane16 * 8;
        vg[p] = load_stream16(row);
        vu[p] = load_stream16(row + I);
      }
    }
    uint4 hv[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint32_t gw[4] = {vg[p].x, vg[p].y, vg[p].z, vg[p].w};
      const uint32_t uw[4] = {vu[p].x, vu[p].y, vu[p].z, vu[p].w};
      uint32_t hw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hw[k] = bf16x2_rne(swiglu1(bf16_lo(gw[k]), bf16_lo(uw[k])), swiglu1(bf16_hi(gw[k]), bf16_hi(uw[k])));
      }
      hv[p] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    }
    // codes of all 8 passes, one scale computation for the wavefront's 32 groups
    uint2 qc[8];
    const float sc = quant_1x128_passes<8, P2>(hv, qc);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = 16 * (p & 1) + dr, g = p >> 1;
      const int64_t m = m0 + r, j = j0 + g;
      if (m < M && j < G) {
        store_stream8(q + m * ldq + j * kGroup + lane16 * 8, qc[p].x, qc[p].y);
        if (h) store_stream16(h + m * ldh + j * kGroup + lane16 * 8, hv[p]);
      }
    }
    {
      // lane L of wavefront w holds the scale of pass L/4, DPP row L%4: row
      // 16*(pass&1) + 4w + L%4 of the unit, group pass/2
      const int lane = threadIdx.x & 63, p = lane >> 2;
      if (p < 8) stg[buf][p >> 1][16 * (p & 1) + 4 * (threadIdx.x >> 6) + (lane & 3)] = sc;
    }
    __syncthreads();
    if (threadIdx.x < 128) {
      const int g = threadIdx.x >> 5, r = threadIdx.x & 31;
      const int64_t m = m0 + r, j = j0 + g;
      if (m < M && j < G) s[j * M + m] = stg[buf][g][r];
    }
  }
}

hipError_t launch_swiglu_quant_1x128(const uint16_t* gu, int64_t M, int64_t I, int64_t ldgu, uint16_t* h,
                                     int64_t ldh, uint8_t* q, int64_t ldq, float* s, hipStream_t st, bool p2) {
  if (M == 0 || I == 0) return hipSuccess;
  if (I % kGroup) return hipErrorInvalidValue;
  constexpr int64_t kMaxBlocks = 2048;
  const int64_t units = ((M + 31) / 32) * ((I / kGroup + 3) / 4);
  const int64_t blocks = std::min<int64_t>(units, kMaxBlocks);
  if (p2)
    hipLaunchKernelGGL(k_swiglu_quant_1x128<true>, dim3((unsigned)blocks), dim3(256), 0, st, gu, M, I, ldgu, h,
                       ldh, q, ldq, s);
  else
    hipLaunchKernelGGL(k_swiglu_quant_1x128<false>, dim3((unsigned)blocks), dim3(256), 0, st, gu, M, I, ldgu, h,
                       ldh, q, ldq, s);
  return hipGetLastError();
}

}  // namespace jet
