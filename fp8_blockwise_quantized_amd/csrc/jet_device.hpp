// Device helpers shared by the gfx950 quantizer and GEMM kernels.
//
// Numerics follow the group-scaling rule of the Jet-RL scheme (gist.science
// explainer, section "Quantisierungsschema"; nmedialink table of section
// "为什么FP8适配线性层？": E4M3 codes with one FP32 scale per group):
//   amax_c = max(amax, 2^-96), s = fl32(amax_c / 448), r = fl32(448 / amax_c),
//   code   = E4M3_rne_sat(fl32(x * r)).
// Built without fast-math: '/' is the correctly rounded IEEE division and FP32
// denormals are preserved (kernel descriptor float_denorm_mode_32 = 3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jet {

constexpr int kGroup = 128;
constexpr float kE4M3Max = 448.0f;
constexpr float kAmaxFloor = 0x1p-96f;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Magnitude maxima.  |bf16| compared as unsigned 15-bit integers is exact for
// finite values, so a group maximum needs no float compare at all: two BF16
// magnitudes per dword go through one v_pk_max_u16.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t max_abs_bf16x2(uint32_t acc, uint32_t w) {
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// Larger of the two BF16 magnitudes held in a dword, as an FP32 value.
__device__ __forceinline__ float fold_bf16x2(uint32_t w) {
  uint32_t lo = w & 0xFFFFu, hi = w >> 16;
  return __uint_as_float((lo > hi ? lo : hi) << 16);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Elementwise maximum over each 16-lane DPP row of the wavefront, applied to
// two packed unsigned 16-bit halves.  After quad_perm [1,0,3,2] and
// [2,3,0,1] every lane holds its quad's maximum; row_half_mirror folds the two
// quads of each half-row, row_mirror the two half-rows.
__device__ __forceinline__ uint32_t row16_max_u16x2(uint32_t v) {
  v = max_abs_bf16x2(v, dpp<0xB1>(v));
  v = max_abs_bf16x2(v, dpp<0x4E>(v));
  v = max_abs_bf16x2(v, dpp<0x141>(v));
  v = max_abs_bf16x2(v, dpp<0x140>(v));
  return v;
}

// Same reduction for non-negative FP32 values (compared as unsigned bits).
__device__ __forceinline__ float row16_max_f32(float f) {
  uint32_t v = __float_as_uint(f);
  v = max(v, dpp<0xB1>(v));
  v = max(v, dpp<0x4E>(v));
  v = max(v, dpp<0x141>(v));
  v = max(v, dpp<0x140>(v));
  return __uint_as_float(v);
}

// ---------------------------------------------------------------------------
// Scale pair of a group.
// ---------------------------------------------------------------------------
struct ScalePair {
  float s;  // stored scale (dequantisation multiplier)
  float r;  // quantisation multiplier
};

__device__ __forceinline__ ScalePair scale_pair(float amax) {
  const float a = fmaxf(amax, kAmaxFloor);
  return ScalePair{a / kE4M3Max, kE4M3Max / a};
}

// ---------------------------------------------------------------------------
// E4M3 conversion.  v_cvt_pk_fp8_f32 on gfx950 converts to OCP E4M3 with
// round-to-nearest-even; the packed byte order is (a, b) into bytes 0/1 of the
// selected half-word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <int BYTE>
__device__ __forceinline__ float e4m3_at(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, BYTE);
}

// BF16 bits of a finite FP32 value, round to nearest even.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace jet
