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

// out[i] = the value of lane i of the caller's 16-lane DPP row, i = 0..7
// (row_newbcast; every lane of the row must be active).
__device__ __forceinline__ void row_bcast8(float v, float out[8]) {
  const int b = __float_as_int(v);
  out[0] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x150, 0xF, 0xF, false));
  out[1] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x151, 0xF, 0xF, false));
  out[2] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x152, 0xF, 0xF, false));
  out[3] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x153, 0xF, 0xF, false));
  out[4] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x154, 0xF, 0xF, false));
  out[5] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x155, 0xF, 0xF, false));
  out[6] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x156, 0xF, 0xF, false));
  out[7] = __int_as_float(__builtin_amdgcn_update_dpp(0, b, 0x157, 0xF, 0xF, false));
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

// Power-of-two scale (the variant for the MFMA's E8M0 operand scales):
// s = 2^e with e the smallest integer for which 448 * 2^e >= a, r = 2^-e.
// a = (1 + f/2^23) * 2^E is a normal FP32 number (a >= 2^-96) and
// 448 = 1.75 * 2^8, so e = E - 8 when f <= 0.75 * 2^23 and E - 7 otherwise;
// -104 <= e <= 120 for finite amax, so both s and r are normal and exact.
__device__ __forceinline__ ScalePair scale_pair_pow2(float amax) {
  const uint32_t b = __float_as_uint(fmaxf(amax, kAmaxFloor));
  const int e = (int)(b >> 23) - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return ScalePair{__uint_as_float((uint32_t)(127 + e) << 23), __uint_as_float((uint32_t)(127 - e) << 23)};
}

template <bool P2>
__device__ __forceinline__ ScalePair scale_rule(float amax) {
  if constexpr (P2) return scale_pair_pow2(amax);
  else return scale_pair(amax);
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

// BF16 bits of two FP32 values, round to nearest even, packed (lo in bits
// 0..15): one v_cvt_pk_bf16_f32.  For every non-NaN input, denormals
// included, it gives the bits of the integer rounding (u + 0x7FFF + bit 16
// of u) >> 16; NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---------------------------------------------------------------------------
// Streaming (non-temporal) global accesses for data touched once: the loads
// and stores bypass the caches' normal allocation, which keeps a kernel that
// runs after a large producer from first evicting that producer's dirty lines.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream8(void* p, uint32_t lo, uint32_t hi) {
  const u32x2_t v = {lo, hi};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void store_stream16(void* p, uint4 w) {
  const u32x4_t v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// 1x128 quantization of BF16 data laid out as NP passes per wavefront, each
// 16-lane DPP row holding one 128-element group per pass (8 values, 4 dwords,
// per lane).  The group maxima of every pass come first; lane L of the
// wavefront then takes the maximum of pass L/4, DPP row L%4, so one scale
// computation covers the wavefront's 4*NP groups, and each pass fetches its
// multiplier back.  Same codes and scales as one scale computation per group.
// Every lane of the wavefront must be active.  Returns the scale s of the
// lane's group (pass lane/4, DPP row lane%4; meaningful for lane < 4*NP).
// ---------------------------------------------------------------------------
template <int NP, bool P2>
__device__ __forceinline__ float quant_1x128_passes(const uint4 (&w)[NP], uint2 (&codes)[NP]) {
  static_assert(NP >= 1 && 4 * NP <= 64, "one group per lane");
  const int lane = threadIdx.x & 63;
  float am[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t a = max_abs_bf16x2(0u, w[p].x);
    a = max_abs_bf16x2(a, w[p].y);
    a = max_abs_bf16x2(a, w[p].z);
    a = max_abs_bf16x2(a, w[p].w);
    am[p] = fold_bf16x2(row16_max_u16x2(a));
  }
  float a_all = 0.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float x = __shfl(am[p], 16 * (lane & 3), 64);
    if ((lane >> 2) == p) a_all = x;
  }
  const ScalePair sp = scale_rule<P2>(a_all);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const float r = __shfl(sp.r, 4 * p + (lane >> 4), 64);
    codes[p].x = e4m3x4(bf16_lo(w[p].x) * r, bf16_hi(w[p].x) * r, bf16_lo(w[p].y) * r, bf16_hi(w[p].y) * r);
    codes[p].y = e4m3x4(bf16_lo(w[p].z) * r, bf16_hi(w[p].z) * r, bf16_lo(w[p].w) * r, bf16_hi(w[p].w) * r);
  }
  return sp.s;
}

// ---------------------------------------------------------------------------
// Segments of a grouped (mixture-of-experts) problem.  seg[0..E] are the
// device row offsets of the experts' segments; each bound is clamped to
// [0, rows] and a segment's end to at least its start, so malformed offsets
// give wrong results but no access outside the matrices.  Segment e owns
// ceil(len_e / unit) consecutive slots (row tiles, 128-row groups) starting
// at slot `first`.  One wavefront computes the prefix sums with shuffles
// (every wavefront of a block may call it; the result is wave-uniform).
// ---------------------------------------------------------------------------
struct SegHit {
  int e;       // segment, or -1 if no segment owns the slot
  int first;   // its first slot
  int lo, hi;  // its rows [lo, hi)
};

// Slots over all segments: the sum of ceil(rows of segment e / unit).
__device__ __forceinline__ int seg_total(const int32_t* seg, int E, int rows, int unit) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int c = 0; c < E; c += 64) {
    const int e = c + lane;
    if (e < E) {
      const int lo = min(max(seg[e], 0), rows);
      const int hi = min(max(seg[e + 1], lo), rows);
      sum += (hi - lo + unit - 1) / unit;
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
  return __builtin_amdgcn_readfirstlane(sum);
}

// At most 128 segments: the segment at position q (0 <= q < E) when they are
// ordered by slot count, largest first, equal counts by index; `first` is its
// first slot in index order, as for seg_find.  Lane l holds segments l and
// l + 64; every offset is loaded in one round.
__device__ __forceinline__ SegHit seg_by_size_128(const int32_t* seg, int E, int rows, int unit, int q) {
  const int lane = threadIdx.x & 63;
  int o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = lane + 64 * (k >> 1) + (k & 1);
    o[k] = (i <= E) ? seg[i] : 0;
  }
  int lo[2], hi[2], cnt[2], excl[2];
  bool in[2];
  int base = 0, top = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    in[h] = lane + 64 * h < E;
    lo[h] = in[h] ? min(max(o[2 * h], 0), rows) : 0;
    hi[h] = in[h] ? min(max(o[2 * h + 1], lo[h]), rows) : 0;
    cnt[h] = (hi[h] - lo[h] + unit - 1) / unit;
    int incl = cnt[h];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    excl[h] = base + incl - cnt[h];
    base += __shfl(incl, 63, 64);
    top = max(top, cnt[h]);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) top = max(top, __shfl_xor(top, d, 64));
  top = __builtin_amdgcn_readfirstlane(top);
  // segments with at least t slots
  auto count_ge = [&](int t) {
    return __popcll(__ballot(in[0] && cnt[0] >= t)) + __popcll(__ballot(in[1] && cnt[1] >= t));
  };
  // the largest count T with more than q segments at or above it
  int T = 0;
  for (int b = 31 - __clz(max(top, 1)); b >= 0; --b)
    if (count_ge(T | (1 << b)) > q) T |= 1 << b;
  // the n-th segment (by index) among those with exactly T slots
  int n = q - count_ge(T + 1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const unsigned long long m = __ballot(in[h] && cnt[h] == T);
    const int c = __popcll(m);
    if (n < c) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      const unsigned long long w = __ballot(((m >> lane) & 1ull) && below == n);
      const int l = __ffsll((long long)w) - 1;
      SegHit s;
      s.e = 64 * h + l;
      s.first = __shfl(excl[h], l, 64);
      s.lo = __shfl(lo[h], l, 64);
      s.hi = __shfl(hi[h], l, 64);
      return s;
    }
    n -= c;
  }
  return SegHit{-1, 0, 0, 0};
}

// by_e = false: the segment owning slot `target`; by_e = true: segment `target`.
__device__ __forceinline__ SegHit seg_find(const int32_t* seg, int E, int rows, int unit,
                                           int target, bool by_e) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int c = 0; c < E; c += 64) {
    const int e = c + lane;
    int lo = 0, hi = 0, cnt = 0;
    if (e < E) {
      lo = min(max(seg[e], 0), rows);
      hi = min(max(seg[e + 1], lo), rows);
      cnt = (hi - lo + unit - 1) / unit;
    }
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int excl = incl - cnt;
    const bool hit = by_e ? (e == target)
                          : (e < E && cnt > 0 && base + excl <= target && target < base + incl);
    const unsigned long long m = __ballot(hit);
    if (m != 0ull) {
      const int l = __ffsll((long long)m) - 1;
      SegHit h;
      h.e = c + l;
      h.first = base + __shfl(excl, l, 64);
      h.lo = __shfl(lo, l, 64);
      h.hi = __shfl(hi, l, 64);
      return h;
    }
    base += __shfl(incl, 63, 64);
  }
  return SegHit{-1, 0, 0, 0};
}

}  // namespace jet
