// E4M3 group quantizers for gfx950 (bandwidth-bound; no MFMA).
//
//  * 1x128 groups along the row (activations, output gradients): gist.science
//    explainer "Jet-RL ...", section "Quantisierungsschema"; nmedialink table
//    in section "为什么FP8适配线性层？" ([1,128], FP32 scale).
//  * 128x128 blocks (weights, re-quantized from the BF16 master on every weight
//    sync): same sources ([128,128]); 66260.cn FP8-RL item, weight-sync paragraph.
//  * 128x1 groups along the token axis, written transposed, for the weight
//    gradient: explainer "Quantisierungsschema" (128x1 for WGrad); 163.com
//    write-up section 五 (1x128 activations re-quantized as 128x1).
//
// Every kernel reads each input byte once from HBM with 16-byte loads, keeps
// the group in registers, reduces the group maximum with integer/DPP
// operations inside one wavefront (plus one LDS exchange for the 128x128
// block), and writes codes with 8-byte stores.  Accesses whose wavefront
// instruction covers whole 128-byte lines that no other wavefront touches use
// the streaming (non-temporal) forms; partial-line accesses keep the normal
// forms, so the L2 merges the pieces of a line.
#include <algorithm>

#include "jet_device.hpp"
#include "jet_launch.hpp"

namespace jet {

// ---------------------------------------------------------------------------
// 1x128.  One 16-lane DPP row handles one group of 128 BF16 values (256 bytes,
// 16 bytes per lane).  Work is cut into units of 32 rows x 4 consecutive
// groups (32 KiB of input): in each of a 256-thread block's 8 passes, the 4
// DPP rows of a wavefront take 4 rows of the same group (whole 128-byte
// lines), all loads issued before any compute.  The unit's 128 scales are
// staged in LDS (double-buffered, one barrier per unit) and written as 4 runs
// of 32 consecutive rows, so the scale stores are whole lines as well.  A
// block strides over the units by the grid size; consecutive units continue
// along the rows.
// ---------------------------------------------------------------------------
template <bool P2>
__global__ __launch_bounds__(256) void k_quant_1x128(const uint16_t* __restrict__ x, int64_t M,
                                                     int64_t K, int64_t ldx,
                                                     uint8_t* __restrict__ q, int64_t ldq,
                                                     float* __restrict__ s) {
  __shared__ float stg[2][4][32];
  const int64_t G = K / kGroup;
  const int64_t ugc = (G + 3) / 4;                 // units along a row block
  const int64_t units = ((M + 31) / 32) * ugc;
  const int dr = threadIdx.x >> 4, lane16 = threadIdx.x & 15;
  int buf = 0;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x, buf ^= 1) {
    const int64_t m0 = (u / ugc) * 32, j0 = (u % ugc) * 4;
    uint4 v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t m = m0 + 16 * (p & 1) + dr, j = j0 + (p >> 1);
      v[p] = make_uint4(0u, 0u, 0u, 0u);
      if (m < M && j < G) v[p] = load_stream16(x + m * ldx + j * kGroup + lane16 * 8);
    }
    // codes of all 8 passes, one scale computation for the wavefront's 32 groups
    uint2 qc[8];
    const float sc = quant_1x128_passes<8, P2>(v, qc);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t m = m0 + 16 * (p & 1) + dr, j = j0 + (p >> 1);
      if (m < M && j < G) store_stream8(q + m * ldq + j * kGroup + lane16 * 8, qc[p].x, qc[p].y);
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

hipError_t launch_quant_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                              int64_t ldq, float* s, hipStream_t st, bool p2) {
  if (M == 0 || K == 0) return hipSuccess;
  constexpr int64_t kMaxBlocks = 2048;
  const int64_t units = ((M + 31) / 32) * ((K / kGroup + 3) / 4);
  const int64_t blocks = std::min<int64_t>(units, kMaxBlocks);
  if (p2)
    hipLaunchKernelGGL(k_quant_1x128<true>, dim3((unsigned)blocks), dim3(256), 0, st, x, M, K, ldx, q, ldq, s);
  else
    hipLaunchKernelGGL(k_quant_1x128<false>, dim3((unsigned)blocks), dim3(256), 0, st, x, M, K, ldx, q, ldq, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x128.  One 256-thread block per block of the weight; thread t owns rows
// 8*(t/16)..+7 and columns 8*(t%16)..+7, i.e. an 8x8 tile held in registers.
// The block maximum: packed-u16 max over the tile, DPP over the 16 lanes of a
// row, then one LDS exchange between the 16 DPP rows of the block.  Row-major
// codes are packed along the tile's rows, transposed codes along its columns.
// ---------------------------------------------------------------------------
// Byte offset in the staged transposed weight tile of byte `b` of row k.
__device__ __forceinline__ int tT_off(int k, int b) {
  return (k ^ ((k >> 3) & 1)) * kGroup + (b ^ (((k >> 3) & 7) << 4));
}

template <bool P2>
__global__ __launch_bounds__(256) void k_quant_128x128(const uint16_t* __restrict__ w, int64_t N,
                                                       int64_t K, int64_t ldw,
                                                       uint8_t* __restrict__ q,
                                                       float* __restrict__ s,
                                                       uint8_t* __restrict__ qT) {
  __shared__ uint32_t red[16];
  __shared__ __attribute__((aligned(16))) uint8_t tT[kGroup * kGroup];
  const int c = threadIdx.x & 15;
  const int ri = threadIdx.x >> 4;
  const int64_t kb = blockIdx.x, nb = blockIdx.y;
  const int64_t n0 = nb * kGroup + 8 * ri;
  const int64_t k0 = kb * kGroup + 8 * c;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = load_stream16(w + (n0 + i) * ldw + k0);
  uint32_t am = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    am = max_abs_bf16x2(am, v[i].x);
    am = max_abs_bf16x2(am, v[i].y);
    am = max_abs_bf16x2(am, v[i].z);
    am = max_abs_bf16x2(am, v[i].w);
  }
  am = row16_max_u16x2(am);
  if (c == 0) red[ri] = am;
  __syncthreads();
  am = red[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) am = max_abs_bf16x2(am, red[i]);
  const ScalePair sp = scale_rule<P2>(fold_bf16x2(am));
  if (threadIdx.x == 0) s[nb * (K / kGroup) + kb] = sp.s;

  float f[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[i][0] = bf16_lo(v[i].x) * sp.r; f[i][1] = bf16_hi(v[i].x) * sp.r;
    f[i][2] = bf16_lo(v[i].y) * sp.r; f[i][3] = bf16_hi(v[i].y) * sp.r;
    f[i][4] = bf16_lo(v[i].z) * sp.r; f[i][5] = bf16_hi(v[i].z) * sp.r;
    f[i][6] = bf16_lo(v[i].w) * sp.r; f[i][7] = bf16_hi(v[i].w) * sp.r;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t lo = e4m3x4(f[i][0], f[i][1], f[i][2], f[i][3]);
    const uint32_t hi = e4m3x4(f[i][4], f[i][5], f[i][6], f[i][7]);
    store_stream8(q + (n0 + i) * K + k0, lo, hi);
  }
  if (qT != nullptr) {
    // Transposed codes through LDS, so every global store covers whole
    // 128-byte lines of qT: a thread holds 8 bytes of each of its 8 qT rows;
    // the block's 128 x 128 qT tile is staged with rows permuted
    // (k ^ ((k >> 3) & 1)) and 16-byte chunks XOR-swizzled by (k >> 3) & 7 to
    // spread the LDS banks, then written back 8 lanes per row.
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int kl = 8 * c + jj;
      const uint32_t lo = e4m3x4(f[0][jj], f[1][jj], f[2][jj], f[3][jj]);
      const uint32_t hi = e4m3x4(f[4][jj], f[5][jj], f[6][jj], f[7][jj]);
      *reinterpret_cast<uint2*>(tT + tT_off(kl, 8 * ri)) = make_uint2(lo, hi);
    }
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int kl = pass * 32 + (threadIdx.x >> 3), chunk = threadIdx.x & 7;
      const uint4 v16 = *reinterpret_cast<const uint4*>(tT + tT_off(kl, 16 * chunk));
      store_stream16(qT + (kb * kGroup + kl) * N + nb * kGroup + 16 * chunk, v16);
    }
  }
}

hipError_t launch_quant_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                float* s, uint8_t* qT, hipStream_t st, bool p2) {
  if (N == 0 || K == 0) return hipSuccess;
  dim3 grid((unsigned)(K / kGroup), (unsigned)(N / kGroup));
  if (p2)
    hipLaunchKernelGGL(k_quant_128x128<true>, grid, dim3(256), 0, st, w, N, K, ldw, q, s, qT);
  else
    hipLaunchKernelGGL(k_quant_128x128<false>, grid, dim3(256), 0, st, w, N, K, ldw, q, s, qT);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 1x128 and 128x1 (transposed) from one read of a BF16 activation.  A block
// of 256*RG threads takes RG 128-row groups of one 128-column block kb; thread
// t owns rows 8*(t/16)..+7 and columns 8*(t%16)..+7, an 8x8 tile in
// registers, as in the 128x128 kernel.  1x128: each of the thread's rows is a
// group spread over one 16-lane DPP row; each lane computes one row's scale
// pair and a DPP broadcast hands it to the row; the codes are 8-byte pieces
// of whole 128-byte lines.  128x1: a column's maximum reduces over the
// thread's 8 rows, the wavefront's 4 row slabs (lane xor 16, 32) and the row
// group's 4 wavefronts (LDS, one thread per column for the scale pair); the
// transposed codes are staged in LDS and leave as whole lines, 128*RG
// contiguous bytes per qT row.
//
// REQUANT (activations): the 128x1 groups quantize the dequantized 1x128
// values fl32(E4M3value(code) * scale), i.e. exactly what the 128x1 kernel
// computes from the 1x128 codes.  Otherwise (output gradients) they quantize
// the BF16 values themselves.  Both sets of outputs equal those of the two
// separate quantizers bit for bit.  Rows at or past M are zeros: they have no
// 1x128 output and encode to zero codes in the transposed padding columns.
// ---------------------------------------------------------------------------
template <bool REQUANT, int RG, bool P2>
__global__ __launch_bounds__(256 * RG) void k_quant_1x128_128x1_T(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ s, uint8_t* __restrict__ qT, int64_t ldqT,
    float* __restrict__ sT) {
  constexpr int CR = REQUANT ? 8 : 4;       // column-maximum words per thread
  __shared__ uint32_t cred[4 * RG][16][CR]; // per wavefront: column maxima of its 16 chunks
  __shared__ float colR[RG][kGroup];        // 128x1 quantisation multipliers of the tile's columns
  __shared__ __attribute__((aligned(16))) uint8_t tT[RG][kGroup * kGroup];
  const int c = threadIdx.x & 15;
  const int ri = threadIdx.x >> 4;          // 8-row slab of the block's 128*RG rows
  const int gi = ri >> 4;                   // row group within the block (wavefronts 4gi..4gi+3)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t G = (M + kGroup - 1) / kGroup;
  const int64_t kb = blockIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * RG * kGroup + 8 * ri;
  const int64_t k0 = kb * kGroup + 8 * c;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (m0 + i < M) v[i] = load_stream16(x + (m0 + i) * ldx + k0);
  }

  // 1x128: the maximum of each of the thread's 8 rows over its DPP row; lane
  // c computes the scale pair of row c % 8 and row_newbcast hands each row's
  // pair to the whole DPP row (one division pair per lane instead of eight).
  uint32_t amr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t am = max_abs_bf16x2(0u, v[i].x);
    am = max_abs_bf16x2(am, v[i].y);
    am = max_abs_bf16x2(am, v[i].z);
    am = max_abs_bf16x2(am, v[i].w);
    amr[i] = row16_max_u16x2(am);
  }
  uint32_t mine = amr[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mine = ((c & 7) == i) ? amr[i] : mine;
  const ScalePair own = scale_rule<P2>(fold_bf16x2(mine));
  if (c < 8 && m0 + c < M) s[kb * M + m0 + c] = own.s;
  float rr[8], rs[8];
  row_bcast8(own.r, rr);
  row_bcast8(own.s, rs);

  // 1x128 codes.  The tile is kept as raw BF16 words (or, for the
  // re-quantisation, as codes and row scales) and its FP32 values are
  // recomputed in each phase: 64 live floats would halve the resident blocks.
  uint32_t cw[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float r = rr[i];
    cw[i][0] = e4m3x4(bf16_lo(v[i].x) * r, bf16_hi(v[i].x) * r, bf16_lo(v[i].y) * r, bf16_hi(v[i].y) * r);
    cw[i][1] = e4m3x4(bf16_lo(v[i].z) * r, bf16_hi(v[i].z) * r, bf16_lo(v[i].w) * r, bf16_hi(v[i].w) * r);
    if (m0 + i < M) store_stream8(q + (m0 + i) * ldq + k0, cw[i][0], cw[i][1]);
  }
  // value of row i, column jj of the thread's tile (jj a compile-time index)
  auto value = [&](int i, int jj) __attribute__((always_inline)) -> float {
    if constexpr (REQUANT) {
      const uint32_t wd = cw[i][jj >> 2];
      float d;
      switch (jj & 3) {
        case 0: d = e4m3_at<0>(wd); break;
        case 1: d = e4m3_at<1>(wd); break;
        case 2: d = e4m3_at<2>(wd); break;
        default: d = e4m3_at<3>(wd); break;
      }
      return d * rs[i];
    } else {
      const uint32_t wd = (jj >> 1) == 0 ? v[i].x : (jj >> 1) == 1 ? v[i].y : (jj >> 1) == 2 ? v[i].z : v[i].w;
      return (jj & 1) ? bf16_hi(wd) : bf16_lo(wd);
    }
  };

  // 128x1 column maxima over the thread's 8 rows and the wavefront's 4 row
  // slabs: packed BF16 magnitudes, or FP32 magnitude bits (re-quantisation)
  uint32_t cm[CR];
#pragma unroll
  for (int d = 0; d < CR; ++d) {
    uint32_t u;
    if constexpr (REQUANT) {
      float a = fabsf(value(0, d));
#pragma unroll
      for (int i = 1; i < 8; ++i) a = fmaxf(a, fabsf(value(i, d)));
      u = __float_as_uint(a);
      u = max(u, (uint32_t)__shfl_xor((int)u, 16, 64));
      u = max(u, (uint32_t)__shfl_xor((int)u, 32, 64));
    } else {
      u = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        u = max_abs_bf16x2(u, d == 0 ? v[i].x : d == 1 ? v[i].y : d == 2 ? v[i].z : v[i].w);
      u = max_abs_bf16x2(u, (uint32_t)__shfl_xor((int)u, 16, 64));
      u = max_abs_bf16x2(u, (uint32_t)__shfl_xor((int)u, 32, 64));
    }
    cm[d] = u;
  }
  if (lane < 16) {
#pragma unroll
    for (int d = 0; d < CR; ++d) cred[wave][c][d] = cm[d];
  }
  __syncthreads();
  // one thread per column of each row group: its maximum over the group's 4
  // wavefronts and its scale pair
  if (threadIdx.x < kGroup * RG) {
    const int cg = threadIdx.x >> 7, col = threadIdx.x & (kGroup - 1), cc = col >> 3, jj = col & 7;
    float amax;
    if constexpr (REQUANT) {
      uint32_t u = cred[4 * cg][cc][jj];
#pragma unroll
      for (int w = 1; w < 4; ++w) u = max(u, cred[4 * cg + w][cc][jj]);
      amax = __uint_as_float(u);
    } else {
      uint32_t u = cred[4 * cg][cc][jj >> 1];
#pragma unroll
      for (int w = 1; w < 4; ++w) u = max_abs_bf16x2(u, cred[4 * cg + w][cc][jj >> 1]);
      amax = __uint_as_float(((jj & 1) ? (u >> 16) : (u & 0xFFFFu)) << 16);
    }
    const ScalePair sp = scale_rule<P2>(amax);
    colR[cg][col] = sp.r;
    const int64_t gg = (int64_t)blockIdx.y * RG + cg;
    if (gg < G) sT[gg * K + kb * kGroup + col] = sp.s;
  }
  __syncthreads();
  float rT[8];
  {
    const float4 r0 = *reinterpret_cast<const float4*>(&colR[gi][8 * c]);
    const float4 r1 = *reinterpret_cast<const float4*>(&colR[gi][8 * c + 4]);
    rT[0] = r0.x; rT[1] = r0.y; rT[2] = r0.z; rT[3] = r0.w;
    rT[4] = r1.x; rT[5] = r1.y; rT[6] = r1.z; rT[7] = r1.w;
  }
  // transposed codes through LDS (layout of the 128x128 kernel's staging);
  // the tile's values are recomputed here, not kept live across the barriers
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (REQUANT) {
      asm volatile("" : "+v"(cw[i][0]), "+v"(cw[i][1]));
    } else {
      asm volatile("" : "+v"(v[i].x), "+v"(v[i].y), "+v"(v[i].z), "+v"(v[i].w));
    }
  }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const float r = rT[jj];
    const uint32_t lo = e4m3x4(value(0, jj) * r, value(1, jj) * r, value(2, jj) * r, value(3, jj) * r);
    const uint32_t hi = e4m3x4(value(4, jj) * r, value(5, jj) * r, value(6, jj) * r, value(7, jj) * r);
    *reinterpret_cast<uint2*>(&tT[gi][tT_off(8 * c + jj, 8 * (ri & 15))]) = make_uint2(lo, hi);
  }
  __syncthreads();
  // each qT row takes 128*RG contiguous bytes (the block's row groups side by side)
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int kl = pass * 32 + (threadIdx.x >> (3 + (RG == 2))), chunk = threadIdx.x & (8 * RG - 1);
    const int h = chunk >> 3;
    const uint4 v16 = *reinterpret_cast<const uint4*>(&tT[h][tT_off(kl, 16 * (chunk & 7))]);
    if ((int64_t)blockIdx.y * RG + h < G)
      store_stream16(qT + (kb * kGroup + kl) * ldqT + (int64_t)blockIdx.y * RG * kGroup + 16 * chunk, v16);
  }
}

hipError_t launch_quant_1x128_128x1_T(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* s, uint8_t* qT,
                                      int64_t ldqT, float* sT, bool requant, hipStream_t st, bool p2) {
  if (M == 0 || K == 0) return hipSuccess;
  // One row group per 256-thread block (128-byte runs in every qT row, still
  // whole lines): with 100 VGPRs per lane four blocks share a CU in different
  // phases of load, reduce and store, against two 512-thread blocks; dY of
  // the Llama-8B gate+up (8192 x 28672) 205.7 -> 185.6 us, bit-identical.
  constexpr int RG = 1;
  const int64_t G = (M + kGroup - 1) / kGroup;
  dim3 grid((unsigned)(K / kGroup), (unsigned)((G + RG - 1) / RG));
#define JET_Q11T(rq_, p2_)                                                                       \
  hipLaunchKernelGGL((k_quant_1x128_128x1_T<rq_, RG, p2_>), grid, dim3(256 * RG), 0, st, x, M, K, \
                     ldx, q, ldq, s, qT, ldqT, sT)
  if (requant) {
    if (p2) JET_Q11T(true, true); else JET_Q11T(true, false);
  } else {
    if (p2) JET_Q11T(false, true); else JET_Q11T(false, false);
  }
#undef JET_Q11T
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 128x1, transposed.  A block handles one 128-row group g and 16*CW columns
// (256 source bytes per row).  Thread t owns rows 8*ri .. 8*ri+7 of the group
// and the CW columns of 16-byte chunk c (ri, c in 0..15), with lane
// (c % 8) + 8 * (ri % 8) of wavefront (ri / 8) + 2 * (c / 8): each wavefront
// load covers 8 rows x 128 contiguous bytes (whole cache lines).  A column's
// maximum is reduced over the thread's 8 rows, across the 8 row slabs of the
// wavefront (lane-index xor 8, 16, 32), then with the one other wavefront
// holding the same columns through LDS.  Codes of column k for the thread's 8
// rows are packed into one 8-byte store at qT[k][128g + 8*ri]; the two
// wavefronts that share columns write the two halves of each 128-byte qT row
// segment.  Rows past the group's end are zeros: they do not change a column
// maximum and they encode to 0x00 in the padding columns.
//
// FP8SRC: the source is the 1x128-quantized activation (codes + [K/128, M]
// scales); the value re-quantized is fl32(E4M3value(code) * scale).
//
// GROUPED: the rows are expert segments seg[e] .. seg[e+1]-1 and groups restart
// at each segment; blockIdx.y is the group's slot g over all segments
// (segment e owns slots first_e .. first_e + ceil(len_e/128) - 1), which is
// also its output column block: the padded layout of the grouped WGrad.
// ---------------------------------------------------------------------------
template <bool FP8SRC, bool GROUPED, bool P2>
__global__ __launch_bounds__(256) void k_quant_128x1_T(const void* __restrict__ src,
                                                       const float* __restrict__ src_s,
                                                       int64_t M, int64_t K, int64_t ldsrc,
                                                       const int32_t* __restrict__ seg, int E,
                                                       uint8_t* __restrict__ qT, int64_t ldqT,
                                                       float* __restrict__ sT) {
  constexpr int CW = FP8SRC ? 16 : 8;
  __shared__ float red[4][8][CW];     // per wavefront: column maxima of its 8 chunks
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ri = (lane >> 3) + 8 * (wave & 1);
  const int c = (lane & 7) + 8 * (wave >> 1);
  const int64_t g = blockIdx.y;
  int64_t row_begin = g * kGroup, row_end = M;
  if constexpr (GROUPED) {
    const SegHit h = seg_find(seg, E, (int)M, kGroup, (int)g, false);
    if (h.e < 0) return;
    row_begin = h.lo + (int64_t)(g - h.first) * kGroup;
    row_end = h.hi;
  }
  const int64_t col0 = (int64_t)blockIdx.x * (16 * CW) + (int64_t)c * CW;
  const bool colok = col0 < K;
  const int64_t m0 = row_begin + 8 * ri;      // first source row of this thread
  const int64_t o0 = g * kGroup + 8 * ri;     // its first output column

  float f[8][CW];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + i;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (colok && m < row_end) {
      if (FP8SRC)
        v = load_stream16(static_cast<const uint8_t*>(src) + m * ldsrc + col0);
      else
        v = load_stream16(static_cast<const uint16_t*>(src) + m * ldsrc + col0);
    }
    if constexpr (FP8SRC) {
      float sc = 0.0f;
      if (colok && m < row_end) sc = src_s[(col0 / kGroup) * M + m];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f[i][4 * d + 0] = e4m3_at<0>(wv[d]) * sc;
        f[i][4 * d + 1] = e4m3_at<1>(wv[d]) * sc;
        f[i][4 * d + 2] = e4m3_at<2>(wv[d]) * sc;
        f[i][4 * d + 3] = e4m3_at<3>(wv[d]) * sc;
      }
    } else {
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f[i][2 * d + 0] = bf16_lo(wv[d]);
        f[i][2 * d + 1] = bf16_hi(wv[d]);
      }
    }
  }

  // column maxima (non-negative floats compared as unsigned integers)
  uint32_t am[CW];
#pragma unroll
  for (int jj = 0; jj < CW; ++jj) {
    float a = fabsf(f[0][jj]);
#pragma unroll
    for (int i = 1; i < 8; ++i) a = fmaxf(a, fabsf(f[i][jj]));
    uint32_t u = __float_as_uint(a);
    u = max(u, (uint32_t)__shfl_xor((int)u, 8, 64));
    u = max(u, (uint32_t)__shfl_xor((int)u, 16, 64));
    u = max(u, (uint32_t)__shfl_xor((int)u, 32, 64));
    am[jj] = u;
  }
  if (lane < 8) {
#pragma unroll
    for (int jj = 0; jj < CW; ++jj) red[wave][lane][jj] = __uint_as_float(am[jj]);
  }
  __syncthreads();
  float rr[CW];
  float ss[CW];
#pragma unroll
  for (int jj = 0; jj < CW; ++jj) {
    const uint32_t other = __float_as_uint(red[wave ^ 1][lane & 7][jj]);
    const ScalePair sp = scale_rule<P2>(__uint_as_float(max(am[jj], other)));
    rr[jj] = sp.r;
    ss[jj] = sp.s;
  }
  if (!colok) return;
  if (ri == 0) {
#pragma unroll
    for (int jj = 0; jj < CW; jj += 4)
      *reinterpret_cast<float4*>(sT + g * K + col0 + jj) =
          make_float4(ss[jj], ss[jj + 1], ss[jj + 2], ss[jj + 3]);
  }
#pragma unroll
  for (int jj = 0; jj < CW; ++jj) {
    const float r = rr[jj];
    const uint32_t lo = e4m3x4(f[0][jj] * r, f[1][jj] * r, f[2][jj] * r, f[3][jj] * r);
    const uint32_t hi = e4m3x4(f[4][jj] * r, f[5][jj] * r, f[6][jj] * r, f[7][jj] * r);
    *reinterpret_cast<uint2*>(qT + (col0 + jj) * ldqT + o0) = make_uint2(lo, hi);
  }
}

template <bool GROUPED, bool P2>
static hipError_t launch_128x1_T(const void* src, bool fp8src, const float* src_s, int64_t M,
                                 int64_t K, int64_t ldsrc, const int32_t* seg, int E,
                                 unsigned groups, uint8_t* qT, int64_t ldqT, float* sT,
                                 hipStream_t st) {
  if (fp8src) {
    dim3 grid((unsigned)((K + 255) / 256), groups);
    hipLaunchKernelGGL((k_quant_128x1_T<true, GROUPED, P2>), grid, dim3(256), 0, st, src, src_s, M, K,
                       ldsrc, seg, E, qT, ldqT, sT);
  } else {
    dim3 grid((unsigned)(K / kGroup), groups);
    hipLaunchKernelGGL((k_quant_128x1_T<false, GROUPED, P2>), grid, dim3(256), 0, st, src, src_s, M,
                       K, ldsrc, seg, E, qT, ldqT, sT);
  }
  return hipGetLastError();
}

hipError_t launch_quant_128x1_T(const void* src, bool fp8src, const float* src_s, int64_t M,
                                int64_t K, int64_t ldsrc, uint8_t* qT, int64_t ldqT, float* sT,
                                hipStream_t st, bool p2) {
  if (M == 0 || K == 0) return hipSuccess;
  const unsigned groups = (unsigned)((M + kGroup - 1) / kGroup);
  if (p2)
    return launch_128x1_T<false, true>(src, fp8src, src_s, M, K, ldsrc, nullptr, 0, groups, qT, ldqT, sT, st);
  return launch_128x1_T<false, false>(src, fp8src, src_s, M, K, ldsrc, nullptr, 0, groups, qT, ldqT, sT,
                                      st);
}

hipError_t launch_quant_128x1_T_grouped(const void* src, bool fp8src, const float* src_s,
                                        int64_t M, int64_t K, int64_t ldsrc, const int32_t* seg,
                                        int E, uint8_t* qT, int64_t ldqT, float* sT,
                                        hipStream_t st, bool p2) {
  if (M == 0 || K == 0) return hipSuccess;
  // at most ceil(M/128) + E groups over all segments
  const unsigned slots = (unsigned)((M + kGroup - 1) / kGroup + E);
  if (p2) return launch_128x1_T<true, true>(src, fp8src, src_s, M, K, ldsrc, seg, E, slots, qT, ldqT, sT, st);
  return launch_128x1_T<true, false>(src, fp8src, src_s, M, K, ldsrc, seg, E, slots, qT, ldqT, sT, st);
}

}  // namespace jet
