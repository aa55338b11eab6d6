// Block-scaled FP8 GEMMs for gfx950:  C[m,n] = sum_kb scale(kb,m,n) * sum_{k in kb} A[m,k]*B[n,k]
//
// A [rows, Kc] and B [cols, Kc] are E4M3 codes with the contraction axis
// contiguous ("NT"); kb runs over 128-wide contraction steps.  The three GEMMs
// of the Jet-RL linear layer (gist.science explainer, section
// "Quantisierungsschema": forward, DGrad and WGrad all in FP8) map onto it:
//
//   forward  Y  = Xq  . Wq^T   scale = sX[kb][m] * sW[n/128][kb]       (ROWBLOCK)
//   dgrad    dX = dYq . WqT^T  scale = sdY[kb][m] * sW[kb][k/128]      (ROWBLOCK)
//   wgrad    dW = dYqT . XqT^T scale = sdYT[kb][n] * sXT[kb][k]         (ROWCOL)
//
// Numerics: each 128-K step is ONE v_mfma_f32_16x16x128_f8f6f4 per 16x16
// output sub-tile, started from zero; its partial is folded into the FP32
// accumulator with one FMA per element using that step's product of scales.
// The FP32 group scales are thus applied exactly once per step and element,
// with no power-of-two restriction, and the MFMA never sums more than 128
// products (it adds them internally at reduced precision).
//
// Tiling (one 256-thread workgroup per CU, 4 wavefronts as 2 x 2):
//   block tile 256 x 128, wave tile 128 x 64 = 8 x 4 MFMA sub-tiles.
//   A three-stage LDS ring is filled by direct global->LDS 16-byte loads
//   (global_load_lds_dwordx4) two K steps ahead of the compute; each stage
//   holds the A and B tiles of one step (16-byte chunks XOR-swizzled by row,
//   conflict-free for both the DMA writes and the 32-byte fragment reads) and
//   that step's row scales and column scales (or, for ROWBLOCK, the block
//   scale).  Every load of the K loop is one of these DMAs; one barrier per
//   K step.
//
// The direct loads are issued with inline asm so that this kernel, not the
// compiler, chooses the vmcnt waits: vector-memory loads retire in issue
// order, so waiting until at most the next stage's loads are outstanding
// means the current stage has landed.  (The compiler would otherwise wait for
// all LDS-bound loads before the first LDS read.)
//
// MFMA operand mapping: lane l supplies row (l % 16) of its 16-row slab and the
// 32 contraction bytes 32*(l/16)..+31 of the step, for A and for B alike; since
// both operands use the same (lane, byte) -> k assignment, every k of the step
// meets its partner exactly once.  Result lane l, element r is row
// 4*(l/16)+r, column l%16 of the sub-tile.
#include "jet_device.hpp"
#include "jet_launch.hpp"

namespace jet {

namespace {

constexpr int kBM = 256, kBN = 128, kBK = 128;
constexpr int kThreads = 256;
constexpr int kStages = 3;
constexpr int kATile = kBM * kBK;                         // 32 KiB
constexpr int kBTile = kBN * kBK;                         // 16 KiB
constexpr int kSA = kBM * 4;                              // row scales of the step
constexpr int kSB = kBN * 4;                              // column scales of the step
constexpr int kStage = kATile + kBTile + kSA + kSB;       // 50688 bytes
constexpr int kEpiF32Pitch = kBN + 4;                     // floats per staged output row
constexpr int kEpiBf16Pitch = kBN + 8;                    // bf16 per staged output row
constexpr int kLdsBytes = (kStages * kStage > kBM * kEpiF32Pitch * 4) ? kStages * kStage
                                                                      : kBM * kEpiF32Pitch * 4;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)(p);
}

// The DMA helpers set M0 (the LDS destination base).  The compiler treats M0
// as reserved and ignores it in clobber lists; nothing else in these kernels
// reads M0 (plain ds_read/ds_write on gfx950 do not use it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// 64 lanes x 16 bytes from sbase + voff (per lane) to LDS [ldsa, ldsa + 1024).
__device__ __forceinline__ void dma16(uint32_t ldsa, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(ldsa), "v"(voff), "s"(sbase) : "memory", "m0");
}

// active lanes x 4 bytes from sbase + voff to LDS [ldsa + 4*lane].
__device__ __forceinline__ void dma4(uint32_t ldsa, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(ldsa), "v"(voff), "s"(sbase) : "memory", "m0");
}

#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ v8i frag32(const uint8_t* tile, int row, int kg) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + swz(row, 2 * kg));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + swz(row, 2 * kg + 1));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format 0 = E4M3 for both operands; scale operands 0 select the unscaled form.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Block index -> output tile.  Workgroups are dealt round-robin to the 8 XCDs;
// renumber so each XCD receives a contiguous range of tiles (shared operand
// panels stay in that XCD's L2), then walk tiles in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_of_block(int nbm, int nbn, int& tm, int& tn) {
  constexpr int kXcds = 8, kGroupM = 4;
  const int total = nbm * nbn;
  int b = blockIdx.x;
  if (total % kXcds == 0) b = (b % kXcds) * (total / kXcds) + b / kXcds;
  const int per_group = kGroupM * nbn;
  const int group = b / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(nbm - first_m, kGroupM);
  const int in_group = b - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

}  // namespace

template <int MODE, int OUT, bool ACCUM, bool FUSEQ>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_fp8(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  constexpr int kLoadsPerStage = 8 + 4 + 1 + 1;   // DMA instructions per wavefront and stage

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 15, kg = lane >> 4;

  const int nbm = (p.M + kBM - 1) / kBM;
  const int nbn = p.N / kBN;
  int tm, tn;
  tile_of_block(nbm, nbn, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int KB = p.Kc / kBK;
  const uint32_t lds0 = lds_addr(lds);

  // ---- per-lane DMA source offsets (bytes from the step's base pointers) ----
  // Instruction t of wave w fills LDS rows 8g..8g+7 (g = group), lane L the
  // physical chunk L%8 of row 8g + L/8, which holds logical chunk (L%8)^(L/8).
  const uint32_t dchunk = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  uint32_t offA[8], offB[4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = (wave * 8 + t) * 8 + (lane >> 3);
    offA[t] = (uint32_t)min(m0 + row, p.M - 1) * (uint32_t)p.lda + dchunk;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = (wave * 4 + t) * 8 + (lane >> 3);
    offB[t] = (uint32_t)(n0 + row) * (uint32_t)p.ldb + dchunk;
  }
  const uint32_t offSA = (uint32_t)min(m0 + wave * 64 + lane, p.M - 1) * 4u;
  const uint32_t offSB = (uint32_t)(n0 + wave * 32 + (lane & 31)) * 4u;
  const float* gsb = p.sB + (int64_t)(n0 / kBN) * p.sB_o;     // ROWBLOCK: this block's scale row

#define JET_ISSUE(stage_, kb_)                                                               \
  do {                                                                                       \
    const uint32_t sbase_ = lds0 + (uint32_t)((stage_) * kStage);                            \
    const uint8_t* ga_ = p.A + (int64_t)(kb_) * kBK;                                         \
    const uint8_t* gb_ = p.B + (int64_t)(kb_) * kBK;                                         \
    _Pragma("unroll") for (int t_ = 0; t_ < 8; ++t_)                                         \
      dma16(sbase_ + (uint32_t)((wave * 8 + t_) * 1024), ga_, offA[t_]);                     \
    _Pragma("unroll") for (int t_ = 0; t_ < 4; ++t_)                                         \
      dma16(sbase_ + (uint32_t)(kATile + (wave * 4 + t_) * 1024), gb_, offB[t_]);            \
    dma4(sbase_ + (uint32_t)(kATile + kBTile + wave * 256), p.sA + (int64_t)(kb_) * p.sA_ld, \
         offSA);                                                                             \
    if (MODE == kRowCol) {                                                                   \
      if (lane < 32)                                                                         \
        dma4(sbase_ + (uint32_t)(kATile + kBTile + kSA + wave * 128),                        \
             p.sB + (int64_t)(kb_) * p.sB_c, offSB);                                         \
    } else if (lane == 0) {                                                                  \
      dma4(sbase_ + (uint32_t)(kATile + kBTile + kSA + wave * 4),                            \
           gsb + (int64_t)(kb_) * p.sB_c, 0u);                                               \
    }                                                                                        \
  } while (0)

  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (KB > 0) JET_ISSUE(0, 0);
  if (KB > 1) JET_ISSUE(1, 1);

  int st = 0;
  for (int kb = 0; kb < KB; ++kb) {
    if (kb + 1 < KB) wait_vmem<kLoadsPerStage>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kb + 2 < KB) {
      const int st2 = (st + 2 >= kStages) ? st + 2 - kStages : st + 2;
      JET_ISSUE(st2, kb + 2);
    }
    const uint8_t* As = lds + st * kStage;
    const uint8_t* Bs = As + kATile;
    const float* sAs = reinterpret_cast<const float*>(Bs + kBTile);
    const float* sBs = sAs + kBM;
    const float sblk = (MODE == kRowBlock) ? sBs[0] : 0.0f;   // the block scale of this step

    v8i bf[4];
    float cb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf[j] = frag32(Bs, wn * 64 + j * 16 + lrow, kg);
      cb[j] = (MODE == kRowCol) ? sBs[wn * 64 + j * 16 + lrow] : sblk;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const v8i af = frag32(As, wm * 128 + i * 16 + lrow, kg);
      const float4 rsc = *reinterpret_cast<const float4*>(sAs + wm * 128 + i * 16 + 4 * kg);
      const float rsv[4] = {rsc.x, rsc.y, rsc.z, rsc.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4f part = mfma_fp8(af, bf[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(part[r], rsv[r] * cb[j], acc[i][j][r]);
      }
    }
    st = (st + 1 == kStages) ? 0 : st + 1;
  }
#undef JET_ISSUE
  __syncthreads();

  // ---- epilogue: stage the 256x128 tile in LDS, then coalesced row stores ----
  const int rbase = wm * 128 + 4 * kg;
  const int cbase = wn * 64 + lrow;
  if (OUT == kOutF32) {
    float* t = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          t[(rbase + i * 16 + r) * kEpiF32Pitch + cbase + j * 16] = acc[i][j][r];
    __syncthreads();
    float* C = static_cast<float*>(p.C);
#pragma unroll 4
    for (int pass = 0; pass < 32; ++pass) {
      const int id = tid + kThreads * pass;
      const int row = id >> 5, c4 = id & 31;
      const int m = m0 + row;
      if (m < p.M) {
        float4 v = *reinterpret_cast<const float4*>(t + row * kEpiF32Pitch + 4 * c4);
        float4* dst = reinterpret_cast<float4*>(C + (int64_t)m * p.ldc + n0 + 4 * c4);
        if (ACCUM) {
          const float4 o = *dst;
          v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
        }
        *dst = v;
      }
    }
  } else {
    uint16_t* t = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          t[(rbase + i * 16 + r) * kEpiBf16Pitch + cbase + j * 16] = (uint16_t)bf16_rne(acc[i][j][r]);
    __syncthreads();
    uint16_t* C = static_cast<uint16_t*>(p.C);
    const int c8 = tid & 15;
#pragma unroll 2
    for (int pass = 0; pass < 16; ++pass) {
      const int row = (tid >> 4) + 16 * pass;
      const int m = m0 + row;
      const uint4 v = *reinterpret_cast<const uint4*>(t + row * kEpiBf16Pitch + 8 * c8);
      if (FUSEQ) {
        // 1x128 quantization of this BF16 output row segment (one DPP row = one group)
        uint32_t am = max_abs_bf16x2(0u, v.x);
        am = max_abs_bf16x2(am, v.y);
        am = max_abs_bf16x2(am, v.z);
        am = max_abs_bf16x2(am, v.w);
        am = row16_max_u16x2(am);
        const ScalePair sp = scale_pair(fold_bf16x2(am));
        const uint32_t q0 = e4m3x4(bf16_lo(v.x) * sp.r, bf16_hi(v.x) * sp.r,
                                   bf16_lo(v.y) * sp.r, bf16_hi(v.y) * sp.r);
        const uint32_t q1 = e4m3x4(bf16_lo(v.z) * sp.r, bf16_hi(v.z) * sp.r,
                                   bf16_lo(v.w) * sp.r, bf16_hi(v.w) * sp.r);
        if (m < p.M) {
          *reinterpret_cast<uint2*>(p.Cq + (int64_t)m * p.ldc + n0 + 8 * c8) = make_uint2(q0, q1);
          if (c8 == 0) p.Cs[(int64_t)(n0 / kBN) * p.M + m] = sp.s;
        }
      }
      if (m < p.M) *reinterpret_cast<uint4*>(C + (int64_t)m * p.ldc + n0 + 8 * c8) = v;
    }
  }
}

template <int MODE, int OUT, bool ACCUM, bool FUSEQ>
static hipError_t launch_one(const GemmArgs& a, hipStream_t st) {
  const int nbm = (a.M + kBM - 1) / kBM;
  const int nbn = a.N / kBN;
  hipLaunchKernelGGL((k_gemm_fp8<MODE, OUT, ACCUM, FUSEQ>), dim3((unsigned)(nbm * nbn)),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int mode, int out, bool accum, bool fuseq,
                       hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (mode == kRowBlock) {
    if (fuseq) return launch_one<kRowBlock, kOutBf16, false, true>(a, st);
    if (out == kOutBf16) return launch_one<kRowBlock, kOutBf16, false, false>(a, st);
    return launch_one<kRowBlock, kOutF32, false, false>(a, st);
  }
  if (out == kOutBf16) return launch_one<kRowCol, kOutBf16, false, false>(a, st);
  if (accum) return launch_one<kRowCol, kOutF32, true, false>(a, st);
  return launch_one<kRowCol, kOutF32, false, false>(a, st);
}

}  // namespace jet
