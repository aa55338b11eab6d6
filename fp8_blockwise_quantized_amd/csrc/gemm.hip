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
// Power-of-two variant (P2): when every group scale is a power of two (the
// pow2 quantizers), each scale is the MFMA's own E8M0 operand scale (lane
// l's byte scales row l % 16 of its slab, the same byte on all four lane
// groups since a scale covers the whole 128-K step), and each step's MFMA
// accumulates straight into the FP32 accumulator, which it adds at full FP32
// precision: no per-step partial, no fold, no scale products.
//
// Structure (the tile shape, wave layout, stage count and LDS layout are the
// compile-time parameters of GemmCfg):
//   * WMW x WNW wavefronts, each owning TM x TN 16x16 sub-tiles; block tile
//     BM x BN = (WMW*TM*16) x (WNW*TN*16); OCC workgroups resident per CU
//     (independent barriers, so one fills the other's per-step ramp).
//   * A ring of STAGES LDS stages filled by direct global->LDS 16-byte loads
//     (global_load_lds_dwordx4), STAGES-1 K steps ahead of the compute.  A
//     stage holds the A and B tiles of one step, that step's row scales
//     (ordered so each lane reads its TM rows with TM/4 contiguous 16-byte
//     loads) and column scales (or, for ROWBLOCK, the 128-column block
//     scales).  Every load of the K loop is one of these DMAs; one barrier per
//     K step, at its start.  The next step's DMAs are issued between this
//     step's MFMAs (one after every other MFMA), so they have almost a whole
//     step to land.  Fragment addresses are compile-time LDS offsets from
//     per-lane bases (no per-step address arithmetic).
//   * Tile layout in LDS, either
//       ROWS: row-major 128-byte rows, 16-byte chunks XOR-swizzled per row
//             (see swz); each DMA reads 8 whole rows;
//       FRAG: MFMA-fragment order, each 16-row slab as two 1 KiB blocks, block
//             h holding at lane l's 16-byte slot the bytes 64*h + 16*(l/16)
//             .. +15 of slab row l%16; each fragment read is one contiguous
//             1 KiB ds_read_b128 and each DMA reads 64 contiguous bytes of
//             16 rows.
//
// The direct loads are issued with inline asm so that this kernel, not the
// compiler, chooses the vmcnt waits: vector-memory loads retire in issue
// order, so waiting until at most the later stages' loads are outstanding
// means the current stage has landed.  (The compiler would otherwise wait for
// every LDS-bound load before the first LDS read.)
//
// MFMA operand mapping: lane l supplies row (l % 16) of its 16-row slab and 32
// contraction bytes chosen by l/16 (the same bytes for A and for B, so every
// k of the step meets its partner exactly once).  The B slab is passed as the
// MFMA's first operand, so result lane l, element r is C row (l % 16) and C
// column 4*(l/16) + r of the sub-tile: each lane owns one row (one row scale)
// and four adjacent columns.
#include "jet_device.hpp"
#include "jet_launch.hpp"
#if JET_PHASE_TIMING
#include "../../include/jetphase.h"
#endif

namespace jet {

#if JET_PHASE_TIMING
// Phase timing, compiled only into the diagnostic build libjetfp8_phase.so
// (include/jetphase.h): while the flag is non-zero, thread 0 of workgroup b
// < kPhaseBlocks of k_gemm_fp8 records in record b: the constant-rate wall
// counter at its entry, before its first DMA, after its K loop and at its
// exit; its hardware ids; and the shader-clock counter before and after the
// K loop.
constexpr int kPhaseBlocks = 16384;
__device__ unsigned long long g_phase[kPhaseBlocks * 8];
__device__ int g_phase_on;
struct PhaseRec {
  unsigned long long t0, t1 = 0, t2 = 0, c1 = 0, c2 = 0;
  __device__ PhaseRec() : t0(wall_clock64()) {}
  __device__ void loop_start() { t1 = wall_clock64(); c1 = clock64(); }
  __device__ void loop_end() { t2 = wall_clock64(); c2 = clock64(); }
  __device__ ~PhaseRec() {
    if (g_phase_on && threadIdx.x == 0 && blockIdx.x < kPhaseBlocks) {
      unsigned long long* r = g_phase + 8 * blockIdx.x;
      r[0] = t0; r[1] = t1; r[2] = t2; r[3] = wall_clock64();
      r[4] = (unsigned long long)__builtin_amdgcn_s_getreg(63492) |     // HW_REG_HW_ID
             ((unsigned long long)__builtin_amdgcn_s_getreg(63508) << 32);   // HW_REG_XCC_ID
      r[5] = gridDim.x | ((unsigned long long)blockDim.x << 32);
      r[6] = c1; r[7] = c2;
    }
  }
};
#endif

template <int WMW_, int WNW_, int TM_, int TN_, int STAGES_, bool FRAG_, int OCC_ = 1>
struct GemmCfg {
  static constexpr int WMW = WMW_, WNW = WNW_, TM = TM_, TN = TN_, STAGES = STAGES_;
  static constexpr int OCC = OCC_;                 // workgroups resident per CU
  static constexpr bool FRAG = FRAG_;
  static constexpr int NW = WMW * WNW;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = WMW * TM * 16, BN = WNW * TN * 16;
  static constexpr int ATILE = BM * 128, BTILE = BN * 128;
  static constexpr int ABLK = ATILE / 1024 / NW;   // A DMA instructions per wave and stage
  static constexpr int BBLK = BTILE / 1024 / NW;
  static constexpr int OA = TM / WNW, OB = TN / WMW;   // A and B slabs of a wave's DMA share
  static constexpr int RQ = BM / 64;                   // row-scale DMAs (64 rows each) per stage
  static constexpr int CQ = BN / 64;                   // column-scale DMAs (ROWCOL) per stage
  static constexpr int SCL = BM * 4 + 1024;            // scale bytes per stage: rows, then columns
  static constexpr int STAGE = ATILE + BTILE + SCL;
  static constexpr int LOADS = ABLK + BBLK;            // tile DMAs per wave and stage (+1 scale DMA
                                                       // for waves 0 .. RQ+CQ-1)
  static constexpr int EPI_PITCH = BN + 8;             // bf16 per staged output row
  static constexpr int EPI_PITCH_F32 = BN + 4;         // floats per staged FP32 output row (one wave row)
  static constexpr int EPI = (BM * EPI_PITCH * 2 > TM * 16 * EPI_PITCH_F32 * 4) ? BM * EPI_PITCH * 2
                                                                              : TM * 16 * EPI_PITCH_F32 * 4;
  static constexpr int LDS = (STAGES * STAGE > EPI) ? STAGES * STAGE : EPI;
  static_assert(ABLK * NW * 1024 == ATILE && BBLK * NW * 1024 == BTILE, "DMA split");
  static_assert(ABLK * 8 == OA * 16 && BBLK * 8 == OB * 16, "a wave's DMA rows are whole slabs");
  static_assert(BM % 64 == 0 && BN % 64 == 0 && BN * 4 <= 1024 && NW >= RQ + CQ, "scale DMA shape");
  static_assert((TM * 16) % 64 == 0 || TM * 16 == 64, "row-scale regions of whole DMAs");
  static_assert(TM % 4 == 0 && (128 % (TN * 16)) == 0 && BN % 128 == 0, "tile shape");
  static_assert((TM & (TM - 1)) == 0 && (TN & (TN - 1)) == 0, "power-of-two slab counts");
  static_assert(LDS * OCC <= 160 * 1024, "LDS");
};

namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)(p);
}

// The DMA helpers set M0 (the LDS destination base).  The compiler treats M0
// as reserved and ignores it in clobber lists; nothing else in these kernels
// reads M0 (plain ds_read/ds_write on gfx950 do not use it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// The LDS address and the base pointer are wave-uniform; readfirstlane puts
// them in SGPRs even where the compiler would keep them in VGPRs (inside
// lane-divergent branches).
__device__ __forceinline__ uint32_t sgpr(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void* sgpr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = sgpr((uint32_t)v), hi = sgpr((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(lo | (hi << 32));
}

// 64 lanes x 16 bytes from sbase + voff (per lane) to LDS [ldsa, ldsa + 1024).
__device__ __forceinline__ void dma16(uint32_t ldsa, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(sgpr(ldsa)), "v"(voff), "s"(sgpr(sbase)) : "memory", "m0");
}

// active lanes x 4 bytes from sbase + voff to LDS [ldsa + 4*lane].
__device__ __forceinline__ void dma4(uint32_t ldsa, const void* sbase, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(sgpr(ldsa)), "v"(voff), "s"(sgpr(sbase)) : "memory", "m0");
}

#pragma clang diagnostic pop

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "i"(N) : "memory");
}

template <bool B> struct BoolC { static constexpr bool value = B; };

// Row-major layout: 16-byte chunk c of tile row r sits at chunk slot
// c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1).  A fragment read has lane l read
// chunk 2*(l/16) (+1) of row l % 16: any 8 consecutive lanes then hit 8
// different chunk slots (all 32 four-byte banks of a 128-byte row), and any
// 16 consecutive lanes hit 16 different (row parity, slot) pairs (all 64 banks
// when rows alternate between the two halves of 64 banks), so the read is
// conflict-free whether the LDS serves 8 or 16 lanes of a b128 read per cycle.
__device__ __forceinline__ int swz_f(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ swz_f(row)) << 4);
}

template <bool FRAG>
__device__ __forceinline__ v8i frag32(const uint8_t* tile, int slab, int lane) {
  uint4 lo, hi;
  if (FRAG) {
    const uint8_t* b = tile + slab * 2048 + lane * 16;
    lo = *reinterpret_cast<const uint4*>(b);
    hi = *reinterpret_cast<const uint4*>(b + 1024);
  } else {
    const int row = slab * 16 + (lane & 15), kg = lane >> 4;
    lo = *reinterpret_cast<const uint4*>(tile + swz(row, 2 * kg));
    hi = *reinterpret_cast<const uint4*>(tile + swz(row, 2 * kg + 1));
  }
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Per-lane global byte offset (within the step's 128 columns) and tile row of
// DMA block g (1 KiB of LDS).
template <bool FRAG>
__device__ __forceinline__ void dma_src(int g, int lane, int& row, uint32_t& col) {
  if (FRAG) {
    row = (g >> 1) * 16 + (lane & 15);
    col = (uint32_t)(64 * (g & 1) + 16 * (lane >> 4));
  } else {
    row = g * 8 + (lane >> 3);
    col = (uint32_t)(((lane & 7) ^ swz_f(row)) << 4);
  }
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format 0 = E4M3 for both operands; scale operands 0 select the unscaled form.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// c + (2^(ea-127) a) . (2^(eb-127) b): per-lane E8M0 operand scales (byte 0 of
// ea / eb; lane l's byte scales row l % 16 of its operand), the sum added to c
// at full FP32 precision.
__device__ __forceinline__ v4f mfma_fp8_e8m0(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// E8M0 byte of a positive power-of-two FP32 scale: its biased exponent field.
__device__ __forceinline__ int e8m0_of(float s) { return (int)(__float_as_uint(s) >> 23); }

// Block index -> output tile.  Workgroups are dealt round-robin to the 8 XCDs
// (block b to XCD b % 8), each with its own L2.  When the tile grid splits
// evenly, each XCD takes one block of a gy x gx split of it, the split that
// minimises the operand panels the XCDs fetch (gx copies of A's rows, gy
// copies of B's columns); a split into row blocks only (gy = 8), or no even
// split, gives each XCD a contiguous range of the grid's walk instead.
// Either way an XCD walks its part in groups of kGroupM tile-rows.
__device__ __forceinline__ void tile_of_block(int nbm, int nbn, int& tm, int& tn) {
  constexpr int kXcds = 8, kGroupM = 4;
  const int total = nbm * nbn;
  int b = blockIdx.x;
  int gy = 0, gx = 0, cost = 0x7fffffff;
  if (total % kXcds == 0) {
#pragma unroll
    for (int y = 1; y <= kXcds; y *= 2) {
      const int x = kXcds / y;
      const int c = x * nbm + y * nbn;
      if (nbm % y == 0 && nbn % x == 0 && c < cost) { cost = c; gy = y; gx = x; }
    }
  }
  int rows = nbm, cols = nbn, r0 = 0, c0 = 0;
  if (gy > 0 && gy < kXcds) {
    const int xcd = b % kXcds;
    b /= kXcds;
    rows = nbm / gy;
    cols = nbn / gx;
    r0 = (xcd / gx) * rows;
    c0 = (xcd % gx) * cols;
  } else if (total % kXcds == 0) {
    b = (b % kXcds) * (total / kXcds) + b / kXcds;
  }
  const int per_group = kGroupM * cols;
  const int group = b / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(rows - first_m, kGroupM);
  const int in_group = b - group * per_group;
  tm = r0 + first_m + in_group % gsz;
  tn = c0 + in_group / gsz;
}

}  // namespace

template <class CFG, int MODE, int OUT, bool ACCUM, bool FUSEQ, int GRP, bool P2>
__global__ __launch_bounds__(CFG::THREADS, CFG::OCC) void k_gemm_fp8(GemmArgs pa) {
  constexpr int TM = CFG::TM, TN = CFG::TN, BM = CFG::BM, BN = CFG::BN;
  constexpr bool FRAG = CFG::FRAG;
  constexpr int64_t kOutBytes = (OUT == kOutF32) ? 4 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[CFG::LDS];
#if JET_PHASE_TIMING
  PhaseRec phase;
#endif

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % CFG::WMW, wn = wave / CFG::WMW;
  const int lrow = lane & 15, kg = lane >> 4;

  // This workgroup's problem: the whole GEMM, or (grouped) one expert's part.
  GemmArgs p = pa;
  int tm, tn;
  if constexpr (GRP == kGrpNone) {
    tile_of_block((p.M + BM - 1) / BM, (p.N + BN - 1) / BN, tm, tn);
  } else if constexpr (GRP == kGrpRows) {
    // tile = (row tile of the concatenated segments) x (column tile), row
    // major.  The grid (a multiple of the 8 XCDs) bounds the tiles from the
    // row count; XCD b%8 takes its contiguous eighth of the tiles that exist
    // (so the segments' rounding leaves no XCD idle while another has twice
    // its share), workgroup b/8 of the XCD its (b/8)-th tile.
    constexpr int kXcds = 8;
    const int nbn = (p.N + BN - 1) / BN;
    const int total = seg_total(p.seg, p.E, p.seg_rows, BM) * nbn;
    const int per = (total + kXcds - 1) / kXcds;
    const int i = (int)blockIdx.x / kXcds;
    const int slot = ((int)blockIdx.x % kXcds) * per + i;
    if (i >= per || slot >= total) return;
    const int r = slot / nbn;
    tn = slot - r * nbn;
    tm = 0;
    const SegHit h = seg_find(p.seg, p.E, p.seg_rows, BM, r, false);
    const int e = __builtin_amdgcn_readfirstlane(h.e);
    if (e < 0) return;
    const int row0 = __builtin_amdgcn_readfirstlane(h.lo + (r - h.first) * BM);
    p.M = __builtin_amdgcn_readfirstlane(h.hi) - row0;
    p.A += (int64_t)row0 * p.lda;
    p.sA += row0;
    p.C = static_cast<uint8_t*>(p.C) + (int64_t)row0 * p.ldc * kOutBytes;
    if (FUSEQ) {
      p.Cq += (int64_t)row0 * p.ldc;
      p.Cs += row0;
    }
    p.B += (int64_t)e * p.bE;
    p.sB += (int64_t)e * p.sbE;
  } else {
    // slot = (expert position) x (output tile); an expert contracts over its
    // padded columns.  Slots keep the hardware's round-robin deal to the
    // XCDs: with a multiple of 8 tiles per expert every XCD gets an equal
    // share of every expert, however unequal the segments (a contiguous
    // range of experts per XCD leaves the XCD with the largest experts doing
    // twice the mean work under a Zipf load), and the XCDs work on the same
    // experts at the same time, so their L2 refills of an expert's operands
    // meet in the MALL.  Experts are taken longest contraction first (up to
    // 128 experts; beyond that in index order), so the last workgroups to
    // start are the shortest and the CUs run out of work together.
    const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
    const int slot = (int)blockIdx.x;
    const int q = slot / (nbm * nbn);
    if (q >= p.E) return;
    const int local = slot - q * (nbm * nbn);
    tm = local / nbn;
    tn = local - tm * nbn;
    // With a multiple of 8 tiles per expert, XCD slot%8 takes one block of a
    // gy x gx split of the expert's tile grid (the split that minimises the
    // operand strips the XCDs fetch, as for the dense grid) instead of every
    // eighth tile of the row-major walk.
    if ((nbm * nbn) % 8 == 0) {
      int gy = 0, gx = 0, cost = 0x7fffffff;
#pragma unroll
      for (int y = 1; y <= 8; y *= 2) {
        const int x = 8 / y, c = x * nbm + y * nbn;
        if (nbm % y == 0 && nbn % x == 0 && c < cost) { cost = c; gy = y; gx = x; }
      }
      if (gy > 0) {
        const int xcd = local % 8, idx = local / 8;
        const int rows = nbm / gy, cols = nbn / gx;
        tm = (xcd / gx) * rows + idx % rows;
        tn = (xcd % gx) * cols + idx / rows;
      }
    }
    const SegHit h = (p.E <= 128) ? seg_by_size_128(p.seg, p.E, p.seg_rows, 128, q)
                                  : seg_find(p.seg, p.E, p.seg_rows, 128, q, true);
    const int e = __builtin_amdgcn_readfirstlane(h.e);
    if (e < 0) return;
    const int first = __builtin_amdgcn_readfirstlane(h.first);
    const int groups = __builtin_amdgcn_readfirstlane((h.hi - h.lo + 127) / 128);
    const int c0 = min(first * 128, p.kcap);
    const int c1 = min((first + groups) * 128, p.kcap);
    p.Kc = c1 - c0;
    p.A += c0;
    p.B += c0;
    p.sA += (int64_t)(c0 / 128) * p.sA_ld;
    p.sB += (int64_t)(c0 / 128) * p.sB_c;
    p.C = static_cast<uint8_t*>(p.C) + (int64_t)e * p.cE * kOutBytes;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int KB = p.Kc / 128;
  const uint32_t lds0 = lds_addr(lds);
  // 64-bit bases at the tile's first row of A and of B (and, for ROWBLOCK, its
  // first weight-block scale row): the 32-bit per-lane DMA offsets then stay
  // below 256 rows times the row stride (< 2^32 for strides up to 2^24 bytes,
  // the limit the entry points check), whatever the operand's size.
  p.A += (int64_t)m0 * p.lda;
  p.B += (int64_t)n0 * p.ldb;
  if (MODE == kRowBlock) p.sB += (int64_t)(n0 / 128) * p.sB_o;

  // ---- the wave's share of every stage ----
  // Wave (wm, wn) DMAs the OA 16-row A slabs wn*OA .. wn*OA+OA-1 of its wave
  // row and the OB 16-row B slabs wm*OB .. of its wave column; the workgroup
  // barrier at the top of each step makes every wave's share visible to all.
  constexpr int OA = CFG::OA, OB = CFG::OB;
  const int gA0 = (wm * TM * 16 + wn * OA * 16) / 8;   // first 1 KiB DMA block (8 rows) of the share
  const int gB0 = (wn * TN * 16 + wm * OB * 16) / 8;
  uint32_t offA[CFG::ABLK], offB[CFG::BBLK];
#pragma unroll
  for (int t = 0; t < CFG::ABLK; ++t) {
    int row; uint32_t col;
    dma_src<FRAG>(gA0 + t, lane, row, col);
    offA[t] = (uint32_t)min(row, p.M - 1 - m0) * (uint32_t)p.lda + col;
  }
#pragma unroll
  for (int t = 0; t < CFG::BBLK; ++t) {
    int row; uint32_t col;
    dma_src<FRAG>(gB0 + t, lane, row, col);
    offB[t] = (uint32_t)min(row, p.N - 1 - n0) * (uint32_t)p.ldb + col;
  }
  // Scales of the stage, shared by the workgroup (the barrier at the top of a
  // step covers them).  Rows: the region of wave row wm holds its TM*16 rows
  // with slot 64*(i/4) + 4*lrow + (i%4) = row i*16 + lrow, so each lane reads
  // its TM row scales as TM/4 16-byte loads.  Columns (after the BM row
  // slots): ROWCOL in natural column order, ROWBLOCK the tile's 128-column
  // block scales (one copy per remaining wave, read from the first).  Every
  // wave issues exactly one scale DMA per stage, its source chosen without a
  // branch, so the K-step body stays one basic block: waves 0..RQ-1 the row
  // scales (64 each), the others the column scales.
  static_assert(MODE == kRowBlock ? (CFG::NW > CFG::RQ && CFG::NW - CFG::RQ <= 4)
                                  : CFG::NW - CFG::RQ == CFG::CQ, "one scale DMA per wave");
  const bool srow = wave < CFG::RQ;
  uint32_t offS, sdst;
  if (srow) {
    const int sl = 64 * wave + lane;
    const int wm_ = sl / (TM * 16), w_ = sl % (TM * 16);
    const int i_ = 4 * (w_ >> 6) + (w_ & 3), lr_ = (w_ >> 2) & 15;
    offS = (uint32_t)min(m0 + wm_ * TM * 16 + i_ * 16 + lr_, p.M - 1) * 4u;
    sdst = (uint32_t)(CFG::ATILE + CFG::BTILE + 256 * wave);
  } else {
    const int c_ = wave - CFG::RQ;
    if (MODE == kRowCol) {
      offS = (uint32_t)min(n0 + 64 * c_ + lane, p.N - 1) * 4u;
    } else {
      // lanes 0..BN/128-1 the tile's blocks (relative to its first); the rest
      // repeat the last one
      const int blk = min(min(lane, CFG::BN / 128 - 1), p.N / 128 - 1 - n0 / 128);
      offS = (uint32_t)blk * (uint32_t)p.sB_o * 4u;
    }
    sdst = (uint32_t)(CFG::ATILE + CFG::BTILE + CFG::BM * 4 + 256 * c_);
  }

  // DMA part t of step kb into stage `stage`: t < ABLK + BBLK is one 1 KiB
  // tile DMA, t == ABLK + BBLK the wave's scale DMA (if it has one).
  constexpr int NT = CFG::ABLK + CFG::BBLK;
#define JET_ISSUE(part_, stage_, kb_)                                                          \
  do {                                                                                         \
    const uint32_t sbase_ = lds0 + (uint32_t)((stage_) * CFG::STAGE);                          \
    if ((part_) < CFG::ABLK) {                                                                 \
      dma16(sbase_ + (uint32_t)((gA0 + (part_)) * 1024), p.A + (int64_t)(kb_) * 128,           \
            offA[(part_) < CFG::ABLK ? (part_) : 0]);                                          \
    } else if ((part_) < NT) {                                                                 \
      const int t_ = (part_) < NT ? (part_) - CFG::ABLK : 0;                                   \
      dma16(sbase_ + (uint32_t)(CFG::ATILE + (gB0 + t_) * 1024), p.B + (int64_t)(kb_) * 128,  \
            offB[t_]);                                                                         \
    } else {                                                                                   \
      const float* sp_ = srow ? p.sA + (int64_t)(kb_) * p.sA_ld : p.sB + (int64_t)(kb_) * p.sB_c; \
      dma4(sbase_ + sdst, sp_, offS);                                                          \
    }                                                                                          \
  } while (0)

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // MFMA order of a step (slab indices of the wave tile): the OA x OB corner
  // block first (its fragments are read first), then the rest of rows
  // 0..OA-1, then rows OA.. in order.  A fragments live in a ring of R buffers
  // (row i in buffer i % R); a row whose buffer is still unused is read after
  // the corner block, any other row right after the last MFMA of row i-R.
  // (With 8 row slabs the outer-product scales of ROWCOL leave no registers
  // for the extra buffer.)
  constexpr int NM = TM * TN;
  constexpr int R = (MODE == kRowCol && TM >= 8) ? OA : OA + 1;
  struct Order { int i[NM]; int j[NM]; int load_after[TM]; };
  constexpr Order ORD = []() {
    Order o{};
    int n = 0;
    for (int i = 0; i < OA; ++i)
      for (int j = 0; j < OB; ++j) { o.i[n] = i; o.j[n] = j; ++n; }
    for (int i = 0; i < OA; ++i)
      for (int j = OB; j < TN; ++j) { o.i[n] = i; o.j[n] = j; ++n; }
    for (int i = OA; i < TM; ++i)
      for (int j = 0; j < TN; ++j) { o.i[n] = i; o.j[n] = j; ++n; }
    for (int i = 0; i < TM; ++i) o.load_after[i] = -1;        // -1: read at the step start
    for (int i = OA; i < TM; ++i) {
      int last = OA * OB - 1;                                   // after the corner block
      for (int m = 0; m < NM; ++m)
        if (i - R >= 0 && o.i[m] == i - R) last = m;
      o.load_after[i] = last;
    }
    return o;
  }();
  constexpr int NCORNER = OA * OB;   // MFMAs of the corner block
  constexpr int LAG = 3;

  constexpr int D = CFG::STAGES - 1;   // prefetch distance in K steps
#if JET_PHASE_TIMING
  phase.loop_start();
#endif
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < KB) {
#pragma unroll
      for (int t = 0; t < NT + 1; ++t) JET_ISSUE(t, s, s);
    }

  int kb = 0, st = 0;
  // One K step.  REFILL: this step also issues the loads of step kb + D into
  // the stage step kb - 1 used.  The body has no data-dependent branches, so
  // the compiler schedules and allocates it as one block.
  auto step = [&](auto refill_tag) __attribute__((always_inline)) {
    constexpr bool REFILL = decltype(refill_tag)::value;
    // This wave's DMAs of step kb have landed (the later steps' may stay);
    // after the barrier every wave's have, and every wave is done with step
    // kb-1, whose stage step kb+D refills.
    if (REFILL) wait_vmem<CFG::LOADS * (D - 1)>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int stn = (st + D) % CFG::STAGES;
    const uint8_t* As = lds + st * CFG::STAGE;
    const uint8_t* Bs = As + CFG::ATILE;
    const float* Sr = reinterpret_cast<const float*>(Bs + CFG::BTILE) + wm * TM * 16;   // row scales
    const float* Sc = reinterpret_cast<const float*>(Bs + CFG::BTILE) + CFG::BM;        // column scales

    v8i bf[TN];
    v8i af[R];
#pragma unroll
    for (int j = 0; j < OB; ++j) bf[j] = frag32<FRAG>(Bs, wn * TN + j, lane);
#pragma unroll
    for (int i = 0; i < OA; ++i) af[i] = frag32<FRAG>(As, wm * TM + i, lane);
    float rsc[TM];
#pragma unroll
    for (int q = 0; q < TM / 4; ++q) {
      const float4 r4 = *reinterpret_cast<const float4*>(Sr + 64 * q + 4 * lrow);
      rsc[4 * q + 0] = r4.x; rsc[4 * q + 1] = r4.y; rsc[4 * q + 2] = r4.z; rsc[4 * q + 3] = r4.w;
    }
    float cb[TN][4];
    int eb[TN], ea[TM];   // P2: E8M0 scales of the lane's B row (column of C) and A row
    if constexpr (P2) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
        eb[j] = e8m0_of(MODE == kRowCol ? Sc[wn * TN * 16 + 16 * j + lrow] : Sc[(wn * TN * 16) / 128]);
#pragma unroll
      for (int i = 0; i < TM; ++i) ea[i] = e8m0_of(rsc[i]);
    } else if (MODE == kRowCol) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const float4 c4 = *reinterpret_cast<const float4*>(Sc + wn * TN * 16 + 16 * j + 4 * kg);
        cb[j][0] = c4.x; cb[j][1] = c4.y; cb[j][2] = c4.z; cb[j][3] = c4.w;
      }
    } else {
      const float sbk = Sc[(wn * TN * 16) / 128];
#pragma unroll
      for (int i = 0; i < TM; ++i) rsc[i] *= sbk;
    }

    v4f part[LAG];
#pragma unroll
    for (int n = 0; n < NM + LAG; ++n) {
      if (!P2 && n >= LAG) {
        const int ii = ORD.i[n - LAG], jj = ORD.j[n - LAG];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float c = (MODE == kRowCol) ? rsc[ii] * cb[jj][r] : rsc[ii];
          acc[ii][jj][r] = fmaf(part[n % LAG][r], c, acc[ii][jj][r]);
        }
      }
      if (n < NM) {
        const int i = ORD.i[n], j = ORD.j[n];
        if constexpr (P2) acc[i][j] = mfma_fp8_e8m0(bf[j], af[i % R], acc[i][j], eb[j], ea[i]);
        else part[n % LAG] = mfma_fp8(bf[j], af[i % R]);
        if (n == 0) {
          // after the first MFMA: the next step's scale DMAs, the remaining
          // B fragments
          if (REFILL) {
#pragma unroll
            for (int t = NT; t < NT + 1; ++t) JET_ISSUE(t, stn, kb + D);
          }
#pragma unroll
          for (int jb = OB; jb < TN; ++jb) bf[jb] = frag32<FRAG>(Bs, wn * TN + jb, lane);
        }
        if (n >= NCORNER - 1) {
#pragma unroll
          for (int ia = OA; ia < TM; ++ia)
            if (ORD.load_after[ia] == n) af[ia % R] = frag32<FRAG>(As, wm * TM + ia, lane);
        }
        // the next step's tile DMAs, one after every other MFMA
        if (REFILL && n >= 1 && ((n - 1) & 1) == 0 && (n - 1) / 2 < NT) JET_ISSUE((n - 1) / 2, stn, kb + D);
      }
    }
    // tile DMAs not yet issued (more DMAs than MFMA slots)
    if (REFILL) {
#pragma unroll
      for (int t = NM / 2; t < NT; ++t) JET_ISSUE(t, stn, kb + D);
    }
    st = (st + 1 == CFG::STAGES) ? 0 : st + 1;
  };
  for (; kb < KB - D; ++kb) step(BoolC<true>{});
  for (; kb < KB; ++kb) step(BoolC<false>{});
#if JET_PHASE_TIMING
  phase.loop_end();
#endif
#undef JET_ISSUE

  // ---- epilogue ----
  // Lane element (i, j, r) of slabs (i, j) is
  // C[m0 + wm*TM*16 + i*16 + lrow][n0 + wn*TN*16 + j*16 + 4*kg + r].
  const int mrow = m0 + wm * TM * 16 + lrow;
  const int ncol = n0 + wn * TN * 16 + 4 * kg;
  if (OUT == kOutF32) {
    // Stage the FP32 tile in LDS one wave row (TM*16 rows) at a time and
    // write it as whole 128-byte lines: each wavefront instruction stores a
    // contiguous piece of one row.  (Stores of each lane's four columns
    // straight from the accumulators write partial lines, which the BF16
    // output measured slower.)
    float* C = static_cast<float*>(p.C);
    float* t = reinterpret_cast<float*>(lds);
    constexpr int FP = CFG::EPI_PITCH_F32;                    // floats per staged row
    constexpr int LPR = BN / 4;                               // lanes per row, 16 bytes each
    constexpr int RPP = CFG::THREADS / LPR;                   // rows per pass
    static_assert((TM * 16) % RPP == 0, "whole passes");
    const int c4 = tid % LPR;
    const int n = n0 + 4 * c4;
#pragma unroll 1
    for (int h = 0; h < CFG::WMW; ++h) {
      __syncthreads();                                        // the ring, or the previous rows, are free
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            *reinterpret_cast<float4*>(t + (i * 16 + lrow) * FP + wn * TN * 16 + j * 16 + 4 * kg) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
      __syncthreads();
#pragma unroll 4
      for (int pass = 0; pass < TM * 16 / RPP; ++pass) {
        const int r = tid / LPR + RPP * pass;
        const int m = m0 + h * TM * 16 + r;
        float4 v = *reinterpret_cast<const float4*>(t + r * FP + 4 * c4);
        if (m < p.M && n < p.N) {
          float4* dst = reinterpret_cast<float4*>(C + (int64_t)m * p.ldc + n);
          if (ACCUM) {
            const float4 o = *dst;
            v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
          }
          *dst = v;
        }
      }
    }
  } else {
    // stage the BF16 tile in LDS, then 16-byte row stores (and the fused 1x128 quantization)
    __syncthreads();
    uint16_t* t = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t lo = bf16x2_rne(acc[i][j][0], acc[i][j][1]);
        const uint32_t hi = bf16x2_rne(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2*>(t + (wm * TM * 16 + i * 16 + lrow) * CFG::EPI_PITCH +
                                  wn * TN * 16 + j * 16 + 4 * kg) = make_uint2(lo, hi);
      }
    __syncthreads();
    uint16_t* C = static_cast<uint16_t*>(p.C);
    constexpr int kLanesPerRow = BN / 8;                      // 16 bytes per lane
    constexpr int kRowsPerPass = CFG::THREADS / kLanesPerRow;
    constexpr int NP = BM / kRowsPerPass;                     // passes over the tile
    const int c8 = tid % kLanesPerRow;
    const int n = n0 + 8 * c8;
    if constexpr (FUSEQ) {
      // 1x128 quantization of the BF16 output: 16 lanes (one DPP row) hold
      // one group per pass; one scale computation per wavefront
      // (quant_1x128_passes), lane L writing the scale of pass L/4, DPP row L%4.
      uint4 v[NP];
      uint2 qc[NP];
#pragma unroll
      for (int pass = 0; pass < NP; ++pass) {
        const int row = tid / kLanesPerRow + kRowsPerPass * pass;
        v[pass] = *reinterpret_cast<const uint4*>(t + row * CFG::EPI_PITCH + 8 * c8);
      }
      const float sc = quant_1x128_passes<NP, P2>(v, qc);
      {
        const int pass = lane >> 2, tq = 64 * wave + 16 * (lane & 3);
        const int m = m0 + tq / kLanesPerRow + kRowsPerPass * pass;
        const int ng = n0 + 8 * (tq % kLanesPerRow);
        if (pass < NP && m < p.M && ng < p.N) p.Cs[(int64_t)(ng / 128) * p.ldcs + m] = sc;
      }
      // row pointers advanced by kRowsPerPass rows per pass
      const int mfirst = m0 + tid / kLanesPerRow;
      const int64_t off0 = (int64_t)mfirst * p.ldc + n, step = (int64_t)kRowsPerPass * p.ldc;
      uint8_t* cq = p.Cq + off0;
      uint16_t* cy = C + off0;
#pragma unroll
      for (int pass = 0; pass < NP; ++pass) {
        if (mfirst + kRowsPerPass * pass < p.M && n < p.N) {
          *reinterpret_cast<uint2*>(cq) = qc[pass];
          *reinterpret_cast<uint4*>(cy) = v[pass];
        }
        cq += step;
        cy += step;
      }
    } else {
#pragma unroll 2
      for (int pass = 0; pass < NP; ++pass) {
        const int row = tid / kLanesPerRow + kRowsPerPass * pass;
        const int m = m0 + row;
        const uint4 v = *reinterpret_cast<const uint4*>(t + row * CFG::EPI_PITCH + 8 * c8);
        if (m < p.M && n < p.N) *reinterpret_cast<uint4*>(C + (int64_t)m * p.ldc + n) = v;
      }
    }
  }
}

template <class CFG, int MODE, int OUT, bool ACCUM, bool FUSEQ, int GRP = kGrpNone, bool P2 = false>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t nbm = (a.M + CFG::BM - 1) / CFG::BM;
  const int64_t nbn = (a.N + CFG::BN - 1) / CFG::BN;
  int64_t blocks = nbm * nbn;
  if (GRP == kGrpRows)            // at most ceil(rows/BM) + E row tiles over all segments
    blocks = ((int64_t)(a.seg_rows + CFG::BM - 1) / CFG::BM + a.E) * nbn;
  else if (GRP == kGrpContraction)
    blocks = (int64_t)a.E * nbm * nbn;
  if (GRP != kGrpNone) blocks = (blocks + 7) / 8 * 8;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_fp8<CFG, MODE, OUT, ACCUM, FUSEQ, GRP, P2>), dim3((unsigned)blocks),
                     dim3(CFG::THREADS), 0, st, a);
  return hipGetLastError();
}

// 8 wavefronts as 2 x 4, wave tile 128 x 64, block tile 256 x 256, two stages.
using CfgMain = GemmCfg<2, 4, 8, 4, 2, false>;
// 4 wavefronts as 2 x 2, wave tile 64 x 64, block tile 128 x 128, two stages,
// two workgroups per CU: for grids whose 256 x 256 tiles leave a last partial
// wave of workgroups.
using CfgSmall = GemmCfg<2, 2, 4, 4, 2, false, 2>;

template <class CFG, int GRP = kGrpNone, bool P2 = false>
hipError_t dispatch(const GemmArgs& a, int mode, int out, bool accum, bool fuseq, hipStream_t st) {
  if (mode == kRowBlock) {
    if (fuseq) return launch_cfg<CFG, kRowBlock, kOutBf16, false, true, GRP, P2>(a, st);
    if (out == kOutBf16) return launch_cfg<CFG, kRowBlock, kOutBf16, false, false, GRP, P2>(a, st);
    return launch_cfg<CFG, kRowBlock, kOutF32, false, false, GRP, P2>(a, st);
  }
  if (out == kOutBf16) return launch_cfg<CFG, kRowCol, kOutBf16, false, false, GRP, P2>(a, st);
  if (accum) return launch_cfg<CFG, kRowCol, kOutF32, true, false, GRP, P2>(a, st);
  return launch_cfg<CFG, kRowCol, kOutF32, false, false, GRP, P2>(a, st);
}

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The output columns [n1, N), or rows [m1, M), of a GEMM as a GEMM of its own.
static GemmArgs column_part(const GemmArgs& a, int mode, int out, bool fuseq, int n1) {
  GemmArgs b = a;
  b.B += (int64_t)n1 * a.ldb;
  b.sB += (mode == kRowBlock) ? (int64_t)(n1 / 128) * a.sB_o : (int64_t)n1;
  b.C = static_cast<uint8_t*>(a.C) + (int64_t)n1 * (out == kOutF32 ? 4 : 2);
  if (fuseq) {
    b.Cq += n1;
    b.Cs += (int64_t)(n1 / 128) * a.ldcs;
  }
  b.N = a.N - n1;
  return b;
}

static GemmArgs row_part(const GemmArgs& a, int out, bool fuseq, int m1) {
  GemmArgs b = a;
  b.A += (int64_t)m1 * a.lda;
  b.sA += m1;
  b.C = static_cast<uint8_t*>(a.C) + (int64_t)m1 * a.ldc * (out == kOutF32 ? 4 : 2);
  if (fuseq) {
    b.Cq += (int64_t)m1 * a.ldc;
    b.Cs += m1;
  }
  b.M = a.M - m1;
  return b;
}

template <class CFG>
static hipError_t dispatch_p2(const GemmArgs& a, int mode, int out, bool accum, bool fuseq, hipStream_t st,
                              bool p2) {
  return p2 ? dispatch<CFG, kGrpNone, true>(a, mode, out, accum, fuseq, st)
            : dispatch<CFG>(a, mode, out, accum, fuseq, st);
}

hipError_t launch_gemm(const GemmArgs& a, int mode, int out, bool accum, bool fuseq,
                       hipStream_t st, bool p2) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  constexpr int BM = CfgMain::BM, BN = CfgMain::BN;
  const int64_t nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
  const int64_t tiles = nbm * nbn;
  const int64_t cus = cu_count();
  const auto small_tiles = [](int64_t m, int64_t n) {
    return ((m + CfgSmall::BM - 1) / CfgSmall::BM) * ((n + CfgSmall::BN - 1) / CfgSmall::BN);
  };
  // Time of a launch plan in waves of big tiles: whole waves of big tiles
  // (one per CU), then whole waves of small ones (CfgSmall::OCC per CU); a
  // wave of small tiles takes about 0.59 of a big one (a quarter of the
  // work at about 85 % of the big tile's rate, two workgroups sharing a CU).
  constexpr double kSmallWave = 0.59;
  const auto plan = [&](int64_t big, int64_t small) {
    return (double)((big + cus - 1) / cus) +
           kSmallWave * (double)((small + cus * CfgSmall::OCC - 1) / (cus * CfgSmall::OCC));
  };
  // One tile for the whole output: the big tile, which keeps the most work
  // per byte staged, unless its grid fills less than 85 % of its waves of
  // workgroups (measured: below that the idle CUs of the big tile's last wave
  // cost more than the small tile's lower rate).
  const int64_t slots = (tiles + cus - 1) / cus * cus;
  const bool big = tiles * 100 >= slots * 85;
  double best = big ? plan(tiles, 0) : plan(0, small_tiles(a.M, a.N));
  // A grid whose big tiles end in a partial wave may instead run its first
  // c1 tile columns (or r1 tile rows) in big tiles and the rest of the
  // output in small ones, as two launches, when that plan is shorter.  Every
  // element is the same chain in either tile, so the bits do not change.
  // (Llama-8B at M = 8192: wgrad of the down projection, 16 x 56 big tiles =
  // 3.5 waves, becomes 16 x 48 big tiles and one wave of 512 small ones;
  // wgrad of QKV, 24 x 16, becomes 16 x 16 and 512 small ones instead of 1536
  // small ones.)
  // (Among equal plans the most big tiles: their waves are the fullest.)
  int64_t c1 = 0, r1 = 0;
  if (tiles % cus != 0) {
    if (a.N % BN == 0)
      for (int64_t c = nbn - 1; c > 0; --c) {
        const double t = plan(nbm * c, small_tiles(a.M, a.N - c * BN));
        if (t < best - 1e-9) { best = t; c1 = c; r1 = 0; }
      }
    if (a.M % BM == 0)
      for (int64_t r = nbm - 1; r > 0; --r) {
        const double t = plan(r * nbn, small_tiles(a.M - r * BM, a.N));
        if (t < best - 1e-9) { best = t; r1 = r; c1 = 0; }
      }
  }
  if (c1 > 0) {
    GemmArgs head = a;
    head.N = (int)(c1 * BN);
    hipError_t e = dispatch_p2<CfgMain>(head, mode, out, accum, fuseq, st, p2);
    if (e != hipSuccess) return e;
    return dispatch_p2<CfgSmall>(column_part(a, mode, out, fuseq, head.N), mode, out, accum, fuseq, st, p2);
  }
  if (r1 > 0) {
    GemmArgs head = a;
    head.M = (int)(r1 * BM);
    hipError_t e = dispatch_p2<CfgMain>(head, mode, out, accum, fuseq, st, p2);
    if (e != hipSuccess) return e;
    return dispatch_p2<CfgSmall>(row_part(a, out, fuseq, head.M), mode, out, accum, fuseq, st, p2);
  }
  if (big) return dispatch_p2<CfgMain>(a, mode, out, accum, fuseq, st, p2);
  return dispatch_p2<CfgSmall>(a, mode, out, accum, fuseq, st, p2);
}

// ---------------------------------------------------------------------------
// Small-M forward (rollout decode, M <= 128): Y = Xq . Wq^T streams the whole
// weight once for a handful of rows, so it is bound by HBM bandwidth and needs
// many weight bytes in flight.  The output is cut into 64*WS-column blocks,
// the K steps into S contiguous ranges and (with one range) the rows into
// groups of MT*16; a workgroup (4 wavefronts) computes the FP32 sum of one
// (block, range, row group) through an NST-stage ring of direct
// global->LDS loads, KS K steps per stage ((NST-1)*KS steps of prefetch).
// With S = 1 it writes Y (BF16 or FP32) and, for BF16, the fused 1x128
// quantization of Y itself.  With S > 1 it writes its partial sum to the
// caller's workspace P[S][M][N] and k_skinny_finish sums the S partials in
// order s = 0..S-1 (deterministic) and writes the same outputs.  (Finishing inside the split kernel, the last
// workgroup of a column block summing the others' partials, measured slower:
// the partials then have to cross the XCDs' separate L2 caches through memory,
// three dependent memory round trips at the end of every workgroup, where the
// second kernel reads them from L2 after one kernel boundary.)  Per 128-K step
// the numerics are those of the main kernel: one MFMA per 16x16 sub-tile from
// zero, folded into FP32 with the product of the row scale and the weight
// block scale.
//
// Stage layout: the X tile (MT*16 rows x 128 bytes, swizzled rows), the W
// tile (64 rows x 128 bytes), then four 256-byte scale slots, one DMA per
// wavefront: slots q < ceil(MT/4) hold X row scales (float 4r + t of slot q
// is row (4q + t)*16 + r, so lane r reads its rows i*16 + r, i < MT, as
// ceil(MT/4) 16-byte loads); the other slots hold 64 copies of the W block
// scale.
// Wavefront w multiplies W slab w (output columns 16w..16w+15 of the block)
// with the MT X slabs.
template <int MT, int NST, int WS, int KS>
struct SkinnyCfg {
  static constexpr int BN = 64 * WS;                   // output columns per workgroup
  static constexpr int XT = MT * 16 * 128, WT = BN * 128;
  static constexpr int SUB = XT + WT + 1024;           // one K step: X tile, W tile, scale slots
  static constexpr int STAGE = KS * SUB;               // KS consecutive K steps per ring stage
  static constexpr int XBLK = XT / 1024, WBLK = WT / 1024;
  static constexpr int BPW = (XBLK + WBLK + 3) / 4;    // tile DMAs per wavefront and K step (slots
                                                       // past the last block repeat it)
  static constexpr int NSX = (MT + 3) / 4;             // scale slots holding X row scales
  static constexpr int LOADS = KS * (BPW + 1);         // DMAs per wavefront and stage
  static constexpr int LDS = NST * STAGE;
  static constexpr int TP = BN + 4;                    // FP32 output tile pitch (floats)
  static_assert(NSX >= 1 && NSX < 4, "scale slots");
  static_assert(BN == 128 || BN == 64, "one weight block scale per workgroup");
  static_assert(MT * 16 * TP * 4 <= LDS, "output tile fits the stage ring");
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <int MT, int NST, int WS, int KS, int OUT, bool FUSEQ, bool P2 = false>
__global__ __launch_bounds__(256) void k_gemm_fp8_skinny(GemmArgs p, float* __restrict__ part,
                                                         int splits) {
  using C = SkinnyCfg<MT, NST, WS, KS>;
  static_assert(C::BN == 128 || !FUSEQ, "the fused 1x128 output needs whole 128-column groups");
  __shared__ __attribute__((aligned(16))) uint8_t lds[C::LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 15, kg = lane >> 4;
  const int n0 = blockIdx.x * C::BN;
  // Row group blockIdx.z: rows MT*16*z .. of X and of the outputs (one K
  // range only; a split launch has a single row group).
  if (blockIdx.z > 0) {
    const int row0 = (int)blockIdx.z * MT * 16;
    if (row0 >= p.M) return;
    p.A += (int64_t)row0 * p.lda;
    p.sA += row0;
    p.C = static_cast<uint8_t*>(p.C) + (int64_t)row0 * p.ldc * (OUT == kOutF32 ? 4 : 2);
    if (FUSEQ) {
      p.Cq += (int64_t)row0 * p.ldc;
      p.Cs += row0;
    }
    p.M -= row0;
  }
  if (p.M > MT * 16) p.M = MT * 16;
  const int sidx = blockIdx.y;
  const int KB = p.Kc / 128;
  const int kb0 = (int)((int64_t)KB * sidx / splits), kb1 = (int)((int64_t)KB * (sidx + 1) / splits);
  const int nsteps = kb1 - kb0;
  const uint32_t lds0 = lds_addr(lds);
  // 64-bit bases at the block's first weight row and weight-block scale row
  // (32-bit per-lane offsets: at most 128 rows times the row stride)
  p.B += (int64_t)n0 * p.ldb;
  p.sB += (int64_t)(n0 / 128) * p.sB_o;

  // this wavefront's DMA blocks: global blocks wave*BPW .. ; X blocks first, then W
  uint32_t off[C::BPW], dst[C::BPW];
  bool isx[C::BPW];
#pragma unroll
  for (int t = 0; t < C::BPW; ++t) {
    // a repeated block writes the same bytes to the same LDS slot again
    const int gb = min(wave * C::BPW + t, C::XBLK + C::WBLK - 1);
    int row; uint32_t col;
    if (gb < C::XBLK) {
      dma_src<false>(gb, lane, row, col);
      off[t] = (uint32_t)min(row, p.M - 1) * (uint32_t)p.lda + col;
      dst[t] = (uint32_t)(gb * 1024);
      isx[t] = true;
    } else {
      dma_src<false>(gb - C::XBLK, lane, row, col);
      off[t] = (uint32_t)row * (uint32_t)p.ldb + col;
      dst[t] = (uint32_t)(C::XT + (gb - C::XBLK) * 1024);
      isx[t] = false;
    }
  }
  uint32_t soff;   // the wavefront's scale DMA
  if (wave < C::NSX) {
    // slot 64q + 4r + t (q = wave, r = lane/4, t = lane%4) holds row (4q + t)*16 + r
    const int row = (4 * wave + (lane & 3)) * 16 + (lane >> 2);
    soff = (uint32_t)min(row, p.M - 1) * 4u;
  } else {
    soff = 0u;
  }
  const uint32_t sdst = (uint32_t)(C::XT + C::WT + 256 * wave);

  // Stage `stage` holds K steps kb .. kb+KS-1 of the range (a step past the
  // range's end loads its last step again and is not computed).  The KS
  // steps' blocks of the same rows are issued back to back, so each weight
  // row is requested KS*128 contiguous bytes at a time.
  auto issue = [&](int stage, int kb) __attribute__((always_inline)) {
    const uint32_t sb = lds0 + (uint32_t)(stage * C::STAGE);
#pragma unroll
    for (int t = 0; t < C::BPW; ++t)
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const int kk = min(kb + u, kb1 - 1);
        dma16(sb + (uint32_t)(u * C::SUB) + dst[t], (isx[t] ? p.A : p.B) + (int64_t)kk * 128, off[t]);
      }
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      const int kk = min(kb + u, kb1 - 1);
      const uint32_t sd = sb + (uint32_t)(u * C::SUB) + sdst;
      if (wave < C::NSX) dma4(sd, p.sA + (int64_t)kk * p.sA_ld, soff);
      else dma4(sd, p.sB + (int64_t)kk * p.sB_c, soff);
    }
  };

  constexpr int D = NST - 1;
  const int nstages = (nsteps + KS - 1) / KS;
#pragma unroll
  for (int s = 0; s < D; ++s)
    if (s < nstages) issue(s, kb0 + s * KS);

  v4f acc[WS][MT];
#pragma unroll
  for (int j = 0; j < WS; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  int st = 0;
  for (int k = 0; k < nstages; ++k) {
    // this wavefront's loads of stage k have landed once at most those of the
    // (up to D-1) later stages already issued are outstanding
    const int later = min(nstages - 1 - k, D - 1);
    if (later >= D - 1) wait_vmem<C::LOADS * (D - 1)>();
    else wait_vmem<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the stage stage k-1 used is free: refill it with stage k + D
    if (k + D < nstages) issue((st + D) % NST, kb0 + (k + D) * KS);
#pragma unroll
    for (int u = 0; u < KS; ++u) {
    if (u > 0 && k * KS + u >= nsteps) break;
    const uint8_t* Xs = lds + st * C::STAGE + u * C::SUB;
    const uint8_t* Ws = Xs + C::XT;
    const float* Sc = reinterpret_cast<const float*>(Xs + C::XT + C::WT);
    float sx[MT];
    if constexpr (MT >= 4) {
#pragma unroll
      for (int q = 0; q < MT / 4; ++q) {
        const float4 r4 = *reinterpret_cast<const float4*>(Sc + 64 * q + 4 * lrow);
        sx[4 * q] = r4.x; sx[4 * q + 1] = r4.y; sx[4 * q + 2] = r4.z; sx[4 * q + 3] = r4.w;
      }
    } else {
      // slot 0 holds rows t*16 + lrow at 4*lrow + t; rows past MT*16 are unused
      const float4 r4 = *reinterpret_cast<const float4*>(Sc + 4 * lrow);
      sx[0] = r4.x;
      if constexpr (MT > 1) sx[1] = r4.y;
    }
    const float swb = Sc[64 * C::NSX + lane];
    if constexpr (P2) {
      // power-of-two scales as the MFMA's E8M0 operand scales, accumulated in
      // place: per element the same MFMA chain as k_gemm_fp8<..., P2>
      int ea[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) ea[i] = e8m0_of(sx[i]);
      const int eb = e8m0_of(swb);
#pragma unroll
      for (int j = 0; j < WS; ++j) {
        const v8i bfr = frag32<false>(Ws, wave * WS + j, lane);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[j][i] = mfma_fp8_e8m0(bfr, frag32<false>(Xs, i, lane), acc[j][i], eb, ea[i]);
      }
      continue;
    }
#pragma unroll
    for (int j = 0; j < WS; ++j) {
      const v8i bfr = frag32<false>(Ws, wave * WS + j, lane);
      v4f pr[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) pr[i] = mfma_fp8(bfr, frag32<false>(Xs, i, lane));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const float c = sx[i] * swb;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][i][r] = fmaf(pr[i][r], c, acc[j][i][r]);
      }
    }
    }
    st = (st + 1 == NST) ? 0 : st + 1;
  }
  wait_vmem<0>();

  if (splits > 1) {
    // partial sums: lane holds row i*16 + lrow, columns n0 + 16*(wave*WS + j) + 4*kg + r
    float* P = part + (int64_t)sidx * p.M * p.N;
#pragma unroll
    for (int j = 0; j < WS; ++j) {
      const int n = n0 + 16 * (wave * WS + j) + 4 * kg;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = i * 16 + lrow;
        if (m < p.M)
          *reinterpret_cast<float4*>(P + (int64_t)m * p.N + n) =
              make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
      }
    }
    return;
  }

  // ---- S = 1: the block's FP32 values into an LDS tile T[MT*16][TP], then
  // the outputs.  Lane element (j, i, r) is row i*16 + lrow, column
  // 16*(wave*WS + j) + 4*kg + r. ----
  float* T = reinterpret_cast<float*>(lds);
  __syncthreads();   // every wavefront is done with the stage ring
#pragma unroll
  for (int j = 0; j < WS; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i)
      *reinterpret_cast<float4*>(T + (i * 16 + lrow) * C::TP + 16 * (wave * WS + j) + 4 * kg) =
          make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
  __syncthreads();

  // ---- outputs: 16 rows per pass, a DPP row of 16 lanes per row (8 columns
  // per lane, one 1x128 group per row) ----
  constexpr int LPR = C::BN / 8;                    // lanes per output row (8 columns each)
  const int c = tid % LPR;
  const int n = n0 + 8 * c;
  for (int m0r = 0; m0r < p.M; m0r += 256 / LPR) {
    const int m = m0r + tid / LPR;
    const bool ok = m < p.M;
    const float* src = T + (ok ? m : p.M - 1) * C::TP + 8 * c;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    if (OUT == kOutF32) {
      if (ok) {
        float* Cf = static_cast<float*>(p.C) + (int64_t)m * p.ldc + n;
        *reinterpret_cast<float4*>(Cf) = a;
        *reinterpret_cast<float4*>(Cf + 4) = b;
      }
      continue;
    }
    uint4 w;
    w.x = bf16x2_rne(a.x, a.y);
    w.y = bf16x2_rne(a.z, a.w);
    w.z = bf16x2_rne(b.x, b.y);
    w.w = bf16x2_rne(b.z, b.w);
    if (FUSEQ) {
      // 1x128 quantization of the BF16 output, as in the main kernel's epilogue
      uint32_t am = max_abs_bf16x2(0u, w.x);
      am = max_abs_bf16x2(am, w.y);
      am = max_abs_bf16x2(am, w.z);
      am = max_abs_bf16x2(am, w.w);
      am = row16_max_u16x2(am);
      const ScalePair sp = scale_rule<P2>(fold_bf16x2(am));
      const uint32_t q0 = e4m3x4(bf16_lo(w.x) * sp.r, bf16_hi(w.x) * sp.r, bf16_lo(w.y) * sp.r, bf16_hi(w.y) * sp.r);
      const uint32_t q1 = e4m3x4(bf16_lo(w.z) * sp.r, bf16_hi(w.z) * sp.r, bf16_lo(w.w) * sp.r, bf16_hi(w.w) * sp.r);
      if (ok) {
        *reinterpret_cast<uint2*>(p.Cq + (int64_t)m * p.ldc + n) = make_uint2(q0, q1);
        if (c == 0) p.Cs[(int64_t)(n / 128) * p.ldcs + m] = sp.s;
      }
    }
    if (ok) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n) = w;
  }
}

// Sum of the S partials, then the output: 16 rows x 128 columns per block, a
// DPP row of 16 lanes per row (8 columns per lane, one 1x128 group per row).
template <int OUT, bool FUSEQ>
__global__ __launch_bounds__(256) void k_skinny_finish(GemmArgs p, const float* __restrict__ part,
                                                       int splits) {
  const int c = threadIdx.x & 15;
  const int m = blockIdx.y * 16 + (threadIdx.x >> 4);
  const int n = blockIdx.x * 128 + 8 * c;
  const bool ok = m < p.M;
  const int mm = ok ? m : p.M - 1;
  float v[8];
  {
    const float* src = part + (int64_t)mm * p.N + n;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  for (int s = 1; s < splits; ++s) {
    const float* src = part + ((int64_t)s * p.M + mm) * p.N + n;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w; v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  if (OUT == kOutF32) {
    if (ok) {
      float* Cf = static_cast<float*>(p.C) + (int64_t)m * p.ldc + n;
      *reinterpret_cast<float4*>(Cf) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(Cf + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    return;
  }
  uint4 w;
  w.x = bf16x2_rne(v[0], v[1]);
  w.y = bf16x2_rne(v[2], v[3]);
  w.z = bf16x2_rne(v[4], v[5]);
  w.w = bf16x2_rne(v[6], v[7]);
  if (FUSEQ) {
    // 1x128 quantization of the BF16 output, as in the main kernel's epilogue
    uint32_t am = max_abs_bf16x2(0u, w.x);
    am = max_abs_bf16x2(am, w.y);
    am = max_abs_bf16x2(am, w.z);
    am = max_abs_bf16x2(am, w.w);
    am = row16_max_u16x2(am);
    const ScalePair sp = scale_pair(fold_bf16x2(am));
    const uint32_t q0 = e4m3x4(bf16_lo(w.x) * sp.r, bf16_hi(w.x) * sp.r, bf16_lo(w.y) * sp.r, bf16_hi(w.y) * sp.r);
    const uint32_t q1 = e4m3x4(bf16_lo(w.z) * sp.r, bf16_hi(w.z) * sp.r, bf16_lo(w.w) * sp.r, bf16_hi(w.w) * sp.r);
    if (ok) {
      *reinterpret_cast<uint2*>(p.Cq + (int64_t)m * p.ldc + n) = make_uint2(q0, q1);
      if (c == 0) p.Cs[(int64_t)(n / 128) * p.ldcs + m] = sp.s;
    }
  }
  if (ok) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.C) + (int64_t)m * p.ldc + n) = w;
}

// Small-M configuration.  One workgroup of this kernel streams its weight
// columns at about 35 GB/s (measured with weights cycled past the 256 MB
// MALL), so HBM bandwidth needs every CU streaming: the K steps are split
// into as many ranges as fit one wave of at most kSkFill workgroups (a
// second, partial wave of workgroups measured slower: Llama-8B decode
// QKV 6 ranges / 288 workgroups 19.1 us against 5 / 240 at 13.9 us).
constexpr int kSkWS = 2;        // W slabs per wavefront: 128 output columns per workgroup
// Ring stages of the 64-row workgroups (M <= 64; 4 for M <= 128): with every
// CU streaming, three stages (two in flight, 48 KB of weights per CU) are
// enough and deeper rings only lengthen the memory queues (Llama-8B decode
// step, weights cycled past the MALL: 2 / 3 / 4 / 6 stages 84.5 / 72.1 /
// 73.5 / 80.8 us).
constexpr int kSkNST64 = 3;
// Two K steps per ring stage, i.e. 256 contiguous bytes of each weight row
// requested at a time, only pay off for the 16-row groups: Llama-8B decode
// with one K range, down projection 14336 -> 4096 in 64-column blocks,
// 35.1 -> 33.0 us (3 stages of 2 steps against 6 of 1; 5 of 1: 34.7 us),
// while for the 64-row gate+up workgroups they cost 32.7 -> 35.0 us.
constexpr int kSkKS64 = 1;      // K steps per ring stage of the 64-row workgroups
constexpr int kSkKS16 = 2;      // ... of the 16-row groups
constexpr int kSkNST = 3;       // ring stages of the 16-row groups (one K range, few column blocks)
constexpr int kSkFill = 256;    // workgroups of one wave on MI355X (one per CU: the ring fills LDS)
constexpr int kSkRowSplitBlocks = 64;   // one K range below this many column blocks: 16-row groups
constexpr int kSkLongK = 64;            // ... of 64 columns from this many K steps on

// K-step ranges of the small-M forward: floor(kSkFill / column blocks), at
// least one K step per range, at most 16 ranges.
int skinny_splits(int64_t M, int64_t N, int64_t K) {
  (void)M;
  const int64_t blocks = N / (64 * kSkWS), kb = K / 128;
  int64_t s = blocks > 0 ? kSkFill / blocks : 1;
  if (s > 16) s = 16;
  if (s > kb) s = kb;
  return (int)(s < 1 ? 1 : s);
}

// Workspace: the S partial sums (S*M*N floats); none when the K steps are not split.
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || M > kSkinnyMaxM || N <= 0 || K <= 0) return 0;
  const int S = skinny_splits(M, N, K);
  return S == 1 ? 0 : (size_t)S * (size_t)M * (size_t)N * sizeof(float);
}

template <int MT, int NST, int WS, int KS, int OUT, bool FUSEQ, bool P2 = false>
static hipError_t launch_skinny_mt(const GemmArgs& a, float* part, int S, hipStream_t st) {
  if (P2 && S != 1) return hipErrorInvalidValue;   // the power-of-two path runs one K range
  // row groups of MT*16 rows (a split launch covers all rows in one group)
  const int R = (a.M + MT * 16 - 1) / (MT * 16);
  if (S > 1 && R != 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm_fp8_skinny<MT, NST, WS, KS, OUT, FUSEQ, P2>),
                     dim3((unsigned)(a.N / (64 * WS)), (unsigned)S, (unsigned)R), dim3(256), 0, st, a,
                     part, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const dim3 g((unsigned)(a.N / 128), (unsigned)((a.M + 15) / 16));
  hipLaunchKernelGGL((k_skinny_finish<OUT, FUSEQ>), g, dim3(256), 0, st, a, part, S);
  return hipGetLastError();
}

// One K range, 16-row groups, 64-column blocks: twice the workgroups of
// 128-column blocks, each streaming half the weight column, for long
// contractions (at least kSkLongK K steps), where the stream dominates.  A
// fused 1x128 output then comes from the 1x128 quantizer run on the BF16 Y,
// which is the fused epilogue's definition, so the bits are the same.
// (Llama-8B decode, one K range, down projection 14336 -> 4096: 42.6 ->
// 35.8 us; for QKV and O, 32 K steps, the extra launch costs more: 15.1 ->
// 18.8 us.)
template <bool P2>
static hipError_t launch_skinny_rows16_64(const GemmArgs& a, int out, bool fuseq, hipStream_t st) {
  const dim3 g((unsigned)(a.N / 64), 1u, (unsigned)((a.M + 15) / 16));
  if (out == kOutF32) {
    hipLaunchKernelGGL((k_gemm_fp8_skinny<1, kSkNST, 1, kSkKS16, kOutF32, false, P2>), g, dim3(256), 0, st, a, nullptr, 1);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_fp8_skinny<1, kSkNST, 1, kSkKS16, kOutBf16, false, P2>), g, dim3(256), 0, st, a, nullptr, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !fuseq) return e;
  return launch_quant_1x128(static_cast<const uint16_t*>(a.C), a.M, a.N, a.ldc, a.Cq, a.ldc, a.Cs, st, P2);
}

template <int MT, int NST, int KS, bool P2 = false>
static hipError_t launch_skinny_out(const GemmArgs& a, int out, bool fuseq, float* part, int S,
                                    hipStream_t st) {
  if (out == kOutF32) return launch_skinny_mt<MT, NST, kSkWS, KS, kOutF32, false, P2>(a, part, S, st);
  if (fuseq) return launch_skinny_mt<MT, NST, kSkWS, KS, kOutBf16, true, P2>(a, part, S, st);
  return launch_skinny_mt<MT, NST, kSkWS, KS, kOutBf16, false, P2>(a, part, S, st);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int out, bool fuseq, void* workspace, hipStream_t st,
                              bool unsplit, bool p2) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.M > kSkinnyMaxM || a.Kc <= 0 || a.N % (64 * kSkWS)) return hipErrorInvalidValue;
  // One K range with few column blocks: each 16-row slab of X is a
  // workgroup of its own.  A workgroup's rate of streaming its weight
  // column is bound by its step (fewer rows, less work per step) and more
  // of them run at once; the workgroups of one column block share an XCD
  // (the block index differs by multiples of the column-block count, a
  // multiple of 8 on every Llama/Qwen shape), so its weight bytes come from
  // that XCD's L2 after the first.  A row's MFMA operands, lanes and chain
  // are those of the 64-row workgroup, so its outputs are the same bits.
  const bool rows16 = a.N / (64 * kSkWS) < kSkRowSplitBlocks;
  if (p2) {   // one K range: the chain of k_gemm_fp8<..., P2> (no workspace)
    if (rows16 && a.Kc / 128 >= kSkLongK) return launch_skinny_rows16_64<true>(a, out, fuseq, st);
    if (rows16) return launch_skinny_out<1, kSkNST, kSkKS16, true>(a, out, fuseq, nullptr, 1, st);
    if (a.M <= 64) return launch_skinny_out<4, kSkNST64, kSkKS64, true>(a, out, fuseq, nullptr, 1, st);
    return launch_skinny_out<8, 4, 1, true>(a, out, fuseq, nullptr, 1, st);
  }
  // unsplit: every output element is the same chain of per-step FMAs, in K
  // order, as in k_gemm_fp8 (bit-identical to the large-M forward)
  const int S = unsplit ? 1 : skinny_splits(a.M, a.N, a.Kc);
  if (S > 1 && workspace == nullptr) return hipErrorInvalidValue;
  float* part = static_cast<float*>(workspace);
  if (S == 1 && rows16 && a.Kc / 128 >= kSkLongK) return launch_skinny_rows16_64<false>(a, out, fuseq, st);
  if (S == 1 && rows16) return launch_skinny_out<1, kSkNST, kSkKS16>(a, out, fuseq, part, 1, st);
  if (a.M <= 64) return launch_skinny_out<4, kSkNST64, kSkKS64>(a, out, fuseq, part, S, st);
  return launch_skinny_out<8, 4, 1>(a, out, fuseq, part, S, st);
}

// Grouped GEMMs use the 256 x 256 tile too: measured on the Qwen3-30B-A3B
// expert layers (128 experts, segments of 72..7380 rows) it is 3-10 % faster
// than the 128 x 128 tile despite the larger ragged remainder per segment.
hipError_t launch_gemm_grouped(const GemmArgs& a, int grp, int mode, int out, bool accum,
                               bool fuseq, hipStream_t st, bool p2) {
  if (a.N == 0 || a.E == 0) return hipSuccess;
  if (grp == kGrpRows) {
    if (a.seg_rows == 0) return hipSuccess;
    if (mode != kRowBlock || accum) return hipErrorInvalidValue;
    if (p2) return dispatch<CfgMain, kGrpRows, true>(a, mode, out, false, fuseq, st);
    return dispatch<CfgMain, kGrpRows>(a, mode, out, false, fuseq, st);
  }
  if (grp == kGrpContraction) {
    if (a.M == 0 || mode != kRowCol || fuseq) return hipErrorInvalidValue;
    if (p2) return dispatch<CfgMain, kGrpContraction, true>(a, mode, out, accum, false, st);
    return dispatch<CfgMain, kGrpContraction>(a, mode, out, accum, false, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace jet

#if JET_PHASE_TIMING
extern "C" int jet_phase_buffers(void** records, void** flag, int* capacity) {
  if (!records || !flag || !capacity) return 1;
  if (hipGetSymbolAddress(records, HIP_SYMBOL(jet::g_phase)) != hipSuccess) return 2;
  if (hipGetSymbolAddress(flag, HIP_SYMBOL(jet::g_phase_on)) != hipSuccess) return 2;
  *capacity = jet::kPhaseBlocks;
  return 0;
}
#endif
