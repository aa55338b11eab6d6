// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Arguments are validated by the caller; these functions only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jet {

enum { kRowBlock = 0, kRowCol = 1 };   // scale modes of the GEMM
enum { kOutBf16 = 0, kOutF32 = 1 };    // GEMM output element types

enum { kGrpNone = 0, kGrpRows = 1, kGrpContraction = 2 };   // grouped (per-expert) modes

// C[M, N] (+)= sum_kb scale * A[M, Kc-slab] . B[N, Kc-slab]^T ; see gemm.hip.
struct GemmArgs {
  const uint8_t* A;      // [M, Kc] E4M3, row stride lda bytes
  const uint8_t* B;      // [N, Kc] E4M3, row stride ldb bytes
  const float* sA;       // row scales: sA[kb * sA_ld + m]
  const float* sB;       // ROWBLOCK: sB[(n/128) * sB_o + kb * sB_c]; ROWCOL: sB[kb * sB_c + n]
  void* C;               // [M, N] output, row stride ldc elements
  uint8_t* Cq;           // fused 1x128 quantization of a BF16 C (or null)
  float* Cs;             //   and its scales: Cs[(n/128) * ldcs + m]
  int64_t lda, ldb, sA_ld, sB_o, sB_c, ldc, ldcs;
  int M, N, Kc;
  // Grouped problems (mixture of experts); unused by the dense GEMMs.
  //   kGrpRows:        the rows of A and C are cut into segments seg[e] .. seg[e+1]-1,
  //                    segment e multiplies expert e's B (B + e*bE, sB + e*sbE).
  //   kGrpContraction: expert e contracts over the 128-padded column range of
  //                    segment e (columns below kcap) and writes C + e*cE.
  const int32_t* seg;
  int E, seg_rows;       // experts; rows the segment offsets index (clamp bound)
  int64_t bE, sbE, cE;
  int kcap;
};

// p2: power-of-two scales (scale_pair_pow2) instead of amax / 448.
hipError_t launch_quant_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                              int64_t ldq, float* s, hipStream_t st, bool p2 = false);
hipError_t launch_quant_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                float* s, uint8_t* qT, hipStream_t st, bool p2 = false);
hipError_t launch_quant_128x1_T(const void* src, bool fp8src, const float* src_s, int64_t M,
                                int64_t K, int64_t ldsrc, uint8_t* qT, int64_t ldqT, float* sT,
                                hipStream_t st, bool p2 = false);
// 1x128 (q, s) and 128x1 transposed (qT, sT) of one BF16 activation in one read;
// requant: the 128x1 groups quantize the dequantized 1x128 values.
hipError_t launch_quant_1x128_128x1_T(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      uint8_t* q, int64_t ldq, float* s, uint8_t* qT,
                                      int64_t ldqT, float* sT, bool requant, hipStream_t st,
                                      bool p2 = false);
// Fused producers of the 1x128 input: RMSNorm (H <= 8192) and SwiGLU; y / h
// (the BF16 tensor) may be null.
hipError_t launch_rmsnorm_quant_1x128(const uint16_t* x, const uint16_t* gamma, int64_t M, int64_t H,
                                      int64_t ldx, float eps, uint16_t* y, int64_t ldy, uint8_t* q,
                                      int64_t ldq, float* s, hipStream_t st, bool p2 = false);
hipError_t launch_swiglu_quant_1x128(const uint16_t* gu, int64_t M, int64_t I, int64_t ldgu, uint16_t* h,
                                     int64_t ldh, uint8_t* q, int64_t ldq, float* s, hipStream_t st, bool p2 = false);
// FP8 KV cache: per-tensor scales (scales[0..3] = s_k, r_k, s_v, r_v; scales[4..5]
// the two amax words) and the quantize-and-append of token rows to cache rows.
hipError_t launch_kv_calibrate(const uint16_t* k, const uint16_t* v, int64_t T, int64_t D, int64_t ldk,
                               int64_t ldv, float* scales, hipStream_t st);
hipError_t launch_kv_append(const uint16_t* k, const uint16_t* v, int64_t T, int64_t D, int64_t ldk,
                            int64_t ldv, const int64_t* slots, const float* scales, uint8_t* kc, uint8_t* vc,
                            int64_t ldc, int64_t rows, hipStream_t st);
// p2: every scale is a power of two and is applied by the MFMA itself (E8M0
// operand scales), accumulating across K steps inside the MFMA; the fused
// 1x128 quantization of the output then uses power-of-two scales too.
hipError_t launch_gemm(const GemmArgs& a, int mode, int out, bool accum, bool fuseq,
                       hipStream_t st, bool p2 = false);
// Small-M forward (M <= kSkinnyMaxM): one kernel when the K steps are not
// split; otherwise split-K partial sums in the caller's workspace
// (skinny_workspace_bytes) and a deterministic finishing pass.
constexpr int64_t kSkinnyMaxM = 128;
int skinny_splits(int64_t M, int64_t N, int64_t K);
size_t skinny_workspace_bytes(int64_t M, int64_t N, int64_t K);
// unsplit: one K range (no workspace), bit-identical to launch_gemm's forward.
// p2: power-of-two scales applied by the MFMA, one K range (bit-identical to
// launch_gemm's p2 forward).
hipError_t launch_gemm_skinny(const GemmArgs& a, int out, bool fuseq, void* workspace, hipStream_t st,
                              bool unsplit = false, bool p2 = false);
// Grouped GEMMs: grp = kGrpRows (forward, dgrad) or kGrpContraction (wgrad).
hipError_t launch_gemm_grouped(const GemmArgs& a, int grp, int mode, int out, bool accum,
                               bool fuseq, hipStream_t st, bool p2 = false);
hipError_t launch_quant_128x1_T_grouped(const void* src, bool fp8src, const float* src_s,
                                        int64_t M, int64_t K, int64_t ldsrc, const int32_t* seg,
                                        int E, uint8_t* qT, int64_t ldqT, float* sT,
                                        hipStream_t st, bool p2 = false);

}  // namespace jet
