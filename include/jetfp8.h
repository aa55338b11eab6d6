/*
 * jetfp8.h -- C ABI of the MI355X (gfx950) unified-precision FP8 linear layer.
 *
 * The method (Jet-RL, "Jet-RL: Enabling On-Policy FP8 Reinforcement Learning
 * with Unified Training and Rollout Precision Flow", gist.science explainer,
 * section "Quantisierungsschema"; and the quantization table of
 * "NVIDIA强化学习加速实操：10分钟提升2倍训练效率", section
 * "为什么FP8适配线性层？") runs every linear layer in FP8 E4M3 with FP32
 * scales: activations and output gradients in 1x128 groups, weights in
 * 128x128 blocks, and a 128x1 grouping for the weight gradient.  The same
 * quantizers and forward GEMM serve rollout and training.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers on the current HIP device, owned by the
 *    caller.  The library never allocates, frees or retains device memory and
 *    keeps no pointer after a call returns.  `stream` is a hipStream_t
 *    (NULL = the null stream).
 *  - Every call only enqueues work on `stream` and returns; it never
 *    synchronizes.  Device faults surface at the caller's next sync.
 *  - Arguments are validated before anything is launched.  On failure a
 *    non-zero jet_status is returned, nothing is launched and no output is
 *    touched; jet_last_error() gives a thread-local description.
 *  - E4M3 is the OCP 8-bit format E4M3 (bias 7, subnormals, max +-448, no
 *    infinities).  Encoding rounds to nearest (ties to even) and saturates at
 *    +-448; the sign of zero is kept.
 *  - Scale of a group with maximum magnitude amax:
 *        amax_c = max(amax, 2^-96),  s = fl32(amax_c / 448),
 *        code   = E4M3(fl32(x * fl32(448 / amax_c))).
 *    s is the stored (dequantisation) scale: value ~= E4M3value(code) * s.
 *  - Inputs must be finite.  Outputs must not alias inputs.
 *  - BF16 is bfloat16 (raw 16-bit storage); outputs rounded to BF16 use
 *    round-to-nearest-even from the FP32 accumulator.
 *  - Identical inputs give bit-identical outputs (no atomics in reductions).
 *  - The library keeps no global mutable state other than the thread-local
 *    error string, and, for jet_fp8_linear_fwd_noalloc only, its static
 *    device scratch and the per-device table of that scratch's address
 *    (filled once under a lock); calls from several host threads are safe,
 *    except overlapping jet_fp8_linear_fwd_noalloc calls on one GPU.
 */
#ifndef JETFP8_H
#define JETFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define JET_ABI_VERSION 10

typedef enum {
  JET_OK = 0,
  JET_ERR_NULL = 1,      /* a required pointer is NULL                          */
  JET_ERR_SHAPE = 2,     /* a size is negative, or not a multiple of 128 where  */
                         /* required, or a leading dimension is too small       */
  JET_ERR_ALIGN = 3,     /* a pointer or leading dimension breaks alignment     */
  JET_ERR_DTYPE = 4,     /* unsupported dtype code                              */
  JET_ERR_WORKSPACE = 5, /* workspace smaller than jet_workspace_bytes()        */
  JET_ERR_HIP = 6        /* a HIP launch or query failed (see jet_last_error)   */
} jet_status;

typedef enum { JET_BF16 = 1, JET_F32 = 2, JET_E4M3 = 3 } jet_dtype;

typedef enum { JET_OP_FWD = 0, JET_OP_DGRAD = 1, JET_OP_WGRAD = 2 } jet_op;

/* ABI version of the loaded library (JET_ABI_VERSION). */
int jet_abi_version(void);
/* Static name of a jet_status code. */
const char* jet_status_string(int status);
/* Thread-local text of the last failure on this host thread ("" if none). */
const char* jet_last_error(void);

/*
 * 1x128 group quantization of an activation or output gradient.
 * Gist.science explainer, "Quantisierungsschema" (activations 1x128);
 * nmedialink table (input activations and output gradients, [1,128], FP32).
 *
 *   x  : BF16 [M, K], row stride ldx elements (ldx >= K, ldx % 8 == 0)
 *   q  : E4M3 [M, K], row stride ldq bytes   (ldq >= K, ldq % 16 == 0)
 *   s  : FP32 [K/128, M]; the scale of row m, columns 128j..128j+127 is s[j*M+m]
 *   M >= 0, K % 128 == 0.  x 16-byte aligned, q 16-byte aligned, s 4-byte aligned.
 */
int jet_quant_act_1x128(const void* x, int64_t M, int64_t K, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* s, void* stream);

/*
 * 128x1 group quantization along the row (token) axis, written transposed, for
 * the weight-gradient GEMM.  Explainer "Quantisierungsschema" (128x1 for WGrad);
 * 163.com write-up section 五 (1x128 activations re-quantized as 128x1).
 *
 *   src_dtype == JET_BF16: src is BF16 [M, K] (row stride ldsrc elements), src_s NULL.
 *   src_dtype == JET_E4M3: src is the E4M3 [M, K] output of jet_quant_act_1x128
 *       (row stride ldsrc bytes) and src_s its scales [K/128, M]; the values
 *       re-quantized are fl32(E4M3value(code) * scale).
 *   qT : E4M3 [K, Mp] with Mp = ceil(M/128)*128, row stride ldqT bytes
 *        (ldqT >= Mp, ldqT % 16 == 0); columns M..Mp-1 receive zero codes.
 *   sT : FP32 [ceil(M/128), K]; scale of rows 128g..min(128g+127, M-1) of
 *        column k is sT[g*K + k].  A partial last group uses its valid rows only.
 *   M >= 0, K % 128 == 0.  ldsrc % 16 bytes, src and qT 16-byte aligned.
 */
int jet_quant_act_128x1_T(const void* src, int src_dtype, const float* src_s,
                          int64_t M, int64_t K, int64_t ldsrc,
                          uint8_t* qT, int64_t ldqT, float* sT, void* stream);

/*
 * FP8 KV cache of the rollout, step 1: recalibrate the scales after a weight
 * update (66260.cn FP8-RL item, KV-cache paragraph: KV-cache scale factors
 * calibrated dynamically and re-adjusted after each model update; nmedialink
 * NeMo-RL repost: FP8 in the KV cache).  One FP32 scale per tensor (the
 * pages give no granularity): from the K and V rows of a calibration batch,
 *   amax_c = max(max|x|, 2^-96), s = amax_c / 448, r = 448 / amax_c
 * (the quantizers' scale rule).
 *
 *   k, v      : BF16 [T, D] (D = KV heads x head dim), row strides ldk, ldv
 *               elements (>= D, % 8) -- e.g. column slices of the QKV output
 *   kv_scales : FP32 device array of 6: [0] s_k, [1] r_k, [2] s_v, [3] r_v
 *               (s dequantizes, r quantizes); [4], [5] working space
 *   T >= 0 (T == 0: the floor scale), D > 0, D % 8 == 0; k, v 16-byte aligned,
 *   kv_scales 4-byte aligned.  Two kernel launches, no memset; during the
 *   call kv_scales[0] also counts the workgroups that have finished.
 */
int jet_kv_calibrate(const void* k, const void* v, int64_t T, int64_t D,
                     int64_t ldk, int64_t ldv, float* kv_scales, void* stream);

/*
 * FP8 KV cache, step 2: quantize T new tokens' K and V rows with the stored
 * multipliers (codes = E4M3 of x * r, round to nearest even, saturating at
 * +-448: values beyond the calibration batch's range saturate) and write
 * them to the cache rows named by slots (a paged cache's block * block_size +
 * offset).
 *
 *   k, v, T, D, ldk, ldv : as jet_kv_calibrate
 *   slots     : int64 device array [T]; a slot outside [0, rows) writes nothing
 *               (-1 marks a padding token)
 *   kv_scales : as written by jet_kv_calibrate
 *   k_cache, v_cache : E4M3 [rows, D], row stride ldc bytes (ldc >= D, % 8)
 *   slots and caches 8-byte aligned.  Rows not named by a slot are unchanged.
 */
int jet_kv_append(const void* k, const void* v, int64_t T, int64_t D,
                  int64_t ldk, int64_t ldv, const int64_t* slots, const float* kv_scales,
                  uint8_t* k_cache, uint8_t* v_cache, int64_t ldc, int64_t rows,
                  void* stream);

/*
 * Fused producer: RMSNorm + 1x128 quantization.  The input of the QKV and
 * gate+up projections comes out of an RMSNorm; this call writes its 1x128 FP8
 * codes and scales directly (explainer "Implementierung": fused RMSNorm
 * kernels; "Quantisierungsschema" and 163.com write-up section 五: the
 * quantization runs fused with the operator that produces the activation).
 * Per row m (the pages give no formula; the Llama RMSNorm is taken):
 *   r = 1 / sqrt(mean_k(x[m,k]^2) + eps)            (FP32)
 *   y[m,k] = bf16((x[m,k] * r) * gamma[k])          (FP32 products, one RNE rounding)
 * and q, s are the 1x128 quantization of y, bit for bit what
 * jet_quant_act_1x128 gives for that BF16 y.
 *
 *   x     : BF16 [M, H], row stride ldx elements (ldx >= H, ldx % 8 == 0)
 *   gamma : BF16 [H]
 *   eps   : finite, >= 0
 *   y     : optional BF16 [M, H] output (NULL: not written), row stride ldy
 *   q     : E4M3 [M, H], row stride ldq bytes (ldq >= H, ldq % 16 == 0)
 *   s     : FP32 [H/128, M]
 *   0 < H <= 8192, H % 128 == 0, M >= 0; x, gamma, y, q 16-byte aligned.
 *   The mean square is summed in FP32 (as in an FP32 RMSNorm): rows whose
 *   squares overflow FP32 (|x| above about 1e19) give a zero scale r.
 *   A row of x is read once; the results are independent of M and of the
 *   other rows.  JET_ERR_SHAPE / NULL / ALIGN as for the quantizers.
 */
int jet_rmsnorm_quant_1x128(const void* x, const void* gamma, int64_t M, int64_t H,
                            int64_t ldx, float eps, void* y, int64_t ldy,
                            uint8_t* q, int64_t ldq, float* s, void* stream);

/*
 * Fused producer: SwiGLU + 1x128 quantization, the input of the down
 * projection (explainer "Implementierung": fused activation kernels).  From
 * the fused gate+up projection's output gu = [gate | up]:
 *   h[m,i] = bf16(gate * sigmoid(gate) * up),  gate = gu[m,i], up = gu[m,I+i]
 * (FP32: sigmoid(g) = 1/(1+e) for g >= 0 and e/(1+e) for g < 0 with
 * e = 2^(-|g| log2(e)) on the hardware exp2 and 1/(1+e) on the hardware
 * reciprocal, each within about 1 ulp; one RNE rounding), and q, s are the
 * 1x128 quantization of h, bit for bit what jet_quant_act_1x128 gives for
 * that BF16 h.
 *
 *   gu : BF16 [M, 2I] (columns 0..I-1 gate, I..2I-1 up), row stride ldgu
 *        elements (ldgu >= 2I, ldgu % 8 == 0)
 *   h  : optional BF16 [M, I] output (NULL: not written), row stride ldh
 *   q  : E4M3 [M, I], row stride ldq bytes (ldq >= I, ldq % 16 == 0)
 *   s  : FP32 [I/128, M]
 *   I % 128 == 0, M >= 0; gu, h, q 16-byte aligned.
 */
int jet_swiglu_quant_1x128(const void* gu, int64_t M, int64_t I, int64_t ldgu,
                           void* h, int64_t ldh, uint8_t* q, int64_t ldq, float* s,
                           void* stream);

/*
 * Both activation groupings from one read of a BF16 activation or output
 * gradient: the 1x128 outputs of jet_quant_act_1x128 and the 128x1 transposed
 * outputs of jet_quant_act_128x1_T, bit for bit, in one pass over x.  The
 * forward needs the 1x128 form and the weight gradient the 128x1 form of the
 * same tensor (explainer "Quantisierungsschema"; 163.com write-up section 五);
 * producing both together saves a read of the tensor in HBM.
 *
 *   x, M, K, ldx, q, ldq, s : as jet_quant_act_1x128.
 *   qT, ldqT, sT            : as jet_quant_act_128x1_T (columns M..Mp-1 of qT
 *                             receive zero codes).
 *   requant == 0 : the 128x1 groups quantize the BF16 values of x (as
 *                  jet_quant_act_128x1_T with src_dtype JET_BF16: output
 *                  gradients).
 *   requant == 1 : they quantize the dequantized 1x128 values
 *                  fl32(E4M3value(q) * s) (as jet_quant_act_128x1_T with
 *                  src_dtype JET_E4M3 on this call's q, s: activations).
 *   M >= 0, K % 128 == 0, ceil(M/128) <= 65535.  x, q, qT, sT 16-byte
 *   aligned, s 4-byte aligned; ldx % 8, ldq % 16, ldqT % 16.
 */
int jet_quant_act_1x128_128x1_T(const void* x, int64_t M, int64_t K, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* s,
                                uint8_t* qT, int64_t ldqT, float* sT,
                                int requant, void* stream);

/*
 * 128x128 block quantization of a BF16 master weight (run on every weight
 * sync).  Explainer "Quantisierungsschema" (weights 128x128) and "Kernarchitektur"
 * (BF16 master weights); 66260.cn FP8-RL item (block-wise re-conversion of the
 * updated parameters at each weight synchronisation).
 *
 *   w  : BF16 [N, K], row stride ldw elements (ldw >= K, ldw % 8 == 0)
 *   q  : E4M3 [N, K], dense (row stride K)
 *   s  : FP32 [N/128, K/128], block (i, j) at s[i*(K/128)+j]
 *   qT : optional E4M3 [K, N], dense (row stride N): the same codes transposed,
 *        used as the B operand of jet_fp8_linear_dgrad.  NULL = not written.
 *   N % 128 == 0, K % 128 == 0.
 */
int jet_quant_weight_128x128(const void* w, int64_t N, int64_t K, int64_t ldw,
                             uint8_t* q, float* s, uint8_t* qT, void* stream);

/*
 * Forward GEMM  Y[m,n] = sum_k Xhat[m,k] * What[n,k]  with Xhat = E4M3(xq)*xs
 * (1x128) and What = E4M3(wq)*ws (128x128); FP32 accumulation, the FP32
 * scales applied at every 128-wide K step.  163.com section 五 (1x128 input
 * times 128x128 weight); explainer "Quantisierungsschema".
 *
 *   xq : E4M3 [M, K] dense; xs : FP32 [K/128, M]
 *   wq : E4M3 [N, K] dense; ws : FP32 [N/128, K/128]
 *   y  : [M, N] dense, y_dtype JET_BF16 or JET_F32
 *   yq, ys : optional fused epilogue (both NULL or both set, y_dtype must be
 *        JET_BF16): yq E4M3 [M, N] dense and ys FP32 [N/128, M] receive
 *        jet_quant_act_1x128 of the BF16 Y -- the next layer's FP8 input
 *        (163.com section 五: quantization fused with the preceding operator).
 *   workspace : device scratch of at least jet_workspace_bytes(JET_OP_FWD, M, N, K)
 *        bytes, 16-byte aligned (may be NULL when that is 0).  For M <= 128
 *        (rollout decode, explainer "Kernarchitektur": rollout runs the same
 *        forward) the call may split the contraction into ranges whose FP32
 *        partial sums live in the workspace, then sums them in a fixed order:
 *        the result is deterministic, and within the GEMM tolerance of the
 *        large-M kernel (the FP32 summation order differs).  Its contents on
 *        entry are ignored and unspecified on return.  The caller owns the
 *        workspace; calls that share one workspace must not overlap.
 *   M >= 0, N % 128 == 0, K % 128 == 0, N and K <= 2^24 (row strides of the
 *   FP8 operands), all pointers 16-byte aligned.
 */
int jet_fp8_linear_fwd(const uint8_t* xq, const float* xs,
                       const uint8_t* wq, const float* ws,
                       int64_t M, int64_t N, int64_t K,
                       void* y, int y_dtype, uint8_t* yq, float* ys,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * The forward of jet_fp8_linear_fwd with a batch-invariant result: every
 * output element is computed by the same chain of operations whatever M is
 * (one MFMA per 128-wide K step from zero, folded into FP32 in K order), so a
 * token's Y, and its fused 1x128 codes, are bit-identical whether it is
 * computed in a rollout batch of a few rows or in a training batch of
 * thousands.  The explainer ("Kernarchitektur") requires the rollout graph to
 * be the training forward graph at the same granularity and precision; this
 * entry point makes the two forwards agree bit for bit, not only in format.
 * For M <= 128 it streams the weight with one K range per output block (no
 * workspace; the split ranges of jet_fp8_linear_fwd are summed in another
 * FP32 order), which is slower there when N/128 blocks leave CUs idle; for
 * M > 128 it is jet_fp8_linear_fwd.  Arguments, layouts and errors as
 * jet_fp8_linear_fwd without the workspace.
 */
int jet_fp8_linear_fwd_batch_invariant(const uint8_t* xq, const float* xs,
                                       const uint8_t* wq, const float* ws,
                                       int64_t M, int64_t N, int64_t K,
                                       void* y, int y_dtype, uint8_t* yq, float* ys,
                                       void* stream);

/*
 * jet_fp8_linear_fwd for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The split-K partial sums of the small-M forward (the only
 * scratch of jet_fp8_linear_fwd) go to a static device array of 16 MiB that
 * the library holds on every GPU it runs on until the process ends, instead
 * of a caller's workspace; the call itself allocates and frees nothing.
 * Arguments, layouts, results (bit for bit) and errors as jet_fp8_linear_fwd
 * without the workspace; JET_ERR_WORKSPACE if jet_workspace_bytes(JET_OP_FWD,
 * M, N, K) exceeds the array (no shape the forward accepts needs more than
 * its 16,777,216 bytes).  The first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress); JET_ERR_HIP if that
 * fails.  All calls on one GPU share its array and nothing in it needs to
 * start at zero (every partial sum is written before it is read), but calls
 * that overlap in time on one GPU -- on different streams, or from several
 * host threads -- race on it: serialise them.
 */
int jet_fp8_linear_fwd_noalloc(const uint8_t* xq, const float* xs,
                               const uint8_t* wq, const float* ws,
                               int64_t M, int64_t N, int64_t K,
                               void* y, int y_dtype, uint8_t* yq, float* ys,
                               void* stream);

/*
 * Data-gradient GEMM  dX[m,k] = sum_n dYhat[m,n] * What[n,k].
 * Explainer "Quantisierungsschema" (DGrad in FP8; BF16 gradients between
 * operators); nmedialink table (output gradients 1x128).
 *
 *   dyq : E4M3 [M, N] dense (jet_quant_act_1x128 of dY); dys : FP32 [N/128, M]
 *   wqT : E4M3 [K, N] dense -- the transposed codes written by
 *         jet_quant_weight_128x128 (its qT output); ws : FP32 [N/128, K/128]
 *         (the same block scales as the forward).
 *   dx  : [M, K] dense, dx_dtype JET_BF16 or JET_F32
 *   M >= 0, N % 128 == 0, K % 128 == 0, N and K <= 2^24, all pointers
 *   16-byte aligned.
 */
int jet_fp8_linear_dgrad(const uint8_t* dyq, const float* dys,
                         const uint8_t* wqT, const float* ws,
                         int64_t M, int64_t N, int64_t K,
                         void* dx, int dx_dtype,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Weight-gradient GEMM  dW[n,k] (+)= sum_m dYhat[m,n] * Xhat[m,k]  with both
 * operands grouped 128x1 along the M tokens (a per-row times per-column FP32
 * scale at every 128-token step).  Explainer "Quantisierungsschema" (WGrad in
 * FP8 with 1x128/128x1 groupings).
 *
 *   dyqT : E4M3 [N, Mp] dense, Mp = ceil(M/128)*128; dysT : FP32 [Mp/128, N]
 *   xqT  : E4M3 [K, Mp] dense;                         xsT  : FP32 [Mp/128, K]
 *          (both as written by jet_quant_act_128x1_T; padding columns hold zeros)
 *   dw   : [N, K] dense, dw_dtype JET_F32 or JET_BF16; accumulate != 0 adds
 *          to the existing contents (JET_F32 only).
 *   M >= 0, N % 128 == 0, K % 128 == 0; M, N and K <= 2^24 (M sets the row
 *   stride of the transposed operands), all pointers 16-byte aligned.
 */
int jet_fp8_linear_wgrad(const uint8_t* dyqT, const float* dysT,
                         const uint8_t* xqT, const float* xsT,
                         int64_t M, int64_t N, int64_t K,
                         void* dw, int dw_dtype, int accumulate,
                         void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes the GEMM `op` (jet_op) needs at this shape (0 = none):
 * nonzero only for the dense forward with 0 < M <= 128 when its contraction is
 * split (S ranges, S <= 16: S * M * N * 4 bytes of partial sums).  The grouped
 * GEMMs need none. */
size_t jet_workspace_bytes(int op, int64_t M, int64_t N, int64_t K);

/*
 * Grouped (mixture-of-experts) layer.  The pages apply the FP8 recipe to MoE
 * models (66260.cn FP8-RL item: expert layers in the compressed format;
 * nmedialink section on the Qwen3-30B MoE experiment) without a layout, so:
 * the M routed rows are sorted by expert and expert e owns the contiguous
 * segment of rows seg_off[e] .. seg_off[e+1]-1; every step of the dense layer
 * applies per segment with expert e's weights.
 *
 *   seg_off : DEVICE int32 [E+1], seg_off[0] = 0, nondecreasing,
 *             seg_off[E] = M.  It is read on the device only (no host sync).
 *             Offsets that break these rules give unspecified results, but
 *             every access stays inside the buffers described here.
 *   1 <= E <= 2^20.  The 1x128 quantization of X and dY, and the 128x128
 *   quantization of the stacked weights [E*N, K], are the dense entry points
 *   (their groups never cross a row or an expert).
 *
 * Padded transposed layout of the grouped WGrad operands: segment e owns the
 * columns col[e] .. col[e+1]-1 with col[e] = 128 * sum_{e'<e} ceil(len_e'/128);
 * its 128x1 groups start at its first row; columns past its rows hold zero
 * codes.  Buffers are sized for the largest possible total,
 * P = 128 * (ceil(M/128) + E) columns; columns past col[E] are not written.
 */

/*
 *   src, src_dtype, src_s, M, K, ldsrc : as jet_quant_act_128x1_T (M = all rows).
 *   qT : E4M3 [K, ldqT] with ldqT >= P (ldqT % 16 == 0);  sT : FP32 [ldqT/128, K],
 *        the scale of slot g (columns 128g..128g+127) of column k at sT[g*K + k].
 *   ceil(M/128) + E <= 65535.
 */
int jet_quant_act_128x1_T_grouped(const void* src, int src_dtype, const float* src_s,
                                  int64_t M, int64_t K, int64_t ldsrc,
                                  const int32_t* seg_off, int64_t E,
                                  uint8_t* qT, int64_t ldqT, float* sT, void* stream);

/*
 * Y rows of segment e = Xhat_e . What_e^T.
 *   xq, xs : as jet_fp8_linear_fwd over all M rows (xs [K/128, M]).
 *   wq : E4M3 [E, N, K] dense; ws : FP32 [E, N/128, K/128].
 *   y, yq, ys : as jet_fp8_linear_fwd ([M, N], ys [N/128, M]).
 */
int jet_fp8_grouped_fwd(const uint8_t* xq, const float* xs,
                        const uint8_t* wq, const float* ws,
                        const int32_t* seg_off, int64_t E,
                        int64_t M, int64_t N, int64_t K,
                        void* y, int y_dtype, uint8_t* yq, float* ys,
                        void* workspace, size_t ws_bytes, void* stream);

/*
 * dX rows of segment e = dYhat_e . What_e.
 *   dyq, dys : as jet_fp8_linear_dgrad over all M rows.
 *   wqT : E4M3 [K, E*N] dense -- the transposed codes jet_quant_weight_128x128
 *         writes for the stacked weights [E*N, K] (expert e: columns e*N..e*N+N-1);
 *   ws  : FP32 [E, N/128, K/128].  E*N <= 2^24.
 *   dx  : [M, K] dense, dx_dtype JET_BF16 or JET_F32.
 */
int jet_fp8_grouped_dgrad(const uint8_t* dyq, const float* dys,
                          const uint8_t* wqT, const float* ws,
                          const int32_t* seg_off, int64_t E,
                          int64_t M, int64_t N, int64_t K,
                          void* dx, int dx_dtype,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * dW_e (+)= dYhat_e^T . Xhat_e for every expert (an empty segment gives 0).
 *   dyqT : E4M3 [N, ldT], dysT : FP32 [ldT/128, N]   (jet_quant_act_128x1_T_grouped of dY)
 *   xqT  : E4M3 [K, ldT], xsT  : FP32 [ldT/128, K]   (of the 1x128-quantized X)
 *   ldT >= P, ldT % 16 == 0, ldT <= 2^24.
 *   dw : [E, N, K] dense, dw_dtype JET_F32 or JET_BF16; accumulate as jet_fp8_linear_wgrad.
 */
int jet_fp8_grouped_wgrad(const uint8_t* dyqT, const float* dysT,
                          const uint8_t* xqT, const float* xsT, int64_t ldT,
                          const int32_t* seg_off, int64_t E,
                          int64_t M, int64_t N, int64_t K,
                          void* dw, int dw_dtype, int accumulate,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * Power-of-two-scale variant.  Not on the pages: their group scale is the FP32
 * value amax/448 (explainer "Quantisierungsschema"; 163.com section 七: scales
 * follow the data).  gfx950's block-scaled MFMA takes its operand scales as
 * 8-bit powers of two (E8M0, 2^(b-127)); with power-of-two group scales the
 * GEMMs hand each scale to the MFMA and accumulate across the 128-wide K steps
 * inside it, so no FP32 rescaling runs per step.  Scale of a group:
 *     amax_c = max(amax, 2^-96),  s = 2^e with e the smallest integer for
 *     which 448 * 2^e >= amax_c,  code = E4M3(x * 2^-e)
 * (-104 <= e <= 120 for finite data; nothing saturates and the group maximum encodes within
 * (224, 448]).  The scales are stored as FP32 values, in the layouts of the
 * FP32-scale entry points, so the two sets of quantizers and GEMMs take the
 * same buffers; but the _pow2 GEMMs read only the exponent field of each
 * scale (a scale that is not a power of two is taken as the power of two
 * below it), so feed them the _pow2 quantizers' output.  Each _pow2 entry point
 * takes the arguments, layouts and limits of its FP32-scale twin and reports
 * the same errors; the GEMMs take no workspace.  The forward at M <= 128
 * streams the weight with one K range, each output element the same chain of
 * MFMAs as in the tiled kernel used for larger M, so it is batch-invariant
 * at every M.
 */
int jet_quant_act_1x128_pow2(const void* x, int64_t M, int64_t K, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, void* stream);
int jet_quant_act_128x1_T_pow2(const void* src, int src_dtype, const float* src_s,
                               int64_t M, int64_t K, int64_t ldsrc,
                               uint8_t* qT, int64_t ldqT, float* sT, void* stream);
int jet_quant_act_1x128_128x1_T_pow2(const void* x, int64_t M, int64_t K, int64_t ldx,
                                     uint8_t* q, int64_t ldq, float* s,
                                     uint8_t* qT, int64_t ldqT, float* sT,
                                     int requant, void* stream);
int jet_quant_weight_128x128_pow2(const void* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* q, float* s, uint8_t* qT, void* stream);
/* yq, ys (optional): the power-of-two 1x128 quantization of the BF16 Y. */
int jet_fp8_linear_fwd_pow2(const uint8_t* xq, const float* xs,
                            const uint8_t* wq, const float* ws,
                            int64_t M, int64_t N, int64_t K,
                            void* y, int y_dtype, uint8_t* yq, float* ys,
                            void* stream);
int jet_fp8_linear_dgrad_pow2(const uint8_t* dyq, const float* dys,
                              const uint8_t* wqT, const float* ws,
                              int64_t M, int64_t N, int64_t K,
                              void* dx, int dx_dtype, void* stream);
int jet_fp8_linear_wgrad_pow2(const uint8_t* dyqT, const float* dysT,
                              const uint8_t* xqT, const float* xsT,
                              int64_t M, int64_t N, int64_t K,
                              void* dw, int dw_dtype, int accumulate, void* stream);
/* The fused producers of the 1x128 input with power-of-two scales. */
int jet_rmsnorm_quant_1x128_pow2(const void* x, const void* gamma, int64_t M, int64_t H,
                                 int64_t ldx, float eps, void* y, int64_t ldy,
                                 uint8_t* q, int64_t ldq, float* s, void* stream);
int jet_swiglu_quant_1x128_pow2(const void* gu, int64_t M, int64_t I, int64_t ldgu,
                                void* h, int64_t ldh, uint8_t* q, int64_t ldq, float* s,
                                void* stream);
/* The grouped (mixture-of-experts) layer with power-of-two scales: the 1x128
 * and 128x128 quantizers are the dense _pow2 ones (as for the FP32-scale
 * grouped layer); these four are the twins of the grouped entry points. */
int jet_quant_act_128x1_T_grouped_pow2(const void* src, int src_dtype, const float* src_s,
                                       int64_t M, int64_t K, int64_t ldsrc,
                                       const int32_t* seg_off, int64_t E,
                                       uint8_t* qT, int64_t ldqT, float* sT, void* stream);
int jet_fp8_grouped_fwd_pow2(const uint8_t* xq, const float* xs,
                             const uint8_t* wq, const float* ws,
                             const int32_t* seg_off, int64_t E,
                             int64_t M, int64_t N, int64_t K,
                             void* y, int y_dtype, uint8_t* yq, float* ys, void* stream);
int jet_fp8_grouped_dgrad_pow2(const uint8_t* dyq, const float* dys,
                               const uint8_t* wqT, const float* ws,
                               const int32_t* seg_off, int64_t E,
                               int64_t M, int64_t N, int64_t K,
                               void* dx, int dx_dtype, void* stream);
int jet_fp8_grouped_wgrad_pow2(const uint8_t* dyqT, const float* dysT,
                               const uint8_t* xqT, const float* xsT, int64_t ldT,
                               const int32_t* seg_off, int64_t E,
                               int64_t M, int64_t N, int64_t K,
                               void* dw, int dw_dtype, int accumulate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JETFP8_H */
