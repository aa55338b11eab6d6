// C ABI of the FP8 linear-layer library (declarations and contracts in
// include/jetfp8.h).  This file validates arguments, maps each entry point
// onto a kernel launch and reports errors; it holds no arithmetic.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/jetfp8.h"
#include "jet_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return JET_OK;
  return fail(JET_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kG = 128;
constexpr int64_t kMaxDim = int64_t(1) << 30;   // GEMM tile indices are 32-bit
// Row stride (bytes) of an FP8 GEMM operand: the kernels address a tile's rows
// with 32-bit offsets from a 64-bit per-tile base, at most 256 rows apart.
constexpr int64_t kMaxLd = int64_t(1) << 24;

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int jet_abi_version(void) { return JET_ABI_VERSION; }

const char* jet_status_string(int status) {
  switch (status) {
    case JET_OK: return "JET_OK";
    case JET_ERR_NULL: return "JET_ERR_NULL";
    case JET_ERR_SHAPE: return "JET_ERR_SHAPE";
    case JET_ERR_ALIGN: return "JET_ERR_ALIGN";
    case JET_ERR_DTYPE: return "JET_ERR_DTYPE";
    case JET_ERR_WORKSPACE: return "JET_ERR_WORKSPACE";
    case JET_ERR_HIP: return "JET_ERR_HIP";
    default: return "JET_ERR_UNKNOWN";
  }
}

const char* jet_last_error(void) { return g_last_error; }

static int quant_1x128(const char* name, bool p2, const void* x, int64_t M, int64_t K, int64_t ldx,
                       uint8_t* q, int64_t ldq, float* s, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || K < 0 || K % kG || M > kMaxDim || K > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need M >= 0 and K a multiple of 128 (M=%lld K=%lld)", name,
                (long long)M, (long long)K);
  if (M == 0 || K == 0) return JET_OK;
  if (!x || !q || !s) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldx < K || ldq < K) return fail(JET_ERR_SHAPE, "%s: leading dimension < K", name);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4) || ldx % 8 || ldq % 16)
    return fail(JET_ERR_ALIGN, "%s: x, q need 16-byte alignment, ldx %% 8, ldq %% 16", name);
  return hip_status(jet::launch_quant_1x128(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq, s,
                                            as_stream(stream), p2),
                    name);
}

int jet_quant_act_1x128(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                        float* s, void* stream) {
  return quant_1x128("quant_act_1x128", false, x, M, K, ldx, q, ldq, s, stream);
}

int jet_quant_act_1x128_pow2(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q, int64_t ldq,
                             float* s, void* stream) {
  return quant_1x128("quant_act_1x128_pow2", true, x, M, K, ldx, q, ldq, s, stream);
}

static int rmsnorm_quant(const char* name, bool p2, const void* x, const void* gamma, int64_t M, int64_t H,
                         int64_t ldx, float eps, void* y, int64_t ldy, uint8_t* q, int64_t ldq, float* s,
                         void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || H <= 0 || H % kG || H > 8192 || M > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need M >= 0 and 0 < H <= 8192, H %% 128 == 0 (M=%lld H=%lld)", name,
                (long long)M, (long long)H);
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(JET_ERR_SHAPE, "%s: eps must be finite and >= 0", name);
  if (M == 0) return JET_OK;
  if (!x || !gamma || !q || !s) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldx < H || ldq < H || (y && ldy < H)) return fail(JET_ERR_SHAPE, "%s: leading dimension < H", name);
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(q, 16) || !aligned(s, 4) || ldx % 8 ||
      ldq % 16 || (y && (!aligned(y, 16) || ldy % 8)))
    return fail(JET_ERR_ALIGN, "%s: x, gamma, y, q need 16-byte alignment, ldx %% 8, ldy %% 8, ldq %% 16", name);
  return hip_status(jet::launch_rmsnorm_quant_1x128(static_cast<const uint16_t*>(x),
                                                    static_cast<const uint16_t*>(gamma), M, H, ldx, eps,
                                                    static_cast<uint16_t*>(y), ldy, q, ldq, s,
                                                    as_stream(stream), p2),
                    name);
}

int jet_rmsnorm_quant_1x128(const void* x, const void* gamma, int64_t M, int64_t H, int64_t ldx,
                            float eps, void* y, int64_t ldy, uint8_t* q, int64_t ldq, float* s,
                            void* stream) {
  return rmsnorm_quant("rmsnorm_quant_1x128", false, x, gamma, M, H, ldx, eps, y, ldy, q, ldq, s, stream);
}

int jet_rmsnorm_quant_1x128_pow2(const void* x, const void* gamma, int64_t M, int64_t H, int64_t ldx,
                                 float eps, void* y, int64_t ldy, uint8_t* q, int64_t ldq, float* s,
                                 void* stream) {
  return rmsnorm_quant("rmsnorm_quant_1x128_pow2", true, x, gamma, M, H, ldx, eps, y, ldy, q, ldq, s, stream);
}

static int swiglu_quant(const char* name, bool p2, const void* gu, int64_t M, int64_t I, int64_t ldgu,
                        void* h, int64_t ldh, uint8_t* q, int64_t ldq, float* s, void* stream) {
  g_last_error[0] = 0;
  if (M < 0 || I < 0 || I % kG || M > kMaxDim || I > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need M >= 0 and I a multiple of 128 (M=%lld I=%lld)", name, (long long)M,
                (long long)I);
  if (M == 0 || I == 0) return JET_OK;
  if (!gu || !q || !s) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldgu < 2 * I || ldq < I || (h && ldh < I))
    return fail(JET_ERR_SHAPE, "%s: need ldgu >= 2*I, ldq >= I, ldh >= I", name);
  if (!aligned(gu, 16) || !aligned(q, 16) || !aligned(s, 4) || ldgu % 8 || ldq % 16 ||
      (h && (!aligned(h, 16) || ldh % 8)))
    return fail(JET_ERR_ALIGN, "%s: gu, h, q need 16-byte alignment, ldgu %% 8, ldh %% 8, ldq %% 16", name);
  return hip_status(jet::launch_swiglu_quant_1x128(static_cast<const uint16_t*>(gu), M, I, ldgu,
                                                   static_cast<uint16_t*>(h), ldh, q, ldq, s,
                                                   as_stream(stream), p2),
                    name);
}

int jet_swiglu_quant_1x128(const void* gu, int64_t M, int64_t I, int64_t ldgu, void* h, int64_t ldh,
                           uint8_t* q, int64_t ldq, float* s, void* stream) {
  return swiglu_quant("swiglu_quant_1x128", false, gu, M, I, ldgu, h, ldh, q, ldq, s, stream);
}

int jet_swiglu_quant_1x128_pow2(const void* gu, int64_t M, int64_t I, int64_t ldgu, void* h, int64_t ldh,
                                uint8_t* q, int64_t ldq, float* s, void* stream) {
  return swiglu_quant("swiglu_quant_1x128_pow2", true, gu, M, I, ldgu, h, ldh, q, ldq, s, stream);
}

static int check_kv_rows(const char* name, const void* k, const void* v, int64_t T, int64_t D, int64_t ldk,
                         int64_t ldv) {
  if (T < 0 || D <= 0 || D % 8 || T > kMaxDim || D > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need T >= 0 and D > 0 a multiple of 8 (T=%lld D=%lld)", name,
                (long long)T, (long long)D);
  if (T > 0 && (!k || !v)) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldk < D || ldv < D) return fail(JET_ERR_SHAPE, "%s: row stride < D", name);
  if (T > 0 && (!aligned(k, 16) || !aligned(v, 16) || ldk % 8 || ldv % 8))
    return fail(JET_ERR_ALIGN, "%s: k, v need 16-byte alignment and row strides %% 8", name);
  return JET_OK;
}

int jet_kv_calibrate(const void* k, const void* v, int64_t T, int64_t D, int64_t ldk, int64_t ldv,
                     float* kv_scales, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_kv_rows("kv_calibrate", k, v, T, D, ldk, ldv)) return st;
  if (!kv_scales) return fail(JET_ERR_NULL, "kv_calibrate: null pointer");
  if (!aligned(kv_scales, 4)) return fail(JET_ERR_ALIGN, "kv_calibrate: kv_scales needs 4-byte alignment");
  return hip_status(jet::launch_kv_calibrate(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                             T, D, ldk, ldv, kv_scales, as_stream(stream)),
                    "kv_calibrate");
}

int jet_kv_append(const void* k, const void* v, int64_t T, int64_t D, int64_t ldk, int64_t ldv,
                  const int64_t* slots, const float* kv_scales, uint8_t* k_cache, uint8_t* v_cache,
                  int64_t ldc, int64_t rows, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_kv_rows("kv_append", k, v, T, D, ldk, ldv)) return st;
  if (rows < 0 || ldc < D) return fail(JET_ERR_SHAPE, "kv_append: need rows >= 0 and ldc >= D");
  if (T == 0 || rows == 0) return JET_OK;
  if (!slots || !kv_scales || !k_cache || !v_cache) return fail(JET_ERR_NULL, "kv_append: null pointer");
  if (!aligned(slots, 8) || !aligned(kv_scales, 4) || !aligned(k_cache, 8) || !aligned(v_cache, 8) || ldc % 8)
    return fail(JET_ERR_ALIGN, "kv_append: slots and caches need 8-byte alignment, ldc %% 8");
  return hip_status(jet::launch_kv_append(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), T, D,
                                          ldk, ldv, slots, kv_scales, k_cache, v_cache, ldc, rows,
                                          as_stream(stream)),
                    "kv_append");
}

static int quant_128x1_T(const char* name, bool p2, const void* src, int src_dtype, const float* src_s,
                         int64_t M, int64_t K, int64_t ldsrc, uint8_t* qT, int64_t ldqT, float* sT,
                         void* stream) {
  g_last_error[0] = 0;
  if (src_dtype != JET_BF16 && src_dtype != JET_E4M3)
    return fail(JET_ERR_DTYPE, "%s: src_dtype must be JET_BF16 or JET_E4M3", name);
  if (M < 0 || K < 0 || K % kG || M > kMaxDim || K > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need M >= 0 and K a multiple of 128", name);
  if (M == 0 || K == 0) return JET_OK;
  const bool fp8 = src_dtype == JET_E4M3;
  if (!src || !qT || !sT || (fp8 && !src_s))
    return fail(JET_ERR_NULL, "%s: null pointer", name);
  const int64_t Mp = (M + kG - 1) / kG * kG;
  if (Mp / kG > 65535) return fail(JET_ERR_SHAPE, "%s: ceil(M/128) must be <= 65535", name);
  if (ldsrc < K || ldqT < Mp)
    return fail(JET_ERR_SHAPE, "%s: ldsrc < K or ldqT < ceil(M/128)*128", name);
  const int64_t ld_bytes = fp8 ? ldsrc : 2 * ldsrc;
  if (!aligned(src, 16) || !aligned(qT, 16) || !aligned(sT, 16) || ld_bytes % 16 || ldqT % 16 ||
      (fp8 && !aligned(src_s, 4)))
    return fail(JET_ERR_ALIGN, "%s: src, qT, sT need 16-byte alignment; row strides 16 bytes", name);
  return hip_status(jet::launch_quant_128x1_T(src, fp8, src_s, M, K, ldsrc, qT, ldqT, sT,
                                              as_stream(stream), p2),
                    name);
}

int jet_quant_act_128x1_T(const void* src, int src_dtype, const float* src_s, int64_t M, int64_t K,
                          int64_t ldsrc, uint8_t* qT, int64_t ldqT, float* sT, void* stream) {
  return quant_128x1_T("quant_act_128x1_T", false, src, src_dtype, src_s, M, K, ldsrc, qT, ldqT, sT, stream);
}

int jet_quant_act_128x1_T_pow2(const void* src, int src_dtype, const float* src_s, int64_t M, int64_t K,
                               int64_t ldsrc, uint8_t* qT, int64_t ldqT, float* sT, void* stream) {
  return quant_128x1_T("quant_act_128x1_T_pow2", true, src, src_dtype, src_s, M, K, ldsrc, qT, ldqT, sT,
                       stream);
}

static int quant_1x128_128x1_T(const char* name, bool p2, const void* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* q, int64_t ldq, float* s, uint8_t* qT, int64_t ldqT, float* sT,
                               int requant, void* stream) {
  g_last_error[0] = 0;
  if (requant != 0 && requant != 1)
    return fail(JET_ERR_DTYPE, "%s: requant must be 0 or 1", name);
  if (M < 0 || K < 0 || K % kG || M > kMaxDim || K > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need M >= 0 and K a multiple of 128", name);
  if (M == 0 || K == 0) return JET_OK;
  if (!x || !q || !s || !qT || !sT) return fail(JET_ERR_NULL, "%s: null pointer", name);
  const int64_t Mp = (M + kG - 1) / kG * kG;
  if (Mp / kG > 65535)
    return fail(JET_ERR_SHAPE, "%s: ceil(M/128) must be <= 65535", name);
  if (ldx < K || ldq < K || ldqT < Mp)
    return fail(JET_ERR_SHAPE, "%s: ldx < K, ldq < K or ldqT < ceil(M/128)*128", name);
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(qT, 16) || !aligned(sT, 16) || !aligned(s, 4) ||
      ldx % 8 || ldq % 16 || ldqT % 16)
    return fail(JET_ERR_ALIGN,
                "%s: x, q, qT, sT need 16-byte alignment, ldx %% 8, ldq %% 16, ldqT %% 16", name);
  return hip_status(jet::launch_quant_1x128_128x1_T(static_cast<const uint16_t*>(x), M, K, ldx, q, ldq,
                                                    s, qT, ldqT, sT, requant == 1, as_stream(stream), p2),
                    name);
}

int jet_quant_act_1x128_128x1_T(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                int64_t ldq, float* s, uint8_t* qT, int64_t ldqT, float* sT,
                                int requant, void* stream) {
  return quant_1x128_128x1_T("quant_act_1x128_128x1_T", false, x, M, K, ldx, q, ldq, s, qT, ldqT, sT, requant,
                             stream);
}

int jet_quant_act_1x128_128x1_T_pow2(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                                     int64_t ldq, float* s, uint8_t* qT, int64_t ldqT, float* sT,
                                     int requant, void* stream) {
  return quant_1x128_128x1_T("quant_act_1x128_128x1_T_pow2", true, x, M, K, ldx, q, ldq, s, qT, ldqT, sT,
                             requant, stream);
}

static int quant_weight(const char* name, bool p2, const void* w, int64_t N, int64_t K, int64_t ldw,
                        uint8_t* q, float* s, uint8_t* qT, void* stream) {
  g_last_error[0] = 0;
  if (N < 0 || K < 0 || N % kG || K % kG || N > kMaxDim || K > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: N and K must be multiples of 128", name);
  if (N == 0 || K == 0) return JET_OK;
  if (!w || !q || !s) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldw < K) return fail(JET_ERR_SHAPE, "%s: ldw < K", name);
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4) || ldw % 8 || (qT && !aligned(qT, 16)))
    return fail(JET_ERR_ALIGN, "%s: w, q, qT need 16-byte alignment, ldw %% 8", name);
  return hip_status(jet::launch_quant_128x128(static_cast<const uint16_t*>(w), N, K, ldw, q, s, qT,
                                              as_stream(stream), p2),
                    name);
}

int jet_quant_weight_128x128(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, float* s,
                             uint8_t* qT, void* stream) {
  return quant_weight("quant_weight_128x128", false, w, N, K, ldw, q, s, qT, stream);
}

int jet_quant_weight_128x128_pow2(const void* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q, float* s,
                                  uint8_t* qT, void* stream) {
  return quant_weight("quant_weight_128x128_pow2", true, w, N, K, ldw, q, s, qT, stream);
}

size_t jet_workspace_bytes(int op, int64_t M, int64_t N, int64_t K) {
  // the dense forward at M <= 128 keeps split-K partial sums in the workspace
  if (op == JET_OP_FWD && M > 0 && M <= jet::kSkinnyMaxM && N > 0 && K > 0 && N % kG == 0 &&
      K % kG == 0 && N <= kMaxDim && K <= kMaxDim)
    return jet::skinny_workspace_bytes(M, N, K);
  return 0;
}

// need: the workspace bytes this call requires (0 for the grouped GEMMs)
static int check_gemm_common(const char* name, int64_t M, int64_t N, int64_t K, size_t need,
                             size_t ws_bytes, const void* workspace) {
  if (M < 0 || N < 0 || K < 0 || N % kG || K % kG || M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: need M >= 0, N and K multiples of 128 (M=%lld N=%lld K=%lld)",
                name, (long long)M, (long long)N, (long long)K);
  if (N > kMaxLd || K > kMaxLd)
    return fail(JET_ERR_SHAPE, "%s: N and K must be <= 2^24 (FP8 operand row strides)", name);
  if (ws_bytes < need || (need && !workspace))
    return fail(JET_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", name, need);
  if (need && !aligned(workspace, 16))
    return fail(JET_ERR_ALIGN, "%s: the workspace needs 16-byte alignment", name);
  return JET_OK;
}

// The forward; invariant: one K range at every M (no workspace), so each
// output element does not depend on M.  p2: power-of-two scales applied by the
// MFMA, one K range at every M (no workspace; batch-invariant as well).
static int linear_fwd(const char* name, const uint8_t* xq, const float* xs, const uint8_t* wq,
                      const float* ws, int64_t M, int64_t N, int64_t K, void* y, int y_dtype, uint8_t* yq,
                      float* ys, void* workspace, size_t ws_bytes, void* stream, bool invariant, bool p2 = false,
                      bool validate_only = false) {
  g_last_error[0] = 0;
  const size_t need = (invariant || p2) ? 0 : jet_workspace_bytes(JET_OP_FWD, M, N, K);
  if (int st = check_gemm_common(name, M, N, K, need, ws_bytes, workspace)) return st;
  if (y_dtype != JET_BF16 && y_dtype != JET_F32)
    return fail(JET_ERR_DTYPE, "%s: y_dtype must be JET_BF16 or JET_F32", name);
  const bool fuse = yq || ys;
  if (fuse && (!yq || !ys)) return fail(JET_ERR_NULL, "%s: yq and ys go together", name);
  if (fuse && y_dtype != JET_BF16)
    return fail(JET_ERR_DTYPE, "%s: the fused 1x128 output needs y_dtype JET_BF16", name);
  if (M == 0 || N == 0) return JET_OK;
  if (!xq || !xs || !wq || !ws || !y) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(xs, 4) || !aligned(ws, 4) ||
      (fuse && (!aligned(yq, 16) || !aligned(ys, 4))))
    return fail(JET_ERR_ALIGN, "%s: operands and outputs need 16-byte alignment", name);
  if (validate_only) return JET_OK;
  jet::GemmArgs a{};
  a.A = xq; a.lda = K;
  a.B = wq; a.ldb = K;
  a.sA = xs; a.sA_ld = M;
  a.sB = ws; a.sB_o = K / kG; a.sB_c = 1;
  a.C = y; a.ldc = N; a.Cq = yq; a.Cs = ys; a.ldcs = M;
  a.M = (int)M; a.N = (int)N; a.Kc = (int)K;
  const int out = y_dtype == JET_BF16 ? jet::kOutBf16 : jet::kOutF32;
  if (M <= jet::kSkinnyMaxM)   // rollout decode: weight-streaming (split-K through the workspace)
    return hip_status(jet::launch_gemm_skinny(a, out, fuse, workspace, as_stream(stream), invariant, p2), name);
  return hip_status(jet::launch_gemm(a, jet::kRowBlock, out, false, fuse, as_stream(stream), p2), name);
}

int jet_fp8_linear_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                       int64_t M, int64_t N, int64_t K, void* y, int y_dtype, uint8_t* yq, float* ys,
                       void* workspace, size_t ws_bytes, void* stream) {
  return linear_fwd("fp8_linear_fwd", xq, xs, wq, ws, M, N, K, y, y_dtype, yq, ys, workspace, ws_bytes,
                    stream, false);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Device scratch of jet_fp8_linear_fwd_noalloc: the split-K partial sums of
// the small-M forward live here instead of in a caller's workspace.  Every
// GPU the library runs on holds its own copy of the array until the process
// ends.  16 MiB covers every split the forward chooses (S * M * N * 4 bytes
// with M <= 128 and S ranges of N/128 column blocks, S * N/128 <= 256: at most
// exactly 16 MiB); the guard below still rejects a larger need.
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up once per
// device (with that device current) and kept.  In host code the array's name
// is only a host-side stand-in, never a device address.
int scratch_address(const char* name, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, name);
  if (dev < 0 || dev >= kMaxDevices) return fail(JET_ERR_HIP, "%s: device %d out of range", name, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, name);
    if (!p) return fail(JET_ERR_HIP, "%s: no device address for the scratch array", name);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return JET_OK;
}

}  // namespace

extern "C" {

int jet_fp8_linear_fwd_noalloc(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                               int64_t M, int64_t N, int64_t K, void* y, int y_dtype, uint8_t* yq,
                               float* ys, void* stream) {
  static const char* const name = "fp8_linear_fwd_noalloc";
  g_last_error[0] = 0;
  const size_t need = jet_workspace_bytes(JET_OP_FWD, M, N, K);
  if (need > kScratchBytes)
    return fail(JET_ERR_WORKSPACE, "%s: this shape needs %zu bytes of scratch; the static scratch holds %zu",
                name, need, kScratchBytes);
  // every argument error before any HIP call; an empty output launches nothing
  void* const fake = reinterpret_cast<void*>(uintptr_t(256));   // aligned stand-in, never dereferenced
  if (int st = linear_fwd(name, xq, xs, wq, ws, M, N, K, y, y_dtype, yq, ys, need ? fake : nullptr,
                          kScratchBytes, stream, false, false, true))
    return st;
  if (M == 0 || N == 0) return JET_OK;
  void* sp = nullptr;
  if (int st = scratch_address(name, &sp)) return st;
  return linear_fwd(name, xq, xs, wq, ws, M, N, K, y, y_dtype, yq, ys, need ? sp : nullptr, kScratchBytes,
                    stream, false);
}

int jet_fp8_linear_fwd_batch_invariant(const uint8_t* xq, const float* xs, const uint8_t* wq,
                                       const float* ws, int64_t M, int64_t N, int64_t K, void* y,
                                       int y_dtype, uint8_t* yq, float* ys, void* stream) {
  return linear_fwd("fp8_linear_fwd_batch_invariant", xq, xs, wq, ws, M, N, K, y, y_dtype, yq, ys, nullptr,
                    0, stream, true);
}

int jet_fp8_linear_fwd_pow2(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                            int64_t M, int64_t N, int64_t K, void* y, int y_dtype, uint8_t* yq, float* ys,
                            void* stream) {
  return linear_fwd("fp8_linear_fwd_pow2", xq, xs, wq, ws, M, N, K, y, y_dtype, yq, ys, nullptr, 0, stream,
                    false, true);
}

static int linear_dgrad(const char* name, bool p2, const uint8_t* dyq, const float* dys, const uint8_t* wqT,
                        const float* ws, int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype, void* workspace,
                        size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_gemm_common(name, M, N, K, jet_workspace_bytes(JET_OP_DGRAD, M, N, K), ws_bytes, workspace))
    return st;
  if (dx_dtype != JET_BF16 && dx_dtype != JET_F32)
    return fail(JET_ERR_DTYPE, "%s: dx_dtype must be JET_BF16 or JET_F32", name);
  if (M == 0 || K == 0) return JET_OK;
  if (!dyq || !dys || !wqT || !ws || !dx) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (!aligned(dyq, 16) || !aligned(wqT, 16) || !aligned(dx, 16) || !aligned(dys, 4) || !aligned(ws, 4))
    return fail(JET_ERR_ALIGN, "%s: operands and output need 16-byte alignment", name);
  jet::GemmArgs a{};
  a.A = dyq; a.lda = N;
  a.B = wqT; a.ldb = N;
  a.sA = dys; a.sA_ld = M;
  a.sB = ws; a.sB_o = 1; a.sB_c = K / kG;
  a.C = dx; a.ldc = K;
  a.M = (int)M; a.N = (int)K; a.Kc = (int)N;
  return hip_status(jet::launch_gemm(a, jet::kRowBlock, dx_dtype == JET_BF16 ? jet::kOutBf16 : jet::kOutF32,
                                     false, false, as_stream(stream), p2),
                    name);
}

int jet_fp8_linear_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wqT, const float* ws,
                         int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype, void* workspace,
                         size_t ws_bytes, void* stream) {
  return linear_dgrad("fp8_linear_dgrad", false, dyq, dys, wqT, ws, M, N, K, dx, dx_dtype, workspace, ws_bytes,
                      stream);
}

int jet_fp8_linear_dgrad_pow2(const uint8_t* dyq, const float* dys, const uint8_t* wqT, const float* ws,
                              int64_t M, int64_t N, int64_t K, void* dx, int dx_dtype, void* stream) {
  return linear_dgrad("fp8_linear_dgrad_pow2", true, dyq, dys, wqT, ws, M, N, K, dx, dx_dtype, nullptr, 0,
                      stream);
}

static int linear_wgrad(const char* name, bool p2, const uint8_t* dyqT, const float* dysT, const uint8_t* xqT,
                        const float* xsT, int64_t M, int64_t N, int64_t K, void* dw, int dw_dtype, int accumulate,
                        void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_gemm_common(name, M, N, K, jet_workspace_bytes(JET_OP_WGRAD, M, N, K), ws_bytes, workspace))
    return st;
  if (dw_dtype != JET_F32 && dw_dtype != JET_BF16)
    return fail(JET_ERR_DTYPE, "%s: dw_dtype must be JET_F32 or JET_BF16", name);
  if (accumulate && dw_dtype != JET_F32)
    return fail(JET_ERR_DTYPE, "%s: accumulate needs dw_dtype JET_F32", name);
  if (N == 0 || K == 0) return JET_OK;
  if (!dw) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (M > 0 && (!dyqT || !dysT || !xqT || !xsT)) return fail(JET_ERR_NULL, "%s: null pointer", name);
  const int64_t Mp = (M + kG - 1) / kG * kG;
  if (Mp > kMaxLd)
    return fail(JET_ERR_SHAPE, "%s: M must be <= 2^24 (row stride of the transposed operands)", name);
  if (!aligned(dw, 16) || (M > 0 && (!aligned(dyqT, 16) || !aligned(xqT, 16) || !aligned(dysT, 4) ||
                                     !aligned(xsT, 4))))
    return fail(JET_ERR_ALIGN, "%s: operands and output need 16-byte alignment", name);
  jet::GemmArgs a{};
  a.A = dyqT; a.lda = Mp;
  a.B = xqT; a.ldb = Mp;
  a.sA = dysT; a.sA_ld = N;
  a.sB = xsT; a.sB_o = 1; a.sB_c = K;
  a.C = dw; a.ldc = K;
  a.M = (int)N; a.N = (int)K; a.Kc = (int)Mp;
  return hip_status(jet::launch_gemm(a, jet::kRowCol, dw_dtype == JET_BF16 ? jet::kOutBf16 : jet::kOutF32,
                                     accumulate != 0, false, as_stream(stream), p2),
                    name);
}

int jet_fp8_linear_wgrad(const uint8_t* dyqT, const float* dysT, const uint8_t* xqT, const float* xsT,
                         int64_t M, int64_t N, int64_t K, void* dw, int dw_dtype, int accumulate,
                         void* workspace, size_t ws_bytes, void* stream) {
  return linear_wgrad("fp8_linear_wgrad", false, dyqT, dysT, xqT, xsT, M, N, K, dw, dw_dtype, accumulate,
                      workspace, ws_bytes, stream);
}

int jet_fp8_linear_wgrad_pow2(const uint8_t* dyqT, const float* dysT, const uint8_t* xqT, const float* xsT,
                              int64_t M, int64_t N, int64_t K, void* dw, int dw_dtype, int accumulate,
                              void* stream) {
  return linear_wgrad("fp8_linear_wgrad_pow2", true, dyqT, dysT, xqT, xsT, M, N, K, dw, dw_dtype, accumulate,
                      nullptr, 0, stream);
}

// ---------------------------------------------------------------------------
// Grouped (mixture-of-experts) entry points
// ---------------------------------------------------------------------------

static int64_t grouped_cols(int64_t M, int64_t E) { return ((M + kG - 1) / kG + E) * kG; }

static int check_grouped_common(const char* name, const int32_t* seg_off, int64_t E, int64_t M) {
  if (E < 1 || E > (int64_t(1) << 20))
    return fail(JET_ERR_SHAPE, "%s: need 1 <= E <= 2^20 experts (E=%lld)", name, (long long)E);
  if (M < 0 || M > kMaxDim) return fail(JET_ERR_SHAPE, "%s: need 0 <= M <= 2^30", name);
  if (!seg_off) return fail(JET_ERR_NULL, "%s: null seg_off", name);
  if (!aligned(seg_off, 4)) return fail(JET_ERR_ALIGN, "%s: seg_off needs 4-byte alignment", name);
  return JET_OK;
}

static int quant_128x1_T_grouped(const char* name, bool p2, const void* src, int src_dtype,
                                 const float* src_s, int64_t M, int64_t K, int64_t ldsrc,
                                 const int32_t* seg_off, int64_t E, uint8_t* qT, int64_t ldqT, float* sT,
                                 void* stream) {
  g_last_error[0] = 0;
  if (src_dtype != JET_BF16 && src_dtype != JET_E4M3)
    return fail(JET_ERR_DTYPE, "%s: src_dtype must be JET_BF16 or JET_E4M3", name);
  if (int st = check_grouped_common(name, seg_off, E, M)) return st;
  if (K < 0 || K % kG || K > kMaxDim)
    return fail(JET_ERR_SHAPE, "%s: K must be a multiple of 128", name);
  if (M == 0 || K == 0) return JET_OK;
  if ((M + kG - 1) / kG + E > 65535)
    return fail(JET_ERR_SHAPE, "%s: ceil(M/128) + E must be <= 65535", name);
  const bool fp8 = src_dtype == JET_E4M3;
  if (!src || !qT || !sT || (fp8 && !src_s))
    return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldsrc < K || ldqT < grouped_cols(M, E))
    return fail(JET_ERR_SHAPE, "%s: ldsrc < K or ldqT < 128*(ceil(M/128)+E)", name);
  const int64_t ld_bytes = fp8 ? ldsrc : 2 * ldsrc;
  if (!aligned(src, 16) || !aligned(qT, 16) || !aligned(sT, 16) || ld_bytes % 16 || ldqT % 16 ||
      (fp8 && !aligned(src_s, 4)))
    return fail(JET_ERR_ALIGN, "%s: src, qT, sT need 16-byte alignment; row strides 16 bytes", name);
  return hip_status(jet::launch_quant_128x1_T_grouped(src, fp8, src_s, M, K, ldsrc, seg_off, (int)E,
                                                      qT, ldqT, sT, as_stream(stream), p2),
                    name);
}

int jet_quant_act_128x1_T_grouped(const void* src, int src_dtype, const float* src_s, int64_t M,
                                  int64_t K, int64_t ldsrc, const int32_t* seg_off, int64_t E,
                                  uint8_t* qT, int64_t ldqT, float* sT, void* stream) {
  return quant_128x1_T_grouped("quant_act_128x1_T_grouped", false, src, src_dtype, src_s, M, K, ldsrc, seg_off, E,
                               qT, ldqT, sT, stream);
}

int jet_quant_act_128x1_T_grouped_pow2(const void* src, int src_dtype, const float* src_s, int64_t M,
                                       int64_t K, int64_t ldsrc, const int32_t* seg_off, int64_t E,
                                       uint8_t* qT, int64_t ldqT, float* sT, void* stream) {
  return quant_128x1_T_grouped("quant_act_128x1_T_grouped_pow2", true, src, src_dtype, src_s, M, K, ldsrc,
                               seg_off, E, qT, ldqT, sT, stream);
}

static int grouped_fwd(const char* name, bool p2, const uint8_t* xq, const float* xs, const uint8_t* wq,
                       const float* ws, const int32_t* seg_off, int64_t E, int64_t M, int64_t N, int64_t K,
                       void* y, int y_dtype, uint8_t* yq, float* ys, void* workspace, size_t ws_bytes,
                       void* stream) {
  g_last_error[0] = 0;
  if (int st = check_grouped_common(name, seg_off, E, M)) return st;
  if (int st = check_gemm_common(name, M, N, K, 0, ws_bytes, workspace)) return st;
  if (y_dtype != JET_BF16 && y_dtype != JET_F32)
    return fail(JET_ERR_DTYPE, "%s: y_dtype must be JET_BF16 or JET_F32", name);
  const bool fuse = yq || ys;
  if (fuse && (!yq || !ys)) return fail(JET_ERR_NULL, "%s: yq and ys go together", name);
  if (fuse && y_dtype != JET_BF16)
    return fail(JET_ERR_DTYPE, "%s: the fused 1x128 output needs y_dtype JET_BF16", name);
  if (M == 0 || N == 0) return JET_OK;
  if (!xq || !xs || !wq || !ws || !y) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(y, 16) || !aligned(xs, 4) || !aligned(ws, 4) ||
      (fuse && (!aligned(yq, 16) || !aligned(ys, 4))))
    return fail(JET_ERR_ALIGN, "%s: operands and outputs need 16-byte alignment", name);
  jet::GemmArgs a{};
  a.A = xq; a.lda = K;
  a.B = wq; a.ldb = K; a.bE = N * K;
  a.sA = xs; a.sA_ld = M;
  a.sB = ws; a.sB_o = K / kG; a.sB_c = 1; a.sbE = (N / kG) * (K / kG);
  a.C = y; a.ldc = N; a.Cq = yq; a.Cs = ys; a.ldcs = M;
  a.M = (int)M; a.N = (int)N; a.Kc = (int)K;
  a.seg = seg_off; a.E = (int)E; a.seg_rows = (int)M;
  return hip_status(jet::launch_gemm_grouped(a, jet::kGrpRows, jet::kRowBlock,
                                             y_dtype == JET_BF16 ? jet::kOutBf16 : jet::kOutF32,
                                             false, fuse, as_stream(stream), p2),
                    name);
}

int jet_fp8_grouped_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                        const int32_t* seg_off, int64_t E, int64_t M, int64_t N, int64_t K, void* y,
                        int y_dtype, uint8_t* yq, float* ys, void* workspace, size_t ws_bytes,
                        void* stream) {
  return grouped_fwd("fp8_grouped_fwd", false, xq, xs, wq, ws, seg_off, E, M, N, K, y, y_dtype, yq, ys,
                     workspace, ws_bytes, stream);
}

int jet_fp8_grouped_fwd_pow2(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                             const int32_t* seg_off, int64_t E, int64_t M, int64_t N, int64_t K, void* y,
                             int y_dtype, uint8_t* yq, float* ys, void* stream) {
  return grouped_fwd("fp8_grouped_fwd_pow2", true, xq, xs, wq, ws, seg_off, E, M, N, K, y, y_dtype, yq, ys,
                     nullptr, 0, stream);
}

static int grouped_dgrad(const char* name, bool p2, const uint8_t* dyq, const float* dys, const uint8_t* wqT,
                         const float* ws, const int32_t* seg_off, int64_t E, int64_t M, int64_t N, int64_t K,
                         void* dx, int dx_dtype, void* workspace, size_t ws_bytes, void* stream) {
  g_last_error[0] = 0;
  if (int st = check_grouped_common(name, seg_off, E, M)) return st;
  if (int st = check_gemm_common(name, M, N, K, 0, ws_bytes, workspace)) return st;
  if (dx_dtype != JET_BF16 && dx_dtype != JET_F32)
    return fail(JET_ERR_DTYPE, "%s: dx_dtype must be JET_BF16 or JET_F32", name);
  if (M == 0 || K == 0) return JET_OK;
  if (E * N > kMaxLd) return fail(JET_ERR_SHAPE, "%s: E*N must be <= 2^24 (row stride of wqT)", name);
  if (!dyq || !dys || !wqT || !ws || !dx) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (!aligned(dyq, 16) || !aligned(wqT, 16) || !aligned(dx, 16) || !aligned(dys, 4) || !aligned(ws, 4))
    return fail(JET_ERR_ALIGN, "%s: operands and output need 16-byte alignment", name);
  jet::GemmArgs a{};
  a.A = dyq; a.lda = N;
  a.B = wqT; a.ldb = E * N; a.bE = N;
  a.sA = dys; a.sA_ld = M;
  a.sB = ws; a.sB_o = 1; a.sB_c = K / kG; a.sbE = (N / kG) * (K / kG);
  a.C = dx; a.ldc = K;
  a.M = (int)M; a.N = (int)K; a.Kc = (int)N;
  a.seg = seg_off; a.E = (int)E; a.seg_rows = (int)M;
  return hip_status(jet::launch_gemm_grouped(a, jet::kGrpRows, jet::kRowBlock,
                                             dx_dtype == JET_BF16 ? jet::kOutBf16 : jet::kOutF32,
                                             false, false, as_stream(stream), p2),
                    name);
}

int jet_fp8_grouped_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wqT, const float* ws,
                          const int32_t* seg_off, int64_t E, int64_t M, int64_t N, int64_t K,
                          void* dx, int dx_dtype, void* workspace, size_t ws_bytes, void* stream) {
  return grouped_dgrad("fp8_grouped_dgrad", false, dyq, dys, wqT, ws, seg_off, E, M, N, K, dx, dx_dtype,
                       workspace, ws_bytes, stream);
}

int jet_fp8_grouped_dgrad_pow2(const uint8_t* dyq, const float* dys, const uint8_t* wqT, const float* ws,
                               const int32_t* seg_off, int64_t E, int64_t M, int64_t N, int64_t K,
                               void* dx, int dx_dtype, void* stream) {
  return grouped_dgrad("fp8_grouped_dgrad_pow2", true, dyq, dys, wqT, ws, seg_off, E, M, N, K, dx, dx_dtype,
                       nullptr, 0, stream);
}

static int grouped_wgrad(const char* name, bool p2, const uint8_t* dyqT, const float* dysT, const uint8_t* xqT,
                         const float* xsT, int64_t ldT, const int32_t* seg_off, int64_t E, int64_t M, int64_t N,
                         int64_t K, void* dw, int dw_dtype, int accumulate, void* workspace, size_t ws_bytes,
                         void* stream) {
  g_last_error[0] = 0;
  if (int st = check_grouped_common(name, seg_off, E, M)) return st;
  if (int st = check_gemm_common(name, M, N, K, 0, ws_bytes, workspace)) return st;
  if (dw_dtype != JET_F32 && dw_dtype != JET_BF16)
    return fail(JET_ERR_DTYPE, "%s: dw_dtype must be JET_F32 or JET_BF16", name);
  if (accumulate && dw_dtype != JET_F32)
    return fail(JET_ERR_DTYPE, "%s: accumulate needs dw_dtype JET_F32", name);
  if (N == 0 || K == 0) return JET_OK;
  if (!dw) return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (M > 0 && (!dyqT || !dysT || !xqT || !xsT))
    return fail(JET_ERR_NULL, "%s: null pointer", name);
  if (ldT < grouped_cols(M, E) || ldT > kMaxLd || ldT % 16)
    return fail(JET_ERR_SHAPE, "%s: need 128*(ceil(M/128)+E) <= ldT <= 2^24, ldT %% 16", name);
  if (!aligned(dw, 16) || (M > 0 && (!aligned(dyqT, 16) || !aligned(xqT, 16) || !aligned(dysT, 4) ||
                                     !aligned(xsT, 4))))
    return fail(JET_ERR_ALIGN, "%s: operands and output need 16-byte alignment", name);
  jet::GemmArgs a{};
  a.A = dyqT; a.lda = ldT;
  a.B = xqT; a.ldb = ldT;
  a.sA = dysT; a.sA_ld = N;
  a.sB = xsT; a.sB_o = 1; a.sB_c = K;
  a.C = dw; a.ldc = K; a.cE = N * K;
  a.M = (int)N; a.N = (int)K; a.Kc = 0;
  a.seg = seg_off; a.E = (int)E; a.seg_rows = (int)M; a.kcap = (int)(ldT / kG * kG);
  return hip_status(jet::launch_gemm_grouped(a, jet::kGrpContraction, jet::kRowCol,
                                             dw_dtype == JET_BF16 ? jet::kOutBf16 : jet::kOutF32,
                                             accumulate != 0, false, as_stream(stream), p2),
                    name);
}

int jet_fp8_grouped_wgrad(const uint8_t* dyqT, const float* dysT, const uint8_t* xqT,
                          const float* xsT, int64_t ldT, const int32_t* seg_off, int64_t E,
                          int64_t M, int64_t N, int64_t K, void* dw, int dw_dtype, int accumulate,
                          void* workspace, size_t ws_bytes, void* stream) {
  return grouped_wgrad("fp8_grouped_wgrad", false, dyqT, dysT, xqT, xsT, ldT, seg_off, E, M, N, K, dw, dw_dtype,
                       accumulate, workspace, ws_bytes, stream);
}

int jet_fp8_grouped_wgrad_pow2(const uint8_t* dyqT, const float* dysT, const uint8_t* xqT,
                               const float* xsT, int64_t ldT, const int32_t* seg_off, int64_t E,
                               int64_t M, int64_t N, int64_t K, void* dw, int dw_dtype, int accumulate,
                               void* stream) {
  return grouped_wgrad("fp8_grouped_wgrad_pow2", true, dyqT, dysT, xqT, xsT, ldT, seg_off, E, M, N, K, dw,
                       dw_dtype, accumulate, nullptr, 0, stream);
}

}  // extern "C"
