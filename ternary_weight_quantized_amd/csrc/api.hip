// C-ABI layer: host-side argument validation, then kernel launches on the caller's stream.
// Nothing is enqueued when validation fails; the library never allocates device memory.
#include <cmath>
#include <mutex>
#include <cstdint>
#include <cstddef>

#include "bl_kernels.h"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0u; }
inline bool eps_ok(float eps) { return std::isfinite(eps) && eps > 0.0f; }
constexpr int64_t kMaxElems = (int64_t)1 << 31;
// Longest reduction the matmuls accept. The int8-core INT4 path holds 1024 * sum(c t) in int32
// (|c| <= 8, |t| <= 1), so K * 8 * 1024 must stay below 2^31; the INT8 path (64 * 127 per term) and
// the fp32 sums of the FP6 / FP4 paths (exact below 2^24) have more room.
constexpr int64_t kMaxMatmulK = ((int64_t)1 << 18) - 128;
// a * b < kMaxElems for non-negative a and b, decided without forming a product that can overflow
bool fits(int64_t a, int64_t b) { return a >= 0 && b >= 0 && (a == 0 || b <= (kMaxElems - 1) / a); }

bl_status hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

// Validation shared by the three matmul entry points.
bl_status check_mm(int32_t fmt, const void* codes, const float* scale, int64_t M, int64_t K, const void* packed,
                   const float* alpha, int64_t N, const float* y, int64_t ldy, const bl_epilogue* epi,
                   bool y_optional = false) {
  if (!codes || !scale || !packed || !alpha || (!y && !y_optional)) return BL_ERR_INVALID_ARGUMENT;
  if (fmt != BL_ACT_INT4 && fmt != BL_ACT_FP4_E2M1 && fmt != BL_ACT_INT8 && fmt != BL_ACT_INT4_E3M2)
    return BL_ERR_INVALID_ARGUMENT;
  if (M < 1 || K < 1 || N < 1) return BL_ERR_UNSUPPORTED_SHAPE;
  if (K % 128 != 0 || N % 16 != 0 || K > kMaxMatmulK) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!fits(M, K) || !fits(N, K) || !fits(M, N)) return BL_ERR_UNSUPPORTED_SHAPE;
  if (y && ldy < N) return BL_ERR_INVALID_ARGUMENT;
  if (!aligned16(codes) || !aligned16(packed)) return BL_ERR_MISALIGNED;
  if (y && (!aligned16(y) || ldy % 4 != 0)) return BL_ERR_MISALIGNED;              // ldy * 4 bytes, a multiple of 16
  if (epi) {
    if (epi->kind == BL_EPI_RESIDUAL) {
      if (!epi->d_residual) return BL_ERR_INVALID_ARGUMENT;
      if (epi->ldr < N) return BL_ERR_INVALID_ARGUMENT;
      if (!aligned16(epi->d_residual) || epi->ldr % 4 != 0) return BL_ERR_MISALIGNED;
    } else if (epi->kind == BL_EPI_RELU2_GLU) {
      if (!epi->d_up_packed || !epi->d_up_alpha) return BL_ERR_INVALID_ARGUMENT;
      if (!aligned16(epi->d_up_packed)) return BL_ERR_MISALIGNED;
    } else if (epi->kind != BL_EPI_NONE) {
      return BL_ERR_INVALID_ARGUMENT;
    }
  }
  return BL_OK;
}

bl_mm_args make_args(int32_t fmt, const void* codes, const float* scale, int64_t M, int64_t K, const void* packed,
                     const float* alpha, int64_t N, float* y, int64_t ldy, const bl_epilogue* epi) {
  bl_mm_args a{};
  a.fmt = fmt; a.A = codes; a.ascale = scale; a.M = (int)M; a.K = (int)K; a.N = (int)N;
  a.W = packed; a.walpha = alpha; a.Y = y; a.ldy = (long)ldy;
  a.epi = epi ? epi->kind : BL_EPI_NONE;
  a.R = nullptr; a.ldr = 0; a.W2 = nullptr; a.w2alpha = nullptr; a.rowmax = nullptr;
  if (epi && epi->kind == BL_EPI_RESIDUAL) { a.R = epi->d_residual; a.ldr = (long)epi->ldr; }
  if (epi && epi->kind == BL_EPI_RELU2_GLU) { a.W2 = epi->d_up_packed; a.w2alpha = epi->d_up_alpha; a.rowmax = epi->d_row_absmax; }
  return a;
}

}  // namespace

extern "C" {

int32_t bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

const char* bitlinear_status_string(int32_t s) {
  switch (s) {
    case BL_OK: return "ok";
    case BL_ERR_INVALID_ARGUMENT: return "invalid argument";
    case BL_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case BL_ERR_MISALIGNED: return "misaligned pointer or stride";
    case BL_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case BL_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  if (!fits(N, K)) return SIZE_MAX;               // beyond every accepted shape
  return (size_t)(N * K / 4);
}

size_t bitlinear_pack_workspace_bytes(void) { return 256 * sizeof(unsigned long long); }

size_t bitlinear_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K) {
  (void)N; (void)K;
  switch (op) {
    case BL_OP_QUANTIZE_ACT:
    case BL_OP_GEMM_W158A4:
    case BL_OP_GEMM_W158A8_SPARSE:
    case BL_OP_GEMV_DECODE:
    case BL_OP_GEMV_DECODE_GLU_CONDITIONAL:
    case BL_OP_KV_QUANTIZE:
      return 0;
    case BL_OP_QUANTIZE_ACT_PER_TENSOR:
      return bitlinear_quantize_per_tensor_workspace_bytes(M);
    case BL_OP_PACK_TERNARY:
    case BL_OP_PACK_TERNARY_ROWS:
    case BL_OP_PACK_TERNARY_A8:
      return bitlinear_pack_workspace_bytes();
    default:
      return SIZE_MAX;
  }
}

bl_status bitlinear_quantize_act(const void* d_x, int32_t in_dtype, int64_t M, int64_t K, int64_t ldx, int32_t fmt,
                                 int32_t topk_keep, float eps, const float* d_row_absmax_hint, void* d_codes,
                                 float* d_scale, uint32_t* d_mask, void* stream) {
  if (!d_x || !d_codes || !d_scale) return BL_ERR_INVALID_ARGUMENT;
  if (in_dtype != BL_IN_BF16 && in_dtype != BL_IN_F32) return BL_ERR_INVALID_ARGUMENT;
  if (fmt != BL_ACT_INT4 && fmt != BL_ACT_FP4_E2M1 && fmt != BL_ACT_INT8 && fmt != BL_ACT_INT4_E3M2 &&
      fmt != BL_ACT_FP4_E2M1_POW2)
    return BL_ERR_INVALID_ARGUMENT;
  if (!eps_ok(eps)) return BL_ERR_INVALID_ARGUMENT;
  if (M < 1 || K < 1) return BL_ERR_UNSUPPORTED_SHAPE;
  if (K % 128 != 0) return BL_ERR_UNSUPPORTED_SHAPE;
  if (ldx < K) return BL_ERR_INVALID_ARGUMENT;
  if (!fits(M, K) || !fits(M, ldx)) return BL_ERR_UNSUPPORTED_SHAPE;
  if (fmt != BL_ACT_INT8 && (topk_keep >= 0 || d_mask)) return BL_ERR_INVALID_ARGUMENT;
  if (topk_keep > K) return BL_ERR_INVALID_ARGUMENT;
  const int64_t esz = in_dtype == BL_IN_F32 ? 4 : 2;
  if (!aligned16(d_x) || !aligned16(d_codes) || ldx % (16 / esz) != 0) return BL_ERR_MISALIGNED;
  if (d_mask && !aligned16(d_mask)) return BL_ERR_MISALIGNED;
  const float* hint = (fmt == BL_ACT_INT4 || fmt == BL_ACT_INT4_E3M2) ? nullptr : d_row_absmax_hint;
  return hip_status(bl_launch_quantize(d_x, in_dtype == BL_IN_F32, (int)M, (int)K, (long)ldx, fmt, (int)topk_keep,
                                       eps, hint, d_codes, d_scale, d_mask, static_cast<hipStream_t>(stream)));
}

size_t bitlinear_quantize_per_tensor_workspace_bytes(int64_t M) {
  if (M <= 0) return 0;
  if (M >= kMaxElems) return SIZE_MAX;            // beyond every accepted shape
  return bl_quantize_per_tensor_ws_bytes((long)M);
}

}  // extern "C"

namespace {

// Validation of the per-tensor quantizer's arguments other than the workspace.
bl_status check_per_tensor(const void* d_x, int32_t in_dtype, int64_t M, int64_t K, int64_t ldx, int32_t fmt,
                           float eps, const void* d_codes, const float* d_scale) {
  if (!d_x || !d_codes || !d_scale) return BL_ERR_INVALID_ARGUMENT;
  if (in_dtype != BL_IN_BF16 && in_dtype != BL_IN_F32) return BL_ERR_INVALID_ARGUMENT;
  if (fmt != BL_ACT_INT4 && fmt != BL_ACT_FP4_E2M1 && fmt != BL_ACT_INT8 && fmt != BL_ACT_INT4_E3M2 &&
      fmt != BL_ACT_FP4_E2M1_POW2)
    return BL_ERR_INVALID_ARGUMENT;
  if (!eps_ok(eps)) return BL_ERR_INVALID_ARGUMENT;
  if (M < 1 || K < 1) return BL_ERR_UNSUPPORTED_SHAPE;
  if (K % 128 != 0) return BL_ERR_UNSUPPORTED_SHAPE;
  if (ldx < K) return BL_ERR_INVALID_ARGUMENT;
  if (!fits(M, K) || !fits(M, ldx)) return BL_ERR_UNSUPPORTED_SHAPE;
  const int64_t esz = in_dtype == BL_IN_F32 ? 4 : 2;
  if (!aligned16(d_x) || !aligned16(d_codes) || ldx % (16 / esz) != 0) return BL_ERR_MISALIGNED;
  return BL_OK;
}

// Scratch of the allocation-free per-tensor quantizer: one fixed array per device, the workspace of
// at most BITLINEAR_NOALLOC_MAX_M rows. Host code never uses the array's name as an address: each
// device's address comes from hipGetSymbolAddress, looked up once per device on its first call.
constexpr size_t kNoallocScratchBytes = bl_quantize_per_tensor_ws_bytes(BITLINEAR_NOALLOC_MAX_M);
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];          // device address of `scratch` on each device (null: not looked up)

// Address of the current device's scratch array, looked up (once per device) with that device current.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

bl_status bitlinear_quantize_act_per_tensor(const void* d_x, int32_t in_dtype, int64_t M, int64_t K, int64_t ldx,
                                            int32_t fmt, float eps, void* d_workspace, size_t ws_bytes,
                                            void* d_codes, float* d_scale, void* stream) {
  if (!d_workspace) return BL_ERR_INVALID_ARGUMENT;
  const bl_status s = check_per_tensor(d_x, in_dtype, M, K, ldx, fmt, eps, d_codes, d_scale);
  if (s != BL_OK) return s;
  if (ws_bytes < bitlinear_quantize_per_tensor_workspace_bytes(M)) return BL_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(d_workspace)) return BL_ERR_MISALIGNED;
  return hip_status(bl_launch_quantize_per_tensor(d_x, in_dtype == BL_IN_F32, (int)M, (int)K, (long)ldx, fmt, eps,
                                                  d_workspace, d_codes, d_scale, static_cast<hipStream_t>(stream)));
}

size_t bitlinear_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

bl_status bitlinear_quantize_act_per_tensor_noalloc(const void* d_x, int32_t in_dtype, int64_t M, int64_t K,
                                                    int64_t ldx, int32_t fmt, float eps, void* d_codes,
                                                    float* d_scale, void* stream) {
  const bl_status s = check_per_tensor(d_x, in_dtype, M, K, ldx, fmt, eps, d_codes, d_scale);
  if (s != BL_OK) return s;
  if (M > BITLINEAR_NOALLOC_MAX_M) return BL_ERR_WORKSPACE_TOO_SMALL;   // beyond the fixed scratch
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return BL_ERR_HIP;
  // every workspace slot is rewritten by the call (nothing needs clearing); no allocation happens
  return hip_status(bl_launch_quantize_per_tensor(d_x, in_dtype == BL_IN_F32, (int)M, (int)K, (long)ldx, fmt, eps,
                                                  ws, d_codes, d_scale, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_pack_ternary(const float* d_w, int64_t N, int64_t K, float eps, void* d_packed, float* d_alpha,
                                 void* d_workspace, size_t ws_bytes, void* stream) {
  if (!d_w || !d_packed || !d_alpha || !d_workspace) return BL_ERR_INVALID_ARGUMENT;
  if (!eps_ok(eps)) return BL_ERR_INVALID_ARGUMENT;
  if (N < 1 || K < 1 || K % 128 != 0 || N % 16 != 0) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!fits(N, K)) return BL_ERR_UNSUPPORTED_SHAPE;
  if (ws_bytes < bitlinear_pack_workspace_bytes()) return BL_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(d_w) || !aligned16(d_packed) || !aligned16(d_workspace)) return BL_ERR_MISALIGNED;
  return hip_status(bl_launch_pack(d_w, (int)N, (int)K, eps, d_packed, d_alpha, d_workspace, BL_PACK_TILES,
                                   static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_pack_ternary_a8(const float* d_w, int64_t N, int64_t K, float eps, void* d_packed, float* d_alpha,
                                    void* d_workspace, size_t ws_bytes, void* stream) {
  if (!d_w || !d_packed || !d_alpha || !d_workspace) return BL_ERR_INVALID_ARGUMENT;
  if (!eps_ok(eps)) return BL_ERR_INVALID_ARGUMENT;
  if (N < 1 || K < 1 || K % 128 != 0 || N % 16 != 0) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!fits(N, K)) return BL_ERR_UNSUPPORTED_SHAPE;
  if (ws_bytes < bitlinear_pack_workspace_bytes()) return BL_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(d_w) || !aligned16(d_packed) || !aligned16(d_workspace)) return BL_ERR_MISALIGNED;
  return hip_status(bl_launch_pack(d_w, (int)N, (int)K, eps, d_packed, d_alpha, d_workspace, BL_PACK_TILES_A8,
                                   static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_pack_ternary_rows(const float* d_w, int64_t N, int64_t K, float eps, void* d_packed,
                                      float* d_alpha, void* d_workspace, size_t ws_bytes, void* stream) {
  if (!d_w || !d_packed || !d_alpha || !d_workspace) return BL_ERR_INVALID_ARGUMENT;
  if (!eps_ok(eps)) return BL_ERR_INVALID_ARGUMENT;
  if (N < 1 || K < 1 || K % 128 != 0 || N % 16 != 0) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!fits(N, K)) return BL_ERR_UNSUPPORTED_SHAPE;
  if (ws_bytes < bitlinear_pack_workspace_bytes()) return BL_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(d_w) || !aligned16(d_packed) || !aligned16(d_workspace)) return BL_ERR_MISALIGNED;
  return hip_status(bl_launch_pack(d_w, (int)N, (int)K, eps, d_packed, d_alpha, d_workspace, BL_PACK_ROWS,
                                   static_cast<hipStream_t>(stream)));
}

static bl_status run_mm(bool decode, int32_t fmt, const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                        const void* d_packed, const float* d_alpha, int64_t N, float* d_y, int64_t ldy,
                        const bl_epilogue* h_epi, void* stream) {
  const hipStream_t st = static_cast<hipStream_t>(stream);
  bl_mm_args a = make_args(fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi);
  if (a.rowmax) {
    const hipError_t e = bl_launch_fill_zero(a.rowmax, (long)M, st);
    if (e != hipSuccess) return BL_ERR_HIP;
  }
  return hip_status(decode ? bl_launch_gemv(a, st) : bl_launch_gemm(a, st));
}

bl_status bitlinear_gemm_w158a4(int32_t fmt, const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                const void* d_packed, const float* d_alpha, int64_t N, float* d_y, int64_t ldy,
                                const bl_epilogue* h_epi, void* stream) {
  const bl_status s = check_mm(fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi);
  if (s != BL_OK) return s;
  if (fmt != BL_ACT_INT4 && fmt != BL_ACT_FP4_E2M1 && fmt != BL_ACT_INT4_E3M2) return BL_ERR_INVALID_ARGUMENT;
  return run_mm(false, fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi, stream);
}

bl_status bitlinear_gemm_w158a8_sparse(const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                       const void* d_packed, const float* d_alpha, int64_t N, float* d_y,
                                       int64_t ldy, const bl_epilogue* h_epi, void* stream) {
  const bl_status s = check_mm(BL_ACT_INT8, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi);
  if (s != BL_OK) return s;
  return run_mm(false, BL_ACT_INT8, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi, stream);
}

bl_status bitlinear_gemv_decode(int32_t fmt, const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                const void* d_packed, const float* d_alpha, int64_t N, float* d_y, int64_t ldy,
                                const bl_epilogue* h_epi, void* stream) {
  const bl_status s = check_mm(fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi);
  if (s != BL_OK) return s;
  if (fmt != BL_ACT_INT4 && fmt != BL_ACT_INT8) return BL_ERR_INVALID_ARGUMENT;
  if (M > 8) return BL_ERR_UNSUPPORTED_SHAPE;
  return run_mm(true, fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, h_epi, stream);
}

bl_status bitlinear_gemv_decode_glu_conditional(const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                                const void* d_gate_packed, const float* d_gate_alpha,
                                                const void* d_up_rows, const float* d_up_alpha, int64_t N,
                                                float* d_gate, int64_t ldg, float* d_h, int64_t ldh,
                                                float* d_row_absmax, void* stream) {
  const bl_status s = check_mm(BL_ACT_INT4, d_codes, d_scale, M, K, d_gate_packed, d_gate_alpha, N, d_gate, ldg,
                               nullptr);
  if (s != BL_OK) return s;
  if (!d_up_rows || !d_up_alpha || !d_h) return BL_ERR_INVALID_ARGUMENT;
  if (ldh < N) return BL_ERR_INVALID_ARGUMENT;
  if (M > 8) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(d_up_rows) || !aligned16(d_h) || ldh % 4 != 0) return BL_ERR_MISALIGNED;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_row_absmax) {
    const hipError_t e = bl_launch_fill_zero(d_row_absmax, (long)M, st);
    if (e != hipSuccess) return BL_ERR_HIP;
  }
  bl_upcond_args u{};
  u.A = d_codes; u.ascale = d_scale; u.M = (int)M; u.K = (int)K; u.N = (int)N;
  u.G = d_gate; u.ldg = (long)ldg; u.Wup = d_up_rows; u.upalpha = d_up_alpha;
  u.H = d_h; u.ldh = (long)ldh; u.rowmax = d_row_absmax;
  return hip_status(bl_launch_glu_conditional_fused(u, d_gate_packed, d_gate_alpha, st));
}

bl_status bitlinear_gemm_w158a4_kv(int32_t fmt, const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                   const void* d_packed, const float* d_alpha, int64_t N, float* d_y, int64_t ldy,
                                   const bl_kv_epilogue* h_kv, void* stream) {
  if (!h_kv) return BL_ERR_INVALID_ARGUMENT;
  if (fmt != BL_ACT_INT4_E3M2 && fmt != BL_ACT_FP4_E2M1) return BL_ERR_INVALID_ARGUMENT;
  // the matmul checks (a null y is allowed: the fp32 projection is then not stored)
  const bl_status s = check_mm(fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, ldy, nullptr, true);
  if (s != BL_OK) return s;
  const bl_kv_epilogue& k = *h_kv;
  if (k.H < 1 || k.H > N / 384 || N != 3 * k.H * 128) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!eps_ok(k.eps)) return BL_ERR_INVALID_ARGUMENT;
  bool any3 = false;
  for (int p = 0; p < 3; ++p) {
    if (k.bits[p] != 3 && k.bits[p] != 4) return BL_ERR_INVALID_ARGUMENT;
    if (!k.d_codes[p] || !k.d_scale[p]) return BL_ERR_INVALID_ARGUMENT;
    if (!aligned16(k.d_codes[p])) return BL_ERR_MISALIGNED;
    any3 = any3 || k.bits[p] == 3;
  }
  if ((k.d_cos == nullptr) != (k.d_sin == nullptr)) return BL_ERR_INVALID_ARGUMENT;
  if (k.d_cos && (!k.d_pos || k.P < 1)) return BL_ERR_INVALID_ARGUMENT;
  if (k.d_cos && (!aligned16(k.d_cos) || !aligned16(k.d_sin))) return BL_ERR_MISALIGNED;
  if (k.d_cos && !fits(k.P, 128)) return BL_ERR_UNSUPPORTED_SHAPE;
  if (k.d_bos_slot) {
    if (!any3 || k.n_bos_slots < 1) return BL_ERR_INVALID_ARGUMENT;
    if (!fits(k.n_bos_slots, k.H * 128)) return BL_ERR_UNSUPPORTED_SHAPE;
    for (int p = 0; p < 3; ++p) {
      if (k.bits[p] != 3) continue;
      if (!k.d_bos_codes[p] || !k.d_bos_scale[p]) return BL_ERR_INVALID_ARGUMENT;
      if (!aligned16(k.d_bos_codes[p])) return BL_ERR_MISALIGNED;
    }
  }
  bl_mm_args a = make_args(fmt, d_codes, d_scale, M, K, d_packed, d_alpha, N, d_y, d_y ? ldy : N, nullptr);
  bl_kv_epi e{};
  e.H = (int)k.H; e.eps = k.eps;
  for (int p = 0; p < 3; ++p) {
    e.bits[p] = k.bits[p];
    e.codes[p] = static_cast<uint8_t*>(k.d_codes[p]);
    e.scale[p] = k.d_scale[p];
    e.bos_codes[p] = static_cast<uint8_t*>(k.d_bos_codes[p]);
    e.bos_scale[p] = k.d_bos_scale[p];
  }
  e.pos = k.d_pos; e.cos = k.d_cos; e.sin = k.d_sin; e.P = (int)k.P;
  e.bos_slot = k.d_bos_slot; e.nslots = (int)k.n_bos_slots;
  return hip_status(bl_launch_gemm_kv(a, e, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_kv_quantize(const void* d_x, int32_t in_dtype, int64_t T, int64_t H, int64_t D, int64_t ldx,
                                const int32_t* d_pos, const float* d_cos, const float* d_sin, int64_t P,
                                int32_t bits, float eps, void* d_codes, float* d_scale,
                                const int32_t* d_bos_slot, int64_t n_bos_slots, void* d_bos_codes,
                                float* d_bos_scale, void* stream) {
  if (in_dtype != BL_IN_BF16 && in_dtype != BL_IN_F32) return BL_ERR_INVALID_ARGUMENT;
  if (bits != 3 && bits != 4) return BL_ERR_INVALID_ARGUMENT;
  if (T == 0 && H >= 1 && (D == 64 || D == 128 || D == 256) && eps_ok(eps)) return BL_OK;   // nothing to do
  if (!d_x || !d_codes || !d_scale) return BL_ERR_INVALID_ARGUMENT;
  if (!eps_ok(eps)) return BL_ERR_INVALID_ARGUMENT;
  if ((d_cos == nullptr) != (d_sin == nullptr)) return BL_ERR_INVALID_ARGUMENT;
  if (d_cos && (!d_pos || P < 1)) return BL_ERR_INVALID_ARGUMENT;
  if (d_bos_slot && (bits != 3 || !d_bos_codes || !d_bos_scale || n_bos_slots < 1)) return BL_ERR_INVALID_ARGUMENT;
  if (T < 0 || H < 1 || H >= kMaxElems) return BL_ERR_UNSUPPORTED_SHAPE;
  if (D != 64 && D != 128 && D != 256) return BL_ERR_UNSUPPORTED_SHAPE;
  if (ldx < H * D) return BL_ERR_INVALID_ARGUMENT;
  if (!fits(T, ldx) || !fits(T, H * D) || (d_cos && !fits(P, D)) || (d_bos_slot && !fits(n_bos_slots, H * D)))
    return BL_ERR_UNSUPPORTED_SHAPE;
  const int64_t esz = in_dtype == BL_IN_F32 ? 4 : 2;
  if (!aligned16(d_x) || ldx % (16 / esz) != 0 || !aligned16(d_codes)) return BL_ERR_MISALIGNED;
  if (d_cos && (!aligned16(d_cos) || !aligned16(d_sin))) return BL_ERR_MISALIGNED;
  if (d_bos_slot && !aligned16(d_bos_codes)) return BL_ERR_MISALIGNED;
  bl_kv_args a{};
  a.x = d_x; a.in_f32 = in_dtype == BL_IN_F32; a.T = (int)T; a.H = (int)H; a.D = (int)D; a.ldx = (long)ldx;
  a.pos = d_pos; a.cos = d_cos; a.sin = d_sin; a.P = (int)P; a.bits = bits; a.eps = eps;
  a.codes = d_codes; a.scale = d_scale;
  a.bos_slot = d_bos_slot; a.nslots = (int)n_bos_slots; a.bos_codes = d_bos_codes; a.bos_scale = d_bos_scale;
  return hip_status(bl_launch_kv_quant(a, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_calibrate_read(const void* d_src, int64_t bytes, uint32_t* d_sink, void* stream) {
  if (!d_src || !d_sink) return BL_ERR_INVALID_ARGUMENT;
  if (bytes < 16 || bytes % 16 != 0 || bytes >= kMaxElems) return BL_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(d_src)) return BL_ERR_MISALIGNED;
  return hip_status(bl_launch_calib_read(d_src, (long)bytes, d_sink, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_calibrate_mfma(int32_t blocks, int32_t iters, float* d_out, void* stream) {
  if (!d_out) return BL_ERR_INVALID_ARGUMENT;
  // at most 2^20 steps (about half a second on a full part): a measurement, not a long-running load
  if (blocks < 1 || blocks > 65536 || iters < 0 || iters > (1 << 20)) return BL_ERR_UNSUPPORTED_SHAPE;
  return hip_status(bl_launch_calib_mfma(blocks, iters, d_out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
