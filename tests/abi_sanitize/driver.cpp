// Host-side run of the C-ABI layer (csrc/api.hip) under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU. The kernel launchers are replaced by stubs that record the
// request, so every entry point's validation, size arithmetic and argument marshalling runs for
// valid calls as well as invalid ones; the buffers are host memory that nothing dereferences (the
// layer never touches device pointers). Extreme sizes exercise the overflow guards.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/bitlinear.h"
#include "../../ternary_weight_quantized_amd/csrc/bl_kernels.h"

namespace {
int g_launches = 0;
long g_M = -1, g_K = -1, g_N = -1;
void note(long M, long K, long N) { ++g_launches; g_M = M; g_K = K; g_N = N; }
}  // namespace

hipError_t bl_launch_quantize(const void*, int, int M, int K, long, int, int, float, const float*, void*, float*,
                              uint32_t*, hipStream_t) { note(M, K, -1); return hipSuccess; }
hipError_t bl_launch_quantize_per_tensor(const void*, int, int M, int K, long, int, float, void*, void*, float*,
                                         hipStream_t) { note(M, K, -1); return hipSuccess; }
hipError_t bl_launch_pack(const float*, int N, int K, float, void*, float*, void*, int, hipStream_t) {
  note(-1, K, N); return hipSuccess;
}
hipError_t bl_launch_gemm(const bl_mm_args& a, hipStream_t) { note(a.M, a.K, a.N); return hipSuccess; }
hipError_t bl_launch_gemm_kv(const bl_mm_args& a, const bl_kv_epi&, hipStream_t) { note(a.M, a.K, a.N); return hipSuccess; }
hipError_t bl_launch_gemv(const bl_mm_args& a, hipStream_t) { note(a.M, a.K, a.N); return hipSuccess; }
hipError_t bl_launch_fill_zero(float*, long n, hipStream_t) { note(n, -1, -1); return hipSuccess; }
hipError_t bl_launch_glu_conditional_fused(const bl_upcond_args& a, const void*, const float*, hipStream_t) {
  note(a.M, a.K, a.N); return hipSuccess;
}
hipError_t bl_launch_kv_quant(const bl_kv_args&, hipStream_t) { note(-1, -1, -1); return hipSuccess; }
hipError_t bl_launch_calib_mfma(int blocks, int iters, float*, hipStream_t) { note(blocks, iters, -1); return hipSuccess; }
hipError_t bl_launch_calib_read(const void*, long bytes, void*, hipStream_t) { note(bytes, -1, -1); return hipSuccess; }

namespace {
int g_checks = 0, g_fails = 0;
alignas(256) unsigned char g_buf[1 << 16];
void* const P = g_buf + 256;          // 16-byte aligned stand-ins for device pointers
void* const PM = g_buf + 260;         // misaligned
float* const F = reinterpret_cast<float*>(g_buf + 512);
const int64_t BIG = INT64_MAX / 2;

void expect(bl_status got, bl_status want, bool launches, const char* what, int line) {
  ++g_checks;
  static int last = 0;
  const bool launched = g_launches != last;
  last = g_launches;
  if (got != want || launched != launches) {
    ++g_fails;
    std::printf("FAIL line %d %s: status %d (want %d), launched %d (want %d)\n", line, what, (int)got, (int)want,
                (int)launched, (int)launches);
  }
}
#define OK(expr) expect((expr), BL_OK, true, #expr, __LINE__)
#define ERR(expr, st) expect((expr), (st), false, #expr, __LINE__)
}  // namespace

int main() {
  const float eps = 1e-5f;
  // ---- quantize_act
  OK(bitlinear_quantize_act(P, BL_IN_BF16, 4, 256, 256, BL_ACT_INT4, -1, eps, nullptr, P, F, nullptr, nullptr));
  OK(bitlinear_quantize_act(P, BL_IN_F32, 7, 384, 384, BL_ACT_INT4_E3M2, -1, eps, nullptr, P, F, nullptr, nullptr));
  OK(bitlinear_quantize_act(P, BL_IN_BF16, 3, 4096, 4096, BL_ACT_INT8, 2048, eps, nullptr, P, F,
                            reinterpret_cast<uint32_t*>(P), nullptr));
  OK(bitlinear_quantize_act(P, BL_IN_F32, 2048, 11008, 11008, BL_ACT_INT8, -1, eps, F, P, F, nullptr, nullptr));
  OK(bitlinear_quantize_act(P, BL_IN_BF16, 1, 262016, 262016, BL_ACT_FP4_E2M1_POW2, -1, eps, nullptr, P, F, nullptr,
                            nullptr));
  ERR(bitlinear_quantize_act(nullptr, 0, 4, 256, 256, 0, -1, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_quantize_act(P, 0, 4, 256, 256, 0, -1, 0.0f, nullptr, P, F, nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_quantize_act(P, 0, 4, 256, 256, 0, -1, NAN, nullptr, P, F, nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_quantize_act(P, 0, 4, 100, 100, 0, -1, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_quantize_act(P, 0, BIG, 4096, 4096, 0, -1, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_quantize_act(P, 0, 4, BIG & ~int64_t(127), BIG, 0, -1, eps, nullptr, P, F, nullptr, nullptr),
      BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_quantize_act(P, 0, 4, 256, BIG, 0, -1, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_quantize_act(P, 0, -4, 256, 256, 0, -1, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_quantize_act(P, 0, 4, 256, 256, 2, 257, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_quantize_act(PM, 0, 4, 256, 256, 0, -1, eps, nullptr, P, F, nullptr, nullptr), BL_ERR_MISALIGNED);
  // ---- per tensor (caller workspace, then the allocation-free form: no device here, so it fails cleanly)
  const size_t ws = bitlinear_quantize_per_tensor_workspace_bytes(64);
  OK(bitlinear_quantize_act_per_tensor(P, 0, 64, 4096, 4096, BL_ACT_INT4, eps, P, ws, P, F, nullptr));
  ERR(bitlinear_quantize_act_per_tensor(P, 0, 64, 4096, 4096, BL_ACT_INT4, eps, P, ws - 1, P, F, nullptr),
      BL_ERR_WORKSPACE_TOO_SMALL);
  ERR(bitlinear_quantize_act_per_tensor(P, 0, BIG, 4096, 4096, BL_ACT_INT4, eps, P, SIZE_MAX, P, F, nullptr),
      BL_ERR_UNSUPPORTED_SHAPE);
  {
    const bl_status s = bitlinear_quantize_act_per_tensor_noalloc(P, 0, 64, 4096, 4096, BL_ACT_INT4, eps, P, F, nullptr);
    expect(s == BL_OK ? BL_ERR_HIP : s, BL_ERR_HIP, false, "noalloc without a device", __LINE__);
  }
  ERR(bitlinear_quantize_act_per_tensor_noalloc(P, 0, BITLINEAR_NOALLOC_MAX_M + 1, 4096, 4096, 0, eps, P, F, nullptr),
      BL_ERR_WORKSPACE_TOO_SMALL);
  // ---- pack
  OK(bitlinear_pack_ternary(F, 32, 256, eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr));
  OK(bitlinear_pack_ternary_rows(F, 11008, 4096, eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr));
  OK(bitlinear_pack_ternary_a8(F, 4096, 11008 & ~int64_t(127), eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr));
  ERR(bitlinear_pack_ternary_a8(F, 24, 256, eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_pack_ternary_a8(nullptr, 32, 256, eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr),
      BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_pack_ternary(F, 10, 256, eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_pack_ternary(F, BIG & ~int64_t(15), 256, eps, P, F, P, bitlinear_pack_workspace_bytes(), nullptr),
      BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_pack_ternary(F, 32, 256, eps, P, F, P, 8, nullptr), BL_ERR_WORKSPACE_TOO_SMALL);
  // ---- matmuls
  bl_epilogue res{BL_EPI_RESIDUAL, F, 32, nullptr, nullptr, nullptr};
  bl_epilogue glu{BL_EPI_RELU2_GLU, nullptr, 0, P, F, F};
  OK(bitlinear_gemm_w158a4(BL_ACT_INT4_E3M2, P, F, 4096, 4096, P, F, 12288, F, 12288, nullptr, nullptr));
  OK(bitlinear_gemm_w158a4(BL_ACT_INT4, P, F, 7, 384, P, F, 32, F, 32, &res, nullptr));
  OK(bitlinear_gemm_w158a4(BL_ACT_FP4_E2M1, P, F, 2048, 4096, P, F, 11008, F, 11008, &glu, nullptr));
  bl_epilogue res_wide{BL_EPI_RESIDUAL, F, 4096, nullptr, nullptr, nullptr};
  OK(bitlinear_gemm_w158a8_sparse(P, F, 8192, 4096, P, F, 4096, F, 4096, &res_wide, nullptr));
  ERR(bitlinear_gemm_w158a8_sparse(P, F, 8192, 4096, P, F, 4096, F, 4096, &res, nullptr), BL_ERR_INVALID_ARGUMENT);
  OK(bitlinear_gemv_decode(BL_ACT_INT4, P, F, 8, 4096, P, F, 11008, F, 11008, &glu, nullptr));
  OK(bitlinear_gemv_decode(BL_ACT_INT8, P, F, 1, 11008, P, F, 4096, F, 4096, nullptr, nullptr));
  ERR(bitlinear_gemm_w158a4(BL_ACT_INT4, P, F, 4, 262144, P, F, 32, F, 32, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_gemm_w158a4(BL_ACT_INT4, P, F, BIG, 256, P, F, 32, F, 32, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_gemm_w158a4(BL_ACT_INT4, P, F, 4, 256, P, F, BIG & ~int64_t(15), F, BIG, nullptr, nullptr),
      BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_gemm_w158a4(BL_ACT_INT4, P, F, 4, 256, P, F, 32, F, 16, nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_gemm_w158a4(BL_ACT_INT8, P, F, 4, 256, P, F, 32, F, 32, nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_gemv_decode(BL_ACT_INT4, P, F, 9, 4096, P, F, 32, F, 32, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_gemm_w158a8_sparse(PM, F, 4, 256, P, F, 32, F, 32, nullptr, nullptr), BL_ERR_MISALIGNED);
  // ---- conditional GLU
  OK(bitlinear_gemv_decode_glu_conditional(P, F, 1, 4096, P, F, P, F, 11008, F, 11008, F, 11008, F, nullptr));
  ERR(bitlinear_gemv_decode_glu_conditional(P, F, 1, 4096, P, F, P, F, 11008, F, 11008, F, 11000, F, nullptr),
      BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_gemv_decode_glu_conditional(P, F, 1, 4096, P, F, nullptr, F, 11008, F, 11008, F, 11008, F, nullptr),
      BL_ERR_INVALID_ARGUMENT);
  // ---- KV cache
  const int32_t* pos = reinterpret_cast<const int32_t*>(P);
  OK(bitlinear_kv_quantize(P, BL_IN_F32, 4096, 32, 128, 12288, pos, F, F, 1024, 4, eps, P, F, nullptr, 0, nullptr,
                           nullptr, nullptr));
  OK(bitlinear_kv_quantize(P, BL_IN_BF16, 5, 3, 64, 192, nullptr, nullptr, nullptr, 0, 3, eps, P, F, pos, 2, P, F,
                           nullptr));
  expect(bitlinear_kv_quantize(nullptr, BL_IN_F32, 0, 32, 128, 4096, nullptr, nullptr, nullptr, 0, 3, eps, nullptr,
                               nullptr, nullptr, 0, nullptr, nullptr, nullptr),
         BL_OK, false, "empty KV input: nothing enqueued", __LINE__);
  ERR(bitlinear_kv_quantize(P, BL_IN_F32, 16, 2, 96, 192, nullptr, nullptr, nullptr, 0, 4, eps, P, F, nullptr, 0,
                            nullptr, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_kv_quantize(P, BL_IN_F32, BIG, 32, 128, 4096, nullptr, nullptr, nullptr, 0, 4, eps, P, F, nullptr, 0,
                            nullptr, nullptr, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_kv_quantize(P, BL_IN_F32, 16, 2, 128, 256, pos, F, nullptr, 64, 4, eps, P, F, nullptr, 0, nullptr,
                            nullptr, nullptr), BL_ERR_INVALID_ARGUMENT);
  // ---- fused QKV + KV
  bl_kv_epilogue kv{};
  kv.H = 32; kv.eps = eps; kv.bits[0] = 4; kv.bits[1] = 3; kv.bits[2] = 3;
  for (int p = 0; p < 3; ++p) { kv.d_codes[p] = P; kv.d_scale[p] = F; kv.d_bos_codes[p] = P; kv.d_bos_scale[p] = F; }
  kv.d_pos = pos; kv.d_cos = F; kv.d_sin = F; kv.P = 1024; kv.d_bos_slot = pos; kv.n_bos_slots = 4;
  OK(bitlinear_gemm_w158a4_kv(BL_ACT_INT4_E3M2, P, F, 4096, 4096, P, F, 12288, nullptr, 0, &kv, nullptr));
  OK(bitlinear_gemm_w158a4_kv(BL_ACT_FP4_E2M1, P, F, 4096, 4096, P, F, 12288, F, 12288, &kv, nullptr));
  ERR(bitlinear_gemm_w158a4_kv(BL_ACT_INT4, P, F, 4096, 4096, P, F, 12288, nullptr, 0, &kv, nullptr),
      BL_ERR_INVALID_ARGUMENT);
  ERR(bitlinear_gemm_w158a4_kv(BL_ACT_INT4_E3M2, P, F, 4096, 4096, P, F, 12160, nullptr, 0, &kv, nullptr),
      BL_ERR_UNSUPPORTED_SHAPE);
  ERR(bitlinear_gemm_w158a4_kv(BL_ACT_INT4_E3M2, P, F, 4096, 4096, P, F, 12288, nullptr, 0, nullptr, nullptr),
      BL_ERR_INVALID_ARGUMENT);
  // ---- measurement aids and helpers
  OK(bitlinear_calibrate_mfma(512, 10, F, nullptr));
  ERR(bitlinear_calibrate_mfma(0, 10, F, nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  OK(bitlinear_calibrate_read(P, 1 << 20, reinterpret_cast<uint32_t*>(F), nullptr));
  ERR(bitlinear_calibrate_read(P, BIG, reinterpret_cast<uint32_t*>(F), nullptr), BL_ERR_UNSUPPORTED_SHAPE);
  for (int32_t op = -2; op < 12; ++op)
    for (int64_t m : {int64_t(0), int64_t(1), int64_t(4096), BIG}) (void)bitlinear_workspace_size(op, m, m, m);
  for (int32_t st = -1; st < 8; ++st) (void)std::strlen(bitlinear_status_string(st));
  (void)bitlinear_packed_bytes(BIG, BIG);
  (void)bitlinear_quantize_per_tensor_workspace_bytes(BIG);
  ++g_checks;
  if (bitlinear_abi_version() != BITLINEAR_ABI_VERSION) { ++g_fails; std::printf("FAIL abi version\n"); }
  std::printf("abi sanitize: %d checks, %d failures\n", g_checks, g_fails);
  return g_fails ? 1 : 0;
}
