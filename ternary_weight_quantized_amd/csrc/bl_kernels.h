// Launchers of the BitLinear kernels (called by the C-ABI layer after argument validation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitlinear.h"

hipError_t bl_launch_quantize(const void* x, int in_f32, int M, int K, long ldx, int fmt, int keep, float eps,
                              const float* hint, void* codes, float* scale, uint32_t* mask, hipStream_t st);

// per-tensor scale variant; ws: 512 block slots of 12 uint64 limb sums, 512 uint32 block maxima, then M floats
constexpr size_t bl_quantize_per_tensor_ws_bytes(long M) { return (size_t)512 * 12 * 8 + 512 * 4 + 4 * (size_t)M; }
hipError_t bl_launch_quantize_per_tensor(const void* x, int in_f32, int M, int K, long ldx, int fmt, float eps,
                                         void* ws, void* codes, float* scale, hipStream_t st);

// packed weight layouts of bl_launch_pack
enum { BL_PACK_TILES = 0, BL_PACK_ROWS = 1, BL_PACK_TILES_A8 = 2 };
hipError_t bl_launch_pack(const float* w, int N, int K, float eps, void* packed, float* alpha,
                          void* ws, int layout, hipStream_t st);

// Arguments shared by the GEMM and the decode GEMV.
struct bl_mm_args {
  int fmt;
  const void* A;
  const float* ascale;
  int M, K, N;
  const void* W;
  const float* walpha;
  float* Y;
  long ldy;
  int epi;
  const float* R;
  long ldr;
  const void* W2;
  const float* w2alpha;
  float* rowmax;
};

hipError_t bl_launch_gemm(const bl_mm_args& a, hipStream_t st);

// KV-cache epilogue of the QKV projection (FP6 / FP4 GEMM, head size 128): parts 0, 1, 2 = Q, K, V
// columns [p H 128, (p+1) H 128); RoPE (cos != null) on Q and K; absmax codes per (token, head);
// 4-bit BOS records of 3-bit parts for tokens with bos_slot[t] in [0, nslots).
constexpr int BL_EPI_KV = 3;        // internal epilogue kind of the fused entry point
struct bl_kv_epi {
  int H;
  float eps;
  int bits[3];
  uint8_t* codes[3];
  float* scale[3];
  const int* pos;
  const float* cos;
  const float* sin;
  int P;
  const int* bos_slot;
  int nslots;
  uint8_t* bos_codes[3];
  float* bos_scale[3];
};
hipError_t bl_launch_gemm_kv(const bl_mm_args& a, const bl_kv_epi& kv, hipStream_t st);
hipError_t bl_launch_gemv(const bl_mm_args& a, hipStream_t st);
hipError_t bl_launch_fill_zero(float* p, long n, hipStream_t st);

// Decode FFN gate and conditional up projection: g = the dequantized gate projection (written to G),
// h = relu(g)^2 * u only where g is positive (+0 elsewhere), u from row-major packed up weights.
struct bl_upcond_args {
  const void* A;          // INT4 codes [M, K/2]
  const float* ascale;
  int M, K, N;
  float* G;               // dequantized gate [M, N] (output), row stride ldg
  long ldg;
  const void* Wup;        // row-major packed up weights
  const float* upalpha;
  float* H;               // [M, N], row stride ldh
  long ldh;
  float* rowmax;          // optional
};
// gate GEMV and conditional up projection in one launch (one block per 16 channels)
hipError_t bl_launch_glu_conditional_fused(const bl_upcond_args& a, const void* Wg, const float* galpha,
                                          hipStream_t st);

// KV-cache quantizer (post-RoPE absmax, 4 or 3 bits, BOS records at 4 bits)
struct bl_kv_args {
  const void* x;          // [T rows of H heads x D], row stride ldx elements
  int in_f32;
  int T, H, D;
  long ldx;
  const int* pos;         // [T] (with cos/sin)
  const float* cos;       // [P, D/2] or null (no rotation)
  const float* sin;
  int P;
  int bits;               // 3 or 4
  float eps;
  void* codes;            // [T][H][D*bits/8]
  float* scale;           // [T][H]
  const int* bos_slot;    // [T] or null; slot >= 0 marks a BOS token (bits == 3 only)
  int nslots;
  void* bos_codes;        // [nslots][H][D/2]
  float* bos_scale;       // [nslots][H]
};
hipError_t bl_launch_kv_quant(const bl_kv_args& a, hipStream_t st);

// measurement aid: FP6 x FP4 matrix-core loop (blocks x 256 threads, out[blocks * 256])
hipError_t bl_launch_calib_mfma(int blocks, int iters, float* out, hipStream_t st);
// measurement aid: plain streaming read of `bytes` bytes (16 per lane); sink: one uint32, never read back
hipError_t bl_launch_calib_read(const void* p, long bytes, void* sink, hipStream_t st);
