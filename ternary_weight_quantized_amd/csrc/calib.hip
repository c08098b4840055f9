// Measurement aid, not part of the BitLinear path: the sustained FP6 x FP4 matrix-core rate of the
// part in the shape of the GEMM's K loop (two 4-wave blocks per CU, 32 independent 16x16 fp32
// accumulators per wave, v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales), so that a kernel's
// MFMA roofline can be read against what this machine sustains as well as against the datasheet.
// The operands change every iteration (one VALU op per subtile) so the loop is not a constant
// repeat; the accumulators are summed into out[] so that no MFMA is dead code.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

__global__ __launch_bounds__(256, 2) void k_calib_mfma(int iters, float* __restrict__ out) {
  v8i a = {(int)(threadIdx.x * 2654435761u), (int)(blockIdx.x * 40503u), 0x5A5A5A5A, 0x3C3C3C3C, 0x12345678,
           0x0F0F0F0F, 0, 0};
  v8i b[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
    b[t] = v8i{(int)(0x4C4C4C4Cu ^ (t * 0x01010101u)), (int)(threadIdx.x * 77u), 0x44444444, 0x0C0C0C0C, 0, 0, 0, 0};
  v4f c[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) c[s][t] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v8i as = a;
      as[0] ^= i * 0x9E3779B9 + s;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        c[s][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[t], as, c[s][t], 4, 3, 0, 127, 0, 127);
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) sum += c[s][t][0] + c[s][t][1] + c[s][t][2] + c[s][t][3];
  out[(long)blockIdx.x * 256 + threadIdx.x] = sum;
}

// Measurement aid: a plain streaming read of `bytes` bytes (16 per lane, one load per lane, 256-lane
// blocks: the fastest of the read shapes measured for an 11 MB buffer), the ceiling a decode GEMV
// reading the same bytes per launch can reach. Each lane folds its 16 bytes into one word, and a
// word is written only when it equals a value the data never produces, so the loads stay live.
__global__ __launch_bounds__(256) void k_calib_read(const uint8_t* __restrict__ p, long bytes,
                                                    uint32_t* __restrict__ sink) {
  const long off = ((long)blockIdx.x * 256 + threadIdx.x) * 16;
  if (off + 16 > bytes) return;
  const uint4 v = *reinterpret_cast<const uint4*>(p + off);
  const uint32_t f = v.x ^ v.y ^ v.z ^ v.w;
  if (f == 0xA5C3E1F7u && v.x == 0x0F1E2D3Cu) sink[0] = f;
}

}  // namespace

hipError_t bl_launch_calib_read(const void* p, long bytes, void* sink, hipStream_t st) {
  const long blocks = (bytes / 16 + 255) / 256;
  hipLaunchKernelGGL(k_calib_read, dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, st,
                     static_cast<const uint8_t*>(p), bytes, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

hipError_t bl_launch_calib_mfma(int blocks, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_calib_mfma, dim3(blocks), dim3(256), 0, st, iters, out);
  return hipGetLastError();
}
