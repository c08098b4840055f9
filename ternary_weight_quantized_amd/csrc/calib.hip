// Measurement aid, not part of the BitLinear path: the sustained FP6 x FP4 matrix-core rate of the
// part in the shape of the GEMM's K loop (two 4-wave blocks per CU, 32 independent 16x16 fp32
// accumulators per wave, v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales), on operands with the
// GEMM's statistics: ternary weights as E2M1 nibbles (0, +2, -2 in about equal shares) and INT4
// codes in E3M2 from a bell-shaped distribution. The matrix cores' sustained rate on this part depends
// on the operand bits (their switching power sets the clock): near-constant operands run far faster
// than these, so the figure is the ceiling for this data, not a datasheet number. Eight weight and
// four activation operand sets alternate, so consecutive MFMAs never see the same bits. Thread 0 of
// every block reports its shader-clock ticks per 100 MHz real-time tick over the loop (s_memtime /
// s_memrealtime); the other lanes store their accumulator sums, so that no MFMA is dead code.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

__device__ __forceinline__ uint32_t calib_hash(uint32_t x) {
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}
// eight E2M1 nibbles of ternary codes: bits 2..3 of a nibble are 00 (0), 01 (+2) or 11 (-2)
__device__ __forceinline__ int calib_w8(uint32_t h) {
  uint32_t w = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t t = ((h >> (4 * j)) & 15u) % 3u;          // 0, 1, 2
    w |= (t == 0u ? 0u : t == 1u ? 0x4u : 0xCu) << (4 * j);
  }
  return (int)w;
}
// E3M2 code of an integer -8 .. 7 (bias 3)
__device__ __forceinline__ uint32_t calib_e3m2(int v) {
  const uint32_t s = v < 0 ? 0x20u : 0u;
  const uint32_t m = (uint32_t)(v < 0 ? -v : v);
  if (m == 0u) return s;
  const int e = 31 - __builtin_clz(m);
  return s | ((uint32_t)(e + 3) << 2) | (((m << 2) >> e) & 3u);
}

__global__ __launch_bounds__(256, 2) void k_calib_mfma(int iters, float* __restrict__ out) {
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u;
  v8i w[8], x[4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    w[t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) w[t][i] = calib_w8(calib_hash(seed + 8u * t + i));
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    // 32 codes of 6 bits, a sum of four uniform nibbles recentred to about -7 .. 7
    uint32_t bits[6] = {0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const uint32_t h = calib_hash(seed + 40u + 1000u * s + e);
      int v = (int)(((h & 15u) + ((h >> 4) & 15u) + ((h >> 8) & 15u) + ((h >> 12) & 15u)) >> 2) - 7;
      v = v > 7 ? 7 : v;
      const uint32_t c = calib_e3m2(v);
      const int bit = 6 * e;
      bits[bit >> 5] |= c << (bit & 31);
      if ((bit & 31) > 26) bits[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
    }
    x[s] = v8i{(int)bits[0], (int)bits[1], (int)bits[2], (int)bits[3], (int)bits[4], (int)bits[5], 0, 0};
  }
  v4f c[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) c[s][t] = v4f{0.f, 0.f, 0.f, 0.f};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        c[s][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w[(t + s) & 7], x[s], c[s][t], 4, 3, 0, 127, 0, 127);
  }
  float sum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) sum += c[s][t][0] + c[s][t][1] + c[s][t][2] + c[s][t][3];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) sum = r1 > r0 ? (float)(t1 - t0) / (float)(r1 - r0) : 0.f;
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
