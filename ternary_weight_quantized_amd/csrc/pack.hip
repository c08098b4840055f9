// Absmean ternary weight quantizer and 2-bit packing.
//
// "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up), section 3.4,
// "Ternary Weight Quantization (BitLinear)": Q_w(W) = alpha * RoundClip(W/(alpha+eps), -1, 1),
// alpha = mean(|W|) over the whole tensor (paper Eq. 2).
//
// alpha is exact: every |w| is split into (biased exponent, 24-bit significand) and the
// significands are summed per exponent in 64-bit integers (LDS per block, then global atomics),
// so the sum is independent of order; one thread turns the 256 bins into the correctly rounded
// double of the exact total and divides by N*K. The pack kernel then writes one 32-bit word
// (16 weights of one row) per thread in the tiled layout of the public header (16 x 128 tiles, with
// the field order of the 4-bit-activation matmuls or of the INT8 ones), or in the row-major layout
// used by the gathered (conditional) up projection.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

__global__ void k_zero_u64(unsigned long long* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__global__ __launch_bounds__(256) void k_abs_bins(const float* __restrict__ w, long n,
                                                  unsigned long long* __restrict__ gbins) {
  __shared__ unsigned long long bins[256];
  bins[threadIdx.x] = 0ull;
  __syncthreads();
  const long stride = (long)gridDim.x * blockDim.x * 4;
  for (long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    const float4 v = *reinterpret_cast<const float4*>(w + i);
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t e, m;
      bl_bin_split(bl_f2u(vv[j]) & 0x7FFFFFFFu, &e, &m);
      if (m) atomicAdd(&bins[e], (unsigned long long)m);
    }
  }
  __syncthreads();
  const unsigned long long b = bins[threadIdx.x];
  if (b) atomicAdd(&gbins[threadIdx.x], b);
}

__global__ __launch_bounds__(256) void k_alpha(const unsigned long long* __restrict__ gbins, double count,
                                               float* __restrict__ alpha) {
  __shared__ unsigned long long limbs[12];
  __shared__ double total;
  const double S = bl_bins_to_double_block(gbins, limbs, &total);
  if (threadIdx.x == 0) *alpha = (float)(S / count);
}

// Bit position of weight q (0..15) of a packed 32-bit word. Standard words (every matmul with 4-bit
// activations): q < 8 at 4 q, q >= 8 at 4 (q - 8) + 2, so that masking the word with 0xCCCCCCCC after
// shifting it by 2 or 0 gives the E2M1 nibbles of q = 0..7 and 8..15 in order. A8 words (the int8
// matmuls with INT8 activations): q at 8 (q % 4) + 2 (q / 4), so that masking it with 0xC0C0C0C0
// after shifting it by 6, 4, 2 or 0 gives the int8 bytes of q = 0..3, 4..7, 8..11 and 12..15 in
// order, the order of the INT8 codes themselves.
__device__ __forceinline__ int field_pos(int q, bool a8) {
  return a8 ? 8 * (q & 3) + 2 * (q >> 2) : (q < 8 ? 4 * q : 4 * (q - 8) + 2);
}

// One thread per packed 32-bit word: tile (kt, G) of 16 rows x 128 columns, lane L = 16 g + r, word i.
template <bool A8>
__global__ __launch_bounds__(256) void k_pack(const float* __restrict__ w, int N, int K, float eps,
                                              const float* __restrict__ alpha, uint32_t* __restrict__ out) {
  const long wid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long nwords = (long)N * K / 16;
  if (wid >= nwords) return;
  const int NG = N >> 4;
  const long tile = wid >> 7;                                    // 128 words per 512-byte tile
  const int t = (int)(wid & 127);
  const int L = t >> 1, i = t & 1;
  const int kt = (int)(tile / NG), G = (int)(tile % NG);         // K-tile-major tile order
  const int n = 16 * G + (L & 15);
  const int k0 = 128 * kt + 32 * (L >> 4) + 16 * i;
  const float den = *alpha + eps;
  const float4* src = reinterpret_cast<const float4*>(w + (long)n * K + k0);
  uint32_t word = 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v = src[c];
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * c + j;                                   // k offset inside the word
      const int code = bl_roundclip(vv[j] / den, -1.f, 1.f);     // IEEE division, half-even
      const uint32_t f = (uint32_t)code & 3u;                    // 0 -> 00, +1 -> 01, -1 -> 11
      word |= f << field_pos(q, A8);
    }
  }
  out[wid] = word;
}

// Row-major variant: one thread per 32-bit word (n, i) holding weights 16 i .. 16 i + 15 of row n,
// with the same placement inside the word; row n occupies K/4 contiguous bytes.
__global__ __launch_bounds__(256) void k_pack_rows(const float* __restrict__ w, int N, int K, float eps,
                                                   const float* __restrict__ alpha, uint32_t* __restrict__ out) {
  const long wid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long nwords = (long)N * K / 16;
  if (wid >= nwords) return;
  const float den = *alpha + eps;
  const float4* src = reinterpret_cast<const float4*>(w + wid * 16);   // row-major: word wid covers 16 * wid
  uint32_t word = 0u;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float4 v = src[c];
    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * c + j;
      const int code = bl_roundclip(vv[j] / den, -1.f, 1.f);
      word |= ((uint32_t)code & 3u) << field_pos(q, false);
    }
  }
  out[wid] = word;
}

}  // namespace

hipError_t bl_launch_pack(const float* w, int N, int K, float eps, void* packed, float* alpha,
                          void* ws, int layout, hipStream_t st) {
  unsigned long long* bins = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(256), 0, st, bins, 256);
  const long n = (long)N * K;
  long blocks = (n / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_abs_bins, dim3((unsigned)blocks), dim3(256), 0, st, w, n, bins);
  hipLaunchKernelGGL(k_alpha, dim3(1), dim3(256), 0, st, bins, (double)n, alpha);
  const long nwords = n / 16;
  const dim3 grid((unsigned)((nwords + 255) / 256));
  if (layout == BL_PACK_ROWS)
    hipLaunchKernelGGL(k_pack_rows, grid, dim3(256), 0, st, w, N, K, eps, alpha, static_cast<uint32_t*>(packed));
  else if (layout == BL_PACK_TILES_A8)
    hipLaunchKernelGGL((k_pack<true>), grid, dim3(256), 0, st, w, N, K, eps, alpha, static_cast<uint32_t*>(packed));
  else
    hipLaunchKernelGGL((k_pack<false>), grid, dim3(256), 0, st, w, N, K, eps, alpha, static_cast<uint32_t*>(packed));
  return hipGetLastError();
}
