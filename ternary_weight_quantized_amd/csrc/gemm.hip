// BitLinear GEMMs on CDNA4 matrix cores: W1.58A4 (INT4 and FP4 E2M1) and W1.58A8 (sparse INT8).
//
// "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up), section 3.4:
//   Y = Q_INT4(X) Q_w(W)^T ("4-Bit Activation Quantization for Gaussian-Like Inputs"),
//   Y = (Q_INT8(X) . M) Q_w(W)^T ("Sparsification Pipeline ...", paper Eq. 1),
//   ReLU^2 GLU epilogue ("Squared ReLU Gating ...", paper Eq. 5), residual add (section 3.2).
//
// Block tile 128 x 128 of Y, K step 256 (one packed weight tile), 4 waves in a 2 x 2 grid, each
// wave 64 x 64 = 4 x 4 MFMA tiles of 16 x 16. Packed operands go global -> registers -> LDS
// (double buffered); each wave expands its fragments in registers right before the MFMA:
//   ternary 2-bit -> int8:  (w << s) & 0xC0C0C0C0 places a code in the top bits of a byte, i.e. 64*t;
//   INT4 nibble   -> int8:  the nibble moved to the top of a byte is 16*c;
//   INT8 codes are used as they are after a byte permutation.
// The int32 accumulator therefore holds 1024*sum(c t) (INT4) or 64*sum(c t) (INT8), both far from
// overflow for K < 2^18, and an exact arithmetic shift recovers sum(c t).
// FP4 uses v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E2M1 and unit block scales;
// a ternary code placed in bits 2..3 of a nibble reads as E2M1 +-2.0, so the fp32 sum is
// 2*sum(e t) = sum(doubled code * t), exact because every partial sum is an integer < 2^24.
//
// The K order inside each 16- or 32-wide MFMA slice follows the packed weight word (see the public
// header); activations are expanded into the same order, which leaves every dot product unchanged.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

constexpr int BM = 128, BN = 128, NTHREADS = 256;

template <int FMT>
struct ATraits {
  static constexpr int ROW = (FMT == BL_ACT_INT8) ? 256 : 128;  // bytes of one A row per K step
  static constexpr int STRIDE = ROW + 16;                       // padded LDS row stride
  static constexpr int BYTES = BM * STRIDE;
  static constexpr int CHUNKS = BM * ROW / 16;                  // 16-byte chunks per stage
  static constexpr int PER_THREAD = CHUNKS / NTHREADS;
};

template <int FMT, int EPI>
struct Smem {
  static constexpr int NB = (EPI == BL_EPI_RELU2_GLU) ? 2 : 1;
  static constexpr int BBYTES = (BN / 16) * 1024;
  static constexpr int STAGE = ATraits<FMT>::BYTES + NB * BBYTES;
};

__device__ __forceinline__ v4i expand_w_i8(uint32_t w) {
  v4i r;
  r[0] = (int)((w << 6) & 0xC0C0C0C0u);   // k 0 2 4 6
  r[1] = (int)((w << 4) & 0xC0C0C0C0u);   // k 8 10 12 14
  r[2] = (int)((w << 2) & 0xC0C0C0C0u);   // k 1 3 5 7
  r[3] = (int)(w & 0xC0C0C0C0u);          // k 9 11 13 15
  return r;
}
__device__ __forceinline__ v4i expand_a_int4(uint32_t p0, uint32_t p1) {
  v4i r;
  r[0] = (int)((p0 << 4) & 0xF0F0F0F0u);  // k 0 2 4 6      (x16)
  r[1] = (int)((p1 << 4) & 0xF0F0F0F0u);  // k 8 10 12 14
  r[2] = (int)(p0 & 0xF0F0F0F0u);         // k 1 3 5 7
  r[3] = (int)(p1 & 0xF0F0F0F0u);         // k 9 11 13 15
  return r;
}
__device__ __forceinline__ v4i expand_a_int8(uint4 q) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(q.y, q.x, 0x06040200u);  // bytes 0 2 4 6
  r[1] = (int)__builtin_amdgcn_perm(q.w, q.z, 0x06040200u);  // 8 10 12 14
  r[2] = (int)__builtin_amdgcn_perm(q.y, q.x, 0x07050301u);  // 1 3 5 7
  r[3] = (int)__builtin_amdgcn_perm(q.w, q.z, 0x07050301u);  // 9 11 13 15
  return r;
}
// two packed words (32 weights) -> four dwords of E2M1 nibbles in natural k order, value 2*t
__device__ __forceinline__ v8i expand_w_fp4(uint32_t w0, uint32_t w1) {
  v8i r;
  r[0] = (int)((w0 << 2) & 0xCCCCCCCCu);
  r[1] = (int)(w0 & 0xCCCCCCCCu);
  r[2] = (int)((w1 << 2) & 0xCCCCCCCCu);
  r[3] = (int)(w1 & 0xCCCCCCCCu);
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

template <int FMT, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm(const uint8_t* __restrict__ A, const float* __restrict__ ascale,
                                                       int M, int K, const uint8_t* __restrict__ W,
                                                       const float* __restrict__ walpha,
                                                       const uint8_t* __restrict__ W2,
                                                       const float* __restrict__ w2alpha, int N,
                                                       float* __restrict__ Y, long ldy,
                                                       const float* R, long ldr,
                                                       float* __restrict__ rowmax) {
  using AT = ATraits<FMT>;
  using SM = Smem<FMT, EPI>;
  constexpr int NB = SM::NB;
  constexpr bool FP4 = (FMT == BL_ACT_FP4_E2M1);
  constexpr bool A8 = (FMT == BL_ACT_INT8);
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * SM::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int KB = K >> 8;
  const long arow = FP4 || !A8 ? (K >> 1) : K;     // bytes per A row in global memory
  const int NG = N >> 4;

  const uint8_t* Wm[2] = {W, W2};

  uint4 ra[AT::PER_THREAD];
  uint4 rb[NB][2];

  auto gload = [&](int kb) {
#pragma unroll
    for (int q = 0; q < AT::PER_THREAD; ++q) {
      const int c = tid + NTHREADS * q;
      const int r = c / (AT::ROW / 16), col = c % (AT::ROW / 16);
      const int m = m0 + r;
      if (m < M)
        ra[q] = *reinterpret_cast<const uint4*>(A + (long)m * arow + (long)kb * AT::ROW + col * 16);
      else
        ra[q] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = tid + NTHREADS * q;
        const int t = c >> 6, L = c & 63;
        const int G = (n0 >> 4) + t;
        if (G < NG)
          rb[mtx][q] = *reinterpret_cast<const uint4*>(Wm[mtx] + ((long)G * KB + kb) * 1024 + L * 16);
        else
          rb[mtx][q] = make_uint4(0u, 0u, 0u, 0u);
      }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * SM::STAGE;
#pragma unroll
    for (int q = 0; q < AT::PER_THREAD; ++q) {
      const int c = tid + NTHREADS * q;
      const int r = c / (AT::ROW / 16), col = c % (AT::ROW / 16);
      *reinterpret_cast<uint4*>(base + r * AT::STRIDE + col * 16) = ra[q];
    }
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = tid + NTHREADS * q;
        *reinterpret_cast<uint4*>(base + AT::BYTES + mtx * SM::BBYTES + c * 16) = rb[mtx][q];
      }
  };

  // accumulators: [matrix][m subtile][n subtile]
  v4i acci[NB][4][4];
  v4f accf[NB][4][4];
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acci[mtx][s][t] = v4i{0, 0, 0, 0};
        accf[mtx][s][t] = v4f{0.f, 0.f, 0.f, 0.f};
      }

  const int r16 = lane & 15, g4 = lane >> 4;

  gload(0);
  sstore(0);
  __syncthreads();

  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    if (kb + 1 < KB) gload(kb + 1);
    const uint8_t* As = smem + buf * SM::STAGE;
    const uint8_t* Bs = As + AT::BYTES;
    uint4 bw[NB][4];
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bw[mtx][t] = *reinterpret_cast<const uint4*>(Bs + mtx * SM::BBYTES + (wn * 4 + t) * 1024 + lane * 16);

    if constexpr (FP4) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v8i bf[NB][4];
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t w0 = j ? bw[mtx][t].z : bw[mtx][t].x;
            const uint32_t w1 = j ? bw[mtx][t].w : bw[mtx][t].y;
            bf[mtx][t] = expand_w_fp4(w0, w1);
          }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int row = wm * 64 + 16 * s + r16;
          const uint4 q = *reinterpret_cast<const uint4*>(As + row * AT::STRIDE + 32 * g4 + 16 * j);
          const v8i a = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
#pragma unroll
          for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              accf[mtx][s][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  a, bf[mtx][t], accf[mtx][s][t], 4, 4, 0, 127, 0, 127);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v4i bf[NB][4];
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t w = i == 0 ? bw[mtx][t].x : i == 1 ? bw[mtx][t].y : i == 2 ? bw[mtx][t].z : bw[mtx][t].w;
            bf[mtx][t] = expand_w_i8(w);
          }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int row = wm * 64 + 16 * s + r16;
          v4i a;
          if constexpr (A8) {
            const uint4 q = *reinterpret_cast<const uint4*>(As + row * AT::STRIDE + 64 * g4 + 16 * i);
            // zero-slice skip: a 16-row x 64-k slice of all-zero codes contributes nothing
            if (__ballot((q.x | q.y | q.z | q.w) != 0u) == 0ull) continue;
            a = expand_a_int8(q);
          } else {
            const uint2 p = *reinterpret_cast<const uint2*>(As + row * AT::STRIDE + 32 * g4 + 8 * i);
            a = expand_a_int4(p.x, p.y);
          }
#pragma unroll
          for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acci[mtx][s][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bf[mtx][t], acci[mtx][s][t], 0, 0, 0);
        }
      }
    }
    if (kb + 1 < KB) sstore(buf ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue (fp32, fixed order)
  const float alpha = *walpha;
  const float alpha2 = (EPI == BL_EPI_RELU2_GLU) ? *w2alpha : 0.f;
  constexpr int SHIFT = A8 ? 6 : 10;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int mb = m0 + wm * 64 + 16 * s + 4 * g4;
    float rmax[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = mb + v;
      const bool mok = m < M;
      const float ds = mok ? ascale[m] : 0.f;
      const float sc = ds * alpha;
      const float sc2 = ds * alpha2;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + wn * 64 + 16 * t + r16;
        if (!mok || n >= N) continue;
        float y0, u0 = 0.f;
        if constexpr (FP4) {
          y0 = (accf[0][s][t][v] * 0.5f) * sc;
          if constexpr (EPI == BL_EPI_RELU2_GLU) u0 = (accf[1][s][t][v] * 0.5f) * sc2;
        } else {
          y0 = (float)(acci[0][s][t][v] >> SHIFT) * sc;
          if constexpr (EPI == BL_EPI_RELU2_GLU) u0 = (float)(acci[NB - 1][s][t][v] >> SHIFT) * sc2;
        }
        float out;
        if constexpr (EPI == BL_EPI_RESIDUAL) {
          out = y0 + R[(long)m * ldr + n];
        } else if constexpr (EPI == BL_EPI_RELU2_GLU) {
          const float gp = y0 > 0.f ? y0 : 0.f;
          out = (gp * gp) * u0;
          const float a = fabsf(out);
          rmax[v] = a > rmax[v] ? a : rmax[v];
        } else {
          out = y0;
        }
        Y[(long)m * ldy + n] = out;
      }
    }
    if constexpr (EPI == BL_EPI_RELU2_GLU) {
      if (rowmax) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float r = rmax[v];
          r = fmaxf(r, __shfl_xor(r, 1, 64));
          r = fmaxf(r, __shfl_xor(r, 2, 64));
          r = fmaxf(r, __shfl_xor(r, 4, 64));
          r = fmaxf(r, __shfl_xor(r, 8, 64));
          const int m = mb + v;
          if (r16 == 0 && m < M) atomicMax(reinterpret_cast<unsigned int*>(rowmax) + m, bl_f2u(r));
        }
      }
    }
  }
}

template <int FMT, int EPI>
hipError_t launch(const bl_mm_args& a, hipStream_t st) {
  const dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM), block(NTHREADS);
  hipLaunchKernelGGL((k_gemm<FMT, EPI>), grid, block, 0, st, static_cast<const uint8_t*>(a.A), a.ascale, a.M, a.K,
                     static_cast<const uint8_t*>(a.W), a.walpha, static_cast<const uint8_t*>(a.W2), a.w2alpha, a.N,
                     a.Y, a.ldy, a.R, a.ldr, a.rowmax);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_epi(const bl_mm_args& a, hipStream_t st) {
  if (a.epi == BL_EPI_RESIDUAL) return launch<FMT, BL_EPI_RESIDUAL>(a, st);
  if (a.epi == BL_EPI_RELU2_GLU) return launch<FMT, BL_EPI_RELU2_GLU>(a, st);
  return launch<FMT, BL_EPI_NONE>(a, st);
}

__global__ void k_fill_zero(float* p, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

hipError_t bl_launch_fill_zero(float* p, long n, hipStream_t st) {
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t bl_launch_gemm(const bl_mm_args& a, hipStream_t st) {
  if (a.fmt == BL_ACT_INT4) return launch_epi<BL_ACT_INT4>(a, st);
  if (a.fmt == BL_ACT_FP4_E2M1) return launch_epi<BL_ACT_FP4_E2M1>(a, st);
  return launch_epi<BL_ACT_INT8>(a, st);
}
