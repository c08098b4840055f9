// Decode BitLinear (1 <= M <= 8 tokens): bandwidth-bound streaming of the packed ternary weights.
//
// "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up), section 3.4: the same
// products as the GEMMs (Y = Q(X) Q_w(W)^T with INT4 or INT8 activations) for a few tokens.
//
// One 256-thread block owns 16 output columns (one packed tile row, n-group G) and splits K over
// its four waves. Every lane loads its 8-byte share of each 512-byte weight tile (a wave reads
// whole tiles, fully coalesced) and issues all of them before any math, so a wave keeps up to
// 4 KB in flight. The tile words feed 16x16x64 int8 MFMAs directly (the M rows are padded to 16
// with zeros); the four partial int32 tiles are summed exactly in LDS.
// INT8 activations (the sparse intermediates) gate the weight loads: a lane skips the 32-wide K
// slice it would load when the codes of all M rows are zero there. INT4 activations do not gate,
// so their weight loads never wait for the activation loads.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

constexpr int WAVES = 4;
constexpr int CH = 8;     // weight tiles in flight per wave and matrix

__device__ __forceinline__ v4i expand_w_i8(uint32_t w) {
  v4i r;
  r[0] = (int)((w << 6) & 0xC0C0C0C0u);
  r[1] = (int)((w << 4) & 0xC0C0C0C0u);
  r[2] = (int)((w << 2) & 0xC0C0C0C0u);
  r[3] = (int)(w & 0xC0C0C0C0u);
  return r;
}
__device__ __forceinline__ v4i expand_a_int4(uint32_t p0, uint32_t p1) {
  v4i r;
  r[0] = (int)((p0 << 4) & 0xF0F0F0F0u);
  r[1] = (int)((p1 << 4) & 0xF0F0F0F0u);
  r[2] = (int)(p0 & 0xF0F0F0F0u);
  r[3] = (int)(p1 & 0xF0F0F0F0u);
  return r;
}
__device__ __forceinline__ v4i expand_a_int8(uint32_t x, uint32_t y, uint32_t z, uint32_t w) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(y, x, 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm(w, z, 0x06040200u);
  r[2] = (int)__builtin_amdgcn_perm(y, x, 0x07050301u);
  r[3] = (int)__builtin_amdgcn_perm(w, z, 0x07050301u);
  return r;
}

template <int FMT, int EPI>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(const uint8_t* __restrict__ A, const float* __restrict__ ascale,
                                                     int M, int K, const uint8_t* __restrict__ W,
                                                     const float* __restrict__ walpha,
                                                     const uint8_t* __restrict__ W2,
                                                     const float* __restrict__ w2alpha, int N,
                                                     float* __restrict__ Y, long ldy, const float* R, long ldr,
                                                     float* __restrict__ rowmax) {
  constexpr bool A8 = (FMT == BL_ACT_INT8);
  constexpr int NB = (EPI == BL_EPI_RELU2_GLU) ? 2 : 1;
  __shared__ v4i red[NB][WAVES - 1][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = blockIdx.x;
  const int KT = K >> 7, NG = N >> 4;            // 128-wide weight tiles along K, 16-row groups
  const int per = (KT + WAVES - 1) / WAVES;
  const int kt_begin = wave * per;
  const int kt_end = min(KT, kt_begin + per);
  const int r = lane & 15, g = lane >> 4;
  const bool row_ok = r < M;
  const long arow = A8 ? K : (K >> 1);
  const uint8_t* Wm[2] = {W, W2};

  v4i acc[NB];
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx) acc[mtx] = v4i{0, 0, 0, 0};

  for (int kt0 = kt_begin; kt0 < kt_end; kt0 += CH) {
    uint2 wt[NB][CH];
    uint4 at[CH][A8 ? 2 : 1];
    bool live[CH];
    if constexpr (A8) {
      // activations first: they decide which weight slices are needed
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int kt = kt0 + c;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        if (kt < kt_end && row_ok) {
          const uint4* p = reinterpret_cast<const uint4*>(A + (long)r * arow + (long)kt * 128 + 32 * g);
          at[c][0] = p[0]; at[c][1] = p[1];
        } else {
          at[c][0] = z; at[c][1] = z;
        }
        const uint32_t nz = at[c][0].x | at[c][0].y | at[c][0].z | at[c][0].w | at[c][1].x | at[c][1].y |
                            at[c][1].z | at[c][1].w;
        const unsigned long long bal = __ballot(nz != 0u);
        live[c] = kt < kt_end && ((bal >> (16 * g)) & 0xFFFFull) != 0ull;
      }
#pragma unroll
      for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int kt = kt0 + c;
          if (live[c])
            wt[mtx][c] = *reinterpret_cast<const uint2*>(Wm[mtx] + ((long)kt * NG + G) * 512 + lane * 8);
          else
            wt[mtx][c] = make_uint2(0u, 0u);
        }
    } else {
      // weights first (the HBM stream), then the small activation slices
#pragma unroll
      for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int kt = kt0 + c;
          if (kt < kt_end)
            wt[mtx][c] = *reinterpret_cast<const uint2*>(Wm[mtx] + ((long)kt * NG + G) * 512 + lane * 8);
          else
            wt[mtx][c] = make_uint2(0u, 0u);
        }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int kt = kt0 + c;
        live[c] = kt < kt_end;
        if (live[c] && row_ok)
          at[c][0] = *reinterpret_cast<const uint4*>(A + (long)r * arow + (long)kt * 64 + 16 * g);
        else
          at[c][0] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (kt0 + c >= kt_end) break;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v4i a;
        if constexpr (A8) {
          a = expand_a_int8(at[c][i].x, at[c][i].y, at[c][i].z, at[c][i].w);
        } else {
          const uint4 q = at[c][0];
          a = i ? expand_a_int4(q.z, q.w) : expand_a_int4(q.x, q.y);
        }
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
          acc[mtx] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, expand_w_i8(i ? wt[mtx][c].y : wt[mtx][c].x), acc[mtx],
                                                           0, 0, 0);
      }
    }
  }

  // exact int32 reduction of the four K partitions
  if (wave > 0) {
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx) red[mtx][wave - 1][lane] = acc[mtx];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w) acc[mtx] += red[mtx][w][lane];

  constexpr int SHIFT = A8 ? 6 : 10;
  const float alpha = *walpha;
  const float alpha2 = (EPI == BL_EPI_RELU2_GLU) ? *w2alpha : 0.f;
  const int n = 16 * G + r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    float out = 0.f;
    if (m < M) {
      const float ds = ascale[m];
      const float y0 = (float)(acc[0][v] >> SHIFT) * (ds * alpha);
      if constexpr (EPI == BL_EPI_RESIDUAL) {
        out = y0 + R[(long)m * ldr + n];
      } else if constexpr (EPI == BL_EPI_RELU2_GLU) {
        const float u0 = (float)(acc[NB - 1][v] >> SHIFT) * (ds * alpha2);
        const float gp = y0 > 0.f ? y0 : 0.f;
        out = (gp * gp) * u0;
      } else {
        out = y0;
      }
      Y[(long)m * ldy + n] = out;
    }
    if constexpr (EPI == BL_EPI_RELU2_GLU) {
      if (rowmax) {
        float a = fabsf(out);
        a = fmaxf(a, __shfl_xor(a, 1, 64));
        a = fmaxf(a, __shfl_xor(a, 2, 64));
        a = fmaxf(a, __shfl_xor(a, 4, 64));
        a = fmaxf(a, __shfl_xor(a, 8, 64));
        if (r == 0 && m < M) atomicMax(reinterpret_cast<unsigned int*>(rowmax) + m, bl_f2u(a));
      }
    }
  }
}

template <int FMT, int EPI>
hipError_t launch(const bl_mm_args& a, hipStream_t st) {
  hipLaunchKernelGGL((k_gemv<FMT, EPI>), dim3(a.N / 16), dim3(WAVES * 64), 0, st, static_cast<const uint8_t*>(a.A),
                     a.ascale, a.M, a.K, static_cast<const uint8_t*>(a.W), a.walpha,
                     static_cast<const uint8_t*>(a.W2), a.w2alpha, a.N, a.Y, a.ldy, a.R, a.ldr, a.rowmax);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_epi(const bl_mm_args& a, hipStream_t st) {
  if (a.epi == BL_EPI_RESIDUAL) return launch<FMT, BL_EPI_RESIDUAL>(a, st);
  if (a.epi == BL_EPI_RELU2_GLU) return launch<FMT, BL_EPI_RELU2_GLU>(a, st);
  return launch<FMT, BL_EPI_NONE>(a, st);
}

}  // namespace

hipError_t bl_launch_gemv(const bl_mm_args& a, hipStream_t st) {
  if (a.fmt == BL_ACT_INT8) return launch_epi<BL_ACT_INT8>(a, st);
  return launch_epi<BL_ACT_INT4>(a, st);
}
