// Decode BitLinear (1 <= M <= 8 tokens): bandwidth-bound streaming of the packed ternary weights.
//
// "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up), section 3.4: the same
// products as the GEMMs (Y = Q(X) Q_w(W)^T with INT4 or INT8 activations) for a few tokens.
//
// One block owns 16 output columns (one packed tile row, n-group G) and splits the K tiles over
// its waves (eight; sixteen when K is long, e.g. the 11008-wide down projection, whose 4096 output
// columns give only 256 blocks); a wave issues all loads of a chunk of four or six K tiles at once (the
// activation slices first, then its 8-byte share of each 512-byte weight tile, so a wave reads
// whole tiles, fully coalesced) and feeds each tile to the matrix cores as soon as it has landed.
// The tile words go to 16x16x64 int8 MFMAs directly; the M token rows occupy the first M of the 16
// MFMA rows and the other rows repeat row M-1 (their outputs are never stored), which keeps every
// load unconditional. The eight partial int32 tiles are summed exactly in LDS. The per-token scales,
// alpha and the residual are fetched at the start so that nothing but the stores follows the sum.
// INT8 activations (the sparse intermediates) gate the weight loads: a lane skips the 32-wide K
// slice it would load when the codes of all M rows are zero there.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

constexpr int WAVES = 8;
constexpr int CH = 4;     // K tiles per chunk and wave

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
__device__ __forceinline__ v4i expand_a_int8(uint4 q) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(q.y, q.x, 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm(q.w, q.z, 0x06040200u);
  r[2] = (int)__builtin_amdgcn_perm(q.y, q.x, 0x07050301u);
  r[3] = (int)__builtin_amdgcn_perm(q.w, q.z, 0x07050301u);
  return r;
}

// One chunk of up to CH K tiles starting at kt0 (kt0 < kt_end). FULL chunks load unconditionally, so
// the compiler can wait for each tile separately; the ragged last chunk clamps its addresses and
// drops the tiles past kt_end. Offsets are 32-bit: N K / 4 < 2^29 bytes of weights, M K < 2^22
// bytes of codes.
template <bool A8, int NB, bool FULL, int CH = 4>
__device__ __forceinline__ void chunk(const uint8_t* arp, const uint8_t* const (&wp)[2], uint32_t wstep, int kt0,
                                      int kt_end, int g, v4i (&acc)[NB][2]) {
  constexpr int AV = A8 ? 2 : 1;              // 16-byte activation vectors per lane and tile
  constexpr uint32_t ABYTES = A8 ? 128 : 64;  // activation bytes per row and tile
  uint4 at[CH][AV];
  uint2 wt[NB][CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const uint32_t kt = FULL ? kt0 + c : min(kt0 + c, kt_end - 1);
#pragma unroll
    for (int v = 0; v < AV; ++v) at[c][v] = *reinterpret_cast<const uint4*>(arp + kt * ABYTES + 16 * v);
  }
  if constexpr (A8) {
    // weights only where some row has a nonzero code in this lane's 32-wide K slice
    bool live[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t nz = at[c][0].x | at[c][0].y | at[c][0].z | at[c][0].w | at[c][1].x | at[c][1].y |
                          at[c][1].z | at[c][1].w;
      const unsigned long long bal = __ballot(nz != 0u);
      live[c] = (FULL || kt0 + c < kt_end) && ((bal >> (16 * g)) & 0xFFFFull) != 0ull;
    }
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        wt[mtx][c] = live[c] ? *reinterpret_cast<const uint2*>(wp[mtx] + (uint32_t)(kt0 + c) * wstep) : make_uint2(0u, 0u);
  } else {
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const uint32_t kt = FULL ? kt0 + c : min(kt0 + c, kt_end - 1);
        wt[mtx][c] = *reinterpret_cast<const uint2*>(wp[mtx] + kt * wstep);
      }
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (!FULL && kt0 + c >= kt_end) break;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4i a;
      if constexpr (A8) a = expand_a_int8(at[c][i]);
      else a = i ? expand_a_int4(at[c][0].z, at[c][0].w) : expand_a_int4(at[c][0].x, at[c][0].y);
#pragma unroll
      for (int mtx = 0; mtx < NB; ++mtx)
        acc[mtx][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, expand_w_i8(i ? wt[mtx][c].y : wt[mtx][c].x),
                                                            acc[mtx][i], 0, 0, 0);
    }
  }
}

template <int FMT, int EPI, int CHN, int NWV>
__global__ __launch_bounds__(NWV * 64) void k_gemv(const uint8_t* __restrict__ A, const float* __restrict__ ascale,
                                                     int M, int K, const uint8_t* __restrict__ W,
                                                     const float* __restrict__ walpha,
                                                     const uint8_t* __restrict__ W2,
                                                     const float* __restrict__ w2alpha, int N,
                                                     float* __restrict__ Y, long ldy, const float* R, long ldr,
                                                     float* __restrict__ rowmax) {
  constexpr bool A8 = (FMT == BL_ACT_INT8);
  constexpr int NB = (EPI == BL_EPI_RELU2_GLU) ? 2 : 1;
  __shared__ v4i red[NB][NWV - 1][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = blockIdx.x;
  const int KT = K >> 7, NG = N >> 4;            // 128-wide weight tiles along K, 16-row groups
  const int per = (KT + NWV - 1) / NWV;
  const int kt_begin = wave * per;
  const int kt_end = min(KT, kt_begin + per);
  const int r = lane & 15, g = lane >> 4;
  const int n = 16 * G + r;
  const uint32_t arow = A8 ? K : (K >> 1);
  const uint8_t* arp = A + (uint32_t)min(r, M - 1) * arow + (A8 ? 32 * g : 16 * g);
  const uint32_t woff = (uint32_t)G * 512u + (uint32_t)lane * 8u;
  const uint8_t* const wp[2] = {W + woff, (NB > 1 ? W2 : W) + woff};
  const uint32_t wstep = (uint32_t)NG * 512u;

  // what the epilogue reads, fetched by the epilogue wave only, before its weight stream (rows past
  // M repeat row M-1; the other waves only stream weights and hand over partial sums)
  float ds[4] = {0.f, 0.f, 0.f, 0.f}, res[4] = {0.f, 0.f, 0.f, 0.f};
  float alpha = 0.f, alpha2 = 0.f;
  if (wave == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = min(4 * g + v, M - 1);
      ds[v] = ascale[m];
      if constexpr (EPI == BL_EPI_RESIDUAL) res[v] = R[(long)m * ldr + n];
    }
    alpha = *walpha;
    if constexpr (EPI == BL_EPI_RELU2_GLU) alpha2 = *w2alpha;
  }

  v4i acc[NB][2];
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx) acc[mtx][0] = acc[mtx][1] = v4i{0, 0, 0, 0};
  for (int kt0 = kt_begin; kt0 < kt_end; kt0 += CHN) {
    if (kt0 + CHN <= kt_end) chunk<A8, NB, true, CHN>(arp, wp, wstep, kt0, kt_end, g, acc);
    else chunk<A8, NB, false, CHN>(arp, wp, wstep, kt0, kt_end, g, acc);
  }

  // exact int32 reduction of the K partitions
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx) acc[mtx][0] += acc[mtx][1];
  if (wave > 0) {
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx) red[mtx][wave - 1][lane] = acc[mtx][0];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
    for (int w = 0; w < NWV - 1; ++w) acc[mtx][0] += red[mtx][w][lane];

  constexpr int SHIFT = A8 ? 6 : 10;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    const float y0 = (float)(acc[0][0][v] >> SHIFT) * (ds[v] * alpha);
    float out;
    if constexpr (EPI == BL_EPI_RESIDUAL) {
      out = y0 + res[v];
    } else if constexpr (EPI == BL_EPI_RELU2_GLU) {
      const float u0 = (float)(acc[NB - 1][0][v] >> SHIFT) * (ds[v] * alpha2);
      const float gp = y0 > 0.f ? y0 : 0.f;
      out = (gp * gp) * u0;
    } else {
      out = y0;
    }
    if (m < M) Y[(long)m * ldy + n] = out;
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

template <int FMT, int EPI, int CHN, int NWV>
hipError_t launch_w(const bl_mm_args& a, hipStream_t st) {
  hipLaunchKernelGGL((k_gemv<FMT, EPI, CHN, NWV>), dim3(a.N / 16), dim3(NWV * 64), 0, st,
                     static_cast<const uint8_t*>(a.A), a.ascale, a.M, a.K, static_cast<const uint8_t*>(a.W),
                     a.walpha, static_cast<const uint8_t*>(a.W2), a.w2alpha, a.N, a.Y, a.ldy, a.R, a.ldr, a.rowmax);
  return hipGetLastError();
}
// eight waves with one chunk of up to four tiles each when K allows it (K <= 4096), else sixteen
// waves with chunks of four or six tiles (K <= 12288 in one chunk per wave)
template <int FMT, int EPI>
hipError_t launch(const bl_mm_args& a, hipStream_t st) {
  const int KT = a.K >> 7;
  if ((KT + WAVES - 1) / WAVES <= CH) return launch_w<FMT, EPI, CH, WAVES>(a, st);
  if ((KT + 15) / 16 <= 4) return launch_w<FMT, EPI, 4, 16>(a, st);
  return launch_w<FMT, EPI, 6, 16>(a, st);
}

template <int FMT>
hipError_t launch_epi(const bl_mm_args& a, hipStream_t st) {
  if (a.epi == BL_EPI_RESIDUAL) return launch<FMT, BL_EPI_RESIDUAL>(a, st);
  if (a.epi == BL_EPI_RELU2_GLU) return launch<FMT, BL_EPI_RELU2_GLU>(a, st);
  return launch<FMT, BL_EPI_NONE>(a, st);
}

// ============================================================================ conditional up projection
// "Squared ReLU Gating and Conditional Computation in the FFN" (section 3.4): once the gate
// projection g is known, the up projection is only needed for channels whose gate is positive
// (relu(g)^2 is zero elsewhere). Up weights come in the row-major 2-bit layout (row n = K/4
// contiguous bytes), so a skipped channel costs no weight traffic.
//
// dot_ternary_int4: sum over one 64-wide K slice (16 weight bytes, 32 code bytes) of c * t. Ternary
// fields f in {00, 01, 11} enter v_dot8 as signed 4-bit values f in {0, 1, 3}; with b the high bit
// of the field, t = f - 4 b, so sum(c t) = dot(c, f) - 4 dot(c, b), exact in int32.
__device__ __forceinline__ int dot_ternary_int4(uint4 w, uint4 a0, uint4 a1, int acc) {
  // word i covers k 16 i .. 16 i + 15: bits 4q..4q+1 -> k = 16 i + q, bits 4q+2..4q+3 -> k = 16 i + 8 + q
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  const uint32_t as[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  int f = 0, b = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = ws[i] & 0x33333333u, hi = (ws[i] >> 2) & 0x33333333u;
    f = __builtin_amdgcn_sdot8((int)as[2 * i], (int)lo, f, false);
    f = __builtin_amdgcn_sdot8((int)as[2 * i + 1], (int)hi, f, false);
    b = __builtin_amdgcn_sdot8((int)as[2 * i], (int)((lo >> 1) & 0x11111111u), b, false);
    b = __builtin_amdgcn_sdot8((int)as[2 * i + 1], (int)((hi >> 1) & 0x11111111u), b, false);
  }
  return acc + f - 4 * b;
}

// Fused form for one block per 16-channel group (the tile row of W_gate): phase 1 is the INT4 decode
// GEMV of the gate (eight waves split K, exact int32 sum in LDS); the block then knows g for its 16
// channels and M rows, and in phase 2 each wave takes two channels and, if the gate of a channel is
// positive in some row, streams its row-major up weights (K/4 bytes; 16 bytes per lane and 64-wide
// K slice) against the INT4 codes with v_dot8 (dot_ternary_int4 above). Rows of W_up whose channel
// is dead in every row are never read. One launch, so the up loads of a block overlap the gate loads
// of others.
__global__ __launch_bounds__(WAVES * 64) void k_glu_cond_fused(const uint8_t* __restrict__ A,
                                                               const float* __restrict__ ascale, int M, int K,
                                                               const uint8_t* __restrict__ Wg,
                                                               const float* __restrict__ galpha,
                                                               const uint8_t* __restrict__ Wup,
                                                               const float* __restrict__ upalpha, int N,
                                                               float* __restrict__ Gout, long ldg,
                                                               float* __restrict__ H, long ldh,
                                                               float* __restrict__ rowmax) {
  __shared__ v4i red[WAVES - 1][64];
  __shared__ float gl[8][16];                   // g[row][channel] of the block
  __shared__ float hmax[8][16];                 // |h| for the row maxima
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = blockIdx.x;
  const int KT = K >> 7, NG = N >> 4;
  const int per = (KT + WAVES - 1) / WAVES;
  const int kt_begin = wave * per;
  const int kt_end = min(KT, kt_begin + per);
  const int r = lane & 15, g4 = lane >> 4;
  const long arow = K >> 1;
  const uint8_t* arp = A + (long)min(r, M - 1) * arow + 16 * g4;
  const uint8_t* const wp[2] = {Wg + (uint32_t)G * 512u + (uint32_t)lane * 8u, Wg + (uint32_t)G * 512u + (uint32_t)lane * 8u};
  const uint32_t wstep = (uint32_t)NG * 512u;
  float ds[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) ds[v] = ascale[min(4 * g4 + v, M - 1)];
  const float alpha = *galpha;

  // ---- phase 1: gate projection of the block's 16 channels
  v4i acc[1][2];
  acc[0][0] = acc[0][1] = v4i{0, 0, 0, 0};
  for (int kt0 = kt_begin; kt0 < kt_end; kt0 += CH) {
    if (kt0 + CH <= kt_end) chunk<false, 1, true>(arp, wp, wstep, kt0, kt_end, g4, acc);
    else chunk<false, 1, false>(arp, wp, wstep, kt0, kt_end, g4, acc);
  }
  acc[0][0] += acc[0][1];
  if (wave > 0) red[wave - 1][lane] = acc[0][0];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w) acc[0][0] += red[w][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g4 + v;
      const float g = (float)(acc[0][0][v] >> 10) * (ds[v] * alpha);
      if (m < 8) gl[m][r] = g;
      if (m < M) Gout[(long)m * ldg + 16 * G + r] = g;
    }
  }
  __syncthreads();

  // ---- phase 2: up projection of the live channels (two per wave)
  const float ualpha = *upalpha;
  const long wrow = K >> 2;
  const int KC = K >> 6;
  const int ch0 = 2 * wave;
  bool live[2] = {false, false};
  for (int m = 0; m < M; ++m) {
    live[0] |= gl[m][ch0] > 0.f;
    live[1] |= gl[m][ch0 + 1] > 0.f;
  }
  int uacc[2][8];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int m = 0; m < 8; ++m) uacc[q][m] = 0;
  if (live[0] || live[1]) {
    const uint8_t* wr0 = Wup + (long)(16 * G + ch0) * wrow;
    for (int c = lane; c < KC; c += 64) {
      // both weight rows first (only the live ones), then the codes of the M rows
      uint4 w[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        w[q] = live[q] ? *reinterpret_cast<const uint4*>(wr0 + q * wrow + 16 * c) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m >= M) break;
        const uint4 a0 = *reinterpret_cast<const uint4*>(A + (long)m * arow + 32 * c);
        const uint4 a1 = *reinterpret_cast<const uint4*>(A + (long)m * arow + 32 * c + 16);
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (live[q]) uacc[q][m] = dot_ternary_int4(w[q], a0, a1, uacc[q][m]);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!live[q]) continue;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m >= M) break;
        int v = uacc[q][m];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
        uacc[q][m] = v;
      }
    }
  }
  if (lane < 2 * M) {
    const int q = lane & 1, m = lane >> 1, ch = ch0 + q;
    int u0 = 0, u1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      u0 = (i == m) ? uacc[0][i] : u0;
      u1 = (i == m) ? uacc[1][i] : u1;
    }
    const float um = (float)(q ? u1 : u0);
    const float g = gl[m][ch];
    const float h = g > 0.f ? (g * g) * (um * (ascale[m] * ualpha)) : 0.f;
    H[(long)m * ldh + 16 * G + ch] = h;
    hmax[m][ch] = fabsf(h);
  }
  if (rowmax) {
    __syncthreads();
    if (wave == 0 && lane < M) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) a = fmaxf(a, hmax[lane][c]);
      atomicMax(reinterpret_cast<unsigned int*>(rowmax) + lane, bl_f2u(a));
    }
  }
}

}  // namespace

hipError_t bl_launch_gemv(const bl_mm_args& a, hipStream_t st) {
  if (a.fmt == BL_ACT_INT8) return launch_epi<BL_ACT_INT8>(a, st);
  return launch_epi<BL_ACT_INT4>(a, st);
}

hipError_t bl_launch_glu_conditional_fused(const bl_upcond_args& a, const void* Wg, const float* galpha,
                                          hipStream_t st) {
  hipLaunchKernelGGL(k_glu_cond_fused, dim3(a.N / 16), dim3(WAVES * 64), 0, st, static_cast<const uint8_t*>(a.A),
                     a.ascale, a.M, a.K, static_cast<const uint8_t*>(Wg), galpha, static_cast<const uint8_t*>(a.Wup),
                     a.upalpha, a.N, a.G, a.ldg, a.H, a.ldh, a.rowmax);
  return hipGetLastError();
}
