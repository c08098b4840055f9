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
// INT4 codes that fit in 32 KiB (M K / 2 bytes) are instead copied once per block into LDS with
// direct-to-LDS loads, issued before the weight loads; one barrier after the first chunk's weight
// loads publishes them, and the waves read their activation tiles from LDS rather than each
// loading them through the vector memory path.
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

// s_waitcnt immediate that waits for vector memory operations only, until at most n are outstanding
constexpr int gemv_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

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
// INT8 codes in memory order: the weights of the INT8 products come in the A8 word layout, whose
// expansion (expand_w_i8) is in that k order
__device__ __forceinline__ v4i expand_a_int8(uint4 q) { return v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w}; }

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

// Register cap of the eight-wave INT4 GLU: at most 80 VGPRs leave room for three blocks of eight
// waves per CU, so the 688 blocks of an 11008-wide FFN are resident at once instead of in two rounds.
// LDS copy of the INT4 codes of the M token rows (M K / 2 bytes), taken when they fit: one 16-byte
// direct-to-LDS load per lane, piece i = NWV 64 j + 64 wave + lane of the contiguous rows, instead of
// every wave of every block loading its activation tiles through the vector memory path.
constexpr int ALDS_BYTES = 32768;
template <int NWV>
__device__ __forceinline__ void stage_codes_lds(const uint8_t* __restrict__ A, uint32_t nbytes, uint8_t* acodes,
                                                int wave, int lane) {
  const uint32_t npc = nbytes >> 4;
  for (uint32_t i0 = 64u * wave; i0 < npc; i0 += NWV * 64) {
    if (i0 + lane < npc)
      __builtin_amdgcn_global_load_lds(A + 16u * (i0 + lane), (__attribute__((address_space(3))) void*)(acodes + 16u * i0),
                                       16, 0, 0);
  }
}

// Weights of one chunk of up to CH K tiles from kt0 (kt0 < kt_end; tiles past kt_end repeat the last).
template <int NB, int CH = 4>
__device__ __forceinline__ void load_w_chunk(const uint8_t* const (&wp)[2], uint32_t wstep, int kt0, int kt_end,
                                             uint2 (&wt)[NB][CH]) {
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
    for (int c = 0; c < CH; ++c) wt[mtx][c] = *reinterpret_cast<const uint2*>(wp[mtx] + (uint32_t)min(kt0 + c, kt_end - 1) * wstep);
}
// Matrix-core work of that chunk with the INT4 codes read from an LDS copy of the rows (alds: this
// lane's row and 16-byte column offset). FULL chunks run straight through, so the reads issue together.
template <int NB, bool FULL, int CH = 4>
__device__ __forceinline__ void mfma_chunk_lds(const uint8_t* alds, const uint2 (&wt)[NB][CH], int kt0, int kt_end,
                                               v4i (&acc)[NB][2]) {
  uint4 at[CH];                                 // all reads first (tiles past kt_end repeat the last)
#pragma unroll
  for (int c = 0; c < CH; ++c) at[c] = *reinterpret_cast<const uint4*>(alds + (uint32_t)min(kt0 + c, kt_end - 1) * 64u);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    if (!FULL && kt0 + c >= kt_end) break;
    const uint4 a = at[c];
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx) {
      acc[mtx][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand_a_int4(a.x, a.y), expand_w_i8(wt[mtx][c].x), acc[mtx][0], 0, 0, 0);
      acc[mtx][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(expand_a_int4(a.z, a.w), expand_w_i8(wt[mtx][c].y), acc[mtx][1], 0, 0, 0);
    }
  }
}

template <int FMT, int EPI, int NWV>
constexpr int kGluWaves = (NWV == 8 && EPI == BL_EPI_RELU2_GLU && FMT != BL_ACT_INT8) ? 6 : 1;

template <int FMT, int EPI, int CHN, int NWV, bool ALDS>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(kGluWaves<FMT, EPI, NWV>))) void k_gemv(const uint8_t* __restrict__ A, const float* __restrict__ ascale,
                                                     int M, int K, const uint8_t* W,
                                                     const float* __restrict__ walpha,
                                                     const uint8_t* W2,
                                                     const float* __restrict__ w2alpha, int N,
                                                     float* __restrict__ Y, long ldy, const float* R, long ldr,
                                                     float* __restrict__ rowmax) {
  constexpr bool A8 = (FMT == BL_ACT_INT8);
  constexpr int NB = (EPI == BL_EPI_RELU2_GLU) ? 2 : 1;
  static_assert(!ALDS || FMT == BL_ACT_INT4, "LDS-staged codes are INT4 only");
  __shared__ v4i red[NB][NWV - 1][64];
  __shared__ __attribute__((aligned(16))) uint8_t acodes[ALDS ? ALDS_BYTES : 16];

  // (the wave index sits in a scalar register in the single-matrix kernels, which measured faster
  // that way; in the two-matrix one it needs registers the three-blocks-per-CU cap does not leave)
  const int lane = threadIdx.x & 63;
  const int wave = NB == 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : (int)(threadIdx.x >> 6);
  const int G = blockIdx.x;
  const int KT = K >> 7, NG = N >> 4;            // 128-wide weight tiles along K, 16-row groups
  const int per = (KT + NWV - 1) / NWV;
  const int kt_begin = wave * per;
  const int kt_end = min(KT, kt_begin + per);
  const int r = lane & 15, g = lane >> 4;
  const int n = 16 * G + r;
  const uint32_t arow = A8 ? K : (K >> 1);
  const uint8_t* arp = A + (uint32_t)min(r, M - 1) * arow + (A8 ? 32 * g : 16 * g);
  // (the weight pointers are not __restrict__: their loads must stay where they are issued, ahead of
  // the barrier below, which a load the compiler may treat as invariant need not)
  const uint32_t woff = (uint32_t)G * 512u + (uint32_t)lane * 8u;
  const uint8_t* const wp[2] = {W + woff, (NB > 1 ? W2 : W) + woff};
  const uint32_t wstep = (uint32_t)NG * 512u;
  if constexpr (ALDS) {
    stage_codes_lds<NWV>(A, (uint32_t)M * arow, acodes, wave, lane);
    asm volatile("" ::: "memory");   // every later load is issued after the copy
  }

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
  if constexpr (ALDS) {
    // the first chunk's weights are in flight across the barrier that publishes the LDS codes
    const uint8_t* alds = acodes + (uint32_t)min(r, M - 1) * arow + 16 * g;
    uint2 wt[NB][CHN];
    // every wave issues the first chunk's NB * CHN weight loads after the copy (a wave without K
    // tiles loads valid, unused words), so the copy has landed once at most those are outstanding;
    // the barrier does not wait for the weights, and each wave starts on a tile as soon as it arrives
    // (the flag is made wave-uniform so that the compiler counts those loads exactly)
    const bool work = __builtin_amdgcn_readfirstlane((int)(kt_begin < kt_end)) != 0;
    load_w_chunk<NB, CHN>(wp, wstep, work ? kt_begin : KT - 1, work ? kt_end : KT, wt);
    __builtin_amdgcn_s_waitcnt(gemv_vmcnt(NB * CHN));
    asm volatile("s_barrier" ::: "memory");
    if (work) {
      if (kt_begin + CHN <= kt_end) mfma_chunk_lds<NB, true, CHN>(alds, wt, kt_begin, kt_end, acc);
      else mfma_chunk_lds<NB, false, CHN>(alds, wt, kt_begin, kt_end, acc);
      for (int kt0 = kt_begin + CHN; kt0 < kt_end; kt0 += CHN) {
        load_w_chunk<NB, CHN>(wp, wstep, kt0, kt_end, wt);
        if (kt0 + CHN <= kt_end) mfma_chunk_lds<NB, true, CHN>(alds, wt, kt0, kt_end, acc);
        else mfma_chunk_lds<NB, false, CHN>(alds, wt, kt0, kt_end, acc);
      }
    }
  } else {
    for (int kt0 = kt_begin; kt0 < kt_end; kt0 += CHN) {
      if (kt0 + CHN <= kt_end) chunk<A8, NB, true, CHN>(arp, wp, wstep, kt0, kt_end, g, acc);
      else chunk<A8, NB, false, CHN>(arp, wp, wstep, kt0, kt_end, g, acc);
    }
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
        // maximum of |h| over the 16 columns (lanes of one DPP row); non-negative floats order
        // as their bit patterns
        uint32_t a = bl_f2u(fabsf(out));
        a = max(a, bl_dpp<0xB1>(a));               // quad_perm(1, 0, 3, 2)
        a = max(a, bl_dpp<0x4E>(a));               // quad_perm(2, 3, 0, 1)
        a = max(a, bl_dpp<0x141>(a));              // row_half_mirror
        a = max(a, bl_dpp<0x140>(a));              // row_mirror
        if (r == 0 && m < M) atomicMax(reinterpret_cast<unsigned int*>(rowmax) + m, a);
      }
    }
  }
}

template <int FMT, int EPI, int CHN, int NWV>
hipError_t launch_w(const bl_mm_args& a, hipStream_t st) {
  const bool alds = FMT == BL_ACT_INT4 && (long)a.M * (a.K / 2) <= ALDS_BYTES;
  hipLaunchKernelGGL((alds ? k_gemv<FMT, EPI, CHN, NWV, FMT == BL_ACT_INT4> : k_gemv<FMT, EPI, CHN, NWV, false>),
                     dim3(a.N / 16), dim3(NWV * 64), 0, st,
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

// Sum of an int32 over the 64 lanes of a wave, returned wave-uniform: DPP exchanges inside each row
// of 16 lanes (xor 1, xor 2, then the half-row and row mirrors), then the four row sums by readlane.
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm(1, 0, 3, 2)
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm(2, 3, 0, 1)
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}

// Fused form for one block per 16-channel group (the tile row of W_gate). At the start the block
// copies the M rows of INT4 codes into LDS (direct-to-LDS loads, when they fit), then phase 1 is
// the INT4 decode GEMV of the gate (eight waves split K, partial int32 tiles in LDS). After one
// barrier each wave sums the partials of its own two channels (lanes 2 m + q: row m, channel
// 2 wave + q), writes g, and if the gate of a channel is positive in some row streams that
// channel's row-major up weights (K/4 bytes; 16 bytes per lane and 64-wide K slice) against the
// codes in LDS with v_dot8 (dot_ternary_int4 above); the row sums are wave reductions by DPP.
// Rows of W_up whose channel is dead in every row are never read. One launch, so the up loads of a
// block overlap the gate loads of others; at most 80 VGPRs keep three blocks per CU resident.
template <bool ALDS>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(6))) void k_glu_cond_fused(
    const uint8_t* __restrict__ A, const float* __restrict__ ascale, int M, int K, const uint8_t* Wg,
    const float* __restrict__ galpha, const uint8_t* __restrict__ Wup, const float* __restrict__ upalpha, int N,
    float* __restrict__ Gout, long ldg, float* __restrict__ H, long ldh, float* __restrict__ rowmax) {
  __shared__ v4i red[WAVES][64];
  __shared__ __attribute__((aligned(16))) uint8_t acodes[ALDS ? ALDS_BYTES : 16];
  __shared__ float hmax[8][16];                 // |h| for the row maxima
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = blockIdx.x;
  const int KT = K >> 7, NG = N >> 4;
  const int per = (KT + WAVES - 1) / WAVES;
  const int kt_begin = wave * per;
  const int kt_end = min(KT, kt_begin + per);
  const int r = lane & 15, g4 = lane >> 4;
  const uint32_t arow = (uint32_t)K >> 1;
  if constexpr (ALDS) {
    stage_codes_lds<WAVES>(A, (uint32_t)M * arow, acodes, wave, lane);
    asm volatile("" ::: "memory");               // every later load is issued after the copy
  }
  const uint8_t* arp = A + (uint32_t)min(r, M - 1) * arow + 16 * g4;
  const uint8_t* const wp[2] = {Wg + (uint32_t)G * 512u + (uint32_t)lane * 8u, Wg + (uint32_t)G * 512u + (uint32_t)lane * 8u};
  const uint32_t wstep = (uint32_t)NG * 512u;
  // lanes 2 m + q < 2 M own (row m, channel 2 wave + q) from the handover on
  const int om = lane >> 1, oq = lane & 1, och = 2 * wave + oq;
  const bool owner = lane < 2 * M;
  const float ods = ascale[min(om, M - 1)];
  const float alpha = *galpha, ualpha = *upalpha;

  // ---- phase 1: gate projection of the block's 16 channels
  v4i acc[1][2];
  acc[0][0] = acc[0][1] = v4i{0, 0, 0, 0};
  if constexpr (ALDS) {
    // every wave issues the first chunk's CH gate-weight loads after the copy (valid addresses also
    // without a K tile), so the copy has landed once at most those are outstanding; the barrier
    // that publishes it does not wait for the weights (the gate pointer is not __restrict__, so
    // the compiler keeps these loads ahead of the barrier)
    const uint8_t* alds = acodes + (uint32_t)min(r, M - 1) * arow + 16 * g4;
    uint2 wt[1][CH];
    const bool work = kt_begin < kt_end;
    load_w_chunk<1>(wp, wstep, work ? kt_begin : KT - 1, work ? kt_end : KT, wt);
    __builtin_amdgcn_s_waitcnt(gemv_vmcnt(CH));
    asm volatile("s_barrier" ::: "memory");
    if (work) {
      if (kt_begin + CH <= kt_end) mfma_chunk_lds<1, true>(alds, wt, kt_begin, kt_end, acc);
      else mfma_chunk_lds<1, false>(alds, wt, kt_begin, kt_end, acc);
      for (int kt0 = kt_begin + CH; kt0 < kt_end; kt0 += CH) {
        load_w_chunk<1>(wp, wstep, kt0, kt_end, wt);
        if (kt0 + CH <= kt_end) mfma_chunk_lds<1, true>(alds, wt, kt0, kt_end, acc);
        else mfma_chunk_lds<1, false>(alds, wt, kt0, kt_end, acc);
      }
    }
  } else {
    for (int kt0 = kt_begin; kt0 < kt_end; kt0 += CH) {
      if (kt0 + CH <= kt_end) chunk<false, 1, true>(arp, wp, wstep, kt0, kt_end, g4, acc);
      else chunk<false, 1, false>(arp, wp, wstep, kt0, kt_end, g4, acc);
    }
  }
  red[wave][lane] = acc[0][0] + acc[0][1];
  __syncthreads();

  // ---- handover: g of the wave's two channels, exact int32 sum of the eight partial tiles (the
  // value of row m, channel c sits in tile lane c + 16 (m / 4), component m % 4)
  float g = 0.f;
  if (owner) {
    const int* rp = reinterpret_cast<const int*>(&red[0][och + 16 * (om >> 2)]) + (om & 3);
    int s = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += rp[w * 64 * 4];
    g = (float)(s >> 10) * (ods * alpha);
    Gout[(long)om * ldg + 16 * G + och] = g;
  }
  const unsigned long long pos = __ballot(owner && g > 0.f);
  const bool live0 = (pos & 0x5555555555555555ull) != 0ull, live1 = (pos & 0xAAAAAAAAAAAAAAAAull) != 0ull;

  // ---- phase 2: up projection of the live channels
  int us[2][8];                                 // wave-uniform row sums
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int m = 0; m < 8; ++m) us[q][m] = 0;
  if (live0 || live1) {
    const uint32_t wrow = (uint32_t)K >> 2;
    const int KC = K >> 6;
    const uint8_t* wr0 = Wup + (long)(16 * G + 2 * wave) * wrow;
    int uacc[2][8];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int m = 0; m < 8; ++m) uacc[q][m] = 0;
    for (int c = lane; c < KC; c += 64) {
      // both weight rows first (only the live ones), then the codes of the M rows
      const uint4 w0 = live0 ? *reinterpret_cast<const uint4*>(wr0 + 16u * c) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 w1 = live1 ? *reinterpret_cast<const uint4*>(wr0 + wrow + 16u * c) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m >= M) break;
        const uint8_t* ap = (ALDS ? acodes : A) + (uint32_t)m * arow + 32u * c;
        const uint4 a0 = *reinterpret_cast<const uint4*>(ap);
        const uint4 a1 = *reinterpret_cast<const uint4*>(ap + 16);
        if (live0) uacc[0][m] = dot_ternary_int4(w0, a0, a1, uacc[0][m]);
        if (live1) uacc[1][m] = dot_ternary_int4(w1, a0, a1, uacc[1][m]);
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m >= M) break;
      if (live0) us[0][m] = wave_sum_i32(uacc[0][m]);
      if (live1) us[1][m] = wave_sum_i32(uacc[1][m]);
    }
  }
  if (owner) {
    int u = 0;
#pragma unroll
    for (int m = 0; m < 8; ++m) u = (m == om) ? (oq ? us[1][m] : us[0][m]) : u;
    const float h = g > 0.f ? (g * g) * ((float)u * (ods * ualpha)) : 0.f;
    H[(long)om * ldh + 16 * G + och] = h;
    hmax[om][och] = fabsf(h);
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
  const bool alds = (long)a.M * (a.K / 2) <= ALDS_BYTES;
  hipLaunchKernelGGL(alds ? k_glu_cond_fused<true> : k_glu_cond_fused<false>, dim3(a.N / 16), dim3(WAVES * 64), 0, st,
                     static_cast<const uint8_t*>(a.A), a.ascale, a.M, a.K, static_cast<const uint8_t*>(Wg), galpha,
                     static_cast<const uint8_t*>(a.Wup), a.upalpha, a.N, a.G, a.ldg, a.H, a.ldh, a.rowmax);
  return hipGetLastError();
}
