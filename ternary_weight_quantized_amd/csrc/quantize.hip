// Per-token activation quantizers: INT4 absmean, FP4 E2M1 (MinMax or power-of-two scale), INT8 absmax
// with Top-K mask.
//
// "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up), section 3.4:
//   "4-Bit Activation Quantization for Gaussian-Like Inputs" (INT4 absmean, paper Eq. 6-7;
//    FP4 MinMax E2M1, paper Eq. 8-9) and "Sparsification Pipeline for Outlier-Heavy
//    Intermediate States" (Top-K mask and INT8 absmax, paper Eq. 1).
//
// Kernels, by case:
//  - k_quant_blk: every format without a Top-K mask, rows of up to 16384 elements. One 256-thread
//    block per row; thread t owns the 8-element chunks t, t + 256, ... of the row.
//  - k_topk_blk: INT8 with the Top-K mask for bf16 rows of up to 8192 elements, one block per row.
//  - k_quant_res / k_quant_stream: the remaining cases (float32 rows with a Top-K mask, longer
//    rows). One wave64 owns one token row, four rows per block; a lane owns four consecutive
//    elements of every 256-element group (group g, elements 256g + 4*lane .. +3; when K % 256 ==
//    128 the last group is half, lanes 32..63 hold nothing). k_quant_res (INT8 with Top-K of float32
//    rows of up to 4096 elements) keeps the row in registers between the threshold search and the
//    codes ("resident"); k_quant_stream reads longer rows again from global memory ("streaming").
//  - k_tensor_*: the statistics of the per-tensor variant.
#include <algorithm>

#include "bl_common.h"
#include "bl_kernels.h"

namespace {

template <int IN_F32>
__device__ __forceinline__ void load4(const void* __restrict__ x, long off, float (&o)[4]) {
  if (IN_F32) {
    const float4 t = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    o[0] = t.x; o[1] = t.y; o[2] = t.z; o[3] = t.w;
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + off);
    o[0] = bl_bf16lo(t.x); o[1] = bl_bf16hi(t.x); o[2] = bl_bf16lo(t.y); o[3] = bl_bf16hi(t.y);
  }
}

__device__ __forceinline__ int ceil_log2(int K) { return K <= 1 ? 0 : 32 - __clz(K - 1); }

// Accumulators of the absmean sum: double sum plus the exponent range of the nonzero terms.
struct AbsSum {
  double s = 0.0;
  // largest magnitude bits, and smallest nonzero magnitude bits minus one (a zero gives 0xFFFFFFFF
  // and never wins the minimum): two integer ops per element, no branch
  uint32_t bmax = 0u, bmin1 = 0xFFFFFFFFu;
  __device__ __forceinline__ void add(float v) {
    const uint32_t b = bl_f2u(v) & 0x7FFFFFFFu;
    s += (double)bl_u2f(b);
    bmax = b > bmax ? b : bmax;
    bmin1 = b - 1u < bmin1 ? b - 1u : bmin1;
  }
  // two bf16 values from one dword (low half first), their floats given: the exponent bounds run on
  // the 16-bit halves at once (a bf16 magnitude is the top half of its float's magnitude bits)
  __device__ __forceinline__ void add_bf16_pair(uint32_t d, float lo, float hi, uint32_t& pmax, uint32_t& pmin1) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    s += (double)fabsf(lo);
    s += (double)fabsf(hi);
    const us2 m = __builtin_bit_cast(us2, d & 0x7FFF7FFFu);
    pmax = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, pmax), m));
    pmin1 = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(us2, pmin1), m - (us2)1));
  }
  // fold the packed bounds of add_bf16_pair into bmax / bmin1 (bmin1 stays 0xFFFFFFFF when every
  // value was zero: m - 1 wraps to 0xFFFF for a zero half)
  __device__ __forceinline__ void fold_bf16(uint32_t pmax, uint32_t pmin1) {
    const uint32_t hmax = max(pmax & 0xFFFFu, pmax >> 16), hmin1 = min(pmin1 & 0xFFFFu, pmin1 >> 16);
    const uint32_t b = hmax << 16, b1 = hmin1 == 0xFFFFu ? 0xFFFFFFFFu : ((hmin1 + 1u) << 16) - 1u;
    bmax = b > bmax ? b : bmax;
    bmin1 = b1 < bmin1 ? b1 : bmin1;
  }
  __device__ __forceinline__ void merge(const AbsSum& o) {
    s += o.s;                          // exact whenever the span check holds for all the terms
    bmax = o.bmax > bmax ? o.bmax : bmax;
    bmin1 = o.bmin1 < bmin1 ? o.bmin1 : bmin1;
  }
  // biased exponents of the largest magnitude and of the smallest nonzero one, packed as
  // (emax << 16) | (255 - emin), so that one packed 16-bit maximum reduces both; all zero -> emin 0xFF
  __device__ __forceinline__ uint32_t exps() const {
    const uint32_t emin = bmin1 == 0xFFFFFFFFu ? 0xFFu : (bmin1 + 1u) >> 23;
    return ((bmax >> 23) << 16) | (255u - emin);
  }
};
__device__ __forceinline__ uint32_t exps_emax(uint32_t p) { return p >> 16; }
__device__ __forceinline__ uint32_t exps_emin(uint32_t p) { return 255u - (p & 0xFFFFu); }
// packed (emax, 255 - emin) maximum over the wave: both halves at once
__device__ __forceinline__ uint32_t wave_max_exps(uint32_t p) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  return bl_wave_reduce_u(p, [](uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
  });
}

// Exact-bins fallback for one wave: called only when the double sum might have rounded.
__device__ __forceinline__ void bins_clear(unsigned long long* bins, int lane) {
  for (int i = lane; i < 256; i += 64) bins[i] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
__device__ __forceinline__ void bins_add(unsigned long long* bins, float v) {
  uint32_t e, m;
  bl_bin_split(bl_f2u(v) & 0x7FFFFFFFu, &e, &m);
  if (m) atomicAdd(&bins[e], (unsigned long long)m);
}
__device__ __forceinline__ double bins_finish(unsigned long long* bins, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  double s = 0.0;
  if (lane == 0) s = bl_bins_to_double(bins);
  return __shfl(s, 0, 64);
}

// Is the double-precision sum of the row exact? All terms are multiples of 2^(max(emin,1)-150+24-sig)
// and the total is below K * 2^(emax-126); exact when that integer count fits in 53 bits.
template <int IN_F32>
__device__ __forceinline__ bool sum_is_exact(uint32_t emax, uint32_t emin, int K) {
  if (emin == 0xFFu) return true;                // all zero
  const int e1 = emin < 1u ? 1 : (int)emin;
  return ((int)emax - e1 + (IN_F32 ? 24 : 8) + ceil_log2(K)) <= 53;
}

// --- per element code functions (float32, one IEEE operation each) ---------------------------
// INT4 code k = RoundClip(RN32(v s), -8, 7). Clamping before rounding gives the same integer (the
// bounds are integers). y + 1.5 2^23 for y in [-8, 7] lies in [2^23, 2^24), where the binary32
// spacing is 1, so that one addition rounds y to the nearest integer with ties to even (as rint)
// and leaves k in the low mantissa bits as a two's complement number: the low nibble of the result
// is the nibble code, its low byte k & 0xFF.
__device__ __forceinline__ uint32_t rne_bits_int4(float v, float s) {
  return bl_f2u(__builtin_amdgcn_fmed3f(v * s, -8.f, 7.f) + 12582912.0f);
}
__device__ __forceinline__ uint32_t code_int4(float v, float s) { return rne_bits_int4(v, s) & 0xFu; }
// Eight INT4 codes as one word, nibble j = the code of v[j]: byte permutes gather the low bytes of
// the even and of the odd elements into two words, whose low nibbles are then interleaved.
__device__ __forceinline__ uint32_t codes_int4_8(const float (&v)[8], float s) {
  uint32_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = rne_bits_int4(v[j], s);
  // selector bytes 0..3 take bytes of the second operand, 4..7 of the first, 12 gives 0
  const uint32_t ev = __builtin_amdgcn_perm(b[2], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[6], b[4], 0x04000C0Cu);
  const uint32_t od = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[5], 0x04000C0Cu);
  return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}
// FP4 E2M1 codes of p = RN32(v * s), two per byte (the first in the low nibble), through the CDNA4
// conversion v_cvt_scalef32_pk_fp4_f32 at scale 1: it rounds to nearest with ties to the even
// mantissa and saturates at 6 (checked against the threshold form on every binary32 value from
// 2^-10 to 2^6 and on zeros, subnormals and values up to the largest finite one). It keeps the
// sign of a negative value that rounds to zero (code 8); fp4_clear_negzero turns those into 0.
__device__ __forceinline__ uint32_t fp4_clear_negzero(uint32_t w) {
  const uint32_t m = w & 0x77777777u;                 // magnitudes; m + 7 carries into bit 3 iff m != 0
  return m | (w & (m + 0x77777777u) & 0x88888888u);
}
__device__ __forceinline__ uint32_t codes_fp4_4(float a, float b, float c, float d, float s) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a * s, b * s, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, c * s, d * s, 1.0f, 1);
  return fp4_clear_negzero(w & 0xFFFFu);
}
__device__ __forceinline__ uint32_t codes_fp4_8(const float (&v)[8], float s) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0] * s, v[1] * s, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * s, v[3] * s, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * s, v[5] * s, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * s, v[7] * s, 1.0f, 3);
  return fp4_clear_negzero(w);
}
__device__ __forceinline__ uint32_t code_int8(float v, float s) {
  return (uint32_t)bl_roundclip(v * s, -128.f, 127.f) & 0xFFu;
}
// INT4 code c = RoundClip(v * s, -8, 7) -> its exact FP6 E3M2 bit pattern (sign bit 5, exponent bias
// 3, 2 mantissa bits), read off the binary32 form of the rounded value: for |c| >= 1 the E3M2
// exponent and mantissa are the binary32 exponent - 124 and its top two mantissa bits, so the
// pattern is (|bits| >> 21) - 496; c = 0 gives 0 (the + 0 turns a -0 into +0).
__device__ __forceinline__ uint32_t code_e3m2(float v, float s) {
  const float r = fminf(fmaxf(__builtin_rintf(v * s), -8.f), 7.f) + 0.0f;
  const uint32_t b = bl_f2u(r);
  const int mag = (int)((b & 0x7FFFFFFFu) >> 21) - 496;
  return (uint32_t)(mag > 0 ? mag : 0) | ((b >> 26) & 0x20u);
}

// The E3M2 patterns of the INT4 codes of two chunks of 8 values (p, then q) through one CDNA4
// conversion: the rounded and clamped codes are exact E3M2 values, so v_cvt_scalef32_2xpk16_bf6_f32
// at scale 1 writes their patterns. It places element i of its first operand at code 2i and element
// i of its second at code 2i + 1 (an in-bounds probe of the instruction on the GPU showed this), so
// the even and the odd elements go to the two operands; codes 16..31 are not used. A rounded -0
// becomes +0 first (the conversion keeps the sign of zero). w[0] and the low half of w[1] hold p's
// 48 bits, the high half of w[1] and w[2] q's (code k at bits 6 k).
typedef float v16f_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ void codes_e3m2_16(const float (&p)[8], const float (&q)[8], float s, uint32_t (&w)[3]) {
  v16f_t a = __builtin_nondeterministic_value(a), b = __builtin_nondeterministic_value(b);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = __builtin_rintf(__builtin_amdgcn_fmed3f(p[2 * j] * s, -8.f, 7.f)) + 0.0f;
    b[j] = __builtin_rintf(__builtin_amdgcn_fmed3f(p[2 * j + 1] * s, -8.f, 7.f)) + 0.0f;
    a[4 + j] = __builtin_rintf(__builtin_amdgcn_fmed3f(q[2 * j] * s, -8.f, 7.f)) + 0.0f;
    b[4 + j] = __builtin_rintf(__builtin_amdgcn_fmed3f(q[2 * j + 1] * s, -8.f, 7.f)) + 0.0f;
  }
  const auto o = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
  w[0] = o[0]; w[1] = o[1]; w[2] = o[2];
}
// 48 bits of 8 E3M2 codes (lo: bits 0..31, hi: bits 32..47) at byte 6 ch of an LDS row
__device__ __forceinline__ void put_e3m2_48(uint8_t* erow, int ch, uint32_t lo, uint32_t hi) {
  uint8_t* d = erow + 6 * ch;
  if ((ch & 1) == 0) {
    *reinterpret_cast<uint32_t*>(d) = lo;
    *reinterpret_cast<uint16_t*>(d + 4) = (uint16_t)hi;
  } else {
    *reinterpret_cast<uint16_t*>(d) = (uint16_t)lo;
    *reinterpret_cast<uint32_t*>(d + 2) = (lo >> 16) | (hi << 16);
  }
}

// Store the 4 codes (24 bits, code j at bits 6j) of elements 256g + 4 lane .. +3 of row m into the
// tiled E3M2 layout (16 rows x 128 codes per 1536-byte tile, 96 bytes per row, code k at bits 6k):
// four lanes make 12 bytes, written as three dwords. Every lane takes part in the shuffle; only lanes
// holding elements (ok, whole groups of four) store.
__device__ __forceinline__ void store_e3m2(uint8_t* __restrict__ codes, int m, int K, int g, int lane, uint32_t v24,
                                           bool ok) {
  const uint32_t nxt = __shfl_down(v24, 1, 64);
  const int i = lane & 3, q = lane >> 2;
  const uint32_t w = i == 0 ? (v24 | (nxt << 24)) : i == 1 ? ((v24 >> 8) | (nxt << 16)) : ((v24 >> 16) | (nxt << 8));
  const long tile = (long)(m >> 4) * (K >> 7) + 2 * g + (q >> 3);
  if (i < 3 && ok) *reinterpret_cast<uint32_t*>(codes + tile * 1536 + (m & 15) * 96 + 12 * (q & 7) + 4 * i) = w;
}

// FP4 scales from the row maximum gamma. MinMax (BL_ACT_FP4_E2M1): the maximum maps to 6,
// s = RN32(6 / RN32(gamma + eps)), dequant gamma / 6. Power of two (BL_ACT_FP4_E2M1_POW2): the dequant
// scale is 2^p with p the smallest integer such that 6 * 2^p >= gamma (p >= -126), s = 2^-p, so
// x * s is exact; an all-zero row gets s = 0 and scale 0.
template <bool POW2>
__device__ __forceinline__ void fp4_scales(float gamma, float eps, float* s, float* dscale) {
  if constexpr (!POW2) {
    *s = 6.0f / (gamma + eps);
    *dscale = gamma / 6.0f;
  } else {
    const uint32_t b = bl_f2u(gamma);
    const int E = (int)(b >> 23);
    int p = E == 0 ? -126 : ((b & 0x7FFFFFu) <= 0x400000u ? E - 129 : E - 128);   // e - 2 or e - 1
    p = p < -126 ? -126 : p;
    *s = gamma == 0.0f ? 0.0f : bl_u2f((uint32_t)(127 - p) << 23);
    *dscale = gamma == 0.0f ? 0.0f : bl_u2f((uint32_t)(127 + p) << 23);
  }
}

// Top-K threshold: the largest key T with count(|x| >= T) >= keep, found bit by bit.
// bf16 inputs have 16 zero low bits in their float32 key, so their search stops at bit 16.
// Ballot + popcount make each count a scalar: no cross-lane reduction is needed.
template <typename CountFn>
__device__ __forceinline__ uint32_t topk_threshold(int keep, int lo_bit, CountFn count_ge) {
  uint32_t T = 0u;
  for (int b = 30; b >= lo_bit; --b) {
    const uint32_t cand = T | (1u << b);
    if (count_ge(bl_u2f(cand)) >= keep) T = cand;
  }
  return T;
}

// Mask word assembly: lane holds a nibble for elements 4*lane..4*lane+3 of a 256-group; eight
// lanes make one 32-bit word (bit k % 32 of word k / 32).
__device__ __forceinline__ void store_mask_nibble(uint32_t* __restrict__ mrow, int g, int lane, uint32_t nib,
                                                  bool ok) {
  uint32_t w = nib << (4 * (lane & 7));
  w |= __shfl_xor(w, 1, 64);
  w |= __shfl_xor(w, 2, 64);
  w |= __shfl_xor(w, 4, 64);
  if ((lane & 7) == 0 && ok) mrow[8 * g + (lane >> 3)] = w;
}

// ============================================================================ resident kernel
// INT8 with a Top-K mask for float32 rows of up to 4096 elements (the only case the block-per-row
// kernels do not take at that length): one wave per row, the row held in registers between the
// threshold search and the codes. Group g holds elements 256 g + 4 lane .. +3; when K % 256 == 128
// the last group is a half group whose lanes 32..63 hold nothing (zeros, excluded from the ties and
// from every store).
template <int IN_F32, int NGMAX>
__global__ __launch_bounds__(256) void k_quant_res(const void* __restrict__ x, int M, int K, long ldx,
                                                   int keep, float eps, const float* __restrict__ hint,
                                                   uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                   uint32_t* __restrict__ mask) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= M) return;                         // wave-uniform; no block barriers below
  const int NG = (K + 255) >> 8;
  const long base = (long)row * ldx + 4 * lane;
  float v[NGMAX][4];
  bool ok[NGMAX];
#pragma unroll
  for (int g = 0; g < NGMAX; ++g) {
    ok[g] = g < NG && 256 * g + 4 * lane < K;
    if (ok[g]) load4<IN_F32>(x, base + 256 * g, v[g]);
    else v[g][0] = v[g][1] = v[g][2] = v[g][3] = 0.0f;
  }
  // gamma = max |x| over the whole row (exact)
  float gamma;
  if (hint) {
    gamma = hint[row];
  } else {
    uint32_t mx = 0u;
#pragma unroll
    for (int g = 0; g < NGMAX; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t b = bl_f2u(v[g][j]) & 0x7FFFFFFFu;
        mx = b > mx ? b : mx;
      }
    gamma = bl_u2f(bl_wave_max_u(mx));
  }
  const float s = 127.0f / (gamma + eps);
  const bool all = keep < 0 || keep >= K;
  const bool none = keep == 0;
  float Tf = 0.0f;
  int need = 0;
  if (!all && !none) {
    // every candidate threshold is > 0, so the zeros of missing lanes never count
    auto count_ge = [&](float c) {
      int n = 0;
#pragma unroll
      for (int g = 0; g < NGMAX; ++g)
        if (g < NG) {
#pragma unroll
          for (int j = 0; j < 4; ++j) n += __popcll(__ballot(fabsf(v[g][j]) >= c));
        }
      return n;
    };
    Tf = bl_u2f(topk_threshold(keep, IN_F32 ? 0 : 16, count_ge));
    int greater = 0;
#pragma unroll
    for (int g = 0; g < NGMAX; ++g)
      if (g < NG) {
#pragma unroll
        for (int j = 0; j < 4; ++j) greater += __popcll(__ballot(fabsf(v[g][j]) > Tf));
      }
    need = keep - greater;                    // >= 1 ties at T survive, lowest index first
  }
  uint32_t* crow = reinterpret_cast<uint32_t*>(codes + (long)row * K) + lane;
  uint32_t* mrow = mask ? mask + (long)row * (K >> 5) : nullptr;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int tie_base = 0;
#pragma unroll
  for (int g = 0; g < NGMAX; ++g)
    if (g < NG) {
      uint32_t keepbits;
      if (all) {
        keepbits = 0xFu;
      } else if (none) {
        keepbits = 0u;
      } else {
        uint32_t gt = 0u, eq = 0u;
        int before = 0, tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = fabsf(v[g][j]);
          gt |= (a > Tf ? 1u : 0u) << j;
          const bool t = ok[g] && a == Tf;
          eq |= (t ? 1u : 0u) << j;
          const unsigned long long bal = __ballot(t);
          before += __popcll(bal & lt);
          tot += __popcll(bal);
        }
        // rank of this lane's ties = ties of earlier groups + of lower lanes + of lower j
        int rank = tie_base + before;
        uint32_t kb = gt;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if ((eq >> j) & 1u) { kb |= (rank < need ? 1u : 0u) << j; ++rank; }
        keepbits = kb;
        tie_base += tot;
      }
      uint32_t c = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if ((keepbits >> j) & 1u) c |= code_int8(v[g][j], s) << (8 * j);
      if (ok[g]) crow[64 * g] = c;
      if (mrow) store_mask_nibble(mrow, g, lane, keepbits, ok[g]);
    }
  if (lane == 0) scale[row] = gamma / 127.0f;
}

// ============================================================================ Top-K, block per row
// INT8 absmax with the Top-K mask for bf16 rows (K <= 8192), one 256-thread block per row. Thread t
// owns the 8-element chunks t, t + 256, ... (one 16-byte load each). The threshold key T (the
// largest 15-bit magnitude key with count(key >= T) >= keep) comes from two radix passes over LDS
// histograms, 8 copies (thread t adds to copy t % 8, so a wave's 64 increments spread over 8
// copies): exponents (key >> 7), then the mantissas of the keys whose exponent is T's. Copies are
// interleaved in groups of four (bin b of copy 4g + i is word 4b + i of group g), so one 16-byte
// read returns a bin of four copies and the clears are 16-byte stores. Bin counts
// are summed over the copies, scanned in descending key order across the block, and the bin where
// the running count reaches keep gives the next digit. Ties at T are ranked by index with one block
// scan of the per-thread tie counts of every chunk. Codes: RN32(x * s) is rounded to an integer by
// adding 1.5 * 2^23 (round to nearest even; |x * s| < 127.5 always, so no clamping is needed) and
// its low byte is the two's-complement code. A 32-element mask word comes from 4 neighbouring threads.
constexpr int TK_COPIES = 8, TK_STRIDE = 264;      // 256 bins + 8 pad words per copy
constexpr int TK_GROUP = 4 * TK_STRIDE;            // words per group of four interleaved copies

// Inclusive scan of one int per thread over the 256-thread block; returns (inclusive, total). The
// caller places a barrier between this scan's reads of wtot and the next write of the same array.
__device__ __forceinline__ int2 tk_block_scan(int v, int* wtot, int t) {
  const int lane = t & 63, wave = t >> 6;
  const int incl = bl_wave_incl_scan(v, lane);
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    off += w < wave ? wtot[w] : 0;
    tot += wtot[w];
  }
  return make_int2(incl + off, tot);
}

typedef unsigned short tk_u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ tk_u16x2 tk_pk(uint32_t v) { return __builtin_bit_cast(tk_u16x2, v); }
__device__ __forceinline__ uint32_t tk_unpk(tk_u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
// Bits 15 and 31 of q0..q3 (one flag per 16-bit half; half h of q_i is element 2i + h of a chunk)
// gathered into bit 2i + h of one byte.
__device__ __forceinline__ uint32_t tk_fold(uint32_t q0, uint32_t q1, uint32_t q2, uint32_t q3) {
  const uint32_t f = (q0 >> 15) | (q1 >> 13) | (q2 >> 11) | (q3 >> 9);   // bits 0,2,4,6 and 16,18,20,22
  return (f | (f >> 15)) & 0xFFu;
}
// 0xFF in byte k where bit k of n (k < 4) is set, else 0x00 (v_perm selector 13 gives 0xFF, 12 gives 0)
__device__ __forceinline__ uint32_t tk_byte_mask(uint32_t n) {
  return __builtin_amdgcn_perm(0u, 0u, 0x0C0C0C0Cu + (((n & 0xFu) * 0x00204081u) & 0x01010101u));
}

template <int NCH>
__global__ __launch_bounds__(256) void k_topk_blk(const uint16_t* __restrict__ x, int M, int K, long ldx, int keep,
                                                  float eps, const float* __restrict__ hint,
                                                  uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                  uint32_t* __restrict__ mask) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[TK_COPIES * TK_STRIDE];
  __shared__ int wtot[4];
  __shared__ int wtot_v[NCH][4];
  __shared__ uint32_t wmax[4];
  __shared__ int sel[2];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x;
  const int nch = K >> 3;
  uint4 w[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (t + 256 * c < nch) w[c] = *reinterpret_cast<const uint4*>(x + (long)row * ldx + 8 * (t + 256 * c));
    else w[c] = make_uint4(0u, 0u, 0u, 0u);
  const bool all = keep < 0 || keep >= K;
  const bool search = !all && keep > 0;            // block-uniform
  uint4* hist4 = reinterpret_cast<uint4*>(hist);
  // the histogram is cleared while the row loads are in flight; the barrier of the row maximum (or
  // the one below, with a given maximum) orders the clear before the first atomic
  if (search)
    for (int i = t; i < TK_COPIES * TK_STRIDE / 4; i += 256) hist4[i] = make_uint4(0u, 0u, 0u, 0u);
  // dword i of chunk c: elements 2i (low half) and 2i + 1 (high half)
  auto dw = [&](int c, int i) -> uint32_t { return i == 0 ? w[c].x : i == 1 ? w[c].y : i == 2 ? w[c].z : w[c].w; };

  float gamma;
  if (hint) {
    gamma = hint[row];
    if (search) __syncthreads();
  } else {
    tk_u16x2 pm = tk_pk(0u);                       // packed maxima of the 15-bit keys
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) pm = __builtin_elementwise_max(pm, tk_pk(dw(c, i) & 0x7FFF7FFFu));
    uint32_t mx = max((uint32_t)pm.x, (uint32_t)pm.y);   // padding chunks hold key 0
    mx = bl_wave_max_u(mx);
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    gamma = bl_u2f(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])) << 16);
  }
  const float s = 127.0f / (gamma + eps);

  uint32_t T = all ? 0u : 0x8000u;                 // 0x8000: above every key (keep == 0)
  int need = 0;
  if (search) {
    uint32_t* hc = hist + ((t & (TK_COPIES - 1)) >> 2) * TK_GROUP + (t & 3);   // bin b at hc[4 b]
    // total of bin b over the copies: one 16-byte read per group of four
    auto bin_total = [&](int b) -> int {
      int n = 0;
#pragma unroll
      for (int g = 0; g < TK_COPIES / 4; ++g) {
        const uint4 q = hist4[(g * TK_GROUP >> 2) + b];
        n += (int)(q.x + q.y + q.z + q.w);
      }
      return n;
    };
    // exponent bin of each key: bits 7..14 (low half) and 23..30 (high half) of a dword
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (t + 256 * c < nch) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          atomicAdd(&hc[4 * __builtin_amdgcn_ubfe(dw(c, i), 7, 8)], 1u);
          atomicAdd(&hc[4 * __builtin_amdgcn_ubfe(dw(c, i), 23, 8)], 1u);
        }
      }
    __syncthreads();
    // pass 1: thread t owns exponent bin 255 - t (descending keys)
    int cnt = bin_total(255 - t);
    int2 sc = tk_block_scan(cnt, wtot, t);
    if (sc.x - cnt < keep && keep <= sc.x) { sel[0] = 255 - t; sel[1] = sc.x - cnt; }
    // clear the mantissa bins (every thread has read its exponent bin above)
    for (int i = t; i < TK_COPIES * 128 / 4; i += 256) hist4[((i >> 7) * TK_GROUP >> 2) + (i & 127)] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const uint32_t e = (uint32_t)sel[0];
    const int above = sel[1];
    // mantissa bin of each key whose exponent is e; every other key adds to bin 128 + its mantissa
    // (bins 128..255 are not read in this pass), so no lane branches. Per 16-bit half: x = key ^
    // (e << 7) is the mantissa when the exponent matches and at least 128 + the mantissa otherwise.
    const uint32_t ee = (e << 7) | (e << 23);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (t + 256 * c < nch) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x = (dw(c, i) & 0x7FFF7FFFu) ^ ee;
          const uint32_t b = tk_unpk(__builtin_elementwise_min(tk_pk(x), tk_pk((x & 0x007F007Fu) | 0x00800080u)));
          atomicAdd(&hc[4 * (b & 0xFFFFu)], 1u);
          atomicAdd(&hc[4 * (b >> 16)], 1u);
        }
      }
    __syncthreads();
    // pass 2: thread t < 128 owns mantissa bin 127 - t
    cnt = t < 128 ? bin_total(127 - t) : 0;
    sc = tk_block_scan(cnt, wtot, t);
    const int ex = above + sc.x - cnt;
    if (t < 128 && ex < keep && keep <= above + sc.x) { sel[0] = 127 - t; sel[1] = ex; }
    __syncthreads();
    T = (e << 7) | (uint32_t)sel[0];
    need = keep - sel[1];                          // >= 1 ties at T survive, lowest index first
  }

  // per chunk: bit j of gt8 / eq8 says whether key j is above / equal to T (packed 16-bit
  // differences T - key: bit 15 of a half is set exactly when key > T, and bit 15 of the difference
  // minus one is set exactly when key >= T, since every key and T are below 2^15)
  uint32_t gt8[NCH], eq8[NCH];
  // tie ranks in index order: chunk c of all threads, then chunk c + 1
  int rank[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) rank[c] = 0;
  if (search) {
    const tk_u16x2 tp = tk_pk(T | (T << 16));
    int tc[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t g[4], q[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t d = tk_unpk(tp - tk_pk(dw(c, i) & 0x7FFF7FFFu));
        const uint32_t e = tk_unpk(tk_pk(d) - tk_pk(0x00010001u));
        g[i] = d & 0x80008000u;
        q[i] = e & ~d & 0x80008000u;
      }
      const bool ok = t + 256 * c < nch;           // padding chunks hold no keys
      gt8[c] = tk_fold(g[0], g[1], g[2], g[3]);
      eq8[c] = ok ? tk_fold(q[0], q[1], q[2], q[3]) : 0u;
      tc[c] = __popc(eq8[c]);
    }
    int incl[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      incl[c] = bl_wave_incl_scan(tc[c], lane);
      if (lane == 63) wtot_v[c][wave] = incl[c];
    }
    __syncthreads();
    int base = 0;                                  // ties of all earlier chunks
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      int off = 0, tot = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        off += q < wave ? wtot_v[c][q] : 0;
        tot += wtot_v[c][q];
      }
      rank[c] = base + off + incl[c] - tc[c];
      base += tot;
    }
  }

  uint32_t* mrow = mask ? mask + (long)row * (K >> 5) : nullptr;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int ch = t + 256 * c;
    if (ch >= nch) continue;                       // whole groups of 4 threads drop out together
    uint32_t kb = all ? 0xFFu : 0u;                // bit j: element j of the chunk survives
    if (search) {
      // the ties of this chunk with ranks below need, lowest index first (most chunks have none)
      uint32_t ke = eq8[c];
      const int room = need - rank[c];
      if (room <= 0) ke = 0u;
      while (__popc(ke) > room) ke &= ~(0x80000000u >> __clz(ke));
      kb = gt8[c] | ke;
    }
    // codes of all eight elements, then the dropped ones cleared byte by byte
    uint32_t rr[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t d = dw(c, i);
      rr[2 * i] = bl_f2u(bl_u2f(d << 16) * s + 12582912.0f);             // low byte = rint(x s)
      rr[2 * i + 1] = bl_f2u(bl_u2f(d & 0xFFFF0000u) * s + 12582912.0f);
    }
    uint32_t lo = __builtin_amdgcn_perm(rr[1], rr[0], 0x0C0C0400u) | __builtin_amdgcn_perm(rr[3], rr[2], 0x04000C0Cu);
    uint32_t hi = __builtin_amdgcn_perm(rr[5], rr[4], 0x0C0C0400u) | __builtin_amdgcn_perm(rr[7], rr[6], 0x04000C0Cu);
    lo &= tk_byte_mask(kb);
    hi &= tk_byte_mask(kb >> 4);
    reinterpret_cast<uint2*>(codes + (long)row * K)[ch] = make_uint2(lo, hi);
    if (mrow) {                                    // the four threads of a quad share one word
      uint32_t mw = kb << (8 * (t & 3));
      mw |= bl_dpp<0xB1>(mw);                      // quad_perm(1, 0, 3, 2)
      mw |= bl_dpp<0x4E>(mw);                      // quad_perm(2, 3, 0, 1)
      if ((t & 3) == 0) mrow[ch >> 2] = mw;
    }
  }
  if (t == 0) scale[row] = gamma / 127.0f;
}

// ============================================================================ block-per-row kernel
// Quantizers without a Top-K mask (INT4 nibbles or E3M2 tiles, FP4 both scale modes, INT8 of the
// whole row), one 256-thread block per row: thread t owns the 8-element chunks t, t + 256, ... of
// the row (16- or 32-byte loads), the row statistic (exact absmean sum or max) is reduced across
// the block, and every chunk's codes leave as one 4- or 8-byte store (E3M2: 12 bytes per thread
// pair). Many more waves are in flight than with one wave per row.
template <int IN_F32>
__device__ __forceinline__ void load8v(const void* __restrict__ x, long off, float (&o)[8]) {
  if (IN_F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    o[0] = bl_bf16lo(t.x); o[1] = bl_bf16hi(t.x); o[2] = bl_bf16lo(t.y); o[3] = bl_bf16hi(t.y);
    o[4] = bl_bf16lo(t.z); o[5] = bl_bf16hi(t.z); o[6] = bl_bf16lo(t.w); o[7] = bl_bf16hi(t.w);
  }
}

template <int FMT, int IN_F32, int NCH>
__global__ __launch_bounds__(256) void k_quant_blk(const void* __restrict__ x, int M, int K, long ldx, float eps,
                                                   const float* __restrict__ hint, uint8_t* __restrict__ codes,
                                                   float* __restrict__ scale) {
  constexpr bool SUM = (FMT == BL_ACT_INT4 || FMT == BL_ACT_INT4_E3M2);
  constexpr bool E3M2 = (FMT == BL_ACT_INT4_E3M2);
  __shared__ double wsum[4];
  __shared__ uint32_t wa[4], wb[4];
  __shared__ unsigned long long bins[SUM ? 256 : 1];
  // E3M2: the row's 6-bit codes (3K/4 bytes, K <= 256 NCH) gathered before the tiled stores
  __shared__ __attribute__((aligned(16))) uint8_t erow[E3M2 ? 256 * NCH * 6 : 16];
  __shared__ unsigned long long limbs[12];
  __shared__ double total;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row = blockIdx.x;
  const int nch = K >> 3;
  float v[NCH][8];
  uint4 raw[NCH];                                                // bf16 nibble rows: the loaded dwords
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if (t + 256 * c < nch) {
      if constexpr (IN_F32 || FMT != BL_ACT_INT4) {
        load8v<IN_F32>(x, (long)row * ldx + 8 * (t + 256 * c), v[c]);
      } else {
        const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (long)row * ldx + 8 * (t + 256 * c));
        raw[c] = q;
        v[c][0] = bl_bf16lo(q.x); v[c][1] = bl_bf16hi(q.x); v[c][2] = bl_bf16lo(q.y); v[c][3] = bl_bf16hi(q.y);
        v[c][4] = bl_bf16lo(q.z); v[c][5] = bl_bf16hi(q.z); v[c][6] = bl_bf16lo(q.w); v[c][7] = bl_bf16hi(q.w);
      }
    }

  // the row statistic: beta (SUM) or gamma
  float st_val;
  if (hint) {
    st_val = hint[row];
  } else if constexpr (SUM) {
    AbsSum acc;
    // bf16 rows of nibble codes track the exponent bounds on packed halves (one vector instruction
    // fewer per element: 12.4-12.8 against 13.9-14.1 us for 4096 x 4096 rows); the E3M2 kernel
    // measured no faster with it (its 2048-row FFN input 0.3 us slower) and keeps the plain form
    if constexpr (IN_F32 || FMT != BL_ACT_INT4) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (t + 256 * c < nch) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc.add(v[c][j]);
        }
    } else {
      uint32_t pmax = 0u, pmin1 = 0xFFFFFFFFu;
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (t + 256 * c < nch) {
          acc.add_bf16_pair(raw[c].x, v[c][0], v[c][1], pmax, pmin1);
          acc.add_bf16_pair(raw[c].y, v[c][2], v[c][3], pmax, pmin1);
          acc.add_bf16_pair(raw[c].z, v[c][4], v[c][5], pmax, pmin1);
          acc.add_bf16_pair(raw[c].w, v[c][6], v[c][7], pmax, pmin1);
        }
      acc.fold_bf16(pmax, pmin1);
    }
    const double ws = bl_wave_sum_d(acc.s);
    const uint32_t ex = wave_max_exps(acc.exps());
    const uint32_t emax = exps_emax(ex), emin = exps_emin(ex);
    if (lane == 0) { wsum[wave] = ws; wa[wave] = emax; wb[wave] = emin; }
    __syncthreads();
    double S = wsum[0] + wsum[1] + wsum[2] + wsum[3];           // exact when the check below holds
    uint32_t e1 = wa[0], e0 = wb[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) { e1 = wa[w] > e1 ? wa[w] : e1; e0 = wb[w] < e0 ? wb[w] : e0; }
    if (!sum_is_exact<IN_F32>(e1, e0, K)) {                      // block-uniform
      bins[t] = 0ull;
      __syncthreads();
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        if (t + 256 * c < nch) {
#pragma unroll
          for (int j = 0; j < 8; ++j) bins_add(bins, v[c][j]);
        }
      __syncthreads();
      S = bl_bins_to_double_block(bins, limbs, &total);
    }
    st_val = (float)(S / (double)K);
  } else {
    uint32_t mx = 0u;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (t + 256 * c < nch) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b = bl_f2u(v[c][j]) & 0x7FFFFFFFu;
          mx = b > mx ? b : mx;
        }
      }
    mx = bl_wave_max_u(mx);
    if (lane == 0) wa[wave] = mx;
    __syncthreads();
    uint32_t g = wa[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) g = wa[w] > g ? wa[w] : g;
    st_val = bl_u2f(g);
  }

  if constexpr (SUM) {
    const float beta = st_val;
    const float s = bl_u2f(BL_SQRT7_BITS) / (beta + eps);
    if constexpr (FMT == BL_ACT_INT4) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int ch = t + 256 * c;
        if (ch >= nch) continue;                                 // whole wave pairs drop out together
        reinterpret_cast<uint32_t*>(codes + (long)row * (K >> 1))[ch] = codes_int4_8(v[c], s);
      }
    } else if constexpr (NCH == 2) {
      // chunks 0 and 1 (8 codes x 6 bits = 6 bytes each, at byte 6 ch of the LDS row) share one
      // conversion (longer rows, whose extra operand registers would lower the occupancy, take the
      // arithmetic form below)
#pragma unroll
      for (int c = 0; c < NCH; c += 2) {
        const int ch = t + 256 * c;
        if (ch >= nch) continue;
        uint32_t w[3];
        codes_e3m2_16(v[c], v[c + 1], s, w);
        put_e3m2_48(erow, ch, w[0], w[1] & 0xFFFFu);
        if (ch + 256 < nch) put_e3m2_48(erow, ch + 256, (w[1] >> 16) | (w[2] << 16), w[2] >> 16);
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int ch = t + 256 * c;
        if (ch >= nch) continue;
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = code_e3m2(v[c][j], s);
        put_e3m2_48(erow, ch, e[0] | (e[1] << 6) | (e[2] << 12) | (e[3] << 18) | (e[4] << 24) | (e[5] << 30),
                    (e[5] >> 2) | (e[6] << 4) | (e[7] << 10));
      }
    }
    if constexpr (E3M2) {
      // 16-byte pieces of the row to the tiles: piece p holds bytes 16 p .. 16 p + 15 of the row, inside
      // the 96-byte row piece of K tile 16 p / 96 (16-row x 128-code tiles of 1536 bytes)
      __syncthreads();
      const int npc = (3 * K) >> 6;
      const long tile0 = (long)(row >> 4) * (K >> 7);
      for (int pc = t; pc < npc; pc += 256) {
        const int kt = pc / 6, off = 16 * (pc - 6 * kt);
        *reinterpret_cast<uint4*>(codes + (tile0 + kt) * 1536 + (row & 15) * 96 + off) =
            *reinterpret_cast<const uint4*>(erow + 16 * pc);
      }
    }
    if (t == 0) scale[row] = beta / bl_u2f(BL_SQRT7_BITS);
  } else if constexpr (FMT == BL_ACT_FP4_E2M1 || FMT == BL_ACT_FP4_E2M1_POW2) {
    float s, dscale;
    fp4_scales<FMT == BL_ACT_FP4_E2M1_POW2>(st_val, eps, &s, &dscale);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = t + 256 * c;
      if (ch >= nch) continue;
      const uint32_t w = codes_fp4_8(v[c], s);
      reinterpret_cast<uint32_t*>(codes + (long)row * (K >> 1))[ch] = w;
    }
    if (t == 0) scale[row] = dscale;
  } else {
    const float gamma = st_val;
    const float s = 127.0f / (gamma + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = t + 256 * c;
      if (ch >= nch) continue;
      uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0 |= code_int8(v[c][j], s) << (8 * j);
        w1 |= code_int8(v[c][j + 4], s) << (8 * j);
      }
      reinterpret_cast<uint2*>(codes + (long)row * K)[ch] = make_uint2(w0, w1);
    }
    if (t == 0) scale[row] = gamma / 127.0f;
  }
}

// ============================================================================ streaming kernels
template <int FMT, int IN_F32>
__global__ __launch_bounds__(256) void k_quant_stream(const void* __restrict__ x, int M, int K, long ldx,
                                                      int keep, float eps, const float* __restrict__ hint,
                                                      uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                      uint32_t* __restrict__ mask) {
  __shared__ unsigned long long bins[(FMT == BL_ACT_INT4 || FMT == BL_ACT_INT4_E3M2) ? 4 : 1][256];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= M) return;
  const int NG = (K + 255) >> 8;                  // the last group is half when K % 256 == 128
  const long base = (long)row * ldx + 4 * lane;
  // elements 256 g + 4 lane .. +3, or zeros for the lanes past the end of a half group
  auto load = [&](int g, float (&v)[4]) {
    if (256 * g + 4 * lane < K) load4<IN_F32>(x, base + 256 * g, v);
    else v[0] = v[1] = v[2] = v[3] = 0.0f;
  };

  if constexpr (FMT == BL_ACT_INT4 || FMT == BL_ACT_INT4_E3M2) {
    float beta;
    if (hint) {
      beta = hint[row];                           // a given beta (per-tensor variant)
    } else {
      AbsSum acc;
      for (int g = 0; g < NG; ++g) {
        float v[4];
        load(g, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc.add(v[j]);
      }
      double S = bl_wave_sum_d(acc.s);
      const uint32_t ex = wave_max_exps(acc.exps());
      const uint32_t emax = exps_emax(ex), emin = exps_emin(ex);
      if (!sum_is_exact<IN_F32>(emax, emin, K)) {
        unsigned long long* b = bins[wave];
        bins_clear(b, lane);
        for (int g = 0; g < NG; ++g) {
          float v[4];
          load(g, v);
#pragma unroll
          for (int j = 0; j < 4; ++j) bins_add(b, v[j]);
        }
        S = bins_finish(b, lane);
      }
      beta = (float)(S / (double)K);
    }
    const float s = bl_u2f(BL_SQRT7_BITS) / (beta + eps);
    for (int g = 0; g < NG; ++g) {
      float v[4];
      load(g, v);
      if constexpr (FMT == BL_ACT_INT4) {
        uint16_t* crow = reinterpret_cast<uint16_t*>(codes + (long)row * (K >> 1)) + lane;
        if (256 * g + 4 * lane < K)
          crow[64 * g] = (uint16_t)(code_int4(v[0], s) | (code_int4(v[1], s) << 4) |
                                     (code_int4(v[2], s) << 8) | (code_int4(v[3], s) << 12));
      } else {
        store_e3m2(codes, row, K, g, lane,
                   code_e3m2(v[0], s) | (code_e3m2(v[1], s) << 6) | (code_e3m2(v[2], s) << 12) |
                       (code_e3m2(v[3], s) << 18),
                   256 * g + 4 * lane < K);
      }
    }
    if (lane == 0) scale[row] = beta / bl_u2f(BL_SQRT7_BITS);
  } else {
    float gamma;
    if (hint) {
      gamma = hint[row];
    } else {
      uint32_t mx = 0u;
      for (int g = 0; g < NG; ++g) {
        float v[4];
        load(g, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t b = bl_f2u(v[j]) & 0x7FFFFFFFu;
          mx = b > mx ? b : mx;
        }
      }
      gamma = bl_u2f(bl_wave_max_u(mx));
    }
    if constexpr (FMT == BL_ACT_FP4_E2M1 || FMT == BL_ACT_FP4_E2M1_POW2) {
      float s, dscale;
      fp4_scales<FMT == BL_ACT_FP4_E2M1_POW2>(gamma, eps, &s, &dscale);
      uint16_t* crow = reinterpret_cast<uint16_t*>(codes + (long)row * (K >> 1)) + lane;   // 2 bytes per lane per group
      for (int g = 0; g < NG; ++g) {
        float v[4];
        load(g, v);
        const uint32_t c = codes_fp4_4(v[0], v[1], v[2], v[3], s);
        if (256 * g + 4 * lane < K) crow[64 * g] = (uint16_t)c;
      }
      if (lane == 0) scale[row] = dscale;
    } else {
      const float s = 127.0f / (gamma + eps);
      const bool all = keep < 0 || keep >= K;
      const bool none = keep == 0;
      float Tf = 0.0f;
      int need = 0;
      if (!all && !none) {
        auto count_cmp = [&](float c, bool strict) {
          int n = 0;
          for (int g = 0; g < NG; ++g) {
            float v[4];
            load(g, v);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float a = fabsf(v[j]);
              n += __popcll(__ballot(strict ? (a > c) : (a >= c)));
            }
          }
          return n;
        };
        Tf = bl_u2f(topk_threshold(keep, IN_F32 ? 0 : 16, [&](float c) { return count_cmp(c, false); }));
        need = keep - count_cmp(Tf, true);
      }
      uint32_t* crow = reinterpret_cast<uint32_t*>(codes + (long)row * K) + lane;
      uint32_t* mrow = mask ? mask + (long)row * (K >> 5) : nullptr;
      const unsigned long long lt = (1ull << lane) - 1ull;
      int tie_base = 0;
      for (int g = 0; g < NG; ++g) {
        float v[4];
        load(g, v);
        uint32_t keepbits;
        if (all) {
          keepbits = 0xFu;
        } else if (none) {
          keepbits = 0u;
        } else {
          uint32_t gt = 0u, eq = 0u;
          int before = 0, tot = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = fabsf(v[j]);
            gt |= (a > Tf ? 1u : 0u) << j;
            const bool t = 256 * g + 4 * lane < K && a == Tf;   // zeros past the end never tie
            eq |= (t ? 1u : 0u) << j;
            const unsigned long long bal = __ballot(t);
            before += __popcll(bal & lt);
            tot += __popcll(bal);
          }
          int rank = tie_base + before;
          uint32_t kb = gt;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if ((eq >> j) & 1u) { kb |= (rank < need ? 1u : 0u) << j; ++rank; }
          keepbits = kb;
          tie_base += tot;
        }
        uint32_t c = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if ((keepbits >> j) & 1u) c |= code_int8(v[j], s) << (8 * j);
        if (256 * g + 4 * lane < K) crow[64 * g] = c;
        if (mrow) store_mask_nibble(mrow, g, lane, keepbits, 256 * g + 4 * lane < K);
      }
      if (lane == 0) scale[row] = gamma / 127.0f;
    }
  }
}

// ============================================================================ per-tensor scale
// Variant of the activation quantizers with one scale for the whole [M, K] tensor (reading of the
// pages' "all entries in X"): beta = RN32(RN64(exact sum |x|) / (M K)) or gamma = max |x| over the
// tensor, then every row is quantized with it (passed to the row kernels as a per-row value).
// The exact sum: each thread adds its values in double, exact whenever the exponent span of its
// terms allows it (else its values go to the bins one by one); the thread's exact double is split
// into three non-negative floats (round down, remainder, remainder) that enter the per-exponent
// integer bins shared with the weight alpha.
__device__ __forceinline__ float round_down_f32(double d) {        // d >= 0, d < FLT_MAX
  float f = (float)d;
  if ((double)f > d) f = bl_u2f(bl_f2u(f) - 1u);
  return f;
}

constexpr int kTensorBlocks = 512;     // blocks of the tensor-wide reduction
constexpr int kTensorThreads = 1024;   // threads per block: two blocks fill a CU's 32 wave slots
constexpr int kTensorLimbs = 12;       // 64-bit limb sums per block slot

template <int IN_F32>
__device__ __forceinline__ void load8(const void* __restrict__ x, long off, float (&o)[8]) {
  if (IN_F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    o[0] = bl_bf16lo(t.x); o[1] = bl_bf16hi(t.x); o[2] = bl_bf16lo(t.y); o[3] = bl_bf16hi(t.y);
    o[4] = bl_bf16lo(t.z); o[5] = bl_bf16hi(t.z); o[6] = bl_bf16lo(t.w); o[7] = bl_bf16hi(t.w);
  }
}

// Adds one non-negative float per lane to the LDS bins: its significand to the bin of its exponent,
// one 64-bit LDS atomic per lane (integer sums, so their order does not matter). Lanes that share an
// exponent are serialized by the LDS, which costs far less than merging them first with shuffles.
__device__ __forceinline__ void lane_bins_add(unsigned long long* bins, float v) {
  uint32_t e, m;
  bl_bin_split(bl_f2u(v) & 0x7FFFFFFFu, &e, &m);
  if (m) atomicAdd(&bins[e], (unsigned long long)m);
}

// Each block writes its exact total as twelve limb sums to slot blockIdx (SUM), or its maximum;
// every slot is rewritten on every call, so the workspace needs no clearing.
// Threads walk 8-element chunks of the row-major tensor with a grid stride.
template <int IN_F32, bool SUM>
__global__ __launch_bounds__(kTensorThreads) void k_tensor_reduce(const void* __restrict__ x, int M, int K, long ldx,
                                                       unsigned long long* __restrict__ gslot,
                                                       uint32_t* __restrict__ gmax) {
  __shared__ unsigned long long bins[SUM ? 256 : 1];
  __shared__ unsigned long long limbs[SUM ? kTensorLimbs : 1];
  __shared__ uint32_t wmax[kTensorThreads / 64];
  const int t = threadIdx.x, lane = t & 63;
  if constexpr (SUM) {
    if (t < 256) bins[t] = 0ull;
    __syncthreads();
  }
  uint32_t mx = 0u;
  AbsSum accs[4];                      // four independent sums shorten the chain of dependent adds
  int cnt = 0;
  const long KO = K >> 3, chunks = (long)M * KO;
  const long q0 = (long)blockIdx.x * blockDim.x + t, qs = (long)gridDim.x * blockDim.x;
  const long drow = qs / KO, dcol = qs % KO;
  {
    long row = q0 / KO, col = q0 % KO;
#pragma unroll 4
    for (long q = q0; q < chunks; q += qs) {
      float v[8];
      load8<IN_F32>(x, row * ldx + 8 * col, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (SUM) {
          accs[j & 3].add(v[j]);
        } else {
          const uint32_t b = bl_f2u(v[j]) & 0x7FFFFFFFu;
          mx = b > mx ? b : mx;
        }
      }
      cnt += 8;
      col += dcol;
      row += drow;
      if (col >= KO) { col -= KO; ++row; }
    }
  }
  if constexpr (SUM) {
    AbsSum acc = accs[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      acc.merge(accs[i]);
    }
    const uint32_t ex = acc.exps();
    const bool exact = sum_is_exact<IN_F32>(exps_emax(ex), exps_emin(ex), cnt) && acc.s < 1.0e38;
    float hi = 0.f, mid = 0.f, lo = 0.f;
    if (exact) {
      hi = round_down_f32(acc.s);
      const double r = acc.s - (double)hi;                          // exact, below ulp(hi)
      mid = round_down_f32(r);
      lo = (float)(r - (double)mid);                                 // exact: at most a few bits
    } else {
      long row = q0 / KO, col = q0 % KO;
      for (long q = q0; q < chunks; q += qs) {
        float v[8];
        load8<IN_F32>(x, row * ldx + 8 * col, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) bins_add(bins, v[j]);
        col += dcol;
        row += drow;
        if (col >= KO) { col -= KO; ++row; }
      }
    }
    lane_bins_add(bins, hi);
    lane_bins_add(bins, mid);
    lane_bins_add(bins, lo);
    __syncthreads();
    bl_bins_to_limb_sums_block(bins, limbs);
    if (t < kTensorLimbs) gslot[blockIdx.x * kTensorLimbs + t] = limbs[t];
  } else {
    mx = bl_wave_max_u(mx);
    if (lane == 0) wmax[t >> 6] = mx;
    __syncthreads();
    if (t == 0) {
      uint32_t m = wmax[0];
      for (int w = 1; w < kTensorThreads / 64; ++w) m = wmax[w] > m ? wmax[w] : m;
      gmax[blockIdx.x] = m;
    }
  }
}

// one value for every row: beta (SUM, from the blocks' limb sums) or gamma (the maximum); 1024 threads
template <bool SUM>
__global__ __launch_bounds__(1024) void k_tensor_scale(const unsigned long long* __restrict__ gslot,
                                                       const uint32_t* __restrict__ gmax, int M, double count,
                                                       float* __restrict__ rowval) {
  __shared__ unsigned long long limbs[kTensorLimbs];
  __shared__ uint32_t wmax[16];
  __shared__ float val;
  const int t = threadIdx.x;
  if constexpr (SUM) {
    // thread (g, i) adds limb i of slots g, g + 64, ...; every sum stays below 2^49 + 2^40
    if (t < kTensorLimbs) limbs[t] = 0ull;
    __syncthreads();
    if (t < kTensorLimbs * 64) {
      const int i = t % kTensorLimbs, g = t / kTensorLimbs;
      unsigned long long b = 0ull;
      for (int k = g; k < kTensorBlocks; k += 64) b += gslot[k * kTensorLimbs + i];
      atomicAdd(&limbs[i], b);
    }
    __syncthreads();
    if (t == 0) val = (float)(bl_limb_sums_to_double(limbs) / count);
  } else {
    uint32_t m = 0u;
    for (int k = t; k < kTensorBlocks; k += 1024) m = gmax[k] > m ? gmax[k] : m;
    m = bl_wave_max_u(m);
    if ((t & 63) == 0) wmax[t >> 6] = m;
    __syncthreads();
    if (t == 0) {
      uint32_t g = wmax[0];
      for (int w = 1; w < 16; ++w) g = wmax[w] > g ? wmax[w] : g;
      val = bl_u2f(g);
    }
  }
  __syncthreads();
  for (int m = t; m < M; m += 1024) rowval[m] = val;
}

template <int FMT, int IN_F32>
hipError_t launch_fmt(const void* x, int M, int K, long ldx, int keep, float eps, const float* hint,
                      uint8_t* codes, float* scale, uint32_t* mask, hipStream_t st) {
  const dim3 grid((M + 3) / 4), block(256);
  // no Top-K mask: one block per row
  const bool plain = FMT != BL_ACT_INT8 || (mask == nullptr && (keep < 0 || keep >= K));
  if (plain && K <= 16384) {
    const int per = (K / 8 + 255) / 256;                 // 8-element chunks per thread
    if (per <= 2)
      hipLaunchKernelGGL((k_quant_blk<FMT, IN_F32, 2>), dim3(M), block, 0, st, x, M, K, ldx, eps, hint, codes, scale);
    else if (per <= 4)
      hipLaunchKernelGGL((k_quant_blk<FMT, IN_F32, 4>), dim3(M), block, 0, st, x, M, K, ldx, eps, hint, codes, scale);
    else
      hipLaunchKernelGGL((k_quant_blk<FMT, IN_F32, 8>), dim3(M), block, 0, st, x, M, K, ldx, eps, hint, codes, scale);
    return hipGetLastError();
  }
  if constexpr (FMT == BL_ACT_INT8) {
    if (!IN_F32 && K <= 8192) {
      // Top-K of bf16 rows: one block per row
      const uint16_t* xb = static_cast<const uint16_t*>(x);
      const int per = (K / 8 + 255) / 256;
      if (per <= 1)
        hipLaunchKernelGGL((k_topk_blk<1>), dim3(M), block, 0, st, xb, M, K, ldx, keep, eps, hint, codes, scale, mask);
      else if (per <= 2)
        hipLaunchKernelGGL((k_topk_blk<2>), dim3(M), block, 0, st, xb, M, K, ldx, keep, eps, hint, codes, scale, mask);
      else
        hipLaunchKernelGGL((k_topk_blk<4>), dim3(M), block, 0, st, xb, M, K, ldx, keep, eps, hint, codes, scale, mask);
      return hipGetLastError();
    }
    if (IN_F32 && K <= 4096) {
      // Top-K of float32 rows: one wave per row, the row in registers
      const int NG = (K + 255) >> 8;
      if (NG <= 4)
        hipLaunchKernelGGL((k_quant_res<IN_F32, 4>), grid, block, 0, st, x, M, K, ldx, keep, eps, hint, codes, scale,
                           mask);
      else if (NG <= 8)
        hipLaunchKernelGGL((k_quant_res<IN_F32, 8>), grid, block, 0, st, x, M, K, ldx, keep, eps, hint, codes, scale,
                           mask);
      else
        hipLaunchKernelGGL((k_quant_res<IN_F32, 16>), grid, block, 0, st, x, M, K, ldx, keep, eps, hint, codes, scale,
                           mask);
      return hipGetLastError();
    }
  }
  // every other case (rows longer than the block kernels take): one wave per row, streaming
  hipLaunchKernelGGL((k_quant_stream<FMT, IN_F32>), grid, block, 0, st, x, M, K, ldx, keep, eps, hint, codes, scale,
                     mask);
  return hipGetLastError();
}

}  // namespace

hipError_t bl_launch_quantize(const void* x, int in_f32, int M, int K, long ldx, int fmt, int keep, float eps,
                              const float* hint, void* codes, float* scale, uint32_t* mask, hipStream_t st) {
  uint8_t* c = static_cast<uint8_t*>(codes);
  if (fmt == BL_ACT_INT4)
    return in_f32 ? launch_fmt<BL_ACT_INT4, 1>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st)
                  : launch_fmt<BL_ACT_INT4, 0>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st);
  if (fmt == BL_ACT_INT4_E3M2)
    return in_f32 ? launch_fmt<BL_ACT_INT4_E3M2, 1>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st)
                  : launch_fmt<BL_ACT_INT4_E3M2, 0>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st);
  if (fmt == BL_ACT_FP4_E2M1)
    return in_f32 ? launch_fmt<BL_ACT_FP4_E2M1, 1>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st)
                  : launch_fmt<BL_ACT_FP4_E2M1, 0>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st);
  if (fmt == BL_ACT_FP4_E2M1_POW2)
    return in_f32 ? launch_fmt<BL_ACT_FP4_E2M1_POW2, 1>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st)
                  : launch_fmt<BL_ACT_FP4_E2M1_POW2, 0>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st);
  return in_f32 ? launch_fmt<BL_ACT_INT8, 1>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st)
                : launch_fmt<BL_ACT_INT8, 0>(x, M, K, ldx, keep, eps, hint, c, scale, mask, st);
}

hipError_t bl_launch_quantize_per_tensor(const void* x, int in_f32, int M, int K, long ldx, int fmt, float eps,
                                         void* ws, void* codes, float* scale, hipStream_t st) {
  // workspace: 512 block slots of 12 limb sums (uint64), 512 block maxima (uint32), then the M row values
  uint8_t* w = static_cast<uint8_t*>(ws);
  unsigned long long* gslot = reinterpret_cast<unsigned long long*>(w);
  uint32_t* gmax = reinterpret_cast<uint32_t*>(w + (size_t)kTensorBlocks * kTensorLimbs * 8);
  float* rowval = reinterpret_cast<float*>(w + (size_t)kTensorBlocks * kTensorLimbs * 8 + (size_t)kTensorBlocks * 4);
  const bool sum = (fmt == BL_ACT_INT4 || fmt == BL_ACT_INT4_E3M2);
  const dim3 grid(kTensorBlocks), block(kTensorThreads);
  if (sum) {
    if (in_f32) hipLaunchKernelGGL((k_tensor_reduce<1, true>), grid, block, 0, st, x, M, K, ldx, gslot, gmax);
    else hipLaunchKernelGGL((k_tensor_reduce<0, true>), grid, block, 0, st, x, M, K, ldx, gslot, gmax);
    hipLaunchKernelGGL((k_tensor_scale<true>), dim3(1), dim3(1024), 0, st, gslot, gmax, M, (double)M * K, rowval);
  } else {
    if (in_f32) hipLaunchKernelGGL((k_tensor_reduce<1, false>), grid, block, 0, st, x, M, K, ldx, gslot, gmax);
    else hipLaunchKernelGGL((k_tensor_reduce<0, false>), grid, block, 0, st, x, M, K, ldx, gslot, gmax);
    hipLaunchKernelGGL((k_tensor_scale<false>), dim3(1), dim3(1024), 0, st, gslot, gmax, M, (double)M * K, rowval);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return bl_launch_quantize(x, in_f32, M, K, ldx, fmt, -1, eps, rowval, codes, scale, nullptr, st);
}
