// Shared device helpers of the BitLinear kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define BL_WAVE 64

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// RN32(sqrt(7)) = 2.6457512f, bit pattern 0x402953FD.
#define BL_SQRT7_BITS 0x402953FDu

__device__ __forceinline__ float bl_u2f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t bl_f2u(float f) { return __float_as_uint(f); }

// bf16 bit pattern (low or high half of a dword) -> exactly equal float32.
__device__ __forceinline__ float bl_bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bl_bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------------ wave reductions (wave64)
// DPP exchanges inside each row of 16 lanes (xor 1, xor 2, the half-row mirror
// i <-> 7 - i of each 8 lanes, the row mirror i <-> 15 - i) leave every lane of a row holding the
// row's result after four steps; readlane of lanes 0, 16, 32 and 48 then combines the four rows, so
// the result is wave-uniform. Callers run with every lane of the wave active.
template <int CTRL>
__device__ __forceinline__ uint32_t bl_dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <typename Op>
__device__ __forceinline__ uint32_t bl_wave_reduce_u(uint32_t v, Op op) {
  v = op(v, bl_dpp<0xB1>(v));      // quad_perm(1, 0, 3, 2)
  v = op(v, bl_dpp<0x4E>(v));      // quad_perm(2, 3, 0, 1)
  v = op(v, bl_dpp<0x141>(v));     // row_half_mirror
  v = op(v, bl_dpp<0x140>(v));     // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float bl_wave_max_f(float v) {
  return bl_u2f(bl_wave_reduce_u(bl_f2u(v), [](uint32_t a, uint32_t b) { return bl_f2u(fmaxf(bl_u2f(a), bl_u2f(b))); }));
}
__device__ __forceinline__ uint32_t bl_wave_max_u(uint32_t v) {
  return bl_wave_reduce_u(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t bl_wave_min_u(uint32_t v) {
  return bl_wave_reduce_u(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
// Inclusive prefix sum of an int over the 64 lanes of a wave: shifts right by 1, 2, 4 and 8 lanes
// inside each row of 16 (a lane with no source adds 0), then the totals of the earlier rows (lanes
// 15, 31, 47) read through readlane. Every lane of the wave must be active.
__device__ __forceinline__ int bl_wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}
// Maximum over the lanes l, l ^ 16, l ^ 32 and l ^ 48 of a wave (the four 16-lane rows at one
// position). v_permlane16_swap with both operands v returns, in its two results, the values of the
// lanes l and l ^ 16; v_permlane32_swap those of l and l ^ 32. Every lane must be active.
__device__ __forceinline__ uint32_t bl_max_across_rows(uint32_t v) {
  const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = p16[0] > p16[1] ? p16[0] : p16[1];
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return p32[0] > p32[1] ? p32[0] : p32[1];
}
template <int CTRL>
__device__ __forceinline__ double bl_dpp_d(double v) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const uint32_t lo = bl_dpp<CTRL>((uint32_t)u), hi = bl_dpp<CTRL>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ double bl_readlane_d(double v, int l) {
  const unsigned long long u = __builtin_bit_cast(unsigned long long, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}
// Sum of doubles; exact whenever every partial sum is representable (the callers check this), so
// the order of the additions does not matter.
__device__ __forceinline__ double bl_wave_sum_d(double v) {
  v += bl_dpp_d<0xB1>(v);
  v += bl_dpp_d<0x4E>(v);
  v += bl_dpp_d<0x141>(v);
  v += bl_dpp_d<0x140>(v);
  return (bl_readlane_d(v, 0) + bl_readlane_d(v, 16)) + (bl_readlane_d(v, 32) + bl_readlane_d(v, 48));
}

// ------------------------------------------------------------------ exact sums of |binary32| values
// A non-negative binary32 value with biased exponent e and significand m (hidden bit included for
// e >= 1) equals m * 2^(max(e,1) - 150). Sums of significands per exponent ("bins") are exact in
// 64-bit integers; bl_bins_to_double turns the 256 bins into the correctly rounded double of the
// exact total with a 384-bit integer in units of 2^-149.
__host__ __device__ inline void bl_bin_split(uint32_t bits, uint32_t* e, uint32_t* m) {
  uint32_t ex = (bits >> 23) & 0xFFu;
  uint32_t mt = bits & 0x7FFFFFu;
  *e = ex;
  *m = ex ? (mt | 0x800000u) : mt;
}

__host__ __device__ inline double bl_bins_to_double(const unsigned long long* bins) {
  uint32_t limb[12];
  for (int i = 0; i < 12; ++i) limb[i] = 0u;
  for (int e = 0; e < 255; ++e) {
    unsigned long long b = bins[e];
    if (!b) continue;
    int sh = (e > 1 ? e : 1) - 1;                    // b * 2^sh in units of 2^-149
    int w = sh >> 5, bit = sh & 31;
    uint32_t p0 = (uint32_t)(b << bit);
    uint32_t p1 = (uint32_t)(bit ? (b >> (32 - bit)) : (b >> 32));
    uint32_t p2 = (uint32_t)(bit ? (b >> (64 - bit)) : 0ull);
    unsigned long long c = 0;
    uint32_t parts[3] = {p0, p1, p2};
    for (int i = 0; i < 12 - w; ++i) {
      unsigned long long add = (i < 3 ? parts[i] : 0u);
      if (i >= 3 && c == 0) break;
      unsigned long long t = (unsigned long long)limb[w + i] + add + c;
      limb[w + i] = (uint32_t)t;
      c = t >> 32;
    }
  }
  int top = -1;
  for (int i = 11; i >= 0; --i) {
    if (limb[i]) {
      int lz = 0;
      uint32_t v = limb[i];
      while (!(v & 0x80000000u)) { v <<= 1; ++lz; }
      top = 32 * i + 31 - lz;
      break;
    }
  }
  if (top < 0) return 0.0;
  // bit accessor
  auto bitat = [&](int p) -> uint32_t { return (p < 0) ? 0u : ((limb[p >> 5] >> (p & 31)) & 1u); };
  if (top <= 52) {
    unsigned long long v = 0;
    for (int p = top; p >= 0; --p) v = (v << 1) | bitat(p);
    return ldexp((double)v, -149);
  }
  unsigned long long mant = 0;
  for (int p = top; p >= top - 52; --p) mant = (mant << 1) | bitat(p);
  uint32_t rbit = bitat(top - 53);
  uint32_t sticky = 0;
  for (int p = top - 54; p >= 0 && !sticky; --p) sticky |= bitat(p);
  int ex = top;
  if (rbit && (sticky || (mant & 1ull))) {
    ++mant;
    if (mant == (1ull << 53)) { mant >>= 1; ++ex; }
  }
  return ldexp((double)mant, ex - 52 - 149);
}

// The same correctly rounded double for a whole block (blockDim.x threads, every thread calls it
// with the same arguments and gets the result): bins are scattered into 32-bit limb sums in LDS in
// parallel (each limb sum stays below 2^42), one thread propagates the carries and rounds.
// lds: 12 unsigned long long of shared memory; out: one shared double.
__device__ inline double bl_limbs_to_double(const uint32_t (&L)[12]) {
  // the three most significant nonzero limbs (a, b, c) and whether anything below them is nonzero
  uint32_t a = 0u, b = 0u, c = 0u;
  int ti = -1, k = 0;
  bool sticky = false;
#pragma unroll
  for (int i = 11; i >= 0; --i) {
    const uint32_t v = L[i];
    if (k == 0) {
      if (v) { a = v; ti = i; k = 1; }
    } else if (k == 1) {
      b = v; k = 2;
    } else if (k == 2) {
      c = v; k = 3;
    } else {
      sticky |= v != 0u;
    }
  }
  if (ti < 0) return 0.0;
  const int lz = __clz(a);
  unsigned long long u = ((unsigned long long)a << 32) | b;
  u = lz ? ((u << lz) | (c >> (32 - lz))) : u;
  const uint32_t c_rest = lz ? (c << lz) : c;                   // bits of c below the window
  int P = 32 * ti + 31 - lz;                                    // position of the leading bit
  unsigned long long mant = u >> 11;                            // 53 bits
  const uint32_t rbit = (uint32_t)(u >> 10) & 1u;
  sticky |= (u & 0x3FFull) != 0ull || c_rest != 0u;
  if (rbit && (sticky || (mant & 1ull))) {
    ++mant;
    if (mant == (1ull << 53)) { mant >>= 1; ++P; }
  }
  return ldexp((double)mant, P - 52 - 149);
}

// Block-parallel first half of the conversion: the bins (256 exponents) added into twelve 64-bit
// sums of 32-bit limb pieces (units of 2^-149, not yet carried) in lds[0..11]. Every thread of the
// block calls it; lds holds the sums when it returns.
__device__ inline void bl_bins_to_limb_sums_block(const unsigned long long* bins, unsigned long long* lds) {
  const int t = threadIdx.x;
  if (t < 12) lds[t] = 0ull;
  __syncthreads();
  for (int e = t; e < 255; e += blockDim.x) {
    const unsigned long long b = bins[e];
    if (!b) continue;
    const int sh = (e > 1 ? e : 1) - 1;                         // b * 2^sh in units of 2^-149
    const int w = sh >> 5, bit = sh & 31;
    atomicAdd(&lds[w], (unsigned long long)(uint32_t)(b << bit));
    atomicAdd(&lds[w + 1], (unsigned long long)(uint32_t)(bit ? (b >> (32 - bit)) : (b >> 32)));
    atomicAdd(&lds[w + 2], (unsigned long long)(uint32_t)(bit ? (b >> (64 - bit)) : 0ull));
  }
  __syncthreads();
}

// Second half: carries through the limb sums (each below 2^63 minus the incoming carry), then the
// correctly rounded double of the 384-bit integer.
__device__ inline double bl_limb_sums_to_double(const unsigned long long* sums) {
  uint32_t L[12];
  unsigned long long carry = 0ull;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const unsigned long long v = sums[i] + carry;
    L[i] = (uint32_t)v;
    carry = v >> 32;
  }
  return bl_limbs_to_double(L);
}

__device__ inline double bl_bins_to_double_block(const unsigned long long* bins, unsigned long long* lds,
                                                 double* out) {
  bl_bins_to_limb_sums_block(bins, lds);
  if (threadIdx.x == 0) *out = bl_limb_sums_to_double(lds);
  __syncthreads();
  return *out;
}

// ------------------------------------------------------------------ quantizer arithmetic
// round-half-even then clamp, as an int
__device__ __forceinline__ int bl_roundclip(float v, float lo, float hi) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, lo), hi);
  return (int)r;
}

