// BitLinear GEMMs on CDNA4 matrix cores: W1.58A4 (INT4 on int8 or FP6 cores, FP4 E2M1) and
// W1.58A8 (sparse INT8).
//
// "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up), section 3.4:
//   Y = Q_INT4(X) Q_w(W)^T ("4-Bit Activation Quantization for Gaussian-Like Inputs"),
//   Y = (Q_INT8(X) . M) Q_w(W)^T ("Sparsification Pipeline ...", paper Eq. 1),
//   ReLU^2 GLU epilogue ("Squared ReLU Gating ...", paper Eq. 5), residual add (section 3.2).
//
// Two kernels share the staging scheme: for every K step of 128 (one packed weight tile) the block
// copies its A rows and B tiles to LDS with 128-bit direct-to-LDS loads (no registers). Four stage
// buffers keep three steps in flight ahead of the matrix cores, which hides the L2/MALL latency
// that one buffered step cannot; A rows are stored with a per-row chunk rotation that makes the
// fragment reads free of bank conflicts. Each wave reads its fragments from LDS and feeds the
// matrix cores; one barrier per step both publishes a step and frees the buffer refilled next.
//
//  k_gemm_mx  FP6 x FP4 / FP4 x FP4 (v_mfma_scale_f32_16x16x128_f8f6f4, unit block scales).
//             4 waves, 128 x 256 block (128 x 128 per matrix for the GLU), 64 x 128 per wave, two
//             blocks per CU. A is used as stored (E3M2 or E2M1);
//             a ternary code placed in bits 2..3 of a nibble reads as E2M1 +-2.0, so the fp32 sum
//             is 2*sum(c t) for E3M2 codes and sum(2e t) for E2M1 codes: integers below 2^24, exact.
//  k_gemm_i8  int8 cores (v_mfma_i32_16x16x64_i8) for INT4 nibbles and INT8 codes. 4 waves, 128 x 256
//             or 128 x 128 block, two blocks per CU. The weight fragment is the first
//             MFMA operand, so a lane ends with four consecutive output columns of one token row and
//             the epilogue moves 16-byte vectors.
//             Fragments are expanded in registers: ternary -> 64*t via (w << s) & 0xC0C0C0C0,
//             INT4 nibble -> 16*c by moving it to the top of a byte, INT8 bytes permuted; the int32
//             accumulator holds 1024*sum(c t) (INT4) or 64*sum(c t) (INT8), exact after a shift.
//
// The K order inside each 16- or 32-wide MFMA slice follows the packed weight word (public header);
// activations enter the MFMAs in the same order, which leaves every dot product unchanged.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Workgroup barrier without a memory fence. A __syncthreads() fence would wait for every
// outstanding global load, including the next stage's prefetch, and so serialize load and compute.
// The only LDS writes here are direct-to-LDS loads, made complete by an explicit vmcnt wait before
// the barrier; LDS reads have returned (their data is consumed) before a wave reaches a barrier.
// The "memory" clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// ----------------------------------------------------------------------------- A storage per format
constexpr int NST = 4;   // stage buffers (three steps in flight)

template <int FMT>
struct AFmt {
  static constexpr int ROW = FMT == BL_ACT_INT8 ? 128 : FMT == BL_ACT_INT4_E3M2 ? 96 : 64;   // bytes per K step
  static constexpr int NCH = ROW / 16;                                                      // 16 B chunks
  // chunk rotation of LDS row r (depends on r % 16 only); chosen so that the 16 lanes of each
  // fragment read (rows r16 = 0..15) hit 16 disjoint bank groups
  __device__ static __forceinline__ int rot(int r) {
    const int r16 = r & 15;
    return FMT == BL_ACT_INT8 ? (r16 >> 1) : FMT == BL_ACT_INT4_E3M2 ? (r16 >> 3) : (r16 >> 2);
  }
  __device__ static __forceinline__ long row_bytes(int K) {
    return FMT == BL_ACT_INT8 ? K : FMT == BL_ACT_INT4_E3M2 ? (3L * K / 4) : (K / 2);
  }
};

// One 16-byte-per-lane direct-to-LDS load: lane i's 16 bytes from gptr land at LDS byte address
// lds_addr + 16 i (lds_addr is wave-uniform, passed in M0). Written as inline assembly so that the
// compiler does not treat later LDS reads of the other stage buffer as dependent on it (it would
// wait for every outstanding load); the kernels order these loads with explicit vmcnt waits and a
// final vmcnt(0) before the waves end.
__device__ __forceinline__ void dma16(const uint8_t* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Per-lane source offsets of this wave's share of the direct-to-LDS copies of one K step: A rows
// [m0, m0+BM) (stored with the chunk rotation) and the 512-byte B tiles of NB matrices x BN/16 tile
// rows (two tiles per 1 KB load). Rows beyond M and tile rows beyond N are clamped to valid memory:
// they load real but unused data (their outputs are never stored). The offsets are fixed for the
// whole K loop; step ks adds ks * ASTEP to A and ks * (N/16) * 512 to B (K-tile-major weights).
// E3M2 activations come in 16-row x 128-code tiles, so a stage of them is 16 contiguous 1536-byte
// runs; the other formats are row-major.
template <int FMT, int BM, int BN, int NB, int NW>
struct StagePlan {
  using F = AFmt<FMT>;
  static constexpr bool TILED = (FMT == BL_ACT_INT4_E3M2);
  static constexpr int ASEG = BM * F::NCH / 64;           // 1 KB LDS segments of A
  static constexpr int BT = NB * (BN / 16);               // 512-byte B tiles
  static constexpr int BSEG = BT / 2;                     // 1 KB LDS segments of B
  static constexpr int BYTES = BM * F::ROW + BT * 512;    // one stage
  static_assert(ASEG % NW == 0 && BSEG % NW == 0, "every wave issues the same number of loads");
  static constexpr int NA = ASEG / NW, NBL = BSEG / NW;
  static constexpr int LOADS = NA + NBL;                  // loads per wave and stage
  uint32_t aoff[NA];                                      // byte offset from A
  uint32_t boff[NBL];                                     // byte offset from its matrix
  uint32_t astep, bstep;                                  // bytes per K step
  __device__ __forceinline__ void init(long arow, int m0, int M, int n0, int NG, int KS, int wave, int lane) {
    const int mlast = TILED ? ((M + 15) & ~15) - 1 : M - 1;   // last row present in the buffer
#pragma unroll
    for (int qi = 0; qi < NA; ++qi) {
      const int q = wave + NW * qi;
      const int p = 64 * q + lane;                         // chunk position in the LDS tile
      const int r = p / F::NCH, slot = p % F::NCH;
      int c = slot - F::rot(r);
      c += c < 0 ? F::NCH : 0;
      const int m = min(m0 + r, mlast);
      aoff[qi] = TILED ? (uint32_t)((m >> 4) * KS * 1536 + (m & 15) * F::ROW + 16 * c)
                       : (uint32_t)(m * arow + 16 * c);
    }
#pragma unroll
    for (int qi = 0; qi < NBL; ++qi) {
      const int T = 2 * (wave + NW * qi) + (lane >> 5);   // B tile of this lane's 16 bytes
      const int t = T % (BN / 16);
      const int G = min((n0 >> 4) + t, NG - 1);
      boff[qi] = (uint32_t)(G * 512 + 16 * (lane & 31));
    }
    astep = TILED ? 1536u : (uint32_t)F::ROW;
    bstep = (uint32_t)NG * 512u;
  }
  // issue the loads of K step ks into the stage buffer at LDS address lds
  __device__ __forceinline__ void issue(uint32_t lds, const uint8_t* __restrict__ A, const uint8_t* const* Wm,
                                        int ks, int wave, int lane) const {
    const uint8_t* abase = A + (long)ks * astep;
#pragma unroll
    for (int qi = 0; qi < NA; ++qi) dma16(abase + aoff[qi], lds + 1024u * (wave + NW * qi));
#pragma unroll
    for (int qi = 0; qi < NBL; ++qi) {
      const int q = wave + NW * qi;
      const int mtx = (2 * q + (lane >> 5)) / (BN / 16);
      dma16(Wm[mtx] + (long)ks * bstep + boff[qi], lds + BM * F::ROW + 1024u * q);
    }
  }
};

// Byte offset, inside an LDS A tile, of byte b (8-byte aligned, within one 16 B chunk) of row r.
template <int FMT>
__device__ __forceinline__ int a_off(int r, int b) {
  using F = AFmt<FMT>;
  int slot = (b >> 4) + F::rot(r);
  slot -= slot >= F::NCH ? F::NCH : 0;
  return r * F::ROW + 16 * slot + (b & 15);
}

// one packed word (16 weights) -> four dwords of int8 values 64 t: a standard word gives k 0 2 4 6,
// 8 10 12 14, 1 3 5 7, 9 11 13 15 (the order of expand_a_int4), an A8 word k 0..3, 4..7, 8..11,
// 12..15 (the order of the INT8 codes in memory)
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
  r[0] = (int)((p0 << 4) & 0xF0F0F0F0u);  // k 0 2 4 6      (x16)
  r[1] = (int)((p1 << 4) & 0xF0F0F0F0u);  // k 8 10 12 14
  r[2] = (int)(p0 & 0xF0F0F0F0u);         // k 1 3 5 7
  r[3] = (int)(p1 & 0xF0F0F0F0u);         // k 9 11 13 15
  return r;
}
// 16 INT8 codes in memory order feed the MFMA as they are: the weights of these matmuls come in the
// A8 word layout, whose expansion is in the same k order
__device__ __forceinline__ v4i expand_a_int8(uint4 q) { return v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w}; }
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

// Block -> tile mapping. Consecutive block ids go to the eight XCDs in turn, so ids are first
// regrouped per XCD; inside an XCD the tiles are visited in groups of GROUP_M tile rows, so that
// the blocks one XCD runs at the same time share A rows and B columns in its L2.
__device__ __forceinline__ void tile_of(int b, int ntm, int ntn, int* tm, int* tn) {
  const int nblocks = ntm * ntn;
  if ((nblocks & 7) == 0) b = (b & 7) * (nblocks >> 3) + (b >> 3);
  constexpr int GROUP_M = 4;
  const int in_group = GROUP_M * ntn;
  const int first_m = (b / in_group) * GROUP_M;
  const int gm = min(ntm - first_m, GROUP_M);
  const int r = b % in_group;
  *tm = first_m + r % gm;
  *tn = r / gm;
}

// Epilogue for accumulators of transposed 16x16 products (weights as the first MFMA operand): the
// lane holds, for token row m, the four consecutive columns n .. n+3 (n % 4 == 0), so every output
// and residual access is one 16-byte vector. Columns come in whole groups of 16 (N % 16 == 0), so
// a lane's four columns are all in range or all out of range. val(mtx, v) is the exact sum of code
// products of matrix mtx for column n + v.
template <int EPI, typename ValFn>
__device__ __forceinline__ void epilogue_vals(bool ok, float sc, float sc2, const float4& res, float& rmax, ValFn val,
                                              float (&o)[4]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float y0 = val(0, v) * sc;
    if constexpr (EPI == BL_EPI_RESIDUAL) {
      o[v] = y0 + (v == 0 ? res.x : v == 1 ? res.y : v == 2 ? res.z : res.w);
    } else if constexpr (EPI == BL_EPI_RELU2_GLU) {
      const float u0 = val(1, v) * sc2;
      const float gp = y0 > 0.f ? y0 : 0.f;
      o[v] = (gp * gp) * u0;
      const float a = fabsf(o[v]);
      rmax = (ok && a > rmax) ? a : rmax;
    } else {
      o[v] = y0;
    }
  }
}

template <int EPI, typename ValFn>
__device__ __forceinline__ void epilogue_cols(int m, int n, bool ok, float sc, float sc2, float* __restrict__ Y,
                                              long ldy, const float4& res, float& rmax, ValFn val) {
  float o[4];
  epilogue_vals<EPI>(ok, sc, sc2, res, rmax, val, o);
  if (ok) *reinterpret_cast<float4*>(Y + (long)m * ldy + n) = make_float4(o[0], o[1], o[2], o[3]);
}

// Stores one 16-row subtile of a wave's outputs (SN tiles of 16 columns) through LDS so that every
// store instruction writes whole rows: lane (r, g) holds row r, columns 4g .. 4g + 3 of each tile;
// the subtile goes to the wave's LDS region in that layout and comes back as two rows of 16 SN
// contiguous floats per instruction (16-byte pieces, lanes 0..31 row 2i, lanes 32..63 row 2i + 1).
template <int SN>
__device__ __forceinline__ void store_subtile_rows(float* __restrict__ Y, long ldy, int M, int N, int m0, int n0,
                                                   const float (&o)[SN][4], float* __restrict__ region, int lane) {
  constexpr int RS = 16 * SN + 4;                  // row stride in floats (4 pad floats)
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < SN; ++t)
    *reinterpret_cast<float4*>(region + r * RS + 16 * t + 4 * g) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  constexpr int LPR = 4 * SN;                      // lanes per row (16 bytes each)
  constexpr int RPI = 64 / LPR;                    // rows per instruction
  const int rr = lane / LPR, cc = lane % LPR;
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int row = RPI * i + rr;
    const float4 q = *reinterpret_cast<const float4*>(region + row * RS + 4 * cc);
    const int m = m0 + row, n = n0 + 4 * cc;
    if (m < M && n < N) *reinterpret_cast<float4*>(Y + (long)m * ldy + n) = q;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();                 // the region is rewritten by the next subtile
}

template <int FMT, int EPI>
struct CfgMx {
  static constexpr bool GLU = (EPI == BL_EPI_RELU2_GLU);
  static constexpr int NB = GLU ? 2 : 1;
  // 4 waves (2 x 2), 128 x 256 block, two blocks per CU (at most 80 KB of LDS and 256 registers
  // per lane each), so one block's loads, LDS reads and epilogue overlap the other's MFMAs.
  static constexpr int NW = 4, WGM = 2, WGN = 2;
  static constexpr int BM = 128, BN = GLU ? 128 : 256;
  static constexpr int SM = BM / WGM / 16, SN = BN / WGN / 16;
  using Plan = StagePlan<FMT, BM, BN, NB, NW>;
};

// ---------------------------------------------------------------------------- fused KV-cache epilogue
// One wave's 128-column strip of a 128 x 256 tile is exactly one head of 128 (strips start at
// multiples of 128), and lane (r, g) holds columns 16 t + 4 g + v (t < 8, v < 4) of row r: the
// rotate-half partner i + 64 of column i = 16 t + 4 g + v (t < 4) is column 16 (t + 4) + 4 g + v of
// the same lane, and the head's absmax is a maximum over the four lanes r, r + 16, r + 32, r + 48.
// Codes, scales and BOS records are written exactly as the stand-alone KV quantizer writes them.
// u = RoundClip(RN32(x s), -Qp-1, Qp) + 2^(b-1) of four values, b bits apart. |x| <= gamma gives
// |RN32(x s)| < Qp + 1/2, so the clip never acts; adding C = 1.5 2^23 + 2^(b-1) rounds to an integer
// (ties to even, like rint: C is even) and leaves rint(x s) + 2^(b-1) in the low mantissa bits.
template <int BITS>
__device__ __forceinline__ uint32_t kv_code4(const float (&x)[4], float s) {
  constexpr float C = 12582912.0f + (float)(1 << (BITS - 1));
  constexpr uint32_t MASK = (1u << BITS) - 1u;
  uint32_t r = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) r |= (bl_f2u(x[j] * s + C) & MASK) << (BITS * j);
  return r;
}

// The head records of one 16-row subtile, assembled in the wave's LDS region and written as 16-byte
// pieces (whole records, one store instruction per subtile). A record holds 128 codes, code k at
// bits BITS k: 64 bytes for 4 bits, 48 for 3. Lane (r, g) holds codes 16 t + 4 g .. + 3 of row r
// for each tile t: 4 bits make the 16-bit group at byte 8 t + 2 g of the record; 3 bits make the
// 12-bit group at bit 48 t + 12 g, which is ORed into zeroed words (it may straddle two).
template <int BITS>
__device__ __forceinline__ void kv_stage_records(uint8_t* __restrict__ region, const float (&x)[8][4], float s, int r,
                                                 int g, int lane) {
  constexpr int RB = BITS * 16;                  // bytes per record
  if constexpr (BITS == 3) {
    if (lane < RB) reinterpret_cast<uint4*>(region)[lane] = make_uint4(0u, 0u, 0u, 0u);   // 16 records
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t c = kv_code4<BITS>(x[t], s);
    if constexpr (BITS == 4) {
      *reinterpret_cast<uint16_t*>(region + r * RB + 8 * t + 2 * g) = (uint16_t)c;
    } else {
      const int o = 48 * t + 12 * g, sh = o & 31;
      uint32_t* w = reinterpret_cast<uint32_t*>(region + r * RB) + (o >> 5);
      atomicOr(w, c << sh);
      if (sh > 20) atomicOr(w + 1, c >> (32 - sh));
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
// lane l < 16 RB / 16 writes piece l % (RB / 16) of record l / (RB / 16), the record of subtile row
// l / (RB / 16), to dst(that row) when the row is stored (keep)
template <int BITS, typename Dst, typename Keep>
__device__ __forceinline__ void kv_write_records(const uint8_t* __restrict__ region, int lane, Dst dst, Keep keep) {
  constexpr int RB = BITS * 16, PPR = RB / 16;
  if (lane < 16 * PPR) {
    const int rr = lane / PPR, pc = lane - PPR * (lane / PPR);
    const uint4 q = *reinterpret_cast<const uint4*>(region + rr * RB + 16 * pc);
    if (keep(rr)) *reinterpret_cast<uint4*>(dst(rr) + 16 * pc) = q;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();                 // the region is rewritten by the next records
}

// The lane's RoPE table entries of one row (columns 16 t + 4 g .. + 3, t < 4), for the row's position
// (clamped into the table, so that no position reads outside it).
__device__ __forceinline__ void kv_rope_tables(const bl_kv_epi& kv, int p, int g, float4 (&cs)[4], float4 (&sn)[4]) {
  p = p < 0 ? 0 : (p >= kv.P ? kv.P - 1 : p);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    cs[t] = *reinterpret_cast<const float4*>(kv.cos + (long)p * 64 + 16 * t + 4 * g);
    sn[t] = *reinterpret_cast<const float4*>(kv.sin + (long)p * 64 + 16 * t + 4 * g);
  }
}

// o: the fp32 outputs of one row of the wave's strip (exactly the values the plain epilogue stores);
// cs, sn: the row's RoPE table entries (used for Q and K when the tables are given); slot: the row's
// BOS slot (or -1); mrow0: the subtile's first row; region: the wave's LDS region
__device__ __forceinline__ void kv_epilogue_row(const bl_kv_epi& kv, int m, bool mok, int nstrip, float (&o)[8][4],
                                                int g, const float4 (&cs)[4], const float4 (&sn)[4], int slot,
                                                int mrow0, int M, uint8_t* __restrict__ region, int lane) {
  const int HD = kv.H * 128;
  const int part = nstrip / HD;
  const int h = (nstrip - part * HD) >> 7;
  const bool rope = kv.cos != nullptr && part < 2;
  if (rope) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float4 c = cs[t], sv = sn[t];
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float a = o[t][v], b = o[t + 4][v];
        o[t][v] = a * cc[v] - b * ss[v];
        o[t + 4][v] = b * cc[v] + a * ss[v];
      }
    }
  }
  // |x| through the float maximum's absolute-value source modifier, one instruction per value (the
  // values are finite, where this equals the largest magnitude bit pattern, +0 for -0)
  float mf = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) mf = fmaxf(mf, fabsf(o[t][v]));
  const uint32_t mx = bl_max_across_rows(bl_f2u(mf));
  const float gamma = bl_u2f(mx);
  const float den = gamma + kv.eps;
  const int r = lane & 15;
  const long rec = (long)m * kv.H + h;
  auto row_ok = [&](int rr) { return mrow0 + rr < M; };
  if (kv.bits[part] == 4) {
    kv_stage_records<4>(region, o, 7.0f / den, r, g, lane);
    uint8_t* base = kv.codes[part];
    kv_write_records<4>(region, lane, [&](int rr) { return base + ((long)(mrow0 + rr) * kv.H + h) * 64; }, row_ok);
    if (mok && g == 0) kv.scale[part][rec] = gamma / 7.0f;
  } else {
    kv_stage_records<3>(region, o, 3.0f / den, r, g, lane);
    uint8_t* base = kv.codes[part];
    kv_write_records<3>(region, lane, [&](int rr) { return base + ((long)(mrow0 + rr) * kv.H + h) * 48; }, row_ok);
    if (mok && g == 0) kv.scale[part][rec] = gamma / 3.0f;
    if (kv.bos_slot) {                                       // uniform over the launch
      const bool wr = mok && slot >= 0 && slot < kv.nslots;
      if (__ballot(wr) != 0ull) {
        // the rows' BOS slots go through LDS to the lanes that write their records
        int* slots = reinterpret_cast<int*>(region + 1024);
        if (lane < 16) slots[lane] = wr ? slot : -1;
        kv_stage_records<4>(region, o, 7.0f / den, r, g, lane);
        uint8_t* bbase = kv.bos_codes[part];
        kv_write_records<4>(region, lane, [&](int rr) { return bbase + ((long)slots[rr] * kv.H + h) * 64; },
                            [&](int rr) { return slots[rr] >= 0; });
        if (wr && g == 0) kv.bos_scale[part][(long)slot * kv.H + h] = gamma / 7.0f;
      }
    }
  }
}

template <int FMT, int EPI>
__global__ __launch_bounds__(256, 2) void k_gemm_mx(
    const uint8_t* __restrict__ A, const float* __restrict__ ascale, int M, int K, const uint8_t* __restrict__ W,
    const float* __restrict__ walpha, const uint8_t* __restrict__ W2, const float* __restrict__ w2alpha, int N,
    float* __restrict__ Y, long ldy, const float* R, long ldr, float* __restrict__ rowmax, const bl_kv_epi kv) {
  using C = CfgMx<FMT, EPI>;
  using F = AFmt<FMT>;
  using P = typename C::Plan;
  constexpr int NB = C::NB, SM = C::SM, SN = C::SN, BM = C::BM;
  constexpr bool FP6 = (FMT == BL_ACT_INT4_E3M2);
  constexpr int AFMT = FP6 ? 3 : 4;                  // activation operand: FP6 E3M2 or FP4 E2M1
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * P::BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int ntm = (M + BM - 1) / BM, ntn = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_of(blockIdx.x, ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * C::BN;
  const int KS = K >> 7, NG = N >> 4;
  const long arow = F::row_bytes(K);
  const uint8_t* Wm[2] = {W, W2};
  const int r16 = lane & 15, g4 = lane >> 4;

  // acc[mtx][s][t] = (weight tile t) x (activation subtile s)^T: lane holds row r16 of subtile s,
  // columns 4 g4 .. 4 g4 + 3 of tile t
  v4f acc[NB][SM][SN];
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
    for (int s = 0; s < SM; ++s)
#pragma unroll
      for (int t = 0; t < SN; ++t) acc[mtx][s][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // lane-constant LDS offsets of the activation fragment (row r16 of the wave's first 16-row
  // subtile): E3M2 24 bytes at 24 g as three 8-byte parts; E2M1 16 bytes at 16 g (one chunk)
  const int arow0 = wm * SM * 16 + r16;
  int aoff[3];
#pragma unroll
  for (int p = 0; p < 3; ++p) aoff[p] = FP6 ? a_off<FMT>(arow0, 24 * g4 + 8 * p) : a_off<FMT>(arow0, 16 * g4);

  // epilogue scalars are fetched before the K loop, which hides their latency
  float dsv[SM];
#pragma unroll
  for (int s = 0; s < SM; ++s) dsv[s] = ascale[min(m0 + wm * SM * 16 + 16 * s + r16, M - 1)];
  const float alpha = *walpha;
  // KV epilogue: the rows' positions and BOS slots, fetched before the K loop as well
  int kvpos[SM], kvslot[SM];
  if constexpr (EPI == BL_EPI_KV) {
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const int m = min(m0 + wm * SM * 16 + 16 * s + r16, M - 1);
      kvpos[s] = kv.cos ? kv.pos[m] : 0;
      kvslot[s] = kv.bos_slot ? kv.bos_slot[m] : -1;
    }
  }
  const float alpha2 = C::GLU ? *w2alpha : 0.f;

  P plan;
  plan.init(arow, m0, M, n0, NG, KS, wave, lane);
  const uint32_t lds0 = lds_addr_of(smem);
  // prologue: steps 0..NST-2 in flight (indices past the end re-fetch the last step, never read)
#pragma unroll
  for (int i = 0; i < NST - 1; ++i) plan.issue(lds0 + i * P::BYTES, A, Wm, min(i, KS - 1), wave, lane);

  for (int ks = 0; ks < KS; ++ks) {
    const uint8_t* cur = smem + (ks % NST) * P::BYTES;
    // step ks has landed when at most NST-2 later steps are still outstanding
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NST - 2) * P::LOADS));
    lds_barrier();

    // weight words of the step, expanded right before their first MFMA (subtile 0)
    const uint8_t* Bs = cur + BM * F::ROW + (wn * SN) * 512 + 8 * lane;
    uint2 bw[NB][SN];
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int t = 0; t < SN; ++t) bw[mtx][t] = *reinterpret_cast<const uint2*>(Bs + mtx * (C::BN / 16) * 512 + t * 512);
    v8i bf[NB][SN];
    // activation fragments are read one 16-row subtile ahead of the MFMAs that use them
    auto load_a = [&](int s) -> v8i {
      const uint8_t* ar = cur + s * 16 * F::ROW;
      if constexpr (FP6) {
        const uint2 p0 = *reinterpret_cast<const uint2*>(ar + aoff[0]);
        const uint2 p1 = *reinterpret_cast<const uint2*>(ar + aoff[1]);
        const uint2 p2 = *reinterpret_cast<const uint2*>(ar + aoff[2]);
        return v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p2.x, (int)p2.y, 0, 0};
      } else {
        const uint4 q = *reinterpret_cast<const uint4*>(ar + aoff[0]);
        return v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
    };
    v8i a_next = load_a(0);
    // refill the buffer every wave finished reading in step ks-1; issued after this step's
    // fragment reads, so that their LDS latency runs under the DMA issue
    plan.issue(lds0 + ((ks + NST - 1) % NST) * P::BYTES, A, Wm, min(ks + NST - 1, KS - 1), wave, lane);
    // the matrix-core phase runs at raised wave priority: while one wave of the CU issues its
    // MFMA chain, the sibling block's waves (stage waits, fragment reads, DMA issue) yield to it
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const v8i a = a_next;
      if (s + 1 < SM) a_next = load_a(s + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
        for (int t = 0; t < SN; ++t) {
          if (s == 0) bf[mtx][t] = expand_w_fp4(bw[mtx][t].x, bw[mtx][t].y);
          acc[mtx][s][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[mtx][t], a, acc[mtx][s][t], 4, AFMT, 0,
                                                                            127, 0, 127);
        }
      if (s == 0) {
#pragma unroll
        for (int k = 0; k < NB * SN; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU: one tile's expansion
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // the trailing (unused) loads land before the waves end
  lds_barrier();                               // every wave is done with the stage buffers (reused below)
  // the epilogue keeps the raised priority: its LDS staging and stores go ahead of the other
  // block's loads and fragment reads
  __builtin_amdgcn_s_setprio(1);

  // fp32 epilogue: the matrix-core sum is 2*sum(c t) (E3M2) or sum(2e t) = sum(doubled code * t)
  // (E2M1); x 0.5 is exact and gives sum(c t), respectively the half-unit count of the oracle.
  const int nw0 = n0 + wn * SN * 16 + 4 * g4;
  // KV epilogue: each subtile's RoPE table rows are fetched while the previous subtile is processed
  float4 kcs[2][4], ksn[2][4];
  if constexpr (EPI == BL_EPI_KV) {
    if (kv.cos) kv_rope_tables(kv, kvpos[0], g4, kcs[0], ksn[0]);
  }
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const int m = m0 + wm * SM * 16 + 16 * s + r16;
    const bool mok = m < M;
    const float sc = dsv[s] * alpha, sc2 = dsv[s] * alpha2;
    if constexpr (EPI == BL_EPI_KV) {
      if (kv.cos && s + 1 < SM) kv_rope_tables(kv, kvpos[s + 1], g4, kcs[(s + 1) & 1], ksn[(s + 1) & 1]);
    }
    float4 res[SN];
    if constexpr (EPI == BL_EPI_RESIDUAL) {
#pragma unroll
      for (int t = 0; t < SN; ++t) {
        const int n = nw0 + 16 * t;
        res[t] = (mok && n < N) ? *reinterpret_cast<const float4*>(R + (long)m * ldr + n) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float rmax = 0.f;
    float o[SN][4];
#pragma unroll
    for (int t = 0; t < SN; ++t) {
      const int n = nw0 + 16 * t;
      epilogue_vals<EPI>(mok && n < N, sc, sc2, res[t], rmax, [&](int mtx, int v) { return acc[mtx][s][t][v] * 0.5f; },
                         o[t]);
    }
    if constexpr (EPI == BL_EPI_RELU2_GLU) {
      // 4 tiles per subtile: the direct 64-byte row pieces measured faster than the staged rows
#pragma unroll
      for (int t = 0; t < SN; ++t) {
        const int n = nw0 + 16 * t;
        if (mok && n < N) *reinterpret_cast<float4*>(Y + (long)m * ldy + n) = make_float4(o[t][0], o[t][1], o[t][2], o[t][3]);
      }
    } else if constexpr (EPI == BL_EPI_KV) {
      static_assert(SN == 8, "one head of 128 per wave strip");
      const int nstrip = n0 + wn * SN * 16;
      if (nstrip < N) {                                      // wave-uniform: a whole strip or none
        if (Y)
          store_subtile_rows<SN>(Y, ldy, M, N, m0 + wm * SM * 16 + 16 * s, nstrip, o,
                                 reinterpret_cast<float*>(smem) + wave * (16 * (16 * SN + 4)), lane);
        kv_epilogue_row(kv, m, mok, nstrip, o, g4, kcs[s & 1], ksn[s & 1], kvslot[s], m0 + wm * SM * 16 + 16 * s, M,
                        reinterpret_cast<uint8_t*>(reinterpret_cast<float*>(smem) + wave * (16 * (16 * SN + 4))), lane);
      }
    } else {
      // whole-row stores through the wave's LDS region
      store_subtile_rows<SN>(Y, ldy, M, N, m0 + wm * SM * 16 + 16 * s, n0 + wn * SN * 16, o,
                             reinterpret_cast<float*>(smem) + wave * (16 * (16 * SN + 4)), lane);
    }
    if constexpr (EPI == BL_EPI_RELU2_GLU) {
      if (rowmax) {
        // |h| >= 0, so the maximum of the bit patterns is the maximum of the values
        const uint32_t rb = bl_max_across_rows(bl_f2u(rmax));
        if (g4 == 0 && mok) atomicMax(reinterpret_cast<unsigned int*>(rowmax) + m, rb);
      }
    }
  }
}

// ============================================================================ int8 matrix cores
template <int FMT, int EPI, int BN0>
struct CfgI8 {
  static constexpr bool A8 = (FMT == BL_ACT_INT8);
  static constexpr bool GLU = (EPI == BL_EPI_RELU2_GLU);
  static constexpr int NB = GLU ? 2 : 1;
  // 4 waves (2 x 2), 128 x BN0 block (per matrix: BN0 / NB), 64 x BN/2 per wave; two blocks share a
  // CU (at most 80 KB of LDS and 256 registers per lane each), so one block's loads, LDS reads and
  // epilogue overlap the other's matrix-core work
  static constexpr int NW = 4, WGM = 2, WGN = 2;
  static constexpr int BM = 128, BN = BN0 / NB;
  static constexpr int SM = BM / WGM / 16, SN = BN / WGN / 16;
  using Plan = StagePlan<FMT, BM, BN, NB, NW>;
  static constexpr int NSTAGE = Plan::BYTES * NST <= 81920 ? NST : 3;
};

template <int FMT, int EPI, int BN0>
__global__ __launch_bounds__(256, 2) void k_gemm_i8(const uint8_t* __restrict__ A, const float* __restrict__ ascale,
                                                     int M, int K, const uint8_t* __restrict__ W,
                                                     const float* __restrict__ walpha,
                                                     const uint8_t* __restrict__ W2,
                                                     const float* __restrict__ w2alpha, int N,
                                                     float* __restrict__ Y, long ldy, const float* R, long ldr,
                                                     float* __restrict__ rowmax) {
  using C = CfgI8<FMT, EPI, BN0>;
  using F = AFmt<FMT>;
  using P = typename C::Plan;
  constexpr int NB = C::NB, SM = C::SM, SN = C::SN, NS = C::NSTAGE, BM = C::BM;
  constexpr bool A8 = C::A8;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * P::BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int ntm = (M + BM - 1) / BM, ntn = (N + C::BN - 1) / C::BN;
  int tm, tn;
  tile_of(blockIdx.x, ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * C::BN;
  const int KS = K >> 7, NG = N >> 4;
  const long arow = F::row_bytes(K);
  const uint8_t* Wm[2] = {W, W2};
  const int r16 = lane & 15, g4 = lane >> 4;

  // acc[mtx][s][t] = (weight tile t) x (activation subtile s)^T: lane holds row r16 of subtile s,
  // columns 4 g4 .. 4 g4 + 3 of tile t
  v4i acc[NB][SM][SN];
#pragma unroll
  for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
    for (int s = 0; s < SM; ++s)
#pragma unroll
      for (int t = 0; t < SN; ++t) acc[mtx][s][t] = v4i{0, 0, 0, 0};

  // lane-constant fragment offsets: INT8 16 bytes at 32 g + 16 i, INT4 16 bytes (both i) at 16 g
  const int arow0 = wm * SM * 16 + r16;
  int aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) aoff[i] = A8 ? a_off<FMT>(arow0, 32 * g4 + 16 * i) : a_off<FMT>(arow0, 16 * g4);

  P plan;
  plan.init(arow, m0, M, n0, NG, KS, wave, lane);
  const uint32_t lds0 = lds_addr_of(smem);
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) plan.issue(lds0 + i * P::BYTES, A, Wm, min(i, KS - 1), wave, lane);

  for (int ks = 0; ks < KS; ++ks) {
    const uint8_t* cur = smem + (ks % NS) * P::BYTES;
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 2) * P::LOADS));
    lds_barrier();

    // weight words of the step; each is expanded right before its first MFMA (subtile 0), so the
    // expansion overlaps the matrix cores instead of delaying the first MFMA of the step
    const uint8_t* Bs = cur + BM * F::ROW + (wn * SN) * 512 + 8 * lane;
    uint2 bw[NB][SN];
#pragma unroll
    for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
      for (int t = 0; t < SN; ++t) bw[mtx][t] = *reinterpret_cast<const uint2*>(Bs + mtx * (C::BN / 16) * 512 + t * 512);
    v4i bf[NB][SN][2];
    // A fragments (both 64-wide K halves of the step) are read one 16-row subtile ahead
    auto load_a = [&](int s, uint4 (&q)[2]) {
      const uint8_t* ar = cur + s * 16 * F::ROW;
      q[0] = *reinterpret_cast<const uint4*>(ar + aoff[0]);
      if constexpr (A8) q[1] = *reinterpret_cast<const uint4*>(ar + aoff[1]);
    };
    uint4 qn[2];
    load_a(0, qn);
    // refill of the buffer freed in step ks-1, issued after this step's fragment reads
    plan.issue(lds0 + ((ks + NS - 1) % NS) * P::BYTES, A, Wm, min(ks + NS - 1, KS - 1), wave, lane);
#pragma unroll
    for (int s = 0; s < SM; ++s) {
      const uint4 q[2] = {qn[0], qn[1]};
      if (s + 1 < SM) load_a(s + 1, qn);
      __builtin_amdgcn_sched_barrier(0);
      if (s > 0 && A8) {
        // zero-slice skip: a 16-row x 128-k slice of all-zero codes contributes nothing (subtile 0
        // always runs: it also expands the step's weights)
        const uint32_t nz = q[0].x | q[0].y | q[0].z | q[0].w | q[1].x | q[1].y | q[1].z | q[1].w;
        if (__ballot(nz != 0u) == 0ull) continue;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v4i a = A8 ? expand_a_int8(q[i]) : (i ? expand_a_int4(q[0].z, q[0].w) : expand_a_int4(q[0].x, q[0].y));
#pragma unroll
        for (int mtx = 0; mtx < NB; ++mtx)
#pragma unroll
          for (int t = 0; t < SN; ++t) {
            if (s == 0) bf[mtx][t][i] = expand_w_i8(i ? bw[mtx][t].y : bw[mtx][t].x);
            acc[mtx][s][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bf[mtx][t][i], a, acc[mtx][s][t], 0, 0, 0);
          }
      }
      if (s == 0) {
        // interleave the weight expansion with the first subtile's MFMAs
#pragma unroll
        for (int k = 0; k < 2 * NB * SN; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);   // VALU
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  lds_barrier();                               // every wave is done with the stage buffers (reused below)

  const float alpha = *walpha;
  const float alpha2 = C::GLU ? *w2alpha : 0.f;
  constexpr int SHIFT = A8 ? 6 : 10;
  const int nw0 = n0 + wn * SN * 16 + 4 * g4;
#pragma unroll
  for (int s = 0; s < SM; ++s) {
    const int m = m0 + wm * SM * 16 + 16 * s + r16;
    const bool mok = m < M;
    const float ds = ascale[mok ? m : M - 1];
    const float sc = ds * alpha, sc2 = ds * alpha2;
    float4 res[SN];
    if constexpr (EPI == BL_EPI_RESIDUAL) {
#pragma unroll
      for (int t = 0; t < SN; ++t) {
        const int n = nw0 + 16 * t;
        res[t] = (mok && n < N) ? *reinterpret_cast<const float4*>(R + (long)m * ldr + n) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float rmax = 0.f;
    if constexpr (EPI == BL_EPI_RELU2_GLU) {
#pragma unroll
      for (int t = 0; t < SN; ++t) {
        const int n = nw0 + 16 * t;
        epilogue_cols<EPI>(m, n, mok && n < N, sc, sc2, Y, ldy, res[t], rmax,
                           [&](int mtx, int v) { return (float)(acc[mtx][s][t][v] >> SHIFT); });
      }
    } else {
      float o[SN][4];
#pragma unroll
      for (int t = 0; t < SN; ++t) {
        const int n = nw0 + 16 * t;
        epilogue_vals<EPI>(mok && n < N, sc, sc2, res[t], rmax,
                           [&](int mtx, int v) { return (float)(acc[mtx][s][t][v] >> SHIFT); }, o[t]);
      }
      store_subtile_rows<SN>(Y, ldy, M, N, m0 + wm * SM * 16 + 16 * s, n0 + wn * SN * 16, o,
                             reinterpret_cast<float*>(smem) + wave * (16 * (16 * SN + 4)), lane);
    }
    if constexpr (EPI == BL_EPI_RELU2_GLU) {
      if (rowmax) {
        // |h| >= 0, so the maximum of the bit patterns is the maximum of the values
        const uint32_t rb = bl_max_across_rows(bl_f2u(rmax));
        if (g4 == 0 && mok) atomicMax(reinterpret_cast<unsigned int*>(rowmax) + m, rb);
      }
    }
  }
}

// ----------------------------------------------------------------------------- launchers
template <int FMT, int EPI>
hipError_t launch(const bl_mm_args& a, hipStream_t st) {
  const uint8_t* A = static_cast<const uint8_t*>(a.A);
  const uint8_t* W = static_cast<const uint8_t*>(a.W);
  const uint8_t* W2 = static_cast<const uint8_t*>(a.W2);
  if constexpr (FMT == BL_ACT_FP4_E2M1 || FMT == BL_ACT_INT4_E3M2) {
    using C = CfgMx<FMT, EPI>;
    const int ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL((k_gemm_mx<FMT, EPI>), dim3(ntm * ntn), dim3(C::NW * 64), 0, st, A, a.ascale, a.M, a.K,
                       W, a.walpha, W2, a.w2alpha, a.N, a.Y, a.ldy, a.R, a.ldr, a.rowmax, bl_kv_epi{});
  } else {
    // 128 x 256 tiles when they give every CU at least two blocks, 128 x 128 tiles otherwise
    using C2 = CfgI8<FMT, EPI, 256>;
    const int ntm = (a.M + 127) / 128;
    const long wide = (long)ntm * ((a.N + C2::BN - 1) / C2::BN);
    if (wide >= 512) {
      hipLaunchKernelGGL((k_gemm_i8<FMT, EPI, 256>), dim3(wide), dim3(C2::NW * 64), 0, st, A, a.ascale, a.M, a.K, W,
                         a.walpha, W2, a.w2alpha, a.N, a.Y, a.ldy, a.R, a.ldr, a.rowmax);
    } else {
      using C1 = CfgI8<FMT, EPI, 128>;
      hipLaunchKernelGGL((k_gemm_i8<FMT, EPI, 128>), dim3((long)ntm * ((a.N + C1::BN - 1) / C1::BN)), dim3(C1::NW * 64),
                         0, st, A, a.ascale, a.M, a.K, W, a.walpha, W2, a.w2alpha, a.N, a.Y, a.ldy, a.R, a.ldr,
                         a.rowmax);
    }
  }
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

hipError_t bl_launch_gemm_kv(const bl_mm_args& a, const bl_kv_epi& kv, hipStream_t st) {
  const uint8_t* A = static_cast<const uint8_t*>(a.A);
  const uint8_t* W = static_cast<const uint8_t*>(a.W);
  if (a.fmt == BL_ACT_INT4_E3M2) {
    using C = CfgMx<BL_ACT_INT4_E3M2, BL_EPI_KV>;
    const int ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL((k_gemm_mx<BL_ACT_INT4_E3M2, BL_EPI_KV>), dim3(ntm * ntn), dim3(C::NW * 64), 0, st, A,
                       a.ascale, a.M, a.K, W, a.walpha, nullptr, nullptr, a.N, a.Y, a.ldy, nullptr, 0L, nullptr, kv);
  } else {
    using C = CfgMx<BL_ACT_FP4_E2M1, BL_EPI_KV>;
    const int ntm = (a.M + C::BM - 1) / C::BM, ntn = (a.N + C::BN - 1) / C::BN;
    hipLaunchKernelGGL((k_gemm_mx<BL_ACT_FP4_E2M1, BL_EPI_KV>), dim3(ntm * ntn), dim3(C::NW * 64), 0, st, A,
                       a.ascale, a.M, a.K, W, a.walpha, nullptr, nullptr, a.N, a.Y, a.ldy, nullptr, 0L, nullptr, kv);
  }
  return hipGetLastError();
}

hipError_t bl_launch_gemm(const bl_mm_args& a, hipStream_t st) {
  switch (a.fmt) {
    case BL_ACT_INT4: return launch_epi<BL_ACT_INT4>(a, st);
    case BL_ACT_FP4_E2M1: return launch_epi<BL_ACT_FP4_E2M1>(a, st);
    case BL_ACT_INT4_E3M2: return launch_epi<BL_ACT_INT4_E3M2>(a, st);
    default: return launch_epi<BL_ACT_INT8>(a, st);
  }
}
