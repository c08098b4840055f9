// KV-cache quantizer of BitNet a4.8 ("Low-Bit KV Cache Quantization", architecture write-up
// section 3.4, and the low-bit attention results of Table 3): after rotary position embedding,
// each (token, head) of Q, K or V is quantized with absmax to 4-bit or 3-bit unsigned integers;
// in a 3-bit cache the heads of beginning-of-sequence tokens are kept at 4 bits.
//
// Readings taken here: the absmax scale is per (token, head) over the head's D values and
// symmetric, Qp = 2^(b-1) - 1, code c = RoundClip(RN32(x * RN32(Qp / RN32(gamma + eps))), -Qp-1, Qp)
// stored as u = c + 2^(b-1); RoPE pairs element i with i + D/2 (rotate-half form) using caller
// cos/sin tables, every product and sum rounded to fp32 on its own.
//
// One pass over HBM: a group of D/8 lanes holds one head, each lane 4 elements of the first half
// and the 4 partner elements of the second half, so the rotation needs no data exchange; the head
// max is a reduction inside the group (DPP row exchanges); codes are packed with lane exchanges and
// written as dwords.
#include "bl_common.h"
#include "bl_kernels.h"

namespace {

template <int IN_F32>
__device__ __forceinline__ void kv_load4(const void* x, long off, float v[4]) {
  if constexpr (IN_F32) {
    const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + off);
    v[0] = bl_bf16lo(q.x); v[1] = bl_bf16hi(q.x); v[2] = bl_bf16lo(q.y); v[3] = bl_bf16hi(q.y);
  }
}

// absmax codes u = RoundClip(rint(x * s), -Qp-1, Qp) + 2^(b-1) of four values, packed b bits apart
template <int BITS>
__device__ __forceinline__ uint32_t kv_codes4(const float v[4], float s) {
  constexpr float QP = (float)((1 << (BITS - 1)) - 1);
  constexpr int OFF = 1 << (BITS - 1);
  uint32_t r = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float y = __builtin_rintf(v[j] * s);
    y = fminf(fmaxf(y, -QP - 1.0f), QP);
    r |= (uint32_t)((int)y + OFF) << (BITS * j);
  }
  return r;
}

// 4-bit record of one head: lane l of the head's group owns codes 4l..4l+3 of each half (16 bits
// each); even lanes write the first-half dword of the lane pair, odd lanes the second-half one.
template <int D>
__device__ __forceinline__ void kv_store4(uint8_t* rec_base, int l, uint32_t a16, uint32_t b16, bool ok) {
  const uint32_t send = (l & 1) ? a16 : b16;
  const uint32_t recv = bl_dpp<0xB1>(send);        // the pair partner (lane xor 1)
  if (!ok) return;
  if ((l & 1) == 0)
    *reinterpret_cast<uint32_t*>(rec_base + 2 * l) = a16 | (recv << 16);
  else
    *reinterpret_cast<uint32_t*>(rec_base + D / 4 + 2 * (l - 1)) = recv | (b16 << 16);
}

// 3-bit record: 8 consecutive lanes hold 32 consecutive codes of a half (12 bits each) = 3 dwords.
// Lane k (< 6) of the 8-lane group assembles dword k % 3 of the first (k < 3) or second half from
// the up to four 12-bit pieces that overlap it.
template <int D>
__device__ __forceinline__ void kv_store3(uint8_t* rec_base, int lane, int l, uint32_t a12, uint32_t b12, bool ok) {
  const uint32_t piece = a12 | (b12 << 12);
  const int k = l & 7;
  const int kk = k < 3 ? k : k - 3;
  const int sel = k < 3 ? 0 : 12;
  const int first = (32 * kk) / 12;
  uint32_t dw = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = first + q;
    const uint32_t pv = (__shfl(piece, (lane & ~7) + (j < 8 ? j : 7), 64) >> sel) & 0xFFFu;
    const int off = 12 * j - 32 * kk;
    if (j < 8) dw |= off >= 0 ? (off < 32 ? pv << off : 0u) : (pv >> (-off));
  }
  if (ok && k < 6)
    *reinterpret_cast<uint32_t*>(rec_base + (k < 3 ? 0 : 3 * D / 16) + 12 * (l >> 3) + 4 * kk) = dw;
}

template <int IN_F32, int D, int BITS, bool ROPE>
__global__ __launch_bounds__(256) void k_kv_quant(const void* __restrict__ x, long ldx, int T, int H,
                                                  const int* __restrict__ pos, const float* __restrict__ cosb,
                                                  const float* __restrict__ sinb, int P, float eps,
                                                  uint8_t* __restrict__ codes, float* __restrict__ scale,
                                                  const int* __restrict__ bos_slot, int nslots,
                                                  uint8_t* __restrict__ bos_codes, float* __restrict__ bos_scale) {
  constexpr int LPH = D / 8;        // lanes per head
  constexpr int HPW = 64 / LPH;     // heads per wave
  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = lane % LPH;
  const long rec = wave * HPW + lane / LPH;
  const bool ok = rec < (long)T * H;
  const int t = ok ? (int)(rec / H) : 0;
  const int h = ok ? (int)(rec % H) : 0;

  float a[4] = {0.f, 0.f, 0.f, 0.f}, b[4] = {0.f, 0.f, 0.f, 0.f};
  if (ok) {
    const long base = (long)t * ldx + (long)h * D + 4 * l;
    kv_load4<IN_F32>(x, base, a);
    kv_load4<IN_F32>(x, base + D / 2, b);
    if constexpr (ROPE) {
      int p = pos[t];
      p = p < 0 ? 0 : (p >= P ? P - 1 : p);              // out-of-range positions never read outside the tables
      const float4 c = *reinterpret_cast<const float4*>(cosb + (long)p * (D / 2) + 4 * l);
      const float4 s = *reinterpret_cast<const float4*>(sinb + (long)p * (D / 2) + 4 * l);
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float na = a[j] * cc[j] - b[j] * ss[j];
        const float nb = b[j] * cc[j] + a[j] * ss[j];
        a[j] = na;
        b[j] = nb;
      }
    }
  }
  uint32_t mx = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t ua = bl_f2u(a[j]) & 0x7FFFFFFFu, ub = bl_f2u(b[j]) & 0x7FFFFFFFu;
    mx = ua > mx ? ua : mx;
    mx = ub > mx ? ub : mx;
  }
  // head maximum over the LPH lanes of the group: DPP exchanges inside rows of 16 lanes (xor 1,
  // xor 2, the mirror of each 8 lanes, the mirror of the row), then one shuffle across rows for D = 256
  mx = max(mx, bl_dpp<0xB1>(mx));                  // quad_perm(1, 0, 3, 2)
  mx = max(mx, bl_dpp<0x4E>(mx));                  // quad_perm(2, 3, 0, 1)
  mx = max(mx, bl_dpp<0x141>(mx));                 // row_half_mirror
  if constexpr (LPH >= 16) mx = max(mx, bl_dpp<0x140>(mx));   // row_mirror
  if constexpr (LPH >= 32) mx = max(mx, (uint32_t)__shfl_xor(mx, 16, 64));
  static_assert(LPH == 8 || LPH == 16 || LPH == 32, "head groups of 8, 16 or 32 lanes");
  const float gamma = bl_u2f(mx);
  const float den = gamma + eps;

  {
    constexpr float QP = (float)((1 << (BITS - 1)) - 1);
    const float s = QP / den;
    const uint32_t ca = kv_codes4<BITS>(a, s), cb = kv_codes4<BITS>(b, s);
    uint8_t* rb = codes + rec * (D * BITS / 8);
    if constexpr (BITS == 4)
      kv_store4<D>(rb, l, ca, cb, ok);
    else
      kv_store3<D>(rb, lane, l, ca, cb, ok);
    if (ok && l == 0) scale[rec] = gamma / QP;
  }
  if constexpr (BITS == 3) {
    if (bos_slot) {                                       // uniform over the launch
      const int slot = ok ? bos_slot[t] : -1;
      const bool wr = slot >= 0 && slot < nslots;
      if (__ballot(wr) != 0ull) {
        const float s4 = 7.0f / den;
        const uint32_t ca = kv_codes4<4>(a, s4), cb = kv_codes4<4>(b, s4);
        const long brec = (long)(wr ? slot : 0) * H + h;
        kv_store4<D>(bos_codes + brec * (D / 2), l, ca, cb, wr);
        if (wr && l == 0) bos_scale[brec] = gamma / 7.0f;
      }
    }
  }
}

template <int IN_F32, int D, int BITS>
hipError_t launch_d(const bl_kv_args& a, hipStream_t st) {
  constexpr int HPW = 64 / (D / 8);
  const long recs = (long)a.T * a.H;
  const long waves = (recs + HPW - 1) / HPW;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (a.cos)
    hipLaunchKernelGGL((k_kv_quant<IN_F32, D, BITS, true>), grid, block, 0, st, a.x, a.ldx, a.T, a.H, a.pos, a.cos,
                       a.sin, a.P, a.eps, static_cast<uint8_t*>(a.codes), a.scale, a.bos_slot, a.nslots,
                       static_cast<uint8_t*>(a.bos_codes), a.bos_scale);
  else
    hipLaunchKernelGGL((k_kv_quant<IN_F32, D, BITS, false>), grid, block, 0, st, a.x, a.ldx, a.T, a.H, a.pos, a.cos,
                       a.sin, a.P, a.eps, static_cast<uint8_t*>(a.codes), a.scale, a.bos_slot, a.nslots,
                       static_cast<uint8_t*>(a.bos_codes), a.bos_scale);
  return hipGetLastError();
}

template <int IN_F32, int BITS>
hipError_t launch_bits(const bl_kv_args& a, hipStream_t st) {
  switch (a.D) {
    case 64: return launch_d<IN_F32, 64, BITS>(a, st);
    case 128: return launch_d<IN_F32, 128, BITS>(a, st);
    case 256: return launch_d<IN_F32, 256, BITS>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t bl_launch_kv_quant(const bl_kv_args& a, hipStream_t st) {
  if (a.T == 0 || a.H == 0) return hipSuccess;
  if (a.in_f32)
    return a.bits == 4 ? launch_bits<1, 4>(a, st) : launch_bits<1, 3>(a, st);
  return a.bits == 4 ? launch_bits<0, 4>(a, st) : launch_bits<0, 3>(a, st);
}
