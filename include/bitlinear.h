/*
 * bitlinear.h -- C ABI of the BitNet a4.8 BitLinear hot path on AMD Instinct MI355X (gfx950).
 *
 * The operations follow "BitNet a4.8: 4-bit Activations for 1-bit LLMs" (architecture write-up,
 * section 3.4 "Detailed, Sentence-Based Technical Breakdown"):
 *   ternary weights      Q_w(W) = alpha * RoundClip(W/(alpha+eps), -1, 1), alpha = mean|W|     (paper Eq. 2)
 *   4-bit activations    Y = Q_INT4(X) Q_w(W)^T, Q_INT4 absmean with sqrt(7)                    (paper Eq. 6-7)
 *                        FP4 E2M1 MinMax quantizer as the floating-point alternative            (paper Eq. 8-9)
 *   sparse 8-bit         Y = (Q_INT8(X) . M) Q_w(W)^T, M = Top_k(|X|), Q_INT8 absmax             (paper Eq. 1)
 *   FFN gate             ReLU^2 GLU(X) = X W_up^T . ReLU^2(X W_gate^T)                           (paper Eq. 5)
 * and section 3.2 "Big-Picture Architecture" (residual add after the output projection).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Pointers named d_* are DEVICE pointers (HIP device memory of the current device); pointers
 *    named h_* are host pointers. The caller allocates and owns every buffer; the library never
 *    allocates, frees or keeps state between calls (it is reentrant).
 *  * `stream` is a hipStream_t passed as void* (NULL = the null stream). All device work is
 *    enqueued on it; BL_OK means "validated and enqueued", results are ready when the stream is.
 *  * Arguments are validated on the host before anything is enqueued. On any error status nothing
 *    is enqueued and no output is touched. BL_ERR_HIP reports a failed launch (hipGetLastError).
 *  * Activations X are row-major [M, K] (tokens x features) with row stride ldx elements.
 *    Weights W are [N, K] as in a linear layer; outputs Y = X W^T are row-major [M, N], row stride ldy.
 *  * Shapes: K % 128 == 0 (one packed weight tile and one matrix-core step are 128 wide),
 *    N % 16 == 0, M >= 1 (any value, ragged tiles are masked); M*K, N*K < 2^31.
 *    The matmuls (GEMM, GEMV, conditional GLU) take K <= 2^18 - 128 = 262016: the int8-core INT4
 *    path keeps 1024 * sum(c t) in int32, which stays exact up to there (all paths do).
 *  * Alignment: code buffers, packed weights, x, y and the residual must be 16-byte aligned;
 *    ldx*elem_size, ldy*4 and ldr*4 must be multiples of 16 bytes.
 *  * Inputs are finite (no NaN or Inf). eps must be finite and > 0.
 *  * Rounding: every float32 operation is a single IEEE operation, round to nearest even, never
 *    fused; round() of the quantizers is round-half-to-even.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 2

typedef enum {
  BL_OK = 0,
  BL_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad enum, eps <= 0, ld too small, keep out of range */
  BL_ERR_UNSUPPORTED_SHAPE = 2,  /* K % 128, N % 16, M > 8 for decode, size limits */
  BL_ERR_MISALIGNED = 3,         /* a pointer or row stride breaks the 16-byte rule */
  BL_ERR_WORKSPACE_TOO_SMALL = 4,
  BL_ERR_HIP = 5
} bl_status;

typedef enum {
  BL_ACT_INT4 = 0, BL_ACT_FP4_E2M1 = 1, BL_ACT_INT8 = 2, BL_ACT_INT4_E3M2 = 3,
  BL_ACT_FP4_E2M1_POW2 = 4   /* quantizer only: FP4 codes with a power-of-two scale (matmuls take them as FP4_E2M1) */
} bl_act_format;
typedef enum { BL_IN_BF16 = 0, BL_IN_F32 = 1 } bl_in_dtype;
typedef enum { BL_EPI_NONE = 0, BL_EPI_RESIDUAL = 1, BL_EPI_RELU2_GLU = 2 } bl_epi_kind;

/* Operations, for bitlinear_workspace_size. */
typedef enum {
  BL_OP_QUANTIZE_ACT = 0, BL_OP_QUANTIZE_ACT_PER_TENSOR = 1, BL_OP_PACK_TERNARY = 2, BL_OP_PACK_TERNARY_ROWS = 3,
  BL_OP_GEMM_W158A4 = 4, BL_OP_GEMM_W158A8_SPARSE = 5, BL_OP_GEMV_DECODE = 6, BL_OP_GEMV_DECODE_GLU_CONDITIONAL = 7,
  BL_OP_KV_QUANTIZE = 8, BL_OP_PACK_TERNARY_A8 = 9
} bl_op;

/* bitlinear_workspace_size: bytes of caller workspace the operation `op` needs for an [M, K] input and
 * N outputs (N and K are accepted for every op; only the per-tensor quantizer depends on M). 0 for the
 * operations that take no workspace; SIZE_MAX for an unknown op. Equals
 * bitlinear_quantize_per_tensor_workspace_bytes(M) and bitlinear_pack_workspace_bytes() for those ops. */
size_t bitlinear_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K);

/*
 * Quantized activation codes (written by bitlinear_quantize_act, read by the matmul entry points):
 *   INT4      M x K/2 bytes, row stride K/2: element 2j in the low nibble of byte j, 2j+1 in the high
 *             nibble; two's-complement nibbles, codes in [-8, 7]. scale[m] = beta_m / sqrt(7).
 *   FP4_E2M1  same nibble layout; nibble = sign<<3 | e, e indexes the E2M1 magnitudes
 *             {0, 0.5, 1, 1.5, 2, 3, 4, 6} (OCP E2M1 encoding); zero is always +0. scale[m] = gamma_m / 6.
 *   FP4_E2M1_POW2 (quantizer output only) the FP4_E2M1 layout with scale[m] = 2^p_m, the power of two
 *             of the scale variant below; the matmul entry points take these codes as BL_ACT_FP4_E2M1.
 *   INT8      M x K bytes, row stride K, codes in [-127, 127] (0 where Top-K masked). scale[m] = gamma_m / 127.
 *   INT4_E3M2 the INT4 absmean codes (same values and scale as INT4) stored 6 bits each as their exact
 *             FP6 E3M2 bit pattern (sign bit 5, 3 exponent bits with bias 3, 2 mantissa bits:
 *             1 = 0x0C, 2 = 0x10, 3 = 0x12, 4 = 0x14, 5 = 0x15, 6 = 0x16, 7 = 0x17, 8 = 0x18, 0 = 0x00),
 *             in tiles of 16 rows x 128 codes (1536 bytes): tile (m/16, k/128) at byte offset
 *             ((m/16) * (K/128) + k/128) * 1536; inside it row m%16 takes 96 bytes and code k%128 sits
 *             in bits [6 (k%128), 6 (k%128) + 6) of those bytes read as a little-endian bit stream.
 *             The buffer holds ceil(M/16) * 16 rows (3K/4 bytes each); rows from M on are padding, never
 *             written and never used. This is the layout the FP6 x FP4 matrix cores stream;
 *             bitlinear_gemm_w158a4 runs INT4 activations given in it on those cores, exactly.
 * Dequantized activation = code value * scale[m].
 *
 * Packed ternary weights (bitlinear_pack_ternary output, N*K/4 bytes, 2 bits per weight):
 *   2-bit field: 00 = 0, 01 = +1, 11 = -1 (10 is never written).
 *   Tiles of 16 rows (n) x 128 columns (k), 512 bytes each, tile (k/128, n/16) at byte offset
 *   ((k/128) * (N/16) + n/16) * 512 (all tiles of one 128-wide K slice are contiguous).
 *   Inside a tile, with r = n % 16 and kk = k % 128:
 *   lane L = 16 * (kk / 32) + r owns bytes [8 L, 8 L + 8) = two little-endian 32-bit words;
 *   word i = (kk % 32) / 16 holds the 16 weights kk0..kk0+15 (kk0 = 16 * (kk / 16)); weight
 *   kk0 + q (q < 8) sits in bits [4q, 4q+2) and weight kk0 + 8 + q in bits [4q+2, 4q+4).
 *   (Each 512-byte tile is exactly two B operands of a 16x16x64 int8 MFMA, or one of a
 *   16x16x128 FP4 MFMA, with no per-element shuffling.)
 */

/* ---------------------------------------------------------------------------------------------
 * bitlinear_quantize_act: per-token activation quantizer (one row of X = one token).
 *   INT4 absmean (section 3.4, 4-bit quantization, paper Eq. 6-7):
 *     beta = RN32(RN64(sum_k |x|) / K) with the sum exact; s = RN32(RN32(sqrt7) / RN32(beta + eps));
 *     code = clamp(rint(RN32(x * s)), -8, 7).
 *     fmt BL_ACT_INT4_E3M2 computes the same codes and stores them in the E3M2 layout above.
 *   FP4 E2M1 MinMax (paper Eq. 8-9; reading: the row max maps to 6): gamma = max|x|;
 *     s = RN32(6 / RN32(gamma + eps)); code = nearest E2M1 value of RN32(x * s), ties to even
 *     mantissa, saturating at 6.
 *     fmt BL_ACT_FP4_E2M1_POW2 (the reading of the same equations with a power-of-two scale): p is the
 *     smallest integer with 6 * 2^p >= gamma (at least -126); s = 2^-p (x * s is exact), the same
 *     rounding, scale[m] = 2^p; eps is not used and an all-zero row gets scale 0.
 *   INT8 absmax with optional Top-K (section 3.4, sparsification, paper Eq. 1): gamma = max|x|
 *     over the whole row; s = RN32(127 / RN32(gamma + eps)); code = clamp(rint(RN32(x * s)), -128, 127)
 *     for the topk_keep entries of largest |x| (ties to the lower index), 0 elsewhere.
 * Arguments:
 *   d_x          [M, K] input, bf16 (in_dtype BL_IN_BF16) or float32 (BL_IN_F32), row stride ldx >= K.
 *                INT4 and FP4 accept bf16 and float32; INT8 accepts both.
 *   fmt          bl_act_format of the output.
 *   topk_keep    INT8 only: number of survivors per row in [0, K]; ANY NEGATIVE VALUE disables the mask
 *                (every entry kept). 0 is not "off": it keeps nothing, so every code is 0. K keeps every
 *                entry, like a negative value. Must be negative for the 4-bit formats.
 *   eps          > 0.
 *   d_row_absmax_hint  optional [M] float32 equal to max_k |x[m, k]| bit for bit (for instance the
 *                row_absmax output of the ReLU^2 GLU epilogue); INT8/FP4 then skip their max pass.
 *                Ignored for INT4. NULL = compute it.
 *   d_codes      output codes (layout above).   d_scale  output [M] float32 dequant scales.
 *   d_mask       optional output [M][K/32] uint32 survivor bitmap (bit k%32 of word k/32); INT8 only.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_quantize_act(const void* d_x, int32_t in_dtype, int64_t M, int64_t K, int64_t ldx,
                                 int32_t fmt, int32_t topk_keep, float eps,
                                 const float* d_row_absmax_hint,
                                 void* d_codes, float* d_scale, uint32_t* d_mask, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_quantize_act_per_tensor: the activation quantizers with ONE scale for the whole [M, K]
 * tensor (the pages' "all entries in X" read per tensor; the per-token form above is the default):
 *   INT4 / INT4_E3M2: beta = RN32(RN64(exact sum over all M K entries of |x|) / (M K)), then every
 *   row as above with that beta; FP4_E2M1 / FP4_E2M1_POW2 / INT8 (no Top-K): gamma = max |x| over the
 *   tensor. scale[m] holds the same value for every row, so the matmuls take these codes unchanged.
 * Arguments as for bitlinear_quantize_act, plus d_workspace of at least
 * bitlinear_quantize_per_tensor_workspace_bytes(M) bytes (16-byte aligned; contents on entry do not
 * matter, the call overwrites it); that query returns 0 for M <= 0 and SIZE_MAX for M >= 2^31.
 * ------------------------------------------------------------------------------------------- */
size_t bitlinear_quantize_per_tensor_workspace_bytes(int64_t M);
bl_status bitlinear_quantize_act_per_tensor(const void* d_x, int32_t in_dtype, int64_t M, int64_t K, int64_t ldx,
                                            int32_t fmt, float eps, void* d_workspace, size_t ws_bytes,
                                            void* d_codes, float* d_scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_quantize_act_per_tensor_noalloc: bitlinear_quantize_act_per_tensor for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and harnesses that forbid
 * hipMalloc): no workspace argument; the call allocates nothing and uses a fixed scratch array the
 * library keeps on each device it runs on (bitlinear_noalloc_scratch_bytes() bytes, held until the
 * process ends), which holds the workspace of at most BITLINEAR_NOALLOC_MAX_M rows.
 *   Arguments, results and other errors as for bitlinear_quantize_act_per_tensor (the outputs are
 *   identical to it); M > BITLINEAR_NOALLOC_MAX_M -> BL_ERR_WORKSPACE_TOO_SMALL, nothing enqueued.
 *   The scratch array's address on a device is looked up on the first call made with that device
 *   current (BL_ERR_HIP if the lookup fails). Every call rewrites all of the scratch it reads, so
 *   what a previous call left there does not matter; but all calls on one device share the one
 *   array, so calls that overlap on one device (concurrent streams or host threads) race and give
 *   undefined results: serialize them.
 * ------------------------------------------------------------------------------------------- */
#define BITLINEAR_NOALLOC_MAX_M 65536
size_t bitlinear_noalloc_scratch_bytes(void);
bl_status bitlinear_quantize_act_per_tensor_noalloc(const void* d_x, int32_t in_dtype, int64_t M, int64_t K,
                                                    int64_t ldx, int32_t fmt, float eps, void* d_codes,
                                                    float* d_scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_pack_ternary: absmean ternary quantizer of a latent weight matrix (section 3.4,
 * "Ternary Weight Quantization (BitLinear)", paper Eq. 2) and 2-bit packing.
 *   alpha = RN32(RN64(sum |w|) / (N K)) with the sum exact over the whole tensor;
 *   code = clamp(rint(RN32(w / RN32(alpha + eps))), -1, 1) (IEEE division per element).
 *   The dequantized weight is alpha * code.
 * Arguments:
 *   d_w          [N, K] float32, row-major, contiguous.
 *   d_packed     output, bitlinear_packed_bytes(N, K) bytes, layout above.
 *   d_alpha      output, one float32 on the device.
 *   d_workspace  scratch of at least bitlinear_pack_workspace_bytes() bytes, 16-byte aligned; its
 *                contents on entry do not matter (the call clears what it uses).
 * bitlinear_packed_bytes returns 0 for N or K <= 0 and SIZE_MAX when N * K is beyond every accepted
 * shape (2^31 elements).
 * ------------------------------------------------------------------------------------------- */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);
size_t bitlinear_pack_workspace_bytes(void);
bl_status bitlinear_pack_ternary(const float* d_w, int64_t N, int64_t K, float eps,
                                 void* d_packed, float* d_alpha,
                                 void* d_workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_pack_ternary_a8: the same ternary quantizer (alpha and codes exactly as
 * bitlinear_pack_ternary) for the weights of the matmuls with INT8 activations (section 3.4,
 * sparsification: the attention output and FFN down projections), in the A8 tile layout: the
 * tiles, lanes and words of the layout above, with weight kk0 + q (q = 0..15) of a word in bits
 * [8 (q % 4) + 2 (q / 4), +2). Expanding such a word to int8 bytes gives the weights in the order
 * of the INT8 codes in memory, so the INT8 matmuls feed the codes to the matrix cores unchanged.
 * bitlinear_gemm_w158a8_sparse and bitlinear_gemv_decode with fmt BL_ACT_INT8 take weights in this
 * layout (and only in it); every other matmul takes the layout of bitlinear_pack_ternary.
 * Arguments, shapes and errors as for bitlinear_pack_ternary.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_pack_ternary_a8(const float* d_w, int64_t N, int64_t K, float eps,
                                    void* d_packed, float* d_alpha,
                                    void* d_workspace, size_t ws_bytes, void* stream);

/* Epilogue of the matmul entry points (a HOST struct; the pointers in it are device pointers).
 *   acc      exact integer sum_k code_x * code_w (FP4: sum of doubled E2M1 codes; counted in halves)
 *   sc[m]    = RN32(scale[m] * alpha)
 *   y0       = RN32(RN32(acc) * sc[m])          (FP4: RN32(RN32(acc * 0.5) * sc[m]))
 *   NONE     y = y0
 *   RESIDUAL y = RN32(y0 + residual[m, n]); d_residual (row stride ldr) may alias y.
 *   RELU2_GLU (section 3.4, squared ReLU gating, paper Eq. 5): the main weights are W_gate,
 *            d_up_packed / d_up_alpha are W_up; g = y0(gate), u = y0(up), g+ = g > 0 ? g : +0,
 *            y = h = RN32(RN32(g+ * g+) * u). If d_row_absmax is non-NULL it receives
 *            max_n |h[m, n]| per row (the call clears it first), which is exactly the gamma of
 *            the following INT8 quantization. (h must stay finite: when g+ * g+ or the product
 *            overflows float32 the row maximum is unspecified.)                                  */
typedef struct {
  int32_t kind;              /* bl_epi_kind */
  const float* d_residual;   /* RESIDUAL */
  int64_t ldr;
  const void* d_up_packed;   /* RELU2_GLU */
  const float* d_up_alpha;
  float* d_row_absmax;       /* RELU2_GLU, optional [M] */
} bl_epilogue;

/* ---------------------------------------------------------------------------------------------
 * bitlinear_gemm_w158a4: Y = Q_4bit(X) Q_w(W)^T (section 3.4, 4-bit activations).
 *   fmt BL_ACT_INT4 runs on int8 matrix cores; BL_ACT_INT4_E3M2 (the same INT4 codes, 6-bit
 *   layout) runs on the block-scaled FP6 x FP4 matrix cores and BL_ACT_FP4_E2M1 on FP4 x FP4 ones,
 *   with unit block scales (the per-token scale is applied in the fp32 epilogue, which keeps the
 *   product exact: every partial sum is an integer, or half-integer for FP4, below 2^24).
 *   d_codes/d_scale  activations from bitlinear_quantize_act, [M, K].
 *   d_packed/d_alpha weights from bitlinear_pack_ternary, [N, K].
 *   d_y              [M, N] float32 output, row stride ldy >= N.
 *   h_epi            NULL or an epilogue description (host pointer).
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_gemm_w158a4(int32_t fmt, const void* d_codes, const float* d_scale,
                                int64_t M, int64_t K,
                                const void* d_packed, const float* d_alpha, int64_t N,
                                float* d_y, int64_t ldy, const bl_epilogue* h_epi, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_gemm_w158a8_sparse: Y = (Q_INT8(X) . M) Q_w(W)^T (section 3.4, sparsification,
 * paper Eq. 1) for the attention output and FFN down projections. Codes are INT8 from
 * bitlinear_quantize_act (masked entries already 0); the weights (and W_up of the RELU2_GLU
 * epilogue) come from bitlinear_pack_ternary_a8. Matrix-core work on 64-wide K slices whose
 * activation codes are all zero for a 16-row group is skipped. Arguments as for the A4 GEMM.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_gemm_w158a8_sparse(const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                       const void* d_packed, const float* d_alpha, int64_t N,
                                       float* d_y, int64_t ldy, const bl_epilogue* h_epi, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_gemv_decode: the same products for decode batches, 1 <= M <= 8, fmt INT4 or INT8.
 * Streams every packed weight tile once from HBM. With INT8 codes a lane skips the load of its
 * 32-wide K slice of a weight tile when the codes of all M rows are zero there. Arguments as for
 * the GEMMs: weights from bitlinear_pack_ternary for fmt BL_ACT_INT4, from
 * bitlinear_pack_ternary_a8 for fmt BL_ACT_INT8.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_gemv_decode(int32_t fmt, const void* d_codes, const float* d_scale,
                                int64_t M, int64_t K,
                                const void* d_packed, const float* d_alpha, int64_t N,
                                float* d_y, int64_t ldy, const bl_epilogue* h_epi, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_pack_ternary_rows: the same ternary quantizer (alpha and codes exactly as
 * bitlinear_pack_ternary) in the row-major 2-bit layout used by the gathered up projection:
 * row n occupies bytes [n K/4, (n+1) K/4); 32-bit word i of the row (little-endian, at byte
 * n K/4 + 4 i) holds weights k0 = 16 i .. 16 i + 15 with weight k0 + q (q < 8) in bits [4q, 4q+2)
 * and weight k0 + 8 + q in bits [4q+2, 4q+4) (the same placement as inside a tile word).
 * Arguments, shapes and errors as for bitlinear_pack_ternary.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_pack_ternary_rows(const float* d_w, int64_t N, int64_t K, float eps,
                                      void* d_packed, float* d_alpha,
                                      void* d_workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_gemv_decode_glu_conditional: the decode FFN gate and up projections with the
 * conditional computation of section 3.4, "Squared ReLU Gating and Conditional Computation in the
 * FFN": the gate projection is computed first, then the up projection only for channels whose
 * gate is positive (relu(g)^2 vanishes elsewhere, so those rows of W_up are never read).
 *   g = y0(gate) as in the epilogue above (INT4 activations, tiled W_gate), written to d_gate;
 *   h[m, n] = RN32(RN32(g * g) * u) where g[m, n] > 0, with u = y0(up) (W_up in the row-major
 *   layout of bitlinear_pack_ternary_rows), and h[m, n] = +0 where g[m, n] <= 0.
 *   (Equal as numbers to the RELU2_GLU epilogue, which yields -0 where g <= 0 and u < 0.)
 *   d_row_absmax, if non-NULL, receives max_n |h[m, n]| per row (cleared first).
 * Arguments: d_codes/d_scale INT4 activations [M, K] (BL_ACT_INT4 layout), 1 <= M <= 8;
 * d_gate [M, N] float32 output (row stride ldg >= N), d_h [M, N] float32 output
 * (row stride ldh >= N, 16-byte aligned, ldh*4 a multiple of 16). Other rules as for the GEMMs.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_gemv_decode_glu_conditional(const void* d_codes, const float* d_scale,
                                                int64_t M, int64_t K,
                                                const void* d_gate_packed, const float* d_gate_alpha,
                                                const void* d_up_rows, const float* d_up_alpha, int64_t N,
                                                float* d_gate, int64_t ldg, float* d_h, int64_t ldh,
                                                float* d_row_absmax, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_kv_quantize: the low-bit KV cache of section 3.4, "Low-Bit KV Cache Quantization"
 * (and the low-bit attention results of Table 3): after rotary position embedding, each
 * (token, head) of Q, K or V is quantized with absmax to unsigned integers, 4 or 3 bits; in a
 * 3-bit cache the heads of beginning-of-sequence (BOS) tokens are also kept at 4 bits.
 *   optional RoPE (d_cos != NULL), rotate-half pairing of element i with i + D/2 (i < D/2):
 *     a' = RN32(RN32(a c) - RN32(b s)),  b' = RN32(RN32(b c) + RN32(a s)),
 *     c = cos[pos[t]][i], s = sin[pos[t]][i]  (caller tables, so any RoPE base or scaling works);
 *   per (t, h): gamma = max_i |x'|, Qp = 2^(bits-1) - 1, s = RN32(Qp / RN32(gamma + eps)),
 *     c_i = RoundClip(RN32(x'_i s), -Qp-1, Qp), stored u_i = c_i + 2^(bits-1) (1 .. 2^bits - 1),
 *     scale[t][h] = RN32(gamma / Qp); the value of a code is (u - 2^(bits-1)) * scale.
 * Arguments:
 *   d_x        [T rows] of H heads x D values (head h at elements [h D, (h+1) D) of a row), bf16
 *              or float32 (in_dtype), row stride ldx >= H D elements; 16-byte aligned, ldx * elem
 *              size a multiple of 16. Typically the K or V columns of the QKV projection output.
 *   D          head size: 64, 128 or 256.  T >= 0, H >= 1; with T == 0 only bits, dtype, H, D
 *              and eps are checked (pointers may be NULL) and nothing is enqueued.
 *   d_pos      [T] int32 positions (required with d_cos); d_cos, d_sin [P][D/2] float32, both or
 *              neither, 16-byte aligned. A position outside [0, P) is out of contract; the kernel
 *              clamps it into that range so it never reads outside the tables.
 *   bits       3 or 4.  eps as for the activation quantizers.
 *   d_codes    out, [T][H][D bits / 8] bytes, 16-byte aligned. 4 bits: code 2j of a head in the
 *              low nibble of its byte j. 3 bits: codes 8g .. 8g+7 in the 24 bits of bytes
 *              3g .. 3g+2 (little-endian), code 8g + q at bits [3q, 3q+3).
 *   d_scale    out, [T][H] float32.
 *   d_bos_slot optional [T] int32 (bits == 3 only): slot >= 0 marks token t as a BOS token whose
 *              4-bit record (the 4-bit layout above) goes to d_bos_codes[slot] ([n_bos_slots][H]
 *              [D/2] bytes, 16-byte aligned) with scales in d_bos_scale[slot][H]; slots outside
 *              [0, n_bos_slots) are skipped. The 3-bit record of a BOS token is written as well.
 * Errors: NULL required pointers, bad dtype or bits, cos without sin or pos, BOS arguments with
 * bits == 4 -> INVALID_ARGUMENT; unsupported D or sizes -> UNSUPPORTED_SHAPE; alignment ->
 * MISALIGNED.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_kv_quantize(const void* d_x, int32_t in_dtype, int64_t T, int64_t H, int64_t D, int64_t ldx,
                                const int32_t* d_pos, const float* d_cos, const float* d_sin, int64_t P,
                                int32_t bits, float eps, void* d_codes, float* d_scale,
                                const int32_t* d_bos_slot, int64_t n_bos_slots, void* d_bos_codes,
                                float* d_bos_scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_calibrate_mfma: a measurement aid, not part of the BitLinear path. Runs a matrix-core-only
 * loop in the shape of the FP6 x FP4 GEMM's K loop (256-thread blocks, two per CU, 32 independent
 * fp32 accumulators per wave, v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales): every block
 * performs iters * 4 waves * 32 MFMAs of 2 * 16 * 16 * 128 ops, i.e. 8388608 * iters ops. The
 * operands have the GEMM's statistics (ternary weights as E2M1 0 / +2 / -2, bell-shaped INT4 codes
 * in E3M2; eight weight and four activation sets alternate), since the sustained matrix-core rate
 * depends on the operand bits. Timing it (HIP events) gives the FP6/FP4 rate this GPU sustains on
 * such data, beside the datasheet peak.
 *   blocks  1 .. 65536 (2 * number of CUs fills the part once);  iters 0 .. 2^20.
 *   d_out   out, blocks * 256 float32: element 256 b holds block b's shader-clock ticks per 100 MHz
 *           real-time tick over its loop (x 0.1 = the clock in GHz); the other elements carry no
 *           meaning.
 * Errors: NULL d_out -> INVALID_ARGUMENT; blocks or iters out of range -> UNSUPPORTED_SHAPE.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_calibrate_mfma(int32_t blocks, int32_t iters, float* d_out, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_gemm_w158a4_kv: the QKV projection of a prefill with the KV-cache quantizer of section 3.4,
 * "Low-Bit KV Cache Quantization" (Table 3), fused into its epilogue: Y = Q_4bit(X) Q_w(W_qkv)^T as
 * bitlinear_gemm_w158a4 computes it (fmt BL_ACT_INT4_E3M2 or BL_ACT_FP4_E2M1), and from each row's
 * fp32 values, exactly as bitlinear_kv_quantize computes them from that fp32 output:
 *   columns [p H 128, (p+1) H 128) are part p = Q, K, V (head size D = 128, N = 3 H 128);
 *   RoPE (when d_cos is given) on Q and K, never on V; per (token, head) absmax codes of bits[p]
 *   bits in the KV record layout above (d_codes[p] [M][H][16 bits[p]] bytes, d_scale[p] [M][H]);
 *   with d_bos_slot, parts with 3 bits also get the 4-bit records of BOS tokens in
 *   d_bos_codes[p] [n_bos_slots][H][64] and d_bos_scale[p] [n_bos_slots][H] (the other parts' BOS
 *   pointers are ignored). The outputs equal bitlinear_gemm_w158a4 followed by three
 *   bitlinear_kv_quantize calls on the Q, K and V columns of Y, bit for bit.
 *   d_y        NULL: the fp32 projection is not stored (its 4 M N bytes never reach memory); else Y as
 *              bitlinear_gemm_w158a4 writes it (row stride ldy).
 * Errors: as for bitlinear_gemm_w158a4 and bitlinear_kv_quantize; N != 3 H 128 -> UNSUPPORTED_SHAPE;
 * other formats -> INVALID_ARGUMENT.
 * ------------------------------------------------------------------------------------------- */
typedef struct {
  int64_t H;                 /* heads per part */
  float eps;
  int32_t bits[3];           /* Q, K, V: 3 or 4 */
  void* d_codes[3];
  float* d_scale[3];
  const int32_t* d_pos;      /* [M] positions (with d_cos) */
  const float* d_cos;        /* [P][64] (or NULL: no RoPE) */
  const float* d_sin;
  int64_t P;
  const int32_t* d_bos_slot; /* optional [M]: slot >= 0 marks a BOS token */
  int64_t n_bos_slots;
  void* d_bos_codes[3];
  float* d_bos_scale[3];
} bl_kv_epilogue;
bl_status bitlinear_gemm_w158a4_kv(int32_t fmt, const void* d_codes, const float* d_scale, int64_t M, int64_t K,
                                   const void* d_packed, const float* d_alpha, int64_t N, float* d_y, int64_t ldy,
                                   const bl_kv_epilogue* h_kv, void* stream);

/* ---------------------------------------------------------------------------------------------
 * bitlinear_calibrate_read: a measurement aid, not part of the BitLinear path. A plain streaming read
 * of `bytes` bytes at d_src (16 bytes per lane, one load per lane), the ceiling for a kernel that
 * reads the same bytes once per launch, e.g. a decode GEMV streaming one packed weight matrix.
 *   bytes   a multiple of 16, 16 .. 2^31 - 16.   d_src 16-byte aligned.
 *   d_sink  one uint32 the kernel may write (its value carries no meaning).
 * Errors: NULL pointers -> INVALID_ARGUMENT; bytes out of range -> UNSUPPORTED_SHAPE; alignment -> MISALIGNED.
 * ------------------------------------------------------------------------------------------- */
bl_status bitlinear_calibrate_read(const void* d_src, int64_t bytes, uint32_t* d_sink, void* stream);

const char* bitlinear_status_string(int32_t status);
int32_t bitlinear_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
