/*
 * mxq.h - C ABI of the MI355X (gfx950) scaled-quantization and block-scaled
 * GEMM library libmxq.so.
 *
 * The library implements the data-parallel hot path of the FP8 / MXFP4
 * low-precision training recipes described by two pages:
 *   [FP8 guide] "Infraestrutura de Treinamento FP8: Precisao Numerica de
 *               Proxima Geracao" (Introl; also published in Indonesian as
 *               "Infrastruktur Pelatihan FP8");
 *   [MoE FP4]   "Practical FP4 Training for Large-Scale MoE Models on Hopper
 *               GPUs" (summary of arXiv 2603.02731), "Resumo tecnico".
 *
 * Conventions shared by every entry point
 *  - Pointers to tensors are DEVICE pointers owned by the caller.  The
 *    library never allocates or frees memory, never synchronises the stream
 *    and never reads device data on the host.  Outputs are fully overwritten.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All work is enqueued asynchronously on it.
 *  - Every call validates its arguments on the host BEFORE touching HIP and
 *    returns an mxq_status.  Device faults surface at the caller's next
 *    synchronisation.  A zero-size problem (no rows, or no columns) returns
 *    MXQ_OK with no launch once its formats and shape rules pass; its data
 *    pointers are then not checked and may be NULL (an empty tensor's).
 *  - All tensors are row-major.  16-byte alignment is required of every
 *    tensor base pointer and of every row pitch in bytes.
 *  - The library holds no state; calls are reentrant.  Calls that write the
 *    same buffers must be ordered by the caller.
 *
 * Encodings
 *  - E4M3: 4 exponent bits (bias 7), 3 mantissa bits, largest finite +-448,
 *    no Inf, S.1111.111 is NaN ([FP8 guide], "O panorama da precisao
 *    numerica").  E5M2: 5 exponent bits (bias 15), 2 mantissa bits, largest
 *    finite +-57344, with Inf and NaN (same section).
 *  - E2M1 (MXFP4 element): sign in bit 3, 2 exponent bits (bias 1), 1
 *    mantissa bit: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.  Two codes per byte,
 *    element 2j in the low nibble.
 *  - E8M0 scale byte b: the power of two 2^(b-127); 0xFF is NaN.
 *  - Casts are saturating round-to-nearest-even: NaN -> 0x7F|sign (FP8),
 *    |v| >= largest finite (Inf included) -> +-largest finite, exact ties go
 *    to the even mantissa, a zero result keeps the input's sign.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXQ_ABI_VERSION 1

/* element formats */
enum { MXQ_E4M3 = 0, MXQ_E5M2 = 1, MXQ_E2M1 = 2 };
/* input element types of the quantizers */
enum { MXQ_SRC_F32 = 0, MXQ_SRC_BF16 = 1 };
/* how an operand of the GEMM is scaled */
enum {
    MXQ_SCALE_TENSOR = 0, /* const float* scale_inv: one factor for the whole operand */
    MXQ_SCALE_BLK32 = 1,  /* const uint8_t* E8M0 [rows, K/32]: one byte per 32 along K */
    MXQ_SCALE_BLK128 = 2  /* const uint8_t* E8M0 [rows, K/128]: one byte per 128 along K */
};
/* GEMM output element type */
enum { MXQ_OUT_F32 = 0, MXQ_OUT_BF16 = 1 };
/* OR into `out` of the GEMMs: exact products, fp32 accumulation (see
 * mxq_scaled_gemm). */
enum { MXQ_OUT_PRECISE = 16 };
/* return codes */
enum {
    MXQ_OK = 0,
    MXQ_ERR_NULL = -1,   /* a required pointer is NULL */
    MXQ_ERR_SHAPE = -2,  /* a size is negative, or violates a divisibility rule */
    MXQ_ERR_ALIGN = -3,  /* a pointer or row pitch is not 16-byte aligned */
    MXQ_ERR_FORMAT = -4, /* unsupported format / scale mode / source combination */
    MXQ_ERR_HIP = -5     /* the HIP runtime reported an error at launch */
};

/*
 * mxq_quantize_per_tensor - amax reduction, per-tensor scale and saturating
 * RNE cast to E4M3 or E5M2, with an optional transposed second output.
 *
 * Defines: [FP8 guide], "Estrategias de escalonamento e estabilidade"
 * (per-tensor scaling: one factor from the tensor's statistics; delayed
 * scaling: the factor comes from earlier iterations' statistics) and
 * "Transformer Engine: a fundacao de software" (recipe: margin 0, amax
 * history of 16, reduced with max; HYBRID = E4M3 forward, E5M2 backward).
 *
 *  x          [rows, cols] input, row pitch ld_x elements (src: F32 or BF16)
 *  fmt        MXQ_E4M3 or MXQ_E5M2
 *  amax_history, history_len
 *             history_len == 0: current scaling, amax_ref = amax(x).
 *             history_len in 1..1024: delayed scaling. amax_history is a
 *             device float[history_len]; entry 0 is the most recent step.
 *             amax_ref = max(history) (NaN propagates); after the cast the
 *             history shifts one slot older and amax(x) enters at entry 0.
 *             A fresh history is all zeros (first step uses scale 1).
 *  amax_out   device float[1]: amax(x) = max |x| (NaN if x holds a NaN).
 *             Also used as the reduction accumulator (overwritten first).
 *  scale_out  device float[1]: scale = fl32(F_max / amax_ref), F_max = 448
 *             or 57344; 1.0 if amax_ref is 0, Inf or NaN; FLT_MAX if the
 *             quotient overflows.  Required.
 *  scale_inv_out device float[1]: fl32(1 / scale) (the dequant factor the
 *             GEMM takes as MXQ_SCALE_TENSOR).  May be NULL.
 *  q_row      [rows, cols] codes q = cast(fl32(x * scale)), or NULL
 *  q_col      [cols, rows] the same codes transposed, or NULL
 * Rules: cols % 16 == 0; if q_col != NULL, rows % 16 == 0; at least one of
 * q_row, q_col non-NULL; ld_x >= cols.  Enqueues three kernels.
 */
int mxq_quantize_per_tensor(const void* x, int src, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                            float* amax_history, int history_len, float* amax_out, float* scale_out,
                            float* scale_inv_out, uint8_t* q_row, uint8_t* q_col, void* stream);

/*
 * mxq_quantize_mx - MX block-32 quantization with E8M0 scales.
 *
 * Defines: [MoE FP4], "Metodologia" (MXFP4: 32-element blocks sharing a
 * power-of-two scale; the BF16->FP4 row quantizer of the forward pass) and
 * [FP8 guide], "Estrategias de escalonamento" / "MXFP8 e NVFP4" (block-level
 * scale factors for FP8).
 * Per block of 32: amax_b = max |x_i|; e = clamp(floor(log2 amax_b) - emax,
 * -127, 127) with emax = 8 (E4M3), 15 (E5M2), 2 (E2M1); scale byte e + 127;
 * q_i = cast(x_i * 2^-e).  An all-zero block gets byte 0x00 and signed-zero
 * codes; a block holding NaN or Inf gets byte 0xFF and codes 0x7F (FP8) or
 * 0x0 (E2M1).
 *
 *  x      [rows, cols], pitch ld_x elements, src F32 or BF16
 *  q_row  rowwise codes (blocks along the contiguous dimension):
 *         [rows, cols] bytes (E2M1: [rows, cols/2]), or NULL
 *  s_row  [rows, cols/32] scale bytes (required with q_row)
 *  q_col  colwise codes (blocks along rows), stored transposed:
 *         [cols, rows] bytes, or NULL.  Not available for E2M1.
 *  s_col  [cols, rows/32] (required with q_col)
 * Rules: cols % 32 == 0; with q_col also rows % 32 == 0 and fmt != E2M1.
 */
int mxq_quantize_mx(const void* x, int src, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                    uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, void* stream);

/*
 * mxq_repack_fp4_to_fp8 - direct MXFP4 -> FP8 (E4M3, block-128 E8M0) repack
 * in the integer domain, with an optional row gather.
 *
 * Defines: [MoE FP4], "Metodologia", direct conversion algorithm (the FP8
 * block of 128 takes the largest of its four FP4 block scales; each
 * element's exponent is adjusted by the difference; no BF16 intermediate) and
 * "Kernels CUDA Otimizados" (the row-layout FP4->FP8 kernel that feeds the
 * GEMM; ragged per-expert rows).
 *  q4, s4     source MXFP4 codes [src_rows, cols/2] and E8M0 [src_rows, cols/32]
 *  gather_idx device int32[rows] (output row r reads source row idx[r]) or
 *             NULL (then rows <= src_rows and row r reads row r).  An index
 *             outside [0, src_rows) yields a NaN group: byte 0xFF, codes 0x7F.
 *  q8, s8     outputs: E4M3 [rows, cols] and E8M0 [rows, cols/128].
 * Per group: s8 = max of the four s4 (0xFF propagates -> all codes 0x7F);
 * q8 = cast_E4M3(v(q4) * 2^(s4 - s8)), exact when s4 - s8 >= -8.
 * Rules: cols % 128 == 0.
 */
int mxq_repack_fp4_to_fp8(const uint8_t* q4, const uint8_t* s4, const int32_t* gather_idx, int64_t src_rows,
                          int64_t rows, int64_t cols, uint8_t* q8, uint8_t* s8, void* stream);

/*
 * mxq_fp4_row_to_fp8_col - MXFP4 rows -> transposed MX E4M3 (block 32 along
 * the new rows), fused: exact dequantization, transpose, requantization.
 *
 * Defines: [MoE FP4], "Metodologia", "Kernels CUDA Otimizados" (besides the
 * row-layout conversion, a kernel fuses FP4 dequantization, the matrix
 * transpose and FP8 requantization, so that MXFP4-cached activations feed
 * the weight-gradient GEMM, which contracts over the tokens).
 *  q4, s4  source MXFP4 codes [rows, cols/2] (element 2j in the low nibble)
 *          and E8M0 scales [rows, cols/32]; 0xFF (NaN) makes every output
 *          block that holds one of its elements a NaN block.
 *  q8, s8  outputs: E4M3 codes [cols, rows] and E8M0 [cols, rows/32].
 * Each output block of 32 source rows: e = floor(log2 amax) - 8 clamped to
 * [-127, 127] over the exact values v = E2M1(code) * 2^(s-127) (all zero:
 * e = -127); codes = saturating RNE E4M3 of v / 2^e; a NaN block gets byte
 * 0xFF and codes 0x7F.
 * Rules: rows % 32 == 0, cols % 32 == 0; q4 and q8 16-byte aligned (s4 and
 * s8 any alignment); at most 2^31 - 1 tiles of 128 rows x 256 columns.  The
 * call writes every byte of q8 and s8 and reads nothing else.
 */
int mxq_fp4_row_to_fp8_col(const uint8_t* q4, const uint8_t* s4, int64_t rows, int64_t cols, uint8_t* q8,
                           uint8_t* s8, void* stream);

/*
 * mxq_swiglu_quantize_mx - the expert MLP's activation between its two
 * grouped GEMMs: h = silu(gate) * up, then MX block-32 quantization of h
 * along the intermediate dimension, the A operand of the down-projection.
 *
 * Defines: [MoE FP4], "Metodologia" (the expert GEMMs run in FP8, so the
 * activation between them is requantized to FP8) and "Kernels CUDA
 * Otimizados" (ragged per-expert rows: the call is row-wise, rows of every
 * expert alike).  The pages do not name the activation; this library reads
 * it as SwiGLU, silu(x) = x / (1 + e^-x), with the gate and up projections
 * side by side in the up-projection's output.
 *  gu     [rows, ld] elements, src F32 or BF16: gate in columns [0, inter),
 *         up in [inter, 2 inter)
 *  q      [rows, inter] FP8 codes (fmt E4M3 or E5M2), dense
 *  s      [rows, inter/32] E8M0 scale bytes
 * h is formed in binary32 (exp and reciprocal each within a few ulps), so a
 * code may differ from one computed on the exact h where h lies within a
 * few binary32 ulps of a rounding boundary; blocks follow mxq_quantize_mx
 * (NaN or Inf in h: byte 0xFF, codes 0x7F).
 * Rules: inter % 32 == 0, ld >= 2 inter; gu and the row pitch 16-byte
 * aligned; q 16-byte aligned.  The call writes every byte of q and s.
 */
int mxq_swiglu_quantize_mx(const void* gu, int src, int64_t rows, int64_t inter, int64_t ld, int fmt, uint8_t* q,
                           uint8_t* s, void* stream);

/*
 * mxq_scaled_gemm - C = dequant(A) . dequant(B)^T with fp32 accumulation on
 * gfx950's block-scaled MFMA.
 *
 * Defines: [MoE FP4], "Metodologia" (the heavy matrix products stay in FP8
 * on the matrix units) and [FP8 guide], "Requisitos de hardware" / "MXFP8 e
 * NVFP4" (FP8 matrix products; hardware block-scaled FP8).
 *  A   [M, K] codes (E2M1: [M, K/2]), K contiguous; fa its format
 *  sA  ma == MXQ_SCALE_TENSOR: const float* (device, 1 value: scale_inv);
 *      MXQ_SCALE_BLK32: E8M0 [M, K/32]; MXQ_SCALE_BLK128: E8M0 [M, K/128]
 *  B   [N, K] codes (E2M1: [N, K/2]), K contiguous; fb, sB, mb likewise
 *  C   [M, N] with row pitch ldc elements; out = MXQ_OUT_F32 or MXQ_OUT_BF16
 *      (bf16: round-to-nearest-even of the fp32 result).  Write-only.
 *      OR MXQ_OUT_PRECISE into `out` for exact products: by default FP8 x FP8
 *      runs on the block-scaled FP8 MFMA, which keeps each aligned run of 8
 *      products to 13 fractional bits below the run's largest; with the flag,
 *      operands are converted to bf16 with their scales folded in (exact while
 *      every dequantized operand is below 2^128 in magnitude; values below
 *      2^-133 become zero) and the bf16 MFMA sums exact products in fp32.
 *      E2M1 x E2M1 is exact either way; the flag with one E2M1 operand and
 *      one FP8 operand is MXQ_ERR_FORMAT.
 * C[m,n] = sum_k deq(A)[m,k] * deq(B)[n,k]; per-tensor factors multiply the
 * fp32 result in the epilogue.  Any mix of E4M3/E5M2/E2M1 operands and scale
 * modes is accepted.
 * Rules: K % 128 == 0 (a multiple of the K step); M, N >= 0; ldc >= N with
 * 16-byte aligned row pitch; A, B and each block-scale array below 4 GiB
 * (else MXQ_ERR_SHAPE).  Scale arrays are read in aligned 4-byte words: a
 * BLK128 array of rows * K/128 bytes that is not a multiple of 4 has the rest
 * of its last word read too (same word, so same page); those bytes are unused.
 */
int mxq_scaled_gemm(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
                    const void* sB, int mb, int64_t M, int64_t N, int64_t K, void* C, int out, int64_t ldc,
                    void* stream);

/*
 * mxq_grouped_scaled_gemm - ragged grouped GEMM: for every group g, rows
 * off[g] .. off[g+1]-1 of A multiply group g's B_g.
 *
 * Defines: [MoE FP4], "Metodologia" and "Kernels CUDA Otimizados" (expert
 * GEMMs in FP8 over ragged per-expert token counts).
 *  A          [total_rows, K] codes with scales as in mxq_scaled_gemm
 *  B          [G, N, K] codes; sB [G, N, K/32] (or [G, N, K/128]) bytes, or
 *             one float for MXQ_SCALE_TENSOR (shared by all groups)
 *  group_off  DEVICE int64[G+1], non-decreasing, off[0] = 0,
 *             off[G] <= total_rows.  Empty groups are allowed.  Rows at or
 *             past off[G] are not written.  Offsets are read on the device
 *             only (no host synchronisation), so they cannot be rejected:
 *             the kernel clamps each to [0, total_rows] (and each group's
 *             end to at least its start).  Offsets that break the rules
 *             give unspecified values in C but never an access outside A,
 *             the scales or C.
 *  C          [total_rows, N] contiguous, fp32 or bf16
 * Rules: as mxq_scaled_gemm (the 4 GiB limit applies to A and to each
 * group's B); G <= 4096.  Rows beyond total_rows are never read, whatever
 * the offsets say.
 */
int mxq_grouped_scaled_gemm(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
                            const void* sB, int mb, const int64_t* group_off, int64_t G, int64_t total_rows,
                            int64_t N, int64_t K, void* C, int out, void* stream);

/*
 * mxq_grouped_gemm_swiglu_quantize_mx - the expert MLP's up-projection with
 * its activation fused into the GEMM's epilogue: for every group g and every
 * row m of it, the gate and up projections gate = deq(A_m) . deq(B_g[c])^T
 * and up = deq(A_m) . deq(B_g[inter + c])^T (fp32 accumulation as
 * mxq_grouped_scaled_gemm, block-scaled FP8 MFMA), h = silu(gate) * up with
 * silu(x) = x / (1 + e^-x) formed in binary32, and h MX block-32 quantized
 * along the intermediate dimension as mxq_swiglu_quantize_mx does.  The
 * gate/up output never reaches memory.
 *
 * Defines: [MoE FP4], "Metodologia" (the expert GEMMs run in FP8 on ragged
 * per-expert rows; the activation between the two expert GEMMs is
 * requantized to FP8 for the down-projection) and "Kernels CUDA Otimizados"
 * (ragged per-expert token counts).  The pages do not name the activation;
 * this library reads it as SwiGLU (see mxq_swiglu_quantize_mx).
 *  A, sA, ma  [total_rows, K] FP8 codes (E4M3 or E5M2) with scales as in
 *             mxq_scaled_gemm (per-tensor, BLK32 or BLK128)
 *  B, sB, mb  [G, 2 inter, K] FP8 codes: rows 0 .. inter-1 of each group are
 *             the gate projection's weights, rows inter .. 2 inter - 1 the up
 *             projection's (the layout of the plain grouped GEMM's B for
 *             N = 2 inter); scales [G, 2 inter, K/32] or [G, 2 inter, K/128],
 *             or one float for MXQ_SCALE_TENSOR
 *  group_off  DEVICE int64[G+1], as mxq_grouped_scaled_gemm (clamped to
 *             [0, total_rows] on the device)
 *  hfmt       MXQ_E4M3 or MXQ_E5M2: the format of h
 *  q_out      [total_rows, inter] codes of h (16-byte aligned); rows outside
 *             every group are not written
 *  s_out      [total_rows, inter/32] E8M0 scale bytes of h
 * h comes from the fp32 accumulators, so a code may differ from one computed
 * on the exact sums where h lies within the GEMM's rounding of a rounding
 * boundary (see mxq_scaled_gemm for what the FP8 MFMA rounds).
 * Rules: inter % 128 == 0, K % 128 == 0; A and each group's B below 4 GiB;
 * G <= 4096; FP8 operands only (E2M1 -> MXQ_ERR_FORMAT).
 */
int mxq_grouped_gemm_swiglu_quantize_mx(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
                                        const void* sB, int mb, const int64_t* group_off, int64_t G,
                                        int64_t total_rows, int64_t inter, int64_t K, int hfmt, uint8_t* q_out,
                                        uint8_t* s_out, void* stream);

/* Human-readable text of a status code (static storage). */
const char* mxq_status_string(int status);

/* MXQ_ABI_VERSION of the loaded library. */
int mxq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
