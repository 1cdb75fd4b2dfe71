/*
 * oracle.c - plain, slow, obviously-correct CPU reference for the
 * scaled-quantization and block-scaled-GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, __graft_entry__.smoke() and
 * the cpu_baseline leg of bench.py load this library.  The GPU library never
 * links, loads or calls it, and the two share no source, header or table.
 *
 * Sources (cited by page title and section):
 *   [FP8 guide]  "Infraestrutura de Treinamento FP8: Precisao Numerica de
 *                Proxima Geracao" (Introl blog; the Indonesian copy
 *                "Infrastruktur Pelatihan FP8" carries the same content).
 *   [MoE FP4]    "Practical FP4 Training for Large-Scale MoE Models on Hopper
 *                GPUs" (summary of arXiv 2603.02731), "Resumo tecnico".
 *
 * Arithmetic.  Every element value and every power-of-two scale is a short
 * dyadic rational, so it is held exactly in double.  Steps that are defined
 * as binary32 operations (the per-tensor scale, its reciprocal, and the
 * scaled product x*scale) are done in float with IEEE round-to-nearest-even.
 * Build: gcc -O2 -ffp-contract=off, no fast-math, so neither contraction nor
 * flush-to-zero can change a rounding.
 *
 * Where the pages leave a rule open, the reading taken is stated at the
 * function that applies it.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define OR_E4M3 0
#define OR_E5M2 1
#define OR_E2M1 2

#define OR_SRC_F32 0
#define OR_SRC_BF16 1
#define OR_SRC_F64 2 /* MX quantizer input only */

#define OR_SCALE_TENSOR 0 /* one float scale_inv for the whole operand */
#define OR_SCALE_BLK32 1  /* one E8M0 byte per 32 elements along K     */
#define OR_SCALE_BLK128 2 /* one E8M0 byte per 128 elements along K    */

/* ------------------------------------------------------------------------ */
/* O1. Decoding of the element and scale encodings.                         */
/* ------------------------------------------------------------------------ */

/* E4M3: [FP8 guide], "O panorama da precisao numerica": 4 exponent bits,
 * 3 mantissa bits, finite range up to +-448.  Reading: the OCP variant whose
 * largest finite value is 448 (exponent bias 7, no infinities, the single
 * all-ones pattern S.1111.111 is NaN).                                      */
static double e4m3_value(unsigned c)
{
    unsigned s = (c >> 7) & 1u, E = (c >> 3) & 15u, M = c & 7u;
    double mag;
    if (E == 15 && M == 7)
        return s ? -NAN : NAN;
    if (E == 0)
        mag = ldexp((double)M / 8.0, 1 - 7); /* subnormal: 0.M x 2^(1-bias) */
    else
        mag = ldexp(1.0 + (double)M / 8.0, (int)E - 7);
    return s ? -mag : mag;
}

/* E5M2: [FP8 guide], same section: 5 exponent bits, 2 mantissa bits, wider
 * range.  Reading: IEEE-style, bias 15, E=31 holds +-Inf (M=0) and NaN.     */
static double e5m2_value(unsigned c)
{
    unsigned s = (c >> 7) & 1u, E = (c >> 2) & 31u, M = c & 3u;
    double mag;
    if (E == 31)
        mag = (M == 0) ? INFINITY : NAN;
    else if (E == 0)
        mag = ldexp((double)M / 4.0, 1 - 15);
    else
        mag = ldexp(1.0 + (double)M / 4.0, (int)E - 15);
    return s ? -mag : mag;
}

/* E2M1 (the MXFP4 element): [MoE FP4], "Metodologia": MXFP4 shares one
 * power-of-two scale across 32 elements.  Element encoding: sign bit 3,
 * exponent bits 2..1 with bias 1, one mantissa bit, no Inf or NaN.         */
static double e2m1_value(unsigned c)
{
    unsigned s = (c >> 3) & 1u, E = (c >> 1) & 3u, M = c & 1u;
    double mag;
    if (E == 0)
        mag = ldexp((double)M / 2.0, 1 - 1);
    else
        mag = ldexp(1.0 + (double)M / 2.0, (int)E - 1);
    return s ? -mag : mag;
}

double or_value(int fmt, unsigned code)
{
    switch (fmt) {
    case OR_E4M3: return e4m3_value(code & 0xFFu);
    case OR_E5M2: return e5m2_value(code & 0xFFu);
    case OR_E2M1: return e2m1_value(code & 0xFu);
    }
    return NAN;
}

/* E8M0 scale byte: the power of two 2^(b-127); 0xFF is NaN.               */
double or_e8m0_value(unsigned b)
{
    b &= 0xFFu;
    if (b == 0xFFu)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------------------------ */
/* O2. Saturating round-to-nearest-even cast.                               */
/* ------------------------------------------------------------------------ */

/* The non-negative finite values of a format, sorted by value, each with its
 * code.  Built once by decoding every code with sign 0.                      */
typedef struct {
    int n;
    double v[128];
    unsigned code[128];
} or_table;

static or_table g_tab[3];
static int g_tab_ready = 0;

static int cmp_entry_by_value(const void* a, const void* b)
{
    const double* x = (const double*)a;
    const double* y = (const double*)b;
    return (*x > *y) - (*x < *y);
}

static void build_tables(void)
{
    for (int f = 0; f < 3; ++f) {
        int ncodes = (f == OR_E2M1) ? 8 : 128; /* sign bit clear */
        struct { double v; unsigned c; } tmp[128];
        int n = 0;
        for (int c = 0; c < ncodes; ++c) {
            double v = or_value(f, (unsigned)c);
            if (isfinite(v)) {
                tmp[n].v = v;
                tmp[n].c = (unsigned)c;
                ++n;
            }
        }
        qsort(tmp, (size_t)n, sizeof(tmp[0]), cmp_entry_by_value);
        g_tab[f].n = n;
        for (int i = 0; i < n; ++i) {
            g_tab[f].v[i] = tmp[i].v;
            g_tab[f].code[i] = tmp[i].c;
        }
    }
    g_tab_ready = 1;
}

/* Built when the library is loaded, before any OpenMP region can race. */
__attribute__((constructor)) static void init_tables(void) { build_tables(); }

static const or_table* table(int fmt)
{
    if (!g_tab_ready)
        build_tables();
    return &g_tab[fmt];
}

double or_max_finite(int fmt)
{
    const or_table* t = table(fmt);
    return t->v[t->n - 1];
}

/* cast_F(v).  BASELINE reading of "saturating round-to-nearest-even":
 *  - NaN -> the NaN code with the input's sign (0x7F / 0xFF in both FP8
 *    formats; E2M1 has no NaN, so the MX quantizer never calls this with NaN);
 *  - |v| >= largest finite value (Inf included) -> +-largest finite;
 *  - otherwise the nearer of the two neighbouring finite values, an exact tie
 *    going to the code whose mantissa LSB is 0;
 *  - a zero result keeps the input's sign.
 * Deliberately a value-table search, not bit manipulation.                 */
unsigned or_cast(int fmt, double v)
{
    const or_table* t = table(fmt);
    unsigned sign_bit = (fmt == OR_E2M1) ? 0x8u : 0x80u;
    unsigned s = signbit(v) ? sign_bit : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (fmt == OR_E2M1) ? 0x7u : (s | 0x7Fu);
    if (a >= t->v[t->n - 1])
        return s | t->code[t->n - 1];
    /* largest i with v[i] <= a; v[0] = 0 <= a always */
    int lo = 0, hi = t->n - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (t->v[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    /* now v[lo] <= a < v[hi] */
    double dlo = a - t->v[lo], dhi = t->v[hi] - a;
    unsigned pick;
    if (dlo < dhi)
        pick = t->code[lo];
    else if (dhi < dlo)
        pick = t->code[hi];
    else
        pick = (t->code[lo] & 1u) == 0 ? t->code[lo] : t->code[hi];
    return s | pick;
}

/* cast_F over an array (convenience for the tests). */
void or_cast_array(int fmt, const double* v, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = (uint8_t)or_cast(fmt, v[i]);
}

/* ------------------------------------------------------------------------ */
/* Input access.                                                            */
/* ------------------------------------------------------------------------ */

static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float load_f(const void* x, int src, int64_t i)
{
    if (src == OR_SRC_BF16)
        return bf16_to_float(((const uint16_t*)x)[i]);
    return ((const float*)x)[i];
}

/* The MX quantizer also takes binary64 input (OR_SRC_F64), for values the
 * oracle computes in double precision (the SwiGLU activation).            */
static double load_d(const void* x, int src, int64_t i)
{
    if (src == OR_SRC_F64)
        return ((const double*)x)[i];
    return (double)load_f(x, src, i);
}

/* ------------------------------------------------------------------------ */
/* O3. amax = max |x|.  [FP8 guide], "Transformer Engine: a fundacao de     */
/* software": the recipe reduces absolute values with "max".  Reading: a NaN */
/* anywhere makes the amax NaN.                                              */
/* ------------------------------------------------------------------------ */
float or_amax(const void* x, int src, int64_t rows, int64_t cols, int64_t ld)
{
    int any_nan = 0;
    float m = 0.0f;
#pragma omp parallel for reduction(max : m) reduction(| : any_nan) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            float v = fabsf(load_f(x, src, r * ld + c));
            if (isnan(v))
                any_nan = 1;
            else if (v > m)
                m = v;
        }
    }
    return any_nan ? NAN : m;
}

/* ------------------------------------------------------------------------ */
/* O4. Per-tensor scale.                                                    */
/* ------------------------------------------------------------------------ */

/* scale = F_max / amax in binary32 ([FP8 guide], "Estrategias de
 * escalonamento e estabilidade": one factor per tensor from its statistics).
 * Readings: amax 0 or non-finite -> 1.0; a quotient that overflows binary32
 * -> FLT_MAX.  F_max is the format's largest finite value.                 */
float or_scale_from_amax(int fmt, float amax)
{
    float fmax = (float)or_max_finite(fmt);
    if (!(amax > 0.0f) || !isfinite(amax))
        return 1.0f;
    float s = fmax / amax;
    if (isinf(s))
        return FLT_MAX;
    return s;
}

/* Delayed scaling, [FP8 guide], "Transformer Engine": the recipe keeps the
 * amaxes of the previous 16 iterations, reduces them with max, margin 0, and
 * the scale for this step comes from that history instead of the current
 * tensor.  Reading: history[0] is the most recent step, history[len-1] the
 * oldest; the current step is excluded; a fresh history is all zeros (so the
 * first step uses scale 1.0); max propagates NaN.  margin = 0 makes the
 * division by 2^margin exact, so it is omitted.                            */
float or_history_amax(const float* history, int len)
{
    float m = 0.0f;
    for (int i = 0; i < len; ++i) {
        if (isnan(history[i]))
            return NAN;
        if (history[i] > m)
            m = history[i];
    }
    return m;
}

/* Push this step's amax: shift every entry one slot older, drop the oldest. */
void or_history_push(float* history, int len, float amax)
{
    for (int i = len - 1; i >= 1; --i)
        history[i] = history[i - 1];
    if (len > 0)
        history[0] = amax;
}

/* ------------------------------------------------------------------------ */
/* O5. Per-tensor quantize: q = cast_F(fl32(x * scale)), two roundings.     */
/* Optional second output: the byte transpose [cols, rows].                 */
/* ------------------------------------------------------------------------ */
void or_quantize_per_tensor(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int fmt,
                            float* history, int hist_len, float* amax_out, float* scale_out,
                            float* scale_inv_out, uint8_t* q_row, uint8_t* q_col)
{
    float amax = or_amax(x, src, rows, cols, ld);
    float amax_ref = hist_len > 0 ? or_history_amax(history, hist_len) : amax;
    float scale = or_scale_from_amax(fmt, amax_ref);
    float scale_inv = 1.0f / scale;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            float y = load_f(x, src, r * ld + c) * scale; /* binary32 product */
            uint8_t q = (uint8_t)or_cast(fmt, (double)y);
            if (q_row)
                q_row[r * cols + c] = q;
            if (q_col)
                q_col[c * rows + r] = q;
        }
    }
    if (hist_len > 0)
        or_history_push(history, hist_len, amax);
    if (amax_out)
        *amax_out = amax;
    if (scale_out)
        *scale_out = scale;
    if (scale_inv_out)
        *scale_inv_out = scale_inv;
}

/* ------------------------------------------------------------------------ */
/* O6. MX block-32 quantize.                                                */
/* ------------------------------------------------------------------------ */

/* emax_F: the exponent of the largest power of two the format represents
 * (E4M3 448 = 1.75*2^8 -> 8; E5M2 57344 = 1.75*2^15 -> 15; E2M1 6 = 1.5*2^2
 * -> 2).  Derived from the decode table, not typed in.                    */
int or_emax(int fmt)
{
    int ex;
    frexp(or_max_finite(fmt), &ex); /* max = m*2^ex, m in [0.5,1) */
    return ex - 1;
}

/* One block of 32 values v[0..31] (exact doubles).  Writes 32 codes and
 * returns the E8M0 byte.
 * [MoE FP4], "Metodologia": MXFP4 blocks are 32 elements with power-of-two
 * scales; [FP8 guide], "Estrategias de escalonamento": MXFP8 gives each block
 * its own factor.  Scale exponent (closed form): e = floor(log2(amax_b)) -
 * emax_F, clamped to [-127, 127]; byte = e + 127; q_i = cast_F(v_i * 2^-e)
 * (exact product).  Readings: a block holding NaN or Inf gets byte 0xFF with
 * codes 0x7F (FP8) or 0x0 (E2M1); an all-zero block gets e = -127 (byte 0)
 * and signed-zero codes.                                                    */
static unsigned quantize_block32(int fmt, const double* v, unsigned* codes)
{
    double amax = 0.0;
    int bad = 0;
    for (int i = 0; i < 32; ++i) {
        double a = fabs(v[i]);
        if (!isfinite(a))
            bad = 1;
        else if (a > amax)
            amax = a;
    }
    if (bad) {
        for (int i = 0; i < 32; ++i)
            codes[i] = (fmt == OR_E2M1) ? 0x0u : 0x7Fu;
        return 0xFFu;
    }
    int e;
    if (amax == 0.0) {
        e = -127;
    } else {
        int ex;
        frexp(amax, &ex); /* amax = m*2^ex, m in [0.5,1): floor(log2) = ex-1 */
        e = (ex - 1) - or_emax(fmt);
        if (e < -127)
            e = -127;
        if (e > 127)
            e = 127;
    }
    for (int i = 0; i < 32; ++i)
        codes[i] = or_cast(fmt, ldexp(v[i], -e));
    return (unsigned)(e + 127);
}

/* Rowwise: blocks along each row (the contiguous dimension); codes
 * [rows, cols] (E2M1: [rows, cols/2], element 2j in the low nibble) and
 * scales [rows, cols/32].  Colwise: blocks along each column, written
 * transposed: codes [cols, rows], scales [cols, rows/32].  Either output may
 * be NULL.  Requires cols % 32 == 0 for rowwise, rows % 32 == 0 for colwise.
 * Reading (nibble order, layouts): element 2j in the low nibble; scales
 * row-major, one byte each.                                                */
void or_quantize_mx(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int fmt,
                    uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col)
{
    if (q_row) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            double v[32];
            unsigned codes[32];
            for (int64_t b = 0; b < cols / 32; ++b) {
                for (int i = 0; i < 32; ++i)
                    v[i] = load_d(x, src, r * ld + b * 32 + i);
                unsigned sb = quantize_block32(fmt, v, codes);
                s_row[r * (cols / 32) + b] = (uint8_t)sb;
                for (int i = 0; i < 32; ++i) {
                    int64_t c = b * 32 + i;
                    if (fmt == OR_E2M1) {
                        uint8_t* p = &q_row[r * (cols / 2) + c / 2];
                        if ((c & 1) == 0)
                            *p = (uint8_t)(codes[i] & 0xFu);
                        else
                            *p = (uint8_t)(*p | ((codes[i] & 0xFu) << 4));
                    } else {
                        q_row[r * cols + c] = (uint8_t)codes[i];
                    }
                }
            }
        }
    }
    if (q_col) {
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < cols; ++c) {
            double v[32];
            unsigned codes[32];
            for (int64_t b = 0; b < rows / 32; ++b) {
                for (int i = 0; i < 32; ++i)
                    v[i] = load_d(x, src, (b * 32 + i) * ld + c);
                unsigned sb = quantize_block32(fmt, v, codes);
                s_col[c * (rows / 32) + b] = (uint8_t)sb;
                for (int i = 0; i < 32; ++i) {
                    int64_t r = b * 32 + i;
                    if (fmt == OR_E2M1) {
                        uint8_t* p = &q_col[c * (rows / 2) + r / 2];
                        if ((r & 1) == 0)
                            *p = (uint8_t)(codes[i] & 0xFu);
                        else
                            *p = (uint8_t)(*p | ((codes[i] & 0xFu) << 4));
                    } else {
                        q_col[c * rows + r] = (uint8_t)codes[i];
                    }
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O7. Direct FP4 -> FP8 repack.                                            */
/* [MoE FP4], "Metodologia", direct conversion algorithm: the FP8 side uses  */
/* blocks of 128 elements, so each FP8 block scale is the largest of the     */
/* four MXFP4 block scales it covers, and every element's exponent is        */
/* shifted by the difference so the represented value is preserved; the      */
/* conversion skips any BF16 intermediate.  [MoE FP4], "Kernels CUDA         */
/* Otimizados": the row-layout variant feeds the GEMM.                       */
/* Readings: the FP8 element format is E4M3; the FP8 scale is exactly        */
/* max(s4) (no headroom shift); when the shift takes a value below E4M3's    */
/* range it rounds to nearest even (exact for shifts >= -8); a group whose    */
/* largest byte is 0xFF (NaN) becomes byte 0xFF with all codes 0x7F.         */
/* With a gather, output row r reads source row idx[r]; an index outside     */
/* [0, src_rows) yields a NaN group (byte 0xFF, codes 0x7F).                 */
/* ------------------------------------------------------------------------ */
void or_repack_fp4_to_fp8(const uint8_t* q4, const uint8_t* s4, const int32_t* idx, int64_t src_rows,
                          int64_t rows, int64_t cols, uint8_t* q8, uint8_t* s8)
{
    int64_t nb32 = cols / 32, ng = cols / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t sr = idx ? (int64_t)idx[r] : r;
        int valid = (sr >= 0 && sr < src_rows);
        for (int64_t g = 0; g < ng; ++g) {
            unsigned smax = 0xFFu;
            if (valid) {
                smax = 0;
                for (int b = 0; b < 4; ++b) {
                    unsigned sb = s4[sr * nb32 + g * 4 + b];
                    if (sb > smax)
                        smax = sb;
                }
            }
            s8[r * ng + g] = (uint8_t)smax;
            for (int64_t k = 0; k < 128; ++k) {
                int64_t c = g * 128 + k;
                uint8_t out;
                if (smax == 0xFFu) {
                    out = 0x7F;
                } else {
                    unsigned sb = s4[sr * nb32 + c / 32];
                    uint8_t byte = q4[sr * (cols / 2) + c / 2];
                    unsigned code = (c & 1) ? (byte >> 4) : (byte & 0xFu);
                    double v = ldexp(or_value(OR_E2M1, code), (int)sb - (int)smax);
                    out = (uint8_t)or_cast(OR_E4M3, v);
                }
                q8[r * cols + c] = out;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O7b. FP4 row -> FP8 col: dequantize, transpose, requantize.              */
/* [MoE FP4], "Metodologia", "Kernels CUDA Otimizados": besides the row-    */
/* layout conversion, one kernel fuses the FP4 dequantization, the matrix   */
/* transpose and the FP8 requantization, so that activations cached in      */
/* MXFP4 (row blocks along the hidden dimension) feed the weight-gradient   */
/* GEMM, whose contraction runs over the tokens.                             */
/* Readings: the dequantization is exact (E2M1 value times 2^(s-127), a     */
/* double); the requantization is MX block-32 E4M3 along the new rows (the  */
/* old columns, 32 tokens per block) by quantize_block32's rule; a source   */
/* block with scale byte 0xFF dequantizes to NaN, so every output block it  */
/* reaches is a NaN block.  In: q4 [rows, cols/2], s4 [rows, cols/32].      */
/* Out: q8 [cols, rows], s8 [cols, rows/32]; rows % 32 == 0, cols % 32 == 0. */
/* ------------------------------------------------------------------------ */
void or_fp4_row_to_fp8_col(const uint8_t* q4, const uint8_t* s4, int64_t rows, int64_t cols, uint8_t* q8,
                           uint8_t* s8)
{
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        double v[32];
        unsigned codes[32];
        for (int64_t b = 0; b < rows / 32; ++b) {
            for (int i = 0; i < 32; ++i) {
                int64_t r = b * 32 + i;
                uint8_t byte = q4[r * (cols / 2) + c / 2];
                unsigned code = (c & 1) ? (byte >> 4) : (byte & 0xFu);
                v[i] = or_value(OR_E2M1, code) * or_e8m0_value(s4[r * (cols / 32) + c / 32]);
            }
            s8[c * (rows / 32) + b] = (uint8_t)quantize_block32(OR_E4M3, v, codes);
            for (int i = 0; i < 32; ++i)
                q8[c * rows + b * 32 + i] = (uint8_t)codes[i];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* O8. Dequantization of one operand element.                               */
/* Element k of row i of an operand stored [rows, K] (E2M1: [rows, K/2]),    */
/* with its scale: per-tensor (a float scale_inv), or one E8M0 byte per 32   */
/* or per 128 elements along K.                                              */
/* ------------------------------------------------------------------------ */
static double deq(const uint8_t* q, int fmt, const void* s, int mode, int64_t K, int64_t i, int64_t k)
{
    unsigned code;
    if (fmt == OR_E2M1) {
        uint8_t byte = q[i * (K / 2) + k / 2];
        code = (k & 1) ? (byte >> 4) : (byte & 0xFu);
    } else {
        code = q[i * K + k];
    }
    double v = or_value(fmt, code);
    double sc;
    if (mode == OR_SCALE_TENSOR)
        sc = (double)((const float*)s)[0];
    else if (mode == OR_SCALE_BLK32)
        sc = or_e8m0_value(((const uint8_t*)s)[i * (K / 32) + k / 32]);
    else
        sc = or_e8m0_value(((const uint8_t*)s)[i * (K / 128) + k / 128]);
    return v * sc;
}

double or_dequant(const uint8_t* q, int fmt, const void* s, int mode, int64_t K, int64_t i, int64_t k)
{
    return deq(q, fmt, s, mode, K, i, k);
}

/* ------------------------------------------------------------------------ */
/* O9. Scaled GEMM: C[m,n] = sum_k deq(A)[m,k] * deq(B)[n,k], A [M,K] and    */
/* B [N,K] both K-contiguous; products and sums in double.                   */
/* [MoE FP4], "Metodologia": the heavy matrix products stay in FP8 on the    */
/* matrix units; [FP8 guide], "MXFP8 e NVFP4": block-scaled FP8 products.    */
/* Computes the listed entries (m_idx[t], n_idx[t]) and, for the tolerance,  */
/* sum_k |deq(A)[m,k]| * |deq(B)[n,k]|.  Either output array may be NULL.    */
/* ------------------------------------------------------------------------ */
void or_gemm_entries(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
                     const void* sB, int mb, int64_t K, const int64_t* m_idx, const int64_t* n_idx,
                     int64_t count, double* c_out, double* abs_out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        double acc = 0.0, aacc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = deq(A, fa, sA, ma, K, m_idx[t], k);
            double b = deq(B, fb, sB, mb, K, n_idx[t], k);
            acc += a * b;
            aacc += fabs(a) * fabs(b);
        }
        if (c_out)
            c_out[t] = acc;
        if (abs_out)
            abs_out[t] = aacc;
    }
}

/* Whole C [M,N] row-major (small shapes only). */
void or_gemm(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
             const void* sB, int mb, int64_t M, int64_t N, int64_t K, double* C, double* Cabs)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = deq(A, fa, sA, ma, K, m, k);
                double b = deq(B, fb, sB, mb, K, n, k);
                acc += a * b;
                aacc += fabs(a) * fabs(b);
            }
            C[m * N + n] = acc;
            if (Cabs)
                Cabs[m * N + n] = aacc;
        }
    }
}

/* Grouped (ragged) GEMM: rows off[g]..off[g+1]-1 of A multiply expert g's
 * B_g [N, K] (B stored [G, N, K]; block scales [G, N, K/32]).  [MoE FP4],
 * "Kernels CUDA Otimizados": ragged per-expert token counts.  Computes the
 * listed (row, n) entries; the group of a row is found from the offsets.   */
void or_grouped_gemm_entries(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B,
                             int fb, const void* sB, int mb, const int64_t* off, int64_t G, int64_t N,
                             int64_t K, const int64_t* m_idx, const int64_t* n_idx, int64_t count,
                             double* c_out, double* abs_out)
{
    int64_t b_elems_bytes = (fb == OR_E2M1) ? N * K / 2 : N * K;
    int64_t b_scale_bytes = (mb == OR_SCALE_BLK32) ? N * (K / 32) : (mb == OR_SCALE_BLK128) ? N * (K / 128) : 0;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        int64_t m = m_idx[t];
        int64_t g = 0;
        while (g < G && !(m >= off[g] && m < off[g + 1]))
            ++g;
        double acc = 0.0, aacc = 0.0;
        if (g < G) {
            const uint8_t* Bg = B + g * b_elems_bytes;
            const void* sBg = (mb == OR_SCALE_TENSOR) ? sB : (const void*)((const uint8_t*)sB + g * b_scale_bytes);
            for (int64_t k = 0; k < K; ++k) {
                double a = deq(A, fa, sA, ma, K, m, k);
                double b = deq(Bg, fb, sBg, mb, K, n_idx[t], k);
                acc += a * b;
                aacc += fabs(a) * fabs(b);
            }
        } else {
            acc = NAN; /* row outside every group: not defined */
        }
        if (c_out)
            c_out[t] = acc;
        if (abs_out)
            abs_out[t] = aacc;
    }
}

/* Threads the OpenMP loops above use (for reporting the oracle's timing). */
int or_num_threads(void) { return omp_get_max_threads(); }
