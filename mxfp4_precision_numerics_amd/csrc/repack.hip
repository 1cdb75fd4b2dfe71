// repack.hip - direct MXFP4 -> FP8 (E4M3, block-128) repack in the integer
// domain, with optional row gather.
//
// MoE FP4 page, "Metodologia", direct conversion algorithm: an FP8 block of
// 128 elements covers four MXFP4 blocks of 32; its power-of-two scale is the
// largest of the four, and each element's exponent is lowered by the gap
// between its own block scale and that maximum, so no BF16 intermediate is
// formed.  "Kernels CUDA Otimizados": the row-layout FP4->FP8 kernel that
// feeds the GEMM, over ragged per-expert rows.
//
// Design: a lane owns one 32-element block: it reads the block's 16 bytes of
// FP4 codes and the group's 4 scale bytes and writes 32 bytes of E4M3 codes.
// Four consecutive lanes make one 128-element group, so that a wave moves
// whole 128-byte lines.  Because every element of a 32-block sees the same
// exponent shift d = s4 - s8 <= 0, the lane first builds the 8-entry table
// T[m] = E4M3(|E2M1 m| * 2^d) and then maps nibbles to bytes with v_perm_b32
// lookups; the sign bit moves from bit 3 to bit 7.  Each thread handles
// RP_PER_THREAD blocks, all loads issued before the first conversion (a row
// index outside the source reads nothing).
#include "common.h"
#include "launch.h"

namespace mxq {

constexpr int RP_THREADS = 256;
constexpr int RP_PER_THREAD = 1;  // more waves in flight hide the index -> data latency chain best

// E4M3 codes of 8 E2M1 codes (one dword, element 0 in the low nibble) through
// the table (tlo: entries 0..3, thi: 4..7); two dwords of 4 codes each.
__device__ __forceinline__ uint2 fp4x8_to_e4m3(uint32_t w, uint32_t tlo, uint32_t thi) {
    const uint32_t lo = w & 0x0F0F0F0Fu;          // nibbles 0,2,4,6
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // nibbles 1,3,5,7
    const uint32_t n01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // elements 0..3
    const uint32_t n23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // elements 4..7
    return make_uint2(__builtin_amdgcn_perm(thi, tlo, n01 & 0x07070707u) | ((n01 & 0x08080808u) << 4),
                      __builtin_amdgcn_perm(thi, tlo, n23 & 0x07070707u) | ((n23 & 0x08080808u) << 4));
}

__global__ void __launch_bounds__(RP_THREADS) k_repack(const uint8_t* __restrict__ q4, const uint8_t* __restrict__ s4,
                                                       const int32_t* __restrict__ idx, int64_t src_rows, int64_t rows,
                                                       int64_t gpr, uint8_t* __restrict__ q8, uint8_t* __restrict__ s8) {
    const int64_t nblk = rows * gpr * 4;  // 32-element blocks of the output
    const int64_t base = (int64_t)blockIdx.x * (RP_THREADS * RP_PER_THREAD) + threadIdx.x;
    uint32_t sw[RP_PER_THREAD];
    uint4 c4[RP_PER_THREAD];
#pragma unroll
    for (int i = 0; i < RP_PER_THREAD; ++i) {
        const int64_t b = base + (int64_t)i * RP_THREADS;
        const int64_t bc = b < nblk ? b : 0;
        const int64_t r = bc / (gpr * 4), g = (bc >> 2) - r * gpr;
        const int64_t sr = idx ? (int64_t)idx[r] : r;
        const bool valid = b < nblk && sr >= 0 && sr < src_rows;
        sw[i] = 0xFFFFFFFFu;  // an invalid row repacks as NaN
        c4[i] = make_uint4(0u, 0u, 0u, 0u);
        if (valid) {
            sw[i] = ld_nt4(s4 + sr * (gpr * 4) + g * 4);
            c4[i] = ld_nt16(q4 + sr * (gpr * 64) + g * 64 + (b & 3) * 16);
        }
    }
#pragma unroll
    for (int i = 0; i < RP_PER_THREAD; ++i) {
        const int64_t b = base + (int64_t)i * RP_THREADS;
        if (b >= nblk) continue;
        const uint32_t w = sw[i];
        const uint32_t b0 = w & 0xFFu, b1 = (w >> 8) & 0xFFu, b2 = (w >> 16) & 0xFFu, b3 = w >> 24;
        uint32_t smax = b0 > b1 ? b0 : b1;
        smax = smax > b2 ? smax : b2;
        smax = smax > b3 ? smax : b3;
        uint4 o0, o1;
        if (smax == 0xFFu) {
            o0 = o1 = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
        } else {
            const uint32_t sb = (w >> (8 * (b & 3))) & 0xFFu;  // this block's scale
            const int d = (int)sb - (int)smax;                 // in [-254, 0]
            // T[m] for m = 0..7: E4M3 code of |E2M1 m| * 2^d.  The product is an
            // exact binary32 for d >= -126; below that every entry rounds to 0.
            uint32_t tlo = 0, thi = 0;
            if (d >= -126) {
                const float p = exp2i(d);
                tlo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(0.0f, 0.5f * p, 0, false) & 0xFFFFu;
                tlo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(1.0f * p, 1.5f * p, (int)tlo, true);
                thi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(2.0f * p, 3.0f * p, 0, false) & 0xFFFFu;
                thi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(4.0f * p, 6.0f * p, (int)thi, true);
            }
            const uint2 e0 = fp4x8_to_e4m3(c4[i].x, tlo, thi), e1 = fp4x8_to_e4m3(c4[i].y, tlo, thi);
            const uint2 e2 = fp4x8_to_e4m3(c4[i].z, tlo, thi), e3 = fp4x8_to_e4m3(c4[i].w, tlo, thi);
            o0 = make_uint4(e0.x, e0.y, e1.x, e1.y);
            o1 = make_uint4(e2.x, e2.y, e3.x, e3.y);
        }
        uint8_t* const dst = q8 + b * 32;  // output rows are dense: block b starts at byte 32 b
        st_nt16(dst, o0);
        st_nt16(dst + 16, o1);
        if ((b & 3) == 0) s8[b >> 2] = (uint8_t)smax;
    }
}

hipError_t launch_repack_fp4_to_fp8(const uint8_t* q4, const uint8_t* s4, const int32_t* idx, int64_t src_rows,
                                    int64_t rows, int64_t cols, uint8_t* q8, uint8_t* s8, hipStream_t st) {
    const int64_t gpr = cols / 128;
    const int64_t nblk = rows * gpr * 4;
    const int64_t per_block = RP_THREADS * RP_PER_THREAD;
    const unsigned grid = (unsigned)((nblk + per_block - 1) / per_block);
    hipLaunchKernelGGL(k_repack, dim3(grid), dim3(RP_THREADS), 0, st, q4, s4, idx, src_rows, rows, gpr, q8, s8);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP4 row -> FP8 col.  MoE FP4 page, "Metodologia", "Kernels CUDA
// Otimizados": one kernel dequantizes cached MXFP4 activations, transposes
// them and requantizes them to FP8, so that the weight-gradient GEMM (which
// contracts over the tokens) reads FP8 blocks along the tokens.  Reading:
// exact dequantization, then MX block-32 E4M3 along the new rows.
//
// One block of 256 threads per tile of 128 source rows (tokens) x 256 source
// columns.  Row phase: the tile's codes reach LDS as 16-byte chunks (whole
// 128-byte lines per 8 lanes) and its scale bytes as a [block][row] array.
// Column phase: lane l of wave w owns tokens 16*(l/8) .. +15 of the 8 columns
// 8*(8w + l%8) .. +7, so every output row gets one 16-byte store per lane and
// 8 lanes write a whole 128-byte line; a 32-token output block spans a lane
// and its partner 8 lanes away (one DPP row rotation).
//
// Two conversion paths, chosen per tile (block-uniform):
//  * converter path, when every scale byte of the tile lies in [12, 254]:
//    gfx950's scaled FP4 converters yield each element divided by 4, exactly
//    (m * 2^(s-129) is a normal number for these bytes).  A first pass
//    converts to bfloat16 and takes the block's largest magnitude as an
//    integer max of the bit patterns; its exponent gives the E8M0 byte
//    e + 127.  A second pass converts to binary32, and the scaled binary32 ->
//    E4M3 converter divides by 2^(e-2) and rounds to nearest even in one
//    step.  The smallest non-zero value, 2^-118 after the division, keeps
//    e >= -124, so 2^(e-2) is a normal binary32 and the converter's scale
//    (its exponent field) holds it.  Converting twice keeps the live values
//    few (66 VGPRs, seven blocks per CU).
//  * integer path otherwise (tiny or NaN scale bytes), one column at a time
//    from LDS: each element's floor(log2 |v|) + 129 is L(m) + s, the block
//    exponent is an integer max, and every element is 2|m| * 2^(s - 128 - e)
//    formed with ldexp and cast by the unscaled converter; a NaN source scale
//    makes the whole output block NaN (codes 0x7F, scale byte 0xFF).
// In both, the block exponent puts the largest magnitude at 256 or 384, so
// nothing saturates, and an all-zero block gets byte 0x00.  The output scale
// bytes gather in LDS as [column][block] and leave as one 4-byte store per
// column (the tile's 4 blocks) where alignment allows, bytes otherwise.
// LDS rows hold 32 dwords; the dword index is XOR-ed with 8 * ((row / 16) % 4)
// so that the column phase's reads (rows 16 apart) spread over the banks.
// ---------------------------------------------------------------------------
// The codes leave through plain (cached) stores: each 16-byte store is part
// of a 128-byte line that 8 lanes complete, and these merge in L2 better
// than streaming stores do (measured 7% faster here).
__device__ __forceinline__ void st_line16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
typedef float v2f __attribute__((ext_vector_type(2)));
constexpr int FC_ROWS = 128, FC_COLS = 256;
constexpr uint32_t FC_FAST_MIN = 12;  // smallest scale byte of the converter path

__device__ __forceinline__ int fc_swz(int r) { return ((r >> 4) & 3) << 3; }

// Scale byte k of w as a binary32 whose exponent field holds it (the other
// bits zero): the scale operand of the scaled converters.
__device__ __forceinline__ float fc_scale_field(uint32_t w, int k) {
    const int sh = 23 - 8 * k;
    const uint32_t v = sh >= 0 ? (w << sh) : (w >> -sh);
    return as_float(v & 0x7F800000u);
}

// Converter path, source columns 2C and 2C+1 of the lane's group (byte C of
// each code dword).  y = element / 4 (exact).  Pass 1 takes the block's
// largest magnitudes from bfloat16 conversions (exact too: bfloat16 has the
// binary32 exponent range), compared as integers; pass 2 converts again to
// binary32 and casts 4 tokens at a time, so few values are live at once.
template <int C>
__device__ __forceinline__ void fc_fast_pair(const uint32_t (&dd)[16], const float (&sf)[16], bool live, bool pair_lo,
                                             uint8_t* qcol, uint8_t* sbuf, int64_t rows) {
    uint32_t mx = 0;  // |bf16| of columns 2C (low half) and 2C+1 (high half), max over tokens
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dd[i], sf[i], C);
        mx = pk_max_u16(mx, __builtin_bit_cast(uint32_t, b) & 0x7FFF7FFFu);
    }
    // the partner lane (8 lanes away, the same DPP row of 16) holds the other 16 tokens of the block
    mx = pk_max_u16(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x128, 0xF, 0xF, false));
    // biased exponents of max|y|: e = eb - 133 (y is a quarter of the value);
    // the codes are y / 2^(e-2), whose exponent field is eb - 8 (>= 1 unless
    // the block is all zero, where any scale gives the zero codes)
    const int ebe = (int)((mx >> 7) & 0xFFu), ebo = (int)(mx >> 23);
    const float sce = as_float((uint32_t)max(ebe - 8, 1) << 23), sco = as_float((uint32_t)max(ebo - 8, 1) << 23);
    uint32_t oe[4], oo[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        v2f y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(dd[4 * p + q], sf[4 * p + q], C);
        v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, y[0][0], y[1][0], sce, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, y[2][0], y[3][0], sce, true);
        oe[p] = __builtin_bit_cast(uint32_t, r);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, y[0][1], y[1][1], sco, false);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, y[2][1], y[3][1], sco, true);
        oo[p] = __builtin_bit_cast(uint32_t, r);
    }
    if (live) {
        st_line16(qcol + (2 * C) * rows, make_uint4(oe[0], oe[1], oe[2], oe[3]));
        st_line16(qcol + (2 * C + 1) * rows, make_uint4(oo[0], oo[1], oo[2], oo[3]));
    }
    if (pair_lo) {
        sbuf[(2 * C) * 4] = (uint8_t)max(ebe - 6, 0);
        sbuf[(2 * C + 1) * 4] = (uint8_t)max(ebo - 6, 0);
    }
}

// Integer path (any scale bytes), one source column at a time; the codes are
// read from LDS again for each column, so that this rare path holds few
// registers.
__device__ __forceinline__ void fc_exact(const uint32_t* codes, int tg, int cg, const uint4 sv, bool live,
                                         bool pair_lo, uint8_t* qcol, uint8_t* sbuf, int64_t rows) {
    const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
        auto code = [&](int i) __attribute__((always_inline)) {
            const int r = 16 * tg + i;
            return codes[r * 32 + (cg ^ fc_swz(r))] >> (4 * j);
        };
        int em = 0;
        uint32_t bad = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int k = (int)code(i) & 7;
            const int s = (int)(sw[i >> 2] >> (8 * (i & 3))) & 0xFF;
            const int l = k < 2 ? k : (k >> 1) + 1;  // floor(log2 2|m|) + 1, 0 for a zero
            em = max(em, k ? l + s : 0);
            bad |= s == 0xFF;
        }
        em = max(em, __builtin_amdgcn_update_dpp(0, em, 0x128, 0xF, 0xF, false));
        bad |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bad, 0x128, 0xF, 0xF, false);
        // floor(log2 amax) - 8 (E4M3 emax), clamped below at -127 (also the
        // all-zero block); it never exceeds 121
        const int e = max(em - 137, -127);
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float y[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = 4 * p + q;
                const uint32_t n = code(i);
                const int k = (int)n & 7;
                const int s = (int)(sw[i >> 2] >> (8 * (i & 3))) & 0xFF;
                const int two_m = k < 2 ? k : (2 + (k & 1)) << ((k >> 1) - 1);
                // |v| / 2^e = 2|m| * 2^(s - 128 - e): exact wherever it can reach
                // E4M3's range, and at most 384
                const float v = __builtin_amdgcn_ldexpf((float)two_m, s - 128 - e);
                y[q] = as_float(as_uint(v) | ((n & 8u) << 28));
            }
            uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)r, true);
            o[p] = bad ? 0x7F7F7F7Fu : r;
        }
        if (live) st_line16(qcol + j * rows, make_uint4(o[0], o[1], o[2], o[3]));
        if (pair_lo) sbuf[j * 4] = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
    }
}

__global__ void __launch_bounds__(256) k_fp4_row_to_fp8_col(const uint8_t* __restrict__ q4,
                                                            const uint8_t* __restrict__ s4, int64_t rows,
                                                            int64_t cols, int64_t ntc, uint8_t* __restrict__ q8,
                                                            uint8_t* __restrict__ s8) {
    __shared__ __attribute__((aligned(16))) uint32_t codes[FC_ROWS * 32];
    __shared__ __attribute__((aligned(16))) uint8_t scales[8 * FC_ROWS];  // [block][row]
    __shared__ __attribute__((aligned(16))) uint8_t sout[FC_COLS * 4];    // output scale bytes [column][block]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t tr = ((int64_t)blockIdx.x / ntc) * FC_ROWS, tc = ((int64_t)blockIdx.x % ntc) * FC_COLS;
    // row phase: codes (zeros outside the tensor)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int id = it * 256 + tid, r = id >> 3, q = id & 7;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tr + r < rows && tc + 32 * q < cols) v = ld_nt16(q4 + (tr + r) * (cols / 2) + tc / 2 + 16 * q);
        *reinterpret_cast<uint4*>(&codes[r * 32 + ((4 * q) ^ fc_swz(r))]) = v;
    }
    // scales: thread -> row tid/2, blocks 4*(tid&1) .. +3; outside the tensor
    // the byte 127 stands in (its codes are zero, so it changes nothing)
    bool exact = false;
    {
        const int r = tid >> 1, b0 = 4 * (tid & 1);
        uint32_t sw = 0x7F7F7F7Fu;
        if (tr + r < rows) {
            const uint8_t* p = s4 + (tr + r) * (cols / 32) + tc / 32 + b0;
            if ((cols & 127) == 0 && (reinterpret_cast<uintptr_t>(s4) & 3) == 0) {
                // 4-byte aligned, and the 4 blocks are all inside or all outside
                if (tc + 32 * b0 < cols) sw = ld_nt4(p);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (tc + 32 * (b0 + k) < cols) sw = (sw & ~(0xFFu << (8 * k))) | ((uint32_t)p[k] << (8 * k));
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t b = (sw >> (8 * k)) & 0xFFu;
            exact |= b < FC_FAST_MIN || b == 0xFFu;
            scales[(b0 + k) * FC_ROWS + r] = (uint8_t)b;
        }
    }
    exact = __syncthreads_or(exact);
    // column phase
    const int tg = lane >> 3, cg = 8 * w + (lane & 7);
    const int64_t c0 = tc + 8 * cg, r0 = tr + 16 * tg;
    const bool live = r0 < rows && c0 < cols, pair_lo = (tg & 1) == 0;
    const uint4 sv = *reinterpret_cast<const uint4*>(&scales[(cg >> 2) * FC_ROWS + 16 * tg]);
    uint8_t* const qcol = q8 + c0 * rows + r0;          // output row c0 + j starts at + j * rows
    uint8_t* const sbuf = sout + 8 * cg * 4 + (tg >> 1);  // column 8 cg + j at + 4 j
    if (!exact) {
        uint32_t dd[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 16 * tg + i;
            dd[i] = codes[r * 32 + (cg ^ fc_swz(r))];
        }
        // 2^(s - 129) per token: exponent field s - 2 (no byte borrows: s >= 12)
        const uint32_t sm[4] = {sv.x - 0x02020202u, sv.y - 0x02020202u, sv.z - 0x02020202u, sv.w - 0x02020202u};
        float sf[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) sf[i] = fc_scale_field(sm[i >> 2], i & 3);
        fc_fast_pair<0>(dd, sf, live, pair_lo, qcol, sbuf, rows);
        fc_fast_pair<1>(dd, sf, live, pair_lo, qcol, sbuf, rows);
        fc_fast_pair<2>(dd, sf, live, pair_lo, qcol, sbuf, rows);
        fc_fast_pair<3>(dd, sf, live, pair_lo, qcol, sbuf, rows);
    } else {
        fc_exact(codes, tg, cg, sv, live, pair_lo, qcol, sbuf, rows);
    }
    // output scale bytes: thread -> column tc + tid, the tile's (up to) 4 blocks
    __syncthreads();
    const int64_t col = tc + tid;
    if (col < cols) {
        const int nb = (int)min((rows - tr) / 32, (int64_t)4);
        uint8_t* const dst = s8 + col * (rows / 32) + tr / 32;
        const uint32_t v = *reinterpret_cast<const uint32_t*>(&sout[4 * tid]);
        if (nb == 4 && ((rows / 32) & 3) == 0 && (reinterpret_cast<uintptr_t>(s8) & 3) == 0) {
            *reinterpret_cast<uint32_t*>(dst) = v;
        } else {
            for (int b = 0; b < nb; ++b) dst[b] = (uint8_t)(v >> (8 * b));
        }
    }
}

hipError_t launch_fp4_row_to_fp8_col(const uint8_t* q4, const uint8_t* s4, int64_t rows, int64_t cols, uint8_t* q8,
                                     uint8_t* s8, hipStream_t st) {
    const int64_t ntc = (cols + FC_COLS - 1) / FC_COLS, ntiles = ntc * ((rows + FC_ROWS - 1) / FC_ROWS);
    hipLaunchKernelGGL(k_fp4_row_to_fp8_col, dim3((unsigned)ntiles), dim3(256), 0, st, q4, s4, rows, cols, ntc, q8,
                       s8);
    return hipGetLastError();
}

}  // namespace mxq
