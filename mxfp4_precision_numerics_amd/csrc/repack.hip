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
// A persistent block of 256 threads walks tiles of 128 source rows x 256
// source columns with the grid's stride; the next tile's loads are in flight
// while the current one is converted from LDS.
//  Row phase: wave w, step it reads source row 16*it + 4*w + l/16, 16 lanes
//  per row, 16 codes (8 bytes) per lane: whole 128-byte lines.  Codes go to
//  LDS as they are (4 bits each); the row's 8 scale bytes too.
//  Column phase (twice, for columns 0..127 and 128..255 of the tile): lane l
//  of wave w takes source rows 8*(l/4) .. +7 and columns 8*(4w + l%4) .. +7,
//  i.e. 8 output rows of 8 tokens; the 16 lanes of a column cover its 128
//  tokens and write a whole line.  An output block (32 tokens) spans the 4
//  lanes that differ in lane bits 2-3.
// Each element is m * 2^(s-127) with m an E2M1 value; its exponent is that of
// m plus s - 127, so the block exponent is an integer max and every element
// divided by the block scale is m * 2^(s-127-e), formed with ldexp from a
// byte table of 2|m| (exact where it can reach E4M3's range) and rounded to
// nearest even by the converter.  The block exponent puts the largest
// magnitude at 256 or 384, so nothing saturates.
// LDS rows hold 32 dwords of codes; dword index bits 2-4 are XOR-ed with the
// row's bits 3-5, which halves the column reads' bank conflicts to 2-way.
// ---------------------------------------------------------------------------
constexpr int FC_ROWS = 128, FC_COLS = 256;
// Persistent blocks, each walking tiles with the grid's stride: three per CU
// of 256, the most the kernel's register use (about 155 VGPRs, three waves
// per SIMD) keeps resident; two per CU were 4% slower, four (with spills to
// fit) 40% slower.
constexpr int FC_GRID = 768;

__device__ __forceinline__ int fc_swz(int r, int dw) { return dw ^ (((r >> 3) & 7) << 2); }

__global__ void __launch_bounds__(256) k_fp4_row_to_fp8_col(const uint8_t* __restrict__ q4,
                                                            const uint8_t* __restrict__ s4, int64_t rows,
                                                            int64_t cols, int64_t ntc, int64_t ntiles,
                                                            uint8_t* __restrict__ q8, uint8_t* __restrict__ s8) {
    __shared__ __attribute__((aligned(16))) uint32_t codes[FC_ROWS * 32];
    __shared__ uint8_t scales[FC_ROWS * 8];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane & 15;
    // the row phase's loads of tile t (zeros outside the tensor)
    uint2 c[8];
    uint32_t sb[8];
    auto load_tile = [&](int64_t t) __attribute__((always_inline)) {
        const int64_t tr = (t / ntc) * FC_ROWS, tc = (t % ntc) * FC_COLS;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 16 * it + 4 * w + (lane >> 4);
            const bool rok = tr + r < rows;
            c[it] = make_uint2(0u, 0u);
            sb[it] = 0;
            if (rok && tc + 16 * ch < cols) c[it] = ld_nt8(q4 + (tr + r) * (cols / 2) + tc / 2 + 8 * ch);
            if (rok && ch < 8 && tc + 32 * ch < cols) sb[it] = s4[(tr + r) * (cols / 32) + tc / 32 + ch];
        }
    };
    int64_t t = blockIdx.x;
    if (t < ntiles) load_tile(t);
    for (; t < ntiles; t += gridDim.x) {
        const int64_t tr = (t / ntc) * FC_ROWS, tc = (t % ntc) * FC_COLS;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 16 * it + 4 * w + (lane >> 4);
            *reinterpret_cast<uint2*>(&codes[r * 32 + fc_swz(r, 2 * ch)]) = c[it];
            if (ch < 8) scales[r * 8 + ch] = (uint8_t)sb[it];
        }
        __syncthreads();
        // the next tile's loads are in flight during this tile's column phase
        if (t + gridDim.x < ntiles) load_tile(t + gridDim.x);
        const int g = lane >> 2;
        // byte tables indexed by an E2M1 magnitude code k (0..7), entries 0..3 in
        // the low word: 2|m| (0, 1, 2, 3, 4, 6, 8, 12) and floor(log2 2|m|) + 1
        // (0 for zero)
        constexpr uint32_t V_LO = 0x03020100u, V_HI = 0x0C080604u;
        constexpr uint32_t L_LO = 0x02020100u, L_HI = 0x04040303u;
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            const int cg = 16 * h + 4 * w + (lane & 3);  // 8-column group of the tile, 0..31
            // Per source row i (one token): 2|m| of columns 0,2,4,6 (vl) and
            // 1,3,5,7 (vh) as bytes, their sign bits (bit 3 of each byte), and
            // s - 128.  An element's floor(log2 |v|) + 129 is L(k) + s for k != 0,
            // so the block exponent per column is a max over rows of L + s,
            // kept on 16-bit lanes: m0 = columns (0, 4), m1 = (2, 6), m2 = (1, 5),
            // m3 = (3, 7); 0 means no non-zero element.
            uint32_t vl[8], vh[8], sl[8], sh[8];
            int a[8];
            uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
            bool bad = false;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * g + i;
                const uint32_t dd = codes[r * 32 + fc_swz(r, cg)];
                const uint32_t sc = scales[r * 8 + (cg >> 2)];
                bad |= sc == 0xFFu;
                const uint32_t klo = dd & 0x07070707u, khi = (dd >> 4) & 0x07070707u;
                sl[i] = dd & 0x08080808u;
                sh[i] = (dd >> 4) & 0x08080808u;
                vl[i] = __builtin_amdgcn_perm(V_HI, V_LO, klo);
                vh[i] = __builtin_amdgcn_perm(V_HI, V_LO, khi);
                const uint32_t ll = __builtin_amdgcn_perm(L_HI, L_LO, klo), lh = __builtin_amdgcn_perm(L_HI, L_LO, khi);
                const uint32_t s2 = sc * 0x00010001u;
                m0 = pk_max_u16(m0, pk_lsum_u16(ll & 0x00FF00FFu, s2));
                m1 = pk_max_u16(m1, pk_lsum_u16((ll >> 8) & 0x00FF00FFu, s2));
                m2 = pk_max_u16(m2, pk_lsum_u16(lh & 0x00FF00FFu, s2));
                m3 = pk_max_u16(m3, pk_lsum_u16((lh >> 8) & 0x00FF00FFu, s2));
                a[i] = (int)sc - 128;
            }
            bad = quad4_max_pk16(bad ? 1u : 0u) != 0u;  // the block's 32 tokens
            m0 = quad4_max_pk16(m0);
            m1 = quad4_max_pk16(m1);
            m2 = quad4_max_pk16(m2);
            m3 = quad4_max_pk16(m3);
            const uint32_t em[8] = {m0 & 0xFFFFu, m2 & 0xFFFFu, m1 & 0xFFFFu, m3 & 0xFFFFu,
                                    m0 >> 16,     m2 >> 16,     m1 >> 16,     m3 >> 16};
            const int64_t c0 = tc + 8 * cg;
            const bool live = tr + 8 * g < rows && c0 < cols;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // floor(log2 amax) - 8 (E4M3 emax), clamped below at -127 (also
                // the all-zero block); it never exceeds 121
                const int e = max((int)em[j] - 137, -127);
                const int b = j >> 1;  // byte of column j in vl / vh
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t vb = (j & 1) ? vh[i] : vl[i], sb = (j & 1) ? sh[i] : sl[i];
                    // |v| / 2^e = 2|m| * 2^(s - 128 - e), exact wherever it can
                    // reach E4M3's range and at most 384 (no saturation)
                    const float v = __builtin_amdgcn_ldexpf((float)((vb >> (8 * b)) & 0xFFu), a[i] - e);
                    y[i] = as_float(as_uint(v) | ((sb << (28 - 8 * b)) & 0x80000000u));
                }
                uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
                uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
                hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
                if (bad) { lo = 0x7F7F7F7Fu; hi = 0x7F7F7F7Fu; }
                if (live) {
                    *reinterpret_cast<uint2*>(q8 + (c0 + j) * rows + tr + 8 * g) = make_uint2(lo, hi);
                    if ((g & 3) == 0) s8[(c0 + j) * (rows / 32) + (tr + 8 * g) / 32] = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
                }
            }
        }
        __syncthreads();  // LDS is free for the next tile
    }
}

hipError_t launch_fp4_row_to_fp8_col(const uint8_t* q4, const uint8_t* s4, int64_t rows, int64_t cols, uint8_t* q8,
                                     uint8_t* s8, hipStream_t st) {
    const int64_t ntc = (cols + FC_COLS - 1) / FC_COLS, ntiles = ntc * ((rows + FC_ROWS - 1) / FC_ROWS);
    const unsigned grid = (unsigned)(ntiles < FC_GRID ? ntiles : FC_GRID);
    hipLaunchKernelGGL(k_fp4_row_to_fp8_col, dim3(grid), dim3(256), 0, st, q4, s4, rows, cols, ntc, ntiles, q8, s8);
    return hipGetLastError();
}

}  // namespace mxq
