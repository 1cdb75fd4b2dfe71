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
constexpr int RP_PER_THREAD = 4;

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

}  // namespace mxq
