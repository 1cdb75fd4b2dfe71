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
// Design: eight lanes share one 128-element group; a lane turns 16 FP4
// codes (8 bytes) into 16 E4M3 codes (16 bytes).  Because every element of a
// 32-block sees the same exponent shift d = s4 - s8 <= 0, the lane first
// builds the 8-entry table T[m] = E4M3(|E2M1 m| * 2^d) and then maps nibbles
// to bytes with v_perm_b32 lookups; the sign bit moves from bit 3 to bit 7.
#include "common.h"
#include "launch.h"

namespace mxq {

constexpr int RP_THREADS = 256;

__global__ void __launch_bounds__(RP_THREADS) k_repack(const uint8_t* __restrict__ q4, const uint8_t* __restrict__ s4,
                                                       const int32_t* __restrict__ idx, int64_t src_rows, int64_t rows,
                                                       int64_t gpr, uint8_t* __restrict__ q8, uint8_t* __restrict__ s8) {
    const int64_t lane_id = (int64_t)blockIdx.x * RP_THREADS + threadIdx.x;
    const int64_t gid = lane_id >> 3;  // group id over [rows, gpr]
    const int j = threadIdx.x & 7;     // 16-element slice of the group
    if (gid >= rows * gpr) return;
    const int64_t r = gid / gpr;
    const int64_t g = gid - r * gpr;
    const int64_t sr = idx ? (int64_t)idx[r] : r;
    const bool valid = sr >= 0 && sr < src_rows;
    uint32_t sw = 0xFFFFFFFFu;
    uint2 code4 = make_uint2(0u, 0u);
    if (valid) {
        sw = *reinterpret_cast<const uint32_t*>(s4 + sr * (gpr * 4) + g * 4);
        code4 = *reinterpret_cast<const uint2*>(q4 + sr * (gpr * 64) + g * 64 + j * 8);
    }
    const uint32_t b0 = sw & 0xFFu, b1 = (sw >> 8) & 0xFFu, b2 = (sw >> 16) & 0xFFu, b3 = sw >> 24;
    uint32_t smax = b0 > b1 ? b0 : b1;
    smax = smax > b2 ? smax : b2;
    smax = smax > b3 ? smax : b3;
    uint4 out;
    if (smax == 0xFFu) {
        out = make_uint4(0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu);
    } else {
        const uint32_t sb = (sw >> (8 * (j >> 1))) & 0xFFu;  // this slice's block scale
        const int d = (int)sb - (int)smax;                   // in [-254, 0]
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
        uint32_t o[4];
        const uint32_t w[2] = {code4.x, code4.y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t lo = w[h] & 0x0F0F0F0Fu;          // nibbles 0,2,4,6 of this dword
            const uint32_t hi = (w[h] >> 4) & 0x0F0F0F0Fu;   // nibbles 1,3,5,7
            const uint32_t n01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // elements 0..3
            const uint32_t n23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // elements 4..7
            o[2 * h] = __builtin_amdgcn_perm(thi, tlo, n01 & 0x07070707u) | ((n01 & 0x08080808u) << 4);
            o[2 * h + 1] = __builtin_amdgcn_perm(thi, tlo, n23 & 0x07070707u) | ((n23 & 0x08080808u) << 4);
        }
        out = make_uint4(o[0], o[1], o[2], o[3]);
    }
    *reinterpret_cast<uint4*>(q8 + r * (gpr * 128) + g * 128 + j * 16) = out;
    if (j == 0) s8[r * gpr + g] = (uint8_t)smax;
}

hipError_t launch_repack_fp4_to_fp8(const uint8_t* q4, const uint8_t* s4, const int32_t* idx, int64_t src_rows,
                                    int64_t rows, int64_t cols, uint8_t* q8, uint8_t* s8, hipStream_t st) {
    const int64_t gpr = cols / 128;
    const int64_t lanes = rows * gpr * 8;
    const unsigned grid = (unsigned)((lanes + RP_THREADS - 1) / RP_THREADS);
    hipLaunchKernelGGL(k_repack, dim3(grid), dim3(RP_THREADS), 0, st, q4, s4, idx, src_rows, rows, gpr, q8, s8);
    return hipGetLastError();
}

}  // namespace mxq
