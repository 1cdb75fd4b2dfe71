// quantize.hip - amax reduction, per-tensor (current / delayed) scaling and
// MX block-32 quantization kernels for gfx950.
//
// Per-tensor path: FP8 guide, "Estrategias de escalonamento e estabilidade"
// (one factor per tensor from its statistics; delayed scaling takes the
// factor from earlier iterations) and "Transformer Engine: a fundacao de
// software" (margin 0, amax history of 16 reduced with max).
// MX path: MoE FP4 page, "Metodologia" (32-element blocks with power-of-two
// scales) and FP8 guide, "MXFP8 e NVFP4" (block-level FP8 scaling).
#include "common.h"
#include "launch.h"

namespace mxq {

// ---------------------------------------------------------------------------
// Tile geometry shared by the per-tensor cast and the dual MX quantizer.
// A thread owns an 8x8 element patch; a wave is 16 (rows) x 4 (cols) lanes,
// i.e. 128 rows x 32 cols; the 4 waves of a block sit side by side along the
// columns, so a block covers 128 x 128.
// ---------------------------------------------------------------------------
constexpr int TILE = 128;

struct Patch {
    int64_t r0;  // first row of the patch
    int64_t c0;  // first column of the patch
};

__device__ __forceinline__ Patch patch_of_thread() {
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    Patch p;
    p.r0 = (int64_t)blockIdx.y * TILE + (l >> 2) * 8;
    p.c0 = (int64_t)blockIdx.x * TILE + w * 32 + (l & 3) * 8;
    return p;
}

// Load an 8x8 patch as binary32 bit patterns (zeros outside the tensor).
template <int SRC>
__device__ __forceinline__ void load_patch(const void* x, int64_t rows, int64_t cols, int64_t ld, Patch p,
                                           uint32_t (&u)[8][8]) {
    const bool cok = p.c0 < cols;  // cols % 8 == 0: a patch row is all-in or all-out
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = p.r0 + i;
        if (cok && r < rows) {
            if (SRC == 1) {
                const uint4 v = *reinterpret_cast<const uint4*>((const uint16_t*)x + r * ld + p.c0);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    u[i][2 * k] = w[k] << 16;
                    u[i][2 * k + 1] = w[k] & 0xFFFF0000u;
                }
            } else {
                const uint4* q = reinterpret_cast<const uint4*>((const float*)x + r * ld + p.c0);
                const uint4 a = q[0], b = q[1];
                u[i][0] = a.x; u[i][1] = a.y; u[i][2] = a.z; u[i][3] = a.w;
                u[i][4] = b.x; u[i][5] = b.y; u[i][6] = b.z; u[i][7] = b.w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) u[i][k] = 0u;
        }
    }
}

// Block-wide max of one value per thread, then one atomicMax per block on the
// bit pattern of a non-negative float (NaN patterns exceed every finite one,
// so a NaN anywhere propagates).
__device__ __forceinline__ void block_atomic_max(uint32_t v, unsigned int* acc) {
    __shared__ uint32_t part[4];
    v = wave_max_u32(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) part[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = part[0];
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = m > part[i] ? m : part[i];
        atomicMax(acc, m);
    }
}

// ---------------------------------------------------------------------------
// Per-tensor scale: scale = fl32(F_max / amax_ref); 1 for amax_ref 0 / Inf /
// NaN; FLT_MAX if the quotient overflows.  IEEE division (no fast math).
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ float scale_from_amax(float amax) {
    const float fmax = as_float(FmtInfo<F>::max_f32);
    if (!(amax > 0.0f) || __builtin_isinf(amax)) return 1.0f;
    float s = fmax / amax;
    if (__builtin_isinf(s)) s = 3.40282347e+38f;
    return s;
}

// Prologue: zero the amax accumulator; for delayed scaling also derive the
// scale from the history (max over the previous steps, NaN propagates).
template <int F>
__global__ void k_pt_prologue(const float* __restrict__ history, int hist_len, unsigned int* amax_acc,
                              float* scale_out, float* scale_inv_out) {
    if (threadIdx.x != 0) return;
    *amax_acc = 0u;
    if (hist_len > 0) {
        float m = 0.0f;
        bool nan = false;
        for (int i = 0; i < hist_len; ++i) {
            const float h = history[i];
            if (__builtin_isnan(h)) nan = true;
            else if (h > m) m = h;
        }
        const float s = scale_from_amax<F>(nan ? __builtin_nanf("") : m);
        scale_out[0] = s;
        if (scale_inv_out) scale_inv_out[0] = 1.0f / s;
    }
}

// amax over the tensor (current scaling, first pass).
template <int SRC>
__global__ void __launch_bounds__(256) k_amax(const void* __restrict__ x, int64_t rows, int64_t cols,
                                              int64_t ld, unsigned int* amax_acc) {
    const Patch p = patch_of_thread();
    uint32_t u[8][8];
    load_patch<SRC>(x, rows, cols, ld, p, u);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t a = u[i][k] & 0x7FFFFFFFu;
            m = m > a ? m : a;
        }
    block_atomic_max(m, amax_acc);
}

// Cast pass.  DELAYED: the scale was written by the prologue and this pass
// also reduces amax(x).  Current: the scale derives from the finished amax.
template <int F, int SRC, bool DELAYED>
__global__ void __launch_bounds__(256) k_pt_cast(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                 int64_t ld, unsigned int* amax_acc, float* scale_out,
                                                 float* scale_inv_out, uint8_t* __restrict__ q_row,
                                                 uint8_t* __restrict__ q_col) {
    float scale;
    if (DELAYED) {
        scale = scale_out[0];
    } else {
        scale = scale_from_amax<F>(as_float(*(volatile unsigned int*)amax_acc));
        if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
            if (scale_out) scale_out[0] = scale;
            if (scale_inv_out) scale_inv_out[0] = 1.0f / scale;
        }
    }
    const Patch p = patch_of_thread();
    uint32_t u[8][8];
    load_patch<SRC>(x, rows, cols, ld, p, u);
    if (DELAYED) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t a = u[i][k] & 0x7FFFFFFFu;
                m = m > a ? m : a;
            }
        block_atomic_max(m, amax_acc);
    }
    // codes: row i -> (lo, hi) dwords holding columns 0..3 and 4..7
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = as_float(u[i][k]) * scale;  // binary32 product
        lo[i] = cast2_sat_f32<F>(y[0], y[1]) | (cast2_sat_f32<F>(y[2], y[3]) << 16);
        hi[i] = cast2_sat_f32<F>(y[4], y[5]) | (cast2_sat_f32<F>(y[6], y[7]) << 16);
    }
    if (p.c0 >= cols) return;
    if (q_row) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = p.r0 + i;
            if (r < rows) *reinterpret_cast<uint2*>(q_row + r * cols + p.c0) = make_uint2(lo[i], hi[i]);
        }
    }
    if (q_col && p.r0 < rows) {  // rows % 16 == 0: a patch is all-in or all-out
        transpose4x4_bytes(lo[0], lo[1], lo[2], lo[3]);  // cols 0..3, rows 0..3
        transpose4x4_bytes(lo[4], lo[5], lo[6], lo[7]);  // cols 0..3, rows 4..7
        transpose4x4_bytes(hi[0], hi[1], hi[2], hi[3]);  // cols 4..7, rows 0..3
        transpose4x4_bytes(hi[4], hi[5], hi[6], hi[7]);  // cols 4..7, rows 4..7
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint2*>(q_col + (p.c0 + j) * rows + p.r0) = make_uint2(lo[j], lo[4 + j]);
            *reinterpret_cast<uint2*>(q_col + (p.c0 + 4 + j) * rows + p.r0) = make_uint2(hi[j], hi[4 + j]);
        }
    }
}

// Epilogue of delayed scaling: shift the history one step older and record
// this step's amax at entry 0.
__global__ void k_pt_history(float* history, int hist_len, const unsigned int* amax_acc) {
    if (threadIdx.x != 0) return;
    for (int i = hist_len - 1; i >= 1; --i) history[i] = history[i - 1];
    history[0] = as_float(*amax_acc);
}

// ---------------------------------------------------------------------------
// MX rowwise quantizer: a lane holds 8 consecutive elements, an aligned quad
// of lanes one 32-element block.  The tensor is walked as a flat sequence of
// 8-element vectors (rows are whole blocks since cols % 32 == 0), so codes and
// scales are written contiguously.
// ---------------------------------------------------------------------------
constexpr int MXR_THREADS = 256;
constexpr int MXR_VEC_PER_THREAD = 4;

template <int F, int SRC>
__global__ void __launch_bounds__(MXR_THREADS) k_mx_row(const void* __restrict__ x, int64_t nvec, int64_t vpr,
                                                        int64_t ld, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const int64_t base = (int64_t)blockIdx.x * (MXR_THREADS * MXR_VEC_PER_THREAD) + threadIdx.x;
    uint32_t u[MXR_VEC_PER_THREAD][8];  // bf16 source: packed pairs in u[.][0..3]
#pragma unroll
    for (int it = 0; it < MXR_VEC_PER_THREAD; ++it) {
        const int64_t v = base + (int64_t)it * MXR_THREADS;
        if (v < nvec) {
            const int64_t row = (vpr == 0) ? 0 : v / vpr;
            const int64_t off = (vpr == 0) ? v * 8 : row * ld + (v - row * vpr) * 8;
            if (SRC == 1) {
                const uint4 a = *reinterpret_cast<const uint4*>((const uint16_t*)x + off);
                u[it][0] = a.x; u[it][1] = a.y; u[it][2] = a.z; u[it][3] = a.w;
            } else {
                const uint4* p = reinterpret_cast<const uint4*>((const float*)x + off);
                const uint4 a = p[0], b = p[1];
                u[it][0] = a.x; u[it][1] = a.y; u[it][2] = a.z; u[it][3] = a.w;
                u[it][4] = b.x; u[it][5] = b.y; u[it][6] = b.z; u[it][7] = b.w;
            }
        }
    }
#pragma unroll
    for (int it = 0; it < MXR_VEC_PER_THREAD; ++it) {
        const int64_t v = base + (int64_t)it * MXR_THREADS;
        if (v >= nvec) continue;  // nvec % 4 == 0: quads stay whole
        uint32_t amax;
        if (SRC == 1) {
            const uint32_t m = pk_max_u16(pk_max_u16(u[it][0] & 0x7FFF7FFFu, u[it][1] & 0x7FFF7FFFu),
                                          pk_max_u16(u[it][2] & 0x7FFF7FFFu, u[it][3] & 0x7FFF7FFFu));
            const uint32_t a = m & 0xFFFFu, b = m >> 16;
            amax = (a > b ? a : b) << 16;
        } else {
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t a = u[it][k] & 0x7FFFFFFFu;
                m = m > a ? m : a;
            }
            amax = m;
        }
        amax = quad_max_u32(amax);
        const bool bad = amax >= 0x7F800000u;  // block holds Inf or NaN
        const int e = block_exp<F>(amax >> 23);
        const float sc = exp2i(e);
        if constexpr (F == E2M1) {
            uint32_t c = 0;
            if (SRC == 1) {
                c = cvt2_bf16_fp4<0>(c, u[it][0], sc);
                c = cvt2_bf16_fp4<1>(c, u[it][1], sc);
                c = cvt2_bf16_fp4<2>(c, u[it][2], sc);
                c = cvt2_bf16_fp4<3>(c, u[it][3], sc);
            } else {
                c = cvt2_f32_fp4<0>(c, as_float(u[it][0]), as_float(u[it][1]), sc);
                c = cvt2_f32_fp4<1>(c, as_float(u[it][2]), as_float(u[it][3]), sc);
                c = cvt2_f32_fp4<2>(c, as_float(u[it][4]), as_float(u[it][5]), sc);
                c = cvt2_f32_fp4<3>(c, as_float(u[it][6]), as_float(u[it][7]), sc);
            }
            if (bad) c = 0u;
            *reinterpret_cast<uint32_t*>(q + v * 4) = c;
        } else {
            uint32_t c0 = 0, c1 = 0;
            if constexpr (SRC == 1) {
                const uint32_t lim = (uint32_t)(e + 127 + FmtInfo<F>::emax) << 7 | FmtInfo<F>::max_mant_bf16;
                const uint32_t lim2 = lim | (lim << 16);
                c0 = cvt2_bf16_fp8<F>(c0, clamp2_bf16(u[it][0], lim2), sc, false);
                c0 = cvt2_bf16_fp8<F>(c0, clamp2_bf16(u[it][1], lim2), sc, true);
                c1 = cvt2_bf16_fp8<F>(c1, clamp2_bf16(u[it][2], lim2), sc, false);
                c1 = cvt2_bf16_fp8<F>(c1, clamp2_bf16(u[it][3], lim2), sc, true);
            } else {
                const uint32_t lim = (uint32_t)(e + 127 + FmtInfo<F>::emax) << 23 | FmtInfo<F>::max_mant_f32;
                float y[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = as_float(clamp_f32(u[it][k], lim));
                c0 = cvt2_f32_fp8<F>(c0, y[0], y[1], sc, false);
                c0 = cvt2_f32_fp8<F>(c0, y[2], y[3], sc, true);
                c1 = cvt2_f32_fp8<F>(c1, y[4], y[5], sc, false);
                c1 = cvt2_f32_fp8<F>(c1, y[6], y[7], sc, true);
            }
            if (bad) { c0 = 0x7F7F7F7Fu; c1 = 0x7F7F7F7Fu; }
            *reinterpret_cast<uint2*>(q + v * 8) = make_uint2(c0, c1);
        }
        if ((threadIdx.x & 3) == 0) s[v >> 2] = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
    }
}

// ---------------------------------------------------------------------------
// MX quantizer with a colwise (transposed) output, optionally also rowwise,
// FP8 only.  Patch geometry as the per-tensor cast: a row block of 32 spans
// the 4 lanes of a quad (lane bits 0-1), a column block of 32 spans 4 lanes
// with lane bits 2-3.
// ---------------------------------------------------------------------------
template <int F>
__device__ __forceinline__ void mx_codes_row8(const uint32_t (&u)[8], uint32_t amax_bits, uint32_t& lo, uint32_t& hi,
                                              uint8_t& sbyte) {
    const bool bad = amax_bits >= 0x7F800000u;
    const int e = block_exp<F>(amax_bits >> 23);
    const float sc = exp2i(e);
    const uint32_t lim = (uint32_t)(e + 127 + FmtInfo<F>::emax) << 23 | FmtInfo<F>::max_mant_f32;
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = as_float(clamp_f32(u[k], lim));
    lo = cvt2_f32_fp8<F>(0u, y[0], y[1], sc, false);
    lo = cvt2_f32_fp8<F>(lo, y[2], y[3], sc, true);
    hi = cvt2_f32_fp8<F>(0u, y[4], y[5], sc, false);
    hi = cvt2_f32_fp8<F>(hi, y[6], y[7], sc, true);
    if (bad) { lo = 0x7F7F7F7Fu; hi = 0x7F7F7F7Fu; }
    sbyte = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
}

template <int F, int SRC>
__global__ void __launch_bounds__(256) k_mx_dual(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                 uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                 uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col) {
    const Patch p = patch_of_thread();
    uint32_t u[8][8];
    load_patch<SRC>(x, rows, cols, ld, p, u);  // rows % 32 == 0, cols % 32 == 0
    const bool live = p.r0 < rows && p.c0 < cols;  // uniform per aligned quad in both directions
    const int lane = threadIdx.x & 63;
    if (q_row) {
        uint32_t am[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t a = u[i][k] & 0x7FFFFFFFu;
                m = m > a ? m : a;
            }
            am[i] = quad_max_u32(m);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t lo, hi;
            uint8_t sb;
            mx_codes_row8<F>(u[i], am[i], lo, hi, sb);
            const int64_t r = p.r0 + i;
            if (live) {
                *reinterpret_cast<uint2*>(q_row + r * cols + p.c0) = make_uint2(lo, hi);
                if ((lane & 3) == 0) s_row[r * (cols / 32) + p.c0 / 32] = sb;
            }
        }
    }
    if (q_col) {
        // column j of the patch: values u[0..7][j]
        uint32_t lo[8], hi[8];  // lo[j]: rows 0..3 of column j, hi[j]: rows 4..7
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t a = u[i][j] & 0x7FFFFFFFu;
                m = m > a ? m : a;
            }
            m = quad4_max_u32(m);
            uint32_t col[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) col[i] = u[i][j];
            uint8_t sb;
            mx_codes_row8<F>(col, m, lo[j], hi[j], sb);
            if (live && ((lane >> 2) & 3) == 0) s_col[(p.c0 + j) * (rows / 32) + p.r0 / 32] = sb;
        }
        if (live) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint2*>(q_col + (p.c0 + j) * rows + p.r0) = make_uint2(lo[j], hi[j]);
        }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int F, int SRC>
static hipError_t launch_pt(const void* x, int64_t rows, int64_t cols, int64_t ld, float* history, int hist_len,
                            float* amax_out, float* scale_out, float* scale_inv_out, uint8_t* q_row,
                            uint8_t* q_col, hipStream_t st) {
    unsigned int* acc = reinterpret_cast<unsigned int*>(amax_out);
    hipLaunchKernelGGL((k_pt_prologue<F>), dim3(1), dim3(64), 0, st, history, hist_len, acc, scale_out, scale_inv_out);
    const dim3 grid((unsigned)((cols + TILE - 1) / TILE), (unsigned)((rows + TILE - 1) / TILE));
    if (hist_len > 0) {
        hipLaunchKernelGGL((k_pt_cast<F, SRC, true>), grid, dim3(256), 0, st, x, rows, cols, ld, acc, scale_out,
                           scale_inv_out, q_row, q_col);
        hipLaunchKernelGGL(k_pt_history, dim3(1), dim3(64), 0, st, history, hist_len, (const unsigned int*)acc);
    } else {
        hipLaunchKernelGGL((k_amax<SRC>), grid, dim3(256), 0, st, x, rows, cols, ld, acc);
        hipLaunchKernelGGL((k_pt_cast<F, SRC, false>), grid, dim3(256), 0, st, x, rows, cols, ld, acc, scale_out,
                           scale_inv_out, q_row, q_col);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_per_tensor(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int fmt,
                                      float* history, int hist_len, float* amax_out, float* scale_out,
                                      float* scale_inv_out, uint8_t* q_row, uint8_t* q_col, hipStream_t st) {
    if (fmt == E4M3)
        return src == 1 ? launch_pt<E4M3, 1>(x, rows, cols, ld, history, hist_len, amax_out, scale_out, scale_inv_out, q_row, q_col, st)
                        : launch_pt<E4M3, 0>(x, rows, cols, ld, history, hist_len, amax_out, scale_out, scale_inv_out, q_row, q_col, st);
    return src == 1 ? launch_pt<E5M2, 1>(x, rows, cols, ld, history, hist_len, amax_out, scale_out, scale_inv_out, q_row, q_col, st)
                    : launch_pt<E5M2, 0>(x, rows, cols, ld, history, hist_len, amax_out, scale_out, scale_inv_out, q_row, q_col, st);
}

template <int F, int SRC>
static void launch_mx_row_t(const void* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* q, uint8_t* s,
                            hipStream_t st) {
    const int64_t nvec = rows * (cols / 8);
    const int64_t vpr = (ld == cols) ? 0 : cols / 8;
    const int64_t per_block = MXR_THREADS * MXR_VEC_PER_THREAD;
    const unsigned grid = (unsigned)((nvec + per_block - 1) / per_block);
    hipLaunchKernelGGL((k_mx_row<F, SRC>), dim3(grid), dim3(MXR_THREADS), 0, st, x, nvec, vpr, ld, q, s);
}

template <int F, int SRC>
static void launch_mx_dual_t(const void* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* q_row, uint8_t* s_row,
                             uint8_t* q_col, uint8_t* s_col, hipStream_t st) {
    const dim3 grid((unsigned)((cols + TILE - 1) / TILE), (unsigned)((rows + TILE - 1) / TILE));
    hipLaunchKernelGGL((k_mx_dual<F, SRC>), grid, dim3(256), 0, st, x, rows, cols, ld, q_row, s_row, q_col, s_col);
}

hipError_t launch_quantize_mx(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int fmt, uint8_t* q_row,
                              uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t st) {
    if (q_col == nullptr) {
        switch (fmt * 2 + src) {
        case E4M3 * 2 + 0: launch_mx_row_t<E4M3, 0>(x, rows, cols, ld, q_row, s_row, st); break;
        case E4M3 * 2 + 1: launch_mx_row_t<E4M3, 1>(x, rows, cols, ld, q_row, s_row, st); break;
        case E5M2 * 2 + 0: launch_mx_row_t<E5M2, 0>(x, rows, cols, ld, q_row, s_row, st); break;
        case E5M2 * 2 + 1: launch_mx_row_t<E5M2, 1>(x, rows, cols, ld, q_row, s_row, st); break;
        case E2M1 * 2 + 0: launch_mx_row_t<E2M1, 0>(x, rows, cols, ld, q_row, s_row, st); break;
        case E2M1 * 2 + 1: launch_mx_row_t<E2M1, 1>(x, rows, cols, ld, q_row, s_row, st); break;
        }
    } else {
        switch (fmt * 2 + src) {
        case E4M3 * 2 + 0: launch_mx_dual_t<E4M3, 0>(x, rows, cols, ld, q_row, s_row, q_col, s_col, st); break;
        case E4M3 * 2 + 1: launch_mx_dual_t<E4M3, 1>(x, rows, cols, ld, q_row, s_row, q_col, s_col, st); break;
        case E5M2 * 2 + 0: launch_mx_dual_t<E5M2, 0>(x, rows, cols, ld, q_row, s_row, q_col, s_col, st); break;
        case E5M2 * 2 + 1: launch_mx_dual_t<E5M2, 1>(x, rows, cols, ld, q_row, s_row, q_col, s_col, st); break;
        }
    }
    return hipGetLastError();
}

}  // namespace mxq
