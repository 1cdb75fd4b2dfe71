// quantize.hip - amax reduction, per-tensor (current / delayed) scaling, MX
// block-32 quantization and the expert MLP's SwiGLU + MX quantization kernels
// for gfx950.
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
// Tiled casts with a transposed output.  A block of 256 threads (4 waves)
// owns a TT x TT tile.
//  Row phase: in step it (0..7) wave w reads tile rows 16*it + 4*w + l/16,
//  16 lanes per row, 8 consecutive elements per lane.  Every load covers
//  whole 256-byte (bf16) or 512-byte (fp32) row segments and every row-code
//  store a whole 128-byte line.  For the transposed output the lane's 8
//  codes (per-tensor) or 8 values (MX) also go to LDS.
//  Column phase: lane l of wave w takes from LDS the 8 x 8 patch at tile
//  rows 8*(l/4) .. +7 and columns 32*w + 8*(l%4) .. +7.  The 16 lanes with
//  the same l%4 then hold 128 consecutive rows of 8 columns, so each column
//  store writes a whole line.
// LDS rows are laid out in chunks of 8 elements; bits 2-3 of a chunk's index
// are XOR-ed with bits 3-4 of its row, so that the column phase's reads of
// 16 lanes (4 row groups x 4 chunks) land on distinct banks.
// ---------------------------------------------------------------------------
constexpr int TT = 128;

__device__ __forceinline__ int chunk_swz(int r, int c) { return c ^ (((r >> 3) & 3) << 2); }

// 8 consecutive elements at `off` as loaded (zeros if !ok): bf16 packed in
// u[0..3] (element 2k in the low half of u[k]), fp32 in u[0..7].  Branch
// free, so that a thread's loads issue back to back: a lane with !ok reads
// the tensor's first elements (always present) and drops them.
template <int SRC>
__device__ __forceinline__ void load_raw8(const void* x, int64_t off, bool ok, uint32_t (&u)[8]) {
    const int64_t o = ok ? off : 0;
    const uint32_t keep = ok ? ~0u : 0u;
    if constexpr (SRC == 1) {
        const uint4 v = ld_nt16((const uint16_t*)x + o);
        u[0] = v.x & keep; u[1] = v.y & keep; u[2] = v.z & keep; u[3] = v.w & keep;
        u[4] = u[5] = u[6] = u[7] = 0u;
    } else {
        const float* q = (const float*)x + o;
        const uint4 a = ld_nt16(q), b = ld_nt16(q + 4);
        u[0] = a.x & keep; u[1] = a.y & keep; u[2] = a.z & keep; u[3] = a.w & keep;
        u[4] = b.x & keep; u[5] = b.y & keep; u[6] = b.z & keep; u[7] = b.w & keep;
    }
}

// Offset of 8-element vector v of a [rows, cols] tensor with row pitch ld:
// DENSE (ld == cols) v * 8, else through its row (vpr = cols / 8 vectors
// per row).
template <bool DENSE>
__device__ __forceinline__ int64_t vec_off(int64_t v, int64_t vpr, int64_t ld) {
    if constexpr (DENSE) {
        return v * 8;
    } else {
        const int64_t row = v / vpr;
        return row * ld + (v - row * vpr) * 8;
    }
}

// Element k of 8 loaded by load_raw8, as a binary32.
template <int SRC>
__device__ __forceinline__ float elem(const uint32_t (&u)[8], int k) {
    if constexpr (SRC == 1) return as_float((k & 1) ? (u[k >> 1] & 0xFFFF0000u) : (u[k >> 1] << 16));
    else return as_float(u[k]);
}

// 8 consecutive elements at `off` as binary32 bit patterns (zeros if !ok).
template <int SRC>
__device__ __forceinline__ void load8(const void* x, int64_t off, bool ok, uint32_t (&u)[8]) {
    uint32_t r[8];
    load_raw8<SRC>(x, off, ok, r);
#pragma unroll
    for (int k = 0; k < 8; ++k) u[k] = as_uint(elem<SRC>(r, k));
}

// Block-wide max of one value per thread, then at most one atomicMax per
// block on the bit pattern of a non-negative float (NaN patterns exceed every
// finite one, so a NaN anywhere propagates).  Atomics on one address are
// serialized (about 8-10 ns each on MI355X), so the kernels that call this
// run few blocks, and a block whose max cannot raise the value already stored
// skips the atomic: the stored value only grows, so a stale read only costs a
// redundant atomic, never a lost one.
__device__ __forceinline__ void block_atomic_max(uint32_t v, unsigned int* acc) {
    __shared__ uint32_t part[4];
    v = wave_max_u32(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) part[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = part[0];
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) m = m > part[i] ? m : part[i];
        if (m > __hip_atomic_load(acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(acc, m);
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
// One wave; lane l reads entries l, l+64, ...
template <int F>
__global__ void __launch_bounds__(64) k_pt_prologue(const float* __restrict__ history, int hist_len,
                                                    unsigned int* amax_acc, float* scale_out, float* scale_inv_out) {
    const int lane = threadIdx.x;
    if (lane == 0) *amax_acc = 0u;
    if (hist_len <= 0) return;
    float m = 0.0f;
    bool nan = false;
    for (int i = lane; i < hist_len; i += 64) {
        const float h = history[i];
        if (__builtin_isnan(h)) nan = true;
        else if (h > m) m = h;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(m, off, 64);
        m = o > m ? o : m;
    }
    nan = __any(nan);
    if (lane == 0) {
        const float s = scale_from_amax<F>(nan ? __builtin_nanf("") : m);
        scale_out[0] = s;
        if (scale_inv_out) scale_inv_out[0] = 1.0f / s;
    }
}

// Largest magnitude of 8 values as a binary32 bit pattern (NaN patterns
// exceed every other): bf16 on packed 16-bit halves, fp32 on whole words.
template <int SRC>
__device__ __forceinline__ uint32_t amax8(const uint32_t (&u)[8]) {
    if constexpr (SRC == 1) {
        const uint32_t m = pk_max_u16(pk_max_u16(u[0] & 0x7FFF7FFFu, u[1] & 0x7FFF7FFFu),
                                      pk_max_u16(u[2] & 0x7FFF7FFFu, u[3] & 0x7FFF7FFFu));
        const uint32_t a = m & 0xFFFFu, b = m >> 16;
        return (a > b ? a : b) << 16;
    } else {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t a = u[k] & 0x7FFFFFFFu;
            m = m > a ? m : a;
        }
        return m;
    }
}

// amax over the tensor (current scaling, first pass), streaming: the tensor
// is walked as a flat sequence of 8-element vectors (vec_off), AMAX_VEC per
// thread per round,
// over at most PERSIST_BLOCKS blocks.
constexpr int AMAX_VEC = 16;
constexpr int PERSIST_BLOCKS = 512;  // 2 blocks of 4 waves per CU (the cast holds two tiles in VGPRs)
template <int SRC, bool DENSE>
__global__ void __launch_bounds__(256) k_amax(const void* __restrict__ x, int64_t nvec, int64_t vpr, int64_t ld,
                                              unsigned int* amax_acc) {
    uint32_t m = 0;
    for (int64_t base = (int64_t)blockIdx.x * (256 * AMAX_VEC) + threadIdx.x; base < nvec;
         base += (int64_t)gridDim.x * (256 * AMAX_VEC)) {
        uint32_t u[AMAX_VEC][8];
#pragma unroll
        for (int it = 0; it < AMAX_VEC; ++it) {
            const int64_t v = base + (int64_t)it * 256;
            load_raw8<SRC>(x, vec_off<DENSE>(v < nvec ? v : 0, vpr, ld), v < nvec, u[it]);
        }
#pragma unroll
        for (int it = 0; it < AMAX_VEC; ++it) {
            const uint32_t a = amax8<SRC>(u[it]);
            m = m > a ? m : a;
        }
    }
    block_atomic_max(m, amax_acc);
}

// Saturating cast of 8 products fl32(x * scale) to FP8 codes (x as loaded
// by load_raw8).  Clamping the product to [-max, max] with v_med3 saturates
// finite overflow and Inf and leaves everything else unchanged; RNE is the
// converter's.  A NaN among the 8 inputs (nan8, rare) sends them through
// cast2_sat_f32, which writes NaN codes with their sign.
template <int F, int SRC>
__device__ __forceinline__ uint2 cast8_pt(const uint32_t (&u)[8], float scale, bool nan8) {
    float y[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = elem<SRC>(u, k) * scale;  // binary32 product
    if (__builtin_expect(nan8, 0)) {
        return make_uint2(cast2_sat_f32<F>(y[0], y[1]) | (cast2_sat_f32<F>(y[2], y[3]) << 16),
                          cast2_sat_f32<F>(y[4], y[5]) | (cast2_sat_f32<F>(y[6], y[7]) << 16));
    }
    const float mx = as_float(FmtInfo<F>::max_f32);
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = __builtin_amdgcn_fmed3f(y[k], -mx, mx);
    uint32_t lo, hi;
    if constexpr (F == E4M3) {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], (int)hi, true);
    } else {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y[4], y[5], 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(y[6], y[7], (int)hi, true);
    }
    return make_uint2(lo, hi);
}

// Cast pass.  DELAYED: the scale was written by the prologue and this pass
// also reduces amax(x).  Current: the scale derives from the finished amax.
// COL: also the transposed codes (rows % 16 == 0).  Blocks walk the ntiles
// tiles (ntc per tile row) with a stride of the grid, loading the next tile
// while casting the current one.
// Tiles are TT rows x PT_TC(SRC) columns: 256 columns for bf16 input, so
// that each row's loads cover 512 contiguous bytes and each row-code store
// 256 (128-column tiles, 256-byte reads, measured 4.0 TB/s on a row-only
// cast against 6.5 TB/s for the MX quantizer's contiguous stream).  In the
// row phase LPR = cols/8 lanes share a tile row; in the column phase (one
// pass per 128 columns) lane l of wave w takes rows 8*(l/4) .. +7 of column
// group 16*pass + 4*w + l%4, so the 16 lanes of a column group write one
// 128-byte line of the transposed output.  LDS rows are chunks of 8 codes;
// the chunk index's bits 2.. are XOR-ed with the row's bits 3.., which keeps
// the column phase's reads free of bank conflicts.
template <int SRC> constexpr int pt_tc() { return SRC == 1 ? 256 : 128; }
template <int TC> __device__ __forceinline__ int pt_swz(int r, int c) {
    return c ^ (((r >> 3) & (TC / 32 - 1)) << 2);
}

template <int F, int SRC, bool DELAYED, bool COL>
__global__ void __launch_bounds__(256) k_pt_cast(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                 int64_t ld, int64_t ntc, int64_t ntiles, unsigned int* amax_acc,
                                                 float* scale_out, float* scale_inv_out,
                                                 uint8_t* __restrict__ q_row, uint8_t* __restrict__ q_col) {
    constexpr int TC = pt_tc<SRC>();
    constexpr int LPR = TC / 8;           // lanes per tile row in the row phase
    constexpr int RPS = 64 / LPR;         // rows per wave and step
    constexpr int NSTEP = TT / (4 * RPS); // row-phase steps
    __shared__ __attribute__((aligned(16))) uint8_t tile[COL ? TT * TC : 16];
    float scale;
    if (DELAYED) {
        scale = scale_out[0];
    } else {
        scale = scale_from_amax<F>(as_float(*(volatile unsigned int*)amax_acc));
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            if (scale_out) scale_out[0] = scale;
            if (scale_inv_out) scale_inv_out[0] = 1.0f / scale;
        }
    }
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane % LPR;  // row phase: chunk of 8 columns
    auto row_of = [&](int it) __attribute__((always_inline)) { return 4 * RPS * it + RPS * w + lane / LPR; };
    auto load_tile = [&](int64_t t, uint32_t (&u)[NSTEP][8]) __attribute__((always_inline)) {
        const int64_t tr = (t / ntc) * TT, tc = (t % ntc) * TC;
        const bool cok = tc + 8 * ch < cols;  // cols % 16 == 0: a chunk is all-in or all-out
#pragma unroll
        for (int it = 0; it < NSTEP; ++it) {
            const int r = row_of(it);
            load_raw8<SRC>(x, (tr + r) * ld + tc + 8 * ch, cok && tr + r < rows, u[it]);
        }
    };
    uint32_t m = 0;
    uint32_t u[NSTEP][8];
    int64_t t = blockIdx.x;
    if (t < ntiles) load_tile(t, u);
    for (; t < ntiles; t += gridDim.x) {
        uint32_t un[NSTEP][8];
        if (t + gridDim.x < ntiles) load_tile(t + gridDim.x, un);
        const int64_t tr = (t / ntc) * TT, tc = (t % ntc) * TC;
        const bool cok = tc + 8 * ch < cols;
#pragma unroll
        for (int it = 0; it < NSTEP; ++it) {
            const int r = row_of(it);
            const uint32_t a = amax8<SRC>(u[it]);
            if (DELAYED) m = m > a ? m : a;
            const uint2 c = cast8_pt<F, SRC>(u[it], scale, a > 0x7F800000u);
            if (q_row && cok && tr + r < rows) st_nt8(q_row + (tr + r) * cols + tc + 8 * ch, c);
            if constexpr (COL) *reinterpret_cast<uint2*>(tile + r * TC + 8 * pt_swz<TC>(r, ch)) = c;
        }
        if constexpr (COL) {
            __syncthreads();
            const int g = lane >> 2;  // 8-row group
#pragma unroll
            for (int pass = 0; pass < TC / 128; ++pass) {
                const int cg = 16 * pass + 4 * w + (lane & 3);  // 8-column group
                uint32_t lo[8], hi[8];                          // patch row i: columns 0..3, 4..7
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * g + i;
                    const uint2 v = *reinterpret_cast<const uint2*>(tile + r * TC + 8 * pt_swz<TC>(r, cg));
                    lo[i] = v.x;
                    hi[i] = v.y;
                }
                if (tr + 8 * g < rows && tc + 8 * cg < cols) {  // rows % 16 == 0: a patch is all-in or all-out
                    transpose4x4_bytes(lo[0], lo[1], lo[2], lo[3]);  // cols 0..3, rows 0..3
                    transpose4x4_bytes(lo[4], lo[5], lo[6], lo[7]);  // cols 0..3, rows 4..7
                    transpose4x4_bytes(hi[0], hi[1], hi[2], hi[3]);  // cols 4..7, rows 0..3
                    transpose4x4_bytes(hi[4], hi[5], hi[6], hi[7]);  // cols 4..7, rows 4..7
                    uint8_t* const dst = q_col + (tc + 8 * cg) * rows + tr + 8 * g;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // plain stores for the transposed output (its 128-byte
                        // segments of neighbouring tiles meet in L2)
                        *reinterpret_cast<uint2*>(dst + j * rows) = make_uint2(lo[j], lo[4 + j]);
                        *reinterpret_cast<uint2*>(dst + (4 + j) * rows) = make_uint2(hi[j], hi[4 + j]);
                    }
                }
            }
            __syncthreads();  // the tile is free for the next round
        }
#pragma unroll
        for (int it = 0; it < NSTEP; ++it)
#pragma unroll
            for (int k = 0; k < 8; ++k) u[it][k] = un[it][k];
    }
    if (DELAYED) block_atomic_max(m, amax_acc);
}

// Epilogue of delayed scaling: shift the history one step older and record
// this step's amax at entry 0.  One wave (hist_len <= 1024): every lane reads
// all its entries before any lane writes.
__global__ void __launch_bounds__(64) k_pt_history(float* history, int hist_len, const unsigned int* amax_acc) {
    const int lane = threadIdx.x;
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int i = lane + 64 * k;
        v[k] = (i == 0) ? as_float(*amax_acc) : (i < hist_len ? history[i - 1] : 0.0f);
    }
    __syncthreads();  // all reads (of every lane) before the first write
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int i = lane + 64 * k;
        if (i < hist_len) history[i] = v[k];
    }
}

// ---------------------------------------------------------------------------
// MX rowwise quantizer: a lane holds 8 consecutive elements, an aligned quad
// of lanes one 32-element block.  The tensor is walked as a flat sequence of
// 8-element vectors (vec_off; rows are whole blocks since cols % 32 == 0), so
// codes and scales are written contiguously.
// ---------------------------------------------------------------------------
constexpr int MXR_THREADS = 256;
constexpr int MXR_VEC_PER_THREAD = 2;

template <int F, int SRC, bool DENSE>
__global__ void __launch_bounds__(MXR_THREADS) k_mx_row(const void* __restrict__ x, int64_t nvec, int64_t vpr,
                                                        int64_t ld, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const int64_t base = (int64_t)blockIdx.x * (MXR_THREADS * MXR_VEC_PER_THREAD) + threadIdx.x;
    uint32_t u[MXR_VEC_PER_THREAD][8];  // bf16 source: packed pairs in u[.][0..3]
#pragma unroll
    for (int it = 0; it < MXR_VEC_PER_THREAD; ++it) {
        const int64_t v = base + (int64_t)it * MXR_THREADS;
        load_raw8<SRC>(x, vec_off<DENSE>(v < nvec ? v : 0, vpr, ld), v < nvec, u[it]);
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
            st_nt4(q + v * 4, c);
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
            st_nt8(q + v * 8, make_uint2(c0, c1));
        }
        if ((threadIdx.x & 3) == 0) s[v >> 2] = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
    }
}

// ---------------------------------------------------------------------------
// MX quantizer with a colwise (transposed) output, optionally also rowwise,
// FP8 only.  Tile phases as the per-tensor cast, with the values (not the
// codes) staged in LDS.  Row phase: a 32-column block spans the 4 lanes of a
// quad (lane bits 0-1).  Column phase: a 32-row block spans the 4 lanes that
// differ in lane bits 2-3.
// ---------------------------------------------------------------------------
template <int F, int SRC>
__global__ void __launch_bounds__(256) k_mx_dual(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                                                 uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                 uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col) {
    // the tile's values as read (bf16 or binary32), rows of TT elements in
    // 16-byte (bf16) or 2 x 16-byte (fp32) chunks of 8
    constexpr int EB = SRC == 1 ? 2 : 4;
    __shared__ __attribute__((aligned(16))) uint8_t tile[TT * TT * EB];
    const int64_t tr = (int64_t)blockIdx.y * TT, tc = (int64_t)blockIdx.x * TT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane & 15;
    const bool cok = tc + 8 * ch < cols;  // rows % 32 == 0, cols % 32 == 0
    auto lds_chunk = [&](int r, int c) __attribute__((always_inline)) -> uint8_t* {
        return tile + (r * TT + 8 * chunk_swz(r, c)) * EB;
    };
    {
        uint32_t u[8][8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 16 * it + 4 * w + (lane >> 4);
            load8<SRC>(x, (tr + r) * ld + tc + 8 * ch, cok && tr + r < rows, u[it]);
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 16 * it + 4 * w + (lane >> 4);
            if (q_row) {
                uint32_t m = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t a = u[it][k] & 0x7FFFFFFFu;
                    m = m > a ? m : a;
                }
                m = quad_max_u32(m);  // the 4 lanes of a 32-column block
                uint32_t lo, hi;
                uint8_t sb;
                mx_codes_row8<F>(u[it], m, lo, hi, sb);
                if (cok && tr + r < rows) {
                    st_nt8(q_row + (tr + r) * cols + tc + 8 * ch, make_uint2(lo, hi));
                    if ((lane & 3) == 0) s_row[(tr + r) * (cols / 32) + (tc + 8 * ch) / 32] = sb;
                }
            }
            uint8_t* const d = lds_chunk(r, ch);
            if constexpr (SRC == 1) {
                const uint4 v = make_uint4((u[it][0] >> 16) | (u[it][1] & 0xFFFF0000u),
                                           (u[it][2] >> 16) | (u[it][3] & 0xFFFF0000u),
                                           (u[it][4] >> 16) | (u[it][5] & 0xFFFF0000u),
                                           (u[it][6] >> 16) | (u[it][7] & 0xFFFF0000u));
                *reinterpret_cast<uint4*>(d) = v;
            } else {
                *reinterpret_cast<uint4*>(d) = make_uint4(u[it][0], u[it][1], u[it][2], u[it][3]);
                *reinterpret_cast<uint4*>(d + 16) = make_uint4(u[it][4], u[it][5], u[it][6], u[it][7]);
            }
        }
    }
    __syncthreads();
    // column phase: patch rows 8g .. 8g+7, columns 8cg .. 8cg+7 of the tile
    const int g = lane >> 2, cg = 4 * w + (lane & 3);
    uint32_t u[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint8_t* const s = lds_chunk(8 * g + i, cg);
        if constexpr (SRC == 1) {
            const uint4 v = *reinterpret_cast<const uint4*>(s);
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                u[i][2 * k] = wd[k] << 16;
                u[i][2 * k + 1] = wd[k] & 0xFFFF0000u;
            }
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(s), b = *reinterpret_cast<const uint4*>(s + 16);
            u[i][0] = a.x; u[i][1] = a.y; u[i][2] = a.z; u[i][3] = a.w;
            u[i][4] = b.x; u[i][5] = b.y; u[i][6] = b.z; u[i][7] = b.w;
        }
    }
    const bool live = tr + 8 * g < rows && tc + 8 * cg < cols;  // uniform over the 4 lanes of a column block
    uint32_t lo[8], hi[8];  // lo[j]: rows 0..3 of column j, hi[j]: rows 4..7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t a = u[i][j] & 0x7FFFFFFFu;
            m = m > a ? m : a;
        }
        m = quad4_max_u32(m);  // lanes l, l^4, l^8, l^12: the 32 rows of the column block
        uint32_t col[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) col[i] = u[i][j];
        uint8_t sb;
        mx_codes_row8<F>(col, m, lo[j], hi[j], sb);
        if (live && (g & 3) == 0) s_col[(tc + 8 * cg + j) * (rows / 32) + (tr + 8 * g) / 32] = sb;
    }
    if (live) {
        uint8_t* const dst = q_col + (tc + 8 * cg) * rows + tr + 8 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint2*>(dst + j * rows) = make_uint2(lo[j], hi[j]);
    }
}

// bf16 input: the same tile phases on the raw bf16 pairs.  Codes come from
// the packed bf16 converter (clamped on the 16-bit patterns), so a lane holds
// its 8 row-phase vectors as loaded (4 registers each) and the column phase
// builds each converter operand (two rows of one column) with one byte
// permute: fewer registers than the binary32 form, so more tiles per CU.
template <int F>
__device__ __forceinline__ uint2 mx_codes_bf16x8(const uint32_t (&w)[4], uint32_t amax16, uint8_t& sbyte) {
    const bool bad = amax16 >= 0x7F80u;
    const int e = block_exp<F>(amax16 >> 7);
    const float sc = exp2i(e);
    const uint32_t lim = (uint32_t)(e + 127 + FmtInfo<F>::emax) << 7 | FmtInfo<F>::max_mant_bf16;
    const uint32_t lim2 = lim | (lim << 16);
    uint32_t c0 = cvt2_bf16_fp8<F>(0u, clamp2_bf16(w[0], lim2), sc, false);
    c0 = cvt2_bf16_fp8<F>(c0, clamp2_bf16(w[1], lim2), sc, true);
    uint32_t c1 = cvt2_bf16_fp8<F>(0u, clamp2_bf16(w[2], lim2), sc, false);
    c1 = cvt2_bf16_fp8<F>(c1, clamp2_bf16(w[3], lim2), sc, true);
    if (bad) { c0 = 0x7F7F7F7Fu; c1 = 0x7F7F7F7Fu; }
    sbyte = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
    return make_uint2(c0, c1);
}

template <int F>
__global__ void __launch_bounds__(256) k_mx_dual_bf16(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                      int64_t ld, uint8_t* __restrict__ q_row,
                                                      uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_col,
                                                      uint8_t* __restrict__ s_col) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[TT * TT * 2];
    const int64_t tr = (int64_t)blockIdx.y * TT, tc = (int64_t)blockIdx.x * TT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int ch = lane & 15;
    const bool cok = tc + 8 * ch < cols;  // rows % 32 == 0, cols % 32 == 0
    auto lds_chunk = [&](int r, int c) __attribute__((always_inline)) -> uint8_t* {
        return tile + (r * TT + 8 * chunk_swz(r, c)) * 2;
    };
    {
        uint32_t raw[8][4];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 16 * it + 4 * w + (lane >> 4);
            uint32_t u[8];
            load_raw8<1>(x, (tr + r) * ld + tc + 8 * ch, cok && tr + r < rows, u);
#pragma unroll
            for (int k = 0; k < 4; ++k) raw[it][k] = u[k];
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int r = 16 * it + 4 * w + (lane >> 4);
            if (q_row) {
                const uint32_t m2 = pk_max_u16(pk_max_u16(raw[it][0] & 0x7FFF7FFFu, raw[it][1] & 0x7FFF7FFFu),
                                               pk_max_u16(raw[it][2] & 0x7FFF7FFFu, raw[it][3] & 0x7FFF7FFFu));
                const uint32_t a = m2 & 0xFFFFu, b = m2 >> 16;
                const uint32_t m = quad_max_u32(a > b ? a : b);  // the 4 lanes of a 32-column block
                uint8_t sb;
                const uint2 c = mx_codes_bf16x8<F>(raw[it], m, sb);
                if (cok && tr + r < rows) {
                    st_nt8(q_row + (tr + r) * cols + tc + 8 * ch, c);
                    if ((lane & 3) == 0) s_row[(tr + r) * (cols / 32) + (tc + 8 * ch) / 32] = sb;
                }
            }
            *reinterpret_cast<uint4*>(lds_chunk(r, ch)) = make_uint4(raw[it][0], raw[it][1], raw[it][2], raw[it][3]);
        }
    }
    __syncthreads();
    // column phase: patch rows 8g .. 8g+7, columns 8cg .. 8cg+7 of the tile;
    // word k of a patch row holds columns 2k (low half) and 2k+1
    const int g = lane >> 2, cg = 4 * w + (lane & 3);
    uint32_t wv[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(lds_chunk(8 * g + i, cg));
        wv[i][0] = v.x; wv[i][1] = v.y; wv[i][2] = v.z; wv[i][3] = v.w;
    }
    const bool live = tr + 8 * g < rows && tc + 8 * cg < cols;  // uniform over the 4 lanes of a column block
    uint8_t* const dst = q_col + (tc + 8 * cg) * rows + tr + 8 * g;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = pk_max_u16(m, wv[i][k] & 0x7FFF7FFFu);
        m = quad4_max_pk16(m);  // lanes l, l^4, l^8, l^12: the 32 rows of the column block
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // rows 2p, 2p+1 of column 2k + h as one bf16 pair
            const uint32_t sel = h ? 0x07060302u : 0x05040100u;
            uint32_t pr[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) pr[p] = __builtin_amdgcn_perm(wv[2 * p + 1][k], wv[2 * p][k], sel);
            uint8_t sb;
            const uint2 c = mx_codes_bf16x8<F>(pr, h ? m >> 16 : m & 0xFFFFu, sb);
            const int j = 2 * k + h;
            if (live) {
                // plain store: the 128-byte column segments of neighbouring
                // tiles meet in L2 (measured 9% faster than streaming stores)
                *reinterpret_cast<uint2*>(dst + j * rows) = c;
                if ((g & 3) == 0) s_col[(tc + 8 * cg + j) * (rows / 32) + (tr + 8 * g) / 32] = sb;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Expert MLP activation: h = silu(gate) * up of the grouped up-projection's
// output, MX block-32 quantized along the intermediate dimension for the
// down-projection GEMM (MoE FP4 page, "Metodologia": the expert GEMMs run
// in FP8; the activation between them is SwiGLU, silu(x) = x / (1 + e^-x),
// a reading).  gu [rows, ld] holds the gate in columns [0, inter) and the up
// projection in [inter, 2 inter).  h is formed in binary32 (expf of -|g|
// and the hardware reciprocal, a few ulps in all) and quantized like k_mx_row: a lane holds 8 consecutive
// intermediate columns, an aligned quad of lanes one 32-element block.
// ---------------------------------------------------------------------------
constexpr int SWG_VEC_PER_THREAD = 2;

template <int F, int SRC>
__global__ void __launch_bounds__(256) k_swiglu_mx(const void* __restrict__ gu, int64_t nvec, int64_t vpr,
                                                   int64_t ld, int64_t inter, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ s) {
    const int64_t base = (int64_t)blockIdx.x * (256 * SWG_VEC_PER_THREAD) + threadIdx.x;
    uint32_t gw[SWG_VEC_PER_THREAD][8], uw[SWG_VEC_PER_THREAD][8];
#pragma unroll
    for (int it = 0; it < SWG_VEC_PER_THREAD; ++it) {
        const int64_t v = base + (int64_t)it * 256;
        const bool ok = v < nvec;
        const int64_t vc = ok ? v : 0;
        const int64_t row = vc / vpr, c = (vc - row * vpr) * 8;
        load8<SRC>(gu, row * ld + c, ok, gw[it]);
        load8<SRC>(gu, row * ld + inter + c, ok, uw[it]);
    }
#pragma unroll
    for (int it = 0; it < SWG_VEC_PER_THREAD; ++it) {
        const int64_t v = base + (int64_t)it * 256;
        if (v >= nvec) continue;  // nvec % 4 == 0: quads stay whole
        uint32_t h[8];
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            h[k] = as_uint(swiglu_f32(as_float(gw[it][k]), as_float(uw[it][k])));
            const uint32_t a = h[k] & 0x7FFFFFFFu;
            m = m > a ? m : a;
        }
        m = quad_max_u32(m);  // the 4 lanes of a 32-column block
        uint32_t lo, hi;
        uint8_t sb;
        mx_codes_row8<F>(h, m, lo, hi, sb);
        st_nt8(q + v * 8, make_uint2(lo, hi));  // rows of q are dense: vector v starts at byte 8 v
        if ((threadIdx.x & 3) == 0) s[v >> 2] = sb;
    }
}

template <int F, int SRC>
static void launch_swiglu_t(const void* gu, int64_t rows, int64_t inter, int64_t ld, uint8_t* q, uint8_t* s,
                            hipStream_t st) {
    const int64_t vpr = inter / 8, nvec = rows * vpr;
    const unsigned grid = (unsigned)((nvec + 256 * SWG_VEC_PER_THREAD - 1) / (256 * SWG_VEC_PER_THREAD));
    hipLaunchKernelGGL((k_swiglu_mx<F, SRC>), dim3(grid), dim3(256), 0, st, gu, nvec, vpr, ld, inter, q, s);
}

hipError_t launch_swiglu_quantize_mx(const void* gu, int src, int64_t rows, int64_t inter, int64_t ld, int fmt,
                                     uint8_t* q, uint8_t* s, hipStream_t st) {
    switch (fmt * 2 + src) {
    case E4M3 * 2 + 0: launch_swiglu_t<E4M3, 0>(gu, rows, inter, ld, q, s, st); break;
    case E4M3 * 2 + 1: launch_swiglu_t<E4M3, 1>(gu, rows, inter, ld, q, s, st); break;
    case E5M2 * 2 + 0: launch_swiglu_t<E5M2, 0>(gu, rows, inter, ld, q, s, st); break;
    case E5M2 * 2 + 1: launch_swiglu_t<E5M2, 1>(gu, rows, inter, ld, q, s, st); break;
    }
    return hipGetLastError();
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
    constexpr int TC = pt_tc<SRC>();
    const int64_t ntc = (cols + TC - 1) / TC, ntiles = ntc * ((rows + TT - 1) / TT);
    const dim3 grid((unsigned)(ntiles < PERSIST_BLOCKS ? ntiles : PERSIST_BLOCKS));
    if (hist_len > 0) {
        if (q_col)
            hipLaunchKernelGGL((k_pt_cast<F, SRC, true, true>), grid, dim3(256), 0, st, x, rows, cols, ld, ntc, ntiles,
                               acc, scale_out, scale_inv_out, q_row, q_col);
        else
            hipLaunchKernelGGL((k_pt_cast<F, SRC, true, false>), grid, dim3(256), 0, st, x, rows, cols, ld, ntc,
                               ntiles, acc, scale_out, scale_inv_out, q_row, q_col);
        hipLaunchKernelGGL(k_pt_history, dim3(1), dim3(64), 0, st, history, hist_len, (const unsigned int*)acc);
    } else {
        const int64_t nvec = rows * (cols / 8);
        const int64_t vpr = (ld == cols) ? 0 : cols / 8;
        const int64_t ab = (nvec + 256 * AMAX_VEC - 1) / (256 * AMAX_VEC);
        const dim3 agrid((unsigned)(ab < PERSIST_BLOCKS ? ab : PERSIST_BLOCKS));
        if (vpr == 0)
            hipLaunchKernelGGL((k_amax<SRC, true>), agrid, dim3(256), 0, st, x, nvec, vpr, ld, acc);
        else
            hipLaunchKernelGGL((k_amax<SRC, false>), agrid, dim3(256), 0, st, x, nvec, vpr, ld, acc);
        if (q_col)
            hipLaunchKernelGGL((k_pt_cast<F, SRC, false, true>), grid, dim3(256), 0, st, x, rows, cols, ld, ntc,
                               ntiles, acc, scale_out, scale_inv_out, q_row, q_col);
        else
            hipLaunchKernelGGL((k_pt_cast<F, SRC, false, false>), grid, dim3(256), 0, st, x, rows, cols, ld, ntc,
                               ntiles, acc, scale_out, scale_inv_out, q_row, q_col);
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
    if (vpr == 0)
        hipLaunchKernelGGL((k_mx_row<F, SRC, true>), dim3(grid), dim3(MXR_THREADS), 0, st, x, nvec, vpr, ld, q, s);
    else
        hipLaunchKernelGGL((k_mx_row<F, SRC, false>), dim3(grid), dim3(MXR_THREADS), 0, st, x, nvec, vpr, ld, q, s);
}

template <int F, int SRC>
static void launch_mx_dual_t(const void* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* q_row, uint8_t* s_row,
                             uint8_t* q_col, uint8_t* s_col, hipStream_t st) {
    const dim3 grid((unsigned)((cols + TT - 1) / TT), (unsigned)((rows + TT - 1) / TT));
    if constexpr (SRC == 1)
        hipLaunchKernelGGL((k_mx_dual_bf16<F>), grid, dim3(256), 0, st, x, rows, cols, ld, q_row, s_row, q_col, s_col);
    else
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
