// gemm.hip - FP8 / MX block-scaled GEMM (dense and ragged grouped) on
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4, fp32 accumulation.
//
// MoE FP4 page, "Metodologia": the heavy matrix products stay in FP8 on the
// matrix units; "Kernels CUDA Otimizados": ragged per-expert token counts.
// FP8 guide, "MXFP8 e NVFP4": block-scaled FP8 products in hardware.
//
// C[m, n] = sum_k deq(A)[m, k] * deq(B)[n, k], A [M, K] and B [N, K] both
// K-contiguous.  Block scales (E8M0, one byte per 32 or 128 along K) enter
// the MFMA's per-lane scale operands; a per-tensor factor enters as scale
// byte 127 (x1) and multiplies the fp32 result in the epilogue.
//
// Operand layout of the 16x16x128 scaled MFMA (pinned on the device with
// one-instruction tests): lane l supplies row l % 16 and the E8M0 scale of
// K block l / 16 (32 elements each).  An FP8 lane holds 32 codes as two
// 16-byte halves: byte j sits at K = 64 * (j / 16) + 16 * (l / 16) + j % 16.
// An FP4 lane holds K = 32 * (l / 16) .. +31 in 16 bytes, element 2i in the
// low nibble of byte i.  The accumulator lane l, register r is row
// 4 * (l / 16) + r, column l % 16.
#include "common.h"
#include "launch.h"

namespace mxq {

constexpr int BM = 128, BN = 128, BK = 128;  // K step in elements
constexpr int NT = 256;                      // 4 waves, 2 x 2, 64 x 64 each

template <int F> struct OpInfo {
    static constexpr int kb = (F == E2M1) ? 64 : 128;  // bytes per row per K step
    static constexpr int chunks = kb / 16;              // 16-byte chunks per row per step
    static constexpr int code = FmtInfo<F>::mfma_code;
};

// LDS byte offset of 16-byte chunk `c` of tile row `r` (XOR swizzle so the
// fragment reads of consecutive rows hit distinct bank groups).
template <int F> __device__ __forceinline__ int lds_off(int r, int c) {
    constexpr int CH = OpInfo<F>::chunks;
    const int sw = (CH == 8) ? (r & 7) : ((r >> 1) & 3);
    return r * OpInfo<F>::kb + ((c ^ sw) << 4);
}

struct Tile {
    int64_t m0, m_end, n0;
    const uint8_t* B;
    const uint8_t* sB;
};

// Map this block to an output tile.  Dense: a grouped ordering of the tile
// grid (GM tile-rows at a time) after spreading consecutive tiles over the
// 8 XCDs; grouped: the m-tiles of all groups, scanned from the offsets.
__device__ __forceinline__ bool tile_of_block(const GemmArgs& g, Tile& t) {
    const int64_t ntn = (g.N + BN - 1) / BN;
    int64_t bid = blockIdx.x;
    t.B = g.B;
    t.sB = (const uint8_t*)g.sB;
    if (g.group_off == nullptr) {
        const int64_t ntm = (g.M + BM - 1) / BM;
        const int64_t nblk = ntm * ntn;
        // blocks are dispatched round-robin over 8 XCDs: give each XCD a
        // contiguous run of logical tiles so neighbours share its L2
        if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
        constexpr int64_t GM = 8;
        const int64_t per_group = GM * ntn;
        const int64_t grp = bid / per_group;
        const int64_t first = grp * GM;
        const int64_t gs = (ntm - first) < GM ? (ntm - first) : GM;
        const int64_t in = bid - grp * per_group;
        const int64_t tm = first + in % gs;
        const int64_t tn = in / gs;
        t.m0 = tm * BM;
        t.m_end = g.M;
        t.n0 = tn * BN;
        return true;
    }
    const int64_t tn = bid % ntn;
    int64_t mt = bid / ntn;
    for (int64_t gi = 0; gi < g.G; ++gi) {
        const int64_t r0 = g.group_off[gi], r1 = g.group_off[gi + 1];
        const int64_t nt = r1 > r0 ? (r1 - r0 + BM - 1) / BM : 0;
        if (mt < nt) {
            t.m0 = r0 + mt * BM;
            t.m_end = r1;
            t.n0 = tn * BN;
            t.B = g.B + gi * g.b_group_stride;
            t.sB = (const uint8_t*)g.sB + gi * g.sb_group_stride;
            return true;
        }
        mt -= nt;
    }
    return false;
}

// E8M0 byte for (row, K step ks, 32-block q of the step) of an operand.
__device__ __forceinline__ uint32_t scale_byte(const uint8_t* s, int mode, int64_t row, int64_t row_end, int64_t K,
                                               int64_t ks, int q) {
    if (mode == 0 || row >= row_end) return 127u;
    if (mode == 1) return s[row * (K / 32) + ks * 4 + q];
    return s[row * (K / 128) + ks];
}

template <int FA, int FB>
__global__ void __launch_bounds__(NT) k_gemm(const GemmArgs g) {
    using IA = OpInfo<FA>;
    using IB = OpInfo<FB>;
    constexpr int A_BYTES = BM * IA::kb, B_BYTES = BN * IB::kb;
    constexpr int NA = A_BYTES / 16 / NT, NB = B_BYTES / 16 / NT;  // chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (A_BYTES + B_BYTES)];

    Tile t;
    if (!tile_of_block(g, t)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t lda = (FA == E2M1) ? g.K / 2 : g.K;  // bytes per row
    const int64_t ldb = (FB == E2M1) ? g.K / 2 : g.K;
    const int64_t nks = g.K / BK;

    // global -> register staging of one K step
    uint4 ra[NA], rb[NB];
    auto gload = [&](int64_t ks) {
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int c = tid + i * NT, r = c / IA::chunks, cc = c % IA::chunks;
            const int64_t m = t.m0 + r;
            ra[i] = (m < t.m_end) ? *reinterpret_cast<const uint4*>(g.A + m * lda + ks * IA::kb + cc * 16)
                                  : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int c = tid + i * NT, r = c / IB::chunks, cc = c % IB::chunks;
            const int64_t n = t.n0 + r;
            rb[i] = (n < g.N) ? *reinterpret_cast<const uint4*>(t.B + n * ldb + ks * IB::kb + cc * 16)
                              : make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int buf) {
        uint8_t* la = lds + buf * (A_BYTES + B_BYTES);
        uint8_t* lb = la + A_BYTES;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int c = tid + i * NT, r = c / IA::chunks, cc = c % IA::chunks;
            *reinterpret_cast<uint4*>(la + lds_off<FA>(r, cc)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int c = tid + i * NT, r = c / IB::chunks, cc = c % IB::chunks;
            *reinterpret_cast<uint4*>(lb + lds_off<FB>(r, cc)) = rb[i];
        }
    };
    // scale bytes of this lane's 4 A fragments and 4 B fragments
    const int q = lane >> 4;
    uint32_t sa[4], sb[4], sa_n[4], sb_n[4];
    auto sload = [&](int64_t ks, uint32_t (&da)[4], uint32_t (&db)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            da[i] = scale_byte((const uint8_t*)g.sA, g.ma, t.m0 + wm * 64 + i * 16 + (lane & 15), t.m_end, g.K, ks, q);
            db[i] = scale_byte(t.sB, g.mb, t.n0 + wn * 64 + i * 16 + (lane & 15), g.N, g.K, ks, q);
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    gload(0);
    sload(0, sa, sb);
    sstore(0);
    __syncthreads();

    for (int64_t ks = 0; ks < nks; ++ks) {
        const int buf = (int)(ks & 1);
        if (ks + 1 < nks) {
            gload(ks + 1);
            sload(ks + 1, sa_n, sb_n);
        }
        const uint8_t* la = lds + buf * (A_BYTES + B_BYTES);
        const uint8_t* lb = la + A_BYTES;
        v8i fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 64 + i * 16 + (lane & 15);
            if constexpr (FA == E2M1) {
                const uint4 x = *reinterpret_cast<const uint4*>(la + lds_off<FA>(r, q));
                fa[i] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            } else {
                const uint4 x = *reinterpret_cast<const uint4*>(la + lds_off<FA>(r, q));
                const uint4 y = *reinterpret_cast<const uint4*>(la + lds_off<FA>(r, 4 + q));
                fa[i] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = wn * 64 + j * 16 + (lane & 15);
            if constexpr (FB == E2M1) {
                const uint4 x = *reinterpret_cast<const uint4*>(lb + lds_off<FB>(r, q));
                fb[j] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
            } else {
                const uint4 x = *reinterpret_cast<const uint4*>(lb + lds_off<FB>(r, q));
                const uint4 y = *reinterpret_cast<const uint4*>(lb + lds_off<FB>(r, 4 + q));
                fb[j] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fa[i], fb[j], acc[i][j], IA::code, IB::code,
                                                                             0, (int)sa[i], 0, (int)sb[j]);
        if (ks + 1 < nks) {
            sstore(buf ^ 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa[i] = sa_n[i];
                sb[i] = sb_n[i];
            }
        }
        __syncthreads();
    }

    // epilogue: per-tensor factors, store fp32 or bf16
    float alpha = 1.0f;
    if (g.ma == 0) alpha *= ((const float*)g.sA)[0];
    if (g.mb == 0) alpha *= ((const float*)g.sB)[0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = t.n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = t.m0 + wm * 64 + i * 16 + 4 * q + r;
                if (row < t.m_end && col < g.N) {
                    const float v = acc[i][j][r] * alpha;
                    if (g.out == 0) {
                        ((float*)g.C)[row * g.ldc + col] = v;
                    } else {
                        const uint32_t u = as_uint(v);
                        // round to nearest even (NaN kept quiet)
                        const uint32_t rb16 = ((u & 0x7FFFFFFFu) > 0x7F800000u)
                                                  ? ((u >> 16) | 0x40u)
                                                  : ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                        ((uint16_t*)g.C)[row * g.ldc + col] = (uint16_t)rb16;
                    }
                }
            }
        }
}

template <int FA, int FB>
static void launch_t(const GemmArgs& a, hipStream_t st) {
    const int64_t ntn = (a.N + BN - 1) / BN;
    int64_t ntm;
    if (a.group_off == nullptr) ntm = (a.M + BM - 1) / BM;
    else ntm = (a.M + BM - 1) / BM + a.G;  // every group may waste one partial tile
    const int64_t nblk = ntm * ntn;
    hipLaunchKernelGGL((k_gemm<FA, FB>), dim3((unsigned)nblk), dim3(NT), 0, st, a);
}

hipError_t launch_scaled_gemm(const GemmArgs& a, hipStream_t st) {
    switch (a.fa * 3 + a.fb) {
    case E4M3 * 3 + E4M3: launch_t<E4M3, E4M3>(a, st); break;
    case E4M3 * 3 + E5M2: launch_t<E4M3, E5M2>(a, st); break;
    case E4M3 * 3 + E2M1: launch_t<E4M3, E2M1>(a, st); break;
    case E5M2 * 3 + E4M3: launch_t<E5M2, E4M3>(a, st); break;
    case E5M2 * 3 + E5M2: launch_t<E5M2, E5M2>(a, st); break;
    case E5M2 * 3 + E2M1: launch_t<E5M2, E2M1>(a, st); break;
    case E2M1 * 3 + E4M3: launch_t<E2M1, E4M3>(a, st); break;
    case E2M1 * 3 + E5M2: launch_t<E2M1, E5M2>(a, st); break;
    case E2M1 * 3 + E2M1: launch_t<E2M1, E2M1>(a, st); break;
    }
    return hipGetLastError();
}

}  // namespace mxq
