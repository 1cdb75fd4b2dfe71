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
// Operand layout of the 32x32x64 scaled MFMA (pinned on the device with
// one-instruction tests): lane l supplies row l % 32 and the E8M0 scale of
// K block g = l / 32 (32 elements each).  An FP8 lane holds 32 codes as two
// 16-byte halves: byte j sits at K = 32 * (j / 16) + 16 * g + j % 16.  An
// FP4 lane holds K = 32 * g .. +31 in 16 bytes, element 2i in the low nibble
// of byte i.  Accumulator lane l, register r is row 8 * (r / 4) + 4 * g +
// r % 4, column l % 32.  The instruction's op_sel picks which byte of the
// 32-bit scale operand is used.
#include <utility>

#include "common.h"
#include "launch.h"

namespace mxq {

constexpr int BK = 128;  // K step in elements
constexpr int NT = 256;  // 4 waves in a 2 x 2 grid, each owning a (BM/2) x (BN/2) sub-tile

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

// Map this block to an output tile.  Dense: blocks are dispatched round-robin
// over the 8 XCDs, so consecutive logical tiles are first gathered onto one
// XCD (sharing its L2), then ordered GM tile-rows at a time.  Grouped: the
// m-tiles of all groups, found by scanning the device offsets.
template <int BM, int BN>
__device__ __forceinline__ bool tile_of_block(const GemmArgs& g, Tile& t) {
    const int64_t ntn = (g.N + BN - 1) / BN;
    int64_t bid = blockIdx.x;
    t.B = g.B;
    t.sB = (const uint8_t*)g.sB;
    if (g.group_off == nullptr) {
        const int64_t ntm = (g.M + BM - 1) / BM;
        const int64_t nblk = ntm * ntn;
        if (nblk % 8 == 0) bid = (bid % 8) * (nblk / 8) + bid / 8;
        constexpr int64_t GM = 4;
        const int64_t per_group = GM * ntn;
        const int64_t grp = bid / per_group;
        const int64_t first = grp * GM;
        const int64_t gs = (ntm - first) < GM ? (ntm - first) : GM;
        const int64_t in = bid - grp * per_group;
        t.m0 = (first + in % gs) * BM;
        t.m_end = g.M;
        t.n0 = (in / gs) * BN;
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

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Raw buffer resource over `bytes` bytes at `p` (gfx9 data format word;
// reads at or past `bytes` return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS copy of one operand tile for K step ks, straight into LDS
// (buffer_load_dwordx4 ... lds: lane L of a wave fills bytes 16L..16L+15 of
// the wave's 1 KiB destination).  Buffer loads are counted by vmcnt alone,
// so LDS reads issued before them can still be waited for one by one.  Each
// lane picks the global chunk that belongs at its LDS slot, so the LDS image
// carries the XOR swizzle of lds_off().  Rows at or past `row_end` read the
// last valid row instead: they only feed output rows (or columns) that are
// never stored.  The per-lane offset is fixed; the K step enters as the
// wave-uniform offset (operands stay below 4 GiB).
template <int F, int ROWS>
struct TileLoader {
    static constexpr int KB = OpInfo<F>::kb, CH = OpInfo<F>::chunks;
    static constexpr int NCHUNK = ROWS * KB / 1024;  // 1 KiB pieces per tile
    static constexpr int PER_WAVE = NCHUNK / 4;
    static_assert(NCHUNK % 4 == 0, "tile must split over 4 waves");
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t off[PER_WAVE];  // per-lane byte offset of its chunk within the operand at K step 0
    __device__ __forceinline__ void init(const uint8_t* base, int64_t bytes, int64_t ld, int64_t row0,
                                         int64_t row_end, int wave, int lane) {
        rsrc = make_rsrc(base, bytes);
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int cid = wave + 4 * i;
            const int o = cid * 1024 + lane * 16;
            const int r = o / KB, p = (o % KB) / 16;
            const int sw = (CH == 8) ? (r & 7) : ((r >> 1) & 3);
            int64_t row = row0 + r;
            row = row < row_end ? row : row_end - 1;
            off[i] = (uint32_t)(row * ld + ((p ^ sw) << 4));
        }
    }
    __device__ __forceinline__ void issue(int64_t ks, uint8_t* lds_tile, int wave) const {
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds_tile + (wave + 4 * i) * 1024), 16,
                                                     (int)off[i], (int)(uint32_t)(ks * KB), 0, 0);
    }
};

// Global -> LDS copy of one scale dword per tile row for K step ks
// (buffer_load_dword ... lds: lane L fills bytes 4L..4L+3).  BLK32: the four
// E8M0 bytes of the step's four 32-blocks (4-aligned because K % 128 == 0).
// BLK128: the aligned dword that contains the step's byte; the reader picks
// byte (row * pitch + ks) % 4.  Per-tensor operands load a dword that is
// never used, so that every mode runs the same straight-line step.
template <int ROWS>
struct ScaleLoader {
    static constexpr int NLOAD = ROWS / 64;  // 64 rows per wave load
    static_assert(NLOAD % 4 == 0 || NLOAD == 2, "scale rows per wave");
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t off[(NLOAD + 3) / 4];
    uint32_t kmul;  // bytes per K step: 4 (BLK32), 1 (BLK128), 0 (per-tensor)
    uint32_t mask;  // ~3 for BLK128 (aligned dword), else ~0
    __device__ __forceinline__ void init(int mode, const void* s, int64_t K, int64_t rows, int64_t row0,
                                         int64_t row_end, int wave, int lane) {
        const int64_t pitch = (mode == 1) ? K / 32 : (mode == 2 ? K / 128 : 0);
        kmul = mode == 1 ? 4u : (mode == 2 ? 1u : 0u);
        mask = mode == 2 ? ~3u : ~0u;
        // a per-tensor operand has a 4-byte float behind `s`: offset 0 is valid
        rsrc = make_rsrc(s, mode == 0 ? 4 : rows * pitch);
#pragma unroll
        for (int i = 0; i < (NLOAD + 3) / 4; ++i) {
            int64_t row = row0 + (wave + 4 * i) * 64 + lane;
            row = row < row_end ? row : row_end - 1;
            off[i] = (uint32_t)(row * pitch);
        }
    }
    __device__ __forceinline__ void issue(int64_t ks, uint8_t* lds_s, int wave) const {
#pragma unroll
        for (int i = 0; i < (NLOAD + 3) / 4; ++i) {
            if (NLOAD % 4 == 0 || wave + 4 * i < NLOAD) {
                const uint32_t o = (off[i] + (uint32_t)ks * kmul) & mask;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds_s + (wave + 4 * i) * 256), 4,
                                                         (int)o, 0, 0, 0);
            }
        }
    }
};

template <int FA, int FB, int BM, int BN>
__global__ void __launch_bounds__(NT, 1) k_gemm(const GemmArgs g) {
    using IA = OpInfo<FA>;
    using IB = OpInfo<FB>;
    constexpr int A_BYTES = BM * IA::kb, B_BYTES = BN * IB::kb;
    constexpr int STAGE = A_BYTES + B_BYTES + 4 * (BM + BN);  // tiles + scale dwords
    constexpr int FM = BM / 64, FN = BN / 64;                  // 32-row fragments per wave
    constexpr int WN = BN / 2;                                 // columns of a wave's sub-tile
    constexpr int EPI = 4 * 32 * WN * 4;                       // epilogue bands, fp32
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE > EPI ? 2 * STAGE : EPI];  // two stages

    Tile t;
    if (!tile_of_block<BM, BN>(g, t)) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t lda = (FA == E2M1) ? g.K / 2 : g.K;  // bytes per row
    const int64_t ldb = (FB == E2M1) ? g.K / 2 : g.K;
    const int64_t nks = g.K / BK;
    const int gq = lane >> 5;  // K block of the instruction this lane feeds
    const int64_t pA = g.ma == 1 ? g.K / 32 : g.K / 128;  // scale pitch of the operand rows
    const int64_t pB = g.mb == 1 ? g.K / 32 : g.K / 128;
    // this lane's fragment rows, as offsets within the tile
    const int rA = wm * (BM / 2) + (lane & 31), rB = wn * (BN / 2) + (lane & 31);

    // operand extents for the buffer resources (validated below 4 GiB); a
    // grouped A has M = total rows, whatever its offsets claim
    const int64_t a_rows = g.M;
    TileLoader<FA, BM> ldA;
    TileLoader<FB, BN> ldB;
    ldA.init(g.A, a_rows * lda, lda, t.m0, t.m_end, wave, lane);
    ldB.init(t.B, g.N * ldb, ldb, t.n0, g.N, wave, lane);
    ScaleLoader<BM> lsA;
    ScaleLoader<BN> lsB;
    lsA.init(g.ma, g.sA, g.K, a_rows, t.m0, t.m_end, wave, lane);
    lsB.init(g.mb, t.sB, g.K, g.N, t.n0, g.N, wave, lane);
    auto issue = [&](int64_t ks, uint8_t* st) {
        ldA.issue(ks, st, wave);
        ldB.issue(ks, st + A_BYTES, wave);
        lsA.issue(ks, st + A_BYTES + B_BYTES, wave);
        lsB.issue(ks, st + A_BYTES + B_BYTES + 4 * BM, wave);
    };
    // Operand fragment for K half h of the step (64 K elements): rows r..r+31.
    auto frag = [&](const uint8_t* base, int r, int h, auto info) -> v8i {
        using I = decltype(info);
        if constexpr (I::kb == 64) {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<E2M1>(r, 2 * h + gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<E4M3>(r, 4 * h + gq));
            const uint4 y = *reinterpret_cast<const uint4*>(base + lds_off<E4M3>(r, 4 * h + 2 + gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        }
    };
    // Scale operand of a fragment row: the staged dword shifted so that the
    // byte for K half h sits at byte 2h (BLK32: blocks 2h + gq; BLK128: the
    // step's byte copied to bytes 0 and 2).  Per-tensor: 127 (x1) everywhere.
    // The mode is folded into a shift, mask, multiplier and OR value chosen
    // once, so the per-step code has no branch:
    //   s = (((d >> ((sh + 8 ks k) & 31)) & mask) * mul) | orv
    struct SMode { uint32_t k, mask, mul, orv; };
    auto smode = [](int mode) -> SMode {
        if (mode == 0) return {0u, 0u, 0u, 0x7F7F7F7Fu};
        if (mode == 1) return {0u, ~0u, 1u, 0u};
        return {1u, 0xFFu, 0x10001u, 0u};
    };
    const SMode smA = smode(g.ma), smB = smode(g.mb);
    uint32_t shA[FM], shB[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
        shA[i] = g.ma == 1 ? 8u * gq : 8u * (uint32_t)(((t.m0 + rA + 32 * i) * pA) & 3);
#pragma unroll
    for (int j = 0; j < FN; ++j)
        shB[j] = g.mb == 1 ? 8u * gq : 8u * (uint32_t)(((t.n0 + rB + 32 * j) * pB) & 3);
    auto sreg = [&](const SMode& m, const uint8_t* lds_s, int r, uint32_t sh, int64_t ks) -> uint32_t {
        const uint32_t d = *reinterpret_cast<const uint32_t*>(lds_s + r * 4);
        return (((d >> ((sh + 8u * (uint32_t)ks * m.k) & 31u)) & m.mask) * m.mul) | m.orv;
    };

    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

    // One K step from stage `cur`: read the first K half's fragments; run the
    // first half's MFMAs while the second half's fragments are read; then, with
    // every read of `cur` issued, start step ks+1 landing in `nxt` (last read
    // before the previous barrier) and run the second half's MFMAs.  No LDS
    // read is ever ordered after an outstanding LDS-bound load.
    auto step = [&](int64_t ks, const uint8_t* cur, uint8_t* nxt, auto more) {
        const uint8_t* la = cur;
        const uint8_t* lb = cur + A_BYTES;
        const uint8_t* lsa = cur + A_BYTES + B_BYTES;
        const uint8_t* lsb = lsa + 4 * BM;
        uint32_t sa[FM], sb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) sa[i] = sreg(smA, lsa, rA + 32 * i, shA[i], ks);
#pragma unroll
        for (int j = 0; j < FN; ++j) sb[j] = sreg(smB, lsb, rB + 32 * j, shB[j], ks);
        v8i fa[2][FM], fb[2][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[0][i] = frag(la, rA + 32 * i, 0, IA{});
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = frag(lb, rB + 32 * j, 0, IB{});
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[1][i] = frag(la, rA + 32 * i, 1, IA{});
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[1][j] = frag(lb, rB + 32 * j, 1, IB{});
        // every read of `cur` is issued: start step ks+1 landing in `nxt` (its
        // last reads were before the previous barrier), so the loads have the
        // whole step's MFMAs to land
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(more)::value) issue(ks + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        static_for<FN>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            static_for<FM>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[0][i], fb[0][j], acc[i][j], IA::code,
                                                                            IB::code, 0, (int)sa[i], 0, (int)sb[j]);
            });
        });
        static_for<FN>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            static_for<FM>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[1][i], fb[1][j], acc[i][j], IA::code,
                                                                            IB::code, 2, (int)sa[i], 2, (int)sb[j]);
            });
        });
        __builtin_amdgcn_sched_barrier(0);  // the wait below must follow every MFMA of the step
        __builtin_amdgcn_s_waitcnt(0);      // this thread's LDS-bound loads for step ks+1 have landed
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
    };

    issue(0, lds);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int64_t ks = 0; ks + 1 < nks; ++ks) {
        const int cur = (int)(ks & 1);
        step(ks, lds + cur * STAGE, lds + (cur ^ 1) * STAGE, std::true_type{});
    }
    step(nks - 1, lds + ((nks - 1) & 1) * STAGE, lds, std::false_type{});

    // Epilogue: per-tensor factors, then fp32 or bf16 (round to nearest even).
    // Each wave stages one 32-row band of its sub-tile at a time in LDS (the
    // operand stages are free once the loop's last barrier has passed) and
    // writes it back as whole rows of 16-byte stores.
    float alpha = 1.0f;
    if (g.ma == 0) alpha *= ((const float*)g.sA)[0];
    if (g.mb == 0) alpha *= ((const float*)g.sB)[0];
    const int64_t row_base = t.m0 + wm * (BM / 2), col_base = t.n0 + wn * WN;
    // rows and columns of this wave's sub-tile that exist in C
    const int mlim = (int)min(t.m_end - row_base, (int64_t)(BM / 2));
    const int nlim = (int)min(g.N - col_base, (int64_t)WN);
    auto store_tile = [&](auto tag) {
        using T = decltype(tag);
        constexpr int PER = 16 / (int)sizeof(T);  // elements per 16-byte chunk
        constexpr int CPR = WN / PER;             // chunks per row
        constexpr int RPI = 64 / CPR;             // rows per wave-wide read
        T* band = reinterpret_cast<T*>(lds + wave * (32 * WN * 4));
        T* cw = (T*)g.C + row_base * g.ldc + col_base;
        const int cc = (lane % CPR) * PER;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            __syncthreads();  // the previous band has been read back
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = acc[i][j][r] * alpha;
                    T o;
                    if constexpr (sizeof(T) == 4) {
                        o = v;
                    } else {
                        const uint32_t u = as_uint(v);
                        const uint32_t rn = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                        o = (T)(((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : rn);
                    }
                    band[(8 * (r / 4) + 4 * gq + (r % 4)) * WN + 32 * j + (lane & 31)] = o;
                }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 32 / RPI; ++q) {
                const int rr = 32 * i + q * RPI + lane / CPR;
                const uint4 d = *reinterpret_cast<const uint4*>(band + (q * RPI + lane / CPR) * WN + cc);
                if (rr < mlim) {
                    T* dst = cw + (int64_t)rr * g.ldc + cc;
                    if (cc + PER <= nlim) {
                        *reinterpret_cast<uint4*>(dst) = d;
                    } else {
                        const T* e = reinterpret_cast<const T*>(&d);
#pragma unroll
                        for (int k = 0; k < PER; ++k)
                            if (cc + k < nlim) dst[k] = e[k];
                    }
                }
            }
        }
    };
    if (g.out == 0)
        store_tile(float{});
    else
        store_tile(uint16_t{});
}

template <int FA, int FB, int BM, int BN>
static hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
    const int64_t ntn = (a.N + BN - 1) / BN;
    const int64_t ntm = (a.group_off == nullptr) ? (a.M + BM - 1) / BM : (a.M + BM - 1) / BM + a.G;
    hipLaunchKernelGGL((k_gemm<FA, FB, BM, BN>), dim3((unsigned)(ntm * ntn)), dim3(NT), 0, st, a);
    return hipGetLastError();
}

// Tile choice: the largest tiles (most operand reuse per LDS byte) unless
// they leave most of the 256 CUs idle.
template <int FA, int FB>
static hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
    const int64_t rows = a.group_off ? (a.M / (a.G > 0 ? a.G : 1)) : a.M;
    if (rows <= 160 || a.N < 256) return launch_tile<FA, FB, 128, 128>(a, st);
    const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (a.group_off == nullptr && t256 < 192) return launch_tile<FA, FB, 128, 128>(a, st);
    if (a.group_off != nullptr) return launch_tile<FA, FB, 128, 256>(a, st);
    return launch_tile<FA, FB, 256, 256>(a, st);
}

hipError_t launch_scaled_gemm(const GemmArgs& a, hipStream_t st) {
    switch (a.fa * 3 + a.fb) {
    case E4M3 * 3 + E4M3: return launch_t<E4M3, E4M3>(a, st);
    case E4M3 * 3 + E5M2: return launch_t<E4M3, E5M2>(a, st);
    case E4M3 * 3 + E2M1: return launch_t<E4M3, E2M1>(a, st);
    case E5M2 * 3 + E4M3: return launch_t<E5M2, E4M3>(a, st);
    case E5M2 * 3 + E5M2: return launch_t<E5M2, E5M2>(a, st);
    case E5M2 * 3 + E2M1: return launch_t<E5M2, E2M1>(a, st);
    case E2M1 * 3 + E4M3: return launch_t<E2M1, E4M3>(a, st);
    case E2M1 * 3 + E5M2: return launch_t<E2M1, E5M2>(a, st);
    case E2M1 * 3 + E2M1: return launch_t<E2M1, E2M1>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxq
