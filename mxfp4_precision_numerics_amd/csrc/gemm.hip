// gemm.hip - FP8 / MX block-scaled GEMM (dense and ragged grouped) on
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation.
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
//
// Pipeline.  K runs in halves of 64 elements (one MFMA deep).  A block
// (4 waves, 2 x 2 over the tile) keeps a ring of four LDS slots, one K half
// of the A and B tiles each, and two slots of scale dwords (one per K step of
// 128).  In half j every wave, after one barrier:
//   * runs the half's MFMAs from fragments already in registers,
//   * reads the next half's fragments (slot j+1, landed) into the other
//     register set, interleaved with the MFMAs,
//   * starts the global->LDS copy of half j+3 into the slot read in half j-2.
// So copies get two halves to land and LDS reads one half, both hidden
// behind MFMAs.  The copies are buffer_load ... lds instructions issued from
// inline assembly: the compiler's wait insertion cannot see them and so
// adds no conservative waits; the kernel waits for them explicitly (vmcnt)
// before the barrier that publishes a slot.
#include <utility>

#include "common.h"
#include "launch.h"

namespace mxq {

constexpr int NT = 256;  // 4 waves in a 2 x 2 grid, each owning a (BM/2) x (BN/2) sub-tile

template <int F> struct OpInfo {
    static constexpr int kh = (F == E2M1) ? 32 : 64;  // bytes per row per K half
    static constexpr int chunks = kh / 16;             // 16-byte chunks per row per half
    static constexpr int code = FmtInfo<F>::mfma_code;
};

// LDS byte offset of 16-byte chunk `c` of row `r` within one half-slot (XOR
// swizzle so that the fragment reads of 8 consecutive rows hit distinct
// 16-byte bank groups).
template <int F> __device__ __forceinline__ int lds_off(int r, int c) {
    constexpr int CH = OpInfo<F>::chunks;
    const int sw = (CH == 4) ? ((r >> 1) & 3) : ((r >> 2) & 1);
    return r * OpInfo<F>::kh + ((c ^ sw) << 4);
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

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// A block-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ int64_t uni64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Raw buffer resource over `bytes` bytes at `p` (stride 0, gfx9 data format
// word; loads at or past `bytes` return zero).
__device__ __forceinline__ v4u make_rsrc(const void* p, int64_t bytes) {
    const uint64_t a = (uint64_t)p;
    return v4u{(unsigned)a, (unsigned)(a >> 32) & 0xFFFFu, (unsigned)(uint32_t)bytes, 0x00020000u};
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LDS and export counters not waited for).
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 32-bit LDS address of a __shared__ object (what M0 takes below).
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}
// Global -> LDS copies: lane L writes bytes [size*L, size*(L+1)) at the
// wave-uniform LDS address `dst`, from buffer offset voff + soff.
__device__ __forceinline__ void dma16(const v4u& rsrc, uint32_t voff, uint32_t soff, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 ::"v"(voff), "s"(rsrc), "s"(dst), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const v4u& rsrc, uint32_t voff, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dword %0, %2, 0 offen lds"
                 ::"v"(voff), "s"(dst), "s"(rsrc) : "memory", "m0");
}

// One K half of an operand tile into a half-slot: each wave copies PER_WAVE
// 1 KiB pieces (piece i of wave w covers tile rows (w + 4i) * RP ...); lane
// L's position holds the global chunk that belongs there under the lds_off()
// swizzle, which is the same for every piece.  Rows past the operand's end
// (a partial last tile) fall outside the buffer's range and read zero; in a
// grouped operand they read the next group's rows.  Either way they only feed
// outputs that are never stored.  The per-lane offset of piece 0 is kept;
// piece i adds i * RP * 4 rows, the K half enters as the uniform offset
// (operands stay below 4 GiB).
template <int F, int ROWS>
struct TileLoader {
    static constexpr int KH = OpInfo<F>::kh, CH = OpInfo<F>::chunks;
    static constexpr int PER_WAVE = ROWS * KH / 1024 / 4;
    static constexpr int RP = 1024 / KH;  // rows per 1 KiB piece
    static_assert(PER_WAVE >= 1 && ROWS * KH % 4096 == 0, "tile half must split over 4 waves");
    v4u rsrc;
    uint32_t off0, step;  // lane offset of piece 0; bytes between pieces
    __device__ __forceinline__ void init(const uint8_t* base, int64_t bytes, int64_t ld, int64_t row0, int wave,
                                         int lane) {
        rsrc = make_rsrc(base, bytes);
        const int o = wave * 1024 + lane * 16;
        const int r = o / KH, p = (o % KH) / 16;
        const int sw = (CH == 4) ? ((r >> 1) & 3) : ((r >> 2) & 1);
        off0 = (uint32_t)((row0 + r) * ld + ((p ^ sw) << 4));
        step = (uint32_t)(4 * RP * ld);
    }
    __device__ __forceinline__ void issue(int i, int64_t half, uint32_t slot, int wave) const {
        dma16(rsrc, off0 + (uint32_t)i * step, (uint32_t)(half * KH), slot + (uint32_t)(wave + 4 * i) * 1024u);
    }
};

// One scale dword per tile row for a K step of 128 (one copy per wave).
// BLK32: the four E8M0 bytes of the step's four 32-blocks (4-aligned since
// K % 128 == 0).  BLK128: the aligned dword that contains the step's byte;
// the reader picks byte (row * pitch + ks) % 4.  Per-tensor operands load the
// dword at offset 0 of their float and never use it, so that every mode runs
// the same code.  With 128 rows, waves w and w+2 copy the same rows.  Rows
// past the end read zero or the next group's scales, as for the tiles.
template <int ROWS>
struct ScaleLoader {
    static_assert(ROWS == 128 || ROWS == 256, "scale rows");
    v4u rsrc;
    uint32_t off, kmul, mask;
    int dst;  // byte offset of this wave's 64 dwords within the scale slot
    __device__ __forceinline__ void init(int mode, const void* s, int64_t K, int64_t rows, int64_t row0, int wave,
                                         int lane) {
        const int64_t pitch = (mode == 1) ? K / 32 : (mode == 2 ? K / 128 : 0);
        kmul = mode == 1 ? 4u : (mode == 2 ? 1u : 0u);
        mask = mode == 2 ? ~3u : ~0u;
        rsrc = make_rsrc(s, mode == 0 ? 4 : rows * pitch);
        const int r = (wave * 64) % ROWS;
        dst = r * 4;
        off = (uint32_t)((row0 + r + lane) * pitch);
    }
    __device__ __forceinline__ void issue(int64_t ks, uint32_t slot) const {
        dma4(rsrc, (off + (uint32_t)ks * kmul) & mask, slot + (uint32_t)dst);
    }
};

template <int FA, int FB, int BM, int BN>
__global__ void __launch_bounds__(NT, 1) k_gemm(const GemmArgs g) {
    using IA = OpInfo<FA>;
    using IB = OpInfo<FB>;
    constexpr int A_H = BM * IA::kh, B_H = BN * IB::kh;  // bytes of one K half of each tile
    constexpr int SLOT = A_H + B_H;
    constexpr int SCB = 4 * (BM + BN);                     // scale dwords of one K step
    constexpr int FM = BM / 64, FN = BN / 64;              // 32-row fragments per wave
    constexpr int WN = BN / 2;                             // columns of a wave's sub-tile
    constexpr int NM = FM * FN;                            // MFMAs per half
    // separate arrays, so the slots are distinct objects to the compiler
    __shared__ __attribute__((aligned(16))) uint8_t s0[SLOT], s1[SLOT], s2[SLOT], s3[SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t c0[SCB], c1[SCB];

    Tile t;
    if (!tile_of_block<BM, BN>(g, t)) return;
    // the tile is the same for the whole block: keep it in scalar registers
    t.m0 = uni64(t.m0);
    t.m_end = uni64(t.m_end);
    t.n0 = uni64(t.n0);
    t.B = (const uint8_t*)uni64((int64_t)t.B);
    t.sB = (const uint8_t*)uni64((int64_t)t.sB);
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: LDS copy destinations stay scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t lda = (FA == E2M1) ? g.K / 2 : g.K;  // bytes per row
    const int64_t ldb = (FB == E2M1) ? g.K / 2 : g.K;
    const int64_t nks = g.K / 128, H = 2 * nks;         // K steps, K halves
    const int gq = lane >> 5;                            // K block of the instruction this lane feeds
    const int64_t pA = g.ma == 1 ? g.K / 32 : g.K / 128;  // scale pitch of the operand rows
    const int64_t pB = g.mb == 1 ? g.K / 32 : g.K / 128;
    const int rA = wm * (BM / 2) + (lane & 31), rB = wn * (BN / 2) + (lane & 31);

    // operand extents for the buffer resources (validated below 4 GiB); a
    // grouped A has M = total rows, whatever its offsets claim
    TileLoader<FA, BM> ldA;
    TileLoader<FB, BN> ldB;
    ldA.init(g.A, g.M * lda, lda, t.m0, wave, lane);
    ldB.init(t.B, g.N * ldb, ldb, t.n0, wave, lane);
    ScaleLoader<BM> lsA;
    ScaleLoader<BN> lsB;
    lsA.init(g.ma, g.sA, g.K, g.M, t.m0, wave, lane);
    lsB.init(g.mb, t.sB, g.K, g.N, t.n0, wave, lane);
    constexpr int TL = TileLoader<FA, BM>::PER_WAVE + TileLoader<FB, BN>::PER_WAVE;  // tile copies per half
    // copies of half h: TL, plus 2 scale copies when h is even (a new K step)
    constexpr int CNT_EVEN = TL + 2, CNT_ODD = TL;

    // Scale operand of a fragment row, from the staged dword: the byte for K
    // half h ends up at byte 2h (BLK32: blocks 2h + gq; BLK128: the step's
    // byte copied to bytes 0 and 2); per-tensor: 127 (x1) everywhere.  The
    // mode is folded into a shift, mask, multiplier and OR value chosen once:
    //   s = (((d >> ((sh + 8 ks k) & 31)) & mask) * mul) | orv
    struct SMode { uint32_t k, mask, mul, orv; };
    auto smode = [](int mode) -> SMode {
        if (mode == 0) return {0u, 0u, 0u, 0x7F7F7F7Fu};
        if (mode == 1) return {0u, ~0u, 1u, 0u};
        return {1u, 0xFFu, 0x10001u, 0u};
    };
    const SMode smA = smode(g.ma), smB = smode(g.mb);
    // (row * pitch) % 4 is the same for every fragment row of this lane: rows
    // differ by multiples of 32
    const uint32_t shA = g.ma == 1 ? 8u * gq : 8u * (uint32_t)(((t.m0 + rA) * pA) & 3);
    const uint32_t shB = g.mb == 1 ? 8u * gq : 8u * (uint32_t)(((t.n0 + rB) * pB) & 3);

    // register sets: fragments of two halves, scale operands of two K steps
    v8i fa[2][FM], fb[2][FN];
    uint32_t sa[2][FM], sb[2][FN];
    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};

    auto frag_a = [&](const uint8_t* slot, int i) -> v8i {
        const uint8_t* base = slot;
        const int r = rA + 32 * i;
        if constexpr (FA == E2M1) {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<E2M1>(r, gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<FA>(r, gq));
            const uint4 y = *reinterpret_cast<const uint4*>(base + lds_off<FA>(r, 2 + gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        }
    };
    auto frag_b = [&](const uint8_t* slot, int j) -> v8i {
        const uint8_t* base = slot + A_H;
        const int r = rB + 32 * j;
        if constexpr (FB == E2M1) {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<E2M1>(r, gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        } else {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<FB>(r, gq));
            const uint4 y = *reinterpret_cast<const uint4*>(base + lds_off<FB>(r, 2 + gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        }
    };
    auto sreg = [&](const SMode& m, uint32_t d, uint32_t sh, int64_t ks) -> uint32_t {
        return (((d >> ((sh + 8u * (uint32_t)ks * m.k) & 31u)) & m.mask) * m.mul) | m.orv;
    };

    // Copies for half h (clamped to the last half: a copy past the end lands
    // in a slot that is never read again), scale dwords with even halves.
    auto issue_tile = [&](int i, int64_t h, uint32_t slot) {
        const int64_t hc = h < H ? h : H - 1;
        if (i < TileLoader<FA, BM>::PER_WAVE)
            ldA.issue(i, hc, slot, wave);
        else
            ldB.issue(i - TileLoader<FA, BM>::PER_WAVE, hc, slot + (uint32_t)A_H, wave);
    };
    auto issue_scales = [&](int64_t ks, uint32_t cs) {
        const int64_t kc = ks < nks ? ks : nks - 1;
        lsA.issue(kc, cs);
        lsB.issue(kc, cs + 4u * BM);
    };

    // One half j.  P: register set holding half j (j % 2); SP: scale set of
    // its K step; CUR/NXT/FREE: slots of halves j, j+1 and j+3; RS: whether
    // half j+1 starts a K step (read its scale dwords from CS into set 1-SP
    // ... the set of step (j+1)/2); NS: whether half j+3 starts a K step
    // (copy its scales into CN).
    auto half = [&](int64_t j, auto P_, auto SP_, auto RS_, auto NS_, const uint8_t* nxt, uint32_t fre,
                    const uint8_t* cs, uint32_t cn) {
        constexpr int P = decltype(P_)::value, SP = decltype(SP_)::value;
        constexpr bool RS = decltype(RS_)::value, NS = decltype(NS_)::value;
        constexpr int Q = 1 - P;                 // register set being filled
        constexpr int SQ = RS ? 1 - SP : SP;     // scale set being filled (if RS)
        // wait for half j+1's copies (issued in half j-2); half j+2's may run on
        // (j has the parity of P; half j+2 has the parity of j)
        if constexpr (P == 0)
            __builtin_amdgcn_s_waitcnt(wait_vm(CNT_EVEN));
        else
            __builtin_amdgcn_s_waitcnt(wait_vm(CNT_ODD));
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        uint32_t da[FM], db[FN];
        if constexpr (RS) {
#pragma unroll
            for (int i = 0; i < FM; ++i) da[i] = *reinterpret_cast<const uint32_t*>(cs + (rA + 32 * i) * 4);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
                db[jj] = *reinterpret_cast<const uint32_t*>(cs + 4 * BM + (rB + 32 * jj) * 4);
        }
        static_for<NM>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            constexpr int i = k % FM, jj = k / FM;
            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[P][i], fb[P][jj], acc[i][jj], IA::code, IB::code, 2 * P, (int)sa[SP][i], 2 * P, (int)sb[SP][jj]);
            // next half's fragments, one per MFMA while they last
            if constexpr (k < FM) fa[Q][k] = frag_a(nxt, k);
            if constexpr (k >= FM && k < FM + FN) fb[Q][k - FM] = frag_b(nxt, k - FM);
            // copies of half j+3, one every other MFMA, scales last
            if constexpr (k % 2 == 1 && k / 2 < TL) issue_tile(k / 2, j + 3, fre);
            if constexpr (NS && k == NM - 1) issue_scales((j + 3) / 2, cn);
            __builtin_amdgcn_sched_barrier(0);
        });
        // copies that did not fit one per two MFMAs
        static_for<TL>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i >= NM / 2) issue_tile(i, j + 3, fre);
        });
        if constexpr (RS) {
            const int64_t ks = (j + 1) / 2;
#pragma unroll
            for (int i = 0; i < FM; ++i) sa[SQ][i] = sreg(smA, da[i], shA, ks);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) sb[SQ][jj] = sreg(smB, db[jj], shB, ks);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using BT = std::true_type;
    using BF = std::false_type;

    // prologue: halves 0, 1, 2 in flight; half 0 and step 0's scales read
    const uint32_t L0 = lds_addr(s0), L1 = lds_addr(s1), L2 = lds_addr(s2), L3 = lds_addr(s3);
    const uint32_t LC0 = lds_addr(c0), LC1 = lds_addr(c1);
    issue_scales(0, LC0);
    static_for<TL>([&](auto ic) { issue_tile(decltype(ic)::value, 0, L0); });
    static_for<TL>([&](auto ic) { issue_tile(decltype(ic)::value, 1, L1); });
    issue_scales(1, LC1);
    static_for<TL>([&](auto ic) { issue_tile(decltype(ic)::value, 2, L2); });
    __builtin_amdgcn_s_waitcnt(wait_vm(CNT_ODD + CNT_EVEN));
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        fa[0][i] = frag_a(s0, i);
        sa[0][i] = sreg(smA, *reinterpret_cast<const uint32_t*>(c0 + (rA + 32 * i) * 4), shA, 0);
    }
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
        fb[0][jj] = frag_b(s0, jj);
        sb[0][jj] = sreg(smB, *reinterpret_cast<const uint32_t*>(c0 + 4 * BM + (rB + 32 * jj) * 4), shB, 0);
    }

    // halves in groups of four (two K steps): slots and register sets are
    // fixed per position in the group
    int64_t j = 0;
    for (; j + 4 <= H; j += 4) {
        half(j + 0, I0{}, I0{}, BF{}, BF{}, s1, L3, c1, LC0);
        half(j + 1, I1{}, I0{}, BT{}, BT{}, s2, L0, c1, LC0);
        half(j + 2, I0{}, I1{}, BF{}, BF{}, s3, L1, c0, LC1);
        half(j + 3, I1{}, I1{}, BT{}, BT{}, s0, L2, c0, LC1);
    }
    if (j < H) {  // an odd number of K steps leaves two halves
        half(j + 0, I0{}, I0{}, BF{}, BF{}, s1, L3, c1, LC0);
        half(j + 1, I1{}, I0{}, BT{}, BT{}, s2, L0, c1, LC0);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // every copy has landed before the slots are reused
    __syncthreads();

    // Epilogue: per-tensor factors, then fp32 or bf16 (round to nearest even).
    // Each wave stages bands of BR rows of its sub-tile in one slot (free
    // once the last barrier has passed) and writes them back as whole rows
    // of 16-byte stores.
    float alpha = 1.0f;
    if (g.ma == 0) alpha *= ((const float*)g.sA)[0];
    if (g.mb == 0) alpha *= ((const float*)g.sB)[0];
    const int64_t row_base = t.m0 + wm * (BM / 2), col_base = t.n0 + wn * WN;
    // rows and columns of this wave's sub-tile that exist in C
    const int mlim = (int)min(t.m_end - row_base, (int64_t)(BM / 2));
    const int nlim = (int)min(g.N - col_base, (int64_t)WN);
    uint8_t* const mine = wave == 0 ? s0 : wave == 1 ? s1 : wave == 2 ? s2 : s3;
    auto store_tile = [&](auto tag) {
        using T = decltype(tag);
        constexpr int PER = 16 / (int)sizeof(T);  // elements per 16-byte chunk
        constexpr int CPR = WN / PER;             // chunks per row
        constexpr int RPI = 64 / CPR;             // rows per wave-wide read
        constexpr int BR = (32 * WN * (int)sizeof(T) <= SLOT) ? 32 : (16 * WN * (int)sizeof(T) <= SLOT ? 16 : 8);
        static_assert(BR * WN * (int)sizeof(T) <= SLOT && BR % RPI == 0, "epilogue band");
        constexpr int RB = BR / 2;                // accumulator registers per band (8 rows <-> 4 registers)
        T* band = reinterpret_cast<T*>(mine);
        T* cw = (T*)g.C + row_base * g.ldc + col_base;
        const int cc = (lane % CPR) * PER;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int b = 0; b < 32 / BR; ++b) {
#pragma unroll
                for (int jj = 0; jj < FN; ++jj)
#pragma unroll
                    for (int r = RB * b; r < RB * (b + 1); ++r) {
                        const float v = acc[i][jj][r] * alpha;
                        T o;
                        if constexpr (sizeof(T) == 4) {
                            o = v;
                        } else {
                            const uint32_t u = as_uint(v);
                            const uint32_t rn = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
                            o = (T)(((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : rn);
                        }
                        band[(8 * (r / 4) + 4 * gq + (r % 4) - BR * b) * WN + 32 * jj + (lane & 31)] = o;
                    }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < BR / RPI; ++q) {
                    const int br = q * RPI + lane / CPR;
                    const int rr = 32 * i + BR * b + br;
                    const uint4 d = *reinterpret_cast<const uint4*>(band + br * WN + cc);
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
                __syncthreads();
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
