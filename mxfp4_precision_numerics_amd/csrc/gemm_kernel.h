// gemm_kernel.h - FP8 / MX block-scaled GEMM (dense and ragged grouped) on
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation.  The kernel
// template and its tile choice; gemm_inst.hip instantiates it once per
// operand-format pair and gemm.hip dispatches on the formats.
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
// Pipeline.  K runs in halves of 64 elements (one MFMA deep), staged in
// ring units of whole 128-byte lines per row for operands of one kind (one
// K step for FP8 x FP8, two for FP4 x FP4) or of one half for mixed
// FP4 x FP8.  A block (4 waves, 2 x 2 over the tile) keeps a ring of
// NSL LDS slots of one unit of the A and B tiles each (two for 256 x 256
// FP8 tiles and for FP4 x FP4, four or eight where they fit), and two slots
// of scale dwords (a group of four K steps each).  In half j every wave:
//   * runs the half's MFMAs from fragments already in registers,
//   * reads the next half's fragments (landed) into the other register set,
//     interleaved with the MFMAs,
//   * in the last half of unit u, after a barrier, starts the global->LDS
//     copies of unit u + NSL into the slot unit u leaves.
// So copies get NSL - 1 units minus one half to land and LDS reads one
// half, both hidden behind MFMAs.  The copies are buffer_load ... lds
// instructions issued from inline assembly: the compiler's wait insertion
// cannot see them and so adds no conservative waits; the kernel waits for
// them explicitly (vmcnt) before the barrier that publishes a slot.
#pragma once
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

// LDS byte offset of 16-byte chunk `c` of row `r` in a slot whose rows hold
// RB bytes (128: eight chunks, 64: four, 32: two).  gfx950's LDS serves a ds_read_b128
// 16 lanes per clock from 64 four-byte banks (256 bytes), so 16 consecutive
// lanes (16 consecutive rows of a fragment) must land on 16 distinct 16-byte
// bank quads; the XOR swizzle on the row bits above those that already
// spread it gives each of the 16 rows its own quad (measured: 4 clocks per
// wave-wide read, against 8 without it).
template <int RB> __device__ __forceinline__ int swz(int r) {
    static_assert(RB == 128 || RB == 64 || RB == 32, "LDS row bytes");
    return (RB == 128) ? ((r >> 1) & 7) : (RB == 64) ? ((r >> 2) & 3) : ((r >> 3) & 1);
}
template <int RB> __device__ __forceinline__ int lds_off(int r, int c) {
    return r * RB + ((c ^ swz<RB>(r)) << 4);
}

struct Tile {
    int64_t m0, m_end, n0;
    const uint8_t* B;
    const uint8_t* sB;
};

// Map this block to an output tile.  Dense: blocks are dispatched round-robin
// over the 8 XCDs, so consecutive logical tiles are first gathered onto one
// XCD (sharing its L2), then ordered GM tile-rows at a time.  Grouped: the
// m-tiles of all groups, found by scanning the device offsets.  With the
// 320-row tiles (one per group) block b runs m-tile (b % 8) + 8 (b / (8 ntn))
// and n-tile (b / 8) % ntn: a group's n-tiles run on one XCD, one after
// another, and read the group's rows of A from that XCD's L2 (the launch
// rounds the m-tiles up to a multiple of 8).  That cut the C4 up-projection's
// fetch from 1.82 to 1.23 GB (time within 1%); for the 256-row tiles of the
// fused call it was 11% slower, so they keep the plain order.
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
    const int64_t tn = BM == 320 ? (bid >> 3) % ntn : bid % ntn;
    int64_t mt = BM == 320 ? (bid & 7) + 8 * ((bid >> 3) / ntn) : bid / ntn;
    for (int64_t gi = 0; gi < g.G; ++gi) {
        // offsets clamped to [0, M] (and each end to at least its start):
        // whatever the device offsets hold, no tile reaches a row outside C
        const int64_t o0 = g.group_off[gi], o1 = g.group_off[gi + 1];
        const int64_t r0 = o0 < 0 ? 0 : (o0 > g.M ? g.M : o0);
        const int64_t r1 = o1 < r0 ? r0 : (o1 > g.M ? g.M : o1);
        const int64_t nt = (r1 - r0 + BM - 1) / BM;
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
// The resource, destination and uniform offset are block-uniform; they are
// passed through readfirstlane so that they sit in scalar registers even
// where the compiler cannot prove uniformity (free where it can).
// STREAM marks the load non-temporal (nt): for bytes that no other tile
// reads, so that they do not push reused operand lines out of the L2.
__device__ __forceinline__ v4u uni(const v4u& r) {
    return v4u{(unsigned)__builtin_amdgcn_readfirstlane(r[0]), (unsigned)__builtin_amdgcn_readfirstlane(r[1]),
               (unsigned)__builtin_amdgcn_readfirstlane(r[2]), (unsigned)__builtin_amdgcn_readfirstlane(r[3])};
}
template <bool STREAM = false>
__device__ __forceinline__ void dma16(const v4u& rsrc, uint32_t voff, uint32_t soff, uint32_t dst) {
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen nt lds"
                     ::"v"(voff), "s"(uni(rsrc)), "s"(__builtin_amdgcn_readfirstlane(dst)),
                       "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                     ::"v"(voff), "s"(uni(rsrc)), "s"(__builtin_amdgcn_readfirstlane(dst)),
                       "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}


// One ring unit (RB bytes of K per row) of an operand tile into a slot:
// each wave copies PER_WAVE 1 KiB pieces (piece i of wave w covers tile rows
// (w + 4i) * RP ...); lane L's position holds the global chunk that belongs
// there under the lds_off() swizzle, which is the same for every piece.
// Rows past the operand's end (a partial last tile) fall outside the
// buffer's range and read zero; A's range ends at the end of the tile's
// group, so rows past a group read zero too, without memory traffic.
// Either way they only feed outputs that are never stored.
// The per-lane offset of piece 0 is kept; piece i adds i * RP * 4 rows.  The
// unit enters as the uniform offset (operands stay below 4 GiB), except with
// LANE_UNIT: the buffer's range check covers the per-lane offset only, and a
// unit that can run past the end of a row (FP4 x FP4 units of two K steps
// when K % 256 == 128) must be range-checked on the last row, so there the
// unit's offset is added to the per-lane offset.
//
// Gate/up tiles of the expert MLP (GU != 0; 128-byte rows), from operand
// rows row0 + .. of the gate half and of the up half (gu bytes further):
//  GU = 1, 256 rows: tile rows [64b, 64b + 64) come from gate rows
//    row0 + 64 (b / 2) + .. for even b and from the up rows of the same 64
//    intermediate columns for odd b (128 columns per tile, each wave column
//    holds gate and up of its own 64).  Piece i (8 rows) lies in block i / 2
//    at rows 32 (i % 2) .. of it.
//  GU = 2, 192 rows: tile rows [0, 96) are gate rows row0 .. row0 + 95,
//    rows [96, 192) the up rows of the same 96 intermediate columns.
//    Pieces 0-2 of a wave are gate rows, 3-5 the up rows 96 further on.
template <int RB, int ROWS, bool LANE_UNIT = false, int GU = 0, bool STREAM = false>
struct TileLoader {
    static constexpr int CH = RB / 16;
    static constexpr int PER_WAVE = ROWS * RB / 1024 / 4;
    static constexpr int RP = 1024 / RB;  // rows per 1 KiB piece
    static_assert(PER_WAVE >= 1 && ROWS * RB % 4096 == 0, "tile unit must split over 4 waves");
    static_assert(GU == 0 || (GU == 1 && RB == 128 && ROWS == 256) || (GU == 2 && RB == 128 && ROWS == 192),
                  "gate/up tiles are 256 or 192 rows of 128 bytes");
    v4u rsrc;
    uint32_t off0, step, gu;  // lane offset of piece 0; bytes between pieces; gate -> up
    __device__ __forceinline__ void init(const uint8_t* base, int64_t bytes, int64_t ld, int64_t row0, int wave,
                                         int lane, int64_t gu_rows = 0) {
        rsrc = make_rsrc(base, bytes);
        const int o = wave * 1024 + lane * 16;
        const int r = o / RB, p = (o % RB) / 16;
        off0 = (uint32_t)((row0 + r) * ld + ((p ^ swz<RB>(r)) << 4));
        step = (uint32_t)(4 * RP * ld);
        gu = (uint32_t)(gu_rows * ld);
    }
    __device__ __forceinline__ uint32_t piece(int i) const {
        if constexpr (GU == 1)
            return (uint32_t)(2 * (i / 4) + (i % 2)) * step + (uint32_t)((i / 2) & 1) * gu;
        else if constexpr (GU == 2)
            return (uint32_t)(i % 3) * step + (uint32_t)(i / 3) * gu;
        else
            return (uint32_t)i * step;
    }
    __device__ __forceinline__ void issue(int i, int64_t unit, uint32_t slot, int wave) const {
        const uint32_t u = (uint32_t)(unit * RB), dst = slot + (uint32_t)(wave + 4 * i) * 1024u;
        if constexpr (LANE_UNIT)
            dma16<STREAM>(rsrc, off0 + piece(i) + u, 0u, dst);
        else
            dma16<STREAM>(rsrc, off0 + piece(i), u, dst);
    }
};

// Scale bytes of a group of SG = 4 K steps, 16 bytes per tile row, copied in
// chunks of 64 rows (one copy each): NCH chunks over the 4 waves, NPW copies
// per wave (a wave with no chunk of its own copies one again: identical bytes
// to the same place).  BLK32: the row's 16 E8M0 bytes of the group's 16
// 32-blocks (4-aligned since K % 128 == 0).  BLK128: the 16 bytes from the
// aligned dword that holds the group's first byte, which covers the group's 4
// bytes.  Per-tensor operands load from offset 0 of their float and never use
// the data, so that every mode runs the same code.  Rows past the end read
// zero or the next group's scales, as for the tiles.  The buffer range check
// drops any dword that is not wholly inside the range, so a BLK128 array
// whose size is not a multiple of 4 gets a range rounded up to the end of its
// last aligned dword: the last row's bytes arrive, the (unused) padding bytes
// share that dword's page.  GU: the tile rows of TileLoader's gate/up modes
// (GU = 1: wave w copies block w; GU = 2: tile row r is a gate row below 96,
// else an up row).
constexpr int SG = 4;
template <int ROWS, int GU = 0>
struct ScaleLoader {
    static constexpr int NCH = (ROWS + 63) / 64;     // chunks of 64 rows
    static constexpr int NPW = (NCH + 3) / 4;        // copies per wave
    static constexpr int SROWS = NCH * 64;           // rows of staging room
    static_assert(ROWS % 32 == 0 && NCH >= 2, "scale rows");
    static_assert(GU == 0 || (GU == 1 && ROWS == 256) || (GU == 2 && ROWS == 192), "gate/up tiles are 256 or 192 rows");
    v4u rsrc;
    uint32_t off[NPW], kmul, mask;
    int dst[NPW];  // byte offsets of this wave's chunks within the operand's part of the slot
    __device__ __forceinline__ void init(int mode, const void* s, int64_t K, int64_t rows, int64_t row0, int wave,
                                         int lane, int64_t gu_rows = 0) {
        const int64_t pitch = (mode == 1) ? K / 32 : (mode == 2 ? K / 128 : 0);
        kmul = mode == 1 ? 4u : (mode == 2 ? 1u : 0u);
        mask = mode == 2 ? ~3u : ~0u;
        rsrc = make_rsrc(s, mode == 0 ? 4 : (rows * pitch + 3) & ~(int64_t)3);
#pragma unroll
        for (int c = 0; c < NPW; ++c) {
            const int ch = (wave + 4 * c) < NCH ? wave + 4 * c : wave % NCH;
            const int r = ch * 64;
            dst[c] = r * 16;
            int64_t grow = row0 + r + lane;
            if constexpr (GU == 1) grow = row0 + 64 * (wave / 2) + (wave % 2) * gu_rows + lane;
            if constexpr (GU == 2) grow = r + lane < 96 ? row0 + r + lane : row0 + gu_rows + r + lane - 96;
            off[c] = (uint32_t)(grow * pitch);
        }
    }
    __device__ __forceinline__ void issue(int64_t grp, uint32_t slot) const {
#pragma unroll
        for (int c = 0; c < NPW; ++c)
            dma16(rsrc, (off[c] + (uint32_t)(grp * SG) * kmul) & mask, 0u, slot + (uint32_t)dst[c]);
    }
};

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Byte k of d as the scale operand of the scaled converters, which read
// only their scale's exponent field, as an E8M0 byte (field 0 is 2^-127,
// field 255 NaN): the byte moved to bits 23..30.  The other bits are left
// as they fall: the converters ignore sign and mantissa (checked on the
// device for every FP8 byte, E4M3 and E5M2, against clean scales).
__device__ __forceinline__ float e8m0_field(uint32_t d, int k) {
    const int sh = 23 - 8 * k;
    return __builtin_bit_cast(float, sh >= 0 ? (d << sh) : (d >> -sh));
}

// Bytes 8q .. 8q+7 of an FP8 fragment (dwords 2q, 2q+1) as 8 bf16 values
// times `scale`.  The packed results are taken whole as 32-bit words.
template <int F> __device__ __forceinline__ v8bf to_bf16(const v8i& f, int q, float scale) {
    const uint32_t d0 = (uint32_t)f[2 * q], d1 = (uint32_t)f[2 * q + 1];
    uint32_t w[4];
    if constexpr (F == E4M3) {
        w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, false));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, scale, true));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, false));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, scale, true));
    } else {
        w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, scale, false));
        w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d0, scale, true));
        w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, scale, false));
        w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(d1, scale, true));
    }
    const uint4 u{w[0], w[1], w[2], w[3]};
    return __builtin_bit_cast(v8bf, u);
}

// Copy instructions a wave issues at the last half (position J mod 8) of a
// ring unit: TL tile copies, plus the NSC scale-group copies at position JS.
constexpr int copies_at(int J, int TL, int JS, int NSC) { return TL + ((J % 8 + 8) % 8 == JS ? NSC : 0); }
// Copies issued at the last halves of the NSL-2 units before the unit that
// ends at position J (still allowed in flight when that half waits for the
// next unit's copies); units are SU halves long.
constexpr int copies_after(int J, int NSL, int SU, int TL, int JS, int NSC) {
    int n = 0;
    for (int d = 1; d <= NSL - 2; ++d) n += copies_at(J - d * SU, TL, JS, NSC);
    return n;
}

// PRECISE: both operands FP8; each FP8 fragment is converted in registers to
// bf16 with its E8M0 scale folded in (exact: the converter rounds value x
// 2^e to bf16, which holds every FP8 value times any power of two inside
// bf16's range), then v_mfma_f32_32x32x16_bf16 accumulates the exact
// products in fp32.  Slower than the block-scaled FP8 MFMA, whose products
// are truncated to 13 fractional bits inside each run of 8 K positions.
//
// HF >= 0 (the expert MLP's up-projection; grouped, FP8 operands): B tiles
// hold gate and up rows of the same intermediate columns (TileLoader's
// gate/up modes).  The epilogue forms h = silu(gate) * up in binary32 and
// writes h MX block-32 quantized to format HF (q_out, s_out) instead of C.
//  * BN = 256 (GU = 1): 128 intermediate columns per tile; each wave's
//    accumulators hold gate in fragments 0, 1 and up of the same columns in
//    2, 3 (same lanes, same registers).
//  * BN = 192 with BM = 320 (GU = 2): 96 intermediate columns per tile; the
//    waves of column 0 hold gate, those of column 1 the up values of the
//    same columns, and the epilogue pairs them through LDS.
template <int FA, int FB, int BM, int BN, bool PRECISE = false, int HF = -1, bool SKIP = false, int SMS = -1>
__global__ void __launch_bounds__(NT, 1) k_gemm(const GemmArgs g) {
    static_assert(!PRECISE || (FA != E2M1 && FB != E2M1), "precise mode takes FP8 operands");
    constexpr int GU = HF < 0 ? 0 : (BN == 256 ? 1 : 2);
    static_assert(GU == 0 || ((BN == 256 || (BM == 320 && BN == 192)) && FA != E2M1 && FB != E2M1 && !PRECISE),
                  "gate/up epilogue configuration");
    constexpr int SM = BM / 2, SN = BN / 2;                // a wave's sub-tile (2 x 2 waves)
    using IA = OpInfo<FA>;
    using IB = OpInfo<FB>;
    // Ring unit: SU K halves.  Copies fetch RB contiguous bytes per row, and
    // partial-line copies cost the CU's address unit about as much as whole
    // ones, so operands of one kind stage whole 128-byte lines per row and
    // unit: one K step for FP8 x FP8, two for FP4 x FP4.  Mixed FP4 x FP8
    // stages one K half.
    constexpr bool SAME = (FA == E2M1) == (FB == E2M1);
    constexpr int SU = SAME ? (FA == E2M1 ? 4 : 2) : 1;
    constexpr int RBA = SU * IA::kh, RBB = SU * IB::kh;  // bytes per row per unit
    constexpr int A_H = BM * RBA, B_H = BN * RBB;        // bytes of one unit of each tile
    constexpr int SLOT = A_H + B_H;
    constexpr int SRA = ScaleLoader<BM>::SROWS, SRB = ScaleLoader<BN>::SROWS;
    constexpr int SCB = 16 * (SRA + SRB);                  // scale bytes of a group of SG K steps
    constexpr int FM = SM / 32, FN = SN / 32;              // 32-row fragments per wave
    constexpr int WN = SN;                                 // columns of a wave's sub-tile
    constexpr int NM = FM * FN;                            // MFMAs per half
    static_assert(SM % 32 == 0 && SN % 32 == 0, "sub-tiles of whole fragments");
    // ring slots: eight, four or two, the most that fit in LDS (a power of
    // two that divides the 8 / SU units of the unrolled group of eight halves)
    constexpr int LDS_BYTES = 160 * 1024;
    constexpr int NSL = (SU == 1 && 8 * SLOT + 2 * SCB <= LDS_BYTES) ? 8
                        : (SU <= 2 && 4 * SLOT + 2 * SCB <= LDS_BYTES ? 4 : 2);
    static_assert(NSL * SLOT + 2 * SCB <= LDS_BYTES, "ring must fit in LDS");
    constexpr int SLOT_MID = NSL >= 4 ? SLOT : 16;
    constexpr int SLOT_HI = NSL == 8 ? SLOT : 16;
    // separate arrays, so the slots are distinct objects to the compiler
    __shared__ __attribute__((aligned(16))) uint8_t s0[SLOT], s1[SLOT], s2[SLOT_MID], s3[SLOT_MID];
    __shared__ __attribute__((aligned(16))) uint8_t s4[SLOT_HI], s5[SLOT_HI], s6[SLOT_HI], s7[SLOT_HI];
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
    // SMS >= 0: both operands carry scales of that mode, known at compile
    // time.  BLK32 (1): the scale operands are the staged dwords themselves,
    // with no per-step mode arithmetic; per-tensor (0): no scale bytes are
    // staged or read at all (the operands' factors act in the epilogue).
    const int gma = SMS >= 0 ? SMS : g.ma, gmb = SMS >= 0 ? SMS : g.mb;
    const int64_t pA = gma == 1 ? g.K / 32 : g.K / 128;  // scale pitch of the operand rows
    const int64_t pB = gmb == 1 ? g.K / 32 : g.K / 128;
    const int rA = wm * SM + (lane & 31), rB = wn * SN + (lane & 31);
    // SKIP (grouped calls on tiles of up to 256 rows, where a group's last
    // tile may hold a few rows): fragments of rows that all lie past the
    // tile's last row are neither read nor multiplied by the FP8 / FP4 MFMA.
    // Elsewhere every fragment is multiplied (rows past the end read zero and
    // their outputs are not stored): the per-fragment branches cost the FP4
    // loops 5-8% and gain nothing where the tile's other wave row is full.
    const int fact = SKIP ? __builtin_amdgcn_readfirstlane(
                                (int)max(min((t.m_end - (t.m0 + wm * SM) + 31) / 32, (int64_t)FM), (int64_t)0))
                          : FM;

    // operand extents for the buffer resources (validated below 4 GiB): A's
    // ends with the tile's rows (the group's end), B's with the operand
    // FP4 x FP4 units are two K steps: the last one may run past a row's end
    constexpr bool LU = SU > 2;
    // The 320-row tiles cover a whole group, so no other tile reads their
    // B panel (the group's weights): it streams past the L2 (measured on
    // the 32-expert up-projection: 9% faster; where a group's panel is read
    // by two 256-row tiles, 6% slower)
    constexpr bool BSTREAM = BM == 320;
    TileLoader<RBA, BM, LU> ldA;
    TileLoader<RBB, BN, LU, GU, BSTREAM> ldB;
    // gate/up tiles: tile n0 (a multiple of BN) covers intermediate columns
    // n0 / 2 .. + BN / 2 - 1, gate rows from n0 / 2, up rows inter further
    const int64_t b_row0 = GU ? t.n0 / 2 : t.n0;
    ldA.init(g.A, t.m_end * lda, lda, t.m0, wave, lane);
    ldB.init(t.B, g.N * ldb, ldb, b_row0, wave, lane, g.inter);
    ScaleLoader<BM> lsA;
    ScaleLoader<BN, GU> lsB;
    lsA.init(gma, g.sA, g.K, t.m_end, t.m0, wave, lane);
    lsB.init(gmb, t.sB, g.K, g.N, b_row0, wave, lane, g.inter);
    constexpr int TLA = TileLoader<RBA, BM, LU>::PER_WAVE;
    constexpr int TL = TLA + TileLoader<RBB, BN, LU, GU, BSTREAM>::PER_WAVE;  // tile copies per unit
    constexpr int NSC = SMS == 0 ? 0 : ScaleLoader<BM>::NPW + ScaleLoader<BN, GU>::NPW;  // scale copies per group

    // Scale operand of a fragment row, from the staged dword: the byte for K
    // half h ends up at byte 2h (BLK32: blocks 2h + gq; BLK128: the step's
    // byte copied to bytes 0 and 2); per-tensor: 127 (x1) everywhere.  The
    // mode is folded into a shift, two masks and an OR value chosen once
    // (full-rate shifts and logic only):
    //   b = (d >> ((sh + 8 ks k) & 31)) & mask;  s = b | ((b << 16) & dup) | orv
    // (precise mode: pd keeps the staged BLK32 dword, pb the BLK128 byte
    // copied to all four bytes)
    struct SMode { uint32_t k, mask, dup, orv, pd, pb; };
    auto smode = [](int mode) __attribute__((always_inline)) -> SMode {
        if (mode == 0) return {0u, 0u, 0u, 0x7F7F7F7Fu, 0u, 0u};
        if (mode == 1) return {0u, ~0u, 0u, 0u, ~0u, 0u};
        return {1u, 0xFFu, 0xFFFF0000u, 0u, 0u, ~0u};
    };
    const SMode smA = smode(gma), smB = smode(gmb);
    // (row * pitch) % 4 is the same for every fragment row of this lane: rows
    // differ by multiples of 32
    const uint32_t rdA = (uint32_t)(((t.m0 + rA) * pA) & 3), rdB = (uint32_t)(((t.n0 + rB) * pB) & 3);
    const uint32_t shA = gma == 1 ? 8u * gq : 8u * rdA;
    const uint32_t shB = gmb == 1 ? 8u * gq : 8u * rdB;
    // byte offset, within a row's 16 staged bytes, of the dword holding step
    // ks's scale(s): BLK32 dword ks % 4; BLK128 the dword of byte rd + ks % 4
    const uint32_t kmA = gma == 1 ? 4u : 1u, kmB = gmb == 1 ? 4u : 1u;
    const uint32_t rdA_ = gma == 2 ? rdA : 0u, rdB_ = gmb == 2 ? rdB : 0u;
    auto dwA = [&](int64_t ks) __attribute__((always_inline)) -> uint32_t { return ((((uint32_t)ks & 3u) * kmA + rdA_) >> 2) * 4u; };
    auto dwB = [&](int64_t ks) __attribute__((always_inline)) -> uint32_t { return ((((uint32_t)ks & 3u) * kmB + rdB_) >> 2) * 4u; };

    // Register sets: fragments of two halves, scale operands of two K steps.
    // The precise mode's 256 x 256 tile keeps one set of FP8 fragments (its
    // bf16 operands take the room of the second): a half's fragments are
    // dead once its last quarter is converted, which happens one quarter
    // ahead, so the next half's are read into the same registers during
    // that last quarter (NM >= 2 (FM + FN) slots: reads, then conversions).
    constexpr bool SB = PRECISE && BM == 256 && BN == 256;
    static_assert(!SB || NM >= 2 * (FM + FN), "single-buffered fragments need two passes of slots");
    v8i fa[SB ? 1 : 2][FM], fb[SB ? 1 : 2][FN];
    uint32_t sa[2][FM], sb[2][FN];
    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v16f{};
    // precise mode: bf16 operands of the current and the next K = 16 quarter
    v8bf ca[2][FM], cb[2][FN];

    // Fragment of rows r .. r+31 for K half `sub` of a unit (chunk indexes
    // within an RB-byte row: FP8 half `sub` is chunks 4*sub + g and
    // 4*sub + 2 + g of a 128-byte row, or g and 2+g of a 64-byte one; FP4
    // half `sub` is chunk 2*sub + g of a 128-byte row, or chunk g of a
    // 32-byte one).
    auto frag = [&](const uint8_t* base, int r, int sub, auto info, auto rb) __attribute__((always_inline)) -> v8i {
        using I = decltype(info);
        constexpr int RB = decltype(rb)::value;
        if constexpr (I::kh == 32) {
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<RB>(r, 2 * sub + gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        } else {
            constexpr int C0 = RB == 128 ? 4 : 0;  // first chunk of half `sub`: C0 * sub
            const uint4 x = *reinterpret_cast<const uint4*>(base + lds_off<RB>(r, C0 * sub + gq));
            const uint4 y = *reinterpret_cast<const uint4*>(base + lds_off<RB>(r, C0 * sub + 2 + gq));
            return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
        }
    };
    auto frag_a = [&](const uint8_t* slot, int i, int sub) __attribute__((always_inline)) -> v8i {
        return frag(slot, rA + 32 * i, sub, IA{}, std::integral_constant<int, RBA>{});
    };
    auto frag_b = [&](const uint8_t* slot, int j, int sub) __attribute__((always_inline)) -> v8i {
        return frag(slot + A_H, rB + 32 * j, sub, IB{}, std::integral_constant<int, RBB>{});
    };
    // shift of step ks for an operand (the same for all its fragment rows)
    auto sshift = [&](const SMode& m, uint32_t sh, int64_t ks) __attribute__((always_inline)) -> uint32_t {
        return (sh + 8u * ((uint32_t)ks & 3u) * m.k) & 31u;
    };
    auto sreg = [&](const SMode& m, uint32_t d, uint32_t shift) __attribute__((always_inline)) -> uint32_t {
        if constexpr (PRECISE) {
            // byte 2h + b holds the scale of K block b of half h: BLK32 the
            // staged dword itself, BLK128 its step byte in all four bytes
            const uint32_t b4 = ((d >> shift) & 0xFFu) * 0x01010101u;
            return (d & m.pd) | (b4 & m.pb) | m.orv;
        } else {
            const uint32_t b = (d >> shift) & m.mask;
            return b | ((b << 16) & m.dup) | m.orv;
        }
    };
    // Quarter q of fragment i of register set `set`, whose half has parity
    // `h` within its K step, as bf16 with the block scale folded in; the
    // scale operand of scale set `ss` holds K block b of half h in byte 2h + b.
    // Quarters 2b and 2b+1 lie in K block b of the half: the float scale is
    // formed at the even quarter and kept for the odd one (conversions run
    // in quarter order per fragment).
    float fsa[FM], fsb[FN];
    auto conv_a = [&](int set, int h, int i, int q, int ss) __attribute__((always_inline)) -> v8bf {
        if ((q & 1) == 0) fsa[i] = e8m0_field(sa[ss][i], 2 * h + q / 2);
        return to_bf16<FA>(fa[set][i], q, fsa[i]);
    };
    auto conv_b = [&](int set, int h, int jj, int q, int ss) __attribute__((always_inline)) -> v8bf {
        if ((q & 1) == 0) fsb[jj] = e8m0_field(sb[ss][jj], 2 * h + q / 2);
        return to_bf16<FB>(fb[set][jj], q, fsb[jj]);
    };

    // slot I of the ring (compile-time I)
    auto slot = [&](auto I_) __attribute__((always_inline)) -> uint8_t* {
        constexpr int I = decltype(I_)::value;
        if constexpr (I == 0) return s0;
        else if constexpr (I == 1) return s1;
        else if constexpr (I == 2) return s2;
        else if constexpr (I == 3) return s3;
        else if constexpr (I == 4) return s4;
        else if constexpr (I == 5) return s5;
        else if constexpr (I == 6) return s6;
        else return s7;
    };
    const uint32_t LC0 = lds_addr(c0), LC1 = lds_addr(c1);
    // ring units; the last one may hold fewer than SU halves (FP4 x FP4 with
    // K % 256 == 128): its copy also fetches the bytes after the row's end
    // (the next row's, or zero past the buffer: the per-lane offset carries
    // the unit there), which no MFMA reads
    const int64_t NU = (H + SU - 1) / SU;
    // Copies of unit v (clamped to the last unit: a copy past the end lands in
    // a slot that is never read again).
    auto issue_tile = [&](int i, int64_t v, uint32_t dst) __attribute__((always_inline)) {
        const int64_t vc = v < NU ? v : NU - 1;
        if (i < TLA)
            ldA.issue(i, vc, dst, wave);
        else
            ldB.issue(i - TLA, vc, dst + (uint32_t)A_H, wave);
    };
    // Scale group u (K steps 4u .. 4u+3) into scale slot u % 2.
    auto issue_scales = [&](int64_t grp) __attribute__((always_inline)) {
        if constexpr (SMS != 0) {
            const uint32_t cs = LC0 + (uint32_t)(grp & 1) * (LC1 - LC0);  // (a select here defeats SROA)
            lsA.issue(grp, cs);
            lsB.issue(grp, cs + 16u * SRA);
        }
    };
    // Schedule: unit v (halves SU*v ..) lives in slot v % NSL.  Its copies are
    // issued in the last half of unit v - NSL, right after that half's
    // barrier (all reads of the slot are done by then); the prologue issues
    // units 0 .. NSL-1.  The scale group that starts at half 8u is issued
    // first, with the copies of the unit holding half 8u; its issuing half
    // sits at position JS (mod 8):
    constexpr int JS = ((8 - NSL * SU + SU - 1) % 8 + 8) % 8;
    static_assert(NSL * TL + NSC <= 63, "copies in flight must fit the vmcnt counter");
    static_assert((8 / SU) % NSL == 0, "slots must repeat within a group of eight halves");

    // One half j at position J = j % 8 of a group of eight halves (four K
    // steps): MFMAs of half j from register set j % 2 while the fragments of
    // half j+1 are read into the other set.  In the last half of a unit the
    // half waits for the next unit's copies, passes a barrier and refills
    // the unit's slot with unit + NSL.  At odd positions half j+1 starts a K
    // step: its scales are read and its scale operands formed.
    auto half = [&](int64_t j, auto J_) __attribute__((always_inline)) {
        constexpr int J = decltype(J_)::value;
        constexpr int P = J & 1, Q = 1 - P;       // register set of half j, of half j+1
        constexpr int SP = (J >> 1) & 1;          // scale set of half j's K step
        constexpr bool RS = (J & 1) == 1;         // read the scales of step (j+1)/2
        constexpr int SQ = ((J + 1) >> 1) & 1;    // their scale set
        constexpr int SUB = J % SU, SUB1 = (J + 1) % SU;       // halves within units
        constexpr bool LAST = SUB == SU - 1;      // last half of its unit
        constexpr int CUR = (J / SU) % NSL, NXT = ((J + 1) / SU) % NSL;
        uint32_t dst = 0;
        if constexpr (LAST) {
            // wait for the next unit's copies; those of the NSL-2 units
            // issued after them may still run
            __builtin_amdgcn_s_waitcnt(wait_vm(copies_after(J, NSL, SU, TL, JS, NSC)));
            __syncthreads();
            __builtin_amdgcn_sched_barrier(0);
            dst = lds_addr(slot(std::integral_constant<int, CUR>{}));
            if constexpr (J == JS) issue_scales((j + 1 + (NSL - 1) * SU) / (2 * SG));
        }
        uint32_t da[FM] = {}, db[FN] = {};
        if constexpr (RS && SMS != 0) {
            const int64_t ks = (j + 1) / 2;
            const uint8_t* cs = ((ks / SG) & 1) ? c1 : c0;
            const uint32_t oa = dwA(ks), ob = dwB(ks);
#pragma unroll
            for (int i = 0; i < FM; ++i) da[i] = *reinterpret_cast<const uint32_t*>(cs + (rA + 32 * i) * 16 + oa);
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
                db[jj] = *reinterpret_cast<const uint32_t*>(cs + 16 * SRA + (rB + 32 * jj) * 16 + ob);
        }
        // scale operands of step (j+1)/2 from the staged dwords
        auto form_scales = [&]() __attribute__((always_inline)) {
            if constexpr (RS) {
                const int64_t ks = (j + 1) / 2;
                const uint32_t xa = sshift(smA, shA, ks), xb = sshift(smB, shB, ks);
#pragma unroll
                for (int i = 0; i < FM; ++i) sa[SQ][i] = sreg(smA, da[i], xa);
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) sb[SQ][jj] = sreg(smB, db[jj], xb);
            }
        };
        const uint8_t* nxt = slot(std::integral_constant<int, NXT>{});
        // MFMA slots of the half: NM for the FP8 instruction, 4 NM for the
        // bf16 one (four K = 16 quarters per fragment pair)
        constexpr int NS = PRECISE ? 4 * NM : NM;
        static_for<NS>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            constexpr int k = s % NM, q = s / NM;
            constexpr int i = k % FM, jj = k / FM;
            if constexpr (!PRECISE) {
                static_assert(!SB, "single-buffered fragments are a precise-mode layout");
                if (i < fact)
                    acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[P][i], fb[P][jj], acc[i][jj], IA::code, IB::code, 2 * P, (int)sa[SP][i], 2 * P,
                        (int)sb[SP][jj]);
            } else {
                // Quarter q of every fragment pair: one bf16 instruction of
                // K = 16 on operands converted during quarter q - 1 (the
                // same bytes of A and B, so the same K positions).  Each
                // accumulator receives its quarters in the order 0..3.  The
                // next quarter's operands are converted in this quarter's
                // slots, one fragment per slot; in the last quarter they are
                // quarter 0 of the next half (fragment set Q, whose scale
                // operands are formed first when that half starts a K step).
                constexpr int CQ = q & 1;
                if constexpr (q == 3 && k == 0) form_scales();
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[CQ][i], cb[CQ][jj], acc[i][jj], 0, 0, 0);
                constexpr int NP = q < 3 ? P : Q;                  // half parity of the next quarter
                constexpr int NR = SB ? 0 : NP;                    // its fragment register set
                constexpr int NSP = q < 3 ? SP : (RS ? SQ : SP);   // its scale set
                constexpr int NQ = (q + 1) & 3;                    // its quarter
                // single-buffered fragments: the next half's are read in the
                // first slots of the last quarter and converted after them
                constexpr int K0 = (SB && q == 3) ? NM / 2 : 0;
                if constexpr (k >= K0 && k < K0 + FM) ca[1 - CQ][k - K0] = conv_a(NR, NP, k - K0, NQ, NSP);
                if constexpr (k >= K0 + FM && k < K0 + FM + FN)
                    cb[1 - CQ][k - K0 - FM] = conv_b(NR, NP, k - K0 - FM, NQ, NSP);
            }
            // next half's fragments, one per MFMA slot while they last (the
            // single-buffered precise tile: in its last quarter, into set 0)
            constexpr int R0 = SB ? 3 * NM : 0;
            if constexpr (s >= R0 && s < R0 + FM) {
                if (PRECISE || s - R0 < fact) fa[SB ? 0 : Q][s - R0] = frag_a(nxt, s - R0, SUB1);
            }
            if constexpr (s >= R0 + FM && s < R0 + FM + FN) fb[SB ? 0 : Q][s - R0 - FM] = frag_b(nxt, s - R0 - FM, SUB1);
            // copies of unit + NSL, spread evenly over the half's MFMA slots
            // (a copy waits for the CU's address unit; bursts stall the MFMAs)
            if constexpr (LAST) {
                static_for<TL>([&](auto ic) __attribute__((always_inline)) {
                    constexpr int c = decltype(ic)::value;
                    if constexpr (TL <= NS) {
                        if constexpr (s == (2 * c + 1) * NS / (2 * TL)) issue_tile(c, j / SU + NSL, dst);
                    } else {
                        if constexpr (s == c * NS / TL) issue_tile(c, j / SU + NSL, dst);
                    }
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (!PRECISE) form_scales();
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: scale group 0 and units 0 .. NSL-1 in flight; half 0 and
    // step 0's scales read
    issue_scales(0);
    static_for<NSL>([&](auto uc) __attribute__((always_inline)) {
        const uint32_t dst = lds_addr(slot(uc));
        static_for<TL>([&](auto ic) __attribute__((always_inline)) {
            issue_tile(decltype(ic)::value, decltype(uc)::value, dst);
        });
    });
    __builtin_amdgcn_s_waitcnt(wait_vm((NSL - 1) * TL));
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        fa[0][i] = frag_a(s0, i, 0);
        sa[0][i] = sreg(smA, SMS == 0 ? 0u : *reinterpret_cast<const uint32_t*>(c0 + (rA + 32 * i) * 16 + dwA(0)),
                        sshift(smA, shA, 0));
    }
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
        fb[0][jj] = frag_b(s0, jj, 0);
        sb[0][jj] = sreg(smB, SMS == 0 ? 0u : *reinterpret_cast<const uint32_t*>(c0 + 16 * SRA + (rB + 32 * jj) * 16 + dwB(0)),
                         sshift(smB, shB, 0));
    }
    if constexpr (PRECISE) {
#pragma unroll
        for (int i = 0; i < FM; ++i) ca[0][i] = conv_a(0, 0, i, 0, 0);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) cb[0][jj] = conv_b(0, 0, jj, 0, 0);
    }

    // groups of eight halves; then the 0, 2, 4 or 6 that remain
    int64_t j = 0;
    for (; j + 8 <= H; j += 8)
        static_for<8>([&](auto Jc) __attribute__((always_inline)) { half(j + decltype(Jc)::value, Jc); });
    static_for<7>([&](auto Jc) __attribute__((always_inline)) {
        if (j + decltype(Jc)::value < H) half(j + decltype(Jc)::value, Jc);
    });
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // every copy has landed before the slots are reused
    __syncthreads();

    // Epilogue: per-tensor factors, then fp32 or bf16 (round to nearest even).
    // Each wave stages bands of BR rows of its sub-tile in one slot (free
    // once the last barrier has passed) and writes them back as whole rows
    // of 16-byte stores.  The stores are non-temporal: C is not read here
    // again, and every CU writes its tile at about the same time, so the
    // write burst should not displace operand lines from the L2 (2-8%
    // faster on the workload GEMMs).
    float alpha = 1.0f;
    if (g.ma == 0) alpha *= ((const float*)g.sA)[0];
    if (g.mb == 0) alpha *= ((const float*)g.sB)[0];
    const int64_t row_base = t.m0 + wm * SM, col_base = t.n0 + wn * WN;
    // rows and columns of this wave's sub-tile that exist in C
    const int mlim = (int)min(t.m_end - row_base, (int64_t)SM);
    const int nlim = (int)min(g.N - col_base, (int64_t)WN);
    // staging room per wave: a slot each, or half of slot 0 / 1 with two slots
    constexpr int CAP = NSL >= 4 ? SLOT : SLOT / 2;
    uint8_t* const mine = NSL >= 4 ? (wave == 0 ? s0 : wave == 1 ? s1 : wave == 2 ? s2 : s3)
                                   : (wave < 2 ? s0 : s1) + (wave & 1) * CAP;
    auto store_tile = [&](auto tag) __attribute__((always_inline)) {
        using T = decltype(tag);
        constexpr int PER = 16 / (int)sizeof(T);  // elements per 16-byte chunk
        constexpr int CPR = WN / PER;             // chunks per row
        // rows per wave-wide read: 64 / CPR rounded down to a power of two (a
        // 96-column sub-tile leaves lanes RPI * CPR .. 63 idle)
        constexpr int RPI = 64 / CPR >= 8 ? 8 : 64 / CPR >= 4 ? 4 : 64 / CPR >= 2 ? 2 : 1;
        constexpr bool IDLE = RPI * CPR != 64;
        constexpr int BR = (32 * WN * (int)sizeof(T) <= CAP) ? 32 : (16 * WN * (int)sizeof(T) <= CAP ? 16 : 8);
        static_assert(BR * WN * (int)sizeof(T) <= CAP && BR % RPI == 0, "epilogue band");
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
                    const uint4 d = *reinterpret_cast<const uint4*>(band + (IDLE ? min(br, BR - 1) : br) * WN + cc);
                    if (rr < mlim && (!IDLE || lane < RPI * CPR)) {
                        T* dst = cw + (int64_t)rr * g.ldc + cc;
                        if (cc + PER <= nlim) {
                            st_nt16(dst, d);
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
    if constexpr (GU == 1) {
        // Expert MLP epilogue.  The wave's 64 intermediate columns: fragment
        // jj < 2 of a row band holds gate columns 32 jj + l % 32, jj + 2 the
        // up values of the same columns.  Per 32-row band: h in binary32 is
        // staged in the wave's LDS room (rows of 64 floats, padded by 4), then
        // read back 8 consecutive columns per lane, so that a quad of lanes
        // holds one MX block of 32 (the same arithmetic as the standalone
        // activation kernel on binary32 input).
        static_assert(FN == 4, "gate and up fragments");
        constexpr int HP = 68;  // floats per staged row
        static_assert(32 * HP * 4 <= CAP, "epilogue band");
        float* band = reinterpret_cast<float*>(mine);
        const int64_t hcol = t.n0 / 2 + wn * 64;  // first intermediate column of the wave
        const int64_t spr = g.inter / 32;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    band[(8 * (r / 4) + 4 * gq + (r % 4)) * HP + 32 * jj + (lane & 31)] =
                        swiglu_f32(acc[i][jj][r] * alpha, acc[i][jj + 2][r] * alpha);
            __syncthreads();
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {
                const int br = 8 * pass + lane / 8, ch = lane % 8;
                const float* src = band + br * HP + 8 * ch;
                const uint4 a = *reinterpret_cast<const uint4*>(src), b = *reinterpret_cast<const uint4*>(src + 4);
                const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                uint32_t m = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t v = u[k] & 0x7FFFFFFFu;
                    m = m > v ? m : v;
                }
                m = quad_max_u32(m);  // lanes 4q .. 4q+3: one row's 32-column block
                uint32_t lo, hi;
                uint8_t sb;
                mx_codes_row8<HF>(u, m, lo, hi, sb);
                const int rr = 32 * i + br;
                if (rr < mlim) {
                    const int64_t row = row_base + rr;
                    st_nt8(g.q_out + row * g.inter + hcol + 8 * ch, make_uint2(lo, hi));
                    if ((lane & 3) == 0) g.s_out[row * spr + (hcol + 8 * ch) / 32] = sb;
                }
            }
            __syncthreads();
        }
    } else if constexpr (GU == 2) {
        // Expert MLP epilogue of the 320 x 192 tile.  Waves of column 0 hold
        // gate, those of column 1 the up values of the same 96 intermediate
        // columns (fragment jj: columns 32 jj + l % 32).  Per 32-row band
        // (fragment row i of both wave rows) every wave stages its values in
        // LDS (binary32 rows of 104 floats: the two half-waves' rows, 4
        // apart, fall on disjoint banks); then each of the 256 lanes takes 8
        // consecutive columns of one row, three times over the band's 64
        // rows x 12 column chunks, so that a quad of lanes holds one MX block
        // of 32, and forms h = silu(gate) * up and its codes (the same
        // arithmetic as the standalone activation kernel on binary32 input).
        static_assert(FM == 5 && FN == 3, "320 x 192 gate/up tile");
        constexpr int HP = 104;  // floats per staged row
        static_assert(4 * 32 * HP * 4 <= SLOT, "epilogue band");
        float* band = reinterpret_cast<float*>(s0);  // [wave row][wave column][32][HP]
        float* mineb = band + (wm * 2 + wn) * 32 * HP;
        const int64_t hcol0 = t.n0 / 2;  // first intermediate column of the tile
        const int64_t spr = g.inter / 32;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mineb[(8 * (r / 4) + 4 * gq + (r % 4)) * HP + 32 * jj + (lane & 31)] = acc[i][jj][r] * alpha;
            __syncthreads();
#pragma unroll
            for (int pass = 0; pass < 3; ++pass) {
                const int task = pass * NT + tid;  // 64 rows x 12 chunks of 8 columns
                const int row = task / 12, ch = task % 12;
                const int wr = row >> 5, br = row & 31;
                const float* gp = band + ((wr * 2) * 32 + br) * HP + 8 * ch;
                const float* up = gp + 32 * HP;
                const uint4 g0 = *reinterpret_cast<const uint4*>(gp), g1 = *reinterpret_cast<const uint4*>(gp + 4);
                const uint4 u0 = *reinterpret_cast<const uint4*>(up), u1 = *reinterpret_cast<const uint4*>(up + 4);
                const uint32_t gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                const uint32_t uv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                uint32_t h[8], m = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    h[k] = as_uint(swiglu_f32(as_float(gv[k]), as_float(uv[k])));
                    const uint32_t v = h[k] & 0x7FFFFFFFu;
                    m = m > v ? m : v;
                }
                m = quad_max_u32(m);  // lanes 4q .. 4q+3: one row's 32-column block
                uint32_t lo, hi;
                uint8_t sb;
                mx_codes_row8<HF>(h, m, lo, hi, sb);
                const int64_t row_g = t.m0 + wr * SM + 32 * i + br, col = hcol0 + 8 * ch;
                if (row_g < t.m_end && col < g.inter) {
                    st_nt8(g.q_out + row_g * g.inter + col, make_uint2(lo, hi));
                    if ((lane & 3) == 0) g.s_out[row_g * spr + col / 32] = sb;
                }
            }
            __syncthreads();
        }
    } else if (g.out == 0) {
        store_tile(float{});
    } else {
        store_tile(uint16_t{});
    }
}

// Compute units of the current device (queried once per process).
inline int64_t cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

template <int FA, int FB, int BM, int BN, bool PRECISE, int HF = -1, bool SKIP = false>
hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
    const int64_t ntn = (a.N + BN - 1) / BN;
    int64_t ntm = (a.group_off == nullptr) ? (a.M + BM - 1) / BM : (a.M + BM - 1) / BM + a.G;
    if (BM == 320 && a.group_off != nullptr) ntm = (ntm + 7) / 8 * 8;  // whole XCD rounds (tile_of_block)
    // both operands BLK32: the precise mode (the mode arithmetic competes
    // with its conversions: 2% faster), FP4 x FP4 (4%), dense FP8 (1-2%)
    // and the grouped 320-row tiles (2% on the down-projection).
    // Both per-tensor (dense FP8 only): no scale staging at all.
    constexpr bool ALL32 = PRECISE || (FA == E2M1 && FB == E2M1);
    constexpr bool CAN32 = ALL32 || (HF < 0 && !SKIP);
    constexpr bool CAN0 = FA != E2M1 && FB != E2M1 && HF < 0 && BM != 320 && !SKIP;
    if (CAN32 && a.ma == 1 && a.mb == 1 && (ALL32 || a.group_off == nullptr || BM == 320))
        hipLaunchKernelGGL((k_gemm<FA, FB, BM, BN, PRECISE, HF, SKIP, CAN32 ? 1 : -1>), dim3((unsigned)(ntm * ntn)), dim3(NT),
                           0, st, a);
    else if (CAN0 && a.ma == 0 && a.mb == 0 && a.group_off == nullptr)
        hipLaunchKernelGGL((k_gemm<FA, FB, BM, BN, PRECISE, HF, SKIP, CAN0 ? 0 : -1>), dim3((unsigned)(ntm * ntn)), dim3(NT),
                           0, st, a);
    else
        hipLaunchKernelGGL((k_gemm<FA, FB, BM, BN, PRECISE, HF, SKIP>), dim3((unsigned)(ntm * ntn)), dim3(NT), 0, st, a);
    return hipGetLastError();
}

// The expert MLP's up-projection with the SwiGLU + MX epilogue (grouped, FP8
// operands, native mode): 256-row tiles once the groups average 192 rows,
// and for groups of 225-320 rows at K >= 2048 the 320 x 192 tile of the
// plain grouped GEMM (one tile per group and 96 intermediate columns).
template <int FA, int FB, int HF>
hipError_t launch_swiglu_h(const GemmArgs& a, hipStream_t st) {
    const int64_t rows = a.M / (a.G > 0 ? a.G : 1);
    if (rows > 224 && rows <= 320 && a.K >= 2048) return launch_tile<FA, FB, 320, 192, false, HF>(a, st);
    return rows < 192 ? launch_tile<FA, FB, 128, 256, false, HF, true>(a, st)
                      : launch_tile<FA, FB, 256, 256, false, HF, true>(a, st);
}
template <int FA, int FB>
hipError_t launch_swiglu_t(const GemmArgs& a, hipStream_t st) {
    return a.hfmt == E5M2 ? launch_swiglu_h<FA, FB, E5M2>(a, st) : launch_swiglu_h<FA, FB, E4M3>(a, st);
}

// Tile choice: the largest tiles (most operand reuse per LDS byte) unless
// they leave most of the 256 CUs idle.  The same for both modes.
template <int FA, int FB, bool PRECISE>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
    static_assert(!PRECISE || (FA != E2M1 && FB != E2M1), "precise mode takes FP8 operands");
    const int64_t rows = a.group_off ? (a.M / (a.G > 0 ? a.G : 1)) : a.M;
    constexpr bool SK = !PRECISE;  // grouped tiles of up to 256 rows skip fragments past a group's end
    if (rows <= 160 || a.N < 256)
        return a.group_off ? launch_tile<FA, FB, 128, 128, PRECISE, -1, SK>(a, st) : launch_tile<FA, FB, 128, 128, PRECISE>(a, st);
    const int64_t t256 = ((a.M + 255) / 256) * ((a.N + 255) / 256);
    if (a.group_off == nullptr && t256 < 192) return launch_tile<FA, FB, 128, 128, PRECISE>(a, st);
    // grouped: 256-row tiles once the groups average 192 rows (fewer passes over
    // each expert's weights), else 128-row tiles
    if (a.group_off != nullptr && rows < 192) return launch_tile<FA, FB, 128, 256, PRECISE, -1, SK>(a, st);
    // Groups of 225-320 rows (an expert's share of a routed batch): one
    // 320-row tile covers a whole group, where 256-row tiles leave a second,
    // nearly empty tile per group that streams the group's weight panel
    // again (320 x 192 keeps the accumulators of 256 x 256 and the same ring
    // slot), and the panel streams past the L2.  Measured on 32 groups of
    // 234-280 rows: 9% faster at K = 7168 and 5% at K = 2048 than 256-row
    // tiles (2% slower at K = 2048 before the weights streamed).
    if constexpr (!PRECISE && (FA == E2M1) == (FB == E2M1)) {
        if (a.group_off != nullptr && rows > 224 && rows <= 320 && a.K >= 2048)
            return launch_tile<FA, FB, 320, 192, false>(a, st);
    }
    if (a.group_off == nullptr) {
        // A last round of 256 x 256 tiles that would leave half the CUs or
        // more idle: the columns of whole rounds run as 256 x 256 tiles, the
        // remaining columns as a second launch of 128 x 256 tiles that fills
        // one round (each element's sum is the same either way).
        const int64_t ncu = cu_count(), tm = (a.M + 255) / 256, t = tm * ((a.N + 255) / 256);
        const int64_t rem = t % ncu, n1 = (t - rem) / tm * 256;
        if (rem != 0 && rem <= ncu / 2 && n1 > 0 && n1 < a.N &&
            ((a.M + 127) / 128) * ((a.N - n1 + 255) / 256) <= ncu) {
            GemmArgs a1 = a, a2 = a;
            a1.N = n1;
            a2.N = a.N - n1;
            a2.B = a.B + n1 * (FB == E2M1 ? a.K / 2 : a.K);
            if (a.mb != 0) a2.sB = (const uint8_t*)a.sB + n1 * (a.K / (a.mb == 1 ? 32 : 128));
            a2.C = (uint8_t*)a.C + n1 * (a.out == 0 ? 4 : 2);
            const hipError_t e = launch_tile<FA, FB, 256, 256, PRECISE>(a1, st);
            if (e != hipSuccess) return e;
            return launch_tile<FA, FB, 128, 256, PRECISE>(a2, st);
        }
    }
    return a.group_off ? launch_tile<FA, FB, 256, 256, PRECISE, -1, SK>(a, st) : launch_tile<FA, FB, 256, 256, PRECISE>(a, st);
}

}  // namespace mxq
