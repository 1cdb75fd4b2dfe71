"""GPU parity of the expert up-projection with its SwiGLU + MX epilogue
(mxq_grouped_gemm_swiglu_quantize_mx).

Two checks per case:
 * the fused call gives the same bytes as the two calls it fuses on the GPU
   (the grouped GEMM with fp32 output, then mxq_swiglu_quantize_mx on that
   fp32 output): every gate/up sum is the same instruction sequence and the
   activation the same binary32 arithmetic;
 * against the oracle (the fp64 GEMM, SwiGLU in fp64, MX quantization): the
   GPU's gate/up sums are within the block-scaled FP8 MFMA's bound of the
   exact ones and h is formed in binary32, so each code may sit on either
   side of a rounding boundary only where h lies within that error of it;
   everything else is identical, and nearly every code bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle as O
import mxfp4_precision_numerics_amd as mxq
import synth
from gpu_helpers import (check_mx_codes_near, dev_u8, gemm_scale_arg, host, mfma_bound, require_gpu,
                         swiglu_delta)

pytestmark = pytest.mark.gpu

# Share of codes that must equal the oracle's own.  The criterion is the
# bound (every code between those of h -+ delta); this floor only guards it.
# The gate/up sums carry the FP8 MFMA's rounding, of the order of 1e-4 of h
# on these operands, and E4M3 codes are 2^-4 apart relative: about 0.3% of
# the values lie that close to a rounding boundary, half of them across.
MIN_SAME = 0.995


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    O.lib()


def log(*a):
    print(*a, flush=True)


def bf16_bits(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def mx_operand(g, rows, K, fmt, mode, std):
    """MX (or per-tensor) codes of seeded normal data through the oracle."""
    x = bf16_bits(std * g.standard_normal((rows, K)).astype(np.float32))
    if mode == 0:
        r = O.quantize_per_tensor(x, fmt)
        return r["q_row"], r["scale_inv"]
    q, s, _, _ = O.quantize_mx(x, fmt)
    if mode == 2:  # one byte per 128 along K: the largest of the four block bytes
        s = np.ascontiguousarray(s.reshape(rows, K // 128, 4).max(axis=2))
    return q, s


def gerr_of(A, fa, sA, ma, B, fb, sB, mb, off, K, rows, inter):
    """Per-entry bound of the GPU gate/up sums (the MFMA's own bound)."""
    N = 2 * inter
    out = np.empty((len(rows), N))
    for k, r in enumerate(rows):
        grp = int(np.searchsorted(off, r, side="right") - 1)
        sa = sA if ma == 0 else sA[r:r + 1]
        out[k] = mfma_bound(A[r:r + 1], fa, sa, ma, B[grp], fb, sB if mb == 0 else sB[grp], mb, K,
                            np.zeros(N, np.int64), np.arange(N))
    return out


def run_fused_and_chain(A, fa, sA, ma, B, fb, sB, mb, off, R, inter, K, hfmt):
    G = B.shape[0]
    dA, dB = dev_u8(A), dev_u8(B)
    dsA, dsB = gemm_scale_arg(sA, ma), gemm_scale_arg(sB, mb)
    doff = torch.from_numpy(off).cuda()
    q = torch.full((R, inter), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((R, inter // 32), 0xAB, dtype=torch.uint8, device="cuda")
    mxq.grouped_gemm_swiglu_quantize_mx(dA, fa, dsA, ma, dB, fb, dsB, mb, doff, G, R, inter, K, hfmt, q, s)
    C = torch.empty((R, 2 * inter), dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dA, fa, dsA, ma, dB, fb, dsB, mb, doff, G, R, 2 * inter, K, C)
    q2 = torch.full((R, inter), 0xAB, dtype=torch.uint8, device="cuda")
    s2 = torch.full((R, inter // 32), 0xAB, dtype=torch.uint8, device="cuda")
    lo, hi = int(off[0]), int(off[-1])
    if hi > lo:
        mxq.swiglu_quantize_mx(C[lo:hi], inter, hfmt, q2[lo:hi], s2[lo:hi])
    return host(q), host(s), host(q2), host(s2)


CASES = [
    # (sizes, fa, ma, fb, mb, hfmt, inter, K): 128-row tiles (groups average
    # < 192 rows) and 256-row tiles at K = 512; 320 x 192 tiles (groups
    # averaging 225-320 rows, K >= 2048: 96 intermediate columns per tile, so
    # inter = 256 and 128 end in a partial tile, 384 does not)
    ([260, 0, 130, 77, 33], 0, 1, 0, 1, 0, 256, 512),
    ([300, 250, 0, 280, 190], 0, 1, 0, 1, 0, 256, 512),
    ([300, 250, 0, 280, 190], 0, 2, 0, 1, 1, 256, 512),
    ([201, 0, 317, 260], 1, 0, 0, 0, 0, 256, 512),
    ([300, 250, 0, 280, 331, 240], 0, 1, 0, 1, 0, 256, 2048),
    ([300, 250, 0, 280, 331, 240], 0, 2, 1, 1, 1, 384, 2176),
    ([260, 0, 317, 229], 1, 0, 0, 0, 0, 128, 2048),
]


@pytest.mark.parametrize("sizes,fa,ma,fb,mb,hfmt,inter,K", CASES)
def test_fused_up_projection_swiglu(sizes, fa, ma, fb, mb, hfmt, inter, K):
    g = np.random.Generator(np.random.PCG64([3000, len(sizes), fa, ma, fb, mb, hfmt, inter, K]))
    G = len(sizes)
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1]) + 9  # trailing rows outside every group stay untouched
    A, sA = mx_operand(g, R, K, fa, ma, 1.0)
    Bs = [mx_operand(g, 2 * inter, K, fb, mb, 0.05) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = Bs[0][1] if mb == 0 else np.stack([s for _, s in Bs])
    q, s, q2, s2 = run_fused_and_chain(A, fa, sA, ma, B, fb, sB, mb, off, R, inter, K, hfmt)
    lo, hi = int(off[0]), int(off[-1])
    assert np.array_equal(q[lo:hi], q2[lo:hi]) and np.array_equal(s[lo:hi], s2[lo:hi]), "fused != GEMM + activation"
    assert np.all(q[hi:] == 0xAB) and np.all(s[hi:] == 0xAB), "rows outside the groups written"
    rows = np.arange(lo, hi)
    oq, os_, h, gu, _ = O.expert_up_swiglu_mx(A, fa, sA, ma, B, fb, sB, mb, off, inter, K, rows, hfmt)
    gerr = gerr_of(A, fa, sA, ma, B, fb, sB, mb, off, K, rows, inter)
    same, same_s = check_mx_codes_near(q[lo:hi], s[lo:hi], h, swiglu_delta(gu, gerr, inter), hfmt,
                                       f"fused {sizes}", min_same=MIN_SAME, oq=oq)
    log(f"fused up-projection {sizes} f{fa}{fb} m{ma}{mb} h{hfmt}: identical codes {same:.6f}, "
        f"scales {float(np.mean(s[lo:hi] == os_)):.6f}")


def test_fused_up_projection_workload4():
    """The MoE share at full size: MXFP4-quantized tokens gathered and
    repacked to E4M3 with BLK128 scales (R routed rows), 32 experts' MXFP8
    gate/up weights [4096, 7168]; inter = 2048.  Whole output against the
    unfused GPU chain; sampled rows against the oracle."""
    x = synth.tensor(synth.c4_x())
    idx, off = synth.c4_routing()
    R = int(off[-1])
    oq4, os4, _, _ = O.quantize_mx(x, O.E2M1)
    A, sA = O.repack_fp4_to_fp8(oq4, os4, idx=idx)
    del x, oq4, os4
    B = np.empty((32, 4096, 7168), np.uint8)
    sB = np.empty((32, 4096, 224), np.uint8)
    for e in range(32):
        B[e], sB[e], _, _ = O.quantize_mx(synth.tensor(synth.c4_w(e)), O.E4M3)
    log(f"workload 4: R = {R}; operands ready")
    q, s, q2, s2 = run_fused_and_chain(A, 0, sA, 2, B, 0, sB, 1, off, R, 2048, 7168, 0)
    assert np.array_equal(q, q2) and np.array_equal(s, s2), "fused != GEMM + activation"
    log("workload 4: fused output bit-identical to the grouped GEMM + activation")
    g = np.random.Generator(np.random.PCG64(3100))
    starts = off[:-1][np.diff(off) > 0]
    rows = np.unique(np.concatenate([starts[:6], starts[:6] + 255, off[1:7] - 1, g.integers(0, R, 12)]))
    rows = rows[rows < R]
    oq, os_, h, gu, _ = O.expert_up_swiglu_mx(A, 0, sA, 2, B, 0, sB, 1, off, 2048, 7168, rows, 0)
    gerr = gerr_of(A, 0, sA, 2, B, 0, sB, 1, off, 7168, rows, 2048)
    same, _ = check_mx_codes_near(q[rows], s[rows], h, swiglu_delta(gu, gerr, 2048), 0, "workload 4 fused",
                                  min_same=MIN_SAME, oq=oq)
    log(f"workload 4 fused up-projection, {len(rows)} sampled rows: identical codes {same:.6f}, "
        f"scales {float(np.mean(s[rows] == os_)):.6f}")
