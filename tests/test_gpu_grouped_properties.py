"""Generated cases (hypothesis, derandomized so every run draws the same
cases) for the ragged grouped GEMM and the fused expert up-projection:
random group counts and sizes (empty groups, groups shorter and longer than
a tile, rows outside every group), widths and depths.

 * grouped GEMM: every row of C against the oracle (the MFMA bound for FP8
   operands, 1e-5 for FP4 x FP4, whose products the instruction sums
   exactly); rows outside every group keep their fill;
 * fused up-projection (SwiGLU + MX in the epilogue): the same bytes as the
   grouped GEMM with fp32 output followed by the activation kernel, and
   rows outside every group untouched.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, example, given, settings
from hypothesis import strategies as st

import oracle as O
import mxfp4_precision_numerics_amd as mxq
from gpu_helpers import check_gemm, dev_u8, host, mfma_bound, require_gpu

pytestmark = pytest.mark.gpu

SET = settings(max_examples=10, deadline=None, derandomize=True,
               suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    O.lib()


def operand(g, fmt, mode, rows, K):
    if fmt == 2:
        q = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    else:
        q = g.integers(0, 256, size=(rows, K), dtype=np.uint8)
        top = 0x7F if fmt == 0 else 0x7C
        q[(q & 0x7F) >= top] &= 0x3F  # finite codes
    s = g.integers(112, 140, size=(rows, K // (32 if mode == 1 else 128)), dtype=np.uint8)
    return q, s


sizes_st = st.lists(st.integers(0, 300), min_size=1, max_size=6)


@SET
@given(sizes=sizes_st, n=st.sampled_from([128, 256, 384]), k=st.sampled_from([128, 256, 384, 512]),
       fmts=st.sampled_from([(0, 0, 1), (0, 0, 2), (1, 0, 1), (2, 2, 1)]), tail=st.integers(0, 40),
       seed=st.integers(0, 2 ** 31))
def test_grouped_gemm_generated(sizes, n, k, fmts, tail, seed):
    fa, fb, ma = fmts
    g = np.random.Generator(np.random.PCG64(seed))
    G = len(sizes)
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    lead = int(g.integers(0, 3))  # the first group may start past row 0
    off += lead
    R = int(off[-1]) + tail
    A, sA = operand(g, fa, ma, R, k)
    Bs = [operand(g, fb, 1, n, k) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    C = torch.full((R, n), 777.0, dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dev_u8(A), fa, dev_u8(sA), ma, dev_u8(B), fb, dev_u8(sB), 1,
                            torch.from_numpy(off).cuda(), G, R, n, k, C)
    Ch = host(C)
    lo, hi = int(off[0]), int(off[-1])
    assert np.all(Ch[:lo] == 777.0) and np.all(Ch[hi:] == 777.0), "rows outside the groups written"
    if hi == lo:
        return
    m_idx = np.repeat(np.arange(lo, hi), n)
    n_idx = np.tile(np.arange(n), hi - lo)
    c, cabs = O.grouped_gemm_entries(A, fa, sA, ma, B, fb, sB, 1, off, n, k, m_idx, n_idx)
    hb = None
    if not (fa == 2 and fb == 2):
        parts = []
        for gi in range(G):
            r0, r1 = int(off[gi]), int(off[gi + 1])
            if r1 > r0:
                mi = np.repeat(np.arange(r1 - r0), n)
                ni = np.tile(np.arange(n), r1 - r0)
                parts.append(mfma_bound(A[r0:r1], fa, sA[r0:r1], ma, B[gi], fb, sB[gi], 1, k, mi, ni))
        hb = np.concatenate(parts).reshape(-1, n)
    check_gemm(Ch[lo:hi], c.reshape(-1, n), cabs.reshape(-1, n), f"grouped {sizes} n{n} k{k} f{fa}{fb} m{ma}",
               hw_bound=hb)


@SET
@given(sizes=sizes_st, inter=st.sampled_from([128, 256]), k=st.sampled_from([128, 256, 512, 2048]),
       ma=st.sampled_from([1, 2]), hfmt=st.sampled_from([0, 1]), tail=st.integers(0, 40),
       seed=st.integers(0, 2 ** 31))
# groups averaging 225-320 rows at K >= 2048: the 320 x 192 tiles
@example(sizes=[300, 251, 0, 290, 290], inter=256, k=2048, ma=1, hfmt=0, tail=7, seed=5)
@example(sizes=[233, 299], inter=128, k=2048, ma=2, hfmt=1, tail=0, seed=6)
def test_fused_up_projection_generated(sizes, inter, k, ma, hfmt, tail, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    G = len(sizes)
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1]) + tail
    A, sA = operand(g, 0, ma, R, k)
    Bs = [operand(g, 0, 1, 2 * inter, k) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    dA, dB, dsA, dsB = dev_u8(A), dev_u8(B), dev_u8(sA), dev_u8(sB)
    doff = torch.from_numpy(off).cuda()
    q = torch.full((R, inter), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((R, inter // 32), 0xAB, dtype=torch.uint8, device="cuda")
    mxq.grouped_gemm_swiglu_quantize_mx(dA, 0, dsA, ma, dB, 0, dsB, 1, doff, G, R, inter, k, hfmt, q, s)
    Cgu = torch.empty((R, 2 * inter), dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dA, 0, dsA, ma, dB, 0, dsB, 1, doff, G, R, 2 * inter, k, Cgu)
    q2 = torch.full((R, inter), 0xAB, dtype=torch.uint8, device="cuda")
    s2 = torch.full((R, inter // 32), 0xAB, dtype=torch.uint8, device="cuda")
    hi = int(off[-1])
    if hi > 0:
        mxq.swiglu_quantize_mx(Cgu[:hi], inter, hfmt, q2[:hi], s2[:hi])
    qh, sh, q2h, s2h = host(q), host(s), host(q2), host(s2)
    assert np.array_equal(qh[:hi], q2h[:hi]) and np.array_equal(sh[:hi], s2h[:hi]), "fused != GEMM + activation"
    assert np.all(qh[hi:] == 0xAB) and np.all(sh[hi:] == 0xAB), "rows outside the groups written"
