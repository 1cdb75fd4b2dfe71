"""Generated dense GEMM cases (hypothesis, derandomized so every run draws
the same cases): random M, N and K, operand formats, scale modes and both
modes, over shapes that reach each tile choice of the launcher (128 x 128
tiles for small or narrow problems, 256 x 256 tiles, the split launch with a
128 x 256 tail).

 * sampled entries (random, plus the last row and column and both sides of
   every tile edge) against the oracle: the precise mode and FP4 x FP4 to
   1e-5 (REL_TOL), FP8 operands in the native mode to the MFMA's own bound;
 * bf16 output equals the fp32 output of the same call rounded to nearest
   even, bit for bit (the epilogue rounds the same accumulators).
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, example, given, settings
from hypothesis import strategies as st

import oracle as O
import mxfp4_precision_numerics_amd as mxq
from gpu_helpers import check_gemm, dev_u8, gemm_scale_arg, host, mfma_bound, require_gpu

pytestmark = pytest.mark.gpu

SET = settings(max_examples=25, deadline=None, derandomize=True,
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
    if mode == 0:
        s = np.float32(g.uniform(0.05, 4.0))
    else:
        s = g.integers(105, 145, size=(rows, K // (32 if mode == 1 else 128)), dtype=np.uint8)
    return q, s


def bf16_rne(c32):
    u = np.ascontiguousarray(c32, np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


@SET
@given(M=st.integers(1, 3000), n8=st.integers(1, 700), ksteps=st.integers(1, 16),
       fmts=st.sampled_from([(0, 0), (0, 1), (1, 0), (1, 1), (2, 2), (0, 2), (2, 1)]),
       ma=st.sampled_from([0, 1, 2]), mb=st.sampled_from([0, 1, 2]), precise=st.booleans(),
       bf16=st.booleans(), seed=st.integers(0, 2 ** 31))
# explicit cases for the large-tile paths: 264 tiles of 256 x 256 (split
# launch with a 128 x 256 tail), and 198 tiles in one 256 x 256 launch
@example(M=3000, n8=700, ksteps=8, fmts=(0, 0), ma=1, mb=1, precise=False, bf16=True, seed=1)
@example(M=3000, n8=700, ksteps=9, fmts=(1, 0), ma=2, mb=1, precise=True, bf16=False, seed=2)
@example(M=2100, n8=675, ksteps=9, fmts=(2, 2), ma=1, mb=2, precise=False, bf16=True, seed=3)
def test_gemm_generated(M, n8, ksteps, fmts, ma, mb, precise, bf16, seed):
    fa, fb = fmts
    precise = precise and fa != 2 and fb != 2
    N, K = 8 * n8, 128 * ksteps
    g = np.random.Generator(np.random.PCG64(seed))
    A, sA = operand(g, fa, ma, M, K)
    B, sB = operand(g, fb, mb, N, K)
    dA, dB, dsA, dsB = dev_u8(A), dev_u8(B), gemm_scale_arg(sA, ma), gemm_scale_arg(sB, mb)
    mode = mxq.OUT_PRECISE if precise else 0
    C32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mxq.scaled_gemm(dA, fa, dsA, ma, dB, fb, dsB, mb, M, N, K, C32, out=mxq.OUT_F32 | mode)
    C = host(C32)
    what = f"gemm {M}x{N}x{K} f{fa}{fb} m{ma}{mb} {'precise' if precise else 'native'}"
    if bf16:
        C16 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        mxq.scaled_gemm(dA, fa, dsA, ma, dB, fb, dsB, mb, M, N, K, C16, out=mxq.OUT_BF16 | mode)
        assert np.array_equal(host(C16), bf16_rne(C)), f"{what}: bf16 output != rounded fp32 output"
    edges_m = np.unique(np.clip(np.concatenate([np.arange(0, M, 128) - 1, np.arange(0, M, 128)]), 0, M - 1))
    edges_n = np.unique(np.clip(np.concatenate([np.arange(0, N, 128) - 1, np.arange(0, N, 128)]), 0, N - 1))
    m = np.concatenate([g.integers(0, M, 600), np.full(16, M - 1), g.choice(edges_m, 200)]).astype(np.int64)
    n = np.concatenate([g.integers(0, N, 600), g.choice(edges_n, 16), np.full(200, N - 1)]).astype(np.int64)
    ref, absum = O.gemm_entries(A, fa, sA, ma, B, fb, sB, mb, K, m, n)
    exact = precise or (fa == 2 and fb == 2)
    hb = None if exact else mfma_bound(A, fa, sA, ma, B, fb, sB, mb, K, m, n)
    check_gemm(C[m, n].astype(np.float64), ref, absum, what, hw_bound=hb)
