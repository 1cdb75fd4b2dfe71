"""Pins of the oracle's dequant (O8) and scaled GEMM (O9).

The reference product here decodes codes with torch's float8 views (an
independent decoder), applies scales with numpy.ldexp and multiplies with
numpy's float64 matmul: nothing in it calls the oracle's own decode.
"""
import numpy as np
import pytest
import torch

TD = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}
E2M1_MAGS = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def indep_decode(q, fmt, K):
    if fmt == 2:
        codes = np.empty((q.shape[0], K), np.uint8)
        codes[:, 0::2], codes[:, 1::2] = q & 0xF, q >> 4
        mag = E2M1_MAGS[codes & 7]
        return np.where(codes & 8, -mag, mag)
    return torch.from_numpy(q).view(TD[fmt]).to(torch.float64).numpy()


def indep_scale(s, mode, rows, K):
    if mode == 0:
        return np.full((rows, K), float(np.float32(s)))
    blk = 32 if mode == 1 else 128
    return np.ldexp(1.0, np.repeat(s.astype(np.int64) - 127, blk, axis=1))


def rand_operand(g, fmt, mode, rows, K):
    if fmt == 2:
        q = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    else:
        q = g.integers(0, 256, size=(rows, K), dtype=np.uint8)
        nan = 0x7F if fmt == 0 else 0x7C   # avoid NaN/Inf codes
        q[(q & 0x7F) >= nan] &= 0x3F
    if mode == 0:
        s = np.float32(g.uniform(0.01, 3.0))
    else:
        s = g.integers(115, 140, size=(rows, K // (32 if mode == 1 else 128)), dtype=np.uint8)
    return q, s


CASES = [(0, 0, 0, 0), (1, 0, 0, 0), (0, 0, 1, 1), (1, 0, 1, 1), (2, 2, 1, 1), (2, 0, 1, 1),
         (0, 0, 2, 1), (0, 1, 1, 0)]


@pytest.mark.parametrize("fa,fb,ma,mb", CASES)
def test_gemm_matches_independent_fp64(O, fa, fb, ma, mb):
    g = np.random.Generator(np.random.PCG64(31 + fa * 7 + fb * 3 + ma + mb))
    M, N, K = 24, 40, 256
    A, sA = rand_operand(g, fa, ma, M, K)
    B, sB = rand_operand(g, fb, mb, N, K)
    C, Cabs = O.gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K)
    Ad = indep_decode(A, fa, K) * indep_scale(sA, ma, M, K)
    Bd = indep_decode(B, fb, K) * indep_scale(sB, mb, N, K)
    ref = Ad @ Bd.T
    refabs = np.abs(Ad) @ np.abs(Bd).T
    assert np.allclose(C, ref, rtol=0, atol=1e-12 * refabs.max())
    assert np.allclose(Cabs, refabs, rtol=1e-14)
    m_idx = g.integers(0, M, 50)
    n_idx = g.integers(0, N, 50)
    c, cabs = O.gemm_entries(A, fa, sA, ma, B, fb, sB, mb, K, m_idx, n_idx)
    assert np.array_equal(c, C[m_idx, n_idx]) and np.array_equal(cabs, Cabs[m_idx, n_idx])


def test_all_ones_closed_form(O):
    M = N = 8
    K = 512
    A = np.full((M, K), 0x38, np.uint8)          # E4M3 1.0
    B = np.full((N, K), 0x3C, np.uint8)          # E5M2 1.0
    sA = np.full((M, K // 32), 130, np.uint8)    # 2^3
    sB = np.full((N, K // 32), 120, np.uint8)    # 2^-7
    C, _ = O.gemm(A, 0, sA, 1, B, 1, sB, 1, M, N, K)
    assert np.all(C == K * 2.0 ** 3 * 2.0 ** -7)
    C, _ = O.gemm(A, 0, np.float32(0.5), 0, B, 1, np.float32(3.0), 0, M, N, K)
    assert np.all(C == K * 1.5)


def test_single_block_isolates_scale(O):
    M, N, K = 4, 4, 256
    A = np.zeros((M, K), np.uint8)
    A[2, 64:96] = 0x40                            # E4M3 2.0 in block 2 of row 2
    B = np.full((N, K), 0x38, np.uint8)
    sA = np.full((M, K // 32), 127, np.uint8)
    sA[2, 2] = 131                                # 2^4
    sB = np.full((N, K // 32), 127, np.uint8)
    C, _ = O.gemm(A, 0, sA, 1, B, 0, sB, 1, M, N, K)
    assert np.all(C[2] == 32 * 2.0 * 16) and np.all(np.delete(C, 2, axis=0) == 0)


def test_identity(O):
    K = 128
    A = np.zeros((K, K), np.uint8)
    np.fill_diagonal(A, 0x38)
    g = np.random.Generator(np.random.PCG64(33))
    B, sB = rand_operand(g, 0, 1, 16, K)
    C, _ = O.gemm(A, 0, np.full((K, K // 32), 127, np.uint8), 1, B, 0, sB, 1, K, 16, K)
    assert np.array_equal(C, (indep_decode(B, 0, K) * indep_scale(sB, 1, 16, K)).T)


def test_grouped_matches_per_group(O):
    g = np.random.Generator(np.random.PCG64(34))
    G, N, K = 4, 32, 256
    off = np.array([0, 5, 5, 17, 30], np.int64)       # group 1 empty
    A, sA = rand_operand(g, 0, 2, 30, K)
    Bs = [rand_operand(g, 0, 1, N, K) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    m_idx = np.repeat(np.arange(30), N)
    n_idx = np.tile(np.arange(N), 30)
    c, _ = O.grouped_gemm_entries(A, 0, sA, 2, B, 0, sB, 1, off, N, K, m_idx, n_idx)
    c = c.reshape(30, N)
    for gi in range(G):
        r0, r1 = off[gi], off[gi + 1]
        if r1 == r0:
            continue
        Cg, _ = O.gemm(A[r0:r1], 0, sA[r0:r1], 2, B[gi], 0, sB[gi], 1, r1 - r0, N, K)
        assert np.array_equal(c[r0:r1], Cg)
