"""Pins of the oracle's expert-MLP activation step (SwiGLU, then MX block-32
quantization of the float64 result), against facts that do not reuse its
formula: the odd/even identities of SiLU (through tanh), exact cases, the
gate/up column layout, and the float32 path of the MX quantizer."""
import numpy as np

import oracle as O


def bf16_bits(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_silu_identities():
    x = np.linspace(-30.0, 30.0, 6001)
    a, b = O.silu(x), O.silu(-x)
    # sigma(x) + sigma(-x) = 1 and sigma(x) - sigma(-x) = tanh(x/2)
    assert np.allclose(a - b, x, rtol=0, atol=1e-13)
    assert np.allclose(a + b, x * np.tanh(x / 2), rtol=1e-13, atol=1e-14)  # cancellation near 0
    assert O.silu(np.array([0.0]))[0] == 0.0
    # the minimum of x sigma(x) lies near x = -1.2785 at about -0.27846
    i = np.argmin(a)
    assert abs(x[i] + 1.2785) < 0.01 and abs(a[i] + 0.27846) < 1e-4


def test_silu_limits_and_specials():
    big = np.array([37.0, 60.0, 1e4])
    assert np.array_equal(O.silu(big), big)                  # sigma rounds to 1 in binary64
    assert np.all(O.silu(-big) <= 0) and np.all(O.silu(-big) > -1e-14)
    r = O.silu(np.array([np.inf, -np.inf, np.nan]))
    assert r[0] == np.inf and np.isnan(r[1]) and np.isnan(r[2])


def test_swiglu_layout():
    rows, inter = 3, 64
    g = np.random.Generator(np.random.PCG64(5))
    gate = g.standard_normal((rows, inter)).astype(np.float32)
    up = g.standard_normal((rows, inter)).astype(np.float32)
    gu = np.concatenate([gate, up, np.full((rows, 32), 7.0, np.float32)], axis=1)  # extra columns unused
    h = O.swiglu(gu, inter)
    assert h.shape == (rows, inter)
    # up = 1 gives silu(gate); gate = 0 gives 0; the halves are not symmetric
    ones = np.concatenate([gate, np.ones_like(up)], axis=1)
    assert np.array_equal(O.swiglu(ones, inter), O.silu(gate.astype(np.float64)))
    zeros = np.concatenate([np.zeros_like(gate), up], axis=1)
    assert np.all(O.swiglu(zeros, inter) == 0)
    swapped = np.concatenate([up, gate], axis=1)
    assert not np.allclose(O.swiglu(swapped, inter), h)


def test_swiglu_quantize_exact_products():
    """For gate >= 37 SiLU is the identity in binary64, so h = gate * up is
    an exact product of two bf16 values, also exact in binary32: the codes
    must equal the float32 path of the MX quantizer on those products."""
    g = np.random.Generator(np.random.PCG64(6))
    rows, inter = 16, 256
    gate = bf16_bits(g.uniform(37, 200, (rows, inter)))
    up = bf16_bits(g.standard_normal((rows, inter)) * np.exp2(g.integers(-20, 20, (rows, 1))))
    up[3, :32] = 0                     # an all-zero block
    gu = np.concatenate([gate, up], axis=1)
    for fmt in (O.E4M3, O.E5M2):
        q, s, h = O.swiglu_quantize_mx(gu, inter, fmt)
        prod = (O.as_f64(gate) * O.as_f64(up)).astype(np.float32)
        assert np.array_equal(prod.astype(np.float64), h)
        q32, s32, _, _ = O.quantize_mx(prod, fmt)
        assert np.array_equal(q, q32) and np.array_equal(s, s32)
        assert s[3, 0] == 0 and np.all(np.isin(q[3, :32], (0x00, 0x80)))


def test_mx_float64_path_block_invariant():
    """On float64 input the block exponent still puts each block's largest
    magnitude in [2^emax, 2^(emax+1)), and every code is the nearest (RNE)
    value of x / 2^e in the format."""
    g = np.random.Generator(np.random.PCG64(7))
    x = g.standard_normal((8, 128)) * np.exp2(g.integers(-30, 30, (8, 4)).repeat(32, axis=1))
    for fmt in (O.E4M3, O.E5M2):
        q, s, _, _ = O.quantize_mx(np.ascontiguousarray(x), fmt)
        tab = O.decode_table(fmt)
        e = s.astype(np.int64) - 127
        amax = np.abs(x).reshape(8, 4, 32).max(axis=2)
        r = amax * np.exp2(-e.astype(np.float64))
        em = O.emax(fmt)
        assert np.all((r >= 2.0 ** em) & (r < 2.0 ** (em + 1)))
        y = x * np.exp2(-np.repeat(e, 32, axis=1).astype(np.float64))
        got = tab[q]
        finite = np.sort(np.unique(np.abs(tab[np.isfinite(tab)])))
        clip = np.clip(np.abs(y), 0, O.max_finite(fmt))
        # distance to the chosen value is the smallest distance to any value
        best = np.min(np.abs(finite[None, :] - clip.reshape(-1, 1)), axis=1).reshape(y.shape)
        assert np.allclose(np.abs(np.abs(got) - clip), best, rtol=0, atol=0)
        assert np.all((got == 0) | (np.sign(got) == np.sign(y)))


def _fused_case(seed):
    """Three groups (one empty) of MX E4M3 activations and gate/up weights."""
    g = np.random.Generator(np.random.PCG64(seed))
    inter, K = 128, 256
    sizes = [40, 0, 25]
    off = np.zeros(4, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1])
    xa = bf16_bits(g.standard_normal((R, K)).astype(np.float32))
    A, sA, _, _ = O.quantize_mx(xa, O.E4M3)
    Bs = [O.quantize_mx(bf16_bits(0.05 * g.standard_normal((2 * inter, K)).astype(np.float32)), O.E4M3)[:2]
          for _ in range(3)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    return A, sA, B, sB, off, inter, K


def test_expert_up_swiglu_is_gemm_then_activation():
    """The fused expert step equals its two steps done apart: the dense GEMM
    of each group's rows against that group's [gate; up] weights, then the
    activation step on the float64 result."""
    A, sA, B, sB, off, inter, K = _fused_case(11)
    rows = np.array([0, 7, 39, 40, 64])
    q, s, h, gu, gabs = O.expert_up_swiglu_mx(A, O.E4M3, sA, 1, B, O.E4M3, sB, 1, off, inter, K, rows, O.E4M3)
    for k, r in enumerate(rows):
        grp = int(np.searchsorted(off, r, side="right") - 1)
        c, cab = O.gemm(A[r:r + 1], O.E4M3, sA[r:r + 1], 1, B[grp], O.E4M3, sB[grp], 1, 1, 2 * inter, K)
        assert np.array_equal(gu[k], c[0]) and np.array_equal(gabs[k], cab[0])
        q1, s1, h1 = O.swiglu_quantize_mx(c, inter, O.E4M3)
        assert np.array_equal(q[k], q1[0]) and np.array_equal(s[k], s1[0]) and np.array_equal(h[k], h1[0])


def test_expert_up_swiglu_gate_up_order():
    """Gate rows are the first half of each group's weights: with identical
    halves h = silu(x) x of the common projection x; exchanging the halves
    changes h (silu(g) u != silu(u) g), and with the up half zero h is +-0."""
    A, sA, B, sB, off, inter, K = _fused_case(12)
    rows = np.arange(0, 65)
    rows = rows[(rows < 40) | (rows >= 40)]
    B2, sB2 = B.copy(), sB.copy()
    B2[:, inter:], sB2[:, inter:] = B[:, :inter], sB[:, :inter]
    _, _, h, gu, _ = O.expert_up_swiglu_mx(A, O.E4M3, sA, 1, B2, O.E4M3, sB2, 1, off, inter, K, rows, O.E4M3)
    x = gu[:, :inter]
    assert np.array_equal(gu[:, inter:], x)
    assert np.allclose(h, x * x / (1.0 + np.exp(-x)), rtol=1e-15, atol=0)
    Bs = B.copy()
    Bs[:, :inter], Bs[:, inter:] = B[:, inter:], B[:, :inter]
    sBs = sB.copy()
    sBs[:, :inter], sBs[:, inter:] = sB[:, inter:], sB[:, :inter]
    _, _, h0, _, _ = O.expert_up_swiglu_mx(A, O.E4M3, sA, 1, B, O.E4M3, sB, 1, off, inter, K, rows, O.E4M3)
    _, _, hs, _, _ = O.expert_up_swiglu_mx(A, O.E4M3, sA, 1, Bs, O.E4M3, sBs, 1, off, inter, K, rows, O.E4M3)
    assert not np.allclose(h0, hs)
    Bz = B.copy()
    Bz[:, inter:] = 0
    qz, sz, hz, _, _ = O.expert_up_swiglu_mx(A, O.E4M3, sA, 1, Bz, O.E4M3, sB, 1, off, inter, K, rows, O.E4M3)
    assert np.all(hz == 0) and np.all(sz == 0) and np.all((qz & 0x7F) == 0)
