"""Generated cases (hypothesis, derandomized so every run draws the same
cases) for the cast kernels, all against the oracle:

 * MX block-32 quantize: row (E4M3, E5M2, E2M1) and dual row + column
   (FP8), bf16 or binary32 input, row pitch wider than the row, values
   spread over many binades per block, with zeros, signed zeros, NaN, Inf
   and subnormals mixed in: codes and scale bytes bit-exact;
 * per-tensor cast, current or delayed scaling, row and column outputs:
   amax, scale, scale_inv, history and codes bit-exact;
 * FP4 -> FP8 repack, with and without a gather (indices out of range
   included): bit-exact;
 * FP4 row -> FP8 col over random scale windows: bit-exact;
 * SwiGLU + MX: the codes within the binary32 bound of the activation.

Shapes are drawn over the kernels' tile edges (ragged rows and columns, a
single block, many tiles).
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O
import mxfp4_precision_numerics_amd as mxq
from gpu_helpers import (check_swiglu_codes, dev_input, dev_u8, empty_u8, gpu_quantize_mx,
                         gpu_quantize_per_tensor, host, require_gpu, same_float)

pytestmark = pytest.mark.gpu

SET = settings(max_examples=30, deadline=None, derandomize=True,
               suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    O.lib()


def to_bf16(x):
    u = np.asarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def values(g, rows, cols, spread, specials):
    """float32 values: normal draws scaled by 2^e per 32-column block (e
    spread over +-spread), with a share of specials."""
    e = g.integers(-spread, spread + 1, size=(rows, (cols + 31) // 32)).repeat(32, axis=1)[:, :cols]
    x = (g.standard_normal((rows, cols)) * np.exp2(e)).astype(np.float32)
    if specials:
        pick = g.random((rows, cols))
        x[pick < 0.02] = 0.0
        x[(pick >= 0.02) & (pick < 0.03)] = -0.0
        x[(pick >= 0.03) & (pick < 0.035)] = np.float32(2.0 ** -140) * np.sign(g.standard_normal())
        x[(pick >= 0.035) & (pick < 0.037)] = np.inf
        x[(pick >= 0.037) & (pick < 0.038)] = np.nan
    return x


@SET
@given(rblk=st.integers(1, 9), cblk=st.integers(1, 12), fmt=st.sampled_from([0, 1, 2]), bf16=st.booleans(),
       dual=st.booleans(), pad=st.sampled_from([0, 32]), spread=st.sampled_from([2, 20, 120]),
       specials=st.booleans(), seed=st.integers(0, 2 ** 31))
def test_mx_generated(rblk, cblk, fmt, bf16, dual, pad, spread, specials, seed):
    dual = dual and fmt != 2
    g = np.random.Generator(np.random.PCG64(seed))
    rows = 32 * rblk if dual else 32 * rblk - int(g.integers(0, 32))
    cols = 32 * cblk
    full = values(g, rows, cols + pad, spread, specials)
    if bf16:
        full = to_bf16(full)
    x = np.ascontiguousarray(full[:, :cols])
    if pad == 0:
        got = gpu_quantize_mx(x, fmt, row=True, col=dual)
    else:
        # the row pitch of the wider array (cols + pad elements)
        xd = dev_input(full)[:, :cols]
        q_row, s_row = empty_u8(rows, cols // 2 if fmt == 2 else cols), empty_u8(rows, cols // 32)
        q_col = s_col = None
        if dual:
            q_col, s_col = empty_u8(cols, rows), empty_u8(cols, rows // 32)
        mxq.quantize_mx(xd, fmt, q_row, s_row, q_col, s_col)
        got = tuple(None if t is None else host(t) for t in (q_row, s_row, q_col, s_col))
    exp = O.quantize_mx(x, fmt, row=True, col=dual)
    what = f"mx f{fmt} {rows}x{cols}+{pad} bf16={bf16} dual={dual} spread={spread}"
    for k in range(4 if dual else 2):
        assert np.array_equal(got[k], exp[k]), (what, k)


@SET
@given(rblk=st.integers(1, 12), cblk=st.integers(1, 40), fmt=st.sampled_from([0, 1]), bf16=st.booleans(),
       col=st.booleans(), delayed=st.booleans(), spread=st.sampled_from([3, 30]),
       seed=st.integers(0, 2 ** 31))
def test_per_tensor_generated(rblk, cblk, fmt, bf16, col, delayed, spread, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = 16 * rblk if col else 16 * rblk - int(g.integers(0, 16))
    cols = 16 * cblk
    x = values(g, rows, cols, spread, False)
    if bf16:
        x = to_bf16(x)
    hist = None
    if delayed:
        hist = np.abs(g.standard_normal(16)).astype(np.float32) * np.float32(2.0 ** g.integers(-10, 10))
        hist[g.integers(0, 16)] = 0.0
    hg = None if hist is None else hist.copy()
    ho = None if hist is None else hist.copy()
    got = gpu_quantize_per_tensor(x, fmt, history=hg, row=True, col=col)
    exp = O.quantize_per_tensor(x, fmt, history=ho, row=True, col=col)
    what = f"pt f{fmt} {rows}x{cols} bf16={bf16} col={col} delayed={delayed}"
    for k in ("amax", "scale", "scale_inv"):
        assert same_float(got[k], exp[k]), (what, k, got[k], exp[k])
    assert np.array_equal(got["q_row"], exp["q_row"]), what
    if col:
        assert np.array_equal(got["q_col"], exp["q_col"]), what
    if delayed:
        assert np.array_equal(hg.view(np.uint32), ho.view(np.uint32)), what


@SET
@given(src_rows=st.integers(1, 300), gblk=st.integers(1, 6), gather=st.booleans(), lo=st.integers(0, 250),
       width=st.sampled_from([1, 9, 40, 255]), nan=st.booleans(), seed=st.integers(0, 2 ** 31))
def test_repack_generated(src_rows, gblk, gather, lo, width, nan, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cols = 128 * gblk
    q4 = g.integers(0, 256, size=(src_rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(lo, min(lo + width, 255), size=(src_rows, cols // 32), endpoint=True).astype(np.uint8)
    if nan:
        s4[g.integers(0, src_rows), g.integers(0, cols // 32)] = 0xFF
    idx = None
    rows = src_rows
    if gather:
        rows = int(g.integers(1, 2 * src_rows + 2))
        idx = g.integers(-2, src_rows + 2, size=rows).astype(np.int32)  # a few out of range
    q8, s8 = empty_u8(rows, cols), empty_u8(rows, cols // 128)
    mxq.repack_fp4_to_fp8(dev_u8(q4), dev_u8(s4), q8, s8,
                          gather_idx=None if idx is None else torch.from_numpy(idx).cuda())
    oq, os_ = O.repack_fp4_to_fp8(q4, s4, idx=idx)
    what = f"repack {src_rows}->{rows}x{cols} gather={gather} s in [{lo}, {lo + width}]"
    assert np.array_equal(host(s8), os_), what
    assert np.array_equal(host(q8), oq), what


@SET
@given(rblk=st.integers(1, 10), cblk=st.integers(1, 20), lo=st.integers(0, 254), width=st.sampled_from([1, 6, 30, 254]),
       zeros=st.booleans(), seed=st.integers(0, 2 ** 31))
def test_fp4_col_generated(rblk, cblk, lo, width, zeros, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    rows, cols = 32 * rblk, 32 * cblk
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    if zeros:
        q4[g.random(q4.shape) < 0.3] = 0
    s4 = g.integers(lo, min(lo + width, 255), size=(rows, cols // 32), endpoint=True).astype(np.uint8)
    q8, s8 = empty_u8(cols, rows), empty_u8(cols, rows // 32)
    mxq.fp4_row_to_fp8_col(dev_u8(q4), dev_u8(s4), q8, s8)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    what = f"fp4col {rows}x{cols} s in [{lo}, {lo + width}]"
    assert np.array_equal(host(s8), os_), what
    assert np.array_equal(host(q8), oq), what


@SET
@given(rows=st.integers(1, 200), iblk=st.integers(1, 10), fmt=st.sampled_from([0, 1]), bf16=st.booleans(),
       gscale=st.sampled_from([0.5, 4.0, 30.0]), seed=st.integers(0, 2 ** 31))
def test_swiglu_generated(rows, iblk, fmt, bf16, gscale, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    inter = 32 * iblk
    gate = g.standard_normal((rows, inter)) * gscale
    up = g.standard_normal((rows, inter)) * np.exp2(g.integers(-20, 20, (rows, inter // 32)).repeat(32, axis=1))
    gu = np.concatenate([gate, up], axis=1).astype(np.float32)
    if bf16:
        gu = to_bf16(gu)
    q, s = empty_u8(rows, inter), empty_u8(rows, inter // 32)
    mxq.swiglu_quantize_mx(dev_input(gu), inter, fmt, q, s)
    check_swiglu_codes(host(q), host(s), gu, inter, fmt, f"swiglu {rows}x{inter} f{fmt} bf16={bf16}")
