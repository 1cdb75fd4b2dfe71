"""Pins of the oracle's MX block-32 quantize (O6) and FP4->FP8 repack (O7)."""
import json
import os

import numpy as np
import pytest
import torch


def _facts():
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")) as f:
        return json.load(f)


def _bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _tq(v, dtype):
    return torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(dtype).view(torch.uint8).numpy()


def test_block_size_from_page(O):
    assert _facts()["mxfp4_block"]["value"] == 32
    x = np.ones((1, 64), np.float32)
    x[0, 32:] = 4.0
    _, s, _, _ = O.quantize_mx(x, O.E4M3)
    assert s.shape == (1, 2) and s[0, 0] + 2 == s[0, 1]   # two independent blocks


def test_worked_examples(O):
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    q, s, _, _ = O.quantize_mx(x, O.E4M3)
    assert s[0, 0] == 127 - 8           # e = floor(log2 1) - 8 = -8
    assert q[0, 0] == 0x78              # 1 * 2^8 = 256
    x[0, 0] = 5.0
    q, s, _, _ = O.quantize_mx(x, O.E2M1)
    assert s[0, 0] == 127               # e = floor(log2 5) - 2 = 0
    assert q[0, 0] & 0xF == 0x6         # 5 ties to 4 (even mantissa)
    x[0, 0] = 7.0                       # 7 in (6, 8): saturates to 6
    q, s, _, _ = O.quantize_mx(x, O.E2M1)
    assert s[0, 0] == 127 and q[0, 0] & 0xF == 0x7


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_scale_invariant_random_blocks(O, fmt):
    """Unclamped: amax_b * 2^-e lies in [2^emax, 2^(emax+1))."""
    g = np.random.Generator(np.random.PCG64(21))
    x = (g.standard_normal((64, 256)) * np.exp2(g.integers(-30, 30, size=(64, 1)))).astype(np.float32)
    _, s, _, _ = O.quantize_mx(x, fmt)
    amax = np.abs(x.reshape(64, 8, 32)).max(axis=2).astype(np.float64)
    e = s.astype(np.int64) - 127
    r = amax * np.exp2(-e.astype(np.float64))
    em = O.emax(fmt)
    assert np.all(r >= 2.0 ** em) and np.all(r < 2.0 ** (em + 1))


@pytest.mark.parametrize("fmt,tdtype", [(0, torch.float8_e4m3fn), (1, torch.float8_e5m2)])
def test_codes_are_rne_of_scaled_values(O, fmt, tdtype):
    """Each code is torch's RNE of x*2^-e where that is inside the finite
    range, and the largest finite code where it is not."""
    g = np.random.Generator(np.random.PCG64(22))
    x = _bf16(g.standard_t(3, size=(32, 512)).astype(np.float32) * 3)
    q, s, _, _ = O.quantize_mx(x, fmt)
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    v = np.ldexp(_f(x), -e)
    mx = O.max_finite(fmt)
    ok = np.abs(v) < mx
    assert np.array_equal(q[ok], _tq(v[ok], tdtype))
    top = 0x7E if fmt == O.E4M3 else 0x7B
    assert np.array_equal(q[~ok], np.where(v[~ok] < 0, top | 0x80, top).astype(np.uint8))


def test_e2m1_packing_and_values(O):
    g = np.random.Generator(np.random.PCG64(23))
    x = _bf16(g.standard_normal((8, 128)).astype(np.float32))
    q, s, _, _ = O.quantize_mx(x, O.E2M1)
    assert q.shape == (8, 64)
    lo, hi = q & 0xF, q >> 4
    codes = np.empty((8, 128), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = lo, hi
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    v = np.ldexp(_f(x), -e)
    # independent E2M1 RNE (fixed step per binade), saturating at 6
    a = np.abs(v)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    r = np.minimum(np.rint(a / step) * step, 6.0)
    got = O.decode_table(O.E2M1)[codes]
    assert np.array_equal(np.abs(got), r)


def test_special_blocks(O):
    x = np.ones((4, 32), np.float32)
    x[0] = 0.0
    x[0, 3] = -0.0
    x[1, 7] = np.nan
    x[2, 9] = -np.inf
    x[3] = np.float32(2.0 ** -140)          # binary32 subnormal block
    x[3, 0] = np.float32(-(2.0 ** -135))
    for fmt in (O.E4M3, O.E5M2, O.E2M1):
        q, s, _, _ = O.quantize_mx(x, fmt)
        assert s[0, 0] == 0                 # all-zero block: e = -127
        assert s[1, 0] == 0xFF and s[2, 0] == 0xFF
        assert s[3, 0] == 0                 # clamped at -127
        if fmt == O.E2M1:
            assert np.all(q[1] == 0) and np.all(q[2] == 0)
            assert q[0, 1] == 0x80          # element 3: high nibble of byte 1 = -0
        else:
            assert np.all(q[1] == 0x7F) and np.all(q[2] == 0x7F)
            assert q[0, 3] == 0x80 and q[0, 0] == 0x00
    # subnormal block scaled by 2^127: -2^-135 -> -2^-8, 2^-140 -> 2^-13
    q, s, _, _ = O.quantize_mx(x, O.E4M3)
    assert O.value(O.E4M3, q[3, 0]) == -(2.0 ** -8)
    assert O.value(O.E4M3, q[3, 1]) == 0.0   # 2^-13 < half of 2^-9
    q, s, _, _ = O.quantize_mx(x, O.E5M2)
    assert O.value(O.E5M2, q[3, 1]) == 2.0 ** -13


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_colwise_is_rowwise_of_transpose(O, fmt):
    g = np.random.Generator(np.random.PCG64(24))
    x = _bf16(g.standard_normal((96, 64)).astype(np.float32))
    _, _, qc, sc = O.quantize_mx(x, fmt, row=False, col=True)
    qr, sr, _, _ = O.quantize_mx(np.ascontiguousarray(x.T), fmt, row=True, col=False)
    assert np.array_equal(qc, qr) and np.array_equal(sc, sr)


# ------------------------------------------------------------------ repack

def _repack_case(O, code, d, base=130):
    """One row of 128 FP4 elements: block 0 carries scale byte `base`, block 1
    carries `base + d` and holds `code` at every position."""
    q4 = np.zeros((1, 64), np.uint8)
    q4[0, 16:32] = code | (code << 4)
    s4 = np.array([[base, base + d, 0, 0]], np.uint8)
    return q4, s4


def test_repack_exhaustive_lossless_region(O):
    """Page claim (direct conversion is lossless) holds exactly while the
    block's scale is within 8 binades of the group maximum."""
    assert _facts()["fp8_repack_block"]["value"] == 128
    for code in range(16):
        for d in range(-254, 1):
            base = 254
            q4, s4 = _repack_case(O, code, d, base)
            q8, s8 = O.repack_fp4_to_fp8(q4, s4)
            assert s8[0, 0] == base
            v4 = O.value(O.E2M1, code) * 2.0 ** (base + d - 127)
            v8 = O.value(O.E4M3, q8[0, 32]) * 2.0 ** (int(s8[0, 0]) - 127)
            exact = O.value(O.E2M1, code) * 2.0 ** d
            if d >= -8:
                assert v8 == v4 and np.signbit(v8) == np.signbit(v4), (code, d)
            else:
                # below E4M3's range: the RNE E4M3 code of the exact value
                assert q8[0, 32] == _tq(np.array([exact]), torch.float8_e4m3fn)[0], (code, d)


def test_repack_nan_and_gather(O):
    g = np.random.Generator(np.random.PCG64(25))
    q4 = g.integers(0, 256, size=(6, 128), dtype=np.uint8)
    s4 = g.integers(100, 140, size=(6, 8), dtype=np.uint8)
    s4[2, 5] = 0xFF
    idx = np.array([5, 2, 2, 0, 7, -1], np.int32)
    q8, s8 = O.repack_fp4_to_fp8(q4, s4, idx=idx)
    full, sfull = O.repack_fp4_to_fp8(q4, s4)
    assert np.array_equal(q8[0], full[5]) and np.array_equal(q8[3], full[0])
    assert s8[1, 1] == 0xFF and np.all(q8[1, 128:] == 0x7F)       # NaN group
    assert s8[1, 0] == sfull[2, 0] and np.array_equal(q8[1, :128], full[2, :128])
    assert np.all(s8[4] == 0xFF) and np.all(q8[4] == 0x7F)        # index out of range
    assert np.all(s8[5] == 0xFF) and np.all(q8[5] == 0x7F)


def test_repack_matches_mx_quantize_of_dequant(O):
    """Repack of MXFP4 data whose four block scales are equal changes no
    value: dequant(FP8) == dequant(FP4) element by element."""
    g = np.random.Generator(np.random.PCG64(26))
    x = _bf16(g.standard_normal((16, 256)).astype(np.float32))
    q4, s4, _, _ = O.quantize_mx(x, O.E2M1)
    q8, s8 = O.repack_fp4_to_fp8(q4, s4)
    d4 = O.dequant_matrix(q4, O.E2M1, s4, O.SCALE_BLK32, 16, 256)
    d8 = O.dequant_matrix(q8, O.E4M3, s8, O.SCALE_BLK128, 16, 256)
    gap = s8.repeat(4, axis=1).astype(int) - s4.astype(int)
    exact_rows = np.all(gap <= 8, axis=1)
    assert exact_rows.any()
    assert np.array_equal(d8[exact_rows], d4[exact_rows])


# --- O7b: FP4 row -> FP8 col --------------------------------------------------

# E2M1 from its definition (sign bit 3; exponent bits 2..1, bias 1; one
# mantissa bit; exponent field 0 is subnormal 0.5 * m)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _fp4_col_reference(q4, s4):
    """Exact dequant in float64, transpose, MX E4M3 along the new rows:
    e = floor(log2 amax) - 8 clamped to [-127, 127]; codes = RNE of the
    saturated v / 2^e by torch's float8_e4m3fn cast."""
    rows, half = q4.shape
    cols = 2 * half
    nib = np.empty((rows, cols), np.uint8)
    nib[:, 0::2], nib[:, 1::2] = q4 & 0xF, q4 >> 4
    mag = _E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sc = np.exp2(s4.astype(np.float64) - 127.0)
    sc[s4 == 0xFF] = np.nan
    v = (mag * np.repeat(sc, 32, axis=1)).T.reshape(cols, rows // 32, 32)   # [cols, blocks, 32]
    amax = np.nanmax(np.abs(v), axis=2)
    bad = np.isnan(v).any(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(amax)) - 8
    e = np.where(amax == 0, -127, np.clip(e, -127, 127))
    y = np.clip(v / np.exp2(e)[..., None], -448.0, 448.0)
    codes = _tq(np.nan_to_num(y), torch.float8_e4m3fn).reshape(cols, rows // 32, 32)
    codes[bad] = 0x7F
    sbyte = np.where(bad, 0xFF, e + 127).astype(np.uint8)
    return codes.reshape(cols, rows), sbyte


def test_fp4_col_matches_independent_reference(O):
    g = np.random.Generator(np.random.PCG64(27))
    for lo, hi in ((120, 135), (0, 255), (200, 255)):
        q4 = g.integers(0, 256, size=(96, 48), dtype=np.uint8)
        s4 = g.integers(lo, hi, size=(96, 3), dtype=np.uint8)
        q8, s8 = O.fp4_row_to_fp8_col(q4, s4)
        rq, rs = _fp4_col_reference(q4, s4)
        assert np.array_equal(s8, rs), (lo, hi)
        assert np.array_equal(q8, rq), (lo, hi)


def test_fp4_col_specials(O):
    q4 = np.zeros((64, 16), np.uint8)
    s4 = np.full((64, 1), 127, np.uint8)
    q4[3, 0] = 0x98            # row 3: column 0 = -0 (code 8), column 1 = -0.5 (code 9)
    s4[40, 0] = 0xFF           # row 40: a NaN source block covering every column
    q8, s8 = O.fp4_row_to_fp8_col(q4, s4)
    # column 0, rows 0..31: only zeros -> byte 0 (e = -127); -0 keeps its sign
    assert s8[0, 0] == 0 and q8[0, 3] == 0x80 and np.count_nonzero(q8[0, :32]) == 1
    # column 1, rows 0..31: amax 0.5 -> e = floor(log2 0.5) - 8 = -9; -0.5 / 2^-9 = -256 = E4M3 0xF8
    assert s8[1, 0] == 127 - 9 and q8[1, 3] == 0xF8
    # rows 32..63 of every column hold row 40's NaN: NaN blocks
    assert np.all(s8[:, 1] == 0xFF) and np.all(q8[:, 32:] == 0x7F)
    # the remaining columns of rows 0..31 are all zero
    assert np.all(s8[2:, 0] == 0) and np.all(q8[2:, :32] == 0)


def test_fp4_col_lossless_when_block_scales_agree(O):
    """When the 32 source rows of an output block share one scale byte, the
    requantized values equal the source values exactly (E2M1 values are E4M3
    values shifted by a power of two)."""
    g = np.random.Generator(np.random.PCG64(28))
    q4 = g.integers(0, 256, size=(64, 32), dtype=np.uint8)
    s4 = np.repeat(g.integers(1, 250, size=(2, 2), dtype=np.uint8), 32, axis=0)
    q8, s8 = O.fp4_row_to_fp8_col(q4, s4)
    d4 = O.dequant_matrix(q4, O.E2M1, s4, O.SCALE_BLK32, 64, 64)
    d8 = O.dequant_matrix(q8, O.E4M3, s8, O.SCALE_BLK32, 64, 64)
    assert np.array_equal(d8.T, d4) and np.array_equal(np.signbit(d8.T), np.signbit(d4))
