"""Pins of the oracle's decode tables (O1) and saturating RNE cast (O2).

Each check ties the oracle to something other than itself: the page's stated
range, torch's independent float8 implementations, the OCP E2M1 value set,
round-to-nearest-even at every midpoint, and an independent fixed-point
rounding of E2M1 with numpy.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


def torch_decode(dtype):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(dtype).to(torch.float64).numpy()


def same_with_nan(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        np.where(np.isnan(a), 0, a), np.where(np.isnan(b), 0, b)) and np.array_equal(
        np.signbit(np.where(np.isnan(a), 0, a)), np.signbit(np.where(np.isnan(b), 0, b)))


# ---------------------------------------------------------------- O1 decode

def test_e4m3_max_is_page_value(O):
    f = facts()
    assert O.max_finite(O.E4M3) == f["e4m3_max_finite"]["value"]
    assert O.value(O.E4M3, 0x7E) == 448.0
    assert O.value(O.E4M3, 0xFE) == -448.0


def test_e4m3_decode_matches_torch(O):
    assert same_with_nan(O.decode_table(O.E4M3), torch_decode(torch.float8_e4m3fn))


def test_e5m2_decode_matches_torch(O):
    assert same_with_nan(O.decode_table(O.E5M2), torch_decode(torch.float8_e5m2))


def test_e2m1_value_set(O):
    # OCP MX E2M1 magnitudes, sign in bit 3.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    t = O.decode_table(O.E2M1)
    assert list(t[:8]) == mags
    assert list(-t[8:]) == mags
    assert all(np.signbit(t[8:]))


def test_e2m1_values_are_e4m3_values(O):
    e4 = set(O.decode_table(O.E4M3)[~np.isnan(O.decode_table(O.E4M3))].tolist())
    assert set(O.decode_table(O.E2M1).tolist()) <= e4


@pytest.mark.parametrize("fmt,nfinite_pos", [(0, 127), (1, 124), (2, 8)])
def test_positive_codes_monotone(O, fmt, nfinite_pos):
    t = O.decode_table(fmt)
    pos = t[: (8 if fmt == O.E2M1 else 128)]
    fin = pos[np.isfinite(pos)]
    assert len(fin) == nfinite_pos
    assert np.all(np.diff(fin) > 0)
    # the finite positive codes are exactly 0..nfinite_pos-1
    assert np.all(np.isfinite(pos[:nfinite_pos]))


def test_named_anchors(O):
    assert O.value(O.E4M3, 0x01) == 2.0 ** -9      # min subnormal
    assert O.value(O.E4M3, 0x08) == 2.0 ** -6      # min normal
    assert np.isnan(O.value(O.E4M3, 0x7F)) and np.isnan(O.value(O.E4M3, 0xFF))
    assert O.value(O.E5M2, 0x7B) == 57344.0
    assert O.value(O.E5M2, 0x01) == 2.0 ** -16
    assert O.value(O.E5M2, 0x7C) == np.inf and O.value(O.E5M2, 0xFC) == -np.inf
    assert np.isnan(O.value(O.E5M2, 0x7D))
    assert O.value(O.E2M1, 0x1) == 0.5 and O.value(O.E2M1, 0x7) == 6.0
    assert O.emax(O.E4M3) == 8 and O.emax(O.E5M2) == 15 and O.emax(O.E2M1) == 2


def test_e8m0(O):
    assert O.e8m0_value(127) == 1.0
    assert O.e8m0_value(0) == 2.0 ** -127
    assert O.e8m0_value(254) == 2.0 ** 127
    assert np.isnan(O.e8m0_value(255))


# ---------------------------------------------------------------- O2 cast

@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_round_trip_every_finite_code(O, fmt):
    n = 16 if fmt == O.E2M1 else 256
    for c in range(n):
        v = O.value(fmt, c)
        if np.isfinite(v):
            assert O.cast(fmt, v) == c, (fmt, hex(c), v)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_midpoints_ties_to_even(O, fmt):
    t = O.decode_table(fmt)
    npos = 8 if fmt == O.E2M1 else 128
    fin = [(t[c], c) for c in range(npos) if np.isfinite(t[c])]
    for (lo, clo), (hi, chi) in zip(fin[:-1], fin[1:]):
        mid = (lo + hi) / 2.0
        even = clo if clo % 2 == 0 else chi
        assert O.cast(fmt, mid) == even
        assert O.cast(fmt, np.nextafter(mid, np.inf)) == chi
        assert O.cast(fmt, np.nextafter(mid, -np.inf)) == clo
        sign = 0x8 if fmt == O.E2M1 else 0x80
        assert O.cast(fmt, -mid) == (even | sign)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_saturation_and_nan(O, fmt):
    mx = O.max_finite(fmt)
    top = 0x7 if fmt == O.E2M1 else (0x7E if fmt == O.E4M3 else 0x7B)
    sign = 0x8 if fmt == O.E2M1 else 0x80
    for v in [mx, mx * 1.0001, mx * 2, 1e30, np.inf]:
        assert O.cast(fmt, v) == top
        assert O.cast(fmt, -v) == top | sign
    if fmt != O.E2M1:
        assert O.cast(fmt, np.nan) == 0x7F
        assert O.cast(fmt, -np.nan) == 0xFF


def test_worked_examples(O):
    assert O.value(O.E2M1, O.cast(O.E2M1, 5.0)) == 4.0     # tie -> even mantissa
    assert O.cast(O.E2M1, 0.25) == 0x0                      # tie between 0 and 0.5
    assert O.cast(O.E2M1, -0.25) == 0x8                     # signed zero kept
    assert O.cast(O.E4M3, 464.0) == 0x7E                    # saturates to 448
    assert O.cast(O.E4M3, 2.0 ** -10) == 0x00               # half of min subnormal: tie to 0
    assert O.cast(O.E4M3, -2.0 ** -10) == 0x80
    assert O.cast(O.E4M3, np.nextafter(2.0 ** -10, 1)) == 0x01
    assert O.cast(O.E5M2, 61440.0) == 0x7B                  # beyond max: saturate, no Inf
    assert O.cast(O.E4M3, 1.0) == 0x38 and O.cast(O.E5M2, 1.0) == 0x3C


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << np.uint32(16)
    return bits.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt,tdtype", [(0, torch.float8_e4m3fn), (1, torch.float8_e5m2)])
def test_cast_matches_torch_on_all_bf16(O, fmt, tdtype):
    """torch's float8 conversion is RNE but not saturating; inside the finite
    range the two must agree on every bf16 input; outside, the oracle must
    saturate and torch gives NaN/Inf."""
    v = _all_bf16_values()
    q = O.cast_array(fmt, v)
    mx = O.max_finite(fmt)
    inrange = np.isfinite(v) & (np.abs(v) < mx)
    tq = torch.from_numpy(v[inrange]).to(tdtype).view(torch.uint8).numpy()
    assert np.array_equal(q[inrange], tq)
    over = np.isfinite(v) & (np.abs(v) >= mx) | np.isinf(v)
    top = 0x7E if fmt == O.E4M3 else 0x7B
    assert np.array_equal(q[over], np.where(np.signbit(v[over]), top | 0x80, top).astype(np.uint8))
    nan = np.isnan(v)
    assert np.array_equal(q[nan], np.where(np.signbit(v[nan]), 0xFF, 0x7F).astype(np.uint8))


@pytest.mark.parametrize("fmt,tdtype", [(0, torch.float8_e4m3fn), (1, torch.float8_e5m2)])
def test_cast_matches_torch_on_random_f32(O, fmt, tdtype):
    g = np.random.Generator(np.random.PCG64(7))
    bits = g.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32).astype(np.float64)
    mx = O.max_finite(fmt)
    v = v[np.isfinite(v) & (np.abs(v) < mx)]
    # spread into the format's range as well
    small = (v * 2.0 ** -100).astype(np.float32).astype(np.float64)
    for arr in (v, small, np.ldexp(np.mod(v, 1.0), -7)):
        arr = arr[np.abs(arr) < mx]
        q = O.cast_array(fmt, arr)
        tq = torch.from_numpy(arr).to(tdtype).view(torch.uint8).numpy()
        assert np.array_equal(q, tq)


def test_e2m1_cast_matches_fixed_point_rounding(O):
    """Independent E2M1 rounding: inside each binade the grid step is fixed,
    so RNE is numpy's half-to-even rint of |x|/step; saturate at 6."""
    g = np.random.Generator(np.random.PCG64(11))
    x = np.concatenate([g.uniform(-9, 9, 100_000), np.arange(-40, 41) / 4.0, np.arange(-16, 17) / 2.0])
    a = np.abs(x)
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    r = np.minimum(np.rint(a / step) * step, 6.0)
    expect = np.where(np.signbit(x), -r, r)
    q = O.cast_array(O.E2M1, x)
    got = O.decode_table(O.E2M1)[q]
    assert np.array_equal(got, expect)
    assert np.array_equal(np.signbit(got), np.signbit(x))
