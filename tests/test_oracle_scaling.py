"""Pins of the oracle's amax (O3), per-tensor/delayed scale (O4) and
per-tensor quantize (O5)."""
import json
import os

import numpy as np
import torch

F32_MAX = np.finfo(np.float32).max


def _facts():
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")) as f:
        return json.load(f)


def test_amax_closed_form(O):
    x = np.array([[1.0, -3.5, 2.0], [0.0, -0.0, 3.25]], np.float32)
    assert O.amax(x) == 3.5
    assert O.amax(np.zeros((4, 4), np.float32)) == 0.0
    y = x.copy()
    y[1, 1] = np.nan
    assert np.isnan(O.amax(y))
    y = x.copy()
    y[0, 0] = -np.inf
    assert O.amax(y) == np.inf


def test_amax_matches_numpy_bf16(O):
    g = np.random.Generator(np.random.PCG64(3))
    bits = g.integers(0, 0x7F80, size=(64, 96), dtype=np.uint16)  # finite positive bf16
    bits |= (g.integers(0, 2, size=bits.shape, dtype=np.uint16) << 15).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    assert O.amax(bits) == np.max(np.abs(f))


def test_scale_examples(O):
    assert O.scale_from_amax(O.E4M3, 1.0) == 448.0
    assert O.scale_from_amax(O.E4M3, 448.0) == 1.0
    assert O.scale_from_amax(O.E5M2, 16.0) == 3584.0
    assert O.scale_from_amax(O.E4M3, 0.0) == 1.0
    assert O.scale_from_amax(O.E4M3, np.inf) == 1.0
    assert O.scale_from_amax(O.E4M3, np.nan) == 1.0
    assert O.scale_from_amax(O.E4M3, 1e-45) == F32_MAX   # quotient overflows binary32


def test_scale_exhaustive_over_bf16_amax(O):
    """Every positive finite bf16 amax: the scale is numpy's binary32 quotient
    (IEEE correctly rounded), FLT_MAX on overflow."""
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << np.uint32(16)
    a = bits.view(np.float32)
    for fmt, fmax in ((O.E4M3, 448.0), (O.E5M2, 57344.0)):
        with np.errstate(over="ignore"):
            expect = np.float32(fmax) / a
        expect = np.where(np.isinf(expect), F32_MAX, expect).astype(np.float32)
        got = np.array([O.scale_from_amax(fmt, float(v)) for v in a], np.float32)
        assert got.size == 32639 and np.array_equal(got, expect)


def test_history_rule_from_page(O):
    f = _facts()
    assert f["delayed_history_len"]["value"] == 16 and f["delayed_margin"]["value"] == 0
    h = np.arange(1, 17, dtype=np.float32)
    assert O.history_amax(h) == 16.0
    # margin 0 -> scale = F_max / max(history): 57344 / 16
    assert O.scale_from_amax(O.E5M2, O.history_amax(h)) == 3584.0
    h[3] = np.nan
    assert np.isnan(O.history_amax(h))


def test_delayed_sequence_by_hand(O):
    """Three steps of delayed E5M2 scaling on tiny tensors."""
    hist = np.zeros(16, np.float32)
    xs = [np.array([[2.0, -8.0]], np.float32), np.array([[1.0, 0.5]], np.float32),
          np.array([[-32.0, 4.0]], np.float32)]
    r0 = O.quantize_per_tensor(xs[0], O.E5M2, history=hist)
    assert r0["scale"] == 1.0 and r0["amax"] == 8.0            # fresh history -> scale 1
    assert hist[0] == 8.0 and np.all(hist[1:] == 0)
    r1 = O.quantize_per_tensor(xs[1], O.E5M2, history=hist)
    assert r1["scale"] == 57344.0 / 8.0 and r1["amax"] == 1.0  # previous step's amax
    assert hist[0] == 1.0 and hist[1] == 8.0
    r2 = O.quantize_per_tensor(xs[2], O.E5M2, history=hist)
    assert r2["scale"] == 57344.0 / 8.0                        # max over history
    # x * 7168: -32*7168 = -229376 saturates to -57344 (0xFB); 4*7168 = 28672 exact (0x77)
    assert list(r2["q_row"][0]) == [0xFB, 0x77]
    assert list(hist[:3]) == [32.0, 1.0, 8.0]


def test_history_drops_oldest(O):
    hist = np.zeros(16, np.float32)
    for t in range(20):
        O.quantize_per_tensor(np.array([[float(t + 1)]], np.float32), O.E4M3, history=hist)
    assert list(hist) == [float(v) for v in range(20, 4, -1)]


def test_per_tensor_worked_example(O):
    x = np.array([[1.0, -2.0], [0.5, 448.0]], np.float32)
    r = O.quantize_per_tensor(x, O.E4M3, row=True, col=True)
    assert r["amax"] == 448.0 and r["scale"] == 1.0 and r["scale_inv"] == 1.0
    assert r["q_row"].tolist() == [[0x38, 0xC0], [0x30, 0x7E]]
    assert r["q_col"].tolist() == [[0x38, 0x30], [0xC0, 0x7E]]


def test_per_tensor_two_roundings(O):
    """q = cast(fl32(x*scale)): the binary32 product is rounded first, then
    cast; checked against torch doing the same two steps."""
    g = np.random.Generator(np.random.PCG64(5))
    x = g.standard_normal((128, 64)).astype(np.float32) * np.float32(3.7)
    r = O.quantize_per_tensor(x, O.E4M3, row=True, col=True)
    amax = np.max(np.abs(x))
    scale = np.float32(448.0) / amax
    assert r["scale"] == scale
    assert r["scale_inv"] == np.float32(1.0) / scale
    y = (x * scale).astype(np.float32)
    yq = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(r["q_row"], yq)
    assert np.array_equal(r["q_col"], yq.T)
