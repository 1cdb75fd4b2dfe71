"""Quantization-error study (oracle only) on small samples of the workload
distributions: the bounds the formats themselves fix.

* RNE to a format with p mantissa bits moves a normal value by at most
  2^-(p+1) of itself: E4M3 2^-4, E5M2 2^-3, so the relative RMS error of
  per-tensor scaling (no value saturates: amax maps to F_max) stays below.
* MX block scaling maps the block's largest magnitude into [2^emax, 2^(emax+1));
  values above F_max saturate, by at most 1 - F_max / 2^(emax+1) of
  themselves (E4M3: 1 - 448/512 = 12.5%; E2M1: 1 - 6/8 = 25%), which with the
  rounding bound caps the relative RMS error.
The share of values flushed to zero is compared too: per-block scales follow
each block's magnitude, and on these samples MX flushes fewer values than
per-tensor scaling (an observation on this data, not a bound: a block holding
the tensor's amax gets up to 1.75x coarser steps under MX).
"""
import numpy as np

import oracle as O
from oracle import error_study as ES
import synth


def test_error_bounds_on_workload_samples():
    rows = ES.study(rows=64, cols=1024)
    assert len(rows) == 5
    for name, fmt, (pe, pu), (me, mu), (fe, _) in rows:
        p = 3 if fmt == O.E4M3 else 2
        assert 0 < pe <= 2.0 ** -(p + 1), name
        sat = 1 - O.max_finite(fmt) / 2.0 ** (O.emax(fmt) + 1)
        assert 0 < me <= max(sat, 2.0 ** -(p + 1)), name
        assert 0 < fe <= 0.25, name
        assert mu <= pu, name


def test_delayed_scale_coarser_than_current_here():
    # the 16 prior steps come from the same distribution, so the history's max
    # exceeds this step's amax (a smaller scale, coarser steps) on this data
    (de, _), (ce, _) = ES.delayed_vs_current(rows=32, cols=1024)
    assert de >= ce > 0
