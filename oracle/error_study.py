"""Quantization-error study on the workloads' synthetic distributions, oracle
only (test infrastructure, like the rest of oracle/).

[FP8 guide], "Estrategias de escalonamento e estabilidade": per-block (MX)
scaling is said to cut quantization error by 30-50% against per-tensor
scaling.  For a sample of each workload tensor this measures

    rel_rms = ||deq(q(x)) - x||_2 / ||x||_2      (over finite x)

for per-tensor current scaling, MX block-32 with the same element format, and
MXFP4, plus the share of non-zero inputs that quantize to zero (underflow).
For the gradients of workload 3 it also compares delayed scaling (scale from
the largest amax of the 16 previous steps) with current scaling.

Dequantization decodes every code with the oracle's own format tables:
per-tensor x^ = value(code) * scale_inv; MX x^ = value(code) * 2^(byte-127).

Run ``python -m oracle.error_study`` for the table of the full-size samples.
"""
import numpy as np

import oracle as O
import synth


def _finite_f32(x):
    v = synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32)
    return v.astype(np.float64)


def _deq_mx(q, s, fmt, cols):
    tab = O.decode_table(fmt)
    if fmt == O.E2M1:
        codes = np.empty((q.shape[0], cols), np.uint8)
        codes[:, 0::2], codes[:, 1::2] = q & 0xF, q >> 4
    else:
        codes = q
    scale = np.exp2(s.astype(np.float64) - 127.0)
    scale[s == 0xFF] = np.nan
    return tab[codes] * np.repeat(scale, 32, axis=1)


def _stats(xhat, x):
    ok = np.isfinite(x)
    err = np.linalg.norm((xhat - x)[ok]) / np.linalg.norm(x[ok])
    nz = ok & (x != 0)
    under = float(np.mean(xhat[nz] == 0)) if nz.any() else 0.0
    return float(err), under


def per_tensor_error(x, fmt, history=None):
    """rel_rms and underflow share of per-tensor scaling (current, or delayed
    with ``history``, which is updated as the oracle updates it)."""
    o = O.quantize_per_tensor(x, fmt, history=history)
    xhat = O.decode_table(fmt)[o["q_row"]] * np.float64(o["scale_inv"])
    return _stats(xhat, _finite_f32(x))


def mx_error(x, fmt):
    q, s, _, _ = O.quantize_mx(x, fmt)
    return _stats(_deq_mx(q, s, fmt, x.shape[1]), _finite_f32(x))


def study(rows=1024, cols=None):
    """One line per tensor: (name, format, per-tensor, MX same format, MXFP4),
    each (rel_rms, underflow); the sample is slab 0 of the tensor cut to
    ``rows`` x ``cols``."""
    specs = [("W2 X (outlier channels)", synth.c2_x(), O.E4M3),
             ("W2 W", synth.c2_w(), O.E4M3),
             ("W3 dY (log-normal)", synth.c3_dy(), O.E5M2),
             ("W5 X (Student-t 3)", synth.c5_x(), O.E4M3),
             ("W5 W_up", synth.c5_w_up(), O.E4M3)]
    out = []
    for name, spec, fmt in specs:
        x = synth.slab(spec, 0)[:rows, :cols]
        x = np.ascontiguousarray(x)
        out.append((name, fmt, per_tensor_error(x, fmt), mx_error(x, fmt), mx_error(x, O.E2M1)))
    return out


def delayed_vs_current(rows=256, cols=None):
    """W3 gradients: after the 16 prior steps fill the history, the error of
    dY's cast with delayed scaling and with current scaling."""
    hist = np.zeros(16, np.float32)
    for t in range(16):
        p = np.ascontiguousarray(synth.slab(synth.c3_prior_dy(t), 0)[:rows, :cols])
        O.quantize_per_tensor(p, O.E5M2, history=hist)
    x = np.ascontiguousarray(synth.slab(synth.c3_dy(), 0)[:rows, :cols])
    return per_tensor_error(x, O.E5M2, history=hist.copy()), per_tensor_error(x, O.E5M2)


def main():
    names = {O.E4M3: "E4M3", O.E5M2: "E5M2"}
    print("| Tensor (slab 0, 1024 rows) | Format | per-tensor rel RMS | MX rel RMS | MX / per-tensor "
          "| MXFP4 rel RMS | underflow per-tensor / MX |")
    print("|---|---|---|---|---|---|---|")
    for name, fmt, (pe, pu), (me, mu), (fe, _) in study():
        print(f"| {name} | {names[fmt]} | {pe:.4g} | {me:.4g} | {me / pe:.3f} | {fe:.4g} | {pu:.3g} / {mu:.3g} |")
    (de, du), (ce, cu) = delayed_vs_current()
    print(f"\nW3 dY E5M2, 256 rows: delayed rel RMS {de:.4g} (underflow {du:.3g}); "
          f"current {ce:.4g} (underflow {cu:.3g})")


if __name__ == "__main__":
    main()
