"""Seeded synthetic inputs for the five workloads (no method arithmetic here).

Shared by the tests (which hand the same bits to the CPU oracle and to the GPU
library) and by ``bench.py``.  Nothing in this module quantizes, scales or
multiplies operands: it only draws random numbers and rounds binary32 samples
to bfloat16 (round-to-nearest-even on the bit pattern), which is how the
inputs are defined.

Seeding: every tensor is cut into row slabs of ``SLAB`` rows; slab ``j`` of
tensor ``t`` in workload ``w`` is drawn from
``numpy.random.Generator(PCG64([w, t, j]))``.  Any slab can therefore be
regenerated alone (the oracle checks sampled slabs of the largest tensors)
and the full tensor is the concatenation of its slabs.

Tensor ids: 0 activations, 1 weights, 2 gradients, 3 routing, 4 outlier-
channel choice, 5 second activation/gradient of a workload, 100+t the t-th
prior gradient draw that fills the amax history.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

SLAB = 1024


def rng(*key):
    return np.random.Generator(np.random.PCG64(list(key)))


def f32_to_bf16_bits(x):
    """binary32 -> bfloat16 bit patterns, round-to-nearest-even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --- distributions of one slab ------------------------------------------------

def _normal(g, shape, std):
    return g.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _lognormal_grad(g, shape, sigma_log2):
    """|g| = 2^(sigma*z), z ~ N(0,1), random sign."""
    z = g.standard_normal(shape, dtype=np.float32)
    mag = np.exp2(np.float32(sigma_log2) * z)
    sign = np.where(g.integers(0, 2, size=shape, dtype=np.int8) == 0, np.float32(1), np.float32(-1))
    return mag * sign


def _student_t(g, shape, nu):
    return g.standard_t(nu, size=shape).astype(np.float32)


@dataclass(frozen=True)
class Spec:
    workload: int
    tensor: int
    rows: int
    cols: int
    dist: str              # "normal" | "lognormal2" | "student_t"
    param: float           # std | sigma in log2 | nu
    outlier_cols: int = 0  # columns multiplied by outlier_mult before rounding
    outlier_mult: float = 1.0
    dtype: str = "bf16"    # "bf16" (uint16 bits) | "f32"


def _outlier_columns(spec):
    if spec.outlier_cols == 0:
        return None
    g = rng(spec.workload, 4)
    return np.sort(g.choice(spec.cols, size=spec.outlier_cols, replace=False))


def slab_f32(spec, j):
    """Slab j (rows [j*SLAB, min((j+1)*SLAB, rows))) as binary32."""
    r0 = j * SLAB
    nr = min(SLAB, spec.rows - r0)
    g = rng(spec.workload, spec.tensor, j)
    shape = (nr, spec.cols)
    if spec.dist == "normal":
        x = _normal(g, shape, spec.param)
    elif spec.dist == "lognormal2":
        x = _lognormal_grad(g, shape, spec.param)
    elif spec.dist == "student_t":
        x = _student_t(g, shape, spec.param)
    else:
        raise ValueError(spec.dist)
    oc = _outlier_columns(spec)
    if oc is not None:
        x[:, oc] *= np.float32(spec.outlier_mult)
    return x


def slab(spec, j):
    x = slab_f32(spec, j)
    return f32_to_bf16_bits(x) if spec.dtype == "bf16" else x


def n_slabs(spec):
    return (spec.rows + SLAB - 1) // SLAB


def rows_of_slab(spec, j):
    return j * SLAB, min((j + 1) * SLAB, spec.rows)


def tensor(spec, threads=None):
    """The whole tensor (uint16 bf16 bits, or float32)."""
    out = np.empty((spec.rows, spec.cols), np.uint16 if spec.dtype == "bf16" else np.float32)
    threads = threads or min(16, os.cpu_count() or 1)

    def fill(j):
        r0, r1 = rows_of_slab(spec, j)
        out[r0:r1] = slab(spec, j)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(n_slabs(spec))))
    return out


# --- the five workloads -------------------------------------------------------
# 1: per-tensor E4M3 of two 256x256 fp32 N(0,1) matrices + 256^3 GEMM.
# 2: MXFP8 forward, Llama-3-8B MLP up-projection: X 4096x4096 N(0,1) with 1%
#    (41) outlier channels x50; W stored [N=14336, K=4096] N(0, 0.02).
# 3: E5M2 backward with delayed scaling: dY [4096, 14336] |g| = 2^(3z) random
#    sign; X [4096, 4096] and W [14336, 4096] as workload 2 without outliers.
# 4: MXFP4 MoE share: X [8192, 7168] N(0,1); 32 local experts with
#    W_g [4096 (gate+up), 7168] and W_down [7168, 2048] N(0, 0.02); routing
#    top-8 of 256 uniform.
# 5: Llama-3-70B MLP, MXFP8: X [8192, 8192], H [8192, 28672] Student-t(3);
#    W_up [28672, 8192], W_down [8192, 28672] N(0, 0.015); dY [8192, 28672],
#    dZ [8192, 8192] gradients as workload 3.

def c1_a():
    return Spec(1, 0, 256, 256, "normal", 1.0, dtype="f32")


def c1_b():
    return Spec(1, 1, 256, 256, "normal", 1.0, dtype="f32")


def c2_x():
    return Spec(2, 0, 4096, 4096, "normal", 1.0, outlier_cols=41, outlier_mult=50.0)


def c2_w():
    return Spec(2, 1, 14336, 4096, "normal", 0.02)


def c3_dy():
    return Spec(3, 2, 4096, 14336, "lognormal2", 3.0)


def c3_x():
    return Spec(3, 0, 4096, 4096, "normal", 1.0)


def c3_w():
    return Spec(3, 1, 14336, 4096, "normal", 0.02)


C3_HISTORY_LEN = 16
C3_PRIOR_ROWS = 256


def c3_prior_dy(t):
    """The t-th earlier gradient draw (t = 0..15, oldest first) whose amax fills
    the delayed-scaling history; a [256, 14336] slice of the same law."""
    return Spec(3, 100 + t, C3_PRIOR_ROWS, 14336, "lognormal2", 3.0)


C4_TOKENS, C4_HIDDEN, C4_INTER = 8192, 7168, 2048
C4_EXPERTS_TOTAL, C4_TOPK, C4_LOCAL = 256, 8, 32


def c4_x():
    return Spec(4, 0, C4_TOKENS, C4_HIDDEN, "normal", 1.0)


def c4_w(expert):
    """Expert weights [2*2048 (gate and up), 7168]; tensor id 1, one Spec per
    expert keyed by 1000 + expert so every expert has its own stream."""
    return Spec(4, 1000 + expert, 2 * C4_INTER, C4_HIDDEN, "normal", 0.02)


def c4_w_down(expert):
    """Expert down-projection weights [7168 (out), 2048 (in)], N(0, 0.02),
    stored N x K like every GEMM B operand; keyed by 2000 + expert."""
    return Spec(4, 2000 + expert, C4_HIDDEN, C4_INTER, "normal", 0.02)


def c4_gate_up(rows):
    """A stand-in for the grouped up-projection's output [rows, 2*2048]
    (gate | up) with its law: X N(0,1) times W N(0, 0.02) summed over 7168
    gives N(0, 0.02^2 * 7168), std 1.693.  Tensor id 5."""
    return Spec(4, 5, rows, 2 * C4_INTER, "normal", 0.02 * float(np.sqrt(C4_HIDDEN)))


def c4_routing():
    """Top-8 distinct experts of 256 per token, uniform.  Returns
    (gather_idx int32 [R], group_off int64 [33]): rows sorted by local expert
    (ids 0..31), token-ascending within an expert; groups may be empty."""
    g = rng(4, 3)
    keys = g.random((C4_TOKENS, C4_EXPERTS_TOTAL))
    top = np.argsort(keys, axis=1, kind="stable")[:, :C4_TOPK]
    tok, slot = np.nonzero(top < C4_LOCAL)
    exp = top[tok, slot]
    order = np.lexsort((tok, exp))
    tok, exp = tok[order], exp[order]
    counts = np.bincount(exp, minlength=C4_LOCAL)
    off = np.zeros(C4_LOCAL + 1, np.int64)
    off[1:] = np.cumsum(counts)
    return tok.astype(np.int32), off


def c5_x():
    return Spec(5, 0, 8192, 8192, "student_t", 3.0)


def c5_h():
    return Spec(5, 5, 8192, 28672, "student_t", 3.0)


def c5_w_up():
    return Spec(5, 1, 28672, 8192, "normal", 0.015)


def c5_w_down():
    return Spec(5, 6, 8192, 28672, "normal", 0.015)


def c5_dy():
    return Spec(5, 2, 8192, 28672, "lognormal2", 3.0)


def c5_dz():
    return Spec(5, 7, 8192, 8192, "lognormal2", 3.0)
