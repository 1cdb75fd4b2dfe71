"""GPU parity: every kernel of libmxq against the CPU oracle, element by
element, through the C ABI.  Codes, scale bytes, amax/scale values and the
delayed-scaling history must match bit for bit; GEMM outputs within the
tolerance of gpu_helpers.check_gemm."""
import numpy as np
import pytest
import torch

import oracle as O
import mxfp4_precision_numerics_amd as mxq
from gpu_helpers import (check_gemm, check_swiglu_codes, dev_bf16, dev_f32, dev_input, dev_u8, empty_u8,
                         gemm_scale_arg, gpu_quantize_mx, gpu_quantize_per_tensor, host, mfma_bound, require_gpu,
                         same_float)

pytestmark = pytest.mark.gpu

FMAX = {0: 448.0, 1: 57344.0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    O.lib()


def all_bf16_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)


def rand_bf16(g, shape, lo_exp=-140, hi_exp=130):
    """bf16 bit patterns with random sign/mantissa and exponent spread."""
    e = g.integers(max(lo_exp + 127, 0), min(hi_exp + 127, 255), size=shape, dtype=np.int64)
    m = g.integers(0, 128, size=shape, dtype=np.int64)
    s = g.integers(0, 2, size=shape, dtype=np.int64)
    return ((s << 15) | (e << 7) | m).astype(np.uint16)


# --------------------------------------------------- expert MLP activation

def gpu_swiglu(gu, inter, fmt, ld=None):
    rows = gu.shape[0]
    xd = dev_input(gu)
    q, sc = empty_u8(rows, inter), empty_u8(rows, inter // 32)
    mxq.swiglu_quantize_mx(xd, inter, fmt, q, sc)
    return host(q), host(sc)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("src", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(96, 96), (33, 2080), (256, 512)])
def test_swiglu_random(fmt, src, shape):
    """Random gate/up values over a wide exponent range, ragged row counts
    and block counts; float32 input also with non-bf16 mantissas."""
    rows, inter = shape
    g = np.random.Generator(np.random.PCG64([30, fmt, rows, inter, src == "bf16"]))
    gate = g.standard_normal((rows, inter)) * 4 * np.exp2(g.integers(-6, 4, (rows, 1)))
    up = g.standard_normal((rows, inter)) * np.exp2(g.integers(-30, 30, (rows, inter // 32)).repeat(32, axis=1))
    gu = np.concatenate([gate, up], axis=1).astype(np.float32)
    if src == "bf16":
        gu = synth_bf16(gu)
    q, sc = gpu_swiglu(gu, inter, fmt)
    check_swiglu_codes(q, sc, gu, inter, fmt, f"swiglu {src} fmt{fmt} {shape}")


def test_swiglu_specials_and_pitch():
    """Inf/NaN gates and ups (NaN blocks), gates far out on both sides, zeros
    with both signs, subnormal products, and a row pitch wider than 2 inter."""
    rows, inter, ld = 64, 128, 320
    g = np.random.Generator(np.random.PCG64(31))
    full = (g.standard_normal((rows, ld)) * 2).astype(np.float32)
    gate, up = full[:, :inter], full[:, inter:2 * inter]
    gate[0, 3] = np.inf              # silu(+inf) * up: +-inf -> NaN block
    gate[1, 40] = -np.inf            # -inf / inf: NaN block
    up[2, 70] = np.nan
    gate[3, :32] = -100.0            # silu(-100) * up is a binary32 subnormal
    gate[4, :32] = 60.0              # sigma = 1
    gate[5, 32:64] = 0.0             # h = +-0: all-zero block
    up[5, 64:96] = -0.0
    gate[6, :] = 1e-30               # products far below binary32's normal range
    up[6, :] = 1e-15
    q, sc = gpu_swiglu(full, inter, 0)
    assert sc[0, 0] == 0xFF and sc[1, 1] == 0xFF and sc[2, 2] == 0xFF
    assert sc[5, 1] == 0 and np.all(np.isin(q[5, 32:64], (0x00, 0x80)))
    check_swiglu_codes(q, sc, np.ascontiguousarray(full), inter, 0, "swiglu specials")


# ------------------------------------------------------------------ per-tensor

def synth_bf16(x):
    """float32 values -> bf16 bit patterns (RNE)."""
    u = np.asarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def compare_pt(got, exp, what):
    assert same_float(got["amax"], exp["amax"]), (what, got["amax"], exp["amax"])
    assert same_float(got["scale"], exp["scale"]), (what, got["scale"], exp["scale"])
    assert same_float(got["scale_inv"], exp["scale_inv"]), (what, got["scale_inv"], exp["scale_inv"])
    for k in ("q_row", "q_col"):
        if exp[k] is not None:
            bad = np.nonzero(got[k] != exp[k])
            assert bad[0].size == 0, (what, k, bad[0].size, got[k][bad][:8], exp[k][bad][:8])


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("ref_amax", [None, "fmax", 3.0, 1e-30, 6e4])
def test_per_tensor_every_bf16_pattern(fmt, ref_amax):
    """All 65,536 bf16 inputs (NaN, Inf, subnormals included) through the
    per-tensor cast, with delayed scaling pinning the scale."""
    x = all_bf16_bits()
    if ref_amax is None:
        hist = None  # current scaling: amax is NaN here -> scale 1
    else:
        a = FMAX[fmt] if ref_amax == "fmax" else ref_amax
        hist = np.zeros(16, np.float32)
        hist[5] = a
    h_gpu = None if hist is None else hist.copy()
    h_or = None if hist is None else hist.copy()
    got = gpu_quantize_per_tensor(x, fmt, history=h_gpu, row=True, col=True)
    exp = O.quantize_per_tensor(x, fmt, history=h_or, row=True, col=True)
    compare_pt(got, exp, f"fmt{fmt} ref{ref_amax}")
    if hist is not None:
        assert np.array_equal(np.isnan(h_gpu), np.isnan(h_or))
        assert np.array_equal(np.nan_to_num(h_gpu), np.nan_to_num(h_or))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [0, 1])
def test_per_tensor_every_fp32_pattern(fmt):
    """The saturating RNE cast on every one of the 2^32 binary32 bit patterns
    (scale pinned to 1 by a history whose max is the format's largest
    value), in chunks of 2^26 generated on each side from the same counter."""
    n = 1 << 26
    rows = n // 4096
    fmax = np.float32(FMAX[fmt])
    amax, sc, si = (torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(3))
    q = empty_u8(rows, 4096)
    for c in range(1 << 32 >> 26):
        xd = torch.arange(c * n, (c + 1) * n, dtype=torch.int64, device="cuda").to(torch.int32).view(torch.float32)
        hist_d = torch.full((16,), float(fmax), dtype=torch.float32, device="cuda")
        mxq.quantize_per_tensor(xd.view(rows, 4096), fmt, amax, sc, si, q, None, amax_history=hist_d)
        got = host(q)
        x = np.arange(c * n, (c + 1) * n, dtype=np.uint64).astype(np.uint32).view(np.float32).reshape(rows, 4096)
        exp = O.quantize_per_tensor(x, fmt, history=np.full(16, fmax, np.float32), row=True)
        assert host(sc)[0] == 1.0 and exp["scale"] == 1.0
        bad = np.nonzero(got != exp["q_row"])
        assert bad[0].size == 0, (c, bad[0].size, x[bad][:4].view(np.uint32), got[bad][:4], exp["q_row"][bad][:4])


@pytest.mark.parametrize("fmt", [0, 1])
def test_per_tensor_random_fp32_bits(fmt):
    g = np.random.Generator(np.random.PCG64(100 + fmt))
    bits = g.integers(0, 2 ** 32, size=(512, 1024), dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).copy()
    x[np.isnan(x)] = 1.0  # keep amax finite so the scale is a real quotient
    for a in (None, 2.5e3, 7e-20):
        hist = None if a is None else np.full(16, np.float32(a) / 2, np.float32)
        if hist is not None:
            hist[0] = a
        hg = None if hist is None else hist.copy()
        ho = None if hist is None else hist.copy()
        got = gpu_quantize_per_tensor(x, fmt, history=hg, row=True, col=True)
        exp = O.quantize_per_tensor(x, fmt, history=ho, row=True, col=True)
        compare_pt(got, exp, f"fp32 fmt{fmt} a{a}")


@pytest.mark.parametrize("shape", [(16, 16), (48, 176), (200, 304), (131, 48)])
def test_per_tensor_ragged_shapes(shape):
    g = np.random.Generator(np.random.PCG64(7))
    x = (g.standard_normal(shape) * 3).astype(np.float32)
    col = shape[0] % 16 == 0
    got = gpu_quantize_per_tensor(x, 0, row=True, col=col)
    exp = O.quantize_per_tensor(x, 0, row=True, col=col)
    compare_pt(got, exp, f"shape {shape}")


@pytest.mark.parametrize("src", ["bf16", "fp32"])
@pytest.mark.parametrize("delayed", [False, True])
def test_per_tensor_persistent_tiles(src, delayed):
    """More tiles than the persistent grid holds blocks (2192 x 7984: 576
    bf16 tiles of 128 x 256, 1134 fp32 tiles of 128 x 128), ragged in both
    directions, so blocks walk several tiles, the last ones partial."""
    g = np.random.Generator(np.random.PCG64([41, int(delayed), src == "bf16"]))
    shape = (2192, 7984)
    x = rand_bf16(g, shape, lo_exp=-20, hi_exp=20)
    if src == "fp32":
        x = (x.astype(np.uint32) << 16).view(np.float32) * np.float32(1.0 + 2.0 ** -10)
    hist = np.full(16, 3.0e5, np.float32) if delayed else None
    got = gpu_quantize_per_tensor(x, 1, history=None if hist is None else hist.copy(), row=True, col=True)
    exp = O.quantize_per_tensor(x, 1, history=None if hist is None else hist.copy(), row=True, col=True)
    compare_pt(got, exp, f"persistent {src} delayed={delayed}")


def test_delayed_sequence_matches_oracle():
    """Twenty delayed-scaling E5M2 steps on log-normal gradients; the history
    evolves identically (checkpoint/resume: restarting from a copied history
    gives the same codes)."""
    hg = np.zeros(16, np.float32)
    ho = np.zeros(16, np.float32)
    for t in range(20):
        g = np.random.Generator(np.random.PCG64([9, t]))
        z = g.standard_normal((64, 256)).astype(np.float32)
        x = (np.exp2(3 * z) * np.where(g.integers(0, 2, z.shape) == 0, 1, -1)).astype(np.float32)
        x = ((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
        if t == 12:  # resume from a copy of the history
            hg = hg.copy()
        got = gpu_quantize_per_tensor(x, 1, history=hg, row=True, col=True)
        exp = O.quantize_per_tensor(x, 1, history=ho, row=True, col=True)
        compare_pt(got, exp, f"step {t}")
        assert np.array_equal(hg, ho)


def test_recipe_state_hybrid_forward_backward():
    """ScalingState under the default DelayedScaling recipe: the forward
    tensor is cast to E4M3 and the gradient to E5M2, each with its own
    history, for 18 steps (beyond the history length), against the oracle."""
    recipe = mxq.DelayedScaling()
    fwd, bwd = mxq.ScalingState(recipe), mxq.ScalingState(recipe)
    ho_f, ho_b = np.zeros(16, np.float32), np.zeros(16, np.float32)
    for t in range(18):
        g = np.random.Generator(np.random.PCG64([11, t]))
        xf = synth_bf16(g.standard_normal((32, 128)).astype(np.float32) * (1 + t))
        z = g.standard_normal((32, 128)).astype(np.float32)
        xb = synth_bf16(np.exp2(3 * z - t % 5) * np.where(g.integers(0, 2, z.shape) == 0, 1, -1))
        for state, x, ho, back in ((fwd, xf, ho_f, False), (bwd, xb, ho_b, True)):
            q = empty_u8(32, 128)
            fmt = state.quantize(dev_bf16(x), q_row=q, backward=back)
            assert fmt == (mxq.E5M2 if back else mxq.E4M3)
            exp = O.quantize_per_tensor(x, fmt, history=ho, row=True)
            assert np.array_equal(host(q), exp["q_row"]), f"step {t} backward={back}"
            assert host(state.scale_inv)[0] == exp["scale_inv"]
            assert np.array_equal(host(state.history), ho)


def test_per_tensor_strided_input():
    g = np.random.Generator(np.random.PCG64(8))
    full = (g.standard_normal((64, 96)) * 10).astype(np.float32)
    xd = dev_f32(full)[:, 16:80]  # row pitch 96 elements
    amax = torch.empty(1, device="cuda")
    sc = torch.empty(1, device="cuda")
    q = empty_u8(64, 64)
    mxq.quantize_per_tensor(xd, 0, amax, sc, None, q)
    exp = O.quantize_per_tensor(np.ascontiguousarray(full[:, 16:80]), 0)
    assert np.array_equal(host(q), exp["q_row"])


# ------------------------------------------------------------------ MX

def mx_blocks_every_exponent(g, src_bf16=True):
    """Blocks whose amax exponent takes every biased value 0..254, filled with
    values down to 24 binades below it (so subnormal codes, underflow to zero
    and saturation all occur), plus special blocks."""
    blocks = []
    for E in range(0, 255):
        for rep in range(4):
            lo = max(E - 24, 0)
            e = g.integers(lo, E + 1, size=32)
            m = g.integers(0, 128, size=32)
            s = g.integers(0, 2, size=32)
            e[0] = E
            m[0] = 127 if rep % 2 == 0 else g.integers(0, 128)
            blocks.append((s << 15) | (e << 7) | m)
    z = np.zeros(32, np.int64)
    blocks.append(z)                                  # all +0
    blocks.append(z | 0x8000)                         # all -0
    nb = z.copy(); nb[3] = 0x7FC0; blocks.append(nb)  # NaN
    ib = z.copy(); ib[9] = 0xFF80; blocks.append(ib)  # -Inf
    sb = g.integers(1, 128, size=32) | (g.integers(0, 2, size=32) << 15); blocks.append(sb)  # subnormal
    arr = np.stack(blocks).astype(np.uint16)
    n = (arr.shape[0] // 4) * 4
    return arr[:n].reshape(n // 4, 128)  # 4 blocks per row


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_mx_row_every_bf16_pattern(fmt):
    x = all_bf16_bits()
    qg, sg, _, _ = gpu_quantize_mx(x, fmt)
    qo, so, _, _ = O.quantize_mx(x, fmt)
    assert np.array_equal(sg, so)
    assert np.array_equal(qg, qo)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_mx_row_every_scale_exponent(fmt):
    g = np.random.Generator(np.random.PCG64(200 + fmt))
    x = mx_blocks_every_exponent(g)
    qg, sg, _, _ = gpu_quantize_mx(x, fmt)
    qo, so, _, _ = O.quantize_mx(x, fmt)
    assert np.array_equal(sg, so)
    bad = np.nonzero(qg != qo)
    assert bad[0].size == 0, (bad[0].size, qg[bad][:8], qo[bad][:8])
    assert set(np.unique(so)) >= set(range(0, 120))   # every low exponent appears


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_mx_row_fp32_input(fmt):
    g = np.random.Generator(np.random.PCG64(300 + fmt))
    bits = g.integers(0, 2 ** 32, size=(96, 256), dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).copy()
    x[:48] = (g.standard_normal((48, 256)) * np.exp2(g.integers(-140, 120, size=(48, 1)))).astype(np.float32)
    qg, sg, _, _ = gpu_quantize_mx(x, fmt)
    qo, so, _, _ = O.quantize_mx(x, fmt)
    assert np.array_equal(sg, so)
    assert np.array_equal(qg, qo)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("shape,row", [((160, 96), True), ((96, 416), True), ((256, 128), False),
                                        ((32, 32), True)])
def test_mx_dual_row_and_col(fmt, shape, row):
    g = np.random.Generator(np.random.PCG64(400 + fmt))
    x = rand_bf16(g, shape, -30, 20)
    x[:, 5] = rand_bf16(g, (shape[0],), -135, -120)  # a subnormal-ish column
    if shape[0] >= 64:
        x[37, 3] = 0x7FC0  # NaN poisons one row block and one column block
    qg, sg, qcg, scg = gpu_quantize_mx(x, fmt, row=row, col=True)
    qo, so, qco, sco = O.quantize_mx(x, fmt, row=row, col=True)
    if row:
        assert np.array_equal(sg, so) and np.array_equal(qg, qo)
    assert np.array_equal(scg, sco)
    assert np.array_equal(qcg, qco)


def test_mx_ragged_rows_and_strided():
    g = np.random.Generator(np.random.PCG64(450))
    full = rand_bf16(g, (37, 224), -10, 10)
    x = np.ascontiguousarray(full[:, :160])
    xd = torch.from_numpy(full.view(np.int16)).cuda().view(torch.bfloat16)[:, :160]
    q = empty_u8(37, 160)
    s = empty_u8(37, 5)
    mxq.quantize_mx(xd, 0, q, s)
    qo, so, _, _ = O.quantize_mx(x, 0)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)


# ------------------------------------------------------------------ repack

def test_repack_every_code_and_shift():
    """16 codes x every shift d in [-254, 0], NaN scales, and a gather."""
    rows = []
    srows = []
    for d in range(-254, 1):
        q = np.zeros(64, np.uint8)
        q[16:32] = np.arange(16, dtype=np.uint8) * 0x11  # every code, both nibbles, block 1
        q[0:16] = np.arange(16, dtype=np.uint8)[::-1] | (np.arange(16, dtype=np.uint8) << 4)
        rows.append(q)
        srows.append([254, 254 + d, 100, 254 + d])
    q4 = np.stack(rows)
    s4 = np.array(srows, np.uint8)
    s4[7, 2] = 0xFF
    q8g = empty_u8(q4.shape[0], 128)
    s8g = empty_u8(q4.shape[0], 1)
    mxq.repack_fp4_to_fp8(dev_u8(q4), dev_u8(s4), q8g, s8g)
    q8o, s8o = O.repack_fp4_to_fp8(q4, s4)
    assert np.array_equal(host(s8g), s8o)
    bad = np.nonzero(host(q8g) != q8o)
    assert bad[0].size == 0, (bad, host(q8g)[bad][:8], q8o[bad][:8])


@pytest.mark.parametrize("gather", [False, True])
def test_repack_random_with_gather(gather):
    g = np.random.Generator(np.random.PCG64(500))
    src_rows, cols = 300, 7168
    q4 = g.integers(0, 256, size=(src_rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(110, 140, size=(src_rows, cols // 32), dtype=np.uint8)
    s4[g.integers(0, src_rows, 5), g.integers(0, cols // 32, 5)] = 0xFF
    idx = None
    rows = src_rows
    if gather:
        idx = g.integers(0, src_rows, size=517).astype(np.int32)
        idx[[3, 400]] = [-1, src_rows]  # out of range -> NaN groups
        rows = len(idx)
    q8g = empty_u8(rows, cols)
    s8g = empty_u8(rows, cols // 128)
    mxq.repack_fp4_to_fp8(dev_u8(q4), dev_u8(s4), q8g, s8g,
                          gather_idx=None if idx is None else torch.from_numpy(idx).cuda())
    q8o, s8o = O.repack_fp4_to_fp8(q4, s4, idx=idx)
    assert np.array_equal(host(s8g), s8o)
    assert np.array_equal(host(q8g), q8o)


# ------------------------------------------------------- FP4 row -> FP8 col

def gpu_fp4_col(q4, s4):
    rows, cols = q4.shape[0], q4.shape[1] * 2
    q8, s8 = empty_u8(cols, rows), empty_u8(cols, rows // 32)
    mxq.fp4_row_to_fp8_col(dev_u8(q4), dev_u8(s4), q8, s8)
    return host(q8), host(s8)


@pytest.mark.parametrize("shape", [(128, 256), (96, 288), (224, 544), (32, 32), (256, 1024)])
@pytest.mark.parametrize("srange", [(120, 136), (0, 255), (230, 255)])
def test_fp4_col_random(shape, srange):
    """Random codes and scale bytes (every code; scale spreads within a
    block of up to 255 binades), ragged tiles both ways: bit-exact."""
    rows, cols = shape
    g = np.random.Generator(np.random.PCG64([17, rows, cols, srange[0]]))
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(srange[0], srange[1], size=(rows, cols // 32), dtype=np.uint8)
    q8, s8 = gpu_fp4_col(q4, s4)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    assert np.array_equal(s8, os_)
    assert np.array_equal(q8, oq)


def test_fp4_col_many_ragged_tiles():
    """5216 x 8224: 1353 tiles of 128 x 256, ragged in both directions,
    mostly mid-range scales with bytes over the whole range sprinkled in (so
    both conversion paths run, tile by tile)."""
    g = np.random.Generator(np.random.PCG64(20))
    rows, cols = 5216, 8224
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(100, 160, size=(rows, cols // 32), dtype=np.uint8)
    s4[g.integers(0, rows, 64), g.integers(0, cols // 32, 64)] = g.integers(0, 255, 64).astype(np.uint8)
    q8, s8 = gpu_fp4_col(q4, s4)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    assert np.array_equal(s8, os_) and np.array_equal(q8, oq)


def test_fp4_col_specials():
    g = np.random.Generator(np.random.PCG64(18))
    rows, cols = 160, 320
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(110, 140, size=(rows, cols // 32), dtype=np.uint8)
    s4[37, 4] = 0xFF               # NaN source block
    q4[64:96, :] = 0               # an all-zero band of tokens
    q4[100, 10] = 0x88             # two negative zeros
    s4[130:160, 2] = 0             # the smallest scale, 2^-127
    s4[128:130, 2] = 254           # next to the largest
    q4[0:32, 40:48] = 0            # zeros in rows with the largest scales
    s4[0:32, 5] = 254
    q8, s8 = gpu_fp4_col(q4, s4)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    assert np.array_equal(s8, os_) and np.array_equal(q8, oq)
    assert np.all(s8[128:160, 1] == 0xFF)


def test_fp4_col_scale_spread_edges():
    """Scale bytes at the ends of the byte range and at spreads of 243-253
    binades within a 32-token block (bytes 0 and 254; column exponents set by
    other tokens' far larger scales), with zero codes, zero rows and signed
    zeros mixed in: bit-exact."""
    g = np.random.Generator(np.random.PCG64(21))
    rows, cols = 256, 512
    edges = np.array([0, 1, 2, 9, 10, 11, 120, 243, 244, 245, 251, 252, 253, 254], np.uint8)
    s4 = edges[g.integers(0, len(edges), size=(rows, cols // 32))]
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    q4[g.random(q4.shape) < 0.3] = 0
    q4[g.random(q4.shape) < 0.05] = 0x88
    q4[g.integers(0, rows, 24), :] = 0
    # 8-token groups whose scales sit at one end, next to groups at the other
    for r0 in range(0, rows, 64):
        s4[r0:r0 + 8] = 254
        s4[r0 + 8:r0 + 16] = g.integers(0, 12, size=(8, cols // 32)).astype(np.uint8)
    q8, s8 = gpu_fp4_col(q4, s4)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    assert np.array_equal(s8, os_)
    assert np.array_equal(q8, oq)


def test_fp4_col_conversion_path_edges():
    """Tiles of 128 tokens x 256 columns on either side of the converter
    path's condition (every scale byte of the tile in [12, 254]): bytes 12 and
    254 inside one 32-token block, a single 11, a single NaN byte, next to
    tiles that convert on the fast path; bit-exact in every tile."""
    g = np.random.Generator(np.random.PCG64(22))
    rows, cols = 384, 768
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(12, 255, size=(rows, cols // 32), dtype=np.uint8)
    s4[0:16, 0:8] = 12                     # tile (0, 0): both edges of the range in one block
    s4[16:32, 0:8] = 254
    s4[5, 3] = 12
    s4[200, 9] = 11                        # tile (1, 1): one byte below the range
    s4[300, 17] = 0xFF                     # tile (2, 2): a NaN block
    s4[128:256, 16:24] = 12                # tile (1, 2): all at the lower edge
    q4[140:150, 64:96] = 0x11              # of it, smallest non-zero codes
    q8, s8 = gpu_fp4_col(q4, s4)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    assert np.array_equal(s8, os_)
    assert np.array_equal(q8, oq)


@pytest.mark.parametrize("shape", [(256, 512), (96, 256)])
def test_fp4_col_unaligned_scale_output(shape):
    """The output scale array at an odd byte address (its 4-byte stores
    fall back to bytes): bit-exact, and the bytes around it untouched."""
    rows, cols = shape
    g = np.random.Generator(np.random.PCG64([23, rows]))
    q4 = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s4 = g.integers(110, 140, size=(rows, cols // 32), dtype=np.uint8)
    n = cols * (rows // 32)
    buf = torch.full((n + 2,), 0xA5, dtype=torch.uint8, device="cuda")
    q8 = empty_u8(cols, rows)
    mxq.fp4_row_to_fp8_col(dev_u8(q4), dev_u8(s4), q8, buf[1:n + 1].view(cols, rows // 32))
    b = host(buf)
    oq, os_ = O.fp4_row_to_fp8_col(q4, s4)
    assert b[0] == 0xA5 and b[-1] == 0xA5
    assert np.array_equal(b[1:n + 1].reshape(cols, rows // 32), os_)
    assert np.array_equal(host(q8), oq)


def test_fp4_col_of_gpu_mx_quantize():
    """BF16 activations -> MXFP4 rows (GPU) -> FP8 columns (GPU) against the
    oracle's own chain."""
    g = np.random.Generator(np.random.PCG64(19))
    x = synth_bf16(g.standard_normal((512, 1024)).astype(np.float32) * np.exp2(g.integers(-4, 5, (1, 1024))))
    q4, s4, _, _ = gpu_quantize_mx(x, mxq.E2M1)
    oq4, os4, _, _ = O.quantize_mx(x, O.E2M1)
    assert np.array_equal(q4, oq4) and np.array_equal(s4, os4)
    q8, s8 = gpu_fp4_col(q4, s4)
    oq, os_ = O.fp4_row_to_fp8_col(oq4, os4)
    assert np.array_equal(s8, os_) and np.array_equal(q8, oq)


# ------------------------------------------------------------------ GEMM

def rand_operand(g, fmt, mode, rows, K, nan_codes=False):
    if fmt == 2:
        q = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    else:
        q = g.integers(0, 256, size=(rows, K), dtype=np.uint8)
        if not nan_codes:
            top = 0x7F if fmt == 0 else 0x7C
            q[(q & 0x7F) >= top] &= 0x3F
    if mode == 0:
        s = np.float32(g.uniform(0.01, 3.0))
    else:
        s = g.integers(110, 140, size=(rows, K // (32 if mode == 1 else 128)), dtype=np.uint8)
    return q, s


def run_gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K, out=0):
    C = torch.empty((M, N), dtype=torch.bfloat16 if out & mxq.OUT_BF16 else torch.float32, device="cuda")
    mxq.scaled_gemm(dev_u8(A), fa, gemm_scale_arg(sA, ma), ma, dev_u8(B), fb, gemm_scale_arg(sB, mb), mb,
                    M, N, K, C, out=out)
    return host(C)


FORMATS = [(0, 0), (1, 0), (0, 1), (1, 1), (2, 2), (2, 0), (0, 2), (1, 2), (2, 1)]


def full_bound(A, fa, sA, ma, B, fb, sB, mb, M, N, K):
    m_idx = np.repeat(np.arange(M), N)
    n_idx = np.tile(np.arange(N), M)
    return mfma_bound(A, fa, sA, ma, B, fb, sB, mb, K, m_idx, n_idx).reshape(M, N)


@pytest.mark.parametrize("fa,fb", FORMATS)
@pytest.mark.parametrize("ma,mb", [(1, 1), (0, 0), (2, 1), (0, 1)])
def test_gemm_formats_and_modes(fa, fb, ma, mb):
    """Random codes over each format's whole range: within the MFMA's own
    bound; FP4 x FP4 (whose products all fit the instruction's alignment
    window) within 1e-5."""
    g = np.random.Generator(np.random.PCG64(600 + fa * 10 + fb + ma * 100 + mb * 1000))
    M, N, K = 160, 200, 384  # two ragged tiles each way, three K steps
    A, sA = rand_operand(g, fa, ma, M, K)
    B, sB = rand_operand(g, fb, mb, N, K)
    C = run_gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K)
    Cref, Cabs = O.gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K)
    if fa == 2 and fb == 2:
        check_gemm(C, Cref, Cabs, f"f{fa}{fb} m{ma}{mb}")
    else:
        check_gemm(C, Cref, Cabs, f"f{fa}{fb} m{ma}{mb}", hw_bound=full_bound(A, fa, sA, ma, B, fb, sB, mb, M, N, K))


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (2, 2), (0, 2)])
def test_gemm_structured_exact(fa, fb):
    """Cases with an exact answer: all-ones codes, a single non-zero block
    (isolates one scale byte), and an identity operand."""
    one = {0: 0x38, 1: 0x3C, 2: 0x22}[fa]      # E2M1 byte 0x22 = two codes of 1.0
    oneb = {0: 0x38, 1: 0x3C, 2: 0x22}[fb]
    M, N, K = 64, 128, 512
    ka = K // 2 if fa == 2 else K
    kb = K // 2 if fb == 2 else K
    A = np.full((M, ka), one, np.uint8)
    B = np.full((N, kb), oneb, np.uint8)
    sA = np.full((M, K // 32), 127, np.uint8)
    sB = np.full((N, K // 32), 127, np.uint8)
    sA[:, 3] = 131
    sB[5, :] = 120
    C = run_gemm(A, fa, sA, 1, B, fb, sB, 1, M, N, K)
    Cref, _ = O.gemm(A, fa, sA, 1, B, fb, sB, 1, M, N, K)
    assert np.array_equal(C.astype(np.float64), Cref)
    # single non-zero block in row 7 of A
    A2 = np.zeros_like(A)
    if fa == 2:
        A2[7, 48:64] = one
    else:
        A2[7, 96:128] = one
    C = run_gemm(A2, fa, sA, 1, B, fb, sB, 1, M, N, K)
    Cref, _ = O.gemm(A2, fa, sA, 1, B, fb, sB, 1, M, N, K)
    assert np.array_equal(C.astype(np.float64), Cref) and np.count_nonzero(C) == N


def test_gemm_identity_fp8():
    g = np.random.Generator(np.random.PCG64(610))
    K = 256
    A = np.zeros((K, K), np.uint8)
    np.fill_diagonal(A, 0x38)
    B, sB = rand_operand(g, 0, 1, 96, K)
    sA = np.full((K, K // 32), 127, np.uint8)
    C = run_gemm(A, 0, sA, 1, B, 0, sB, 1, K, 96, K)
    Cref, _ = O.gemm(A, 0, sA, 1, B, 0, sB, 1, K, 96, K)
    assert np.array_equal(C.astype(np.float64), Cref)


def test_gemm_nan_propagation_and_bf16_out():
    g = np.random.Generator(np.random.PCG64(650))
    M, N, K = 64, 96, 256
    A, sA = rand_operand(g, 0, 1, M, K)
    B, sB = rand_operand(g, 0, 1, N, K)
    A[5, 17] = 0x7F        # NaN code
    sB[9, 3] = 0xFF        # NaN scale
    C = run_gemm(A, 0, sA, 1, B, 0, sB, 1, M, N, K)
    Cref, Cabs = O.gemm(A, 0, sA, 1, B, 0, sB, 1, M, N, K)
    check_gemm(C, Cref, Cabs, "nan", hw_bound=full_bound(A, 0, sA, 1, B, 0, sB, 1, M, N, K))
    # bf16 output: within bf16 rounding (2^-9 relative, RNE) of the fp32 tolerance
    A2, sA2 = rand_operand(g, 0, 1, M, K)
    B2, sB2 = rand_operand(g, 1, 1, N, K)
    Cb = run_gemm(A2, 0, sA2, 1, B2, 1, sB2, 1, M, N, K, out=1)
    Cref, Cabs = O.gemm(A2, 0, sA2, 1, B2, 1, sB2, 1, M, N, K)
    Cf = (Cb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    hb = full_bound(A2, 0, sA2, 1, B2, 1, sB2, 1, M, N, K)
    # bf16 keeps 8 significant bits: RNE moves a value by at most 2^-8 of itself
    assert np.all(np.abs(Cf - Cref) <= 2.0 ** -8 * (np.abs(Cref) + hb) + hb)


def test_gemm_c1_per_tensor_end_to_end():
    """Workload 1: per-tensor E4M3 of two 256x256 fp32 N(0,1) matrices
    (current scaling), then the 256^3 GEMM with the dequant factors."""
    import synth
    a = synth.tensor(synth.c1_a())
    b = synth.tensor(synth.c1_b())
    ra = gpu_quantize_per_tensor(a, 0)
    rb = gpu_quantize_per_tensor(b, 0, col=True)
    oa = O.quantize_per_tensor(a, 0)
    ob = O.quantize_per_tensor(b, 0, col=True)
    compare_pt(ra, oa, "A")
    compare_pt(rb, ob, "B")
    # C = A . B (B stored K-contiguous as B^T = the colwise output)
    C = run_gemm(ra["q_row"], 0, ra["scale_inv"], 0, rb["q_col"], 0, rb["scale_inv"], 0, 256, 256, 256)
    Cref, Cabs = O.gemm(oa["q_row"], 0, oa["scale_inv"], 0, ob["q_col"], 0, ob["scale_inv"], 0, 256, 256, 256)
    hb = full_bound(oa["q_row"], 0, oa["scale_inv"], 0, ob["q_col"], 0, ob["scale_inv"], 0, 256, 256, 256)
    check_gemm(C, Cref, Cabs, "c1", hw_bound=hb)


def test_grouped_gemm_fp4_x_fp4():
    """MXFP4 activations x MXFP4 expert weights (the variant that skips the
    repack), ragged groups with 256-row tiles: FP4 x FP4 products are exact
    in the MFMA, so 1e-5 holds."""
    g = np.random.Generator(np.random.PCG64(701))
    sizes = [260, 0, 330, 250]  # 210 rows per group on average: 256-row tiles
    G, N, K = len(sizes), 256, 512
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1])
    A, sA = rand_operand(g, 2, 1, R, K)
    Bs = [rand_operand(g, 2, 1, N, K) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    C = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dev_u8(A), 2, dev_u8(sA), 1, dev_u8(B), 2, dev_u8(sB), 1,
                            torch.from_numpy(off).cuda(), G, R, N, K, C)
    m_idx = np.repeat(np.arange(R), N)
    n_idx = np.tile(np.arange(N), R)
    c, cabs = O.grouped_gemm_entries(A, 2, sA, 1, B, 2, sB, 1, off, N, K, m_idx, n_idx)
    check_gemm(host(C), c.reshape(-1, N), cabs.reshape(-1, N), "grouped fp4")


@pytest.mark.parametrize("sizes", [[0, 37, 256, 0, 129, 1], [300, 0, 517, 258]])
def test_grouped_gemm_ragged_with_empty_groups(sizes):
    """Ragged groups, empty ones included; the second set averages more than
    192 rows per group, which selects 256-row tiles (one group spans three)."""
    g = np.random.Generator(np.random.PCG64([700, len(sizes)]))
    G, N, K = len(sizes), 256, 512
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1]) + 13  # trailing rows outside every group stay untouched
    A, sA = rand_operand(g, 0, 2, R, K)
    Bs = [rand_operand(g, 0, 1, N, K) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    C = torch.full((R, N), 12345.0, dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dev_u8(A), 0, dev_u8(sA), 2, dev_u8(B), 0, dev_u8(sB), 1,
                            torch.from_numpy(off).cuda(), G, R, N, K, C)
    Ch = host(C)
    m_idx = np.repeat(np.arange(int(off[-1])), N)
    n_idx = np.tile(np.arange(N), int(off[-1]))
    c, cabs = O.grouped_gemm_entries(A, 0, sA, 2, B, 0, sB, 1, off, N, K, m_idx, n_idx)
    hb = np.concatenate([full_bound(A[off[gi]:off[gi + 1]], 0, sA[off[gi]:off[gi + 1]], 2, B[gi], 0, sB[gi], 1,
                                    int(off[gi + 1] - off[gi]), N, K) for gi in range(G)])
    check_gemm(Ch[:int(off[-1])], c.reshape(-1, N), cabs.reshape(-1, N), "grouped", hw_bound=hb)
    assert np.all(Ch[int(off[-1]):] == 12345.0)


def run_grouped_case(g, off_dev, off_ref, R, N, K):
    """Grouped MXFP8 GEMM with device offsets `off_dev`; every row of C
    against the oracle on the offsets `off_ref` (rows outside every group
    keep their fill value)."""
    G = len(off_ref) - 1
    A, sA = rand_operand(g, 0, 2, R, K)
    B = g.integers(0, 256, size=(G, N, K), dtype=np.uint8)
    B[(B & 0x7F) == 0x7F] &= 0x3F
    sB = g.integers(118, 136, size=(G, N, K // 32), dtype=np.uint8)
    C = torch.full((R, N), 12345.0, dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dev_u8(A), 0, dev_u8(sA), 2, dev_u8(B), 0, dev_u8(sB), 1,
                            torch.from_numpy(np.asarray(off_dev, np.int64)).cuda(), G, R, N, K, C)
    Ch = host(C)
    lo, hi = int(off_ref[0]), int(off_ref[-1])
    m_idx = np.repeat(np.arange(lo, hi), N)
    n_idx = np.tile(np.arange(N), hi - lo)
    c, cabs = O.grouped_gemm_entries(A, 0, sA, 2, B, 0, sB, 1, off_ref, N, K, m_idx, n_idx)
    hb = np.concatenate([full_bound(A[off_ref[gi]:off_ref[gi + 1]], 0, sA[off_ref[gi]:off_ref[gi + 1]], 2, B[gi], 0,
                                    sB[gi], 1, int(off_ref[gi + 1] - off_ref[gi]), N, K)
                         for gi in range(G) if off_ref[gi + 1] > off_ref[gi]])
    check_gemm(Ch[lo:hi], c.reshape(-1, N), cabs.reshape(-1, N), "grouped", hw_bound=hb)
    assert np.all(Ch[:lo] == 12345.0) and np.all(Ch[hi:] == 12345.0)


def test_grouped_gemm_offsets_clamped_to_the_rows():
    """Device offsets that break the contract (a negative start, an end past
    total_rows) cannot be rejected on the host; the kernel clamps them to
    [0, total_rows], so the result is that of the clamped offsets."""
    g = np.random.Generator(np.random.PCG64(710))
    R, N, K = 200, 256, 256
    run_grouped_case(g, [-5, 40, 40, 100, R + 50], np.array([0, 40, 40, 100, R]), R, N, K)


def test_grouped_gemm_most_groups():
    """G = 4096 (the largest accepted), most groups empty, 1000 rows spread
    over 60 of them: every block scans the whole offset array."""
    g = np.random.Generator(np.random.PCG64(711))
    G, N, K = 4096, 256, 128
    sizes = np.zeros(G, np.int64)
    live = np.sort(g.choice(G, 60, replace=False))
    sizes[live] = g.multinomial(1000 - 60, np.full(60, 1 / 60)) + 1
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    run_grouped_case(g, off, off, int(off[-1]) + 7, N, K)


# ---------------------------------------------------- GEMM, precise mode

FP8_PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


@pytest.mark.parametrize("fa,fb", FP8_PAIRS)
@pytest.mark.parametrize("ma,mb", [(1, 1), (0, 0), (2, 1), (0, 1)])
def test_gemm_precise_within_1e5(fa, fb, ma, mb):
    """MXQ_OUT_PRECISE: the same random codes over each FP8 format's whole
    range, now held to 1e-5 of the fp64 oracle (elementwise and normwise)."""
    g = np.random.Generator(np.random.PCG64(1600 + fa * 10 + fb + ma * 100 + mb * 1000))
    M, N, K = 160, 200, 384
    A, sA = rand_operand(g, fa, ma, M, K)
    B, sB = rand_operand(g, fb, mb, N, K)
    C = run_gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K, out=mxq.OUT_PRECISE)
    Cref, Cabs = O.gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K)
    check_gemm(C, Cref, Cabs, f"precise f{fa}{fb} m{ma}{mb}")


def test_gemm_precise_wide_scales_nan_and_bf16_out():
    """Scale bytes over 80..170 (dequantized operands from about 2^-63 to
    2^59, sums up to about 2^110, inside fp32), a NaN code and a NaN scale,
    fp32 and bf16 outputs."""
    g = np.random.Generator(np.random.PCG64(1650))
    M, N, K = 96, 160, 512
    A, _ = rand_operand(g, 0, 1, M, K)
    B, _ = rand_operand(g, 1, 1, N, K)
    sA = g.integers(80, 171, size=(M, K // 32), dtype=np.uint8)
    sB = g.integers(80, 171, size=(N, K // 32), dtype=np.uint8)
    A[5, 17] = 0x7F
    sB[9, 3] = 0xFF
    C = run_gemm(A, 0, sA, 1, B, 1, sB, 1, M, N, K, out=mxq.OUT_PRECISE)
    Cref, Cabs = O.gemm(A, 0, sA, 1, B, 1, sB, 1, M, N, K)
    check_gemm(C, Cref, Cabs, "precise wide")
    Cb = run_gemm(A, 0, sA, 1, B, 1, sB, 1, M, N, K, out=mxq.OUT_BF16 | mxq.OUT_PRECISE)
    Cf = (Cb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok = ~np.isnan(Cref)
    assert np.array_equal(np.isnan(Cf), ~ok)
    # bf16 keeps 8 significant bits: RNE moves a value by at most 2^-8 of itself
    assert np.all(np.abs(Cf - Cref)[ok] <= (2.0 ** -8 * np.abs(Cref) + 2e-5 * Cabs)[ok])


def test_gemm_precise_tiny_operands():
    """Dequantized A operands between 2^-130 and 2^-118 (scale bytes 0..8,
    byte 0 being 2^-127) against B near 2^123: every A value is a multiple of
    2^-130, so its bf16 form is exact, subnormal or not, and so is the sum."""
    g = np.random.Generator(np.random.PCG64(1660))
    M, N, K = 64, 96, 256
    A = g.integers(0x38, 0x40, size=(M, K), dtype=np.uint8)          # E4M3 values in [1, 2)
    A[g.random((M, K)) < 0.5] |= 0x80
    sA = g.integers(0, 9, size=(M, K // 32), dtype=np.uint8)
    B = g.integers(0x38, 0x40, size=(N, K), dtype=np.uint8)
    sB = g.integers(245, 252, size=(N, K // 32), dtype=np.uint8)
    C = run_gemm(A, 0, sA, 1, B, 0, sB, 1, M, N, K, out=mxq.OUT_PRECISE)
    Cref, Cabs = O.gemm(A, 0, sA, 1, B, 0, sB, 1, M, N, K)
    check_gemm(C, Cref, Cabs, "precise tiny")


@pytest.mark.parametrize("ma,mb", [(2, 1), (1, 1), (0, 0)])
def test_grouped_gemm_precise(ma, mb):
    """Grouped precise mode with BLK128 x BLK32 scales (the general kernel),
    BLK32 on both operands (the kernel specialised for them) and per-tensor
    factors on both (one factor for every group's B)."""
    g = np.random.Generator(np.random.PCG64([1700, ma, mb]))
    G, N, K = 5, 192, 384
    sizes = [40, 0, 131, 7, 64]
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1])
    A, sA = rand_operand(g, 0, ma, R, K)
    Bs = [rand_operand(g, 0, mb, N, K) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = Bs[0][1] if mb == 0 else np.stack([s for _, s in Bs])
    C = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_scaled_gemm(dev_u8(A), 0, gemm_scale_arg(sA, ma), ma, dev_u8(B), 0, gemm_scale_arg(sB, mb), mb,
                            torch.from_numpy(off).cuda(), G, R, N, K, C, out=mxq.OUT_PRECISE)
    m_idx = np.repeat(np.arange(R), N)
    n_idx = np.tile(np.arange(N), R)
    c, cabs = O.grouped_gemm_entries(A, 0, sA, ma, B, 0, sB, mb, off, N, K, m_idx, n_idx)
    check_gemm(host(C), c.reshape(-1, N), cabs.reshape(-1, N), f"grouped precise m{ma}{mb}")


@pytest.mark.parametrize("out", [0, 16])
def test_gemm_blk128_last_row_in_partial_word(out):
    """BLK128 A of 131 rows, K = 384: 393 scale bytes, so the last row's
    bytes sit in a 4-byte word that the array only partly covers."""
    g = np.random.Generator(np.random.PCG64(1750 + out))
    M, N, K = 131, 64, 384
    A, sA = rand_operand(g, 0, 2, M, K)
    B, sB = rand_operand(g, 1, 1, N, K)
    C = run_gemm(A, 0, sA, 2, B, 1, sB, 1, M, N, K, out=out)
    Cref, Cabs = O.gemm(A, 0, sA, 2, B, 1, sB, 1, M, N, K)
    hb = None if out else full_bound(A, 0, sA, 2, B, 1, sB, 1, M, N, K)
    check_gemm(C, Cref, Cabs, f"blk128 partial word out={out}", hw_bound=hb)


def test_gemm_deterministic():
    g = np.random.Generator(np.random.PCG64(800))
    M, N, K = 256, 384, 1024
    A, sA = rand_operand(g, 0, 1, M, K)
    B, sB = rand_operand(g, 1, 1, N, K)
    C1 = run_gemm(A, 0, sA, 1, B, 1, sB, 1, M, N, K)
    C2 = run_gemm(A, 0, sA, 1, B, 1, sB, 1, M, N, K)
    assert np.array_equal(C1.view(np.uint32), C2.view(np.uint32))
