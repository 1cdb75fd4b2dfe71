"""GPU parity past the 32-bit index ranges.

Each kernel runs on a tensor of more than 2^31 elements (or, for the GEMM, an
operand just under its 4 GiB addressing limit), so that any 32-bit element or
byte offset in a kernel would wrap.  The inputs come from torch's seeded
device generator; the oracle checks sampled rows and columns, chosen on both
sides of element 2^31 and at the very end, bit for bit (GEMM entries within
the MFMA's own bound).
"""
import numpy as np
import pytest
import torch

import oracle as O
import mxfp4_precision_numerics_amd as mxq
from gpu_helpers import check_gemm, check_swiglu_codes, host, mfma_bound, require_gpu

pytestmark = pytest.mark.gpu

# 65600 x 32768 = 2,149,580,800 elements; row 65536 starts at element 2^31
ROWS, COLS = 65600, 32768


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    O.lib()
    yield
    torch.cuda.empty_cache()


def log(*a):
    print(*a, flush=True)


def gen(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def pick(g, n, fixed, k):
    extra = g.integers(0, n, k)
    return np.unique(np.concatenate([np.asarray(fixed), extra])).astype(np.int64)


def rows_of(t, idx):
    return host(t.index_select(0, torch.from_numpy(idx).cuda()))


def cols_of(t, idx):
    return host(t.index_select(1, torch.from_numpy(idx).cuda()).contiguous())


def big_bf16(seed, row_binades=0):
    x = torch.randn((ROWS, COLS), dtype=torch.bfloat16, device="cuda", generator=gen(seed))
    if row_binades:
        k = torch.randint(-row_binades, row_binades + 1, (ROWS, 1), device="cuda", generator=gen(seed + 1))
        x.mul_(torch.exp2(k.float()).to(torch.bfloat16))  # powers of two: exact in bf16
    return x


def host_amax_bf16(x):
    """max |x| of a NaN-free bf16 device tensor, on the host in chunks."""
    flat = x.view(-1)
    m = 0
    for c in flat.split(1 << 28):
        b = host(c)
        m = max(m, int((b & 0x7FFF).max()))
    return np.array([m << 16], np.uint32).view(np.float32)[0]


@pytest.mark.parametrize("fmt", [0, 1])
def test_per_tensor_current_scaling_past_2_31(fmt):
    """Current scaling (amax pass + row and column casts) on 2.15e9 bf16
    elements: amax, scale, scale_inv and sampled rows and columns."""
    x = big_bf16(70 + fmt)
    amax, sc, si = (torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(3))
    q_row = torch.empty((ROWS, COLS), dtype=torch.uint8, device="cuda")
    q_col = torch.empty((COLS, ROWS), dtype=torch.uint8, device="cuda")
    mxq.quantize_per_tensor(x, fmt, amax, sc, si, q_row, q_col)
    log(f"per-tensor fmt{fmt}: launched")
    ref_amax = host_amax_bf16(x)
    assert host(amax)[0] == ref_amax
    hist = np.array([ref_amax], np.float32)  # delayed scaling from the same amax gives the same scale
    g = np.random.Generator(np.random.PCG64(71))
    r = pick(g, ROWS, [0, 1, 65535, 65536, 65537, ROWS - 1], 10)
    exp = O.quantize_per_tensor(rows_of(x, r), fmt, history=hist.copy(), row=True)
    assert host(sc)[0] == exp["scale"] and host(si)[0] == exp["scale_inv"]
    assert exp["scale"] == O.scale_from_amax(fmt, ref_amax)
    assert np.array_equal(rows_of(q_row, r), exp["q_row"])
    c = pick(g, COLS, [0, 31, 16384, COLS - 1], 12)
    exp = O.quantize_per_tensor(cols_of(x, c), fmt, history=hist.copy(), row=False, col=True)
    assert np.array_equal(rows_of(q_col, c), exp["q_col"])
    log(f"per-tensor fmt{fmt}: {len(r)} rows and {len(c)} columns bit-exact")


@pytest.mark.parametrize("fmt,col", [(2, False), (0, True)])
def test_mx_past_2_31(fmt, col):
    """MX block-32 quantization, row-only E2M1 (one pass) and row + column
    E4M3 (the tiled two-output kernel), rows spread over 41 binades."""
    x = big_bf16(80 + fmt, row_binades=20)
    q_row = torch.empty((ROWS, COLS // 2 if fmt == 2 else COLS), dtype=torch.uint8, device="cuda")
    s_row = torch.empty((ROWS, COLS // 32), dtype=torch.uint8, device="cuda")
    q_col = s_col = None
    if col:
        q_col = torch.empty((COLS, ROWS), dtype=torch.uint8, device="cuda")
        s_col = torch.empty((COLS, ROWS // 32), dtype=torch.uint8, device="cuda")
    mxq.quantize_mx(x, fmt, q_row, s_row, q_col, s_col)
    log(f"mx fmt{fmt} col={col}: launched")
    g = np.random.Generator(np.random.PCG64(81))
    r = pick(g, ROWS, [0, 65535, 65536, ROWS - 1], 12)
    oq, os_, _, _ = O.quantize_mx(rows_of(x, r), fmt, row=True)
    assert np.array_equal(rows_of(s_row, r), os_)
    assert np.array_equal(rows_of(q_row, r), oq)
    if col:
        c = pick(g, COLS, [0, 16384, COLS - 1], 12)
        _, _, oqc, osc = O.quantize_mx(cols_of(x, c), fmt, row=False, col=True)
        assert np.array_equal(rows_of(s_col, c), osc)
        assert np.array_equal(rows_of(q_col, c), oqc)
    log(f"mx fmt{fmt} col={col}: sampled rows{' and columns' if col else ''} bit-exact")


def test_fp4_row_to_fp8_col_past_2_31():
    """FP4 rows [65568, 32768] -> FP8 columns [32768, 65568]: 2.15e9 output
    bytes; sampled 32-column blocks (the oracle needs whole columns)."""
    rows = 65568
    g_d = gen(90)
    q4 = torch.randint(0, 256, (rows, COLS // 2), dtype=torch.uint8, device="cuda", generator=g_d)
    s4 = torch.randint(100, 160, (rows, COLS // 32), dtype=torch.uint8, device="cuda", generator=g_d)
    q8 = torch.empty((COLS, rows), dtype=torch.uint8, device="cuda")
    s8 = torch.empty((COLS, rows // 32), dtype=torch.uint8, device="cuda")
    mxq.fp4_row_to_fp8_col(q4, s4, q8, s8)
    g = np.random.Generator(np.random.PCG64(91))
    for b in pick(g, COLS // 32, [0, 512, COLS // 32 - 1], 3):
        oq, os_ = O.fp4_row_to_fp8_col(host(q4[:, 16 * b:16 * b + 16].contiguous()),
                                       host(s4[:, b:b + 1].contiguous()))
        assert np.array_equal(host(s8[32 * b:32 * b + 32]), os_), b
        assert np.array_equal(host(q8[32 * b:32 * b + 32]), oq), b
    log("fp4 row -> fp8 col: sampled column blocks bit-exact")


def test_repack_gather_past_2_31():
    """Gathered FP4 -> FP8 repack into 300,000 rows x 7168 (2.15e9 bytes)."""
    src_rows, cols, rows = 8192, 7168, 300000
    g_d = gen(100)
    q4 = torch.randint(0, 256, (src_rows, cols // 2), dtype=torch.uint8, device="cuda", generator=g_d)
    s4 = torch.randint(110, 140, (src_rows, cols // 32), dtype=torch.uint8, device="cuda", generator=g_d)
    idx = torch.randint(0, src_rows, (rows,), dtype=torch.int32, device="cuda", generator=g_d)
    q8 = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s8 = torch.empty((rows, cols // 128), dtype=torch.uint8, device="cuda")
    mxq.repack_fp4_to_fp8(q4, s4, q8, s8, gather_idx=idx)
    g = np.random.Generator(np.random.PCG64(101))
    r = pick(g, rows, [0, 299520, rows - 1], 16)  # row 299520 starts past byte 2^31
    oq, os_ = O.repack_fp4_to_fp8(host(q4), host(s4), idx=host(idx)[r])
    assert np.array_equal(rows_of(s8, r), os_)
    assert np.array_equal(rows_of(q8, r), oq)
    log("repack with gather: sampled rows bit-exact")


def test_swiglu_past_2_31():
    """SwiGLU + MX E4M3 on gate|up [1048640, 4096] bf16: h has 2.15e9
    elements."""
    rows, inter = 1048640, 2048
    gu = torch.randn((rows, 2 * inter), dtype=torch.bfloat16, device="cuda", generator=gen(110)).mul_(1.6875)
    q = torch.empty((rows, inter), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, inter // 32), dtype=torch.uint8, device="cuda")
    mxq.swiglu_quantize_mx(gu, inter, 0, q, s)
    g = np.random.Generator(np.random.PCG64(111))
    r = pick(g, rows, [0, 1048575, 1048576, rows - 1], 12)  # row 2^20 starts at element 2^31 of h
    check_swiglu_codes(rows_of(q, r), rows_of(s, r), rows_of(gu, r), inter, 0, "swiglu past 2^31")
    log("swiglu: sampled rows within the checker's bound")


def test_gemm_operand_just_under_4gib():
    """MXFP8 GEMM with A = 524,272 x 8192 bytes (4 GiB - 128 KiB), the
    largest operand the 32-bit buffer offsets address; sampled rows of C
    (all 512 columns) at the start, around byte 2^31 and at the end."""
    M, N, K = 524272, 512, 8192
    g_d = gen(120)

    def operand(rows):
        q = torch.randint(0, 256, (rows, K), dtype=torch.uint8, device="cuda", generator=g_d)
        q.sub_(((q & 0x7F) == 0x7F).to(torch.uint8))  # NaN codes -> the largest finite code
        s = torch.randint(118, 136, (rows, K // 32), dtype=torch.uint8, device="cuda", generator=g_d)
        return q, s

    A, sA = operand(M)
    B, sB = operand(N)
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mxq.scaled_gemm(A, 0, sA, mxq.SCALE_BLK32, B, 0, sB, mxq.SCALE_BLK32, M, N, K, C)
    g = np.random.Generator(np.random.PCG64(121))
    r = pick(g, M, [0, 262143, 262144, M - 129, M - 1], 7)
    Ah, sAh, Bh, sBh = rows_of(A, r), rows_of(sA, r), host(B), host(sB)
    m_idx = np.repeat(np.arange(len(r)), N)
    n_idx = np.tile(np.arange(N), len(r))
    got = rows_of(C, r).reshape(-1).astype(np.float64)
    ref, absum = O.gemm_entries(Ah, 0, sAh, 1, Bh, 0, sBh, 1, K, m_idx, n_idx)
    hb = mfma_bound(Ah, 0, sAh, 1, Bh, 0, sBh, 1, K, m_idx, n_idx)
    ratio = check_gemm(got, ref, absum, "gemm 4 GiB operand", hw_bound=hb)
    log(f"gemm A just under 4 GiB: {len(r)} rows x {N} within the MFMA bound (err / 1e-5 sum|ab| = {ratio:.3f})")
