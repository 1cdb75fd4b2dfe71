"""GPU parity of the GEMM on the tile shapes and ring lengths of the large
workloads, at sizes where the oracle checks sampled entries in seconds.

 * 256 x 256 tiles (and the 128 x 256 tiles of a last-round launch) in both
   modes, ragged in M and N, with K long enough that every ring slot is
   refilled several times: FP8 x FP8, FP4 x FP4 (units of two K steps, also
   with K % 256 == 128, where the last unit is half a unit) and mixed
   FP4 x FP8 (units of one K half, more units than ring slots).
 * The split launch (256 x 256 tiles over the columns of whole rounds, a
   128 x 256 launch for the rest) gives the same bits as unsplit calls over
   the same columns, which run other tile shapes: each element's sum is the
   same instruction sequence whatever the tile.
 * Grouped GEMM with MXFP4 operands at K = 7168 (the expert GEMM's depth),
   for both the 256-row and the 128-row tile choices.
 * Grouped GEMM on the 320 x 192 tiles (groups averaging 225-320 rows, one
   tile per group up to 320 rows, two above): every group's rows equal, bit
   for bit, a dense call on that group alone (other tile shapes, the same
   per-element instruction sequence), and sampled entries meet the oracle.

Tolerances: the precise mode and FP4 x FP4 (whose products fit the FP8
MFMA's alignment window) are held to 1e-5 (REL_TOL); FP8 operands through the
block-scaled FP8 MFMA to the instruction's derived bound (random codes span
each format's whole range, which is where that bound and 1e-5 part).
"""
import numpy as np
import pytest
import torch

import oracle as O
import mxfp4_precision_numerics_amd as mxq
from gpu_helpers import check_gemm, dev_u8, gemm_scale_arg, host, mfma_bound, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    O.lib()


def log(*a):
    print(*a, flush=True)


def rand_operand(g, fmt, mode, rows, K):
    """Random codes over the format's whole finite range; BLK32/BLK128 scale
    bytes in 110..139, or one per-tensor factor."""
    if fmt == 2:
        q = g.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    else:
        q = g.integers(0, 256, size=(rows, K), dtype=np.uint8)
        top = 0x7F if fmt == 0 else 0x7C
        q[(q & 0x7F) >= top] &= 0x3F
    if mode == 0:
        s = np.float32(g.uniform(0.01, 3.0))
    else:
        s = g.integers(110, 140, size=(rows, K // (32 if mode == 1 else 128)), dtype=np.uint8)
    return q, s


def sample_entries(g, M, N, n=3000, tile=256):
    """Random entries plus the last row and column, and rows and columns on
    both sides of every tile edge."""
    edges_m = np.unique(np.clip(np.concatenate([np.arange(0, M, tile) - 1, np.arange(0, M, tile)]), 0, M - 1))
    edges_n = np.unique(np.clip(np.concatenate([np.arange(0, N, tile) - 1, np.arange(0, N, tile)]), 0, N - 1))
    m = np.concatenate([g.integers(0, M, n), np.full(64, M - 1), g.choice(edges_m, 256),
                        g.integers(0, M, 64)])
    k = np.concatenate([g.integers(0, N, n), g.integers(0, N, 64), g.integers(0, N, 256),
                        np.full(64, N - 1)])
    return m.astype(np.int64), k.astype(np.int64)


def run(A, fa, sA, ma, B, fb, sB, mb, M, N, K, out=0):
    C = torch.empty((M, N), dtype=torch.bfloat16 if out & mxq.OUT_BF16 else torch.float32, device="cuda")
    mxq.scaled_gemm(dev_u8(A), fa, gemm_scale_arg(sA, ma), ma, dev_u8(B), fb, gemm_scale_arg(sB, mb), mb,
                    M, N, K, C, out=out)
    return host(C)


def check_sampled(C, A, fa, sA, ma, B, fb, sB, mb, K, m, n, what, exact):
    got = C[m, n].astype(np.float64)
    ref, absum = O.gemm_entries(A, fa, sA, ma, B, fb, sB, mb, K, m, n)
    hb = None if exact else mfma_bound(A, fa, sA, ma, B, fb, sB, mb, K, m, n)
    r = check_gemm(got, ref, absum, what, hw_bound=hb)
    log(f"{what}: max |err| / (1e-5 sum|a||b|) = {r:.3f}")
    return r


# (fa, fb, ma, mb, K): FP8 pairs with every scale mode, FP4 x FP4 over whole and
# half last units, mixed FP4 x FP8 with many more units than slots
DENSE_CASES = [
    (0, 0, 1, 1, 1152),
    (1, 0, 0, 0, 1152),
    (0, 1, 2, 1, 1408),
    (1, 1, 1, 0, 1152),
    (2, 2, 1, 1, 2048),
    (2, 2, 1, 2, 2176),
    (2, 0, 1, 1, 1152),
    (0, 2, 2, 1, 1280),
]


@pytest.mark.parametrize("fa,fb,ma,mb,K", DENSE_CASES)
@pytest.mark.parametrize("precise", [False, True])
def test_gemm_256_tiles(fa, fb, ma, mb, K, precise):
    """M = 2100, N = 5400: 9 x 22 tiles of 256 x 256 (198, one launch; the
    last tile row holds 52 rows, the last column 24 columns)."""
    if precise and (fa == 2 or fb == 2):
        pytest.skip("the precise mode takes FP8 operands (E2M1 x E2M1 is exact natively)")
    g = np.random.Generator(np.random.PCG64([2000, fa, fb, ma, mb, K, int(precise)]))
    M, N = 2100, 5400
    A, sA = rand_operand(g, fa, ma, M, K)
    B, sB = rand_operand(g, fb, mb, N, K)
    C = run(A, fa, sA, ma, B, fb, sB, mb, M, N, K, out=mxq.OUT_PRECISE if precise else 0)
    m, n = sample_entries(g, M, N)
    exact = precise or (fa == 2 and fb == 2)
    check_sampled(C, A, fa, sA, ma, B, fb, sB, mb, K, m, n,
                  f"256x256 f{fa}{fb} m{ma}{mb} K={K} {'precise' if precise else 'native'}", exact)


@pytest.mark.parametrize("fa,fb,ma,mb,K", [(0, 0, 1, 1, 1024), (1, 0, 0, 0, 768), (2, 2, 1, 1, 2176)])
@pytest.mark.parametrize("precise", [False, True])
def test_gemm_split_launch_same_bits_as_unsplit(fa, fb, ma, mb, K, precise):
    """M = 2048, N = 8448: 264 tiles of 256 x 256 on 256 CUs, so the call runs
    the first 8192 columns as 256 x 256 tiles and the last 256 as a 128 x 256
    launch.  The same columns computed by separate calls (8192 columns: one
    whole round of 256 x 256 tiles; 256 columns: 128 x 128 tiles) give
    bit-identical results, and the whole is within tolerance."""
    if precise and (fa == 2 or fb == 2):
        pytest.skip("the precise mode takes FP8 operands")
    g = np.random.Generator(np.random.PCG64([2100, fa, fb, ma, mb, K, int(precise)]))
    M, N, n1 = 2048, 8448, 8192
    out = mxq.OUT_PRECISE if precise else 0
    A, sA = rand_operand(g, fa, ma, M, K)
    B, sB = rand_operand(g, fb, mb, N, K)
    C = run(A, fa, sA, ma, B, fb, sB, mb, M, N, K, out=out)
    sB1 = sB if mb == 0 else np.ascontiguousarray(sB[:n1])
    sB2 = sB if mb == 0 else np.ascontiguousarray(sB[n1:])
    C1 = run(A, fa, sA, ma, np.ascontiguousarray(B[:n1]), fb, sB1, mb, M, n1, K, out=out)
    C2 = run(A, fa, sA, ma, np.ascontiguousarray(B[n1:]), fb, sB2, mb, M, N - n1, K, out=out)
    assert np.array_equal(C[:, :n1].view(np.uint32), C1.view(np.uint32)), "256x256 columns differ"
    assert np.array_equal(C[:, n1:].view(np.uint32), C2.view(np.uint32)), "128x256 columns differ"
    m, n = sample_entries(g, M, N, 2000)
    exact = precise or (fa == 2 and fb == 2)
    check_sampled(C, A, fa, sA, ma, B, fb, sB, mb, K, m, n,
                  f"split f{fa}{fb} K={K} {'precise' if precise else 'native'}", exact)


@pytest.mark.parametrize("sizes", [[300, 17, 256, 250, 211], [150, 0, 190, 120, 260, 97]])
def test_grouped_gemm_mxfp4_k7168(sizes):
    """MXFP4 x MXFP4 grouped GEMM at the expert GEMM's K = 7168: 28 ring units
    of two K steps through two slots.  The first group set averages more than
    192 rows (256-row tiles), the second fewer (128-row tiles).  FP4 x FP4
    products are exact in the MFMA, so 1e-5 holds."""
    g = np.random.Generator(np.random.PCG64([2200, len(sizes)]))
    G, N, K = len(sizes), 512, 7168
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
    Ch = host(C)
    m, n = sample_entries(g, R, N, 2500)
    c, cabs = O.grouped_gemm_entries(A, 2, sA, 1, B, 2, sB, 1, off, N, K, m, n)
    r = check_gemm(Ch[m, n].astype(np.float64), c, cabs, "grouped MXFP4 K=7168")
    log(f"grouped MXFP4 K=7168 sizes {sizes}: ratio {r:.3f}")


@pytest.mark.parametrize("fa,fb,ma,mb,out,K", [(0, 0, 1, 1, 0, 4224), (1, 0, 2, 1, 0, 4224), (0, 1, 1, 2, 1, 4224),
                                                (2, 2, 1, 1, 0, 4224), (0, 0, 1, 1, 1, 2176), (2, 2, 2, 1, 0, 2304)])
def test_grouped_gemm_320x192_tiles(fa, fb, ma, mb, out, K):
    """Groups of 300, 0, 250, 331, 229 and 280 rows (average 232: 320 x 192
    tiles; the 331-row group takes a 320-row and an 11-row tile), N = 504 (the
    last n-tile holds 120 columns), K = 4224 (33 K steps through a two-slot
    ring), 2176 or 2304 (the tile serves K >= 2048), fp32 or bf16 output."""
    sizes = [300, 0, 250, 331, 229, 280]
    g = np.random.Generator(np.random.PCG64([2300, fa, fb, ma, mb, out, K]))
    G, N = len(sizes), 504
    off = np.zeros(G + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    R = int(off[-1])
    A, sA = rand_operand(g, fa, ma, R, K)
    Bs = [rand_operand(g, fb, mb, N, K) for _ in range(G)]
    B = np.stack([b for b, _ in Bs])
    sB = np.stack([s for _, s in Bs])
    dt = torch.bfloat16 if out else torch.float32
    C = torch.full((R, N), 7.0, dtype=dt, device="cuda")
    mxq.grouped_scaled_gemm(dev_u8(A), fa, dev_u8(sA), ma, dev_u8(B), fb, dev_u8(sB), mb,
                            torch.from_numpy(off).cuda(), G, R, N, K, C, out=mxq.OUT_BF16 if out else mxq.OUT_F32)
    Ch = host(C)
    for gi in range(G):
        r0, r1 = int(off[gi]), int(off[gi + 1])
        if r1 == r0:
            continue
        Cg = run(np.ascontiguousarray(A[r0:r1]), fa, np.ascontiguousarray(sA[r0:r1]), ma, B[gi], fb, sB[gi], mb,
                 r1 - r0, N, K, out=mxq.OUT_BF16 if out else 0)
        view = np.uint16 if out else np.uint32
        assert np.array_equal(Ch[r0:r1].view(view), Cg.view(view)), f"group {gi}: grouped != dense"
    if out == 0:
        m, n = sample_entries(g, R, N, 2500, tile=320)
        c, cabs = O.grouped_gemm_entries(A, fa, sA, ma, B, fb, sB, mb, off, N, K, m, n)
        hb = None
        if not (fa == 2 and fb == 2):
            hb = np.empty(len(m))
            for gi in range(G):
                r0, r1 = int(off[gi]), int(off[gi + 1])
                sel = (m >= r0) & (m < r1)
                if sel.any():
                    hb[sel] = mfma_bound(A[r0:r1], fa, sA[r0:r1], ma, B[gi], fb, sB[gi], mb, K, m[sel] - r0, n[sel])
        r = check_gemm(Ch[m, n].astype(np.float64), c, cabs, f"grouped 320x192 f{fa}{fb} m{ma}{mb}", hw_bound=hb)
        log(f"grouped 320x192 f{fa}{fb} m{ma}{mb}: ratio {r:.3f}")
