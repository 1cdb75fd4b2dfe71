"""ctypes wrapper of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
cpu_baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library and never imports it.

All arrays are numpy, C-contiguous.  bf16 inputs are passed as their uint16
bit patterns.  Codes and E8M0 scale bytes are uint8.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# MXQ_ORACLE_LIB selects another build of oracle.c (the sanitizer build of
# the CPU hygiene tests); the default is the optimized one.
_LIB_PATH = os.environ.get("MXQ_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

E4M3, E5M2, E2M1 = 0, 1, 2
SRC_F32, SRC_BF16, SRC_F64 = 0, 1, 2  # float64 input: MX quantizer only
SCALE_TENSOR, SCALE_BLK32, SCALE_BLK128 = 0, 1, 2

_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.or_num_threads.restype = ctypes.c_int
        L.or_num_threads.argtypes = []
        L.or_value.restype = ctypes.c_double
        L.or_value.argtypes = [_i, ctypes.c_uint]
        L.or_e8m0_value.restype = ctypes.c_double
        L.or_e8m0_value.argtypes = [ctypes.c_uint]
        L.or_cast.restype = ctypes.c_uint
        L.or_cast.argtypes = [_i, ctypes.c_double]
        L.or_cast_array.restype = None
        L.or_cast_array.argtypes = [_i, _p, _i64, _p]
        L.or_max_finite.restype = ctypes.c_double
        L.or_max_finite.argtypes = [_i]
        L.or_emax.restype = _i
        L.or_emax.argtypes = [_i]
        L.or_amax.restype = ctypes.c_float
        L.or_amax.argtypes = [_p, _i, _i64, _i64, _i64]
        L.or_scale_from_amax.restype = ctypes.c_float
        L.or_scale_from_amax.argtypes = [_i, ctypes.c_float]
        L.or_history_amax.restype = ctypes.c_float
        L.or_history_amax.argtypes = [_p, _i]
        L.or_history_push.restype = None
        L.or_history_push.argtypes = [_p, _i, ctypes.c_float]
        L.or_quantize_per_tensor.restype = None
        L.or_quantize_per_tensor.argtypes = [_p, _i, _i64, _i64, _i64, _i, _p, _i, _p, _p, _p, _p, _p]
        L.or_quantize_mx.restype = None
        L.or_quantize_mx.argtypes = [_p, _i, _i64, _i64, _i64, _i, _p, _p, _p, _p]
        L.or_repack_fp4_to_fp8.restype = None
        L.or_repack_fp4_to_fp8.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p, _p]
        L.or_fp4_row_to_fp8_col.restype = None
        L.or_fp4_row_to_fp8_col.argtypes = [_p, _p, _i64, _i64, _p, _p]
        L.or_dequant.restype = ctypes.c_double
        L.or_dequant.argtypes = [_p, _i, _p, _i, _i64, _i64, _i64]
        L.or_gemm_entries.restype = None
        L.or_gemm_entries.argtypes = [_p, _i, _p, _i, _p, _i, _p, _i, _i64, _p, _p, _i64, _p, _p]
        L.or_gemm.restype = None
        L.or_gemm.argtypes = [_p, _i, _p, _i, _p, _i, _p, _i, _i64, _i64, _i64, _p, _p]
        L.or_grouped_gemm_entries.restype = None
        L.or_grouped_gemm_entries.argtypes = [_p, _i, _p, _i, _p, _i, _p, _i, _p, _i64, _i64, _i64,
                                              _p, _p, _i64, _p, _p]
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _src_of(x):
    if x.dtype == np.float32:
        return SRC_F32
    if x.dtype == np.uint16:
        return SRC_BF16
    if x.dtype == np.float64:
        return SRC_F64
    raise TypeError("oracle input must be float32, float64 or uint16 (bf16 bits)")


# --- O1/O2 ---------------------------------------------------------------

def value(fmt, code):
    return lib().or_value(fmt, int(code))


def e8m0_value(b):
    return lib().or_e8m0_value(int(b))


def cast(fmt, v):
    return lib().or_cast(fmt, float(v))


def max_finite(fmt):
    return lib().or_max_finite(fmt)


def emax(fmt):
    return lib().or_emax(fmt)


def decode_table(fmt):
    n = 16 if fmt == E2M1 else 256
    return np.array([value(fmt, c) for c in range(n)], dtype=np.float64)


def cast_array(fmt, v):
    """cast_F of each element of an array (taken as float64)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().or_cast_array(fmt, _ptr(v), v.size, _ptr(out))
    return out


# --- O3/O4/O5 ------------------------------------------------------------

def amax(x):
    x = np.ascontiguousarray(x)
    r, c = x.shape
    return lib().or_amax(_ptr(x), _src_of(x), r, c, c)


def scale_from_amax(fmt, a):
    return lib().or_scale_from_amax(fmt, float(a))


def history_amax(history):
    h = np.ascontiguousarray(history, dtype=np.float32)
    return lib().or_history_amax(_ptr(h), len(h))


def quantize_per_tensor(x, fmt, history=None, row=True, col=False):
    """Returns dict(amax, scale, scale_inv, q_row, q_col); ``history`` (float32
    array, updated in place) selects delayed scaling."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    out = {}
    amax_o = np.zeros(1, np.float32)
    sc = np.zeros(1, np.float32)
    si = np.zeros(1, np.float32)
    q_row = np.empty((rows, cols), np.uint8) if row else None
    q_col = np.empty((cols, rows), np.uint8) if col else None
    if history is not None:
        assert history.dtype == np.float32 and history.flags["C_CONTIGUOUS"]
    lib().or_quantize_per_tensor(_ptr(x), _src_of(x), rows, cols, cols, fmt,
                                 _ptr(history), 0 if history is None else len(history),
                                 _ptr(amax_o), _ptr(sc), _ptr(si), _ptr(q_row), _ptr(q_col))
    out.update(amax=amax_o[0], scale=sc[0], scale_inv=si[0], q_row=q_row, q_col=q_col)
    return out


# --- O6 --------------------------------------------------------------------

def quantize_mx(x, fmt, row=True, col=False):
    """Returns (q_row, s_row, q_col, s_col); unrequested outputs are None.
    ``x`` is bf16 bits (uint16), float32 or float64."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q_row = s_row = q_col = s_col = None
    if row:
        assert cols % 32 == 0
        q_row = np.zeros((rows, cols // 2 if fmt == E2M1 else cols), np.uint8)
        s_row = np.zeros((rows, cols // 32), np.uint8)
    if col:
        assert rows % 32 == 0
        q_col = np.zeros((cols, rows // 2 if fmt == E2M1 else rows), np.uint8)
        s_col = np.zeros((cols, rows // 32), np.uint8)
    lib().or_quantize_mx(_ptr(x), _src_of(x), rows, cols, cols, fmt,
                         _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col))
    return q_row, s_row, q_col, s_col


# --- expert MLP activation ----------------------------------------------------

def as_f64(x):
    """bf16 bits (uint16) or float32 -> float64 (exact)."""
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def silu(x):
    """SiLU (swish) x * sigma(x) = x / (1 + e^-x), float64 (NaN stays NaN,
    -inf gives NaN like inf/inf, +inf gives +inf)."""
    with np.errstate(over="ignore", invalid="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(gu, inter):
    """SwiGLU activation of a gate/up projection output ``gu`` [rows, >= 2
    inter] (bf16 bits or float32): h = silu(gate) * up, gate in columns
    [0, inter), up in [inter, 2 inter), float64 [rows, inter]."""
    v = as_f64(np.ascontiguousarray(gu))
    with np.errstate(invalid="ignore", over="ignore"):
        return silu(v[:, :inter]) * v[:, inter:2 * inter]


def swiglu_quantize_mx(gu, inter, fmt):
    """The expert MLP's activation step: h = swiglu(gu) in float64, then MX
    block-32 quantization along the intermediate dimension (O6 on the
    float64 values).  Returns (q [rows, inter], s [rows, inter/32], h)."""
    h = np.ascontiguousarray(swiglu(gu, inter))
    q, s, _, _ = quantize_mx(h, fmt)
    return q, s, h


# --- O7 --------------------------------------------------------------------

def repack_fp4_to_fp8(q4, s4, idx=None, rows=None):
    q4 = np.ascontiguousarray(q4, dtype=np.uint8)
    s4 = np.ascontiguousarray(s4, dtype=np.uint8)
    src_rows = q4.shape[0]
    cols = q4.shape[1] * 2
    assert cols % 128 == 0 and s4.shape == (src_rows, cols // 32)
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        rows = len(idx)
    elif rows is None:
        rows = src_rows
    q8 = np.empty((rows, cols), np.uint8)
    s8 = np.empty((rows, cols // 128), np.uint8)
    lib().or_repack_fp4_to_fp8(_ptr(q4), _ptr(s4), _ptr(idx), src_rows, rows, cols, _ptr(q8), _ptr(s8))
    return q8, s8


# --- O7b -------------------------------------------------------------------

def fp4_row_to_fp8_col(q4, s4):
    """MXFP4 rows [rows, cols] -> MX E4M3 columns: (q8 [cols, rows], s8 [cols, rows/32])."""
    q4 = np.ascontiguousarray(q4, dtype=np.uint8)
    s4 = np.ascontiguousarray(s4, dtype=np.uint8)
    rows, cols = q4.shape[0], q4.shape[1] * 2
    assert rows % 32 == 0 and cols % 32 == 0 and s4.shape == (rows, cols // 32)
    q8 = np.empty((cols, rows), np.uint8)
    s8 = np.empty((cols, rows // 32), np.uint8)
    lib().or_fp4_row_to_fp8_col(_ptr(q4), _ptr(s4), rows, cols, _ptr(q8), _ptr(s8))
    return q8, s8


# --- O8/O9 -----------------------------------------------------------------

def _scale_arg(s, mode):
    if mode == SCALE_TENSOR:
        return np.ascontiguousarray(np.asarray(s, dtype=np.float32).reshape(1))
    return np.ascontiguousarray(s, dtype=np.uint8)


def dequant(q, fmt, s, mode, K, i, k):
    s = _scale_arg(s, mode)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    return lib().or_dequant(_ptr(q), fmt, _ptr(s), mode, K, i, k)


def dequant_matrix(q, fmt, s, mode, rows, K):
    """Whole dequantized operand as float64 [rows, K] (small shapes)."""
    s = _scale_arg(s, mode)
    q = np.ascontiguousarray(q, dtype=np.uint8)
    L = lib()
    out = np.empty((rows, K), np.float64)
    for i in range(rows):
        for k in range(K):
            out[i, k] = L.or_dequant(_ptr(q), fmt, _ptr(s), mode, K, i, k)
    return out


def gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K):
    """Full C [M,N] and sum|a||b| [M,N] in float64 (small shapes)."""
    sA = _scale_arg(sA, ma)
    sB = _scale_arg(sB, mb)
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    C = np.empty((M, N), np.float64)
    Cabs = np.empty((M, N), np.float64)
    lib().or_gemm(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, M, N, K, _ptr(C), _ptr(Cabs))
    return C, Cabs


def gemm_entries(A, fa, sA, ma, B, fb, sB, mb, K, m_idx, n_idx):
    sA = _scale_arg(sA, ma)
    sB = _scale_arg(sB, mb)
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    c = np.empty(len(m_idx), np.float64)
    cabs = np.empty(len(m_idx), np.float64)
    lib().or_gemm_entries(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, K,
                          _ptr(m_idx), _ptr(n_idx), len(m_idx), _ptr(c), _ptr(cabs))
    return c, cabs


def grouped_gemm_entries(A, fa, sA, ma, B, fb, sB, mb, off, N, K, m_idx, n_idx):
    sA = _scale_arg(sA, ma)
    sB = _scale_arg(sB, mb)
    A = np.ascontiguousarray(A, dtype=np.uint8)
    B = np.ascontiguousarray(B, dtype=np.uint8)
    off = np.ascontiguousarray(off, dtype=np.int64)
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    c = np.empty(len(m_idx), np.float64)
    cabs = np.empty(len(m_idx), np.float64)
    lib().or_grouped_gemm_entries(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, _ptr(off),
                                  len(off) - 1, N, K, _ptr(m_idx), _ptr(n_idx), len(m_idx),
                                  _ptr(c), _ptr(cabs))
    return c, cabs


def expert_up_swiglu_mx(A, fa, sA, ma, B, fb, sB, mb, off, inter, K, rows, hfmt):
    """The expert MLP's up-projection followed by its activation step, for
    the listed rows of A ([MoE FP4] "Metodologia": the expert GEMMs in FP8,
    the activation between them requantized; activation read as SwiGLU):
    gate and up = the grouped GEMM (O9, fp64 sums of exact products) over the
    2 inter columns of each row's group (gate columns [0, inter), up
    [inter, 2 inter)), then h = silu(gate) * up in fp64 and MX block-32
    quantization of h (O6).  Rows must lie in a group.  Returns (q [n, inter],
    s [n, inter/32], h [n, inter], gu [n, 2 inter], gu_abs [n, 2 inter]), the
    last being sum |a||b| of each gate/up entry."""
    rows = np.asarray(rows, np.int64)
    N = 2 * inter
    m_idx = np.repeat(rows, N)
    n_idx = np.tile(np.arange(N, dtype=np.int64), len(rows))
    c, cabs = grouped_gemm_entries(A, fa, sA, ma, B, fb, sB, mb, off, N, K, m_idx, n_idx)
    gu = c.reshape(len(rows), N)
    q, s, h = swiglu_quantize_mx(gu, inter, hfmt)
    return q, s, h, gu, cabs.reshape(len(rows), N)


def num_threads():
    """OpenMP threads the oracle's loops run on."""
    return int(lib().or_num_threads())
