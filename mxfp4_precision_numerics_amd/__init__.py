"""Thin Python binding of libmxq.so (the gfx950 HIP library behind include/mxq.h).

Argument marshalling only: every step of the path runs in the HIP kernels.
Tensors are torch tensors on the GPU (torch supplies device memory and the
current stream); each function passes their device pointers and the current
HIP stream to the C entry point of the same name (``mxq_<name>``) and raises
``MxqError`` on a non-zero status.  There is no CPU fallback: if the library
is not built, the first call raises.
"""
import ctypes
import dataclasses
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxq.so")

E4M3, E5M2, E2M1 = 0, 1, 2
SRC_F32, SRC_BF16 = 0, 1
SCALE_TENSOR, SCALE_BLK32, SCALE_BLK128 = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1
OUT_PRECISE = 16  # OR into `out`: exact products (see include/mxq.h)

_lib = None


class MxqError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def lib():
    """Load libmxq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python -m mxfp4_precision_numerics_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mxq_abi_version.restype = i
        L.mxq_abi_version.argtypes = []
        L.mxq_status_string.restype = ctypes.c_char_p
        L.mxq_status_string.argtypes = [i]
        L.mxq_quantize_per_tensor.restype = i
        L.mxq_quantize_per_tensor.argtypes = [p, i, i64, i64, i64, i, p, i, p, p, p, p, p, p]
        L.mxq_quantize_mx.restype = i
        L.mxq_quantize_mx.argtypes = [p, i, i64, i64, i64, i, p, p, p, p, p]
        L.mxq_repack_fp4_to_fp8.restype = i
        L.mxq_repack_fp4_to_fp8.argtypes = [p, p, p, i64, i64, i64, p, p, p]
        L.mxq_fp4_row_to_fp8_col.restype = i
        L.mxq_fp4_row_to_fp8_col.argtypes = [p, p, i64, i64, p, p, p]
        L.mxq_swiglu_quantize_mx.restype = i
        L.mxq_swiglu_quantize_mx.argtypes = [p, i, i64, i64, i64, i, p, p, p]
        L.mxq_scaled_gemm.restype = i
        L.mxq_scaled_gemm.argtypes = [p, i, p, i, p, i, p, i, i64, i64, i64, p, i, i64, p]
        L.mxq_grouped_scaled_gemm.restype = i
        L.mxq_grouped_scaled_gemm.argtypes = [p, i, p, i, p, i, p, i, p, i64, i64, i64, i64, p, i, p]
        _lib = L
    return _lib


def abi_version():
    return lib().mxq_abi_version()


def status_string(status):
    return lib().mxq_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn, st):
    if st != 0:
        raise MxqError(fn, st)


def _src_of(x):
    import torch
    if x.dtype == torch.bfloat16:
        return SRC_BF16
    if x.dtype == torch.float32:
        return SRC_F32
    raise TypeError("input must be bfloat16 or float32")


def quantize_per_tensor(x, fmt, amax_out, scale_out, scale_inv_out=None, q_row=None, q_col=None,
                        amax_history=None, stream=None):
    """amax + per-tensor scale + saturating RNE cast (mxq_quantize_per_tensor).
    ``x`` [rows, cols] (row pitch x.stride(0)); outputs are preallocated
    tensors; ``amax_history`` (float32 [len]) selects delayed scaling."""
    rows, cols = x.shape
    assert x.stride(1) == 1
    hl = 0 if amax_history is None else amax_history.numel()
    st = lib().mxq_quantize_per_tensor(_ptr(x), _src_of(x), rows, cols, x.stride(0), fmt, _ptr(amax_history), hl,
                                       _ptr(amax_out), _ptr(scale_out), _ptr(scale_inv_out), _ptr(q_row),
                                       _ptr(q_col), _stream(stream))
    _check("mxq_quantize_per_tensor", st)


def quantize_mx(x, fmt, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """MX block-32 quantization (mxq_quantize_mx) into preallocated outputs."""
    rows, cols = x.shape
    assert x.stride(1) == 1
    st = lib().mxq_quantize_mx(_ptr(x), _src_of(x), rows, cols, x.stride(0), fmt, _ptr(q_row), _ptr(s_row),
                               _ptr(q_col), _ptr(s_col), _stream(stream))
    _check("mxq_quantize_mx", st)


def repack_fp4_to_fp8(q4, s4, q8, s8, gather_idx=None, stream=None):
    """Direct MXFP4 -> E4M3/block-128 repack (mxq_repack_fp4_to_fp8)."""
    src_rows = q4.shape[0]
    cols = q4.shape[1] * 2
    rows = q8.shape[0]
    st = lib().mxq_repack_fp4_to_fp8(_ptr(q4), _ptr(s4), _ptr(gather_idx), src_rows, rows, cols, _ptr(q8),
                                     _ptr(s8), _stream(stream))
    _check("mxq_repack_fp4_to_fp8", st)


def fp4_row_to_fp8_col(q4, s4, q8, s8, stream=None):
    """MXFP4 rows [rows, cols] -> MX E4M3 columns q8 [cols, rows], s8
    [cols, rows/32] (mxq_fp4_row_to_fp8_col)."""
    rows, cols = q4.shape[0], q4.shape[1] * 2
    st = lib().mxq_fp4_row_to_fp8_col(_ptr(q4), _ptr(s4), rows, cols, _ptr(q8), _ptr(s8), _stream(stream))
    _check("mxq_fp4_row_to_fp8_col", st)


def swiglu_quantize_mx(gu, inter, fmt, q, s, stream=None):
    """h = silu(gate) * up of ``gu`` [rows, >= 2 inter] (gate columns [0,
    inter), up [inter, 2 inter)), MX block-32 quantized into q [rows, inter]
    and s [rows, inter/32] (mxq_swiglu_quantize_mx)."""
    rows = gu.shape[0]
    assert gu.stride(1) == 1
    st = lib().mxq_swiglu_quantize_mx(_ptr(gu), _src_of(gu), rows, inter, gu.stride(0), fmt, _ptr(q), _ptr(s),
                                      _stream(stream))
    _check("mxq_swiglu_quantize_mx", st)


def scaled_gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K, C, out=OUT_F32, ldc=None, stream=None):
    """C = deq(A) . deq(B)^T (mxq_scaled_gemm)."""
    ldc = C.stride(0) if ldc is None else ldc
    st = lib().mxq_scaled_gemm(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, M, N, K, _ptr(C), out, ldc,
                               _stream(stream))
    _check("mxq_scaled_gemm", st)


def grouped_scaled_gemm(A, fa, sA, ma, B, fb, sB, mb, group_off, G, total_rows, N, K, C, out=OUT_F32,
                        stream=None):
    """Ragged grouped GEMM over device offsets (mxq_grouped_scaled_gemm)."""
    st = lib().mxq_grouped_scaled_gemm(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, _ptr(group_off), G,
                                       total_rows, N, K, _ptr(C), out, _stream(stream))
    _check("mxq_grouped_scaled_gemm", st)


# --------------------------------------------------------------------------
# Delayed-scaling recipe (argument marshalling around quantize_per_tensor)

HYBRID = "HYBRID"  # E4M3 in the forward pass, E5M2 for gradients


@dataclasses.dataclass(frozen=True)
class DelayedScaling:
    """The delayed-scaling recipe of the FP8 guide ("Transformer Engine: a
    fundacao de software"): each step's scale comes from the largest amax of
    the previous ``amax_history_len`` steps (``amax_compute_algo="max"``)
    with margin 0; ``fmt`` HYBRID casts forward tensors to E4M3 and
    gradients to E5M2.  The library computes scale = F_max / amax, so only
    margin 0 and the "max" reduction are accepted."""
    margin: int = 0
    fmt: str = HYBRID
    amax_history_len: int = 16
    amax_compute_algo: str = "max"

    def __post_init__(self):
        if self.margin != 0:
            raise ValueError("only margin 0 is supported")
        if self.amax_compute_algo != "max":
            raise ValueError("only amax_compute_algo='max' is supported")
        if self.fmt not in (HYBRID, "E4M3", "E5M2"):
            raise ValueError("fmt must be HYBRID, E4M3 or E5M2")
        if not 1 <= self.amax_history_len <= 1024:
            raise ValueError("amax_history_len must be in 1 .. 1024")

    def format_for(self, backward=False):
        """FP8 format of a forward tensor (backward=False) or a gradient."""
        if self.fmt == HYBRID:
            return E5M2 if backward else E4M3
        return E4M3 if self.fmt == "E4M3" else E5M2


class ScalingState:
    """One tensor's delayed-scaling state on the GPU: the amax history
    (float32 [amax_history_len], zeros at the start, so the first step uses
    scale 1) and the last amax, scale and scale_inv (float32 [1] each).
    quantize() casts with the scale from the history and then records this
    step's amax in it, all inside mxq_quantize_per_tensor."""

    def __init__(self, recipe, device="cuda"):
        import torch
        self.recipe = recipe
        f32 = dict(dtype=torch.float32, device=device)
        self.history = torch.zeros(recipe.amax_history_len, **f32)
        self.amax = torch.zeros(1, **f32)
        self.scale = torch.ones(1, **f32)
        self.scale_inv = torch.ones(1, **f32)

    def quantize(self, x, q_row=None, q_col=None, backward=False, stream=None):
        """Cast ``x`` into the preallocated ``q_row`` / ``q_col``; returns
        the FP8 format used."""
        fmt = self.recipe.format_for(backward)
        quantize_per_tensor(x, fmt, self.amax, self.scale, self.scale_inv, q_row, q_col,
                            amax_history=self.history, stream=stream)
        return fmt
