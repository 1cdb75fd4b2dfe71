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
        L.mxq_grouped_gemm_swiglu_quantize_mx.restype = i
        L.mxq_grouped_gemm_swiglu_quantize_mx.argtypes = [p, i, p, i, p, i, p, i, p, i64, i64, i64, i64, i, p, p,
                                                          p]
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


# Argument checks.  The C entry points validate sizes, divisibility and
# alignment, but they see raw pointers: a tensor smaller than the region a
# kernel addresses, of another element type or not laid out as the kernel
# assumes would become an out-of-bounds device access.  Every wrapper
# therefore checks each tensor's dtype, layout, extent and device before the
# call and raises ValueError / TypeError instead.

def _dtype(name, t, dtypes):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {', '.join(str(d) for d in dtypes)}")


def _on_gpu(**tensors):
    """Checked last, once every extent is known to be right."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _buf(name, t, dtypes, numel):
    """A dense buffer of at least `numel` elements of one of `dtypes`."""
    if t is None:
        raise ValueError(f"{name} is required")
    _dtype(name, t, dtypes)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call addresses {numel}")


def _matrix(name, t, dtypes, rows, cols):
    """A row-major matrix view of at least [rows, cols], unit column stride
    (the row pitch is the view's own stride)."""
    _dtype(name, t, dtypes)
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError(f"{name} is {tuple(t.shape)}; the call addresses [{rows}, {cols}]")


def _u8():
    import torch
    return (torch.uint8,)


def _f32():
    import torch
    return (torch.float32,)


def _scale(name, s, mode, rows, K):
    """GEMM operand scales: one float (per-tensor) or E8M0 bytes."""
    if mode == SCALE_TENSOR:
        _buf(name, s, _f32(), 1)
    elif mode in (SCALE_BLK32, SCALE_BLK128):
        _buf(name, s, _u8(), rows * (K // (32 if mode == SCALE_BLK32 else 128)))
    # any other mode is refused by the library (MXQ_ERR_FORMAT)


def _codes_per_row(fmt, K):
    return K // 2 if fmt == E2M1 else K


def quantize_per_tensor(x, fmt, amax_out, scale_out, scale_inv_out=None, q_row=None, q_col=None,
                        amax_history=None, stream=None):
    """amax + per-tensor scale + saturating RNE cast (mxq_quantize_per_tensor).
    ``x`` [rows, cols] (row pitch x.stride(0)); outputs are preallocated
    tensors; ``amax_history`` (float32 [len]) selects delayed scaling."""
    L = lib()
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    _matrix("x", x, (torch.bfloat16, torch.float32), rows, cols)
    _buf("amax_out", amax_out, _f32(), 1)
    _buf("scale_out", scale_out, _f32(), 1)
    if scale_inv_out is not None:
        _buf("scale_inv_out", scale_inv_out, _f32(), 1)
    if q_row is not None:
        _buf("q_row", q_row, _u8(), rows * cols)
    if q_col is not None:
        _buf("q_col", q_col, _u8(), rows * cols)
    if amax_history is not None:
        _buf("amax_history", amax_history, _f32(), 1)
    _on_gpu(x=x, amax_out=amax_out, scale_out=scale_out, scale_inv_out=scale_inv_out, q_row=q_row, q_col=q_col,
            amax_history=amax_history)
    hl = 0 if amax_history is None else amax_history.numel()
    st = L.mxq_quantize_per_tensor(_ptr(x), _src_of(x), rows, cols, x.stride(0), fmt, _ptr(amax_history), hl,
                                   _ptr(amax_out), _ptr(scale_out), _ptr(scale_inv_out), _ptr(q_row),
                                   _ptr(q_col), _stream(stream))
    _check("mxq_quantize_per_tensor", st)


def quantize_mx(x, fmt, q_row=None, s_row=None, q_col=None, s_col=None, stream=None):
    """MX block-32 quantization (mxq_quantize_mx) into preallocated outputs."""
    L = lib()
    import torch
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    _matrix("x", x, (torch.bfloat16, torch.float32), rows, cols)
    if q_row is not None:
        _buf("q_row", q_row, _u8(), rows * _codes_per_row(fmt, cols))
        _buf("s_row", s_row, _u8(), rows * (cols // 32))
    if q_col is not None:
        _buf("q_col", q_col, _u8(), rows * cols)
        _buf("s_col", s_col, _u8(), cols * (rows // 32))
    _on_gpu(x=x, q_row=q_row, s_row=s_row, q_col=q_col, s_col=s_col)
    st = L.mxq_quantize_mx(_ptr(x), _src_of(x), rows, cols, x.stride(0), fmt, _ptr(q_row), _ptr(s_row),
                           _ptr(q_col), _ptr(s_col), _stream(stream))
    _check("mxq_quantize_mx", st)


def repack_fp4_to_fp8(q4, s4, q8, s8, gather_idx=None, stream=None):
    """Direct MXFP4 -> E4M3/block-128 repack (mxq_repack_fp4_to_fp8).
    q4 [src_rows, cols/2], s4 [src_rows, cols/32]; q8 [rows, cols],
    s8 [rows, cols/128]; gather_idx int32 [rows] or None."""
    L = lib()
    import torch
    if q4.dim() != 2 or q8.dim() != 2:
        raise ValueError("q4 and q8 must be 2-D")
    src_rows, cols = q4.shape[0], q4.shape[1] * 2
    rows = q8.shape[0]
    _buf("q4", q4, _u8(), src_rows * (cols // 2))
    _buf("s4", s4, _u8(), src_rows * (cols // 32))
    _buf("q8", q8, _u8(), rows * cols)
    _buf("s8", s8, _u8(), rows * (cols // 128))
    if gather_idx is not None:
        _buf("gather_idx", gather_idx, (torch.int32,), rows)
    _on_gpu(q4=q4, s4=s4, q8=q8, s8=s8, gather_idx=gather_idx)
    st = L.mxq_repack_fp4_to_fp8(_ptr(q4), _ptr(s4), _ptr(gather_idx), src_rows, rows, cols, _ptr(q8),
                                 _ptr(s8), _stream(stream))
    _check("mxq_repack_fp4_to_fp8", st)


def fp4_row_to_fp8_col(q4, s4, q8, s8, stream=None):
    """MXFP4 rows [rows, cols] -> MX E4M3 columns q8 [cols, rows], s8
    [cols, rows/32] (mxq_fp4_row_to_fp8_col)."""
    L = lib()
    if q4.dim() != 2:
        raise ValueError("q4 must be 2-D")
    rows, cols = q4.shape[0], q4.shape[1] * 2
    _buf("q4", q4, _u8(), rows * (cols // 2))
    _buf("s4", s4, _u8(), rows * (cols // 32))
    _buf("q8", q8, _u8(), rows * cols)
    _buf("s8", s8, _u8(), cols * (rows // 32))
    _on_gpu(q4=q4, s4=s4, q8=q8, s8=s8)
    st = L.mxq_fp4_row_to_fp8_col(_ptr(q4), _ptr(s4), rows, cols, _ptr(q8), _ptr(s8), _stream(stream))
    _check("mxq_fp4_row_to_fp8_col", st)


def swiglu_quantize_mx(gu, inter, fmt, q, s, stream=None):
    """h = silu(gate) * up of ``gu`` [rows, >= 2 inter] (gate columns [0,
    inter), up [inter, 2 inter)), MX block-32 quantized into q [rows, inter]
    and s [rows, inter/32] (mxq_swiglu_quantize_mx)."""
    L = lib()
    import torch
    if gu.dim() != 2:
        raise ValueError("gu must be 2-D")
    rows = gu.shape[0]
    _matrix("gu", gu, (torch.bfloat16, torch.float32), rows, 2 * inter)
    _buf("q", q, _u8(), rows * inter)
    _buf("s", s, _u8(), rows * (inter // 32))
    _on_gpu(gu=gu, q=q, s=s)
    st = L.mxq_swiglu_quantize_mx(_ptr(gu), _src_of(gu), rows, inter, gu.stride(0), fmt, _ptr(q), _ptr(s),
                                  _stream(stream))
    _check("mxq_swiglu_quantize_mx", st)


def _gemm_out(C, out, rows, N, ldc):
    import torch
    kind = out & ~OUT_PRECISE
    _dtype("C", C, (torch.float32,) if kind == OUT_F32 else (torch.bfloat16, torch.int16, torch.uint16))
    if C.dim() != 2 or C.stride(1) != 1 or C.stride(0) != ldc:
        raise ValueError("C must be a 2-D tensor with unit column stride and row pitch ldc")
    if C.shape[0] < rows or C.shape[1] < N:
        raise ValueError(f"C is {tuple(C.shape)}; the call writes [{rows}, {N}]")


def scaled_gemm(A, fa, sA, ma, B, fb, sB, mb, M, N, K, C, out=OUT_F32, ldc=None, stream=None):
    """C = deq(A) . deq(B)^T (mxq_scaled_gemm).  A [M, K] codes (E2M1:
    [M, K/2]), B [N, K] likewise, scales per mode; C [M, N] (row pitch ldc,
    default C.stride(0)), float32 or bfloat16 per ``out``."""
    L = lib()
    ldc = C.stride(0) if ldc is None else ldc
    _buf("A", A, _u8(), M * _codes_per_row(fa, K))
    _buf("B", B, _u8(), N * _codes_per_row(fb, K))
    _scale("sA", sA, ma, M, K)
    _scale("sB", sB, mb, N, K)
    _gemm_out(C, out, M, N, ldc)
    _on_gpu(A=A, sA=sA, B=B, sB=sB, C=C)
    st = L.mxq_scaled_gemm(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, M, N, K, _ptr(C), out, ldc,
                           _stream(stream))
    _check("mxq_scaled_gemm", st)


def grouped_scaled_gemm(A, fa, sA, ma, B, fb, sB, mb, group_off, G, total_rows, N, K, C, out=OUT_F32,
                        stream=None):
    """Ragged grouped GEMM over device offsets (mxq_grouped_scaled_gemm).
    A [total_rows, K] codes, B [G, N, K], sB per group (or one float),
    group_off int64 [G+1] on the device, C [total_rows, N] dense."""
    L = lib()
    import torch
    _buf("A", A, _u8(), total_rows * _codes_per_row(fa, K))
    _buf("B", B, _u8(), G * N * _codes_per_row(fb, K))
    _scale("sA", sA, ma, total_rows, K)
    _scale("sB", sB, mb, G * N if mb != SCALE_TENSOR else 1, K)
    _buf("group_off", group_off, (torch.int64,), G + 1)
    if not C.is_contiguous():
        raise ValueError("C must be contiguous")
    _gemm_out(C, out, total_rows, N, N)
    _on_gpu(A=A, sA=sA, B=B, sB=sB, group_off=group_off, C=C)
    st = L.mxq_grouped_scaled_gemm(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, _ptr(group_off), G,
                                   total_rows, N, K, _ptr(C), out, _stream(stream))
    _check("mxq_grouped_scaled_gemm", st)


def grouped_gemm_swiglu_quantize_mx(A, fa, sA, ma, B, fb, sB, mb, group_off, G, total_rows, inter, K, hfmt, q,
                                    s, stream=None):
    """Expert up-projection with the SwiGLU + MX epilogue
    (mxq_grouped_gemm_swiglu_quantize_mx).  B [G, 2 inter, K] holds each
    group's gate rows then its up rows; q [total_rows, inter] and s
    [total_rows, inter/32] receive h = silu(gate) * up, MX quantized."""
    L = lib()
    import torch
    _buf("A", A, _u8(), total_rows * K)
    _buf("B", B, _u8(), G * 2 * inter * K)
    _scale("sA", sA, ma, total_rows, K)
    _scale("sB", sB, mb, G * 2 * inter if mb != SCALE_TENSOR else 1, K)
    _buf("group_off", group_off, (torch.int64,), G + 1)
    _buf("q", q, _u8(), total_rows * inter)
    _buf("s", s, _u8(), total_rows * (inter // 32))
    _on_gpu(A=A, sA=sA, B=B, sB=sB, group_off=group_off, q=q, s=s)
    st = L.mxq_grouped_gemm_swiglu_quantize_mx(_ptr(A), fa, _ptr(sA), ma, _ptr(B), fb, _ptr(sB), mb, _ptr(group_off),
                                               G, total_rows, inter, K, hfmt, _ptr(q), _ptr(s), _stream(stream))
    _check("mxq_grouped_gemm_swiglu_quantize_mx", st)


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
