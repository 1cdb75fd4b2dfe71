"""The Python binding checks every tensor before it calls the library: an
undersized, mistyped, non-contiguous or host-resident tensor raises in
Python, and no entry point is reached (CPU checks; the library is replaced by
a stub that fails if any of its functions is called)."""
import pytest
import torch

import mxfp4_precision_numerics_amd as mxq


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"{name} was reached with invalid arguments")


@pytest.fixture
def stub(monkeypatch):
    monkeypatch.setattr(mxq, "_lib", _NoCalls())


def u8(*s):
    return torch.zeros(s, dtype=torch.uint8)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


X = torch.zeros((64, 128), dtype=torch.bfloat16)


def cases():
    """(label, call, expected exception) - each call has exactly one defect."""
    return [
        ("mx q_row short", lambda: mxq.quantize_mx(X, mxq.E4M3, u8(64, 127), u8(64, 4)), ValueError),
        ("mx s_row short", lambda: mxq.quantize_mx(X, mxq.E4M3, u8(64, 128), u8(64, 3)), ValueError),
        ("mx e2m1 q_row short", lambda: mxq.quantize_mx(X, mxq.E2M1, u8(63, 64), u8(64, 4)), ValueError),
        ("mx q_col short", lambda: mxq.quantize_mx(X, mxq.E4M3, None, None, u8(128, 63), u8(128, 2)), ValueError),
        ("mx s_col missing", lambda: mxq.quantize_mx(X, mxq.E4M3, None, None, u8(128, 64), None), ValueError),
        ("mx q_row dtype", lambda: mxq.quantize_mx(X, mxq.E4M3, f32(64, 128), u8(64, 4)), TypeError),
        ("mx x dtype", lambda: mxq.quantize_mx(X.to(torch.float16), mxq.E4M3, u8(64, 128), u8(64, 4)), TypeError),
        ("mx x column stride", lambda: mxq.quantize_mx(X.t(), mxq.E4M3, u8(128, 64), u8(128, 2)), ValueError),
        ("mx q_row non-contiguous", lambda: mxq.quantize_mx(X, mxq.E4M3, u8(128, 64).t(), u8(64, 4)), ValueError),
        ("mx host tensors", lambda: mxq.quantize_mx(X, mxq.E4M3, u8(64, 128), u8(64, 4)), ValueError),
        ("pt q_col short", lambda: mxq.quantize_per_tensor(X, mxq.E4M3, f32(1), f32(1), f32(1), None, u8(100, 64)),
         ValueError),
        ("pt amax dtype", lambda: mxq.quantize_per_tensor(X, mxq.E4M3, u8(4), f32(1), f32(1), u8(64, 128)),
         TypeError),
        ("pt scale missing", lambda: mxq.quantize_per_tensor(X, mxq.E4M3, f32(1), None, None, u8(64, 128)),
         ValueError),
        ("pt history dtype", lambda: mxq.quantize_per_tensor(X, mxq.E4M3, f32(1), f32(1), f32(1), u8(64, 128),
                                                              amax_history=torch.zeros(16, dtype=torch.float64)),
         TypeError),
        ("repack q8 short", lambda: mxq.repack_fp4_to_fp8(u8(64, 64), u8(64, 4), u8(64, 127), u8(64, 1)),
         ValueError),
        ("repack s4 short", lambda: mxq.repack_fp4_to_fp8(u8(64, 64), u8(64, 3), u8(64, 128), u8(64, 1)),
         ValueError),
        ("repack idx dtype", lambda: mxq.repack_fp4_to_fp8(u8(64, 64), u8(64, 4), u8(64, 128), u8(64, 1),
                                                           gather_idx=torch.zeros(64, dtype=torch.int64)),
         TypeError),
        ("repack idx short", lambda: mxq.repack_fp4_to_fp8(u8(64, 64), u8(64, 4), u8(64, 128), u8(64, 1),
                                                           gather_idx=torch.zeros(63, dtype=torch.int32)),
         ValueError),
        ("fp4 col s8 short", lambda: mxq.fp4_row_to_fp8_col(u8(64, 64), u8(64, 4), u8(128, 64), u8(128, 1)),
         ValueError),
        ("swiglu gu narrow", lambda: mxq.swiglu_quantize_mx(X, 96, mxq.E4M3, u8(64, 96), u8(64, 3)), ValueError),
        ("swiglu s short", lambda: mxq.swiglu_quantize_mx(X, 64, mxq.E4M3, u8(64, 64), u8(64, 1)), ValueError),
        ("gemm A short", lambda: mxq.scaled_gemm(u8(127, 128), 0, u8(128, 4), 1, u8(64, 128), 0, u8(64, 4), 1,
                                                 128, 64, 128, f32(128, 64)), ValueError),
        ("gemm fp4 B short", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(64, 63), 2, u8(64, 4), 1,
                                                     128, 64, 128, f32(128, 64)), ValueError),
        ("gemm sB short", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(64, 128), 0, u8(64, 3), 1,
                                                  128, 64, 128, f32(128, 64)), ValueError),
        ("gemm blk128 sA short", lambda: mxq.scaled_gemm(u8(128, 256), 0, u8(255), 2, u8(64, 256), 0, u8(64, 8), 1,
                                                         128, 64, 256, f32(128, 64)), ValueError),
        ("gemm tensor scale dtype", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(4), 0, u8(64, 128), 0, f32(1), 0,
                                                            128, 64, 128, f32(128, 64)), TypeError),
        ("gemm C small", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(64, 128), 0, u8(64, 4), 1,
                                                 128, 64, 128, f32(127, 64)), ValueError),
        ("gemm C dtype", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(64, 128), 0, u8(64, 4), 1,
                                                 128, 64, 128, f32(128, 64), out=mxq.OUT_BF16), TypeError),
        ("gemm C pitch", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(64, 128), 0, u8(64, 4), 1,
                                                 128, 64, 128, f32(128, 64), ldc=72), ValueError),
        ("gemm host tensors", lambda: mxq.scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(64, 128), 0, u8(64, 4), 1,
                                                      128, 64, 128, f32(128, 64)), ValueError),
        ("grouped B short", lambda: mxq.grouped_scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(2, 64, 127), 0,
                                                            u8(2, 64, 4), 1, torch.tensor([0, 64, 128]), 2, 128,
                                                            64, 128, f32(128, 64)), ValueError),
        ("grouped offsets short", lambda: mxq.grouped_scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(2, 64, 128), 0,
                                                                  u8(2, 64, 4), 1, torch.tensor([0, 64]), 2, 128,
                                                                  64, 128, f32(128, 64)), ValueError),
        ("grouped offsets dtype", lambda: mxq.grouped_scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(2, 64, 128), 0,
                                                                  u8(2, 64, 4), 1,
                                                                  torch.tensor([0, 64, 128], dtype=torch.int32),
                                                                  2, 128, 64, 128, f32(128, 64)), TypeError),
        ("grouped C rows", lambda: mxq.grouped_scaled_gemm(u8(128, 128), 0, u8(128, 4), 1, u8(2, 64, 128), 0,
                                                           u8(2, 64, 4), 1, torch.tensor([0, 64, 128]), 2, 128,
                                                           64, 128, f32(120, 64)), ValueError),
    ]


@pytest.mark.parametrize("label,call,exc", cases(), ids=[c[0] for c in cases()])
def test_invalid_tensor_raises_before_the_library(stub, label, call, exc):
    with pytest.raises(exc) as e:
        call()
    # the defect itself is named; the device is checked only after every extent
    assert ("GPU tensor" in str(e.value)) == ("host" in label), str(e.value)
