"""The product path runs the HIP library or nothing: without libmxq.so every
entry point raises before any work, and no package module reaches the
oracle (CPU checks)."""
import ast
import os

import pytest
import torch

import mxfp4_precision_numerics_amd as mxq

PKG = os.path.dirname(os.path.abspath(mxq.__file__))


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(mxq, "LIB_PATH", os.path.join(PKG, "does-not-exist", "libmxq.so"))
    monkeypatch.setattr(mxq, "_lib", None)


def test_missing_library_raises(no_library):
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    f32 = lambda: torch.zeros(1, dtype=torch.float32)
    calls = [
        lambda: mxq.lib(),
        lambda: mxq.quantize_mx(x, mxq.E4M3, u8(32, 64), u8(32, 2)),
        lambda: mxq.quantize_per_tensor(x, mxq.E4M3, f32(), f32(), f32(), u8(32, 64)),
        lambda: mxq.repack_fp4_to_fp8(u8(32, 64), u8(32, 4), u8(32, 128), u8(32, 1)),
        lambda: mxq.fp4_row_to_fp8_col(u8(32, 64), u8(32, 4), u8(128, 32), u8(128, 1)),
        lambda: mxq.swiglu_quantize_mx(x, 32, mxq.E4M3, u8(32, 32), u8(32, 1)),
        lambda: mxq.scaled_gemm(u8(128, 128), mxq.E4M3, u8(128, 4), mxq.SCALE_BLK32, u8(128, 128), mxq.E4M3,
                                u8(128, 4), mxq.SCALE_BLK32, 128, 128, 128, torch.zeros((128, 128))),
        lambda: mxq.grouped_scaled_gemm(u8(128, 128), mxq.E4M3, u8(128, 4), mxq.SCALE_BLK32, u8(2, 128, 128),
                                        mxq.E4M3, u8(2, 128, 4), mxq.SCALE_BLK32,
                                        torch.tensor([0, 64, 128]), 2, 128, 128, 128, torch.zeros((128, 128))),
    ]
    for c in calls:
        with pytest.raises(RuntimeError, match="is missing"):
            c()


def test_package_never_imports_the_oracle():
    for root, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(root, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                assert not any(n == "oracle" or n.startswith("oracle.") for n in names), (f, names)
