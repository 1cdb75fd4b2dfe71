"""Build libmxq.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled for gfx950 only.  Flags:
  -ffp-contract=off                  no fused multiply-add merges the scale
                                     product with anything else
  -fno-gpu-flush-denormals-to-zero   binary32 subnormals are kept (block
                                     scales reach 2^-127; bf16 inputs can be
                                     subnormal)
  -target-feature -packed-fp32-ops   no packed fp32 instructions are emitted
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxq.so")
# (source, object name, extra defines): gemm_inst.hip once per operand-format
# pair and mode (E4M3 = 0, E5M2 = 1, E2M1 = 2; the precise mode takes FP8
# operands only), so that the GEMM's instantiations compile in parallel
SOURCES = [(s, s, []) for s in ("mxq_api.hip", "quantize.hip", "repack.hip", "gemm.hip")]
SOURCES += [("gemm_inst.hip", f"gemm_inst_{fa}{fb}{p}.hip", [f"-DMXQ_FA={fa}", f"-DMXQ_FB={fb}", f"-DMXQ_PRECISE={p}"])
            for p in (0, 1) for fa in range(3) for fb in range(3) if p == 0 or (fa < 2 and fb < 2)]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(job, verbose):
    src, name, defs = job
    out = os.path.join(OBJ, name + ".o")
    cmd = [HIPCC, *FLAGS, *defs, "-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature: harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
