"""Benchmark of the scaled-quantization + block-scaled GEMM hot path on one MI355X.

Headline step (workload "llama3-70b-mlp-mxfp8-fwd-bwd"): one training step's
worth of the Llama-3-70B MLP's FP8 work on one GPU, inputs resident in HBM:
  * dual (row + column) MX block-32 quantization of the six bf16 tensors the
    MLP's GEMMs consume: X [8192, 8192], W_up [28672, 8192], H [8192, 28672],
    W_down [8192, 28672] to E4M3 and the gradients dY [8192, 28672],
    dZ [8192, 8192] to E5M2 (each operand blocked along its own contraction
    dimension);
  * the six GEMMs, fp32 output: forward up (8192 x 28672 x 8192) and down
    (8192 x 8192 x 28672), dgrad and wgrad of both.
The GEMMs run in the library's precise mode (MXQ_OUT_PRECISE: FP8 operands
converted exactly to bf16 with their block scales, bf16 MFMA, fp32
accumulation), the mode that holds these six GEMMs within 1e-5 of the fp64
oracle; the block-scaled FP8 MFMA does not on this data (its truncation
inside each run of 8 products adds up over K).  `value` is the step's GEMM
work (6 x 2MNK) per step time, TFLOP/s.

Also reported on the one JSON line: the roofline of the dominant kernel (the
step's six GEMM launches, timed with HIP events on the stream they run on,
against the bf16 dense MFMA peak), every other row of the hot path on its
own workload with a cold cache (each GEMM row says whether its mode meets
1e-5 on that workload), and the CPU oracle timed on a bounded sample of the
headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows]
       [--no-cpu-baseline] [--row-reps 50] [--row-warmup 10]
       [--only ROW-ID[,ROW-ID...]] [--copy-probe]

--only runs just the named rows ("headline" for the step; row ids are the
keys of the "rows" object), which is how each row is profiled on its own.
roofline.traffic is the step's GEMM HBM bytes from the committed rocprofv3
FETCH_SIZE / WRITE_SIZE summary under profiles/ (each counter scaled by what
it reads for a plain copy of known size, --copy-probe), and null when the
GEMM kernel source has changed since those counters were taken.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
BF16_PEAK_TFLOPS = 2500.0

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemm_precise_llama70b_mlp_step_hbm_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "mxfp4_precision_numerics_amd", "csrc", "gemm_kernel.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-reps", type=int, default=50, help="timed repetitions per row (median, p10/p90)")
    ap.add_argument("--row-warmup", type=int, default=10, help="untimed repetitions per row")
    ap.add_argument("--only", default=None, help="comma-separated row ids to run ('headline' for the step)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (reference for the traffic counters)")
    return ap.parse_args()


def gemm_traffic():
    """HBM bytes of the step's GEMM launches from the committed counter
    summary, or None if there is none or the kernel source differs from the
    one counted."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if kv.get("gemm_source_sha256") != sha or "traffic_bytes_per_step" not in kv:
        return None
    return int(float(kv["traffic_bytes_per_step"]))


class Ctx:
    """Device, binding, timing helpers shared by the rows."""

    def __init__(self, args):
        import torch
        import mxfp4_precision_numerics_amd as mxq
        import synth
        self.torch, self.mxq, self.synth = torch, mxq, synth
        self.dev = torch.device("cuda:0")
        self.stream = torch.cuda.current_stream()
        self.args = args
        self.only = None if args.only is None else set(s.strip() for s in args.only.split(","))
        self._flush = None

    def want(self, rid):
        return self.only is None or rid in self.only

    def bf16(self, spec):
        bits = self.synth.tensor(spec)
        return self.torch.from_numpy(bits.view(np.int16)).to(self.dev).view(self.torch.bfloat16)

    def u8(self, *shape):
        return self.torch.empty(shape, dtype=self.torch.uint8, device=self.dev)

    def f32(self, *shape):
        return self.torch.empty(shape, dtype=self.torch.float32, device=self.dev)

    def timed(self, fn):
        """Median and p10/p90 (ms) of `row_reps` calls, each after a 1 GiB fill
        (outside the timed interval) that evicts the 256 MB last-level cache;
        `row_warmup` untimed calls first."""
        torch = self.torch
        if self._flush is None:
            self._flush = torch.empty(2 ** 30, dtype=torch.uint8, device=self.dev)
        for _ in range(self.args.row_warmup):
            fn()
        ts = []
        for _ in range(self.args.row_reps):
            self._flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)), [round(float(np.percentile(ts, q)), 4) for q in (10, 90)]

    @staticmethod
    def bw(what, nbytes, t):
        ms, sp = t
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"what": what, "bound": "hbm", "ms": round(ms, 4), "ms_p10_p90": sp, "bytes": int(nbytes),
                "GB/s": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "peak": HBM_PEAK_GBS}

    @staticmethod
    def fl(what, nflop, t, peak, meets, nbytes=None):
        ms, sp = t
        tf = nflop / (ms * 1e-3) / 1e12
        r = {"what": what, "bound": "mfma", "ms": round(ms, 4), "ms_p10_p90": sp, "flop": nflop,
             "TFLOP/s": round(tf, 1), "frac": round(tf / peak, 4), "peak": peak, "meets_1e-5": meets}
        if nbytes is not None:
            gbs = nbytes / (ms * 1e-3) / 1e9
            r.update({"bytes": int(nbytes), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        return r


# ----------------------------------------------------------------- headline

C5_SHAPES = {"x": (8192, 8192), "w_up": (28672, 8192), "h": (8192, 28672), "w_down": (8192, 28672),
             "dy": (8192, 28672), "dz": (8192, 8192)}
# (name, A tensor, A layout, B tensor, B layout): C = A . B^T, both K-contiguous
C5_GEMMS = [("fwd_up", "x", "row", "w_up", "row"), ("fwd_down", "h", "row", "w_down", "row"),
            ("dgrad_up", "dy", "row", "w_up", "col"), ("wgrad_up", "x", "col", "dy", "col"),
            ("dgrad_down", "dz", "row", "w_down", "col"), ("wgrad_down", "h", "col", "dz", "col")]


def headline(ctx):
    torch, mxq, synth = ctx.torch, ctx.mxq, ctx.synth
    specs = {"x": synth.c5_x(), "w_up": synth.c5_w_up(), "h": synth.c5_h(), "w_down": synth.c5_w_down(),
             "dy": synth.c5_dy(), "dz": synth.c5_dz()}
    fmt = {k: (mxq.E5M2 if k in ("dy", "dz") else mxq.E4M3) for k in specs}
    src, q = {}, {}
    for k, spec in specs.items():
        r, c = C5_SHAPES[k]
        src[k] = ctx.bf16(spec)
        q[k] = {"row": (ctx.u8(r, c), ctx.u8(r, c // 32)), "col": (ctx.u8(c, r), ctx.u8(c, r // 32))}
    gemms = []
    for name, an, al, bn, bl in C5_GEMMS:
        A, sA = q[an][al]
        B, sB = q[bn][bl]
        M, K, N = A.shape[0], A.shape[1], B.shape[0]
        gemms.append((name, A, fmt[an], sA, B, fmt[bn], sB, M, N, K, ctx.f32(M, N)))
    flops = sum(2.0 * g[7] * g[8] * g[9] for g in gemms)
    qbytes = sum(C5_SHAPES[k][0] * C5_SHAPES[k][1] * (2 + 2 + 2 / 32) for k in specs)
    stream = ctx.stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for k in specs:
            mxq.quantize_mx(src[k], fmt[k], *q[k]["row"], *q[k]["col"])
        for i, (name, A, fa, sA, B, fb, sB, M, N, K, C) in enumerate(gemms):
            if ev is not None:
                ev[1 + i].record(stream)
            mxq.scaled_gemm(A, fa, sA, mxq.SCALE_BLK32, B, fb, sB, mxq.SCALE_BLK32, M, N, K, C,
                            out=mxq.OUT_F32 | mxq.OUT_PRECISE)
        if ev is not None:
            ev[1 + len(gemms)].record(stream)

    for _ in range(ctx.args.warmup):
        step()
    torch.cuda.synchronize()
    nev = 2 + len(gemms)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(ctx.args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(ctx.args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / ctx.args.steps
    q_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    g_ms = {g[0]: float(np.mean([e[1 + i].elapsed_time(e[2 + i]) for e in evs])) for i, g in enumerate(gemms)}
    gemm_ms = sum(g_ms.values())
    gemm_tf = flops / (gemm_ms * 1e-3) / 1e12
    res = {
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "ms_per_step": round(ms_step, 4),
        "roofline": {"kernel": "k_gemm, precise mode (FP8 operands -> bf16 with block scales, bf16 MFMA, fp32 "
                               "accumulation), the step's six GEMM launches", "bound": "mfma",
                     "achieved": round(gemm_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tf / BF16_PEAK_TFLOPS, 4), "traffic": gemm_traffic()},
        "kernels_ms": {"quantize_mx_dual_x6": round(q_ms, 4), **{f"gemm_{k}": round(v, 4) for k, v in g_ms.items()}},
        "quantize_gbs": round(qbytes / (q_ms * 1e-3) / 1e9, 1),
        "gemm_flop_per_step": flops,
    }
    del src, q, gemms
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------- rows

def rows_c1(ctx, rows):
    """Workload 1: per-tensor E4M3 (current scaling) of two 256 x 256 fp32
    matrices and the 256^3 GEMM: latency-bound (the data fit in cache)."""
    if not (ctx.want("c1_pt_cast") or ctx.want("c1_gemm")):
        return
    torch, mxq, synth = ctx.torch, ctx.mxq, ctx.synth
    a = torch.from_numpy(synth.tensor(synth.c1_a())).to(ctx.dev)
    b = torch.from_numpy(synth.tensor(synth.c1_b())).to(ctx.dev)
    amax, sc, sia, sib = (ctx.f32(1) for _ in range(4))
    qa, qbc = ctx.u8(256, 256), ctx.u8(256, 256)
    if ctx.want("c1_pt_cast"):
        t = ctx.timed(lambda: mxq.quantize_per_tensor(a, mxq.E4M3, amax, sc, sia, qa))
        rows["c1_pt_cast"] = ctx.bw("a1-a3 per-tensor current E4M3 (amax pass + cast), A 256x256 fp32 "
                                    "(latency-bound, fits in cache)", 256 * 256 * 9, t)
    mxq.quantize_per_tensor(a, mxq.E4M3, amax, sc, sia, qa)
    mxq.quantize_per_tensor(b, mxq.E4M3, amax, sc, sib, None, qbc)
    if ctx.want("c1_gemm"):
        C = ctx.f32(256, 256)
        t = ctx.timed(lambda: mxq.scaled_gemm(qa, mxq.E4M3, sia, 0, qbc, mxq.E4M3, sib, 0, 256, 256, 256, C))
        rows["c1_gemm"] = ctx.fl("a6 per-tensor E4M3 GEMM 256x256x256, FP8 MFMA (latency-bound)",
                                 2.0 * 256 ** 3, t, FP8_PEAK_TFLOPS, True)


def rows_c2(ctx, rows):
    """Workload 2: Llama-3-8B MLP up-projection, MXFP8 forward."""
    ids = ("c2_mx_x", "c2_mx_w", "c2_gemm_precise", "c2_gemm_native")
    if not any(ctx.want(i) for i in ids):
        return
    mxq, synth = ctx.mxq, ctx.synth
    M, N, K = 4096, 14336, 4096
    x, w = ctx.bf16(synth.c2_x()), ctx.bf16(synth.c2_w())
    qx, sx, qw, sw = ctx.u8(M, K), ctx.u8(M, K // 32), ctx.u8(N, K), ctx.u8(N, K // 32)
    if ctx.want("c2_mx_x"):
        rows["c2_mx_x"] = ctx.bw("a4 MX E4M3 row quantize, X 4096x4096 bf16 (41 outlier columns)",
                                 M * K * (2 + 1 + 1 / 32), ctx.timed(lambda: mxq.quantize_mx(x, mxq.E4M3, qx, sx)))
    if ctx.want("c2_mx_w"):
        rows["c2_mx_w"] = ctx.bw("a4 MX E4M3 row quantize, W 14336x4096 bf16", N * K * (2 + 1 + 1 / 32),
                                 ctx.timed(lambda: mxq.quantize_mx(w, mxq.E4M3, qw, sw)))
    if not (ctx.want("c2_gemm_precise") or ctx.want("c2_gemm_native")):
        return
    mxq.quantize_mx(x, mxq.E4M3, qx, sx)
    mxq.quantize_mx(w, mxq.E4M3, qw, sw)
    C = ctx.f32(M, N)
    for rid, out, peak, meets, what in (
            ("c2_gemm_precise", mxq.OUT_PRECISE, BF16_PEAK_TFLOPS, True,
             "a6 MXFP8 GEMM 4096x14336x4096 fp32 out, precise mode (bf16 MFMA; within 1e-5)"),
            ("c2_gemm_native", 0, FP8_PEAK_TFLOPS, False,
             "a6 MXFP8 GEMM 4096x14336x4096 fp32 out, block-scaled FP8 MFMA (misses 1e-5 on this data)")):
        if ctx.want(rid):
            t = ctx.timed(lambda: mxq.scaled_gemm(qx, mxq.E4M3, sx, 1, qw, mxq.E4M3, sw, 1, M, N, K, C, out=out))
            rows[rid] = ctx.fl(what, 2.0 * M * N * K, t, peak, meets)


def rows_c3(ctx, rows):
    """Workload 3: E5M2 backward with delayed per-tensor scaling (history 16)."""
    ids = ("c3_pt_delayed", "c3_pt_current", "c3_dgrad_precise", "c3_dgrad_native", "c3_wgrad_precise",
           "c3_wgrad_native")
    if not any(ctx.want(i) for i in ids):
        return
    torch, mxq, synth = ctx.torch, ctx.mxq, ctx.synth
    hist = torch.zeros(16, dtype=torch.float32, device=ctx.dev)
    amax, sc, si = ctx.f32(1), ctx.f32(1), ctx.f32(1)
    for t in range(16):
        p = ctx.bf16(synth.c3_prior_dy(t))
        mxq.quantize_per_tensor(p, mxq.E5M2, amax, sc, si, ctx.u8(*p.shape), amax_history=hist)
    dy = ctx.bf16(synth.c3_dy())
    qr, qc = ctx.u8(4096, 14336), ctx.u8(14336, 4096)
    if ctx.want("c3_pt_delayed"):
        # each repetition pushes dY's amax into the history; the work of a
        # call does not depend on the history's values
        rows["c3_pt_delayed"] = ctx.bw(
            "a1-a3 per-tensor delayed E5M2 cast, dY 4096x14336 bf16, row + col (fused amax; prologue, cast, "
            "history launches)", dy.numel() * 4,
            ctx.timed(lambda: mxq.quantize_per_tensor(dy, mxq.E5M2, amax, sc, si, qr, qc, amax_history=hist)))
    if ctx.want("c3_pt_current"):
        amax_c = ctx.f32(1)
        rows["c3_pt_current"] = ctx.bw(
            "a1-a3 per-tensor current E5M2 (amax pass, then cast), dY 4096x14336 bf16, row + col (6 B/el)",
            dy.numel() * 6, ctx.timed(lambda: mxq.quantize_per_tensor(dy, mxq.E5M2, amax_c, sc, si, qr, qc)))
    mxq.quantize_per_tensor(dy, mxq.E5M2, amax, sc, si, qr, qc, amax_history=hist)
    w = ctx.bf16(synth.c3_w())
    qwr, qwc, sw = ctx.u8(14336, 4096), ctx.u8(4096, 14336), ctx.f32(1)
    mxq.quantize_per_tensor(w, mxq.E4M3, amax, sc, sw, qwr, qwc, amax_history=torch.zeros(16, device=ctx.dev))
    x = ctx.bf16(synth.c3_x())
    qxr, qxc, sx = ctx.u8(4096, 4096), ctx.u8(4096, 4096), ctx.f32(1)
    mxq.quantize_per_tensor(x, mxq.E4M3, amax, sc, sx, qxr, qxc, amax_history=torch.zeros(16, device=ctx.dev))
    Cd, Cw = ctx.f32(4096, 4096), ctx.f32(4096, 14336)
    for kind, out, peak, meets, tag in ((
            "precise", mxq.OUT_PRECISE, BF16_PEAK_TFLOPS, True, "precise mode (bf16 MFMA; within 1e-5)"),
            ("native", 0, FP8_PEAK_TFLOPS, False, "block-scaled FP8 MFMA (misses 1e-5 on this data)")):
        if ctx.want(f"c3_dgrad_{kind}"):
            t = ctx.timed(lambda: mxq.scaled_gemm(qr, mxq.E5M2, si, 0, qwc, mxq.E4M3, sw, 0, 4096, 4096, 14336, Cd,
                                                  out=out))
            rows[f"c3_dgrad_{kind}"] = ctx.fl(f"a6 dgrad E5M2 x E4M3 per-tensor, 4096x4096x14336 fp32 out, {tag}",
                                              2.0 * 4096 * 4096 * 14336, t, peak, meets)
        if ctx.want(f"c3_wgrad_{kind}"):
            t = ctx.timed(lambda: mxq.scaled_gemm(qxc, mxq.E4M3, sx, 0, qc, mxq.E5M2, si, 0, 4096, 14336, 4096, Cw,
                                                  out=out))
            rows[f"c3_wgrad_{kind}"] = ctx.fl(f"a6 wgrad E4M3 x E5M2 per-tensor, 4096x14336x4096 fp32 out, {tag}",
                                              2.0 * 4096 * 14336 * 4096, t, peak, meets)


def rows_c4(ctx, rows):
    """Workload 4: one GPU's share of a 671B-class MoE: MXFP4 quantize,
    gather + repack, grouped expert GEMM; the expert MLP's activation and
    down-projection."""
    ids = ("c4_mx_e2m1", "c4_repack", "c4_fp4col", "c4_grouped", "c4_up_swiglu_fused", "c4_grouped_fp4",
           "c4_swiglu", "c4_down")
    if not any(ctx.want(i) for i in ids):
        return
    torch, mxq, synth = ctx.torch, ctx.mxq, ctx.synth
    x = ctx.bf16(synth.c4_x())
    idx, off = synth.c4_routing()
    R = int(off[-1])
    q4, s4 = ctx.u8(8192, 3584), ctx.u8(8192, 224)
    if ctx.want("c4_mx_e2m1"):
        rows["c4_mx_e2m1"] = ctx.bw("a4 MX E2M1 row quantize, X 8192x7168 bf16", x.numel() * (2 + 0.5 + 1 / 32),
                                    ctx.timed(lambda: mxq.quantize_mx(x, mxq.E2M1, q4, s4)))
    mxq.quantize_mx(x, mxq.E2M1, q4, s4)
    q8, s8 = ctx.u8(R, 7168), ctx.u8(R, 56)
    idx_d = torch.from_numpy(idx).to(ctx.dev)
    if ctx.want("c4_repack"):
        rows["c4_repack"] = ctx.bw(f"a5 FP4 -> FP8 repack with routing gather, R={R} rows x 7168",
                                   R * (3584 + 224 + 4 + 7168 + 56),
                                   ctx.timed(lambda: mxq.repack_fp4_to_fp8(q4, s4, q8, s8, gather_idx=idx_d)))
    mxq.repack_fp4_to_fp8(q4, s4, q8, s8, gather_idx=idx_d)
    if ctx.want("c4_fp4col"):
        q8c, s8c = ctx.u8(7168, 8192), ctx.u8(7168, 256)
        rows["c4_fp4col"] = ctx.bw("f1 FP4 row -> FP8 col (dequant, transpose, MX E4M3), X 8192x7168",
                                   x.numel() * (0.5 + 1 / 32 + 1 + 1 / 32),
                                   ctx.timed(lambda: mxq.fp4_row_to_fp8_col(q4, s4, q8c, s8c)))
        del q8c, s8c
    del x
    off_d = torch.from_numpy(off).to(ctx.dev)
    Cg = torch.empty((R, 4096), dtype=torch.bfloat16, device=ctx.dev)
    if any(ctx.want(i) for i in ("c4_grouped", "c4_up_swiglu_fused", "c4_swiglu", "c4_down")):
        qw, sw = ctx.u8(32, 4096, 7168), ctx.u8(32, 4096, 224)
        for e in range(32):
            mxq.quantize_mx(ctx.bf16(synth.c4_w(e)), mxq.E4M3, qw[e], sw[e])
        if ctx.want("c4_up_swiglu_fused"):
            qhf, shf = ctx.u8(R, 2048), ctx.u8(R, 64)
            t = ctx.timed(lambda: mxq.grouped_gemm_swiglu_quantize_mx(
                q8, mxq.E4M3, s8, mxq.SCALE_BLK128, qw, mxq.E4M3, sw, mxq.SCALE_BLK32, off_d, 32, R, 2048, 7168,
                mxq.E4M3, qhf, shf))
            rows["c4_up_swiglu_fused"] = ctx.fl(
                f"f2 expert up-projection with SwiGLU + MX E4M3 in the epilogue (gate/up never stored), 32 "
                f"experts, R={R}, inter=2048, K=7168, block-scaled FP8 MFMA", 2.0 * R * 4096 * 7168, t,
                FP8_PEAK_TFLOPS, True,
                nbytes=32 * 4096 * 7168 * (1 + 1 / 32) + R * 7168 * (1 + 1 / 128) + R * 2048 * (1 + 1 / 32))
            del qhf, shf

        def grouped():
            mxq.grouped_scaled_gemm(q8, mxq.E4M3, s8, mxq.SCALE_BLK128, qw, mxq.E4M3, sw, mxq.SCALE_BLK32, off_d,
                                    32, R, 4096, 7168, Cg, out=mxq.OUT_BF16)
        if ctx.want("c4_grouped"):
            rows["c4_grouped"] = ctx.fl(
                f"a7 grouped GEMM MXFP8, 32 experts, R={R}, N=4096 (gate+up), K=7168, bf16 out, block-scaled FP8 "
                "MFMA (within 1e-5 with fp32 out)", 2.0 * R * 4096 * 7168, ctx.timed(grouped), FP8_PEAK_TFLOPS, True,
                nbytes=32 * 4096 * 7168 * (1 + 1 / 32) + R * 7168 * (1 + 1 / 128) + R * 4096 * 2)
        grouped()
        del qw, sw
    if ctx.want("c4_grouped_fp4"):
        # variant beyond the pages (which keep the expert GEMMs in FP8): MXFP4
        # weights and activations, no repack; seeded random activation codes
        qw4, sw4 = ctx.u8(32, 4096, 3584), ctx.u8(32, 4096, 224)
        for e in range(32):
            mxq.quantize_mx(ctx.bf16(synth.c4_w(e)), mxq.E2M1, qw4[e], sw4[e])
        gen = torch.Generator(device=ctx.dev)
        gen.manual_seed(41)
        qa4 = torch.randint(0, 256, (R, 3584), generator=gen, dtype=torch.uint8, device=ctx.dev)
        sa4 = torch.full((R, 224), 127, dtype=torch.uint8, device=ctx.dev)
        Cg4 = torch.empty((R, 4096), dtype=torch.bfloat16, device=ctx.dev)
        t = ctx.timed(lambda: mxq.grouped_scaled_gemm(qa4, mxq.E2M1, sa4, 1, qw4, mxq.E2M1, sw4, 1, off_d, 32, R,
                                                      4096, 7168, Cg4, out=mxq.OUT_BF16))
        rows["c4_grouped_fp4"] = ctx.fl(
            f"a7 variant beyond the pages: grouped GEMM MXFP4 x MXFP4 (no repack), 32 experts, R={R}, N=4096, "
            "K=7168, bf16 out (FP4 products exact: within 1e-5)", 2.0 * R * 4096 * 7168, t, FP4_PEAK_TFLOPS, True,
            nbytes=32 * 4096 * 7168 * (0.5 + 1 / 32) + R * 7168 * (0.5 + 1 / 32) + R * 4096 * 2)
        del qw4, sw4, qa4, sa4, Cg4
    qh, sh = ctx.u8(R, 2048), ctx.u8(R, 64)
    if ctx.want("c4_swiglu"):
        rows["c4_swiglu"] = ctx.bw(f"f2 SwiGLU + MX E4M3 of the gate/up output, R={R} x 2048",
                                   R * (4096 * 2 + 2048 * (1 + 1 / 32)),
                                   ctx.timed(lambda: mxq.swiglu_quantize_mx(Cg, 2048, mxq.E4M3, qh, sh)))
    if ctx.want("c4_down"):
        mxq.swiglu_quantize_mx(Cg, 2048, mxq.E4M3, qh, sh)
        qd, sd = ctx.u8(32, 7168, 2048), ctx.u8(32, 7168, 64)
        for e in range(32):
            mxq.quantize_mx(ctx.bf16(synth.c4_w_down(e)), mxq.E4M3, qd[e], sd[e])
        Cd = torch.empty((R, 7168), dtype=torch.bfloat16, device=ctx.dev)
        t = ctx.timed(lambda: mxq.grouped_scaled_gemm(qh, mxq.E4M3, sh, 1, qd, mxq.E4M3, sd, 1, off_d, 32, R, 7168,
                                                      2048, Cd, out=mxq.OUT_BF16))
        rows["c4_down"] = ctx.fl(
            f"f2 down-projection grouped GEMM MXFP8, 32 experts, R={R}, N=7168, K=2048, bf16 out, block-scaled FP8 "
            "MFMA (within 1e-5 with fp32 out)", 2.0 * R * 7168 * 2048, t, FP8_PEAK_TFLOPS, True,
            nbytes=32 * 7168 * 2048 * (1 + 1 / 32) + R * 2048 * (1 + 1 / 32) + R * 7168 * 2)
        del qd, sd, Cd


def rows_c5(ctx, rows):
    """Workload 5: the 70B MLP tensors' dual quantization on their own, the
    up-projection on the block-scaled FP8 MFMA, and the same shape in MXFP4."""
    ids = ("c5_dual_h", "c5_dual_dy", "c5_fwd_up_native", "c5_fwd_up_mxfp4")
    if not any(ctx.want(i) for i in ids):
        return
    mxq, synth = ctx.mxq, ctx.synth
    for rid, spec, fmt, name in (("c5_dual_h", synth.c5_h(), mxq.E4M3, "E4M3, H"),
                                 ("c5_dual_dy", synth.c5_dy(), mxq.E5M2, "E5M2, dY")):
        if ctx.want(rid):
            v = ctx.bf16(spec)
            r, c = v.shape
            q, s, qc, sc = ctx.u8(r, c), ctx.u8(r, c // 32), ctx.u8(c, r), ctx.u8(c, r // 32)
            rows[rid] = ctx.bw(f"a4 MX {name} {r}x{c} bf16, row + col (dual)", v.numel() * (2 + 2 + 2 / 32),
                               ctx.timed(lambda: mxq.quantize_mx(v, fmt, q, s, qc, sc)))
            del v, q, s, qc, sc
    if not (ctx.want("c5_fwd_up_native") or ctx.want("c5_fwd_up_mxfp4")):
        return
    x5, wu = ctx.bf16(synth.c5_x()), ctx.bf16(synth.c5_w_up())
    C = ctx.f32(8192, 28672)
    for rid, fmt, peak, what in (
            ("c5_fwd_up_native", mxq.E4M3, FP8_PEAK_TFLOPS,
             "a6 MXFP8 GEMM 8192x28672x8192 fp32 out, block-scaled FP8 MFMA (misses 1e-5 normwise on this data)"),
            ("c5_fwd_up_mxfp4", mxq.E2M1, FP4_PEAK_TFLOPS,
             "a6 MXFP4 GEMM 8192x28672x8192 fp32 out (FP4 products exact: within 1e-5)")):
        if not ctx.want(rid):
            continue
        kb = 8192 // 2 if fmt == mxq.E2M1 else 8192
        qa, sa, qb, sb = ctx.u8(8192, kb), ctx.u8(8192, 256), ctx.u8(28672, kb), ctx.u8(28672, 256)
        mxq.quantize_mx(x5, fmt, qa, sa)
        mxq.quantize_mx(wu, fmt, qb, sb)
        t = ctx.timed(lambda: mxq.scaled_gemm(qa, fmt, sa, 1, qb, fmt, sb, 1, 8192, 28672, 8192, C))
        rows[rid] = ctx.fl(what, 2.0 * 8192 * 28672 * 8192, t, peak, fmt == mxq.E2M1)
        del qa, sa, qb, sb


def measure_rows(ctx):
    rows = {}
    for fn in (rows_c1, rows_c2, rows_c3, rows_c4, rows_c5):
        fn(ctx, rows)
        ctx.torch.cuda.empty_cache()
    return rows


# ----------------------------------------------------------------- CPU oracle

def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline():
    """The oracle as it stands, on a bounded sample of the headline workload:
    dual MX E4M3 quantization of all of X [8192, 8192], then the fp64 GEMM
    on the 1024 x 1024 entries C[0:1024, 0:1024] of the forward
    up-projection (K = 8192; W_up's first 1024 rows quantized for it).
    Reported in the headline unit (GEMM FLOP/s of the sample) with the
    quantize throughput beside it."""
    import oracle as O
    import synth
    O.lib()
    x = synth.tensor(synth.c5_x())
    w0 = synth.slab(synth.c5_w_up(), 0)  # rows 0..1023 of W_up
    t0 = time.perf_counter()
    qx, sx, _, _ = O.quantize_mx(x, O.E4M3, row=True, col=True)
    t1 = time.perf_counter()
    qw, sw, _, _ = O.quantize_mx(w0, O.E4M3)
    m = np.repeat(np.arange(1024), 1024)
    n = np.tile(np.arange(1024), 1024)
    t2 = time.perf_counter()
    O.gemm_entries(qx[:1024], O.E4M3, sx[:1024], O.SCALE_BLK32, qw, O.E4M3, sw, O.SCALE_BLK32, 8192, m, n)
    t3 = time.perf_counter()
    model, aff = cpu_info()
    q_bytes = x.size * (2 + 2 + 2 / 32)
    return {"value": round(2.0 * 8192 * len(m) / (t3 - t2) / 1e12, 6), "unit": "TFLOP/s", "cores": O.num_threads(),
            "kind": "oracle", "cpu_model": model, "affinity_cores": aff,
            "quantize_gbs": round(q_bytes / (t1 - t0) / 1e9, 4),
            "sample": "dual MX E4M3 quantize of all of X 8192x8192 (bf16), fp64 GEMM on the 1024x1024 entries "
                      f"C[0:1024, 0:1024] of the up-projection (K=8192); quantize {t1 - t0:.1f} s, "
                      f"GEMM {t3 - t2:.1f} s"}


def copy_probe(torch, dev):
    """A plain elementwise kernel that reads and writes exactly 1 GiB each
    (the reference for the traffic counters), timed: what a bandwidth-bound
    kernel that reads and writes equal amounts reaches on this GPU."""
    src = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(10):
        torch.cuda.synchronize()
        e0.record()
        torch.bitwise_not(src, out=dst)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2.0 * 2 ** 30 / (best * 1e-3) / 1e9
    return {"kernel": "elementwise bitwise_not, 1 GiB in + 1 GiB out", "ms": round(best, 4),
            "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the quantizers and "
              "GEMMs shard over rows or columns with no communication, which is not run here.", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    ctx = Ctx(args)
    ctx.mxq.lib()
    result = {
        "metric": "scaled-GEMM TFLOPS + quantize GB/s, % of MI355X FP8/FP4 & HBM peak",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3/e5m2 operands, bf16 MFMA, fp32 accumulation",
        "data": "synthetic (seeded numpy PCG64): Student-t(3) activations, N(0,0.015) weights, gradients "
                "|g| = 2^(3z) with random sign, bf16",
        "config": {"workload": "llama3-70b-mlp-mxfp8-fwd-bwd", "tokens": 8192, "hidden": 8192, "intermediate": 28672,
                   "step": "6 dual MX quantizes (X, W_up, H, W_down E4M3; dY, dZ E5M2) + 6 GEMMs (fwd up/down, "
                           "dgrad and wgrad of both), precise mode, fp32 out",
                   "parallelism": "none (1 GPU)"},
    }
    if ctx.want("headline"):
        result.update(headline(ctx))
    if args.copy_probe or not args.no_rows:
        result["hbm_copy"] = copy_probe(torch, ctx.dev)
    if not args.no_rows:
        result["rows"] = measure_rows(ctx)
        result["row_timing"] = {"reps": args.row_reps, "warmup": args.row_warmup,
                                "flush": "1 GiB fill before each timed repetition"}
    if not args.no_cpu_baseline and ctx.want("headline"):
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
