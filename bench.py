"""Benchmark of the scaled-quantization + block-scaled GEMM hot path on one MI355X.

Headline step (workload "llama3-8b-mlp-up-mxfp8-fwd"): MX block-32 E4M3
quantization of the activations X [4096, 4096] and of the weights
W [14336, 4096] (bf16 inputs), then the MXFP8 scaled GEMM M=4096, N=14336,
K=4096 with fp32 output.  `value` is the step's whole-job throughput
2*M*N*K / step time (TFLOP/s) with inputs resident in HBM.

Also reported (one JSON line): the dominant kernel's roofline (the GEMM,
timed with HIP events on the stream it runs on), the other rows of the hot
path measured on their own workloads, and the CPU oracle timed on a bounded
sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows]
       [--no-cpu-baseline] [--copy-probe]

roofline.traffic is the GEMM's HBM bytes per launch from the committed
rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/ (each counter
scaled by what it reads for a plain copy of known size, --copy-probe), and
null when the GEMM source has changed since those counters were taken.
"""
import hashlib
import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row measurements")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--row-reps", type=int, default=10, help="timed repetitions per row (median, p10/p90)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (reference for the traffic counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_gemm_mxfp8_4096x14336x4096_hbm_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "mxfp4_precision_numerics_amd", "csrc", "gemm.hip")


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    if there is none or the kernel source differs from the one counted."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    sha = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
    if kv.get("gemm_source_sha256") != sha or "traffic_bytes" not in kv:
        return None
    return int(float(kv["traffic_bytes"]))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the quantizers and "
              "GEMMs shard over rows or columns with no communication, which is not run here.", file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp4_precision_numerics_amd as mxq
    import synth

    assert torch.cuda.is_available(), "bench.py needs the MI355X"
    mxq.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---------------- headline workload -----------------------------------
    M, N, K = 4096, 14336, 4096
    x = bf16(synth.tensor(synth.c2_x()))
    w = bf16(synth.tensor(synth.c2_w()))
    u8 = dict(dtype=torch.uint8, device=dev)
    qx, sx = torch.empty((M, K), **u8), torch.empty((M, K // 32), **u8)
    qw, sw = torch.empty((N, K), **u8), torch.empty((N, K // 32), **u8)
    C = torch.empty((M, N), dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        mxq.quantize_mx(x, mxq.E4M3, qx, sx)
        if ev is not None:
            ev[1].record(stream)
        mxq.quantize_mx(w, mxq.E4M3, qw, sw)
        if ev is not None:
            ev[2].record(stream)
        mxq.scaled_gemm(qx, mxq.E4M3, sx, mxq.SCALE_BLK32, qw, mxq.E4M3, sw, mxq.SCALE_BLK32, M, N, K, C)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    qx_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    qw_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    gemm_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    qbytes_x = M * K * (2 + 1 + 1 / 32)
    qbytes_w = N * K * (2 + 1 + 1 / 32)

    result = {
        "metric": "scaled-GEMM TFLOPS + quantize GB/s, % of MI355X FP8/FP4 & HBM peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3",
        "data": "synthetic (seeded numpy PCG64; bf16 N(0,1) activations with 41 outlier columns x50, "
                "N(0,0.02) weights)",
        "config": {"workload": "llama3-8b-mlp-up-mxfp8-fwd", "M": M, "N": N, "K": K,
                   "step": "quantize_mx(X) + quantize_mx(W) + scaled_gemm", "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "k_gemm<E4M3,E4M3> (256x256 tiles + a 128x256 launch for the last round)", "bound": "mfma", "achieved": round(gemm_tflops, 1),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": gemm_traffic()},
        "kernels_ms": {"quantize_mx_x": round(qx_ms, 4), "quantize_mx_w": round(qw_ms, 4),
                       "scaled_gemm": round(gemm_ms, 4)},
        "quantize_gbs": {"x": round(qbytes_x / (qx_ms * 1e-3) / 1e9, 1),
                         "w": round(qbytes_w / (qw_ms * 1e-3) / 1e9, 1)},
    }
    del C
    torch.cuda.empty_cache()

    if args.copy_probe:
        # an elementwise kernel that reads and writes exactly 1 GiB each
        src = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    if not args.no_rows:
        result["rows"] = measure_rows(torch, mxq, synth, dev, args.row_reps)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth)

    print(json.dumps(result), flush=True)


def measure_rows(torch, mxq, synth, dev, reps):
    """Every other row of the hot path on its own workload, cold cache (a
    512 MiB fill runs between repetitions, outside the timed interval).
    Algorithmic bytes per element are those the method itself must move."""
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
    u8 = dict(dtype=torch.uint8, device=dev)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            flush.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        spread[0] = [round(float(np.percentile(ts, q)), 4) for q in (10, 90)]
        return float(np.median(ts))

    spread = [None]  # p10 / p90 of the last timed() call, ms

    def bw(nbytes, ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 4), "ms_p10_p90": spread[0], "GB/s": round(gbs, 1),
                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}

    def fl(nflop, ms, peak):
        tf = nflop / (ms * 1e-3) / 1e12
        return {"ms": round(ms, 4), "ms_p10_p90": spread[0], "TFLOP/s": round(tf, 1), "frac_peak": round(tf / peak, 4),
                "peak": peak}

    rows = {}
    # a1-a3: per-tensor delayed E5M2 cast of dY [4096, 14336] with row + col outputs
    hist = torch.zeros(16, dtype=torch.float32, device=dev)
    amax, sc, si = (torch.empty(1, device=dev) for _ in range(3))
    for t in range(16):
        p = bf16(synth.tensor(synth.c3_prior_dy(t)))
        mxq.quantize_per_tensor(p, mxq.E5M2, amax, sc, si, torch.empty(p.shape, **u8), amax_history=hist)
    dy = bf16(synth.tensor(synth.c3_dy()))
    qr, qc = torch.empty((4096, 14336), **u8), torch.empty((14336, 4096), **u8)
    ms = timed(lambda: mxq.quantize_per_tensor(dy, mxq.E5M2, amax, sc, si, qr, qc, amax_history=hist))
    rows["a1-a3 per-tensor delayed E5M2 cast, dY 4096x14336 bf16, row+col"] = bw(dy.numel() * 4, ms)
    # current scaling must see the whole tensor's amax before casting: the amax
    # pass reads dY once more (6 B per element: 2 reads, two 1-byte outputs)
    amax_c = torch.empty(1, device=dev)
    ms = timed(lambda: mxq.quantize_per_tensor(dy, mxq.E5M2, amax_c, sc, si, qr, qc))
    rows["a1-a3 per-tensor current E5M2 (amax pass + cast), dY 4096x14336 bf16, row+col"] = bw(dy.numel() * 6, ms)
    # a6 per-tensor FP8 GEMMs of the backward pass (E5M2 x E4M3)
    w = bf16(synth.tensor(synth.c3_w()))
    qwr, qwc = torch.empty((14336, 4096), **u8), torch.empty((4096, 14336), **u8)
    hw = torch.zeros(16, dtype=torch.float32, device=dev)
    sw = torch.empty(1, device=dev)
    mxq.quantize_per_tensor(w, mxq.E4M3, amax, sc, sw, qwr, qwc, amax_history=hw)
    C = torch.empty((4096, 4096), dtype=torch.float32, device=dev)
    ms = timed(lambda: mxq.scaled_gemm(qr, mxq.E5M2, si, 0, qwc, mxq.E4M3, sw, 0, 4096, 4096, 14336, C))
    rows["a6 dgrad GEMM E5M2xE4M3 per-tensor, M=4096 N=4096 K=14336"] = fl(2.0 * 4096 * 4096 * 14336, ms,
                                                                            FP8_PEAK_TFLOPS)
    x3 = bf16(synth.tensor(synth.c3_x()))
    qxr, qxc = torch.empty((4096, 4096), **u8), torch.empty((4096, 4096), **u8)
    sx = torch.empty(1, device=dev)
    mxq.quantize_per_tensor(x3, mxq.E4M3, amax, sc, sx, qxr, qxc, amax_history=torch.zeros(16, device=dev))
    C2 = torch.empty((4096, 14336), dtype=torch.float32, device=dev)
    ms = timed(lambda: mxq.scaled_gemm(qxc, mxq.E4M3, sx, 0, qc, mxq.E5M2, si, 0, 4096, 14336, 4096, C2))
    rows["a6 wgrad GEMM E4M3xE5M2 per-tensor, M=4096 N=14336 K=4096"] = fl(2.0 * 4096 * 14336 * 4096, ms,
                                                                           FP8_PEAK_TFLOPS)
    del dy, qr, qc, w, qwr, qwc, x3, qxr, qxc, C, C2
    torch.cuda.empty_cache()

    # workload 4: MXFP4 quantize, gather + repack, grouped GEMM
    x = bf16(synth.tensor(synth.c4_x()))
    idx, off = synth.c4_routing()
    R = int(off[-1])
    q4, s4 = torch.empty((8192, 3584), **u8), torch.empty((8192, 224), **u8)
    ms = timed(lambda: mxq.quantize_mx(x, mxq.E2M1, q4, s4))
    rows["a4 MX quantize bf16->E2M1, X 8192x7168"] = bw(x.numel() * (2 + 0.5 + 1 / 32), ms)
    q8, s8 = torch.empty((R, 7168), **u8), torch.empty((R, 56), **u8)
    idx_d = torch.from_numpy(idx).to(dev)
    ms = timed(lambda: mxq.repack_fp4_to_fp8(q4, s4, q8, s8, gather_idx=idx_d))
    rows[f"a5 FP4->FP8 repack with gather, R={R} rows x 7168"] = bw(R * (3584 + 224 + 4 + 7168 + 56), ms)
    q8c, s8c = torch.empty((7168, 8192), **u8), torch.empty((7168, 256), **u8)
    ms = timed(lambda: mxq.fp4_row_to_fp8_col(q4, s4, q8c, s8c))
    rows["f1 FP4 row -> FP8 col (dequant, transpose, MX E4M3), X 8192x7168"] = bw(
        x.numel() * (0.5 + 1 / 32 + 1 + 1 / 32), ms)
    del x, q8c, s8c
    qw = torch.empty((32, 4096, 7168), **u8)
    sw4 = torch.empty((32, 4096, 224), **u8)
    for e in range(32):
        we = bf16(synth.tensor(synth.c4_w(e)))
        mxq.quantize_mx(we, mxq.E4M3, qw[e], sw4[e])
    del we
    off_d = torch.from_numpy(off).to(dev)
    Cg = torch.empty((R, 4096), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: mxq.grouped_scaled_gemm(q8, mxq.E4M3, s8, mxq.SCALE_BLK128, qw, mxq.E4M3, sw4,
                                               mxq.SCALE_BLK32, off_d, 32, R, 4096, 7168, Cg, out=mxq.OUT_BF16))
    gflop = 2.0 * R * 4096 * 7168
    gbytes = 32 * 4096 * 7168 * (1 + 1 / 32) + R * 7168 * (1 + 1 / 128) + R * 4096 * 2
    r = fl(gflop, ms, FP8_PEAK_TFLOPS)
    r["GB/s"] = round(gbytes / (ms * 1e-3) / 1e9, 1)
    r["frac_hbm"] = round(r["GB/s"] / HBM_PEAK_GBS, 4)
    rows[f"a7 grouped GEMM MXFP8, 32 experts, R={R}, N=4096, K=7168, bf16 out"] = r
    del qw, sw4
    # variant beyond the pages (which keep the expert GEMMs in FP8): the same
    # grouped GEMM with MXFP4 weights and MXFP4 activations; the R activation
    # rows are seeded random E2M1 codes with unit scales (values do not change
    # the timing)
    qw4 = torch.empty((32, 4096, 3584), **u8)
    sw44 = torch.empty((32, 4096, 224), **u8)
    for e in range(32):
        we = bf16(synth.tensor(synth.c4_w(e)))
        mxq.quantize_mx(we, mxq.E2M1, qw4[e], sw44[e])
    del we
    Cg4 = torch.empty((R, 4096), dtype=torch.bfloat16, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    qa4 = torch.randint(0, 256, (R, 3584), generator=gen, **u8)
    sa4 = torch.full((R, 224), 127, **u8)
    ms = timed(lambda: mxq.grouped_scaled_gemm(qa4, mxq.E2M1, sa4, mxq.SCALE_BLK32, qw4, mxq.E2M1, sw44,
                                               mxq.SCALE_BLK32, off_d, 32, R, 4096, 7168, Cg4, out=mxq.OUT_BF16))
    gbytes4 = 32 * 4096 * 7168 * (0.5 + 1 / 32) + R * 7168 * (0.5 + 1 / 32) + R * 4096 * 2
    r = fl(gflop, ms, FP4_PEAK_TFLOPS)
    r["GB/s"] = round(gbytes4 / (ms * 1e-3) / 1e9, 1)
    r["frac_hbm"] = round(r["GB/s"] / HBM_PEAK_GBS, 4)
    rows[f"a7 variant: grouped GEMM MXFP4 x MXFP4 (no repack), 32 experts, R={R}, N=4096, K=7168, bf16 out"] = r
    del qw4, sw44, Cg4, qa4, sa4
    # the rest of the expert MLP on the up-projection's output: SwiGLU + MX
    # E4M3, then the down-projection grouped GEMM (N = 7168, K = 2048)
    qh, sh = torch.empty((R, 2048), **u8), torch.empty((R, 64), **u8)
    ms = timed(lambda: mxq.swiglu_quantize_mx(Cg, 2048, mxq.E4M3, qh, sh))
    rows[f"f2 SwiGLU + MX E4M3 of the gate/up output, R={R} x 2048"] = bw(R * (4096 * 2 + 2048 * (1 + 1 / 32)), ms)
    qd = torch.empty((32, 7168, 2048), **u8)
    sd = torch.empty((32, 7168, 64), **u8)
    for e in range(32):
        wd = bf16(synth.tensor(synth.c4_w_down(e)))
        mxq.quantize_mx(wd, mxq.E4M3, qd[e], sd[e])
    del wd
    Cd = torch.empty((R, 7168), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: mxq.grouped_scaled_gemm(qh, mxq.E4M3, sh, mxq.SCALE_BLK32, qd, mxq.E4M3, sd,
                                               mxq.SCALE_BLK32, off_d, 32, R, 7168, 2048, Cd, out=mxq.OUT_BF16))
    gflop = 2.0 * R * 7168 * 2048
    gbytes = 32 * 7168 * 2048 * (1 + 1 / 32) + R * 2048 * (1 + 1 / 32) + R * 7168 * 2
    r = fl(gflop, ms, FP8_PEAK_TFLOPS)
    r["GB/s"] = round(gbytes / (ms * 1e-3) / 1e9, 1)
    r["frac_hbm"] = round(r["GB/s"] / HBM_PEAK_GBS, 4)
    rows[f"f2 down-projection grouped GEMM MXFP8, 32 experts, R={R}, N=7168, K=2048, bf16 out"] = r
    del q4, s4, q8, s8, Cg, qh, sh, qd, sd, Cd
    torch.cuda.empty_cache()

    # workload 5: dual MX quantize of H and the 70B up-projection GEMM (MXFP8, and MXFP4 variant)
    h = bf16(synth.tensor(synth.c5_h()))
    qh, sh = torch.empty((8192, 28672), **u8), torch.empty((8192, 896), **u8)
    qhc, shc = torch.empty((28672, 8192), **u8), torch.empty((28672, 256), **u8)
    ms = timed(lambda: mxq.quantize_mx(h, mxq.E4M3, qh, sh, qhc, shc))
    rows["a4 MX quantize bf16->E4M3 row+col, H 8192x28672"] = bw(h.numel() * (2 + 2 + 2 / 32), ms)
    del h, qh, sh, qhc, shc
    x5 = bf16(synth.tensor(synth.c5_x()))
    wu = bf16(synth.tensor(synth.c5_w_up()))
    res = {}
    for fmt, name in ((mxq.E4M3, "MXFP8"), (mxq.E2M1, "MXFP4")):
        kb = 8192 // 2 if fmt == mxq.E2M1 else 8192
        qa, sa = torch.empty((8192, kb), **u8), torch.empty((8192, 256), **u8)
        qb, sb = torch.empty((28672, kb), **u8), torch.empty((28672, 256), **u8)
        mxq.quantize_mx(x5, fmt, qa, sa)
        mxq.quantize_mx(wu, fmt, qb, sb)
        C5 = torch.empty((8192, 28672), dtype=torch.bfloat16, device=dev)
        ms = timed(lambda: mxq.scaled_gemm(qa, fmt, sa, 1, qb, fmt, sb, 1, 8192, 28672, 8192, C5, out=mxq.OUT_BF16))
        peak = FP4_PEAK_TFLOPS if fmt == mxq.E2M1 else FP8_PEAK_TFLOPS
        rows[f"a6 {name} GEMM, M=8192 N=28672 K=8192, bf16 out"] = fl(2.0 * 8192 * 28672 * 8192, ms, peak)
        del qa, sa, qb, sb, C5
        torch.cuda.empty_cache()
    return rows


def cpu_baseline(synth):
    """The oracle as it stands, on a bounded sample of the headline workload:
    MX E4M3 quantization of all of X [4096, 4096] and W [14336, 4096], then
    the fp64 GEMM on the 1024 x 1536 entries C[0:1024, 0:1536] (K=4096).
    Reported in the headline unit (GEMM FLOP/s of the sample) with the
    quantize throughput beside it."""
    import oracle as O
    O.lib()
    x = synth.tensor(synth.c2_x())
    w = synth.tensor(synth.c2_w())
    t0 = time.perf_counter()
    qx, sx, _, _ = O.quantize_mx(x, O.E4M3)
    qw, sw, _, _ = O.quantize_mx(w, O.E4M3)
    t1 = time.perf_counter()
    m = np.repeat(np.arange(1024), 1536)
    n = np.tile(np.arange(1536), 1024)
    O.gemm_entries(qx, O.E4M3, sx, O.SCALE_BLK32, qw, O.E4M3, sw, O.SCALE_BLK32, 4096, m, n)
    t2 = time.perf_counter()
    q_bytes = (x.size + w.size) * (2 + 1 + 1 / 32)
    gemm_flops = 2.0 * 4096 * len(m)
    return {"value": round(gemm_flops / (t2 - t1) / 1e12, 6), "unit": "TFLOP/s", "cores": O.num_threads(),
            "kind": "oracle", "quantize_gbs": round(q_bytes / (t1 - t0) / 1e9, 4),
            "sample": "MX E4M3 quantize of all of X 4096x4096 and W 14336x4096 (bf16), fp64 GEMM on the "
                      f"1024x1536 entries C[0:1024, 0:1536] (K=4096); quantize {t1 - t0:.1f} s, GEMM {t2 - t1:.1f} s"}


if __name__ == "__main__":
    main()
