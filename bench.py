"""Benchmark of the scaled FP8 GEMM hot path on one MI355X.

One step = the whole path over one batch of synthetic input already resident in
HBM: quantise A and B (amax / scale and e4m3 encoding) and run the GEMM (MFMA
mainloop, scale/cast epilogue, tile scheduling); the grouped workload runs the
grouped GEMM instead.  Untimed steps for at least --settle-ms (a GPU that was
idle runs its first ~25 ms of load up to 15 % slower, so a short run would time
that ramp rather than the kernels), then W untimed warm-up steps, then K timed
steps between two ``torch.cuda.synchronize()``; one JSON line goes to stdout.

``value`` is 2*M*N*K per step over the wall time of the timed steps (TFLOP/s,
the formula of the Cutlass-named Triton FP8 post's monitoring list).  The
``roofline`` object describes the dominant kernel (the GEMM): its algorithmic
FLOPs per launch over its average duration, measured with HIP events recorded
on the stream it is launched on, against the MI355X dense FP8 MFMA peak.
``cpu_baseline`` times the CPU oracle (numpy, float64) on a bounded sample of
the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import WORKLOADS, dense_inputs, grouped_inputs  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 MFMA peak (no sparsity)
PEAK_FP4_TFLOPS = 10100.0         # MI355X dense FP4 (MXFP4) MFMA peak
PEAK_FP6_TFLOPS = 10100.0         # MI355X dense FP6 (MXFP6) MFMA peak
PEAK_HBM_GBS = 8000.0             # MI355X HBM3E
DEFAULT_WORKLOAD = "mx8192"
# the pages' own figures, measured on other hardware: context, not targets
PAGES_CONTEXT = {
    "h100_sxm5_fp8_dense_peak_tflops": 1979,
    "h100_m128_n4096_k4096_fp8_gemm_tbs": {"cuBLAS": 1.55, "Triton+TMA": 1.45,
                                           "Triton cp.async": 0.95},
    "source": "Hopper/Blackwell architecture features, 12.1.1 and 12.2.4 (H100 SXM5)",
}
KERNEL_SOURCES = ["block_scaled_gemm_fp8gemm_amd/csrc/gemm_tile.h",
                  "block_scaled_gemm_fp8gemm_amd/csrc/gemm.hip",
                  "block_scaled_gemm_fp8gemm_amd/csrc/grouped.hip",
                  "block_scaled_gemm_fp8gemm_amd/csrc/tile_order.h",
                  "block_scaled_gemm_fp8gemm_amd/csrc/device_utils.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary.

    None when there is no summary for this workload or the kernel sources have
    changed since the counters were taken.
    """
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_CAL_BYTES = 1 << 30          # plain device copy used to calibrate the byte counters


def copy_calibration(dev):
    """A plain device-to-device copy of COPY_CAL_BYTES, three times, for the counter
    runs: FETCH_SIZE / WRITE_SIZE of its dispatches give the scale between the
    counters and true bytes."""
    import torch
    src = torch.ones(COPY_CAL_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 copies of {COPY_CAL_BYTES} bytes")


def _counter_values(csv_path, counter):
    """Per-kernel list of one rocprofv3 counter over its dispatches (KiB for
    FETCH_SIZE / WRITE_SIZE)."""
    import csv
    import collections
    vals = collections.defaultdict(list)
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            if row.get("Counter_Name") != counter:
                continue
            vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
    return vals


GEMM_KERNELS = ("gemm_kernel", "gemm_persistent_kernel", "splitk_kernel", "grouped_kernel")


def summarize_traffic(workload: str, fetch_csv: str, write_csv: str, command: str):
    """Write profiles/gemm_<workload>_traffic.json from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE) of `bench.py --copy-calibration`.

    The GEMM figure is the mean over its dispatches.  The copy kernel also serves
    the bench's own small host-to-device and device copies, so its scale comes
    from its three largest dispatches, the 1 GiB calibration copies."""
    fetch = _counter_values(fetch_csv, "FETCH_SIZE")
    write = _counter_values(write_csv, "WRITE_SIZE")
    gemm_name = [k for k in fetch if "fp8gemm" in k and any(g in k for g in GEMM_KERNELS)]
    copy_name = [k for k in fetch if "copy" in k.lower() and "fp8gemm" not in k]
    if len(gemm_name) != 1 or len(copy_name) != 1:
        raise SystemExit(f"expected one GEMM and one copy kernel, got {gemm_name} / {copy_name}")
    g, c = gemm_name[0], copy_name[0]
    mean = lambda v: sum(v) / len(v)
    top3 = lambda v: mean(sorted(v)[-3:])
    fg, wg = mean(fetch[g]), mean(write[g])
    fc, wc = top3(fetch[c]), top3(write[c])
    fetch_scale = COPY_CAL_BYTES / (fc * 1024.0)
    write_scale = COPY_CAL_BYTES / (wc * 1024.0)
    fetch_b = fg * 1024.0 * fetch_scale
    write_b = wg * 1024.0 * write_scale
    rec = {"workload": workload, "kernel": g, "kernel_source_digest": kernel_source_digest(),
           "gemm_dispatches": len(fetch[g]),
           "fetch_kib_per_launch_raw": fg, "write_kib_per_launch_raw": wg,
           "copy_kernel": c, "copy_bytes": COPY_CAL_BYTES,
           "copy_fetch_kib_raw": fc, "copy_write_kib_raw": wc,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "hbm_fetch_bytes_per_launch": round(fetch_b), "hbm_write_bytes_per_launch": round(write_b),
           "hbm_bytes_per_launch": round(fetch_b + write_b), "command": command}
    out = os.path.join(ROOT, "profiles", f"gemm_{workload}_traffic.json")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))


def gemm_bytes(w, code_bytes: float = 1.0) -> int:
    """Algorithmic bytes of one GEMM launch: A + B codes (code_bytes per element:
    1, 0.75 for FP6 or 0.5 for FP4), scales, C."""
    mb = int((w.M * w.K + (w.groups or 1) * w.N * w.K) * code_bytes)
    if w.mode == "mx32":
        mb += (w.M + (w.groups or 1) * w.N) * (w.K // 32)
    elif w.mode == "rowwise":
        mb += 4 * (w.M + (w.groups or 1) * w.N)
    else:
        mb += 8
    return mb + 2 * w.M * w.N


def gemm_bytes_mxout(w, code_bytes: float = 1.0) -> int:
    """The same with the output as e4m3 codes plus one E8M0 code per 32 columns."""
    return gemm_bytes(w, code_bytes) - 2 * w.M * w.N + w.M * w.N + w.M * (w.N // 32)


def gemm_bytes_qout(w, code_bytes: float = 1.0) -> int:
    """The same with the output as e4m3 codes plus fp32 scales (one per row; the
    per-tensor case counts the same): the result's own bytes, not the bf16 y the
    implementation writes and reads back between its two kernels."""
    return gemm_bytes(w, code_bytes) - 2 * w.M * w.N + w.M * w.N + 4 * w.M


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, rows: int, fmt: str = "e4m3", runs: int = 3):
    """Oracle on a bounded sample: quantise `rows` rows of A and of B (element
    format fmt), then the float64 GEMM reference of that rows x rows x K block
    (value and sum|a*b|); the median of `runs` runs, and the full problem's time
    extrapolated from it at the same rate."""
    import numpy as np
    import oracle as O
    from oracle import quant as Q
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    if w.groups:
        counts, A, W = grouped_inputs(w, experts=(0,))
        Bs = W[0][:rows]
    else:
        A, B = dense_inputs(w)
        Bs = B[:rows]
    As = A[:rows]
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        qa, sa = Q.quantize(As, w.mode, fmt)
        qb, sb = Q.quantize(Bs, w.mode, fmt)
        O.gemm_reference(qa, sa, qb, sb, w.mode, fmt_a=fmt, fmt_b=fmt)
        times.append(time.perf_counter() - t0)
    dt = sorted(times)[len(times) // 2]
    flops = 2.0 * rows * rows * w.K
    rate = flops / dt
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(), "runs": runs, "median_s": round(dt, 3),
            "run_s": [round(t, 3) for t in times],
            "extrapolated_full_problem_s": round(w.flops / rate, 1),
            "extrapolation": "extrapolated: the full problem's FLOPs at the sample's measured rate "
                             "(quantisation and GEMM counted as one rate)",
            "sample": f"{rows} rows of A and {rows} columns of B (K={w.K}, {fmt}): quantise "
                      f"both, float64 GEMM reference with sum|a*b|; median of {runs} runs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--formats", default="e4m3,e4m3", metavar="A,B",
                    help="element formats of the A and B codes (e4m3 or e5m2; e2m1,e2m1 for "
                         "MXFP4; e2m3 or e3m2 in any pairing for MXFP6, dense mx32 workloads "
                         "with K % 128 == 0)")
    ap.add_argument("--epilogue", default="none", choices=["none", "bias", "bias+relu",
                                                           "bias+gelu", "bias+silu", "mxout",
                                                           "qrow", "qtensor"],
                    help="fused epilogue of the GEMM (dense only); mxout: the output quantised "
                         "for the next layer (e4m3 + E8M0 per 32 columns); qrow / qtensor: "
                         "quantised with a fresh fp32 scale per row / for the whole output "
                         "(the timed GEMM then includes the requantising kernel)")
    ap.add_argument("--b-layout", default="nk", choices=["nk", "kn"],
                    help="kn: B row-major [K, N] (fp8gemm_run_kn, its transposing copy timed "
                         "with the GEMM); B is then quantised once before timing (resident "
                         "weights) and a step is quantise A + GEMM")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="before the warm-up steps, run untimed steps for at least this long "
                         "(a GPU that was idle runs its first ~25 ms of load up to 15 %% "
                         "slower); 0: none")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="rows of A / columns of B in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/gemm_<workload>_traffic.json from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE); no GPU work")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command, recorded in the traffic summary")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args.workload, *args.summarize_traffic, command=args.traffic_command)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_gemm_fp8gemm_amd as F

    w = WORKLOADS[args.workload]
    fmt_a, fmt_b = args.formats.split(",")
    act = args.epilogue.split("+")[1] if "+" in args.epilogue else "none"
    mxout = args.epilogue == "mxout"
    qout = args.epilogue in ("qrow", "qtensor")
    kn = args.b_layout == "kn"
    if kn and (w.groups or mxout or qout):
        raise SystemExit("--b-layout kn applies to the dense workloads with a 16-bit output")
    use_bias = args.epilogue not in ("none", "mxout", "qrow", "qtensor")
    fp4 = "e2m1" in (fmt_a, fmt_b)
    if w.groups and ((args.formats != "e4m3,e4m3" and not fp4) or use_bias or mxout or qout):
        raise SystemExit("--epilogue applies to the dense workloads; the grouped one takes "
                         "--formats e2m1,e2m1 only")
    if fp4 and w.groups:       # MXFP4 experts: the same shapes and inputs with MX scales
        w = dataclasses.replace(w, mode="mx32")
    if fp4 and (fmt_a != fmt_b or w.mode != "mx32"):
        raise SystemExit("e2m1 (MXFP4) runs as e2m1,e2m1 on an mx32 workload")
    fp6_fmts = ("e2m3", "e3m2")
    fp6 = fmt_a in fp6_fmts or fmt_b in fp6_fmts
    if fp6 and (fmt_a not in fp6_fmts or fmt_b not in fp6_fmts or w.mode != "mx32" or w.groups
                or kn or w.K % 128):
        raise SystemExit("MXFP6 runs as e2m3 / e3m2 pairs on a dense mx32 workload, K % 128 == 0")
    kq = w.K // 2 if fp4 else w.K * 3 // 4 if fp6 else w.K     # code bytes per row
    peak = PEAK_FP4_TFLOPS if fp4 else PEAK_FP6_TFLOPS if fp6 else PEAK_FP8_TFLOPS
    code_bytes = 0.5 if fp4 else 0.75 if fp6 else 1.0
    dev = torch.device("cuda:0")
    F.load_library()
    log(f"workload {w.name}: M={w.M} N={w.N} K={w.K} mode={w.mode} out={w.out} groups={w.groups}")

    # ---- synthetic inputs, resident in HBM before timing -------------------------
    if w.groups:
        counts, A, W = grouped_inputs(w)
        import numpy as np
        offsets = torch.from_numpy(
            np.concatenate([[0], np.cumsum(counts)]).astype("int32")).to(dev)
        Ad = torch.from_numpy(A).to(dev)
        Bd = torch.from_numpy(W).to(dev).view(w.groups * w.N, w.K)
        del A, W
    else:
        A, B = dense_inputs(w)
        Ad = torch.from_numpy(A).to(dev)
        Bd = torch.from_numpy(B).to(dev)
        del A, B
    rows_b = Bd.shape[0]

    # ---- outputs and workspaces allocated once ---------------------------------
    qa = torch.empty((w.M, kq), dtype=torch.uint8, device=dev)
    qb = torch.empty((rows_b, kq), dtype=torch.uint8, device=dev)
    if w.mode == "tensor":
        sa = torch.empty(1, dtype=torch.float32, device=dev)
        sb = torch.empty(1, dtype=torch.float32, device=dev)
    elif w.mode == "rowwise":
        sa = torch.empty(w.M, dtype=torch.float32, device=dev)
        sb = torch.empty(rows_b, dtype=torch.float32, device=dev)
    else:
        sa = torch.empty((w.M, w.K // 32), dtype=torch.uint8, device=dev)
        sb = torch.empty((rows_b, w.K // 32), dtype=torch.uint8, device=dev)
    mode_id = F.SCALE_MODES[w.mode]
    ws_a = ws_b = None
    if F.fp8gemm_quantize_workspace_size(w.M, w.K, mode_id):
        ws_a = torch.empty(F.fp8gemm_quantize_workspace_size(w.M, w.K, mode_id),
                           dtype=torch.uint8, device=dev)
        ws_b = torch.empty_like(ws_a)
    tdt = torch.bfloat16 if w.out == "bf16" else torch.float16
    C = torch.empty((w.M, w.N), dtype=tdt, device=dev)
    if mxout:
        Cq = torch.empty((w.M, w.N), dtype=torch.uint8, device=dev)
        Cs = torch.empty((w.M, w.N // 32), dtype=torch.uint8, device=dev)
    if qout:
        qmode = "rowwise" if args.epilogue == "qrow" else "tensor"
        Cq = torch.empty((w.M, w.N), dtype=torch.uint8, device=dev)
        Cs = torch.empty(w.M if qmode == "rowwise" else 1, dtype=torch.float32, device=dev)
        ws_q = torch.zeros(F.fp8gemm_qout_workspace_size(w.M, w.N, w.K, mode_id),
                           dtype=torch.uint8, device=dev)
    bias = None
    if use_bias:
        import numpy as np
        bias = torch.from_numpy(
            np.random.default_rng(w.seed + 1).standard_normal(w.N).astype("float32")).to(dev)

    def run_gemm():
        if w.groups:
            if w.mode == "tensor":
                raise SystemExit("grouped per-tensor benchmarking is not configured")
            F.grouped_gemm(qa, sa, offsets, qb.view(w.groups, w.N, kq),
                           sb.view(w.groups, -1) if w.mode == "mx32" else sb.view(w.groups, w.N),
                           w.mode, w.out, out=C, fmt=fmt_a)
        elif kn:
            F.gemm(qa, sa, qb_kn, sb_kn, w.mode, w.out, out=C, fmt_a=fmt_a, fmt_b=fmt_b,
                   bias=bias, activation=act, b_layout="kn")
        elif mxout:
            F.gemm_mxout(qa, sa, qb, sb, w.mode, out=Cq, out_scales=Cs, fmt_a=fmt_a, fmt_b=fmt_b)
        elif qout:
            F.gemm_qout(qa, sa, qb, sb, w.mode, qmode, out=Cq, out_scales=Cs, workspace=ws_q,
                        fmt_a=fmt_a, fmt_b=fmt_b)
        else:
            F.gemm(qa, sa, qb, sb, w.mode, w.out, out=C, fmt_a=fmt_a, fmt_b=fmt_b, bias=bias,
                   activation=act)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        F.quantize(Ad, w.mode, out=qa, scales=sa, workspace=ws_a, fmt=fmt_a)
        if ev is not None:
            ev[1].record()
        if not kn:
            F.quantize(Bd, w.mode, out=qb, scales=sb, workspace=ws_b, fmt=fmt_b)
        if ev is not None:
            ev[2].record()
        run_gemm()
        if ev is not None:
            ev[3].record()

    if kn:   # resident row-major weights: quantised and laid out once, before timing
        F.quantize(Bd, w.mode, out=qb, scales=sb, workspace=ws_b, fmt=fmt_b)
        if fp4:   # packed [N, K/2] along K -> [K, N/2] packed along N (low nibble first)
            codes = torch.stack((qb & 15, qb >> 4), dim=2).reshape(rows_b, w.K).t()
            qb_kn = (codes[:, 0::2] | (codes[:, 1::2] << 4)).contiguous()
        else:
            qb_kn = qb.t().contiguous()
        sb_kn = sb.t().contiguous() if w.mode == "mx32" else sb
        torch.cuda.synchronize()
    # settle: untimed steps until the GPU has run the hot path for settle_ms, so
    # that the timed steps see its steady state whatever the warm-up count
    settle_steps = 0
    t_settle = time.perf_counter()
    while args.settle_ms > 0:
        for _ in range(8):
            step()
        settle_steps += 8
        torch.cuda.synchronize()
        if (time.perf_counter() - t_settle) * 1e3 >= args.settle_ms:
            break
    settle_ms = (time.perf_counter() - t_settle) * 1e3 if settle_steps else 0.0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"settled ({settle_steps} steps, {settle_ms:.0f} ms), warm-up done ({args.warmup} steps)")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {elapsed * 1e3:.2f} ms")

    qa_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    qb_ms = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    gemm_each = sorted(e[2].elapsed_time(e[3]) for e in events)
    gemm_ms = sum(gemm_each) / args.steps
    gemm_med, gemm_min = gemm_each[len(gemm_each) // 2], gemm_each[0]
    ms_per_step = elapsed * 1e3 / args.steps
    flops = w.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    quant_bytes_a = w.M * w.K * 4 + w.M * kq + (w.M * w.K // 32 if w.mode == "mx32" else 4 * w.M)
    quant_bytes_b = rows_b * w.K * 4 + rows_b * kq + (rows_b * w.K // 32 if w.mode == "mx32"
                                                      else 4 * rows_b)
    if w.mode == "tensor":  # the amax pass reads the input once more
        quant_bytes_a += w.M * w.K * 4
        quant_bytes_b += rows_b * w.K * 4

    # HBM-bound shapes (arithmetic intensity below the MFMA/HBM ridge): the roofline
    # is bytes over time; a cold-cache rate is measured as well, cycling the GEMM
    # over enough distinct operand copies (>= 512 MiB) that none is cache resident
    gbytes = (gemm_bytes_mxout if mxout else gemm_bytes_qout if qout else gemm_bytes)(w, code_bytes)
    hbm_bound = flops / gbytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    cold = None
    if not w.groups and not mxout and not qout and not kn and rows_b * kq >= (4 << 20):
        # >= 512 MiB of distinct operands (at least three sets): no launch finds
        # its operands in the 256 MB Infinity Cache
        nsets = max(3, -(-(512 << 20) // (rows_b * kq + w.M * kq)))
        qbs = [qb.clone() for _ in range(nsets)]
        qas = [qa.clone() for _ in range(nsets)]
        for i in range(nsets):
            F.gemm(qas[i], sa, qbs[i], sb, w.mode, w.out, out=C, fmt_a=fmt_a, fmt_b=fmt_b,
                   bias=bias, activation=act)
        torch.cuda.synchronize()
        reps = 4 if hbm_bound else 2
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for i in range(nsets):
                F.gemm(qas[i], sa, qbs[i], sb, w.mode, w.out, out=C, fmt_a=fmt_a, fmt_b=fmt_b,
                       bias=bias, activation=act)
        e1.record()
        torch.cuda.synchronize()
        cold_ms = e0.elapsed_time(e1) / (reps * nsets)
        cold = {"ms": round(cold_ms, 5), "gbs_algorithmic": round(gbytes / (cold_ms * 1e-3) / 1e9, 1),
                "tflops": round(flops / (cold_ms * 1e-3) / 1e12, 1),
                "operand_sets": nsets, "launches": reps * nsets,
                "note": "back-to-back launches over distinct operand copies (HIP events on the "
                        "launch stream)"}
        del qbs, qas
        log(f"cold-cache GEMM: {cold}")
    if cold is not None and hbm_bound:
        # context: a plain device read of the same number of bytes from HBM,
        # rotated over distinct buffers, and of 1 GiB: torch row sums over 16 KiB
        # rows of int64 words (one workgroup per row, no cross-workgroup reduction)
        def read_rate(nbytes, sets, reps):
            rows = nbytes // 16384
            bufs = [torch.ones((rows, 2048), dtype=torch.int64, device=dev) for _ in range(sets)]
            for b in bufs:
                b.sum(dim=1)
            torch.cuda.synchronize()
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            r0.record()
            for _ in range(reps):
                for b in bufs:
                    b.sum(dim=1)
            r1.record()
            torch.cuda.synchronize()
            ms = r0.elapsed_time(r1) / (reps * sets)
            del bufs
            nb = rows * 16384
            return {"bytes": nb, "ms": round(ms, 5), "gbs": round(nb / (ms * 1e-3) / 1e9, 1)}
        gb = gbytes // 8 * 8
        cold["hbm_read_context"] = {
            "kernel": "torch row sums over 16 KiB rows of int64 words (a plain device read)",
            "same_bytes": read_rate(gb, max(2, -(-(512 << 20) // gb)), 4),
            "one_gib": read_rate(1 << 30, 2, 3)}
        log(f"plain read context: {cold['hbm_read_context']}")
    gemm_gbs = gbytes / (gemm_ms * 1e-3) / 1e9
    # the committed counter summaries are of the default e4m3 GEMM without epilogue
    default_variant = args.formats == "e4m3,e4m3" and args.epilogue == "none" and not kn
    traffic = measured_traffic(w.name) if default_variant else None
    if hbm_bound:
        # against HBM, the launches whose operands come from HBM (in the step the
        # GEMM reads the codes the quantiser has just written, likely still in the
        # Infinity Cache); the step timing stays in kernels.gemm
        gbs = cold["gbs_algorithmic"] if cold is not None else gemm_gbs
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic,
                    "timing": "cold-cache launches (kernels.gemm_cold_cache)" if cold is not None
                              else "the timed steps (kernels.gemm)"}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                    "traffic": traffic}

    result = {
        "metric": "FP8 GEMM TFLOPS (% of MI355X FP8 peak) at 4096^3/8192^3; GB/s at M=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1),
                   "note": "untimed steps before the warm-up, until the GPU has run the hot "
                           "path for --settle-ms (steady state)"},
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": fmt_a if fmt_a == fmt_b else f"{fmt_a}x{fmt_b}",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "scale": w.mode,
                   "out": w.out, "groups": w.groups, "formats": [fmt_a, fmt_b],
                   "epilogue": args.epilogue, "b_layout": args.b_layout,
                   "step": "quantize A + GEMM (row-major B resident, transposing copy inside "
                           "the GEMM call)" if kn else
                           "quantize A + quantize B + GEMM (zero the maxima, GEMM storing fp32 y "
                           "with atomic maxima, requantise)" if qout else
                           "quantize A + quantize B + GEMM"},
        "roofline": roofline,
        "kernels": {
            "gemm": {"ms": round(gemm_ms, 5), "ms_median": round(gemm_med, 5),
                     "ms_min": round(gemm_min, 5), "tflops": round(achieved, 1),
                     "gbs_algorithmic": round(gemm_gbs, 1)},
            "quantize_a": {"ms": round(qa_ms, 4),
                           "gbs": round(quant_bytes_a / (qa_ms * 1e-3) / 1e9, 1)},
            "quantize_b": None if kn else {"ms": round(qb_ms, 4),
                                           "gbs": round(quant_bytes_b / (qb_ms * 1e-3) / 1e9, 1)},
        },
    }
    if cold is not None:
        result["kernels"]["gemm_cold_cache"] = cold
    result["context"] = PAGES_CONTEXT
    if args.copy_calibration:
        del Ad, Bd
        copy_calibration(dev)
        Ad = Bd = None
    if not args.no_cpu_baseline:
        del Ad, Bd
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_rows, fmt_a if fmt_a == fmt_b else "e4m3")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
