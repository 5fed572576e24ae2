"""Benchmark of the batched OKLS preconditioner step on one MI355X.

One step = one okls_step over every matrix of the workload (factor updates,
10-step Newton-Schulz roots, whitening, momentum and the weight update).
Default workload: the 1.2B-class model's optimizer step, 24 layers of
{4x 2048x2048, 2x 5632x2048, 1x 2048x5632} (168 matrices, 1.23e9
parameters), fp32 gradients 0.02*(sqrt(0.9) rank-32 + sqrt(0.1) noise)
generated on the device, OKLS defaults, fp16 Newton-Schulz and factor GEMM
inputs with fp32 accumulation.  Gradients are generated once and kept
resident in HBM; the timed steps cycle through them.

Prints one JSON line: matrices/s, step latency, the dominant kernel's
roofline (gemm_nt_kernel: algorithmic FLOPs over the union of its launches'
intervals, measured with HIP events on the launch streams during the timed
steps; the average launch duration is reported beside it for comparison
with rocprofv3) and the CPU oracle's time on a bounded sample of the same
workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "preconditioned matrices/sec + step latency (ms); % fp16 MFMA peak on NS chain"
PEAK_FP16_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
PEAK_HBM_GBS = 8000.0


# the GEMM's traffic depends on its kernel and on the planner's launch shapes
KERNEL_SRCS = [os.path.join(ROOT, "kronecker_factored_second_amd", "csrc", f)
               for f in ("okls_kernels.hip", "okls_types.h", "okls_api.cpp")]
def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"gemm_nt_kernel_{workload}_fp16_hbm_traffic.txt")
COPY_PROBE_BYTES = 1 << 30


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed steps before the timed ones (default 5; soap mode: --precond-freq, so that the "
                        "first eigenbasis refresh, a cold start from the identity, is not timed)")
    p.add_argument("--workload", default="c3")
    p.add_argument("--precision", default="fp16", choices=["fp16", "fp32"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-seconds", type=float, default=90.0)
    p.add_argument("--device-grads", action="store_true",
                   help="gradients of the workload's recipe drawn on the GPU (the default for "
                        "workloads above 1e9 parameters, whose host recipes would take minutes per step)")
    p.add_argument("--mode", choices=["okls", "shampoo", "muon", "soap", "nystrom"], default=None,
                   help="optimizer mode (default: the workload's); muon runs the polar iteration of the momentum "
                        "on the same matrices, the pages' throughput comparison; soap runs Adam in the factors' "
                        "eigenbasis (bases refreshed every --precond-freq steps)")
    p.add_argument("--nys-rank", type=int, default=32, help="nystrom mode: eigenpairs kept per factor")
    p.add_argument("--nys-oversample", type=int, default=8, help="nystrom mode: extra sketch columns")
    p.add_argument("--nys-passes", type=int, default=1, help="nystrom mode: subspace-iteration passes")
    p.add_argument("--precond-freq", type=int, default=10,
                   help="soap mode: refresh the eigenbases after every this many steps (the Clean paper's Table 6: 10)")
    p.add_argument("--root-period", type=int, default=None,
                   help="recompute the roots every this many steps (default 1: every step); nystrom mode: "
                        "refresh the low-rank factors every this many steps (default 10, the Clean paper's T)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 10 times (HBM counter calibration)")
    p.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV_DIR", "WRITE_CSV_DIR", "COMMANDS"),
                   help="write the GEMM's HBM traffic summary of --workload from two rocprofv3 --pmc runs")
    p.add_argument("--summarize-sq", nargs=2, metavar=("SQ_CSV_DIR", "COMMANDS"),
                   help="write the GEMM's SQ counter table of --workload from a rocprofv3 --pmc run of SQ_COUNTERS")
    return p.parse_args()


def copy_probe():
    """A plain copy of COPY_PROBE_BYTES: FETCH_SIZE and WRITE_SIZE of this
    kernel calibrate the counters (each should read the copy's size)."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": 10}), flush=True)


def _counter_rows(d, counter, prefix):
    """{kernel name: [values]} of one counter from the rocprofv3 --pmc csv
    files <prefix>_counter_collection.csv under directory d."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", f"{prefix}_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_counters(fetch_dir, write_dir, commands, workload):
    """HBM bytes per gemm_nt_kernel launch from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch) of the benchmark run ('bench' files), each scaled by the
    factor that makes the counter of the plain 1 GiB copy ('copy' files, the
    runtime's copy kernel) read the copy's size."""

    def avg(d, counter, prefix, key):
        vals = [v for k, vs in _counter_rows(d, counter, prefix).items() if key(k) for v in vs]
        if not vals:
            raise SystemExit(f"no {counter} rows for {prefix} in {d}")
        return sum(vals) / len(vals), len(vals)

    is_copy = lambda k: k.startswith("__amd_rocclr_copyBuffer")
    is_gemm = lambda k: "gemm_nt_kernel" in k
    cf, ncf = avg(fetch_dir, "FETCH_SIZE", "copy", is_copy)
    cw, ncw = avg(write_dir, "WRITE_SIZE", "copy", is_copy)
    gf, ngf = avg(fetch_dir, "FETCH_SIZE", "bench", is_gemm)
    gw, ngw = avg(write_dir, "WRITE_SIZE", "bench", is_gemm)
    kf = COPY_PROBE_BYTES / (cf * 1024.0)
    kw = COPY_PROBE_BYTES / (cw * 1024.0)
    traffic = gf * 1024.0 * kf + gw * 1024.0 * kw
    others = []
    for kern in ("stats_kernel", "cast_kernel"):
        of, nof = avg(fetch_dir, "FETCH_SIZE", "bench", lambda k: kern in k)
        ow, _ = avg(write_dir, "WRITE_SIZE", "bench", lambda k: kern in k)
        others.append(f"{kern}_hbm_bytes_per_launch {of * 1024.0 * kf + ow * 1024.0 * kw:.6e} "
                      f"(fetch {of * 1024.0 * kf:.4e}, write {ow * 1024.0 * kw:.4e}, {nof} dispatches)")
    from kronecker_factored_second_amd import workloads as WL
    w = WL.workload(workload)
    lines = [
        "# HBM traffic of gemm_nt_kernel (both block tiles, every launch of a step),",
        f"# workload {w.name}: " + ", ".join(f"{b}x {m}x{n}" for m, n, b in w.groups) + ", fp16 path",
        f"# kernel_source_sha256_16 {kernel_source_hash()} (okls_kernels.hip, okls_types.h, okls_api.cpp)",
        "# commands (repository root as $REPO, output directory OUT; cd /tmp first):",
        *[f"#   {c.strip()}" for c in commands.split(";")],
        f"copy_probe_bytes {COPY_PROBE_BYTES}",
        f"copy_fetch_kib_avg {cf:.1f} over {ncf} dispatches -> fetch factor {kf:.4f}",
        f"copy_write_kib_avg {cw:.1f} over {ncw} dispatches -> write factor {kw:.4f}",
        f"gemm_fetch_kib_avg {gf:.1f} over {ngf} dispatches",
        f"gemm_write_kib_avg {gw:.1f} over {ngw} dispatches",
        f"gemm_hbm_bytes_per_launch {traffic:.6e}",
        *others,
    ]
    open(traffic_file(workload), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


EPI_NAMES = ["STORE32", "SYRK", "NS_T", "NS_Y1", "STORE16", "NS_FINAL", "UPDATE", "POLAR", "POLAR_UPDATE", "NS_T_RES"]
SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F16",
               "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CU_CYCLES"]


def sq_file(workload):
    return os.path.join(ROOT, "profiles", f"gemm_nt_kernel_{workload}_fp16_sq_counters.txt")


def summarize_sq(sq_dir, commands, workload):
    """Per-instantiation table of gemm_nt_kernel from one rocprofv3 --pmc pass
    of SQ_COUNTERS (with --kernel-trace, so every counter row carries its
    dispatch's start and end): duration, MFMA rate, the shader clock the
    launch ran at (GRBM_GUI_ACTIVE cycles over 8 XCDs per microsecond) and
    the matrix cores' busy share at that clock."""
    import csv
    import glob
    import re
    disp = {}
    for f in glob.glob(os.path.join(sq_dir, "**", "bench_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "gemm_nt_kernel" not in r["Kernel_Name"]:
                continue
            d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                         "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
    if not disp:
        raise SystemExit(f"no gemm_nt_kernel counter rows in {sq_dir}")
    groups = {}
    for d in disp.values():
        m = re.search(r"TileCfg<(\d+), \d+, \d+, \w+>, (\d+), (\w+)>", d["name"])
        groups.setdefault((int(m.group(1)), EPI_NAMES[int(m.group(2))], m.group(3) == "true"), []).append(d)
    lines = [
        f"# gemm_nt_kernel SQ counters per launch, workload {workload}, fp16 path",
        f"# kernel_source_sha256_16 {kernel_source_hash()} (okls_kernels.hip, okls_types.h, okls_api.cpp)",
        "# commands (repository root as $REPO, output directory OUT; cd /tmp first):",
        *[f"#   {c.strip()}" for c in commands.split(";")],
        "# Under counters the launches run one at a time (no overlap of two chains).",
        "# Columns (averages over the launches of one instantiation):",
        "#   gflop     = SQ_INSTS_VALU_MFMA_MOPS_F16 * 512 (the planner's algorithmic FLOPs of these launches)",
        "#   frac      = TFLOP/s / 2500 (dense fp16 peak at 2.4 GHz)",
        "#   clk_mhz   = GRBM_GUI_ACTIVE / 8 XCDs / us: the shader clock the launch ran at",
        "#   mfma@2.4  = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (us * 2400): matrix-core busy share at the peak clock",
        "#   mfma@clk  = the same share at clk_mhz",
        "#   wait_any  = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: share of wave time stalled in s_waitcnt",
        "#   lds_confl = SQ_LDS_BANK_CONFLICT / 256 CUs / (us * clk_mhz): bank-conflict cycles per CU cycle",
        "tile epilogue      lo launches        us    gflop  TFLOP/s  frac clk_mhz mfma@2.4 mfma@clk wait_any lds_confl",
    ]
    tot_fl = tot_us = 0.0
    for (tile, epi, wl), ds in sorted(groups.items()):
        n = len(ds)
        us = sum(d["us"] for d in ds) / n
        fl = sum(d["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512 for d in ds) / n
        clk = sum(d["GRBM_GUI_ACTIVE"] / 8 / d["us"] for d in ds) / n
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / n / 1024
        wait = sum(d["SQ_WAIT_INST_ANY"] for d in ds) / max(sum(d["SQ_WAVE_CYCLES"] for d in ds), 1)
        confl = sum(d["SQ_LDS_BANK_CONFLICT"] for d in ds) / n / 256 / (us * clk)
        tf = fl / us / 1e6
        tot_fl += fl * n
        tot_us += us * n
        lines.append(f"{tile:4d} {epi:>12s} {int(wl):3d} {n:8d} {us:9.1f} {fl / 1e9:8.1f} {tf:8.1f} {tf / PEAK_FP16_TFLOPS:5.3f} "
                     f"{clk:7.0f} {busy / (us * 2400):8.3f} {busy / (us * clk):8.3f} {wait:8.3f} {confl:9.4f}")
    lines.append(f"# all gemm_nt_kernel launches: {len(disp)}, {tot_fl / tot_us / 1e6:.1f} TFLOP/s "
                 f"({tot_fl / tot_us / 1e6 / PEAK_FP16_TFLOPS:.3f} of peak) over their summed durations")
    open(sq_file(workload), "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_traffic(workload):
    """HBM bytes per GEMM launch from the committed counter summary of this
    workload, or None when it is missing or was taken on another version of
    the kernels."""
    f = traffic_file(workload)
    if not os.path.exists(f):
        return None
    txt = open(f).read()
    if f"kernel_source_sha256_16 {kernel_source_hash()} " not in txt:
        return None
    for line in txt.splitlines():
        if line.startswith("gemm_hbm_bytes_per_launch"):
            return float(line.split()[1])
    return None


def progress(msg):
    """One line per finished phase on stderr (stdout carries only the JSON line)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def cpu_baseline_nys(w, budget_s, args):
    """The fp64 Nystrom oracle on the same bounded sample as cpu_baseline:
    per shape class one step that refreshes the factors and one that keeps
    them, averaged over one period and scaled to the workload's counts."""
    from oracle import nystrom_oracle as Y
    from kronecker_factored_second_amd import workloads as WL
    T = max(args.root_period, 1)
    hp = Y.NysHyper(rank=args.nys_rank, oversample=args.nys_oversample, passes=args.nys_passes, period=T)
    rng = np.random.default_rng(0)
    total_s, step_s, sampled, timed = 0.0, 0.0, [], {}
    for gi, (m, n, b) in enumerate(w.groups):
        key = (min(m, n), max(m, n))
        if key in timed:
            sampled.append(f"{m}x{n}: as {timed[key][0]}")
            step_s += timed[key][1] * b
            continue
        G = WL.gradient(w, gi, 0, 1).astype(np.float64)
        k = args.nys_rank + args.nys_oversample
        psa, psb = rng.standard_normal((m, min(k, m))), rng.standard_normal((n, min(k, n)))
        t0 = time.perf_counter()
        r = Y.nys_step(Y.init_state(np.zeros((m, n))), G, hp, 1, psa, psb)
        dt_ref = time.perf_counter() - t0
        t0 = time.perf_counter()
        Y.nys_step(r.state, G, hp, 2 if T > 1 else 1, psa, psb)
        dt_keep = time.perf_counter() - t0 if T > 1 else dt_ref
        total_s += dt_ref + dt_keep
        dt = (dt_ref + (T - 1) * dt_keep) / T
        sampled.append(f"{m}x{n}:{dt:.3f}s")
        timed[key] = (f"{m}x{n}", dt)
        step_s += dt * b
        if total_s > budget_s:
            return None
    return {"value": w.n_matrices / step_s, "unit": "matrices/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": f"per shape class one fp64 oracle step refreshing the factors and one keeping them, averaged "
                      f"over {T} steps ({', '.join(sampled)}), scaled to the {w.n_matrices}-matrix workload: "
                      f"{step_s:.3f} s/step"}


def cpu_baseline_soap(w, budget_s, freq):
    """The fp64 eigenbasis-Adam oracle on the same bounded sample as
    cpu_baseline: per shape class one step that keeps the bases and one that
    refreshes them (eigh of both factors), averaged over one period of freq
    steps and scaled to the workload's matrix counts."""
    from oracle import soap_oracle as S
    from kronecker_factored_second_amd import workloads as WL
    hp = S.SoapHyper(freq=freq)
    total_s, step_s, sampled, timed = 0.0, 0.0, [], {}
    for gi, (m, n, b) in enumerate(w.groups):
        key = (min(m, n), max(m, n))
        if key in timed:
            sampled.append(f"{m}x{n}: as {timed[key][0]}")
            step_s += timed[key][1] * b
            continue
        G = WL.gradient(w, gi, 0, 1).astype(np.float64)
        st = S.init_state(np.zeros((m, n)))
        t0 = time.perf_counter()
        S.soap_step(st, G, hp, 1)
        dt_keep = time.perf_counter() - t0
        t0 = time.perf_counter()
        S.soap_step(st, G, hp, freq)
        dt_ref = time.perf_counter() - t0
        total_s += dt_keep + dt_ref
        dt = (dt_ref + (freq - 1) * dt_keep) / freq
        sampled.append(f"{m}x{n}:{dt:.2f}s")
        timed[key] = (f"{m}x{n}", dt)
        step_s += dt * b
        if total_s > budget_s:
            return None
    return {"value": w.n_matrices / step_s, "unit": "matrices/s", "cores": os.cpu_count(), "kind": "oracle",
            "sample": f"per shape class one fp64 oracle step keeping the bases and one refreshing them, averaged "
                      f"over {freq} steps ({', '.join(sampled)}), scaled to the {w.n_matrices}-matrix workload: "
                      f"{step_s:.2f} s/step"}


def cpu_baseline(w, budget_s, root_period=1, mode=None):
    """The fp64 oracle, as it stands, on a bounded sample: one matrix of each
    distinct shape class of the workload, a full oracle step each (exact eigh
    roots plus the fp64 Newton-Schulz iteration), scaled to the whole
    workload's matrix counts.  An m x n class and its n x m transpose run the
    same products and eigendecompositions (the same two factor sides), so the
    second takes the first one's time.  With a root period p > 1 the step
    that keeps the roots is timed too and the two are averaged over one
    period."""
    from oracle import okls_oracle as O
    from kronecker_factored_second_amd import workloads as WL
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                         for i in info if i.get("user_api") == "blas") or blas
    except Exception:
        threads = os.cpu_count()
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    mode = mode or w.mode
    hp = O.muon_hyper() if mode == "muon" else O.Hyper(root_period=root_period)
    total_s, sampled, step_s = 0.0, [], 0.0
    timed = {}
    for gi, (m, n, b) in enumerate(w.groups):
        key = (min(m, n), max(m, n))
        if key in timed:
            sampled.append(f"{m}x{n}: as {timed[key][0]}")
            step_s += timed[key][1] * b
            continue
        G = WL.gradient(w, gi, 0, 1).astype(np.float64)
        st = O.init_state(np.zeros((m, n)), hp.eps)
        t0 = time.perf_counter()
        r = O.step(st, G, hp, 1, mode)
        dt = time.perf_counter() - t0
        total_s += dt
        if root_period > 1:
            t0 = time.perf_counter()
            O.step(r.state, G, hp, 2, mode)
            dt2 = time.perf_counter() - t0
            total_s += dt2
            dt = (dt + (root_period - 1) * dt2) / root_period
        sampled.append(f"{m}x{n}:{dt:.2f}s")
        timed[key] = (f"{m}x{n}", dt)
        step_s += dt * b
        if total_s > budget_s:
            step_s = None
            break
    if step_s is None:
        return None
    return {"value": w.n_matrices / step_s, "unit": "matrices/s", "cores": threads, "kind": "oracle",
            "host_cpu": cpu, "host_cpus_visible": os.cpu_count(), "blas": blas,
            "sample": f"one full fp64 oracle step per shape class ({', '.join(sampled)}), "
                      f"scaled by the class counts to the {w.n_matrices}-matrix workload: {step_s:.1f} s/step"}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload)
        return
    if args.summarize_sq:
        summarize_sq(*args.summarize_sq, args.workload)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the preconditioner step runs on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    import torch
    from kronecker_factored_second_amd import okls, workloads as WL

    w = WL.workload(args.workload)
    mode = args.mode or w.mode
    if args.root_period is None:
        args.root_period = 10 if mode == "nystrom" else 1
    if args.warmup is None:
        args.warmup = args.precond_freq if mode == "soap" else 5
    dev = torch.device("cuda:0")
    bf16 = w.grad_dtype == "bf16"
    big = w.n_params > 1e9
    device_grads = args.device_grads or big
    params = [torch.zeros(b, m, n, device=dev) for (m, n, b) in w.groups]
    for gi, (m, n, b) in enumerate(w.groups):
        std = 0.07539 * (m / n) ** 0.5 / (n ** 0.5 + m ** 0.5)
        if big:
            params[gi].copy_(WL.device_filler(std, (b, m, n), seed=1000 + gi))
        else:
            for i in range(b):
                params[gi][i].copy_(torch.from_numpy(WL.initial_weights(w, gi, i)))
    n_bufs = 1 if big else 3
    scale = {"gauss1": 1.0, "rowscaled": 0.02, "lowrank": 0.02, "gauss1e-3": 1e-3, "illcond": 0.07}[w.grad]
    grads = []
    for t in range(1, n_bufs + 1):
        gs = []
        for gi, (m, n, b) in enumerate(w.groups):
            if device_grads and w.grad == "lowrank":      # the recipe itself, on the device
                g = WL.device_lowrank((b, m, n), seed_fixed=(1 << 16) + gi, seed_t=(t << 8) + gi, scale=scale)
            elif device_grads:
                g = WL.device_filler(scale, (b, m, n), seed=(t << 8) + gi)
            else:
                g = torch.from_numpy(np.stack([WL.gradient(w, gi, i, t) for i in range(b)])).to(dev)
            gs.append(g.to(torch.bfloat16) if bf16 else g)
        grads.append(gs)
    progress(f"{w.name}: inputs ready ({len(grads)} gradient set(s))")
    limit = None
    if big:   # leave room for the caller's tensors: the workspace takes what the card has left
        limit = torch.cuda.mem_get_info(0)[0] - sum(b * (m * n + 2 * m * m + 2 * n * n) * 4 for m, n, b in w.groups) \
            - (8 << 30)
    extra = dict(precond_freq=args.precond_freq) if mode == "soap" else dict(root_period=args.root_period)
    if mode == "nystrom":
        extra.update(nys_rank=args.nys_rank, nys_oversample=args.nys_oversample, nys_passes=args.nys_passes)
    opt = okls.OKLS(params, mode=mode, precision=args.precision,
                    grad_dtype=torch.bfloat16 if bf16 else torch.float32, workspace_limit=limit, **extra)
    progress(f"{w.name}: optimizer ready (workspace {opt.workspace.numel() / 2**30:.1f} GiB)")
    for i in range(args.warmup):
        opt.step(grads=grads[i % n_bufs])
    torch.cuda.synchronize()
    progress(f"{w.name}: {args.warmup} warm-up step(s) done")

    # the timed steps run as a user runs them: the library's per-launch
    # profiling events are off
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        opt.step(grads=grads[i % n_bufs])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    progress(f"{w.name}: {args.steps} timed step(s), {ms_step:.2f} ms/step")
    # per-step latencies (an event on the caller's stream after every step):
    # their median and maximum, beside the mean of the timed block above
    lat_steps = min(args.steps, 3) if big else args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(lat_steps + 1)]
    evs[0].record()
    for i in range(lat_steps):
        opt.step(grads=grads[(args.steps + i) % n_bufs])
        evs[i + 1].record()
    torch.cuda.synchronize()
    lat = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(lat_steps))
    lat_median = float(np.median(lat))
    progress(f"{w.name}: per-step latency pass done")
    # then the same steps again with a HIP event pair around every launch:
    # per-category busy times, the GEMM roofline and the HBM kernels' rates
    prof_steps = min(args.steps, 3) if big else args.steps
    okls.profile_enable(opt.handle, True)
    okls.profile_read(opt.handle)       # clear
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    for i in range(prof_steps):
        opt.step(grads=grads[(args.steps + lat_steps + i) % n_bufs])
    p1.record()
    torch.cuda.synchronize()
    prof = okls.profile_read(opt.handle)
    progress(f"{w.name}: instrumented pass done")
    okls.profile_enable(opt.handle, False)
    ms_step_profiled = p0.elapsed_time(p1) / prof_steps
    finite = opt.check_finite()

    g_ms = sum(prof[k]["ms"] for k in ("ns_gemm", "factor_gemm", "whiten_gemm"))
    # the three GEMM categories run in different phases of the step, so their
    # busy times add; within the Newton-Schulz phase two chains overlap
    g_busy = sum(prof[k]["busy_ms"] for k in ("ns_gemm", "factor_gemm", "whiten_gemm"))
    g_fl = sum(prof[k]["flops"] for k in ("ns_gemm", "factor_gemm", "whiten_gemm"))
    g_n = sum(prof[k]["launches"] for k in ("ns_gemm", "factor_gemm", "whiten_gemm"))
    g_b = sum(prof[k]["bytes"] for k in ("ns_gemm", "factor_gemm", "whiten_gemm"))
    achieved = g_fl / (g_busy * 1e-3) / 1e12 if g_busy > 0 else 0.0
    per_launch = g_fl / (g_ms * 1e-3) / 1e12 if g_ms > 0 else 0.0
    ns = prof["ns_gemm"]
    ns_tflops = ns["flops"] / (ns["busy_ms"] * 1e-3) / 1e12 if ns["busy_ms"] > 0 else 0.0
    nys_roofline = None
    if mode == "nystrom":
        # every step's preconditioning (thin_kernel launches: the momentum
        # with X = N U_b, U_a^T N, the weight update) streams the m x n data
        # three times: bound by HBM
        wb = prof["whiten_gemm"]
        ach = wb["bytes"] / (wb["busy_ms"] * 1e-3) / 1e9 if wb["busy_ms"] > 0 else 0.0
        nys_roofline = {"kernel": "thin_kernel (per-step preconditioning)", "bound": "hbm",
                        "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                        "traffic": None,
                        "method": "algorithmic bytes of the per-step preconditioning launches (the momentum read and "
                                  "written once, N read twice more, W read and written) over their busy time from HIP "
                                  "events on the launch stream, in a second pass of the same steps",
                        "avg_launch_us": wb["ms"] * 1e3 / max(wb["launches"], 1),
                        "launches_per_step": wb["launches"] / max(prof["steps"], 1),
                        "algorithmic_bytes_per_step": wb["bytes"] / max(prof["steps"], 1),
                        "algorithmic_flops_per_step": wb["flops"] / max(prof["steps"], 1)}
    line = {
        "metric": METRIC,
        "value": w.n_matrices / (ms_step * 1e-3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if args.precision == "fp16" else "fp16x3-split",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: " + ", ".join(f"{b}x {m}x{n}" for m, n, b in w.groups) +
                   f" ({w.n_matrices} matrices, {w.n_params / 1e6:.1f}M params), {mode}, "
                   f"{w.grad_dtype} gradients" + ((" (low-rank recipe drawn on the device)" if w.grad == "lowrank" else
                                                   " (device Gaussian)") if device_grads else "") +
                   f", precision {args.precision}" +
                   (f", chunks of {opt.cfg.chunk_matrices} matrices" if opt.cfg.chunk_matrices else "") +
                   (f", roots every {args.root_period} steps" if args.root_period > 1 and mode not in ("soap", "nystrom") else "") +
                   (f", Nystrom rank {args.nys_rank} + {args.nys_oversample}, {args.nys_passes} pass(es), factors "
                    f"refreshed every {args.root_period} steps" if mode == "nystrom" else "") +
                   (f", eigenbases refreshed every {args.precond_freq} steps" if mode == "soap" else ""),
                   "matrices": w.n_matrices, "parallelism": "single GPU"},
        "step_latency_ms": ms_step,
        "step_latency_ms_median": lat_median,
        "step_latency_ms_max": lat[-1],
        "ms_per_step_with_launch_events": ms_step_profiled,
        "ns_chain": {"tflops": ns_tflops, "frac_fp16_peak": ns_tflops / PEAK_FP16_TFLOPS,
                     "ms_per_step": ns["busy_ms"] / max(prof["steps"], 1), "launches_per_step": ns["launches"] / max(prof["steps"], 1)},
        "roofline": nys_roofline if mode == "nystrom" else {"kernel": "gemm_nt_kernel",
                     "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_FP16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP16_TFLOPS,
                     "traffic": measured_traffic(args.workload) if (args.precision == "fp16" and mode == w.mode and
                                                                    args.root_period == 1 and mode != "nystrom") else None,
                     "method": "algorithmic FLOPs of every gemm_nt_kernel launch over the union of their intervals, "
                               "from HIP events on the launch streams in a second pass of the same steps (the timed "
                               "pass runs without them); where the plan runs two Newton-Schulz chains their launches overlap",
                     "avg_launch_us": g_ms * 1e3 / max(g_n, 1), "achieved_per_launch_duration": per_launch,
                     "launches_per_step": g_n / max(prof["steps"], 1),
                     "algorithmic_flops_per_step": g_fl / max(prof["steps"], 1),
                     "algorithmic_bytes_per_launch": g_b / max(g_n, 1)},
        "profile_ms_per_step": {k: prof[k]["busy_ms"] / max(prof["steps"], 1) for k in okls.PROFILE_CATEGORIES},
        "hbm_kernels": {kern: {"bound": "hbm", "achieved": prof[cat]["bytes"] / (prof[cat]["busy_ms"] * 1e-3) / 1e9,
                               "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": prof[cat]["bytes"] / (prof[cat]["busy_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                               "bytes_per_step": prof[cat]["bytes"] / max(prof["steps"], 1),
                               "launches_per_step": prof[cat]["launches"] / max(prof["steps"], 1)}
                        for kern, cat in (("stats_kernel", "stats"), ("cast_kernel", "cast")) if prof[cat]["busy_ms"] > 0},
        "state_finite": finite,
        "host_wall_s": wall,
    }
    if mode in ("okls", "shampoo") and prof["stats"]["busy_ms"] + prof["cast"]["busy_ms"] > 0:
        # the statistics and cast launches against the method's own bytes, not
        # the staging copies the GEMMs read: the momentum reads G and M and
        # writes M and the fp16 N (bytes_G + 10 per element), and the root's
        # start reads each factor and writes its fp16 Y_0 (6 per entry)
        gb = 2 if bf16 else 4
        mb = sum(b * (m * n * (gb + 10) + 6 * (m * m + n * n)) for m, n, b in w.groups)
        sc_ms = (prof["stats"]["busy_ms"] + prof["cast"]["busy_ms"]) / max(prof["steps"], 1)
        line["hbm_kernels_method_bytes"] = {"kernels": "stats_kernel + cast_kernel", "bytes_per_step": mb,
                                            "ms_per_step": sc_ms, "achieved": mb / (sc_ms * 1e-3) / 1e9,
                                            "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                            "frac": mb / (sc_ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if mode in ("okls", "shampoo"):
        # convergence of the roots: ||Z_{K-1} Y_{K-1} - I||_F of every chain of the last step
        r = np.array([x for g in opt.ns_residuals() for mat in g for side in mat for x in side], dtype=np.float64)
        r = r[np.isfinite(r)]
        if r.size:
            line["ns_residual"] = {"chains": int(r.size), "median": float(np.median(r)), "max": float(r.max())}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline_soap(w, args.cpu_sample_seconds, args.precond_freq) if mode == "soap"
                                else cpu_baseline_nys(w, args.cpu_sample_seconds, args) if mode == "nystrom"
                                else cpu_baseline(w, args.cpu_sample_seconds, args.root_period, mode))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
