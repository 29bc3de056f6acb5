"""Benchmark of the LaplacianFormer attention forward pass on one MI355X.

A step is one lf_attn_fwd call over one batch of synthetic input that is already resident in HBM. The call is
landmark pooling -> fused L1-distance+exp kernel for C_K and W_eps -> Newton-Schulz pseudo-inverse, with
S = C_K^T V and the C_Q distance pass in the same launch -> output GEMM (landmark mix P = X S inside it) with the
depthwise-conv epilogue. The default workload is the PVT stage-1 shape: B=8, one head,
56x56 tokens, d=64, r=8 (m=49), lambda=4, eps=1e-3, 12 Newton-Schulz steps, fp32.

It prints one JSON line with the whole-job throughput (tokens/s = B*heads*N per step). It also prints the roofline
of the dominant kernel (laplace_l1_exp: VALU-bound, timed with HIP events on its own stream) and the fp64 CPU
oracle timed on a bounded sample of the same workload on the host cores.

--workload picks another shape; for the training shape (whitening on) a step is lf_attn_fwd with the saved buffer
followed by lf_attn_bwd_ex (dQ, dK, dV and the DWC weight and lambda gradients). Besides the hot figure (one
buffer set, as the contract's value) it reports a "cold" one:
the same steps rotating over enough input/output/workspace sets (>= 512 MB in all) that no step finds its data in
the 256 MB last-level cache (--no-cold skips it).

--solver measures the solver comparison of the pages instead (Newton-Schulz against conjugate gradients for
W_eps X = I, at the workload's landmark matrices and at synthetic kappa = 50 SPD matrices of the same batch): one JSON
line with, per solver and step count, the residual ||W_eps X - I||_F (mean and max over the batch), the matrix
products spent and the time per launch (HIP events), and the CG kernel's MFMA roofline.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Laplacian-Nyström attention fwd tokens/s (B·heads·N) + % VALU/MFMA roofline"
METRIC_TRAIN = "Laplacian-Nyström attention fwd+bwd tokens/s (B·heads·N) + % VALU/MFMA roofline"
METRIC_GAUSS = "Gaussian-kernel Nyström attention fwd tokens/s (B·heads·N) + % MFMA roofline"
COLD_BYTES = 512 << 20

# HBM traffic of the distance kernel, from two rocprofv3 counter passes over `bench.py --counters` (FETCH_SIZE,
# then WRITE_SIZE), each scaled by what the same counter reads for a device copy of known size. The file records a
# hash of the kernel's source; when the source has changed since, the bench reports the traffic as unknown.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "laplace_l1_exp_pvt_s1_56x56_m49_traffic.json")
CALIB_COPY_MIB = 256
COUNTER_LAUNCHES = 10

# MI355X: the published fp32 vector peak is 157.3 TFLOP/s, an FMA counted as two flops: 256 CUs x 4 SIMDs x 32
# lanes per clock at 2.4 GHz, i.e. 78.6e12 fp32 lane-operations per second, which a stream of independent
# v_add_f32 with register operands reaches to 80 % (63 T measured). The distance kernel's v_sub_f32 and
# v_add_f32 |.| are one operation each.
VALU_PEAK_TFLOPS = 256 * 4 * 32 * 2.4e9 / 1e12
# MI355X published dense fp32 MFMA peak.
MFMA_F32_PEAK_TFLOPS = 157.3


def laplace_source_hash():
    """Hash of the distance kernel (its block, kernel wrapper and launcher) as it stands in the source tree (None if
    not found)."""
    import hashlib

    csrc = os.path.join(ROOT, "laplacian_nystr_vit_amd", "csrc")
    try:
        blk = open(os.path.join(csrc, "lf_laplace.h")).read()
        src = open(os.path.join(csrc, "lf_fwd.hip")).read()
        z = blk.index("template <int D>\nconstexpr int kLaplaceLds")
        a = src.index("__global__ __launch_bounds__(512) void k_laplace(")
        b = src.index("\n}\n", a)
        c = src.index("struct LaplacePlan {")
        e = src.index("static void laplace_d(", c)
    except (OSError, ValueError):
        return None
    return hashlib.sha256((blk[z:] + src[a:b] + src[c:e]).encode()).hexdigest()[:16]


def load_traffic():
    """Bytes per launch of the distance kernel from the committed counter summary, if it matches the source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != laplace_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def read_counter_csv(d, counter):
    """Per-dispatch (kernel name, value) pairs of one counter from a rocprofv3 --pmc csv output directory."""
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for row in csv.DictReader(open(files[0])):
        if row.get("Counter_Name") != counter:
            continue
        key = row["Dispatch_Id"]
        name, val = per.get(key, (row["Kernel_Name"], 0.0))
        per[key] = (name, val + float(row["Counter_Value"]))
    return list(per.values())


def ingest_counters(fetch_dir, write_dir):
    """Writes the traffic summary (JSON + markdown) from a FETCH_SIZE pass and a WRITE_SIZE pass."""
    out = {"workload": "pvt_s1_56x56_m49", "kernel": "lf::k_laplace<float, 64>", "source_hash": laplace_source_hash(),
           "calib_copy_bytes": CALIB_COPY_MIB * 2**20}
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = read_counter_csv(d, counter)
        lap = [v for n, v in rows if "k_laplace" in n]
        cal = [v for n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        if not lap or not cal:
            raise SystemExit(f"{counter}: laplace dispatches {len(lap)}, copy dispatches {len(cal)}")
        raw = sum(lap) / len(lap) * 1024.0            # bytes per launch as the counter reads them
        cal_raw = max(cal) * 1024.0                   # the big copy is the largest copy dispatch
        factor = out["calib_copy_bytes"] / cal_raw    # counter bytes -> true bytes, from the copy of known size
        out[f"{label}_launches"] = len(lap)
        out[f"{label}_raw_bytes_per_launch"] = raw
        out[f"{label}_calib_raw_bytes"] = cal_raw
        out[f"{label}_factor"] = factor
        out[f"{label}_bytes_per_launch"] = raw * factor
    out["traffic_bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out))


def counters_workload():
    """The distance kernel COUNTER_LAUNCHES times on the stage-1 shape, then one device copy of known size."""
    import numpy as np
    import torch

    from laplacian_nystr_vit_amd import lf
    from laplacian_nystr_vit_amd import workloads as WL

    wl = WL.ALL["pvt_s1_56x56_m49"]
    inp = WL.make_inputs(wl, seed=0)
    Q, K = torch.from_numpy(inp["Q_raw"]).cuda(), torch.from_numpy(inp["K_raw"]).cuda()
    p = lf.make_params(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.r, wl.lam, wl.eps, wl.ns_iters, wl.whiten, wl.whiten_eps,
                       torch.float32)
    G, N, m, d = p.G, p.N, p.m, p.d
    L = torch.empty(G * m * d, device="cuda")
    CQ = torch.empty(G * N * m, device="cuda")
    CK = torch.empty_like(CQ)
    We = torch.empty(G * m * m, device="cuda")
    lf.lf_landmark_pool(p, Q, L)
    for _ in range(COUNTER_LAUNCHES):
        lf.lf_laplace_l1_exp(p, Q, K, L, CQ, CK, We)
    n = CALIB_COPY_MIB * 2**20 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"counters workload done: {COUNTER_LAUNCHES} distance launches, copy of {CALIB_COPY_MIB} MiB", flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 2000 untimed steps (about 0.1 s at the stage-1 shape): after 20 the same 200 timed steps still measured about
    # 1 us per step slower (44.2 against 43.05 us) while the clocks settle
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", default="pvt_s1_56x56_m49")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall time budget of the oracle sample")
    ap.add_argument("--kernel-reps", type=int, default=100)
    ap.add_argument("--no-cold", action="store_true", help="skip the timing over rotating buffer sets")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the 1.5 s shader-clock observation (for profiler and counter runs)")
    ap.add_argument("--solver", action="store_true",
                    help="measure Newton-Schulz against conjugate gradients on the workload's W_eps batch")
    ap.add_argument("--counters", action="store_true",
                    help="run only the distance kernel and a calibration copy (for rocprofv3 --pmc passes)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from the two rocprofv3 --pmc output directories")
    return ap.parse_args()


# ---------------------------------------------------------------------------------------------- CPU baseline
_ORACLE_STATE = {}


def _oracle_init(wl):
    """Worker set-up: the workload's inputs, once per worker process, and BLAS limited to one thread."""
    from threadpoolctl import threadpool_limits

    from laplacian_nystr_vit_amd import workloads as WL

    _ORACLE_STATE["wl"] = wl
    _ORACLE_STATE["inp"] = WL.make_inputs(wl, seed=0, with_dy=bool(wl.whiten))
    _ORACLE_STATE["limits"] = threadpool_limits(limits=1)


def _oracle_run(args):
    """One worker's share of a timed run: whole (batch, head) slices from `first` on, until `budget_s` has passed
    (at least one). Returns (slices, seconds)."""
    import oracle as O

    first, budget_s = args
    wl, inp = _ORACLE_STATE["wl"], _ORACLE_STATE["inp"]
    op = O.Params(B=wl.B, heads=wl.heads, H=wl.H, W=wl.W, d=wl.d, r=wl.r, lam=wl.lam, eps=wl.eps,
                  ns_iters=wl.ns_iters, whiten=wl.whiten, whiten_eps=wl.whiten_eps, kernel=wl.kernel)
    slices = 0
    t0 = time.perf_counter()
    while True:
        b, h = divmod((first + slices) % wl.G, wl.heads)
        args = (inp["Q"][b, h], inp["K"][b, h], inp["V"][b, h], inp["w64"][h * wl.d:(h + 1) * wl.d])
        fwd = O.forward_slice(*args, op)
        if wl.whiten:
            O.backward_slice(*args, inp["dY"][b, h], op, fwd)
        slices += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return slices, time.perf_counter() - t0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_workers():
    """Host cores the oracle may use: the process's CPU affinity, capped by the thread budget the environment sets
    (OMP_NUM_THREADS) and at 16, the host share of one GPU."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, min(n, 16))


def cpu_baseline(wl, budget_s):
    """The fp64 oracle as it stands, one single-threaded process per host core (spawned, so no child inherits GPU
    state), over whole slices of the same workload. Three timed runs of budget_s / 3 each; the median is reported."""
    import multiprocessing as mp

    workers = oracle_workers()
    ctx = mp.get_context("spawn")
    runs = []
    with ctx.Pool(workers, initializer=_oracle_init, initargs=(wl,)) as pool:
        pool.map(_oracle_run, [(k, 0.0) for k in range(workers)])  # start-up and first-touch outside the timing
        for _ in range(3):
            res = pool.map(_oracle_run, [(k * 7, budget_s / 3) for k in range(workers)])
            slices = sum(r[0] for r in res)
            secs = max(r[1] for r in res)
            runs.append((slices * wl.N / secs, slices, secs))
    runs.sort()
    value, slices, secs = runs[1]
    what = "forward + backward" if wl.whiten else "forward"
    return {"value": value, "unit": "tokens/s", "cores": workers, "kind": "oracle", "cpu_model": cpu_model(),
            "runs_tokens_per_s": [r[0] for r in runs],
            "sample": f"{what} of whole (batch, head) slices of {wl.name} ({wl.N} tokens each), fp64 numpy, "
                      f"{workers} single-threaded processes; median of 3 runs of {budget_s / 3:.1f} s "
                      f"(median run: {slices} slices in {secs:.2f} s)"}


def observed_sclk_mhz(run_for_s, work):
    """Highest shader clock rocm-smi reports while `work` runs for about run_for_s seconds (None if unavailable)."""
    import re
    import subprocess
    import threading

    samples = []
    done = threading.Event()

    def poll():
        while not done.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            for line in out.splitlines():
                if "sclk" in line.lower():
                    m = re.search(r"\((\d+)\s*Mhz\)", line, flags=re.I)
                    if m:
                        samples.append(int(m.group(1)))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < run_for_s:
        work()
    done.set()
    th.join(timeout=15)
    return max(samples) if samples else None


def distance_stage(wl, lf):
    """The stage entry point that forms C_Q, C_K and W_eps for the workload's kernel."""
    return lf.lf_gauss_l2_exp if wl.kernel == "gauss" else lf.lf_laplace_l1_exp


def solver_compare(args):
    import numpy as np
    import torch

    from laplacian_nystr_vit_amd import lf
    from laplacian_nystr_vit_amd import workloads as WL

    wl = WL.ALL[args.workload]
    if wl.m > 64:
        sys.exit(f"bench.py --solver: the CG kernel covers m <= 64 landmarks; {wl.name} has m = {wl.m}")
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    inp = WL.make_inputs(wl, seed=0)
    dt = torch.bfloat16 if wl.dtype == WL.BF16 else torch.float32
    p0 = lf.make_params(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.r, wl.lam, wl.eps, wl.ns_iters, False, 1e-5, dt,
                        wl.kernel)
    G, N, m, d = p0.G, p0.N, p0.m, p0.d

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    # the workload's landmark matrices, by the library's pooling and distance stages
    Q, K = dev(inp["Q_raw"]), dev(inp["K_raw"])
    L = torch.empty(G * m * d, device="cuda")
    CQ = torch.empty(G * N * m, device="cuda")
    CK = torch.empty_like(CQ)
    We = torch.empty(G * m * m, device="cuda")
    lf.lf_landmark_pool(p0, Q, L, stream)
    distance_stage(wl, lf)(p0, Q, K, L, CQ, CK, We, stream)
    torch.cuda.synchronize()
    del CQ, CK
    batches = {"landmark_W_eps": We.cpu().numpy().astype(np.float64).reshape(G, m, m),
               "spd_kappa50": np.stack([WL.spd_matrix(m, 50.0, 1000 + g) for g in range(G)])}

    def event_us(fn, reps):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    out = {"metric": "W_eps solver comparison: Newton-Schulz vs conjugate gradients (residual, products, us)",
           "unit": "us per launch", "n_gpus": 1, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{wl.name} W_eps batch", "G": G, "m": m}, "batches": {}}
    X = torch.empty(G * m * m, device="cuda")
    for name, W64 in batches.items():
        Wd = torch.from_numpy(np.ascontiguousarray(W64.astype(np.float32))).cuda()
        ev = np.linalg.eigvalsh(W64)
        rows = {"kappa_mean": float(np.mean(ev[:, -1] / ev[:, 0])), "ns": [], "cg": []}
        for K in (8, 12, 16, 20, 24):
            p = lf.make_params(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.r, wl.lam, wl.eps, K, False, 1e-5, dt, wl.kernel)
            fwd_b, _, _ = lf.lf_attn_query(p)
            ws = torch.empty(max(fwd_b, 1), dtype=torch.uint8, device="cuda")
            res = torch.empty(G, device="cuda")
            lf.lf_ns_pinv(p, Wd, X, None, None, res, ws, stream)
            torch.cuda.synchronize()
            r = res.cpu().numpy()
            us = event_us(lambda: lf.lf_ns_pinv(p, Wd, X, None, None, None, ws, stream), args.kernel_reps)
            rows["ns"].append({"steps": K, "products": 2 * K, "resid_mean": float(r.mean()),
                               "resid_max": float(r.max()), "us": round(us, 2)})
        p = p0
        for k in (12, 24, 36, 49, 64, 98):
            res = torch.empty(G * k, device="cuda")
            lf.lf_cg_pinv(p, Wd, X, res, k, stream)
            torch.cuda.synchronize()
            r = res.view(G, k)[:, -1].cpu().numpy()
            us = event_us(lambda: lf.lf_cg_pinv(p, Wd, X, None, k, stream), args.kernel_reps)
            rows["cg"].append({"steps": k, "products": k, "resid_mean": float(r.mean()), "resid_max": float(r.max()),
                               "us": round(us, 2)})
        out["batches"][name] = rows
    # CG kernel roofline: one W*P product (2 m^3 flops per slice) per step, at the longest run.
    last = out["batches"]["spd_kappa50"]["cg"][-1]
    flops = 2.0 * G * m ** 3 * last["steps"]
    achieved = flops / (last["us"] * 1e-6) / 1e12
    out["roofline"] = {"kernel": "cg_pinv", "bound": "mfma", "achieved": achieved, "peak": MFMA_F32_PEAK_TFLOPS,
                       "unit": "TFLOP/s", "frac": achieved / MFMA_F32_PEAK_TFLOPS, "traffic": None,
                       "avg_us": last["us"], "flops_per_launch": flops}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the B*heads slices are "
              "independent, so a multi-GPU run would shard them with no communication.", file=sys.stderr)
        sys.exit(2)

    if args.counters:
        counters_workload()
        return
    if args.solver:
        solver_compare(args)
        return

    import numpy as np
    import torch

    from laplacian_nystr_vit_amd import lf
    from laplacian_nystr_vit_amd import workloads as WL

    wl = WL.ALL[args.workload]
    torch.cuda.set_device(0)
    inp = WL.make_inputs(wl, seed=0)
    dt = torch.bfloat16 if wl.dtype == WL.BF16 else torch.float32

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    p = lf.make_params(wl.B, wl.heads, wl.H, wl.W, wl.d, wl.r, wl.lam, wl.eps, wl.ns_iters, wl.whiten, wl.whiten_eps,
                       dt, wl.kernel)
    train = bool(wl.whiten)
    fwd_b, saved_b, bwd_b = lf.lf_attn_query(p)
    stream = torch.cuda.current_stream()

    def make_set():
        """One set of every buffer a step touches: inputs, outputs, workspaces (and the saved buffer, dY and the
        gradients for a training step)."""
        t = {"Q": dev(inp["Q_raw"]), "K": dev(inp["K_raw"]), "V": dev(inp["V_raw"]), "w": dev(inp["w"])}
        t["Y"] = torch.empty_like(t["Q"])
        t["ws"] = torch.empty(max(fwd_b, bwd_b if train else 0), dtype=torch.uint8, device="cuda")
        if train:
            t["saved"] = torch.empty(saved_b, dtype=torch.uint8, device="cuda")
            t["dY"] = dev(inp["dY_raw"])
            for g in ("dQ", "dK", "dV"):
                t[g] = torch.empty_like(t["Q"])
            t["dw"] = torch.empty(wl.heads * wl.d * 9, device="cuda")
            t["dlam"] = torch.empty(1, device="cuda")
        return t

    # the training op lends the library a second stream for the backward's independent parts
    aux = lf.AuxStream() if train else None

    def run_step(t):
        if train:
            # the full training op: dQ, dK, dV and the DWC weight and lambda gradients
            lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], t["Y"], t["saved"], t["ws"], stream)
            lf.lf_attn_bwd_ex(p, t["Q"], t["K"], t["V"], t["w"], t["saved"], t["dY"], t["dQ"], t["dK"], t["dV"],
                              t["dw"], t["dlam"], 0, t["ws"], stream, aux=aux)
        else:
            lf.lf_attn_fwd(p, t["Q"], t["K"], t["V"], t["w"], t["Y"], None, t["ws"], stream)

    def timed(sets, steps, warmup):
        for i in range(warmup):
            run_step(sets[i % len(sets)])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run_step(sets[i % len(sets)])
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    hot = make_set()
    Q, K, V, w, Y, ws = hot["Q"], hot["K"], hot["V"], hot["w"], hot["Y"], hot["ws"]
    elapsed = timed([hot], args.steps, args.warmup)
    ms_per_step = elapsed / args.steps * 1e3
    tokens_per_s = wl.tokens * args.steps / elapsed

    # The same steps with a HIP event recorded on the stream between consecutive steps: the distribution of the
    # device time per step (its median is robust to a stray slow step, which the wall-clock mean is not).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        run_step(hot)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    step_events = {"median_ms": per[len(per) // 2], "p10_ms": per[len(per) // 10],
                   "p90_ms": per[min(len(per) - 1, (9 * len(per)) // 10)], "steps": len(per),
                   "median_tokens_per_s": wl.tokens / (per[len(per) // 2] * 1e-3)}
    sclk = None if args.no_sclk else observed_sclk_mhz(1.5, lambda: run_step(hot))
    torch.cuda.synchronize()

    cold = None
    if not args.no_cold:
        set_bytes = sum(x.numel() * x.element_size() for x in hot.values())
        nsets = max(2, -(-COLD_BYTES // set_bytes))
        sets = [hot] + [make_set() for _ in range(nsets - 1)]
        el = timed(sets, max(args.steps, 2 * nsets), 2 * nsets)
        nsteps = max(args.steps, 2 * nsets)
        cold = {"value": wl.tokens * nsteps / el, "ms_per_step": el / nsteps * 1e3, "sets": nsets,
                "bytes_per_set": set_bytes}
        del sets

    # Dominant kernel: the distance stage (laplace_l1_exp, or gauss_l2_exp for the Gaussian variant), through its
    # own entry point on the same stream, bracketed by HIP events.
    G, N, m, d = p.G, p.N, p.m, p.d
    gauss = wl.kernel == "gauss"
    dist = distance_stage(wl, lf)
    L = torch.empty(G * m * d, device="cuda")
    CQ = torch.empty(G * N * m, device="cuda")
    CK = torch.empty_like(CQ)
    We = torch.empty(G * m * m, device="cuda")
    lf.lf_landmark_pool(p, Q, L, stream)
    for _ in range(5):
        dist(p, Q, K, L, CQ, CK, We, stream)
    # Back-to-back launches between two events on the kernel's own stream: the average is the kernel's duration
    # (the GPU never idles between launches), which is what rocprofv3's kernel trace reports for it.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.kernel_reps):
        dist(p, Q, K, L, CQ, CK, We, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    lap_us = e0.elapsed_time(e1) / args.kernel_reps * 1e3
    # Algorithmic work over the 2N + m rows per slice, per (row, landmark, channel): Laplacian, one subtract and one
    # |.|-add (VALU operations); Gaussian, one multiply-add of x.l (2 flops, fp32 MFMA).
    ops = 2.0 * G * (2 * N + m) * m * d
    achieved = ops / (lap_us * 1e-6) / 1e12
    if gauss:
        roof = {"kernel": "gauss_l2_exp", "bound": "mfma", "achieved": achieved, "peak": MFMA_F32_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_F32_PEAK_TFLOPS, "traffic": None, "avg_us": lap_us,
                "flops_per_launch": ops}
    else:
        roof = {"kernel": "laplace_l1_exp", "bound": "alu", "achieved": achieved, "peak": VALU_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / VALU_PEAK_TFLOPS,
                "traffic": load_traffic() if args.workload == "pvt_s1_56x56_m49" else None,
                "avg_us": lap_us, "ops_per_launch": ops}

    # Per-stage event times (each stage entry point alone, same stream), for context.
    stages = {}

    def time_stage(name, fn, reps=50):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        stages[name] = round(e0.elapsed_time(e1) / reps * 1e3, 2)

    X = torch.empty(G * m * m, device="cuda")
    S = torch.empty(G * m * d, device="cuda")
    P = torch.empty(G * m * d, device="cuda")
    time_stage("landmark_pool", lambda: lf.lf_landmark_pool(p, Q, L, stream))
    time_stage("gauss_l2_exp" if gauss else "laplace_l1_exp", lambda: dist(p, Q, K, L, CQ, CK, We, stream))
    time_stage("ns_pinv", lambda: lf.lf_ns_pinv(p, We, X, None, None, None, ws, stream))
    time_stage("ckv_reduce", lambda: lf.lf_ckv_reduce(p, CK, V, S, ws, stream))
    time_stage("landmark_mix", lambda: lf.lf_landmark_mix(p, X, S, None, P, stream))
    time_stage("out_gemm_dwc", lambda: lf.lf_out_gemm_dwc(p, CQ, P, None, V, w, Y, stream))
    # The forward's solver launch as lf_attn_fwd makes it (m <= 64: Newton-Schulz with S = C_K^T V beside it),
    # through the stage entry points: the solver's own share is ns_pinv above.
    # MFMA stages against the fp32 MFMA peak, algorithmic flops per call: Newton-Schulz 4 K m^3 per slice (two
    # m x m products per step), C_K^T V and the output product 2 N m d, the landmark mix 2 m^2 d. The solver's
    # fraction is chip-wide; it holds one CU per slice, so per_cu_frac scales it by the CUs it occupies.
    flops = {"ns_pinv": 4.0 * G * wl.ns_iters * m ** 3, "ckv_reduce": 2.0 * G * N * m * d,
             "landmark_mix": 2.0 * G * m * m * d, "out_gemm_dwc": 2.0 * G * N * m * d}
    mfma = {}
    for name, fl in flops.items():
        us = stages[name]
        ach = fl / (us * 1e-6) / 1e12
        mfma[name] = {"flops": fl, "us": us, "achieved_tflops": round(ach, 3),
                      "frac": round(ach / MFMA_F32_PEAK_TFLOPS, 5)}
    if m <= 64:
        mfma["ns_pinv"]["per_cu_frac"] = round(mfma["ns_pinv"]["frac"] * 256 / min(256, G), 5)

    rec = {
        "metric": METRIC_TRAIN if train else (METRIC_GAUSS if gauss else METRIC),
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == WL.F32 else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} {'forward+backward' if train else 'forward'}", "B": wl.B,
                   "heads": wl.heads, "H": wl.H, "W": wl.W, "d": wl.d, "r": wl.r, "m": wl.m, "lambda": wl.lam,
                   "eps": wl.eps, "ns_iters": wl.ns_iters, "kernel": wl.kernel, "tokens_per_step": wl.tokens},
        "roofline": roof,
        "mfma_stages": mfma,
        "stages_us": stages,
        "step_events": step_events,
        "sclk_mhz": sclk,
    }
    if cold is not None:
        rec["cold"] = cold
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
