#!/usr/bin/env python3
"""Benchmark of the block-quantized GEMV on one MI355X.

Metric: effective weight-read GB/s (quantized weight bytes / time) and the
fraction of MI355X HBM peak. Default workload: the Q6_K output projection,
k=2560, n=262144 (vocabulary), m=1, y = x @ W; one step is one launch over
all rows. W is rotated over enough copies that HBM, not the 256 MB
last-level cache, serves it. The same rows as 8 row-range tiles accumulating
into y are timed as well and reported under "tiled".

--op t times the transposed (backward-input) product dx = dy @ W over the
same weights instead (dy of length n in, dx of length k out); --op moe the
expert-indexed product of an expert workload (top_k of the stacked experts per
position; the expert sets rotate with the weight copies so that HBM serves
them).

Prints ONE JSON line. Extra modes:
  --summarize-pmc CSV...   turn rocprofv3 counter CSVs of this script into
                           the traffic summary under profiles/
"""
from __future__ import annotations

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
MFMA_F16_PEAK_TFS = 2500.0    # dense f16/bf16 matrix-core peak of MI355X
# Sources of each kernel family (the traffic summary of a workload is valid
# only for the sources it was measured on).
COMMON_SOURCES = ["block_quantized_matvec_gguf_amd/csrc/qmv_api.cpp",
                  "block_quantized_matvec_gguf_amd/csrc/qmv_internal.h"]
FAMILY_SOURCES = {"gemv": ["block_quantized_matvec_gguf_amd/csrc/qmv_gemv.hip",
                           "block_quantized_matvec_gguf_amd/csrc/qmv_units.h"],
                  "gemv_t": ["block_quantized_matvec_gguf_amd/csrc/qmv_gemv_t.hip",
                             "block_quantized_matvec_gguf_amd/csrc/qmv_units.h"],
                  "affine": ["block_quantized_matvec_gguf_amd/csrc/qmv_gemv.hip",
                             "block_quantized_matvec_gguf_amd/csrc/qmv_units.h"],
                  "mfma": ["block_quantized_matvec_gguf_amd/csrc/qmv_mfma.hip"],
                  "simple": ["block_quantized_matvec_gguf_amd/csrc/qmv_simple.hip"]}
# the dispatches whose counters and durations are the family's (not x staging
# or the partial-sum reduction)
MAIN_KERNEL = {"gemv": "qmv_gemv", "gemv_t": "qmv_gemv_t_staged", "mfma": "qmv_mfma_",
               "simple": "qmv_simple", "affine": "qmv_affine_gemv"}


def is_main_kernel(family: str, name: str) -> bool:
    return MAIN_KERNEL[family] in name and "prep_x" not in name
METRIC = "effective weight-read GB/s and % of MI355X HBM peak for quantized GEMV"


def kernel_family(kernel_name: str) -> str:
    return ("mfma" if kernel_name.startswith("qmv_mfma") else
            "affine" if kernel_name.startswith("qmv_affine") else
            "simple" if kernel_name.startswith("qmv_simple") else
            "gemv_t" if kernel_name.startswith("qmv_gemv_t") else "gemv")


def kernel_name_of(qb, fmt, k: int, m: int, algo: int, op: str) -> str:
    if op == "affine":
        return qb.qmv_affine_kernel_name(fmt, k)
    if op == "t":
        return qb.qmv_t_kernel_name(fmt, k, algo)
    if op == "moe":
        return qb.qmv_moe_kernel_name(fmt, k, algo)
    return qb.qmv_kernel_name(fmt, k, m, algo)


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for rel in COMMON_SOURCES + FAMILY_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(workload: str, op: str = "fwd") -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s%s.json" % (workload,
                                                                "_t" if op == "t" else ""))


def load_traffic(workload: str, family: str, op: str = "fwd"):
    """HBM bytes per launch from committed counter runs, or None when absent
    or taken on a different kernel source."""
    p = traffic_path(workload, op)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash(family):
        return None
    return t


def summarize_pmc(args):
    """Average FETCH_SIZE / WRITE_SIZE per dispatch of the GEMV kernel and of
    the calibration copy (torch copy of a known byte count) and write the
    traffic summary for the workload."""
    import csv
    from block_quantized_matvec_gguf_amd import binding as qb
    from block_quantized_matvec_gguf_amd import synth
    spec = synth.WORKLOADS[args.workload]
    fmt_ = spec["bits"] if args.op == "affine" else synth.fmt_id(spec["fmt"])
    family = kernel_family(kernel_name_of(qb, fmt_, spec["k"], spec["m"], qb.ALGOS[args.algo],
                                          args.op))
    per = {}
    for path in args.summarize_pmc:
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            key = "gemv" if is_main_kernel(family, name) else ("copy" if "neg_kernel" in name or
                                                      ("elementwise" in name and "neg" in name)
                                                      else None)
            if key is None:
                continue
            per.setdefault((key, r["Counter_Name"]), []).append(float(r["Counter_Value"]))

    def avg(key, c):
        v = per.get((key, c), [])
        return sum(v) / len(v) if v else None

    copy_bytes = args.calib_bytes
    cf, cw = avg("copy", "FETCH_SIZE"), avg("copy", "WRITE_SIZE")
    gf, gw = avg("gemv", "FETCH_SIZE"), avg("gemv", "WRITE_SIZE")
    out = {"workload": args.workload, "op": args.op, "kernel_family": family,
           "kernel_source_sha256": kernel_source_hash(family),
           "gemv_fetch_kib_per_dispatch": gf, "gemv_write_kib_per_dispatch": gw,
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw}
    if cf and gf is not None:
        out["fetch_factor"] = copy_bytes / (cf * 1024.0)
        out["fetch_bytes_per_launch"] = gf * 1024.0 * out["fetch_factor"]
    if cw and gw is not None:
        out["write_factor"] = copy_bytes / (cw * 1024.0)
        out["write_bytes_per_launch"] = gw * 1024.0 * out["write_factor"]
    if "fetch_bytes_per_launch" in out and "write_bytes_per_launch" in out:
        out["bytes_per_launch"] = out["fetch_bytes_per_launch"] + out["write_bytes_per_launch"]
    os.makedirs(os.path.dirname(traffic_path(args.workload, args.op)), exist_ok=True)
    with open(traffic_path(args.workload, args.op), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def host_threads():
    """Host threads for the oracle baseline: every CPU this process may run
    on (its affinity mask), capped by OMP_NUM_THREADS when that is set (the
    GPU machine sets it to the host share of one GPU)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = min(avail, int(omp)) if omp and omp.isdigit() and int(omp) > 0 else avail
    return max(1, threads), avail, omp


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_entry(value, threads, avail, omp, sample):
    return {"value": value, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample, "nproc": os.cpu_count(), "cpus_in_affinity": avail,
            "omp_num_threads": omp, "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The device's clock controller reacts to a sustained launch stream within
    # a few milliseconds: the first ~10 vocabulary launches run at the boost
    # clock (about 96 us each), the next ones dip (up to 140 us) and the clock
    # settles after ~10 ms (103-110 us). 100 untimed launches (~12 ms) put the
    # timed region in the settled state.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="q6_k_vocab_outproj")
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--op", choices=["fwd", "t", "moe", "affine"], default=None,
                    help="fwd: y = x @ W; t: the transposed product dx = dy @ W; moe: the "
                         "expert-indexed product (default: moe for expert workloads, else fwd)")
    ap.add_argument("--tiles", type=int, default=None, help="tiles of the auxiliary run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-tiled", action="store_true",
                    help="skip the tiled run (profiling runs: one launch shape only)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain copy of --calib-bytes (counter calibration)")
    ap.add_argument("--calib-bytes", type=int, default=512 * 1024 * 1024)
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9,
                    help="bytes of weight copies the steps rotate over (default 1.1 GB: more "
                         "than the 256 MB last-level cache; counter runs use less, since every "
                         "copy is one more dispatch under the profiler)")
    ap.add_argument("--summarize-pmc", nargs="*", default=None)
    args = ap.parse_args()

    if args.op is None:
        from block_quantized_matvec_gguf_amd import synth as _s
        spec_ = _s.WORKLOADS[args.workload]
        args.op = "moe" if "experts" in spec_ else "affine" if "bits" in spec_ else "fwd"
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; runs on several GPUs are not implemented (the "
              "product would shard by output rows with no exchange inside it). Requested "
              "--gpus %d, WORLD_SIZE %d." % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_matvec_gguf_amd import binding as qb
    from block_quantized_matvec_gguf_amd import synth

    op_t = args.op == "t"
    op_moe = args.op == "moe"
    op_aff = args.op == "affine"
    if op_aff:  # three arrays: code words, bf16 scales, bf16 biases
        spec = synth.WORKLOADS[args.workload]
        words, scales, biases, x = synth.affine_workload(args.workload)
        fmt = spec["bits"]
        W = np.concatenate([words.view(np.uint8).reshape(-1), scales.view(np.uint8).reshape(-1),
                            biases.view(np.uint8).reshape(-1)])
    else:
        fmt, W, x, spec = synth.workload(args.workload)
    k, n, m = spec["k"], spec["n"], spec["m"]
    if op_t:  # the transposed product reads dy (m x n) and writes dx (m x k)
        x = synth.gen_x(np.random.default_rng(0x51A72000 + spec["id"]), m, n)
    tiles = args.tiles if args.tiles is not None else spec.get("tiles", 8)
    algo = qb.ALGOS[args.algo]
    wbytes = W.nbytes
    copies = max(1, int(np.ceil(args.rotate_bytes / wbytes)))
    if op_moe:
        E, top_k = spec["experts"], spec["top_k"]
        slab = W.nbytes // E
        # disjoint expert sets, one per step in turn (each set: top_k experts
        # per position, all positions drawn from the set's experts)
        perm = np.random.default_rng(0x51A73000 + spec["id"]).permutation(E)
        nsets = max(1, E // (top_k * m))
        id_sets = [perm[s_ * top_k * m:(s_ + 1) * top_k * m].astype(np.int32)
                   for s_ in range(nsets)]
        wbytes = len(np.unique(id_sets[0])) * slab       # weight bytes one call reads
        copies = max(1, int(np.ceil(args.rotate_bytes / (wbytes * nsets))))
    dev = torch.device("cuda:0")
    Wd = [torch.from_numpy(W).to(dev)]
    for _ in range(copies - 1):
        Wd.append(Wd[0].clone())
    xd = torch.from_numpy(x).to(dev)
    yd = torch.zeros((m * (top_k if op_moe else 1), k if op_t else n), dtype=torch.float32,
                     device=dev)
    qb.ensure_context()
    lib = qb.load()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    wp = [w.data_ptr() for w in Wd]
    xp, yp = xd.data_ptr(), yd.data_ptr()

    entry = lib.qmv_run_t_ex if op_t else lib.qmv_run_ex
    if op_aff:  # the three arrays sit back to back in each weight copy
        o_s, o_b = words.nbytes, words.nbytes + scales.nbytes
    if op_moe:
        idd = [torch.from_numpy(a).to(dev) for a in id_sets]
        idp = [t.data_ptr() for t in idd]

    def run(i, j0=0, j1=n, acc=0):
        if op_aff:
            wb = wp[i % copies]
            rc = lib.qmv_run_affine(fmt, wb, wb + o_s, wb + o_b, xp, yp, k, n, m, j0, j1, acc, sp)
        elif op_moe:
            # step i: weight copy i % copies, expert set (i // copies) % nsets
            rc = lib.qmv_run_moe_ex(fmt, wp[i % copies], idp[(i // copies) % nsets], xp, yp, k,
                                    n, E, m, top_k, acc, sp, algo)
        else:
            rc = entry(fmt, wp[i % copies], xp, yp, k, n, m, j0, j1, acc, sp, algo)
        if rc != 0:
            raise RuntimeError("qmv run: %s %s" % (qb.qmv_status_string(rc), qb.qmv_last_error()))

    # ---- main timed region: one launch over all rows per step
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        run(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) * 1e-3
    step_s = max(wall, gpu_s) / args.steps
    launch_s = gpu_s / args.steps
    y_main = yd.cpu().numpy()
    last_ids = id_sets[((args.steps - 1) // copies) % nsets] if op_moe else None

    # ---- auxiliary: the same rows as row-range tiles accumulating into y
    edges = [t * n // tiles for t in range(tiles + 1)]
    tstep = None
    if not args.no_tiled and not op_moe:
        yd.zero_()
        # forward: every tile adds into y; transposed: tile 0 writes dx and
        # tiles 1.. add (the partial-sum convention of the backward pass)
        def tacc(t):
            return (1 if t > 0 else 0) if op_t else 1

        for i in range(max(1, args.warmup // 4)):
            for t in range(tiles):
                run(i, edges[t], edges[t + 1], tacc(t))
        torch.cuda.synchronize()
        tsteps = max(1, args.steps // 2)
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e2.record(stream)
        for i in range(tsteps):
            for t in range(tiles):
                run(i, edges[t], edges[t + 1], tacc(t))
        e3.record(stream)
        torch.cuda.synchronize()
        twall = time.perf_counter() - t0
        tgpu = e2.elapsed_time(e3) * 1e-3
        tstep = max(twall, tgpu) / tsteps

    if args.calibrate_copy:
        # a plain elementwise kernel that reads and writes calib_bytes each
        a = torch.ones(args.calib_bytes // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    # W read + x + y (dy + dx) once
    alg_bytes = wbytes + m * k * 4 + m * (top_k if op_moe else 1) * n * 4
    achieved = alg_bytes / launch_s / 1e9
    value = wbytes / step_s / 1e9
    kname = kernel_name_of(qb, fmt, k, m, algo, args.op)
    traffic = load_traffic(args.workload, kernel_family(kname), args.op)
    traffic_bytes = (round(traffic["bytes_per_launch"])
                     if traffic and "bytes_per_launch" in traffic else None)
    hbm = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_bytes,
           "algorithmic_bytes_per_launch": alg_bytes, "launch_us": round(launch_s * 1e6, 3)}
    if kname.startswith("qmv_mfma"):
        # matrix-core kernel: 2*m*k*n algorithmic flops against the dense f16
        # (bf16) peak; x enters as two terms, and the weights of the scaled
        # formats as two more (no lo*lo product), so the units execute two or
        # three times that
        flops = 2.0 * m * k * n
        terms = 2 if fmt in (synth.F16, synth.BF16, synth.Q4_K) else 3
        tf = flops / launch_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_F16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(tf / MFMA_F16_PEAK_TFS, 4),
                    "traffic": traffic_bytes, "algorithmic_flops_per_launch": flops,
                    "executed_mfma_flops_per_launch": terms * flops,
                    "launch_us": round(launch_s * 1e6, 3),
                    "hbm": {k_: hbm[k_] for k_ in ("achieved", "peak", "unit", "frac",
                                                   "algorithmic_bytes_per_launch")}}
    else:
        roofline = hbm
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; value distributions of the measured workload)",
        "config": {"workload": args.workload + ("_transposed" if op_t else ""),
                   **({"experts": E, "top_k": top_k, "expert_sets_rotated": nsets}
                      if op_moe else {}),
                   "format": ("affine%d_group64" % fmt) if op_aff else synth.FORMAT_NAMES[fmt],
                   "k": k,
                   "n": n, "m_tokens": m, "accumulate": 0, "weight_bytes": wbytes,
                   "weight_copies_rotated": copies,
                   "kernel": kname},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "rows_per_s": round(m * (top_k if op_moe else 1) * n / step_s, 1),
        "roofline": roofline,
    }
    if tstep is not None:
        out["tiled"] = {"tiles": tiles, "accumulate": "tiles 1.. add" if op_t else 1,
                        "ms_per_step": round(tstep * 1e3, 5),
                        "value": round(wbytes / tstep / 1e9, 1),
                        "pct_hbm_peak": round(100.0 * wbytes / tstep / 1e9 / HBM_PEAK_GBS, 2)}

    if not args.no_cpu_baseline and op_aff:
        import oracle
        threads, avail, omp = host_threads()
        t0 = time.perf_counter()
        yref, sref = oracle.affine_gemv(fmt, words, scales, biases, x, k, n, threads=threads)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = cpu_baseline_entry(
            round(wbytes / dt / 1e9, 3), threads, avail, omp,
            "all %d rows, m=%d, f64 accumulation; %.2f s" % (n, m, dt))
        res = oracle.check_parity(y_main, yref, sref)
        out["parity"] = {"ok": res["ok"], "max_err_over_tol": round(res["max_ratio"], 5),
                         "cosine": res["cosine"], "outputs": res["n"]}
    elif not args.no_cpu_baseline and op_moe:
        import oracle
        threads, avail, omp = host_threads()
        t0 = time.perf_counter()
        yref, sref = oracle.moe(fmt, W, last_ids, x, k, n, E, top_k, threads=threads)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = cpu_baseline_entry(
            round(wbytes / dt / 1e9, 3), threads, avail, omp,
            "the whole call (%d expert rows x %d), f64 accumulation; %.2f s"
            % (len(last_ids) * n, k, dt))
        res = oracle.check_parity(y_main, yref, sref)
        out["parity"] = {"ok": res["ok"], "max_err_over_tol": round(res["max_ratio"], 5),
                         "cosine": res["cosine"], "outputs": res["n"]}
    elif not args.no_cpu_baseline and op_t:
        import oracle
        threads, avail, omp = host_threads()
        # a bounded sample of columns (each needs every row of the range)
        ncols = max(1, min(k, 400_000_000 // max(1, n * m)))
        cols = np.linspace(0, k - 1, ncols).astype(np.int64)
        t0 = time.perf_counter()
        dref, sref = oracle.gemv_t_cols(fmt, W, x, k, n, cols, threads=threads)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = cpu_baseline_entry(
            round(wbytes * ncols / k / dt / 1e9, 3), threads, avail, omp,
            "%d of %d columns (evenly spaced), all %d rows, m=%d, f64 accumulation; %.2f s"
            % (ncols, k, n, m, dt))
        res = oracle.check_parity(y_main[:, cols], dref, sref)
        out["parity"] = {"ok": res["ok"], "max_err_over_tol": round(res["max_ratio"], 5),
                         "cosine": res["cosine"], "outputs": res["n"]}
    elif not args.no_cpu_baseline:
        import oracle
        threads, avail, omp = host_threads()
        # the whole workload when it is small enough, else a bounded row sample
        rows = n if k * n * m <= 4_000_000_000 else max(1, 4_000_000_000 // (k * m))
        t0 = time.perf_counter()
        yref, sref = oracle.gemv(fmt, W, x, k, n, 0, rows, threads=threads)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = cpu_baseline_entry(
            round(rows * (wbytes / n) / dt / 1e9, 3), threads, avail, omp,
            "rows 0..%d of %d (%s), m=%d, f64 accumulation; %.2f s" % (
                rows, n, "all" if rows == n else "first rows", m, dt))
        res = oracle.check_parity(y_main[:, :rows], yref, sref)
        out["parity"] = {"ok": res["ok"], "max_err_over_tol": round(res["max_ratio"], 5),
                         "cosine": res["cosine"], "outputs": res["n"]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
