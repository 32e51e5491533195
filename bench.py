"""Benchmark: dense and VSA self-attention at the 480p Wan2.2 shape on one MI355X.

One step = one pass of the whole hot path on synthetic inputs already resident
in HBM:
  * dense attention, CFG pair x 40 heads x 32,760 tokens x d128 (one call);
  * VSA, 1 x 40 heads, grid 21x30x52 padded to 624 cubes, top-32: the coarse
    call (gather + pool, scores, top-k) and the fine call.
Prints one JSON line.  ms_per_step is the time of exactly --steps steps over
their count.  The per-kernel times are means over those steps, from HIP events
the library records on the launch stream around each kernel; the per-call
medians come from events recorded on the same stream around each call.  After
the timed steps, extra records are taken (not part of the step): VSA at
top-78, VSA with the gated coarse branch, the 3D RoPE (standalone and fused),
the softmax reference policies, sliding-tile attention, the 720p shape, and
the step's kernels on one GPU's share of the heads when eight GPUs split them
(--no-extra skips them).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import subprocess
import sys
import time
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
PEAK_CLOCK_GHZ = 2.4        # engine clock the published MFMA peak assumes
DENSE = "dense_480p_cfg"
VSA = "vsa_480p"
# HBM traffic of the dense kernel, measured with rocprofv3 FETCH_SIZE / WRITE_SIZE; used only while
# the kernel sources hash to the value recorded with the measurement
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_dense_fwd_480p_cfg.json")
DENSE_SOURCES = [os.path.join(ROOT, "video_diffusion_dit_amd", "csrc", f)
                 for f in ("dense.hip", "wf_device.hpp", "wf_tiles.hpp")]


def sources_sha256(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_counters():
    """The committed rocprofv3 counter summary of wf_dense_fwd, or {} if missing or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    if t.get("source_sha256") != sources_sha256(DENSE_SOURCES):
        return {}
    return t


def measured_traffic():
    """Bytes per launch of wf_dense_fwd from the committed counter summary, or None if stale."""
    return measured_counters().get("bytes_per_launch")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip timing the CPU oracle (used for profiler runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--cpu-full", action="store_true",
                   help="also time the oracle per measured configuration (whole calls where they take "
                        "seconds to a minute, one head scaled otherwise) and add the record 'cpu_oracle_calls'")
    p.add_argument("--traffic-json", metavar="ROCPROF_DIR", default=None,
                   help="write the dense kernel's calibrated traffic, clock and MFMA busy fraction from a "
                        "rocprofv3 run directory to profiles/ and exit (no GPU)")
    p.add_argument("--summarize", metavar="ROCPROF_DIR", default=None,
                   help="print a text summary of rocprofv3 CSV output under ROCPROF_DIR and exit")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the extra records after the timed steps (VSA top-78, one GPU's share of "
                        "heads); profiling runs use it to keep per-kernel averages to the step's own launches")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="before timing, run one plain device copy of this many MiB (a known-size "
                        "kernel that calibrates the profiler's HBM byte counters)")
    return p.parse_args()


def git_rev() -> str:
    """The source revision: git's, or (where the tree travels without .git) the one the build
    step recorded next to the library it built."""
    try:
        rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True, timeout=10).stdout.strip()
        if rev:
            return rev
    except Exception:
        pass
    try:
        with open(os.path.join(ROOT, "video_diffusion_dit_amd", "build_info.json")) as f:
            info = json.load(f)
        return info.get("git", "unknown") + ("+dirty" if info.get("dirty") else "") + " (recorded at build)"
    except (OSError, ValueError):
        return "unknown"


def dense_flops(wl) -> float:
    return 4.0 * wl.B * wl.Hh * wl.N * wl.N * wl.D


def vsa_flops(wl, C) -> dict:
    fine = 4.0 * wl.B * wl.Hh * wl.N * 64 * wl.topk * wl.D        # padded queries excluded
    coarse = 2.0 * wl.B * wl.Hh * C * C * wl.D
    return dict(fine=fine, coarse=coarse, total=fine + coarse)


IDEAL_CONVENTION = ("dense FLOPs / VSA FLOPs at the same shape, real tokens: 4 N^2 D / (4 N (64 k) D + "
                    "2 C^2 D) per head (gather, top-k and padding excluded)")


def ideal_speedup(wl, C) -> float:
    """The dense call's FLOPs over the VSA call's (fine on real queries + coarse scores), per head."""
    return dense_flops(wl) / vsa_flops(wl, C)["total"]


def vsa_bytes(wl, C, gated=False) -> dict:
    """Algorithmic HBM bytes per call of each VSA kernel (Cs: C rounded up to 32).  The cube means
    of Q and K are stored as three bf16 parts (6 bytes per element), V's as two."""
    Np, Cs = 64 * C, (C + 31) // 32 * 32
    BH = wl.B * wl.Hh
    means_qk, means_v = 2 * C * wl.D * 6, 2 * wl.D * Cs * 2
    gather = BH * (3 * wl.N * wl.D * 2 + 3 * Np * wl.D * 2 + means_qk + means_v)
    # the one-call path's gather writes no cube-ordered Q, K or V, and reads V only for V's mean,
    # which only the gated coarse branch needs
    gather_one_call = BH * ((3 if gated else 2) * wl.N * wl.D * 2 + means_qk + (means_v if gated else 0))
    scores = BH * (2 * C * wl.D * 6 + C * Cs * 4)
    topk = BH * (C * C * 4 + C * wl.topk * 4 + C * 8)
    # coarse-branch output: scores + row statistics + hi/lo cube means of V in, O_coarse out
    coarse_out = BH * (C * Cs * 4 + C * 8 + 2 * wl.D * Cs * 2 + C * wl.D * 4)
    # the gated merge adds the gate (bf16, every real token) to the fine stage's traffic
    merge = BH * wl.N * wl.D * 2
    return dict(gather=gather, gather_one_call=gather_one_call, scores=scores, topk=topk, coarse_out=coarse_out,
                merge=merge)


def blas_info() -> dict:
    """The BLAS numpy's matrix products run on, and its thread count."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return {"library": f"{i.get('internal_api')} {i.get('version')}", "threads": int(i.get("num_threads", 1))}
    except Exception:
        pass
    return {"library": "unknown", "threads": os.cpu_count() or 1}


def cpu_baseline(seconds: float) -> dict:
    """The fp64 oracle on a bounded sample of the step's workload, about `seconds` of CPU.

    Whole dense heads of the dense workload (most of the budget) and whole VSA heads
    (pool, scores, top-k, fine) of the VSA workload; the rate is the step's FLOPs over
    the step's time extrapolated from the per-head times, the same convention as
    `value`."""
    import oracle
    import synth
    blas = blas_info()
    wd, wv = synth.WORKLOADS[DENSE], synth.WORKLOADS[VSA]

    def heads_within(wl, budget, run, least=1):
        phi = synth.field_for(wl)
        n, dt = 0, 0.0
        for bh in range(wl.B * wl.Hh):          # whole heads until the time budget is spent
            b, h = divmod(bh, wl.Hh)
            q, k, v = (synth.bits_to_f64(synth.make_slice(wl, t, b, h, phi)) for t in ("q", "k", "v"))
            t0 = time.perf_counter()
            run(wl, q, k, v)
            dt += time.perf_counter() - t0
            n += 1
            if n >= least and dt >= budget:
                break
        return n, dt

    nd, td = heads_within(wd, 0.85 * seconds, lambda wl, q, k, v: oracle.attention(q, k, v, wl.scale))
    nv, tv = heads_within(wv, 0.15 * seconds,
                          lambda wl, q, k, v: oracle.vsa(q, k, v, wl.T, wl.H, wl.W, wl.topk, wl.scale), least=2)
    C = int(oracle.geometry(wv.T, wv.H, wv.W)["C"])
    step_flops = dense_flops(wd) + vsa_flops(wv, C)["total"]
    step_s = td / nd * wd.B * wd.Hh + tv / nv * wv.B * wv.Hh
    return {"value": step_flops / step_s / 1e12, "unit": "TFLOP/s", "cores": blas["threads"], "kind": "oracle",
            "sample": f"fp64 numpy oracle ({blas['library']}, {blas['threads']} threads): dense attention of "
                      f"{nd} whole head(s) ({wd.N} x {wd.N} x d{wd.D}) of the {DENSE} workload in {td:.1f} s, and "
                      f"the whole VSA pass of {nv} head(s) of the {VSA} workload (top-{wv.topk} of {C} cubes) in "
                      f"{tv:.1f} s; one step extrapolated: {step_s:.0f} s",
            "blas": blas["library"], "host_cpus": os.cpu_count()}


def cpu_oracle_calls() -> dict:
    """The fp64 oracle per measured configuration: whole calls of the 512-token, 12-head 480p
    and VSA 480p workloads, and one (batch, head) of the CFG-pair and 720p workloads scaled by
    their head counts (labelled extrapolated).  Minutes of CPU; run on request (--cpu-full)."""
    import oracle
    import synth
    blas = blas_info()
    out = {"blas": blas["library"], "threads": blas["threads"], "host_cpus": os.cpu_count(), "configs": {}}

    def slices(wl, heads):
        phi = synth.field_for(wl)
        for b, h in heads:
            yield tuple(synth.bits_to_f64(synth.make_slice(wl, t, b, h, phi)) for t in ("q", "k", "v"))

    def dense_call(name, heads):
        wl = synth.WORKLOADS[name]
        dt = 0.0
        for q, k, v in slices(wl, heads):
            t0 = time.perf_counter()
            oracle.attention(q, k, v, wl.scale)
            dt += time.perf_counter() - t0
        return wl, dt

    def vsa_call(name, heads):
        wl = synth.WORKLOADS[name]
        dt = 0.0
        for q, k, v in slices(wl, heads):
            t0 = time.perf_counter()
            oracle.vsa(q, k, v, wl.T, wl.H, wl.W, wl.topk, wl.scale)
            dt += time.perf_counter() - t0
        return wl, dt

    for name, kind, whole in (("dense_512_iid", "dense", True), ("dense_480p_12h", "dense", True),
                              ("dense_480p_cfg", "dense", False), ("vsa_480p", "vsa", True),
                              ("dense_720p_cfg", "dense", False), ("vsa_720p", "vsa", False)):
        wl = synth.WORKLOADS[name]
        heads = [(b, h) for b in range(wl.B) for h in range(wl.Hh)] if whole else [(0, 0)]
        wl, dt = (dense_call if kind == "dense" else vsa_call)(name, heads)
        C = int(oracle.geometry(wl.T, wl.H, wl.W)["C"])
        flops = dense_flops(wl) if kind == "dense" else vsa_flops(wl, C)["total"]
        call_s = dt if whole else dt * wl.B * wl.Hh
        print(f"cpu oracle {name}: {call_s:.1f} s per call ({'whole call' if whole else 'extrapolated from one head'})",
              file=sys.stderr, flush=True)
        out["configs"][name] = {"seconds_per_call": call_s, "measured": "whole call" if whole else
                                f"one (b, h) of {wl.B * wl.Hh}, scaled (extrapolated)",
                                "tflops": flops / call_s / 1e12}
    return out


def _short(name: str) -> str:
    base = name.split("(")[0]
    return base.replace("void ", "").strip()


def summarize(rocprof_dir: str) -> None:
    """Summarise rocprofv3 --kernel-trace --stats and --pmc CSV files (no GPU needed)."""
    for path in sorted(glob.glob(os.path.join(rocprof_dir, "**", "*_kernel_stats.csv"), recursive=True)):
        print(f"# kernel stats: {os.path.relpath(path, rocprof_dir)}")
        print(f"{'kernel':44s} {'calls':>6s} {'avg_ms':>10s} {'min_ms':>10s} {'max_ms':>10s} {'pct':>6s}")
        for r in csv.DictReader(open(path)):
            print(f"{_short(r['Name'])[:44]:44s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:10.4f} "
                  f"{float(r['MinNs']) / 1e6:10.4f} {float(r['MaxNs']) / 1e6:10.4f} {float(r['Percentage']):6.2f}")
    for path in sorted(glob.glob(os.path.join(rocprof_dir, "**", "*_counter_collection.csv"), recursive=True)):
        print(f"# counters: {os.path.relpath(path, rocprof_dir)} (mean per dispatch)")
        agg = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(path)):
            agg[_short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, cs in agg.items():
            vals = "  ".join(f"{c}={sum(v) / len(v):.6g}" for c, v in sorted(cs.items()))
            print(f"{k[:44]:44s} n={len(next(iter(cs.values())))}  {vals}")


def write_traffic(rocprof_dir: str, out_path: str = TRAFFIC_FILE) -> dict:
    """Write the traffic summary (TRAFFIC_FILE) from a rocprofv3 run directory (no GPU needed).

    The directory holds the passes the committed profiles name: kt/ (kernel
    trace), FETCH_SIZE/ and WRITE_SIZE/ (one --pmc counter each) and sq1/
    (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES), all of the same bench command
    with --copy-probe-mib 1024.  The 1 GiB device copy in that command
    calibrates the byte counters: each is scaled so that the copy reads as 1 GiB
    fetched and 1 GiB written.
    """
    def counter(run, name, kern):
        path = os.path.join(rocprof_dir, run, f"{run}_counter_collection.csv")
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if kern in r["Kernel_Name"] and r["Counter_Name"] == name]
        if not vals:
            raise SystemExit(f"{path}: no {name} for {kern}")
        return sum(vals) / len(vals)

    def avg_ms(kern):
        for r in csv.DictReader(open(os.path.join(rocprof_dir, "kt", "kt_kernel_stats.csv"))):
            if kern in r["Name"]:
                return float(r["AverageNs"]) / 1e6
        raise SystemExit(f"no {kern} in the kernel trace")

    copy, kern = "__amd_rocclr_copyBuffer", "wf_dense_fwd"
    cf, cw = counter("FETCH_SIZE", "FETCH_SIZE", copy), counter("WRITE_SIZE", "WRITE_SIZE", copy)
    fs, ws = round((1 << 30) / (cf * 1024), 2), round((1 << 30) / (cw * 1024), 2)
    fe, wr = counter("FETCH_SIZE", "FETCH_SIZE", kern), counter("WRITE_SIZE", "WRITE_SIZE", kern)
    gui = counter("sq1", "GRBM_GUI_ACTIVE", kern)            # summed over the 8 XCDs
    busy = counter("sq1", "SQ_VALU_MFMA_BUSY_CYCLES", kern)  # summed over the 1,024 SIMDs
    out = {"kernel": kern, "workload": "dense MHA 2x40x32760xd128",
           "source_sha256": sources_sha256(DENSE_SOURCES),
           "clock_ghz": round(gui / 8 / (avg_ms(kern) * 1e-3) / 1e9, 3),
           "mfma_busy": round(busy / 1024 / (gui / 8), 3),
           "fetch_kib_per_dispatch": round(fe, 2), "write_kib_per_dispatch": round(wr, 2),
           "calibration": {"copy_bytes": 1 << 30, "copy_fetch_kib": round(cf), "copy_write_kib": round(cw),
                           "fetch_scale": fs, "write_scale": ws},
           "bytes_per_launch": fe * 1024 * fs + wr * 1024 * ws,
           "summary": "profiles/hbm_bytes_dense_2x40x32760_vsa_1x40_top32.txt",
           "command": "python3 bench.py --traffic-json <rocprofv3 run directory>"}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return out


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.traffic_json:
        print(json.dumps(write_traffic(args.traffic_json)))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py times one GPU (one GPU's share of the heads): --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import video_diffusion_dit_amd as wf

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    wd, wv = synth.WORKLOADS[DENSE], synth.WORKLOADS[VSA]
    qd, kd, vd = (to_dev(x) for x in synth.make_qkv(wd))
    qv, kv, vv = (to_dev(x) for x in synth.make_qkv(wv))
    C = wf.num_cubes(wv.T, wv.H, wv.W)
    od = torch.empty((wd.B, wd.Hh, wd.N, wd.D), dtype=torch.float32, device=dev)
    ws_d = torch.empty(wf.dense_workspace_bytes(wd.B, wd.Hh, wd.N, wd.D), dtype=torch.uint8, device=dev)
    ov = torch.empty((wv.B, wv.Hh, wv.N, wv.D), dtype=torch.float32, device=dev)
    idx = torch.empty((wv.B, wv.Hh, C, wv.topk), dtype=torch.int32, device=dev)
    ws_v = torch.empty(wf.vsa_workspace_bytes(wv.B, wv.Hh, wv.T, wv.H, wv.W, wv.D), dtype=torch.uint8,
                       device=dev)
    grid = (wv.T, wv.H, wv.W)

    def step(ev=None):
        # ev: three events recorded on the launch stream around the step's two calls; the VSA call is
        # the one-call path (wf_vsa: coarse and fine stage, no cube-ordered copies of Q and K)
        if ev:
            ev[0].record()
        wf.wf_attn_dense(qd, kd, vd, out=od, workspace=ws_d)
        if ev:
            ev[1].record()
        wf.wf_vsa(qv, kv, vv, grid, wv.topk, idx=idx, out=ov, workspace=ws_v)
        if ev:
            ev[2].record()

    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wf.profile_enable(True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    call_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(call_ev[i])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    # per-call medians over the timed steps (the means come from the library's per-kernel events)
    per_call = np.array([[ev[j].elapsed_time(ev[j + 1]) for j in range(2)] for ev in call_ev])
    med_dense, med_vsa = (float(np.median(per_call[:, j])) for j in range(2))
    kern = {}
    for name in ("wf_transpose_v", "wf_dense_fwd", "wf_vsa_gather", "wf_vsa_scores", "wf_vsa_topk",
                 "wf_vsa_fine"):
        n, tot = wf.profile_query(name)
        kern[name] = tot / n
    wf.profile_enable(False)

    dense_tf_step = dense_flops(wd) / (kern["wf_dense_fwd"] * 1e-3) / 1e12  # for dense-equivalent times

    def vsa_kernel_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        wf.profile_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        out_ms = {}
        for name in ("wf_vsa_gather", "wf_vsa_scores", "wf_vsa_topk", "wf_vsa_fine"):
            n, tot = wf.profile_query(name)
            out_ms[name] = tot / n
        wf.profile_enable(False)
        return out_ms

    # extra records (not part of the step): the same VSA call through the two-call path
    # (wf_vsa_coarse_topk + wf_vsa_fine, with cube-ordered copies of Q and K), and both paths at
    # the review's 78-of-624 operating point
    k78, k78_ms, k78_two_ms, two_ms = synth.WORKLOADS["vsa_480p_k78"].topk, None, None, None
    if not args.no_extra:
        idx78 = torch.empty((wv.B, wv.Hh, C, k78), dtype=torch.int32, device=dev)
        reps = max(3, args.steps // 2)

        def two_calls(kk, ix):
            wf.wf_vsa_coarse_topk(qv, kv, vv, grid, kk, idx=ix, workspace=ws_v)
            wf.wf_vsa_fine(ws_v, ix, (wv.B, wv.Hh, wv.N, wv.D), grid, out=ov)

        two_ms = vsa_kernel_ms(lambda: two_calls(wv.topk, idx), reps)
        k78_ms = vsa_kernel_ms(lambda: wf.wf_vsa(qv, kv, vv, grid, k78, idx=idx78, out=ov, workspace=ws_v), reps)
        k78_two_ms = vsa_kernel_ms(lambda: two_calls(k78, idx78), reps)

    # extra record (not part of the step): VSA with the gated merge (coarse-branch output plus
    # gate * O_coarse added in the fine stage's epilogue), same inputs and top-k, gate ~ U[0, 1),
    # through the one-call path
    gated_ms, plain_fine_ms = None, None
    if not args.no_extra:
        gate = to_dev(synth.make_gate(wv))

        def vsa_gated():  # the one-call path with a gate, as the step's VSA call
            wf.wf_vsa(qv, kv, vv, grid, wv.topk, idx=idx, out=ov, workspace=ws_v, gate=gate)

        vsa_gated()
        torch.cuda.synchronize()
        wf.profile_enable(True)
        for _ in range(max(3, args.steps // 2)):
            vsa_gated()
        torch.cuda.synchronize()
        gated_ms = {}
        for name in ("wf_vsa_gather", "wf_vsa_scores", "wf_vsa_topk", "wf_vsa_coarse_out", "wf_vsa_fine_gated"):
            n, tot = wf.profile_query(name)
            gated_ms[name] = tot / n
        wf.profile_enable(False)
        # the plain call right after, in the same conditions, for the merge's extra time
        plain_fine_ms = vsa_kernel_ms(lambda: wf.wf_vsa(qv, kv, vv, grid, wv.topk, idx=idx, out=ov,
                                                         workspace=ws_v), max(3, args.steps // 2))["wf_vsa_fine"]
        del gate

    # extra record (not part of the step): 3D RoPE of Q and K, standalone (wf_rope_qk, the form dense
    # attention takes) and fused into VSA's gather (the coarse stage with RoPE, then the fine stage)
    rope = None
    if not args.no_extra:
        qr, kr = torch.empty_like(qv), torch.empty_like(kv)

        def rope_runs():
            wf.wf_rope_qk(qv, kv, grid, q_out=qr, k_out=kr)
            wf.wf_rope_qk(qv, kv, grid, precision=64, q_out=qr, k_out=kr)
            wf.wf_vsa_coarse_topk(qv, kv, vv, grid, wv.topk, idx=idx, workspace=ws_v, rope_theta=10000.0)
            wf.wf_vsa_fine(ws_v, idx, (wv.B, wv.Hh, wv.N, wv.D), grid, out=ov)
            # the same gather without RoPE (it writes the same cube-ordered copies), for the fusion's cost
            wf.wf_vsa_coarse_topk(qv, kv, vv, grid, wv.topk, idx=idx, workspace=ws_v)

        rope_runs()
        torch.cuda.synchronize()
        wf.profile_enable(True)
        for _ in range(max(3, args.steps // 2)):
            rope_runs()
        torch.cuda.synchronize()
        rk = {}
        for name in ("wf_rope_qk", "wf_rope_qk_fp64", "wf_vsa_gather_rope", "wf_vsa_gather", "wf_vsa_scores",
                     "wf_vsa_topk", "wf_vsa_fine"):
            n, tot = wf.profile_query(name)
            rk[name] = tot / n
        wf.profile_enable(False)
        rope_bytes = 4.0 * wv.B * wv.Hh * wv.N * wv.D * 2   # Q and K, read and written
        rope = {"theta": 10000.0, "precision_fused_and_rope_qk": 32,
                "rope_qk_ms": rk["wf_rope_qk"],
                "rope_qk_gbs": rope_bytes / (rk["wf_rope_qk"] * 1e-3) / 1e9,
                "rope_qk_frac_hbm": rope_bytes / (rk["wf_rope_qk"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "rope_qk_fp64_ms": rk["wf_rope_qk_fp64"],
                "rope_qk_fp64_frac_hbm": rope_bytes / (rk["wf_rope_qk_fp64"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "vsa_ms_per_call_fused_rope": rk["wf_vsa_gather_rope"] + rk["wf_vsa_scores"] + rk["wf_vsa_topk"] + rk["wf_vsa_fine"],
                "gather_rope_ms": rk["wf_vsa_gather_rope"],
                "gather_plain_ms": rk["wf_vsa_gather"],
                "fused_rope_extra_ms": rk["wf_vsa_gather_rope"] - rk["wf_vsa_gather"],
                "kernel_ms": rk}
        del qr, kr

    # extra record (not part of the step): the softmax reference policies on the step's dense and
    # VSA fine kernels -- guarded integer reference (the default), running max, fixed first tile
    policies = None
    if not args.no_extra:
        wf.wf_vsa_coarse_topk(qv, kv, vv, grid, wv.topk, idx=idx, workspace=ws_v)
        pk = {}
        for mode, tag in ((1, "_running_max"), (2, "_fixed_first"), (0, "")):
            wf.wf_attn_dense(qd, kd, vd, out=od, workspace=ws_d, softmax_mode=mode)
            wf.wf_vsa_fine(ws_v, idx, (wv.B, wv.Hh, wv.N, wv.D), grid, out=ov, softmax_mode=mode)
            torch.cuda.synchronize()
            wf.profile_enable(True)
            for _ in range(3):
                wf.wf_attn_dense(qd, kd, vd, out=od, workspace=ws_d, softmax_mode=mode)
                for _ in range(4):
                    wf.wf_vsa_fine(ws_v, idx, (wv.B, wv.Hh, wv.N, wv.D), grid, out=ov, softmax_mode=mode)
            torch.cuda.synchronize()
            for name in ("wf_dense_fwd" + tag, "wf_vsa_fine" + tag):
                n, tot = wf.profile_query(name)
                pk[name] = tot / n
            wf.profile_enable(False)
        policies = {"kernel_ms": pk,
                    "dense_running_max_over_guarded": pk["wf_dense_fwd_running_max"] / pk["wf_dense_fwd"],
                    "dense_fixed_first_over_guarded": pk["wf_dense_fwd_fixed_first"] / pk["wf_dense_fwd"],
                    "vsa_fine_running_max_over_guarded": pk["wf_vsa_fine_running_max"] / pk["wf_vsa_fine"],
                    "vsa_fine_fixed_first_over_guarded": pk["wf_vsa_fine_fixed_first"] / pk["wf_vsa_fine"]}

    # extra record (not part of the step): sliding-tile attention on the two tuned grids, 40 heads,
    # 3x3x3 windows of 6x8x8-token tiles (own inputs; the step's tensors are unchanged)
    sta = None
    if not args.no_extra:
        sta = {}
        for name in ("sta_36x48x48", "sta_18x48x80"):
            ws_ = synth.WORKLOADS[name]
            qs_, ks2, vs2 = (to_dev(x) for x in synth.make_qkv(ws_))
            gs = (ws_.T, ws_.H, ws_.W)
            os2 = torch.empty((ws_.B, ws_.Hh, ws_.N, ws_.D), dtype=torch.float32, device=dev)
            wsb = torch.empty(wf.lib.wf_sta_workspace_bytes(ws_.B, ws_.Hh, *gs, ws_.D, *ws_.window),
                              dtype=torch.uint8, device=dev)
            wf.wf_sta(qs_, ks2, vs2, gs, ws_.window, out=os2, workspace=wsb)
            torch.cuda.synchronize()
            wf.profile_enable(True)
            for _ in range(5):
                wf.wf_sta(qs_, ks2, vs2, gs, ws_.window, out=os2, workspace=wsb)
            torch.cuda.synchronize()
            sk2 = {}
            for kname in ("wf_sta_gather", "wf_sta_plan", "wf_sta_fine"):
                n, tot = wf.profile_query(kname)
                sk2[kname] = tot / n
            wf.profile_enable(False)
            kk = ws_.window[0] * ws_.window[1] * ws_.window[2]
            tiles = (ws_.T // 6) * (ws_.H // 8) * (ws_.W // 8)
            fine_fl = 4.0 * ws_.B * ws_.Hh * ws_.N * 384 * kk * ws_.D   # every query against 384 kk keys
            ms = sum(sk2.values())
            dense_ms = dense_flops(ws_) / (dense_tf_step * 1e12) * 1e3  # dense at this shape, at the step's rate
            sta[name] = {"grid": list(gs), "heads": ws_.Hh, "tiles": tiles, "tile": [6, 8, 8],
                         "window_tiles": list(ws_.window), "key_tiles_per_query_tile": kk,
                         "density": kk / tiles, "ms_per_call": ms, "kernel_ms": sk2,
                         "fine_tflops": fine_fl / (sk2["wf_sta_fine"] * 1e-3) / 1e12,
                         "dense_equivalent_ms_at_step_rate": dense_ms,
                         "dense_equivalent_speedup": dense_ms / ms,
                         "ideal_speedup": tiles / kk}
            del qs_, ks2, vs2, os2, wsb

    # extra record (not part of the step): the 720p shape -- dense attention on the CFG pair at
    # 21x45x80 = 75,600 tokens and VSA top-64 of 1,440 cubes on the same tensors
    r720 = None
    if not args.no_extra:
        wd7, wv7 = synth.WORKLOADS["dense_720p_cfg"], synth.WORKLOADS["vsa_720p"]
        q7, k7, v7 = (to_dev(x) for x in synth.make_qkv(wv7))
        g7 = (wv7.T, wv7.H, wv7.W)
        C7 = wf.num_cubes(*g7)
        o7 = torch.empty((wv7.B, wv7.Hh, wv7.N, wv7.D), dtype=torch.float32, device=dev)
        wsd7 = torch.empty(wf.dense_workspace_bytes(wd7.B, wd7.Hh, wd7.N, wd7.D), dtype=torch.uint8, device=dev)
        wsv7 = torch.empty(wf.vsa_workspace_bytes(wv7.B, wv7.Hh, *g7, wv7.D), dtype=torch.uint8, device=dev)
        idx7 = torch.empty((wv7.B, wv7.Hh, C7, wv7.topk), dtype=torch.int32, device=dev)

        def run720():
            wf.wf_attn_dense(q7, k7, v7, out=o7, workspace=wsd7)
            wf.wf_vsa(q7, k7, v7, g7, wv7.topk, idx=idx7, out=o7, workspace=wsv7)

        run720()
        torch.cuda.synchronize()
        wf.profile_enable(True)
        for _ in range(3):
            run720()
        torch.cuda.synchronize()
        k7ms = {}
        for name in ("wf_transpose_v", "wf_dense_fwd", "wf_vsa_gather", "wf_vsa_scores", "wf_vsa_topk", "wf_vsa_fine"):
            n, tot = wf.profile_query(name)
            k7ms[name] = tot / n
        wf.profile_enable(False)
        d7 = k7ms["wf_transpose_v"] + k7ms["wf_dense_fwd"]
        v7ms = k7ms["wf_vsa_gather"] + k7ms["wf_vsa_scores"] + k7ms["wf_vsa_topk"] + k7ms["wf_vsa_fine"]
        f7 = vsa_flops(wv7, C7)
        r720 = {"grid": list(g7), "B": wv7.B, "heads": wv7.Hh, "tokens": wv7.N, "cubes": C7, "topk": wv7.topk,
                "dense_ms_per_call": d7,
                "dense_tflops_kernel": dense_flops(wd7) / (k7ms["wf_dense_fwd"] * 1e-3) / 1e12,
                "dense_frac_bf16_peak": dense_flops(wd7) / (k7ms["wf_dense_fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "vsa_ms_per_call": v7ms,
                "vsa_fine_tflops": f7["fine"] / (k7ms["wf_vsa_fine"] * 1e-3) / 1e12,
                "dense_equivalent_speedup": d7 / v7ms, "ideal_speedup": ideal_speedup(wv7, C7),
                "kernel_ms": k7ms}
        del q7, k7, v7, o7, wsd7, wsv7, idx7

    # extra record (not part of the step): one GPU's share of the heads when 8 GPUs split them
    # (5 of 40 per CFG branch): the same kernels at Hh = 5 and full N
    share = None
    if not args.no_extra:
        hs = wd.Hh // 8
        qs, ks_, vs_ = (x[:, :hs].contiguous() for x in (qd, kd, vd))
        os_ = torch.empty((wd.B, hs, wd.N, wd.D), dtype=torch.float32, device=dev)
        ws_s = torch.empty(wf.dense_workspace_bytes(wd.B, hs, wd.N, wd.D), dtype=torch.uint8, device=dev)
        qvs, kvs, vvs = (x[:, :hs].contiguous() for x in (qv, kv, vv))
        ovs = torch.empty((wv.B, hs, wv.N, wv.D), dtype=torch.float32, device=dev)
        idxs = torch.empty((wv.B, hs, C, wv.topk), dtype=torch.int32, device=dev)
        ws_vs = torch.empty(wf.vsa_workspace_bytes(wv.B, hs, wv.T, wv.H, wv.W, wv.D), dtype=torch.uint8, device=dev)

        def step_share():
            wf.wf_attn_dense(qs, ks_, vs_, out=os_, workspace=ws_s)
            wf.wf_vsa(qvs, kvs, vvs, grid, wv.topk, idx=idxs, out=ovs, workspace=ws_vs)

        for _ in range(3):
            step_share()
        torch.cuda.synchronize()
        wf.profile_enable(True)
        for _ in range(10):
            step_share()
        torch.cuda.synchronize()
        sk = {}
        for name in ("wf_transpose_v", "wf_dense_fwd", "wf_vsa_gather", "wf_vsa_scores", "wf_vsa_topk", "wf_vsa_fine"):
            n, tot = wf.profile_query(name)
            sk[name] = tot / n
        wf.profile_enable(False)
        sd = sk["wf_transpose_v"] + sk["wf_dense_fwd"]
        share = {"heads": hs, "of_gpus": 8,
                 "dense_ms_per_call": sd,
                 "dense_tflops_kernel": 4.0 * wd.B * hs * wd.N * wd.N * wd.D / (sk["wf_dense_fwd"] * 1e-3) / 1e12,
                 "vsa_ms_per_call": sk["wf_vsa_gather"] + sk["wf_vsa_scores"] + sk["wf_vsa_topk"] + sk["wf_vsa_fine"],
                 "kernel_ms": sk}

    fl_d = dense_flops(wd)
    fl_v = vsa_flops(wv, C)
    by_v = vsa_bytes(wv, C)
    ms_dense = kern["wf_transpose_v"] + kern["wf_dense_fwd"]
    ms_vsa = kern["wf_vsa_gather"] + kern["wf_vsa_scores"] + kern["wf_vsa_topk"] + kern["wf_vsa_fine"]
    dense_tf = fl_d / (kern["wf_dense_fwd"] * 1e-3) / 1e12
    # dense attention at the VSA call's own shape (B=1, 40 heads) is half the CFG-pair call
    ms_dense_same = ms_dense * wv.B / wd.B
    counters = measured_counters()
    out = {
        "metric": "attention TFLOP/s and ms/call at 32,760 tok x 40 heads x d128 (dense, VSA)",
        "value": (fl_d + fl_v["total"]) / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "dense MHA 2x40x32760xd128 (CFG pair, grid 21x30x52) + VSA 1x40 heads, "
                        "grid 21x30x52 -> 24x32x52, 624 cubes, top-32",
            "dense": {"B": wd.B, "heads": wd.Hh, "tokens": wd.N, "head_dim": wd.D},
            "vsa": {"B": wv.B, "heads": wv.Hh, "tokens": wv.N, "cubes": C, "topk": wv.topk,
                    "head_dim": wv.D},
            "inputs": "bf16 N(0,1) + 2*phi(t,h,w), seeded random Fourier features",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "wf_dense_fwd",
            "achieved": dense_tf,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": dense_tf / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic(),
        },
        "dense": {
            "profiled_clock_ghz": counters.get("clock_ghz"),
            "frac_peak_at_profiled_clock": (dense_tf / (PEAK_BF16_TFLOPS * counters["clock_ghz"] / PEAK_CLOCK_GHZ)
                                            if counters.get("clock_ghz") else None),
            "ms_per_call": ms_dense,
            "ms_per_call_median": med_dense,
            "kernel_ms": {"wf_transpose_v": kern["wf_transpose_v"], "wf_dense_fwd": kern["wf_dense_fwd"]},
            "tflops_call": fl_d / (ms_dense * 1e-3) / 1e12,
            "tflops_kernel": dense_tf,
            "frac_bf16_peak": dense_tf / PEAK_BF16_TFLOPS,
            "algorithmic_tflop": fl_d / 1e12,
        },
        "vsa": {
            "path": "one call (wf_vsa): the gather writes V^T and the cube means only, the fine stage reads Q and K "
                    "from the token grid",
            "ms_per_call": ms_vsa,
            "ms_per_call_median": med_vsa,
            "coarse_ms": kern["wf_vsa_gather"] + kern["wf_vsa_scores"] + kern["wf_vsa_topk"],
            "kernel_ms": {k: kern[k] for k in ("wf_vsa_gather", "wf_vsa_scores", "wf_vsa_topk", "wf_vsa_fine")},
            "fine_tflops": fl_v["fine"] / (kern["wf_vsa_fine"] * 1e-3) / 1e12,
            "fine_tflops_padded_queries": fl_v["fine"] * C * 64 / wv.N / (kern["wf_vsa_fine"] * 1e-3) / 1e12,
            "fine_frac_bf16_peak": fl_v["fine"] / (kern["wf_vsa_fine"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "gather_gbs": by_v["gather_one_call"] / (kern["wf_vsa_gather"] * 1e-3) / 1e9,
            "topk_gbs": by_v["topk"] / (kern["wf_vsa_topk"] * 1e-3) / 1e9,
            "gather_frac_hbm": by_v["gather_one_call"] / (kern["wf_vsa_gather"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "topk_frac_hbm": by_v["topk"] / (kern["wf_vsa_topk"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "scores_gbs": by_v["scores"] / (kern["wf_vsa_scores"] * 1e-3) / 1e9,
            "dense_equivalent_speedup": ms_dense_same / ms_vsa,
            "dense_equivalent_tflops": fl_d * wv.B / wd.B / (ms_vsa * 1e-3) / 1e12,
            "ideal_speedup": ideal_speedup(wv, C),
            "ideal_speedup_convention": IDEAL_CONVENTION,
        },
        "vsa_gated": None if gated_ms is None else {
            "topk": wv.topk,
            "ms_per_call": sum(gated_ms.values()),
            "kernel_ms": gated_ms,
            "coarse_out_gbs": by_v["coarse_out"] / (gated_ms["wf_vsa_coarse_out"] * 1e-3) / 1e9,
            "coarse_out_frac_hbm": by_v["coarse_out"] / (gated_ms["wf_vsa_coarse_out"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "merge_extra_ms": gated_ms["wf_vsa_fine_gated"] - plain_fine_ms,
            "merge_extra_floor_ms": by_v["merge"] / PEAK_HBM_GBS / 1e6,
        },
        "shape_720p": r720,
        "sta": sta,
        "rope": rope,
        "softmax_policies": policies,
        "vsa_two_calls": None if two_ms is None else {
            "topk": wv.topk,
            "ms_per_call": sum(two_ms.values()),
            "kernel_ms": two_ms,
            "gather_gbs": by_v["gather"] / (two_ms["wf_vsa_gather"] * 1e-3) / 1e9,
            "fine_tflops": fl_v["fine"] / (two_ms["wf_vsa_fine"] * 1e-3) / 1e12,
        },
        "vsa_k78": None if k78_ms is None else {
            "topk": k78,
            "ms_per_call": sum(k78_ms.values()),
            "kernel_ms": k78_ms,
            "fine_tflops_page_convention": 4.0 * wv.N * 64 * k78 * wv.D * wv.Hh / (k78_ms["wf_vsa_fine"] * 1e-3) / 1e12,
            "dense_equivalent_speedup": ms_dense_same / sum(k78_ms.values()),
            "ideal_speedup": ideal_speedup(synth.WORKLOADS["vsa_480p_k78"], C),
            "two_calls": {
                "ms_per_call": sum(k78_two_ms.values()),
                "kernel_ms": k78_two_ms,
                "fine_tflops_page_convention": (4.0 * wv.N * 64 * k78 * wv.D * wv.Hh
                                                / (k78_two_ms["wf_vsa_fine"] * 1e-3) / 1e12),
            },
        },
        "per_gpu_share": share,
        "context": {"pages_dense_ms_b200": 17.0,
                    "our_dense_ms_one_cfg_branch": ms_dense_same,
                    "pages_vsa_k78_ms_b200_persistent_cuda": 4.719},
        "wall_s_timed_region": wall,
        "device": torch.cuda.get_device_name(dev),
        "git": git_rev(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    if args.cpu_full:
        out["cpu_oracle_calls"] = cpu_oracle_calls()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
