#!/usr/bin/env python3
"""Throughput of the branch-attention hot path on one MI355X.

One step = one forward and one backward pass of the whole path over one batch:
main-sequence attention of every row over its causal main prefix, the
branch-local attention, the log-sum-exp merge, the backward preprocess, and the
main-sequence and branch-local backward passes. Default workload: one rank's
share of a 256K-token sequence in a 16-chunk zigzag layout (rank 3 of CP=8:
chunks 3 and 12 hold the queries, keys 0..212991), GQA 32q/8kv, head_dim 128,
EAGLE-3 TTT depth-7 branches on every local position, bf16, synthetic seeded
inputs already resident in HBM.

Prints one JSON line. value = algorithmic fwd+bwd TFLOP/s: 4*d*Hq and 10*d*Hq
flops per visible (row, key) pair for the forward and the backward.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3  # published fp32 vector peak
CLOCK_PEAK_MHZ = 2400.0  # the clock the peaks are quoted at
METRIC = "branch-attention fwd+bwd TFLOP/s and % bf16 MFMA peak, 256K-ctx 1-GPU share"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _sclk_path(pci=None):
    """sysfs file that lists the shader clock levels of this process's GPU, with
    the current one marked by '*': the PCI device of torch's device 0 when it
    is known, else the only AMD card with such a file; None otherwise."""
    import glob
    if pci is not None:
        p = "/sys/bus/pci/devices/%04x:%02x:%02x.0/pp_dpm_sclk" % pci
        return p if os.path.exists(p) else None
    found = []
    for dev in glob.glob("/sys/class/drm/card*/device"):
        try:
            with open(os.path.join(dev, "vendor")) as f:
                if f.read().strip() != "0x1002":
                    continue
        except OSError:
            continue
        if os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
            found.append(os.path.realpath(os.path.join(dev, "pp_dpm_sclk")))
    found = sorted(set(found))
    return found[0] if len(found) == 1 else None


def parse_sclk(text):
    """Current shader clock in MHz from the text of pp_dpm_sclk (the line marked
    '*', e.g. '1: 1900Mhz *'), or None."""
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            tok = line.split(":", 1)[-1].strip().rstrip("*").strip().lower()
            if tok.endswith("mhz"):
                try:
                    return float(tok[:-3])
                except ValueError:
                    return None
    return None


class ClockSampler:
    """Shader clock during the timed steps, read in this process from sysfs
    (pp_dpm_sclk of the GPU, polled every 0.2 s by a thread; no tool is
    started): the mean of the samples above 1 GHz, or None when the file is
    not there or not readable, or when disabled."""

    def __init__(self, enabled=True, pci=None):
        import threading
        self.path = _sclk_path(pci) if enabled else None
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self.stop.is_set():
            try:
                with open(self.path) as f:
                    v = parse_sclk(f.read())
            except OSError:
                return
            if v is not None and v > 1000.0:
                self.samples.append(v)
            self.stop.wait(0.2)

    def __enter__(self):
        if self.path:
            self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        if self.thread.is_alive():
            self.thread.join(timeout=30)

    def mhz(self):
        return round(sum(self.samples) / len(self.samples), 1) if self.samples else None


def kernel_source_hash(names):
    """Hash of the code of the kernel's sources: line comments, trailing blanks
    and empty lines are left out, so an edit of comments alone keeps it."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "speculative_draft_branch_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update((code + "\n").encode())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"main_fwd": ["main_fwd.hip", "common.hpp", "plan.hpp"],
                  "main_bwd_dq": ["main_bwd.hip", "common.hpp", "plan.hpp"],
                  "main_bwd_dkdv": ["main_bwd.hip", "common.hpp", "plan.hpp"]}


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
        if d.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kernel]):
            return None
        return float(d["hbm_bytes_per_launch"])
    except Exception:
        return None


def row_pairs(w, rows):
    """Visible keys of each combined row (main prefix plus own branch keys)."""
    import numpy as np
    out = []
    for r in rows:
        if r < w.Nq:
            t = int(w.q_pos[r])
            s = int(np.searchsorted(w.cu_seqlens, t, side="right") - 1)
            out.append(t - int(w.cu_seqlens[s]) + 1)
        else:
            b = r - w.Nq
            m = int(np.searchsorted(w.cu_branch, b, side="right") - 1)
            a = int(w.anchors[m])
            s = int(np.searchsorted(w.cu_seqlens, a, side="right") - 1)
            L = int(w.cu_branch[m + 1] - w.cu_branch[m])
            j = b - int(w.cu_branch[m]) + 1
            out.append(a - int(w.cu_seqlens[s]) + 1 + (L if w.modes[m] == 1 else j))
    return out


def stratified_rows(w, n=512, seed=0):
    """A seeded sample of n combined rows in four strata, interleaved so that
    every prefix of the list is itself stratified: (1) the first and last main
    rows of each sequence and of each contiguous run of query positions (the
    chunks of a zigzag share); (2) the branch rows of anchors at sequence
    starts and at the starts of those runs; (3) depth 1 and the deepest row of
    the first and last anchor of each sequence and of random anchors; (4)
    uniformly drawn rows."""
    import numpy as np
    rng = np.random.default_rng(seed)
    R = w.Nq + w.Rb
    s1, s2, s3 = [], [], []
    qp = w.q_pos.astype(np.int64)
    for s in range(w.num_seqs):
        lo, hi = int(w.cu_seqlens[s]), int(w.cu_seqlens[s + 1])
        q0, q1 = (int(x) for x in np.searchsorted(qp, [lo, hi]))
        run_starts = {lo}
        if q1 > q0:
            run = qp[q0:q1]
            breaks = np.nonzero(np.diff(run) != 1)[0]
            starts = np.concatenate([[0], breaks + 1])
            ends = np.concatenate([breaks, [len(run) - 1]])
            for a, b in zip(starts, ends):
                s1 += [q0 + int(a), q0 + int(b)]
                run_starts.add(int(run[a]))
        m0, m1 = (int(x) for x in np.searchsorted(w.anchors, [lo, hi]))
        for pos in sorted(run_starts):
            m = int(np.searchsorted(w.anchors, pos))
            if m < w.A and int(w.anchors[m]) == pos:
                s2 += list(range(w.Nq + int(w.cu_branch[m]), w.Nq + int(w.cu_branch[m + 1])))
        if m1 > m0:
            for m in {m0, m1 - 1}:
                b0, b1 = int(w.cu_branch[m]), int(w.cu_branch[m + 1])
                if b1 > b0:
                    s3 += [w.Nq + b0, w.Nq + b1 - 1]
    if w.A:
        for m in rng.integers(0, w.A, size=64):
            b0, b1 = int(w.cu_branch[m]), int(w.cu_branch[m + 1])
            if b1 > b0:
                s3 += [w.Nq + b0, w.Nq + b1 - 1]
    s4 = [int(x) for x in rng.integers(0, R, size=4 * n)]
    strata = [list(dict.fromkeys(x)) for x in (s1, s2, s3, s4)]
    out, seen, i = [], set(), 0
    while len(out) < min(n, R) and any(i < len(x) for x in strata):
        for x in strata:
            if i < len(x) and x[i] not in seen and len(out) < n:
                seen.add(x[i])
                out.append(x[i])
        i += 1
    return out


def cpu_info():
    """Host facts recorded with the CPU baseline: core counts, CPU model and the
    BLAS that numpy uses."""
    import numpy as np
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name')} {b.get('version')}".strip()
    except Exception:
        pass
    threads = 0
    try:
        from threadpoolctl import threadpool_info
        for x in threadpool_info():
            if x.get("user_api") == "blas":
                threads = max(threads, int(x.get("num_threads", 0)))
                blas = f"{blas} ({x.get('internal_api')}, {x.get('num_threads')} threads)"
    except Exception:
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count(),
            "blas_threads": threads or None, "cpu_model": model, "blas": blas}


def cpu_baseline(w, t, seconds, downscaled=()):
    """The CPU oracle as it stands, timed on the machine's host cores: forward and
    backward of a bounded prefix of a stratified 512-row sample of the same
    workload (all heads), extrapolated to the whole problem by visible-pair
    count; then, if given, the full dense oracle on downscaled versions of the
    workloads."""
    import numpy as np
    import oracle
    import workloads as W
    from workloads.inputs import make_inputs, to_f32

    class View:
        def __init__(self, a):
            self.a, self.shape = a, a.shape

        def __getitem__(self, i):
            return to_f32(self.a[i])

    info = cpu_info()
    cores = info["blas_threads"] or info["affinity_cores"]
    p = oracle.Problem.from_workload(w)
    tv = {k: View(v) for k, v in t.items()}
    hm = oracle.branch_attention._HeadMajor(p, tv, np.float64)   # one-time layout copy, not timed
    acc = {"dk": np.zeros((w.N, w.num_kv_heads, w.head_dim)), "dv": np.zeros((w.N, w.num_kv_heads, w.head_dim)),
           "dkb": np.zeros((w.Rb, w.num_kv_heads, w.head_dim)), "dvb": np.zeros((w.Rb, w.num_kv_heads, w.head_dim))}
    sample = stratified_rows(w, 512)
    done, t0 = [], time.perf_counter()
    for r in sample:
        if done and time.perf_counter() - t0 >= seconds:
            break
        oracle.forward_rows(p, tv, [r], _hm=hm)
        oracle.backward_rows(p, tv, [r], acc, _hm=hm)
        done.append(r)
    el = time.perf_counter() - t0
    n_pairs = sum(row_pairs(w, done))
    full_pairs = sum(oracle.pair_counts(p).values())
    fl = (4 + 10) * w.head_dim * w.num_q_heads
    extrap_s = el * full_pairs / n_pairs
    res = {"value": n_pairs * fl / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": (f"first {len(done)} rows of a seeded stratified sample of 512 rows (sequence and chunk "
                      f"ends, anchors at sequence starts, depth 1 and deepest branch rows, uniform rows) of "
                      f"{w.name}, all {w.num_q_heads} heads: fp64 numpy forward + backward of each row over its "
                      f"{n_pairs} visible row-key pairs in {el:.1f} s, extrapolated by pair count"),
           "seconds": round(el, 2),
           "extrapolated CPU time (%d cores)" % cores: round(extrap_s, 1),
           "extrapolated_cpu_s": round(extrap_s, 1),
           "rows_timed": len(done), "pairs_timed": n_pairs, "pairs_full": full_pairs,
           "host": info, "downscaled": []}
    for name in downscaled:
        wd = W.get(name)
        td = {k: to_f32(v).astype(np.float64) for k, v in make_inputs(wd, grads=True).items()}
        pd = oracle.Problem.from_workload(wd)
        t1 = time.perf_counter()
        f = oracle.forward(pd, td)
        t2 = time.perf_counter()
        oracle.backward(pd, td, f)
        t3 = time.perf_counter()
        pairs = sum(oracle.pair_counts(pd).values())
        res["downscaled"].append({"workload": wd.name, "fwd_s": round(t2 - t1, 2), "bwd_s": round(t3 - t2, 2),
                                  "tflops": round((4 + 10) * wd.head_dim * wd.num_q_heads * pairs / (t3 - t1) / 1e12,
                                                  5),
                                  "what": "full dense fp64 oracle forward + backward"})
        log(f"cpu downscaled {wd.name}: fwd {t2 - t1:.1f} s, bwd {t3 - t2:.1f} s")
    return res


def hbm_kernels(w, kern):
    """HBM-bound kernels (bf16): algorithmic bytes per launch and the rate
    against the 8 TB/s peak. Branch-local backward (dK, dV of the branch keys),
    per (branch row, q head): Q, dO 4d, LSE and D 8; per (branch row, kv head):
    K, V in and dK, dV out 8d. (The backward preprocess -- D and the staged
    query tiles -- runs inside the dq kernel.)"""
    rb, hq, hkv, d = w.Rb, w.num_q_heads, w.num_kv_heads, w.head_dim
    byt = {"branch_local_bwd": rb * hq * (4 * d + 8) + rb * hkv * 8 * d}
    out = {}
    for k, b in byt.items():
        if k in kern and kern[k][1]:
            ms = kern[k][0] / kern[k][1]
            gbs = b / (ms * 1e-3) / 1e9
            out[k] = {"ms": round(ms, 3), "bytes": b, "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def ring_sim(sda, plan, g, w, stream, kern):
    """The main-key forward as rank 3 of a CP=8 zigzag ring computes it: the 16
    chunks arrive in ring order (pair r, 15-r from rank r), each from its own K/V
    buffer, through ba_ring_step_fwd into one running (O, LSE). Chunks 13-15 lie
    past the rank's last key and arrive empty. Untimed: the chunk copies and one
    warmup pass. Compared with the single pass (V transpose + main forward)."""
    import torch
    chunk = w.N // 13
    wins = []
    for s in range(8):
        r = (3 - s) % 8
        for c in (r, 15 - r):
            wins.append((min(c * chunk, w.N), min((c + 1) * chunk, w.N)))
    bufs = [(g["k"][lo:hi].clone(), g["v"][lo:hi].clone()) for lo, hi in wins]
    R = w.Nq + w.Rb
    o_run = torch.empty((R, w.num_q_heads, w.head_dim), dtype=torch.float32, device=g["q"].device)
    lse_run = torch.empty((w.num_q_heads, R), dtype=torch.float32, device=g["q"].device)
    ws = sda.workspace(plan, 2, g["q"].device)

    def run():
        o_run.zero_()
        lse_run.fill_(float("-inf"))
        for (lo, hi), (kw, vw) in zip(wins, bufs):
            sda.ba_ring_step_fwd(plan, g["q"], g["qb"], kw, vw, lo, hi, o_run, lse_run, ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    single = (kern["main_fwd"][0] + kern["vt_transpose"][0]) / max(1, kern["main_fwd"][1])
    log(f"ring simulation: {len(wins)} windows in {ms:.1f} ms (single pass {single:.1f} ms)")
    del bufs, o_run, lse_run, ws
    return {"windows": len(wins), "nonempty": sum(hi > lo for lo, hi in wins), "ms": round(ms, 3),
            "single_pass_ms": round(single, 3), "ratio": round(ms / single, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="ctx256k_rank3")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cpu-downscaled", action="store_true",
                    help="skip the full dense oracle on the downscaled workloads (part of the CPU baseline)")
    ap.add_argument("--kernel-steps", type=int, default=2,
                    help="steps of the separate pass, after the timed steps, that times each kernel launch "
                         "with HIP events (per-kernel split and roofline)")
    ap.add_argument("--no-ring-sim", action="store_true",
                    help="skip the ring-step simulation measured after the timed steps")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the shader clock (sysfs) during the timed steps")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the warmup, copy a buffer of this many MiB once (a plain copy kernel of known "
                         "size, for scaling hardware byte counters); not part of the timed region")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the path runs one GPU's share; "
                                   "run with --gpus 1", "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import speculative_draft_branch_amd as sda
    import workloads as W
    from workloads.inputs import make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = W.get(args.workload)
    log(f"workload {w.name}: N={w.N} Nq={w.Nq} Rb={w.Rb} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim}")
    t_gen = time.time()
    t = make_inputs(w, grads=True)
    log(f"inputs generated in {time.time() - t_gen:.1f} s")
    if w.dtype == "bf16":
        g = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda() for k, v in t.items()}
    else:
        g = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in t.items()}
    t_plan = time.time()
    plan = sda.Plan.from_workload(w)
    log(f"plan built in {time.time() - t_plan:.2f} s: {plan.n_qtiles} query tiles, {plan.n_ktiles} key tiles")
    dev = g["q"].device
    hq, d = w.num_q_heads, w.head_dim
    o, ob = torch.empty_like(g["q"]), torch.empty_like(g["qb"])
    lse = torch.empty((hq, w.Nq), dtype=torch.float32, device=dev)
    lseb = torch.empty((hq, w.Rb), dtype=torch.float32, device=dev)
    gr = [torch.empty_like(g[k]) for k in ("q", "k", "v", "qb", "kb", "vb")]
    ws_f, ws_b = sda.workspace(plan, 0, dev), sda.workspace(plan, 1, dev)
    stream = torch.cuda.current_stream()

    def step():
        sda.branch_attn_fwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"], o, lse, ob, lseb, ws_f)
        sda.branch_attn_bwd(plan, g["q"], g["k"], g["v"], g["qb"], g["kb"], g["vb"], o, lse, ob, lseb,
                            g["do"], g["dob"], *gr, ws_b)

    if args.calibration_copy_mib > 0:
        n = args.calibration_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {args.calibration_copy_mib} MiB done")
        del src, dst

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i} done")
    # Timed region: exactly `steps` steps, one event between consecutive steps on
    # the launch stream, the library's per-launch timing off.
    props = torch.cuda.get_device_properties(dev)
    pci = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id) if hasattr(props, "pci_bus_id") else None
    sda.timing_enable(False)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler(enabled=not args.no_clock, pci=pci) as clk:
        ev[0].record(stream)
        for i in range(args.steps):
            step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    clock_mhz = clk.mhz()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = float(np.median(per_step))
    total_ms = ev[0].elapsed_time(ev[-1])
    log(f"timed {args.steps} steps: median {ms:.1f} ms/step, total {total_ms:.1f} ms, clock {clock_mhz} MHz")
    # Per-kernel split: a separate pass of the same steps with every launch
    # bracketed by HIP events on the launch stream.
    sda.timing_reset()
    sda.timing_enable(True)
    for i in range(max(1, args.kernel_steps)):
        step()
    torch.cuda.synchronize()
    sda.timing_enable(False)
    kern = sda.timing_read()
    nks = max(1, args.kernel_steps)

    pairs = sum(plan.pairs)
    flops_fwd, flops_bwd = plan.flops_fwd(), plan.flops_bwd()
    value = (flops_fwd + flops_bwd) / (ms * 1e-3) / 1e12
    fwd_kernels = ("metadata_upload", "vt_transpose", "vbt_transpose", "main_fwd", "branch_local_fwd", "lse_merge")
    fwd_ms = sum(kern[k][0] for k in fwd_kernels if k in kern) / nks
    bwd_ms = sum(v[0] for k, v in kern.items() if k not in fwd_kernels) / nks
    main_pairs = plan.pairs[0] + plan.pairs[1]
    # contraction flops each kernel must do per visible (row, key) pair and q head:
    # forward QK^T + PV (4d); dq kernel QK^T, dO V^T, dS K (6d); dkdv kernel
    # QK^T, dO V^T, P^T dO, dS^T Q (8d)
    algo = {"main_fwd": 4 * d * hq * main_pairs, "main_bwd_dq": 6 * d * hq * main_pairs,
            "main_bwd_dkdv": 8 * d * hq * main_pairs}
    peak, bound = PEAK_BF16_TFLOPS, "mfma"
    if w.dtype != "bf16":  # float32: plain vector kernels, one backward kernel does dQ, dK and dV (10d)
        algo = {"main_fwd": 4 * d * hq * main_pairs, "main_bwd_dkdv": 10 * d * hq * main_pairs}
        peak, bound = PEAK_FP32_TFLOPS, "alu"
    dominant = max(algo, key=lambda k: kern[k][0])
    dom_ms = kern[dominant][0] / max(1, kern[dominant][1])
    achieved = algo[dominant] / (dom_ms * 1e-3) / 1e12
    traffic = traffic_from_profile(dominant, w.name)
    fwd_main_ms = kern["main_fwd"][0] / max(1, kern["main_fwd"][1])
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_per_step_steps": [round(x, 3) for x in per_step],
        "ms_total_timed": round(total_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "tokens_total": 16 * 16384 if w.name == "ctx256k_rank3" else w.N,
                   "main_keys": w.N, "main_query_rows": w.Nq, "branch_rows": w.Rb,
                   "q_heads": hq, "kv_heads": w.num_kv_heads, "head_dim": d,
                   "description": w.description},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        # fwd_ms, bwd_ms and the per-kernel figures come from the separate
        # kernel pass (kernel_steps steps, per-launch events)
        "kernel_steps": nks,
        "fwd_ms": round(fwd_ms, 3),
        "bwd_ms": round(bwd_ms, 3),
        "fwd_tflops": round(flops_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_tflops": round(flops_bwd / (bwd_ms * 1e-3) / 1e12, 2),
        "main_fwd_frac_peak": round(4 * d * hq * main_pairs / (fwd_main_ms * 1e-3) / 1e12 / peak, 4),
        "kernels_ms_per_launch": {k: round(v[0] / max(1, v[1]), 3) for k, v in kern.items() if v[1]},
        "roofline": {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic},
        # shader clock while the steps ran, and the dominant kernel's fraction of
        # the peak scaled to that clock (the peak assumes 2.4 GHz)
        "clock_mhz": clock_mhz,
        "frac_at_clock": (round(achieved / (peak * clock_mhz / CLOCK_PEAK_MHZ), 4) if clock_mhz else None),
        "hbm_bound_kernels": hbm_kernels(w, kern) if w.dtype == "bf16" else None,
        "cpu_baseline": None,
    }
    if not args.no_ring_sim and w.name == "ctx256k_rank3":
        res["ring_sim"] = ring_sim(sda, plan, g, w, stream, kern)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on stratified sampled rows for ~{args.cpu_seconds:.0f} s")
        down = () if args.no_cpu_downscaled or w.name != "ctx256k_rank3" else ("ctx256k_rank3_chunk256",
                                                                                 "qwen3_8b_16k_div16")
        del g, gr, ws_f, ws_b, o, ob, lse, lseb
        res["cpu_baseline"] = cpu_baseline(w, t, args.cpu_seconds, down)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
