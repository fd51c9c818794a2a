#!/usr/bin/env python3
"""Throughput of batched lossless draft verification on one MI355X.

A step is one spec_verify call over the block-diffusion workload: B=64 requests,
gamma=15 draft positions, V=129280, bf16 target logits, T=1 (every request
verifies all 15 drafts, so a step verifies 960 draft positions).  Inputs are
seeded synthetic arrays resident in HBM before the timed region; several
independent copies rotate so that HBM, not the 256 MB last-level cache, serves
the reads.  After the W warm-up steps, K calls are timed cold; the step then
runs for --settle-ms of wall time (the device's steady operating point), and
the K calls timed after that give the reported value.  Prints one JSON line,
with the roofline of the whole call, the cold figure and the float64 oracle
timed on host cores beside it.

    python bench.py [--steps K] [--warmup W] [--settle-ms MS] [--gpus 1] [--workload NAME] [--no-cpu-baseline]
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

import workloads as W  # noqa: E402

PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
CSRC = os.path.join(ROOT, "lossless_draft_verification_verify_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "verify_kernels.hip")
# rocprofv3 counter summaries of each workload's dominant kernel, and the
# source file that kernel is built from
TRAFFIC_FILES = {
    "block": (os.path.join(ROOT, "profiles", "k_verify_sampled_block_traffic.md"), KERNEL_SRC),
    "greedy": (os.path.join(ROOT, "profiles", "k_verify_greedy_traffic.md"), KERNEL_SRC),
    "logits": (os.path.join(ROOT, "profiles", "k_rows_sampled_logits_traffic.md"), KERNEL_SRC),
    "acceptance": (os.path.join(ROOT, "profiles", "k_acceptance_traffic.md"),
                   os.path.join(CSRC, "acceptance_kernel.hip")),
}


def algorithmic_bytes(B, G, V, lens, n_rej, esize=2):
    """Bytes the method must move per call: every read target row once, one
    fp32 draft row per rejecting request, the per-position gathers (token id,
    q(x), uniform) and the per-request final uniform and outputs."""
    lens = np.asarray(lens, np.int64)
    rows = int((lens + 1).sum())
    return rows * V * esize + n_rej * V * 4 + int(lens.sum()) * 12 + B * (4 + 4 + 4 * (G + 1))


def row_pass_bytes(V, lens, esize=2):
    """Algorithmic bytes of the row pass (the dominant kernel): one target row
    of V * esize bytes per read row (sum of len_b + 1 rows), plus the token id
    and q(x_k) it gathers per verified position."""
    lens = np.asarray(lens, np.int64)
    return int((lens + 1).sum()) * V * esize + int(lens.sum()) * 8


def kernel_sha(src=KERNEL_SRC):
    """Hash of a kernel source's code: comments and blank lines removed, so
    that only a change to the code itself makes recorded counters stale."""
    import re
    with open(src) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(line.rstrip() for line in src.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload="block"):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, scaled by a
    plain copy of known size), if they were taken on the current kernel
    source; else None."""
    if workload not in TRAFFIC_FILES:
        return None
    path, src = TRAFFIC_FILES[workload]
    try:
        with open(path) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        key, sep, val = line.strip().partition(": ")
        if sep and key in ("kernel_sha", "kernel", "bytes_per_launch"):
            kv[key] = val.strip()
    if kv.get("kernel_sha") != kernel_sha(src) or "bytes_per_launch" not in kv:
        return None
    return int(kv["bytes_per_launch"])


class HipEvents:
    """Timing events created directly in the HIP runtime torch loaded, with the
    system-scope fence disabled: a record is then a device-scope marker and does
    not write back the L2 to host-coherent memory, so it adds less delay."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")          # already loaded by torch: the same runtime
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(h.value)

    def record(self, i, stream):
        if self.hip.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i, j):
        t = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(t), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return t.value

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


_CPU = {}


def _cpu_job(part):
    lo, hi = part
    t0 = time.perf_counter()
    units = _CPU["fn"](lo, hi)
    return time.perf_counter() - t0, units


def cpu_baseline(fn, n_items, unit, what, budget_s=12.0, max_workers=16):
    """Time the float64 oracle, as it stands, on host cores.

    fn(lo, hi) runs the oracle on items [lo, hi) of the workload (requests, or
    sample chunks) and returns the units of work done (verified positions,
    ...).  First one core runs slices in turn for about 2 s (the 1-core
    figure); then a fork pool of min(max_workers, affinity cores) workers runs
    slices that cover the workload, repeated to about budget_s seconds of
    summed worker time.  Must run before anything initialises the GPU."""
    import multiprocessing as mp
    _CPU["fn"] = fn
    per = max(1, n_items // 16)
    slices = [(lo, min(n_items, lo + per)) for lo in range(0, n_items, per)]
    t0 = time.perf_counter()
    units1, done = 0, 0
    while True:
        lo, hi = slices[done % len(slices)]
        units1 += fn(lo, hi)
        done += 1
        if time.perf_counter() - t0 >= 2.0:
            break
    t1 = time.perf_counter() - t0
    affinity = len(os.sched_getaffinity(0))
    workers = min(max_workers, affinity)
    nparts = max(workers, int(round(budget_s / (t1 / done))))
    parts = [slices[k % len(slices)] for k in range(nparts)]
    ctx = mp.get_context("fork")                 # before any GPU initialisation
    t0 = time.perf_counter()
    with ctx.Pool(processes=workers) as pool:
        res = pool.map(_cpu_job, parts, chunksize=1)
    wall = time.perf_counter() - t0
    units = sum(u for _, u in res)
    return {"value": round(units / wall, 2), "unit": unit, "cores": workers, "kind": "oracle",
            "one_core_value": round(units1 / t1, 2), "affinity_cores": affinity,
            "sample": f"{what}: {len(parts)} slices of up to {per} of {n_items} items over a {workers}-process "
                      f"fork pool, wall {wall:.2f} s, summed worker time {sum(t for t, _ in res):.2f} s; "
                      f"one core: {done} slices in {t1:.2f} s"}


def oracle_fn(kind, w, lens=None):
    """The oracle's work for requests [lo, hi) of workload w, and its unit count."""
    import oracle
    T = np.float32(w.get("T", 0.0))
    G = w.get("G", 0)
    if kind in ("block", "tiny", "mtp", "greedy"):
        def fn(lo, hi):
            oracle.verify(w["logits"][lo:hi], w.get("draft_probs")[lo:hi] if w.get("draft_probs") is not None
                          else None, w["draft_tokens"][lo:hi],
                          None if w.get("uniforms") is None else w["uniforms"][lo:hi], T)
            return (hi - lo) * G
        return fn
    if kind in ("scheduled", "static", "dcut"):
        def fn(lo, hi):
            if lo == 0:                           # the batch-wide length choice, once per pass over the batch
                if kind == "scheduled":
                    oracle.schedule(w["confidence"], w["cost_table"], w["budget"])
                elif kind == "static":
                    from oracle import calibration as C
                    C.static_threshold(w["confidence"], 0.5)
                else:
                    from oracle import dcut as OD
                    OD.dcut(w["confidence"], w["ratios"], w["ratio_cost"])
            oracle.verify(w["logits"][lo:hi], w["draft_probs"][lo:hi], w["draft_tokens"][lo:hi],
                          w["uniforms"][lo:hi], T, lens[lo:hi])
            return int(np.sum(lens[lo:hi]))
        return fn
    if kind == "logits":
        from oracle import acceptance as OA

        def fn(lo, hi):
            OA.verify_logits(w["logits"][lo:hi], w["draft_logits"][lo:hi], w["draft_tokens"][lo:hi],
                             w["uniforms"][lo:hi], T)
            return (hi - lo) * G
        return fn
    if kind == "acceptance":
        from oracle import acceptance as OA

        def fn(lo, hi):
            OA.acceptance(w["logits"][lo:hi], w["draft_logits"][lo:hi], T, draft_is_logits=True)
            return (hi - lo) * G
        return fn
    if kind == "tree":
        from oracle import tree as OT

        def fn(lo, hi):
            OT.tree_verify_greedy(w["logits"][lo:hi], w["parents"][lo:hi], w["node_tokens"][lo:hi])
            return (hi - lo) * (w["M"] - 1)
        return fn
    raise ValueError(kind)


def sts_fit_bench(args):
    """spec_sts_fit on the calibration recipe: 2^20 samples x 15 positions,
    the 100-point grid linspace(0.1, 10, 100), 15 bins (3 launches per position)."""
    N, G = 1 << 20, 15
    conf, L, _ = W.calibration(N, G=G)
    temps = [float(np.float32(t)) for t in np.linspace(0.1, 10.0, 100)]
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import calibration as C
        chunk = 1 << 12

        def fn(lo, hi):
            C.sts_fit(conf[lo * chunk:hi * chunk], L[lo * chunk:hi * chunk], temps)
            return (hi - lo) * chunk * G
        cpu = cpu_baseline(fn, N // chunk, "sample-positions/s",
                           f"the float64 oracle's fit on chunks of {chunk} of the {N} samples (all {G} positions, "
                           "the same grid and bins)")
    import torch
    import lossless_draft_verification_verify_amd as sv
    sv.load()
    dev = torch.device("cuda:0")
    c, l = torch.from_numpy(conf).to(dev), torch.from_numpy(L).to(dev)
    for _ in range(args.warmup):
        sv.sts_fit(c, l, temps)
    torch.cuda.synchronize()
    K = max(1, min(args.steps, 20))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        sv.sts_fit(c, l, temps)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    evals = N * G * len(temps)
    # ALU peak of the accumulate kernel's inner step: one fp64 exp2 per grid evaluation is
    # the costliest op; the chip's fp64 vector rate is 78.6 TFLOP/s and an fp64 exp2 is about
    # 20 fp64 operations, so at most ~3.9 T evaluations/s.
    alu_peak = 78.6e12 / 20 / 1e9
    print(json.dumps({
        "metric": "STS fit: sample-positions per second", "value": round(N * G / (ms * 1e-3), 1),
        "unit": "sample-positions/s", "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"Sequential Temperature Scaling fit: N={N} samples, G={G} positions, "
                               "100-point grid, 15 bins, 45 launches", "N": N, "G": G, "grid": len(temps)},
        "roofline": {"bound": "alu", "achieved": round(evals / (ms * 1e-3) / 1e9, 3), "unit": "G grid evaluations/s",
                     "peak": round(alu_peak, 1), "frac": round(evals / (ms * 1e-3) / 1e9 / alu_peak, 4),
                     "traffic": None,
                     "peak_derivation": "fp64 vector peak 78.6 TFLOP/s / ~20 fp64 operations per exp2 evaluation",
                     "kernel": "k_fit_accumulate (one fp64 exp2, a bin and three LDS atomics per sample, position "
                               "and grid point)"},
        "cpu_baseline": cpu}), flush=True)


def tree_bench(args):
    """spec_verify_tree on the layered 64-node tree: B=8, V=152064, bf16 (512 node rows per call, the bytes of
    the greedy workload).  Rotating input copies; HIP events around each call."""
    w = W.tree()
    B, M, V = w["B"], w["M"], w["V"]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(oracle_fn("tree", w), B, "verified candidate nodes/s",
                           f"the float64 oracle's greedy tree walk on the {B} requests of the same workload")
    import torch
    import lossless_draft_verification_verify_amd as sv
    sv.load()
    dev = torch.device("cuda:0")
    z0 = torch.from_numpy(w["logits"].view(np.int16)).to(dev).view(torch.bfloat16)
    par = torch.from_numpy(w["parents"]).to(dev)
    tok = torch.from_numpy(w["node_tokens"]).to(dev)
    sets = [z0] + [z0.clone() for _ in range(args.sets - 1)]
    acc = None
    for i in range(args.warmup):
        acc, _, _ = sv.verify_tree(sets[i % len(sets)], par, tok)
    torch.cuda.synchronize()
    K = args.steps
    stream = torch.cuda.current_stream(dev)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        acc, _, _ = sv.verify_tree(sets[i % len(sets)], par, tok)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / K
    a = acc.cpu().numpy()
    algo = B * M * V * 2 + B * M * 8 + B * (4 + 8 * M)
    nodes = B * (M - 1)
    print(json.dumps({
        "metric": "verified draft positions/sec and achieved HBM GB/s (% peak), B=64 gamma=15 V=129k",
        "value": round(nodes / (ms_step * 1e-3), 1), "unit": "verified candidate nodes/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"greedy tree verification: B={B} requests, a {M}-node layered candidate tree "
                               f"(8/16/24/15 nodes per level), V={V}, bf16 logits N(0,4), T=0",
                   "B": B, "nodes": M, "V": V, "rotating_sets": len(sets), "mean_accepted": float(a.mean())},
        "roofline": {"bound": "hbm", "achieved": round(algo / (ms_step * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(algo / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": None,
                     "kernel": "whole spec_verify_tree call: k_verify_greedy row workgroups over every node row, "
                               "then k_tree_walk",
                     "algorithmic_bytes_per_launch": algo, "launch_ms_mean": round(ms_step, 5)},
        "cpu_baseline": cpu}), flush=True)


def acceptance_stats(acc, lens):
    """Mean accepted drafts, mean tokens per request (accepted + 1), and the
    acceptance rate at each draft position: the share of the requests that
    reached and verified position k whose draft k was accepted."""
    acc, lens = np.asarray(acc, np.int64), np.asarray(lens, np.int64)
    ok = acc >= 0
    acc, lens = acc[ok], lens[ok]
    rate = []
    for k in range(int(lens.max()) if lens.size else 0):
        tested = (acc >= k) & (lens > k)
        rate.append(round(float((acc[tested] > k).mean()), 4) if tested.any() else None)
    return {"mean_accepted": round(float(acc.mean()), 4), "mean_tokens_per_request": round(float((acc + 1).mean()), 4),
            "acceptance_by_position": rate}


DESCRIPTIONS = {
    "block": ("block-diffusion draft verification: B=64, gamma=15, V=129280, bf16 logits "
              "(Zipf(1.1) over a per-row permutation), fp32 draft probabilities, T=1"),
    "tiny": "tiny verification: B=4, gamma=4, V=1024, fp32 logits N(0,2), fp32 draft probabilities, T=1",
    "mtp": ("MTP-style short drafts: B=16, gamma=3, V=32000, bf16 logits N(0,3) with a 1-in-8 peaked token (+8), "
            "fp32 draft probabilities, T=0.7"),
    "greedy": "greedy draft verification: B=64, gamma=7, V=152064, bf16 logits N(0,4), T=0",
    "logits": ("draft-logits verification: B=64, gamma=15, V=129280, bf16 target logits (Zipf(1.1) over a "
               "per-row permutation) and bf16 draft logits, q = softmax(draft logits / T) on the device, T=1"),
    "acceptance": ("acceptance diagnostics: alpha = sum min(p, q) per position, B=64, gamma=15, V=129280, bf16 target "
                   "and draft logits, T=1 (two passes over each row pair)"),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The first 10-30 ms of calls after start run up to 10% slower (the chip's
    # clocks and caches settling), so the defaults warm up for about 11 ms.
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="wall time the step runs between the cold timing and the timed calls")
    ap.add_argument("--sets", type=int, default=4, help="independent input copies rotated in HBM")
    ap.add_argument("--workload", choices=("block", "tiny", "mtp", "greedy", "scheduled", "dcut", "logits",
                                           "acceptance", "static", "sts_fit", "tree"),
                    default="block",
                    help="block: B=64 gamma=15 V=129280 T=1 (default); tiny: B=4 gamma=4 V=1024 fp32 T=1; "
                         "mtp: B=16 gamma=3 V=32000 T=0.7; greedy: B=64 gamma=7 "
                         "V=152064 T=0; scheduled: spec_schedule then spec_verify, gamma=15 V=129280; "
                         "dcut: spec_dcut then spec_verify_packed over the packed rows, gamma=15 V=129280; "
                         "logits: spec_verify_logits with bf16 draft logits, B=64 gamma=15 V=129280 T=1; "
                         "acceptance: spec_acceptance (alpha per position) on the same draft-logits workload; "
                         "static: spec_schedule_static (threshold 0.5) then spec_verify, gamma=15 V=129280; "
                         "sts_fit: spec_sts_fit on 2^20 samples x 15 positions, 100-point grid, 15 bins; "
                         "tree: spec_verify_tree, B=8 requests x a 64-node candidate tree, V=152064, T=0")
    ap.add_argument("--calibrated", action="store_true",
                    help="scheduled / dcut / static: apply per-position STS temperatures as confidences load")
    ap.add_argument("--batch", type=int, default=64, help="B of the scheduled, static and dcut workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 20 plain device-to-device copies of MIB MiB (a known-size kernel "
                         "for scaling the HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(requests shard across GPUs with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload == "sts_fit":
        return sts_fit_bench(args)
    if args.workload == "tree":
        return tree_bench(args)

    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 20}), flush=True)
        return

    kind = args.workload
    if kind == "block":
        w = W.block()
    elif kind == "tiny":
        w = W.tiny()
    elif kind == "mtp":
        w = W.mtp()
    elif kind == "greedy":
        w = W.greedy()
    elif kind in ("scheduled", "static"):
        w = W.scheduled(args.batch)
    elif kind in ("logits", "acceptance"):
        w = W.block_logits()
    else:
        w = W.ratio_budgeted(args.batch)
    B, G, V = w["B"], w["G"], w["V"]
    T = float(w["T"])
    esize = 2 if w["dtype"] == "bf16" else 4
    # stand-in fitted temperatures (the calibration recipe's per-position values)
    calib = W.calibration(2, G=G)[2].astype(np.float32).tolist() if args.calibrated else None

    # The oracle's lengths for the scheduled workloads (the GPU's are checked equal below).
    lens_o = None
    if kind == "scheduled":
        import oracle
        from oracle import calibration as C
        conf_o = w["confidence"] if calib is None else C.sts_apply(w["confidence"], calib)
        lens_o = np.asarray(oracle.schedule(conf_o, w["cost_table"], w["budget"])[0], np.int64)
    elif kind == "static":
        from oracle import calibration as C
        lens_o = C.static_threshold(w["confidence"] if calib is None else C.sts_apply(w["confidence"], calib), 0.5)
    elif kind == "dcut":
        from oracle import calibration as C
        from oracle import dcut as OD
        lens_o = np.asarray(OD.dcut(w["confidence"] if calib is None else C.sts_apply(w["confidence"], calib),
                                    w["ratios"], w["ratio_cost"])["verify_len"], np.int64)

    cpu = None
    if not args.no_cpu_baseline:
        unit = "alpha positions/s" if kind == "acceptance" else "verified draft positions/s"
        cpu = cpu_baseline(oracle_fn(kind, w, lens_o), B, unit,
                           f"the float64 oracle on the {B} requests of the same workload"
                           + (" (its own length choice once per pass over the batch, then verification)"
                              if lens_o is not None else ""))

    import torch
    import lossless_draft_verification_verify_amd as sv
    sv.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    def to_dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if w["dtype"] == "bf16":
        z0 = torch.from_numpy(w["logits"].view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        z0 = to_dev(w["logits"])
    q0, x0, u0 = to_dev(w["draft_probs"]), to_dev(w["draft_tokens"]), to_dev(w["uniforms"])
    if w.get("draft_logits") is not None:        # draft logits travel in the q slot
        q0 = torch.from_numpy(w["draft_logits"].view(np.int16)).to(dev).view(torch.bfloat16)
    clone = (lambda t: None if t is None else t.clone())
    sets = [(z0, q0, x0, u0)] + [tuple(clone(t) for t in (z0, q0, x0, u0)) for _ in range(args.sets - 1)]
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, G + 1, dtype=torch.int32, device=dev)
    static = None
    if kind == "static":
        static = (to_dev(w["confidence"]), 0.5, torch.empty(B, dtype=torch.int32, device=dev),
                  torch.empty(1, dtype=torch.int32, device=dev))
    sched = None
    if kind == "scheduled":
        conf, cost = to_dev(w["confidence"]), to_dev(w["cost_table"])
        vlen = torch.empty(B, dtype=torch.int32, device=dev)
        tot = torch.empty(1, dtype=torch.int32, device=dev)
        tau = torch.empty(1, dtype=torch.float32, device=dev)
        sched = (conf, cost, w["budget"], vlen, tot, tau)
    dcut = None
    if kind == "dcut":
        conf = to_dev(w["confidence"])
        vlen = torch.empty(B, dtype=torch.int32, device=dev)
        offs = torch.empty(B + 1, dtype=torch.int32, device=dev)
        ridx = torch.empty(1, dtype=torch.int32, device=dev)
        rows = torch.empty(1, dtype=torch.int32, device=dev)
        sv.dcut(conf, w["ratios"], w["ratio_cost"], out_verify_len=vlen, out_row_offsets=offs, out_ratio=ridx,
                out_rows=rows, utility=False, calib_temps=calib)
        torch.cuda.synchronize()
        # The target's logits of the packed batch: the kept rows of each set,
        # gathered once before timing (buffer sized for full depth).
        off_h = offs.cpu().numpy()
        idx = torch.tensor([b * (G + 1) + k for b in range(B) for k in range(int(off_h[b + 1] - off_h[b]))],
                           dtype=torch.long, device=dev)
        packed = []
        for zz, _, _, _ in sets:
            zp = torch.zeros(B * (G + 1), V, dtype=zz.dtype, device=dev)
            zp[: idx.numel()] = zz.reshape(B * (G + 1), V)[idx]
            packed.append(zp)
        dcut = (conf, vlen, offs, ridx, rows, packed)

    alpha = torch.empty(B, G, dtype=torch.float32, device=dev)

    def step(i, row_event=None):
        zz, qq, xx, uu = sets[i % len(sets)]
        vl = None
        if kind == "logits":
            sv.verify(zz, None, xx, uu, T, None, out_accepted=acc, out_tokens=tok, row_pass_event=row_event,
                      draft_logits=qq)
            return
        if kind == "acceptance":
            sv.acceptance(zz, qq, T, None, draft_is_logits=True, out_alpha=alpha)
            return
        if dcut is not None:
            conf, vlen, offs, ridx, rows, packed = dcut
            sv.dcut(conf, w["ratios"], w["ratio_cost"], out_verify_len=vlen, out_row_offsets=offs, out_ratio=ridx,
                    out_rows=rows, utility=False, calib_temps=calib)
            sv.verify_packed(packed[i % len(packed)], offs, qq, xx, uu, T, out_accepted=acc, out_tokens=tok,
                             row_pass_event=row_event)
            return
        if static is not None:
            vl, _, _ = sv.schedule_static(static[0], threshold=static[1], calib_temps=calib, row_offsets=False,
                                          out_verify_len=static[2], out_total=static[3])
        if sched is not None:
            conf, cost, budget, vlen, tot, tau = sched
            sv.schedule(conf, cost, budget, out_verify_len=vlen, out_total=tot, out_expected=tau, calib_temps=calib)
            vl = vlen
        sv.verify(zz, qq, xx, uu, T, vl, out_accepted=acc, out_tokens=tok, row_pass_event=row_event)

    # The verify workloads, and the scheduler workloads without calibration,
    # call the C ABI directly in the timed loops, with every argument marshalled
    # once beforehand, so the Python binding's per-call checks (tens of
    # microseconds) cannot starve the GPU between calls.
    fast = None
    fast_path = kind in ("block", "tiny", "mtp", "greedy") or (kind in ("scheduled", "static", "dcut") and calib is None)
    if kind in ("block", "tiny", "mtp", "greedy"):
        import ctypes
        from lossless_draft_verification_verify_amd import _capi
        lib = _capi.load()
        code = _capi.SPEC_DTYPE_BF16 if z0.dtype == torch.bfloat16 else _capi.SPEC_DTYPE_F32
        nbytes = _capi.verify_workspace_bytes(B, G, V, code)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        st_handle = torch.cuda.current_stream(dev).cuda_stream
        ptr = (lambda t: None if t is None else t.data_ptr())
        fast = [(ptr(zz), code, ptr(qq), ptr(xx), ptr(uu), None, B, G, V, ctypes.c_float(T), acc.data_ptr(),
                 tok.data_ptr(), None, ws.data_ptr(), ws.numel(), st_handle) for zz, qq, xx, uu in sets]
        fn = lib.spec_verify

        def step_fast(i):
            rc = fn(*fast[i % len(fast)])
            if rc != 0:
                raise RuntimeError(f"spec_verify: {_capi.status_string(rc)}")
    elif kind in ("scheduled", "static", "dcut") and calib is None:
        # The scheduler, then the verify over its lengths: the same two C ABI
        # calls the Python binding makes, marshalled once.
        import ctypes
        from lossless_draft_verification_verify_amd import _capi
        lib = _capi.load()
        code = _capi.SPEC_DTYPE_BF16 if z0.dtype == torch.bfloat16 else _capi.SPEC_DTYPE_F32
        nbytes = _capi.verify_workspace_bytes(B, G, V, code)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        st_handle = torch.cuda.current_stream(dev).cuda_stream
        ptr = (lambda t: None if t is None else t.data_ptr())
        cT = ctypes.c_float(T)
        if kind == "scheduled":
            conf, cost, budget, vlen, tot, tau = sched
            first = (lib.spec_schedule, "spec_schedule",
                     (conf.data_ptr(), cost.data_ptr(), int(cost.shape[0]), B, G, int(budget), ctypes.c_float(0.0),
                      vlen.data_ptr(), tot.data_ptr(), tau.data_ptr(), None, 0, st_handle))
            second = (lib.spec_verify, "spec_verify",
                      [(ptr(zz), code, ptr(qq), ptr(xx), ptr(uu), vlen.data_ptr(), B, G, V, cT, acc.data_ptr(),
                        tok.data_ptr(), None, ws.data_ptr(), ws.numel(), st_handle) for zz, qq, xx, uu in sets])
        elif kind == "static":
            sconf, thr, slen, stot = static
            first = (lib.spec_schedule_static, "spec_schedule_static",
                     (sconf.data_ptr(), B, G, _capi.SPEC_STATIC_THRESHOLD, 0, ctypes.c_float(thr), None,
                      slen.data_ptr(), stot.data_ptr(), None, st_handle))
            second = (lib.spec_verify, "spec_verify",
                      [(ptr(zz), code, ptr(qq), ptr(xx), ptr(uu), slen.data_ptr(), B, G, V, cT, acc.data_ptr(),
                        tok.data_ptr(), None, ws.data_ptr(), ws.numel(), st_handle) for zz, qq, xx, uu in sets])
        else:
            dconf, dlen, doffs, dridx, drows, packed = dcut
            nr = len(w["ratios"])
            rat = (ctypes.c_float * nr)(*[float(r) for r in w["ratios"]])
            rco = (ctypes.c_float * nr)(*[float(r) for r in w["ratio_cost"]])
            first = (lib.spec_dcut, "spec_dcut",
                     (dconf.data_ptr(), B, G, rat, rco, nr, None, dlen.data_ptr(), doffs.data_ptr(),
                      dridx.data_ptr(), drows.data_ptr(), None, st_handle))
            second = (lib.spec_verify_packed, "spec_verify_packed",
                      [(zp.data_ptr(), code, int(zp.shape[0]), doffs.data_ptr(), ptr(qq), ptr(xx), ptr(uu), B, G, V,
                        cT, acc.data_ptr(), tok.data_ptr(), None, ws.data_ptr(), ws.numel(), st_handle)
                       for zp, (_, qq, xx, uu) in zip(packed, sets)])
        f1, n1, a1 = first
        f2, n2, a2 = second

        def step_fast(i):
            rc = f1(*a1)
            if rc != 0:
                raise RuntimeError(f"{n1}: {_capi.status_string(rc)}")
            rc = f2(*a2[i % len(a2)])
            if rc != 0:
                raise RuntimeError(f"{n2}: {_capi.status_string(rc)}")
    else:
        step_fast = step

    # outputs of one call fix the data-dependent counts (verify lengths, rejecting requests)
    step(0)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    if sched is not None:
        lens = sched[3].cpu().numpy().astype(np.int64)
    elif static is not None:
        lens = static[2].cpu().numpy().astype(np.int64)
    elif dcut is not None:
        lens = dcut[1].cpu().numpy().astype(np.int64)
    else:
        lens = np.full(B, G, np.int64)
    if lens_o is not None and not np.array_equal(lens, lens_o):
        raise RuntimeError("the device's verify lengths differ from the oracle's")
    n_rej = int((a < lens).sum()) if T > 0 and kind != "acceptance" else 0
    algo = algorithmic_bytes(B, G, V, lens, n_rej, esize)
    if T == 0:                                   # no q rows, no uniforms
        algo = int((lens + 1).sum()) * V * esize + int(lens.sum()) * 4 + B * (4 + 4 * (G + 1))
    row_algo = row_pass_bytes(V, lens, esize)
    if kind in ("logits", "acceptance"):
        # draft rows 0..len_b-1 are read too; every q(x) and residual comes
        # from rows already read, so no fp32 q row is compulsory
        drafts = int(lens.sum()) * V * esize
        row_algo = row_algo + drafts
        algo = int((lens + 1).sum()) * V * esize + drafts + int(lens.sum()) * 8 + B * (4 + 4 + 4 * (G + 1))
        if kind == "acceptance":                   # one read of target row k and draft row k per position
            row_algo = algo = 2 * int(lens.sum()) * V * esize

    for i in range(args.warmup):
        step_fast(i)
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.current_stream(dev)       # the stream the library launches on
    sh = stream.cuda_stream

    # Cold: K calls right after the warm-up steps.  Then settle: the device
    # reaches its steady operating point only after some milliseconds of this
    # step's traffic (block workload: batches of 20 calls at 55-66 us over the
    # first ~250 calls, 53.0-53.4 us after; a neutral 50 ms memory fill before
    # them shortens that only partly), and a serving loop runs in that steady
    # state, so the step runs for --settle-ms of wall time before the timed
    # calls.  Both are reported.
    c_start = torch.cuda.Event(enable_timing=True)
    c_end = torch.cuda.Event(enable_timing=True)
    c_start.record(stream)
    for i in range(K):
        step_fast(i)
    c_end.record(stream)
    torch.cuda.synchronize()
    cold_ms = c_start.elapsed_time(c_end) / K
    n_settle = 0
    s0 = time.perf_counter()
    while time.perf_counter() - s0 < args.settle_ms * 1e-3:
        for _ in range(16):
            step_fast(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - s0) * 1e3

    # Throughput: exactly K calls back to back, nothing else on the stream.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    h0 = time.perf_counter()
    for i in range(K):
        step_fast(i)
    host_ms = (time.perf_counter() - h0) * 1e3
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)

    # Per-call spread and the row pass alone: K more calls, each bracketed by
    # events on the same stream, plus the event the library records right
    # after the row-pass launch.
    hev = HipEvents(3 * K)
    torch.cuda.synchronize()
    for i in range(K):
        hev.record(3 * i, sh)
        if kind == "acceptance":                 # a single kernel: its own interval
            step(i)
            hev.record(3 * i + 1, sh)
        else:
            step(i, row_event=hev.ev[3 * i + 1])
        hev.record(3 * i + 2, sh)
    torch.cuda.synchronize()
    call = np.array([hev.ms(3 * i, 3 * i + 2) for i in range(K)])      # ms per call
    rows_ms = np.array([hev.ms(3 * i, 3 * i + 1) for i in range(K)])   # ms up to the row-pass event
    req_ms = np.array([hev.ms(3 * i + 1, 3 * i + 2) for i in range(K)])  # ms after it
    hev.close()
    ms_step = total_ms / K
    positions = int(lens.sum())
    value = positions / (ms_step * 1e-3)
    call_gbps = algo / (ms_step * 1e-3) / 1e9
    row_gbps = row_algo / (float(rows_ms.mean()) * 1e-3) / 1e9
    traffic = measured_traffic(kind)
    if kind in DESCRIPTIONS:
        desc = DESCRIPTIONS[kind]
    elif kind == "scheduled":
        desc = (f"confidence-scheduled verification: spec_schedule{'_calibrated' if calib else ''} (token budget "
                f"{w['budget']}, cost 1 + 0.02 T) then spec_verify, B={B}, gamma=15, V=129280, bf16, T=1")
    elif kind == "static":
        desc = (f"static-threshold verification: spec_schedule_static (confidence > 0.5"
                f"{', STS-calibrated' if calib else ''}) then spec_verify, B={B}, gamma=15, V=129280, bf16, T=1")
    else:
        r_idx = int(dcut[3].item())
        desc_cal = ", STS-calibrated" if calib else ""
        desc = (f"ratio-budgeted verification: spec_dcut (ratios {list(w['ratios'])}, cost 1 + 0.02 rho B (G+1); "
                f"chosen ratio {w['ratios'][r_idx]}, {int(dcut[4].item())} packed rows{desc_cal}) then "
                f"spec_verify_packed, B={B}, gamma=15, V=129280, bf16, T=1")
    one_launch = "k_verify_sampled (one launch: row groups, a decision workgroup per request, request workgroups)"
    launches = {"acceptance": "k_acceptance (one launch)",
                "greedy": "k_verify_greedy (one launch: argmax row workgroups, then one workgroup per request)",
                "block": one_launch, "tiny": one_launch, "mtp": one_launch}
    call_kernels = launches.get(kind, "the whole call: row pass (k_rows_sampled" +
                                ("_vl" if lens_o is not None else "") + "), then request pass (k_requests_sampled)" +
                                (", after the length choice" if lens_o is not None else ""))
    two_launches = kind not in launches
    out = {
        "metric": "verified draft positions/sec and achieved HBM GB/s (% peak), B=64 gamma=15 V=129k",
        "value": round(value, 1),
        "unit": "alpha positions/s" if kind == "acceptance" else "verified draft positions/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": desc, "B": B, "gamma": G, "V": V, "temperature": T, "logits": w["dtype"],
                   "rotating_sets": len(sets), "verified_positions_per_step": positions,
                   "rejecting_requests": n_rej, "host_enqueue_ms_per_step": round(host_ms / K, 5),
                   "call_path": "C ABI, arguments marshalled once" if fast_path else "Python binding"},
        # The roofline of the verify call as a whole (every launch it makes):
        # its algorithmic bytes over its time per call in the throughput loop.
        "roofline": {"bound": "hbm", "achieved": round(call_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(call_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "kernel": call_kernels,
                     "algorithmic_bytes_per_launch": algo,
                     "launch_ms_mean": round(ms_step, 5),
                     "call_ms_p10_p50_p90_event_timed": [round(float(np.percentile(call, p)), 5)
                                                         for p in (10, 50, 90)]},
        "row_pass": ({"algorithmic_bytes": row_algo, "ms_mean_event_timed": round(float(rows_ms.mean()), 5),
                      "achieved_GBps": round(row_gbps, 1), "frac": round(row_gbps / PEAK_HBM_GBPS, 4),
                      "after_row_pass_ms_mean": round(float(req_ms.mean()), 5),
                      "note": "interval from the call's start to the library's event after the row-pass launch"}
                     if two_launches else None),
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "settle": {"cold_ms_per_step": round(cold_ms, 5), "settle_ms": round(settle_ms, 1), "settle_calls": n_settle,
                   "note": "cold: the K calls right after the warm-up steps; the timed K calls follow settle_calls "
                           "more calls of the same step"},
    }
    if kind != "acceptance":
        out["acceptance"] = acceptance_stats(a, lens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
