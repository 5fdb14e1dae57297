"""Benchmark of the DDTree tree-verify step on one MI355X.

A step is one pass of the whole hot path over one batch: tree build -> tree-
verify attention (prefix stream, masked tree part, split merge) -> greedy
accept, enqueued back to back on one stream (captured once into a HIP graph and
replayed).  The headline workload is batch 1, H=64, bf16 latent KV 512+64,
prefix 2048, drafter depth 8 x top-8, budget 8.  The same JSON line also carries
the attention roofline of that workload, the other benchmark workloads as extra
measurements, and the CPU oracle timed on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only-primary]
Prints exactly one JSON line on stdout (progress goes to stderr).
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

METRIC = ("verify-attn TFLOP/s + HBM GB/s (% roofline); "
          "tree-verify steps/s at batch 1/64")
PRIMARY = "b1_l2k_q9"
EXTRA = ["tiny_fp32", "b4_l4k_q17", "b4_l4k_q33", "b64_l2k_q9", "b8_l32k_q65"]
# MI355X published peaks.
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "tree_verify_mla_ddt_amd", "csrc", "verify_attn.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_work(wl, tree):
    """Algorithmic flops and bytes of one verify-attention call.

    flops: every visible (row, key) pair costs 2*(d_lat+d_rope) for the score and
    2*d_lat for the value product; a node sees the prefix and its depth+1 root
    path entries.  bytes: each KV entry read once, queries read once, fp32
    output + lse written once, visibility rows and slot ids read once."""
    elt = 4 if wl.dtype == "f32" else 2
    dk = wl.d_lat + wl.d_rope
    n_nodes = tree["n_nodes"]
    depth = tree["depth"]
    pairs = 0
    kv_entries = 0
    for b in range(wl.B):
        n = int(n_nodes[b])
        L = int(wl.prefix_len[b])
        pairs += n * L + int((depth[b, :n] + 1).sum())
        kv_entries += L + n
    flops = wl.H * pairs * (2 * dk + 2 * wl.d_lat)
    W = (wl.Q + 63) // 64
    rows = wl.B * wl.Q * wl.H
    nbytes = (kv_entries * dk * elt + rows * dk * elt + rows * (wl.d_lat + 1) * 4
              + wl.B * wl.Q * W * 8 + kv_entries * 4)
    return float(flops), float(nbytes)


def source_digest():
    with open(ATTN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


COPY_BYTES = 256 << 20  # the --copy-calibration copy
ATTN_KERNELS = ("verify_attn_kernel", "verify_merge_kernel", "verify_merge_wide_kernel")


def _counter_rows(directory):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    return rows


def _per_launch_kib(rows, counter):
    """(attention-call KiB per launch, copy KiB) for one counter: the verify_attn
    call's kernels summed per launch (mean over launches), and the 256 MiB copy."""
    per_kernel, copy = {}, []
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        name, v = r["Kernel_Name"], float(r["Counter_Value"])
        for k in ATTN_KERNELS:
            if k in name:
                per_kernel.setdefault(k, []).append(v)
        if "copyBuffer" in name and int(r["Grid_Size"]) * 2048 == COPY_BYTES:
            copy.append(v)  # the calibration copy moves 2 KiB per work-item
    if "verify_attn_kernel" not in per_kernel or not copy:
        raise SystemExit(f"{counter}: attention kernel or calibration copy missing")
    att = sum(sum(v) / len(v) for v in per_kernel.values())
    return att, sum(copy) / len(copy)


def write_traffic(workload, fetch_dir, write_dir):
    """Record HBM bytes per verify_attn call from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE), each counter scaled by what it reads for a plain
    copy of COPY_BYTES (read once, written once)."""
    f_att, f_copy = _per_launch_kib(_counter_rows(fetch_dir), "FETCH_SIZE")
    w_att, w_copy = _per_launch_kib(_counter_rows(write_dir), "WRITE_SIZE")
    f_scale, w_scale = COPY_BYTES / (f_copy * 1024.0), COPY_BYTES / (w_copy * 1024.0)
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    if rec.get("source_sha256_16") != source_digest():
        rec = {"source_sha256_16": source_digest(), "workloads": {}}
    rec["workloads"][workload] = {
        "bytes_per_launch": round(f_att * 1024.0 * f_scale + w_att * 1024.0 * w_scale),
        "fetch_kib_raw": round(f_att, 1), "write_kib_raw": round(w_att, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec["workloads"][workload]))


def measured_traffic(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, or
    None when absent or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256_16") != source_digest():
        return None
    w = rec.get("workloads", {}).get(workload)
    return None if w is None else float(w["bytes_per_launch"])


class StepRunner:
    """Device-resident inputs of one workload and its captured step graphs."""

    def __init__(self, name, torch, ddt, workloads):
        self.torch, self.ddt = torch, ddt
        t0 = time.time()
        wl = workloads.make_workload(name)
        self.wl = wl
        dev = torch.device("cuda:0")
        cuda = lambda a: torch.as_tensor(a).contiguous().to(dev)
        self.logp, self.ids = cuda(wl.topk_logp), cuda(wl.topk_ids)
        self.root, self.plen = cuda(wl.root_token), cuda(wl.prefix_len)
        self.q_lat, self.q_pe = cuda(wl.q_lat), cuda(wl.q_pe)
        self.c_kv, self.k_pe = cuda(wl.c_kv), cuda(wl.k_pe)
        self.r2s = cuda(wl.req_to_slot)
        B, Q, H = wl.B, wl.Q, wl.H
        self.out = torch.empty((B, Q, H, wl.d_lat), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
        self.ws = torch.empty((max(1, ddt.workspace_size(B, Q, H, self.r2s.shape[1], wl.d_lat)),),
                              dtype=torch.uint8, device=dev)
        # Build once to get the tree the target tokens are synthesized for.
        self.tree = ddt.tree_build(self.logp, self.ids, self.root, self.plen, wl.budget)
        torch.cuda.synchronize()
        host_tree = {k: v.cpu().numpy() for k, v in self.tree.items()}
        self.host_tree = host_tree
        tgt = workloads.synth_target_argmax(wl, host_tree["node_token"], host_tree["parent"],
                                            host_tree["depth"], host_tree["n_nodes"])
        self.tgt = cuda(tgt)
        self.acc = ddt.tree_accept(self.tree["node_token"], self.tree["parent"],
                                   self.tree["n_nodes"], self.tgt)
        torch.cuda.synchronize()
        self.flops, self.nbytes = attn_work(wl, host_tree)
        log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s "
            f"(attention {self.flops / 1e9:.2f} GFLOP, {self.nbytes / 1e6:.1f} MB per call)")

    def attn(self):
        self.ddt.verify_attn(self.q_lat, self.q_pe, self.c_kv, self.k_pe, self.r2s, self.plen,
                             self.tree["n_nodes"], self.tree["vis"], self.wl.sm_scale,
                             out=self.out, lse=self.lse, workspace=self.ws)

    def step(self):
        self.ddt.tree_build(self.logp, self.ids, self.root, self.plen, self.wl.budget,
                            out=self.tree)
        self.attn()
        self.ddt.tree_accept(self.tree["node_token"], self.tree["parent"], self.tree["n_nodes"],
                             self.tgt, out=self.acc)

    def capture(self, fn):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_graph(self, g, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            g.replay()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps  # ms

    def time_eager(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            fn()
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    def commit_ms(self, steps=200):
        """What ddt_kv_commit adds to a step: graph replays of (step, restore
        prefix_len, commit) minus replays of (step, restore).  The commit rewrites
        the table in place, so prefix_len is reset every time and each replay
        commits the same accepted paths."""
        torch, ddt = self.torch, self.ddt
        r2s, plen0 = self.r2s.clone(), self.plen.clone()
        plen = plen0.clone()
        fo = {"freed_slots": torch.empty_like(self.acc["accept_nodes"]),
              "n_freed": torch.empty_like(self.acc["accept_len"])}

        def without():
            self.step()
            plen.copy_(plen0)

        def with_commit():
            without()
            ddt.kv_commit(r2s, plen, self.tree["n_nodes"], self.acc["accept_len"],
                          self.acc["accept_nodes"], out=fo)

        g_w, g_c = self.capture(without), self.capture(with_commit)
        t_w = self.time_graph(g_w, steps, 10)
        t_c = self.time_graph(g_c, steps, 10)
        t_w2 = self.time_graph(g_w, steps, 10)
        return max(t_c - 0.5 * (t_w + t_w2), 0.0)

    def topk_stats(self, steps=200):
        """ddt_draft_topk on this workload's drafter shape: D depths of logits over
        the workload's vocabulary (bf16, or fp32 for the fp32 workload), timed by
        graph replays; HBM-bound, so the roofline is bytes read and written."""
        torch, ddt, wl = self.torch, self.ddt, self.wl
        dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        g = torch.Generator(device="cuda").manual_seed(11)
        logits = (torch.randn((wl.B, wl.D, wl.vocab), generator=g, device="cuda") * 2).to(dt)
        out = {"topk_logp": torch.empty((wl.B, wl.D, wl.K), dtype=torch.float32, device="cuda"),
               "topk_ids": torch.empty((wl.B, wl.D, wl.K), dtype=torch.int32, device="cuda")}
        ws = torch.empty((int(ddt.load_library().ddt_draft_topk_workspace_size(
            wl.B, wl.D, wl.vocab, wl.K)),), dtype=torch.uint8, device="cuda")
        gr = self.capture(lambda: ddt.draft_topk(logits, wl.K, out=out, workspace=ws))
        ms = self.time_graph(gr, steps, 10)
        nbytes = logits.numel() * logits.element_size() + wl.B * wl.D * wl.K * 8
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "bytes": nbytes, "gbs": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "vocab": wl.vocab, "K": wl.K,
                "D": wl.D}

    def sampling_stats(self, steps=200):
        """ddt_tree_accept_sampling on this workload's drafted tree at temperature 1:
        target logits N(0, 2) over the workload's vocabulary at every tree node (bf16,
        or fp32 for the fp32 workload), with each node's lowest-index child's token set
        to 16 (about 0.9 of the node's mass at V = 160000) so that drafts are accepted;
        timed by graph replays.  The
        statistics pass reads every live node's logits once, so the roofline is HBM
        bytes."""
        torch, ddt, wl = self.torch, self.ddt, self.wl
        dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        g = torch.Generator(device="cuda").manual_seed(12)
        B, Q, V = wl.B, wl.Q, wl.vocab
        logits = (torch.randn((B, Q, V), generator=g, device="cuda") * 2).to(dt)
        ht = self.host_tree
        for b in range(B):
            seen = set()
            for c in range(1, int(ht["n_nodes"][b])):
                p = int(ht["parent"][b, c])
                if p not in seen:
                    seen.add(p)
                    logits[b, p, int(ht["node_token"][b, c])] = 16.0
        temp = torch.ones((B,), dtype=torch.float32, device="cuda")
        coins = torch.rand((B, Q), generator=g, device="cuda")
        cfin = torch.rand((B,), generator=g, device="cuda")
        out = {k: torch.empty_like(v) for k, v in self.acc.items()}
        ws = torch.empty((max(1, int(ddt.load_library().ddt_tree_accept_sampling_workspace_size(
            B, Q, V))),), dtype=torch.uint8, device="cuda")
        tr = self.tree
        fn = lambda: ddt.tree_accept_sampling(logits, temp, tr["node_token"], tr["parent"],
                                              tr["n_nodes"], coins, cfin, out=out, workspace=ws)
        gr = self.capture(fn)
        ms = self.time_graph(gr, steps, 10)
        live = int(ht["n_nodes"][:B].sum())
        nbytes = live * V * logits.element_size() + B * Q * 4 * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        mean_len = float(out["accept_len"].float().mean())
        return {"ms": round(ms, 5), "bytes": nbytes, "gbs": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "vocab": V,
                "mean_accept_len": round(mean_len, 3)}

    def roofline(self, attn_ms, name):
        wl = self.wl
        peak = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
        achieved = self.flops / (attn_ms * 1e-3) / 1e12
        gbs = self.nbytes / (attn_ms * 1e-3) / 1e9
        return {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(name),
                "kernel": "verify_attn (attention + split-merge kernels)",
                "flops_per_launch": self.flops, "bytes_per_launch": self.nbytes,
                "hbm_gbs_algorithmic": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                "launch_ms": round(attn_ms, 5)}


def cpu_baseline(name, wl, host_tree, tgt_host, budget_s=12.0):
    """The oracle on the host cores: one full step of the workload (tree build,
    attention over every row, accept), repeated until about `budget_s` of work."""
    import oracle
    f = lambda t: t.float().numpy()
    q_lat, q_pe, c_kv, k_pe = f(wl.q_lat), f(wl.q_pe), f(wl.c_kv), f(wl.k_pe)
    reps, t_total = 0, 0.0
    t_build = t_attn = t_acc = 0.0
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
        t1 = time.perf_counter()
        oracle.verify_attn(q_lat, q_pe, c_kv, k_pe, wl.req_to_slot, wl.prefix_len, t["n_nodes"],
                           t["vis"], wl.sm_scale)
        t2 = time.perf_counter()
        oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"], tgt_host)
        t3 = time.perf_counter()
        t_build += t1 - t0
        t_attn += t2 - t1
        t_acc += t3 - t2
        t_total += t3 - t0
        reps += 1
    per_step = t_total / reps
    return {"value": round(1.0 / per_step, 3), "unit": "steps/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": (f"{reps} full steps of {name} (tree build, attention over all "
                       f"{wl.B * wl.Q * wl.H} rows in fp64, accept), {t_total:.1f}s total; "
                       f"per step build {t_build / reps * 1e3:.2f} ms, attention "
                       f"{t_attn / reps * 1e3:.1f} ms, accept {t_acc / reps * 1e3:.3f} ms")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-primary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP graph replays (for profilers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for byte counters)")
    ap.add_argument("--workload", default=PRIMARY,
                    help="headline workload (default: the batch-1 configuration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="record the workload's HBM bytes per attention call from two "
                         "rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.workload, *args.traffic_from)
        return
    if args.gpus != 1:
        print(f"bench.py: the verify step runs on one GPU; --gpus {args.gpus} is not "
              f"supported (no sharding or collectives across GPUs).", file=sys.stderr)
        sys.exit(2)

    import torch
    import tree_verify_mla_ddt_amd as ddt
    from tree_verify_mla_ddt_amd import workloads
    ddt.load_library()
    log(f"[bench] device {torch.cuda.get_device_name(0)}, {ddt.version()}")

    primary = args.workload
    runner = StepRunner(primary, torch, ddt, workloads)
    if args.copy_calibration:
        src = torch.empty((256 << 20,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.eager:
        ms_step = runner.time_eager(runner.step, args.steps, args.warmup)
        ms_attn = runner.time_eager(runner.attn, args.steps, args.warmup)
    else:
        g_step = runner.capture(runner.step)
        g_attn = runner.capture(runner.attn)
        torch.cuda.synchronize()
        ms_step = runner.time_graph(g_step, args.steps, args.warmup)
        ms_attn = runner.time_graph(g_attn, args.steps, args.warmup)
    ms_eager = runner.time_eager(runner.step, min(args.steps, 100), 5)
    log(f"[bench] {primary}: step {ms_step * 1e3:.1f} us (graph), {ms_eager * 1e3:.1f} us "
        f"(eager), attention {ms_attn * 1e3:.1f} us")
    roof = runner.roofline(ms_attn, primary)
    wl = runner.wl
    result = {
        "metric": METRIC, "value": round(1000.0 / ms_step, 2), "unit": "steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": primary, "batch": wl.B, "heads": wl.H, "prefix": int(wl.prefix_len[0]),
                   "q_len": wl.Q, "drafter": f"{wl.D}x{wl.K}",
                   "kv": f"{wl.dtype} {wl.d_lat}+{wl.d_rope}",
                   "step": "tree_build -> verify_attn -> tree_accept, HIP graph replay"},
        "roofline": roof,
        "step_eager_ms": round(ms_eager, 5),
        "kv_commit_step_ms": round(runner.commit_ms(), 5),
        "draft_topk": runner.topk_stats(),
        "accept_sampling": runner.sampling_stats(),
    }

    extras = {}
    if not args.only_primary:
        for name in [n for n in [PRIMARY] + EXTRA if n != primary]:
            r = StepRunner(name, torch, ddt, workloads)
            gs, ga = r.capture(r.step), r.capture(r.attn)
            k = max(10, min(args.steps, 200))
            ms_s = r.time_graph(gs, k, 5)
            ms_a = r.time_graph(ga, k, 5)
            rf = r.roofline(ms_a, name)
            extras[name] = {"steps_per_s": round(1000.0 / ms_s, 2), "ms_per_step": round(ms_s, 5),
                            "requests_per_s": round(r.wl.B * 1000.0 / ms_s, 1),
                            "attn_ms": round(ms_a, 5), "attn_tflops": rf["achieved"],
                            "attn_frac_peak": rf["frac"], "attn_hbm_gbs": rf["hbm_gbs_algorithmic"],
                            "traffic": rf["traffic"], "dtype": r.wl.dtype,
                            "kv_commit_step_ms": round(r.commit_ms(), 5),
                            "draft_topk": r.topk_stats(),
                            "accept_sampling": r.sampling_stats()}
            log(f"[bench] {name}: step {ms_s * 1e3:.1f} us, attention {ms_a * 1e3:.1f} us = "
                f"{rf['achieved']:.1f} TFLOP/s ({100 * rf['frac']:.1f}% of {rf['peak']})")
            del r, gs, ga
            torch.cuda.empty_cache()
        result["extra_workloads"] = extras

    if not args.no_cpu:
        log("[bench] timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(primary, wl, runner.host_tree,
                                              runner.tgt.cpu().numpy())
        log(f"[bench] oracle: {result['cpu_baseline']['value']} steps/s on "
            f"{result['cpu_baseline']['cores']} threads")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
