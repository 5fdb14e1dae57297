"""Benchmark of the DDTree tree-verify step on one MI355X.

A step is one pass of the whole hot path over one batch: tree build -> tree-
verify attention (prefix stream, masked tree part, split merge) -> greedy
accept, enqueued back to back on one stream (captured once into a HIP graph and
replayed).  The headline workload is batch 1, H=64, bf16 latent KV 512+64,
prefix 2048, drafter depth 8 x top-8, budget 8.  The same JSON line also carries
the attention roofline of that workload, the other benchmark workloads as extra
measurements, and the CPU oracle timed on the host cores.

Every GPU figure is the median of 5 repeats of back-to-back graph replays (the
headline step: --steps replays per repeat; everything else: at least 100), with
the repeats' minimum and maximum beside it.  The attention roofline is given
for the attention kernel alone (HIP events around back-to-back launches of that
kernel) and for the whole call (attention kernel + split merge).

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
EXTRA = ["tiny_fp32", "b4_l4k_q17", "b4_l4k_q33", "b64_l2k_q9", "b8_l32k_q65",
         "b64_l2k_q9_h8", "b8_l32k_q65_h8"]
REPEATS = 5        # timed repeats per figure; the median is reported
MIN_REPLAYS = 100  # replays per repeat for every figure but the headline step
# MI355X published peaks.
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_attn_traffic.json")
# The attention kernels and the work split they run: the traffic record is
# valid for exactly these sources.
ATTN_SOURCES = [os.path.join(ROOT, "tree_verify_mla_ddt_amd", "csrc", f)
                for f in ("verify_attn.hip", "attn_split.h")]


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
    h = hashlib.sha256()
    for path in ATTN_SOURCES:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()[:16]


COPY_BYTES = 256 << 20  # the --copy-calibration copy
ATTN_KERNELS = ("verify_attn_kernel", "verify_attn_wide_kernel", "verify_attn_narrow_kernel",
                "verify_merge_kernel", "verify_merge_wide_kernel")


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
    if not ({"verify_attn_kernel", "verify_attn_wide_kernel", "verify_attn_narrow_kernel"}
            & set(per_kernel)) or not copy:
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


class Timing:
    """Per-launch milliseconds of each timed repeat; `ms` is their median."""

    def __init__(self, per_repeat, n):
        self.per = sorted(float(x) for x in per_repeat)
        self.n = n
        self.ms = float(np.median(self.per))

    def summary(self, scale=1e3, unit="us"):
        return {"median": round(self.ms * scale, 3), "min": round(self.per[0] * scale, 3),
                "max": round(self.per[-1] * scale, 3), "unit": unit,
                "replays_per_repeat": self.n, "repeats": len(self.per)}


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

    def _time(self, launch, n, warmup, repeats=REPEATS):
        """`repeats` timed runs of n back-to-back launches, each bracketed by a
        device synchronization and HIP events on the current stream (where the
        graphs are replayed and the library enqueues its kernels).  Returns the
        per-launch milliseconds of every repeat and their median."""
        torch = self.torch
        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
        per = []
        for _ in range(repeats):
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for _ in range(n):
                launch()
            stop.record()
            torch.cuda.synchronize()
            per.append(start.elapsed_time(stop) / n)
        return Timing(per, n)

    def time_graph(self, g, n, warmup, repeats=REPEATS):
        return self._time(g.replay, n, warmup, repeats)

    def steps_in_one_graph(self, copies, n=MIN_REPLAYS):
        """Per-step time of graph replays that hold `copies` consecutive steps."""
        g = self.capture(lambda: [self.step() for _ in range(copies)])
        t = self.time_graph(g, n, 5)
        return Timing([x / copies for x in t.per], n * copies)

    def time_eager(self, fn, n, warmup, repeats=REPEATS):
        return self._time(fn, n, warmup, repeats)

    def kernel_times(self, reps=MIN_REPLAYS, repeats=REPEATS):
        """Per-launch milliseconds of the attention kernel and of the merge kernel,
        each launched `reps` times back to back between HIP events on the current
        stream; `repeats` runs, medians."""
        a = self.wl
        att, mrg = [], []
        for _ in range(repeats):
            ms_a, ms_m, _, _ = self.ddt.verify_attn_kernel_times(
                self.q_lat, self.q_pe, self.c_kv, self.k_pe, self.r2s, self.plen,
                self.tree["n_nodes"], self.tree["vis"], a.sm_scale, reps, out=self.out,
                lse=self.lse, workspace=self.ws)
            att.append(ms_a)
            mrg.append(ms_m)
        return Timing(att, reps), Timing(mrg, reps)

    def commit_ms(self, steps=MIN_REPLAYS):
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
        t_w = self.time_graph(g_w, steps, 10).ms
        t_c = self.time_graph(g_c, steps, 10).ms
        t_w2 = self.time_graph(g_w, steps, 10).ms
        return max(t_c - 0.5 * (t_w + t_w2), 0.0)

    def topk_stats(self, steps=MIN_REPLAYS):
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
        ms = self.time_graph(gr, steps, 10).ms
        nbytes = logits.numel() * logits.element_size() + wl.B * wl.D * wl.K * 8
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "bytes": nbytes, "gbs": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "vocab": wl.vocab, "K": wl.K,
                "D": wl.D}

    def sampling_stats(self, steps=MIN_REPLAYS):
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
        ms = self.time_graph(gr, steps, 10).ms
        live = int(ht["n_nodes"][:B].sum())
        nbytes = live * V * logits.element_size() + B * Q * 4 * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        mean_len = float(out["accept_len"].float().mean())
        return {"ms": round(ms, 5), "bytes": nbytes, "gbs": round(gbs, 1),
                "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "vocab": V,
                "mean_accept_len": round(mean_len, 3)}

    def roofline(self, kernel_ms, merge_ms, call_ms, name):
        """Roofline of one verify_attn call's algorithmic work (flops and bytes as
        attn_work counts them), over the attention kernel's mean launch time
        (the dominant kernel: `frac`) and over the whole call (`call_frac`).  The
        bound is the one the algorithmic intensity falls under: MFMA when
        flops / bytes is at least the peak ratio, else HBM."""
        wl = self.wl
        peak_f = PEAK_F32_TFLOPS if wl.dtype == "f32" else PEAK_BF16_TFLOPS
        ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
        mfma = self.flops / self.nbytes >= ridge
        tf = lambda ms: self.flops / (ms * 1e-3) / 1e12
        gb = lambda ms: self.nbytes / (ms * 1e-3) / 1e9
        if mfma:
            ach, peak, unit, call_ach = tf(kernel_ms), peak_f, "TFLOP/s", tf(call_ms)
        else:
            ach, peak, unit, call_ach = gb(kernel_ms), PEAK_HBM_GBS, "GB/s", gb(call_ms)
        return {"bound": "mfma" if mfma else "hbm", "achieved": round(ach, 3), "peak": peak,
                "unit": unit, "frac": round(ach / peak, 4),
                "traffic": measured_traffic(name),
                "kernel": self.attn_kernel_name(),
                "kernel_us": round(kernel_ms * 1e3, 3), "merge_kernel_us": round(merge_ms * 1e3, 3),
                "call_us": round(call_ms * 1e3, 3), "call_achieved": round(call_ach, 3),
                "call_frac": round(call_ach / peak, 4),
                "flops_per_launch": self.flops, "bytes_per_launch": self.nbytes,
                "kernel_tflops": round(tf(kernel_ms), 3),
                "kernel_mfma_frac": round(tf(kernel_ms) / peak_f, 4),
                "kernel_hbm_gbs": round(gb(kernel_ms), 1),
                "kernel_hbm_frac": round(gb(kernel_ms) / PEAK_HBM_GBS, 4)}

    def attn_kernel_name(self):
        """The attention kernel the library launches for this workload: the
        512-wide bf16 form runs four 32-row workgroups per range (narrow) when
        its row tiles number at most a sixteenth of the CUs, else 128-row ones
        (wide); the 64-wide forms run the paired-wave kernel."""
        wl = self.wl
        if not (wl.dtype == "bf16" and wl.d_lat == 512):
            return "verify_attn_kernel"
        units = wl.B * ((wl.Q * wl.H + 127) // 128)
        cus = self.torch.cuda.get_device_properties(0).multi_processor_count
        return "verify_attn_narrow_kernel" if units * 16 <= cus else "verify_attn_wide_kernel"

    def measure(self, steps, warmup, kernel_reps=MIN_REPLAYS):
        """Step and attention-call graph replays plus kernel times; returns the
        timings and the roofline."""
        g_step, g_attn = self.capture(self.step), self.capture(self.attn)
        self.torch.cuda.synchronize()
        t_step = self.time_graph(g_step, steps, warmup)
        t_call = self.time_graph(g_attn, max(steps, MIN_REPLAYS), warmup)
        t_kern, t_merge = self.kernel_times(kernel_reps)
        roof = self.roofline(t_kern.ms, t_merge.ms, t_call.ms, self.wl.name)
        del g_step, g_attn
        return t_step, t_call, t_kern, t_merge, roof


CEILING_MODES = {0: "MFMA only (16 accumulators, operands in registers)",
                 1: "attention tile operand traffic (LDS reads, one barrier per tile)",
                 2: "attention tile operand traffic + next tile's global->LDS loads"}


def run_ceiling(iters=4000):
    """What one CU's four waves sustain on v_mfma_f32_32x32x16_bf16 alone and with
    the attention tile's operand traffic, on random and on zero operand values
    (libddt_ceiling.so, csrc/ceiling.hip); prints one JSON line."""
    import ctypes
    from tree_verify_mla_ddt_amd import build as libbuild
    if not os.path.exists(libbuild.CEILING_PATH):
        raise SystemExit("libddt_ceiling.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(libbuild.CEILING_PATH)
    lib.ddt_ceiling_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.ddt_ceiling_run.restype = ctypes.c_int
    res = {}
    for random in (1, 0):
        for mode, label in CEILING_MODES.items():
            tf, cyc = ctypes.c_double(), ctypes.c_double()
            n = iters if mode == 0 else iters // 2
            rc = lib.ddt_ceiling_run(mode, n, random, ctypes.byref(tf), ctypes.byref(cyc))
            if rc != 0:
                raise SystemExit(f"ddt_ceiling_run failed ({rc})")
            key = f"mode{mode}_{'random' if random else 'zero'}"
            res[key] = {"what": label, "tflops": round(tf.value, 1),
                        "frac_of_2500": round(tf.value / PEAK_BF16_TFLOPS, 4),
                        "cycles_per_mfma": round(cyc.value, 2)}
            log(f"[ceiling] {key}: {tf.value:.0f} TFLOP/s, {cyc.value:.1f} cycles per MFMA ({label})")
    print(json.dumps({"ceiling": res}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_inputs(wl):
    f = lambda t: t.float().numpy()
    return f(wl.q_lat), f(wl.q_pe), f(wl.c_kv), f(wl.k_pe)


def cpu_full_steps(wl, tgt_host, budget_s, max_reps=1000):
    """The oracle running whole steps of the workload (tree build, attention over
    every row in fp64, accept) until about `budget_s` of work; at least one."""
    import oracle
    q_lat, q_pe, c_kv, k_pe = _oracle_inputs(wl)
    reps, t_total = 0, 0.0
    t_build = t_attn = t_acc = 0.0
    while (t_total < budget_s or reps == 0) and reps < max_reps:
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
    return {"steps_per_s": round(reps / t_total, 4), "steps": reps, "seconds": round(t_total, 2),
            "build_ms": round(t_build / reps * 1e3, 3), "attn_ms": round(t_attn / reps * 1e3, 2),
            "accept_ms": round(t_acc / reps * 1e3, 4)}


def cpu_sampled_step(wl, tgt_host, budget_s, seed=0):
    """A whole oracle step of the workload estimated from a bounded sample: the
    tree build and the accept run in full; the attention is timed on rows drawn
    uniformly from all B*Q*H rows (doubling the sample until it takes about
    `budget_s`) and scaled to every row."""
    import oracle
    q_lat, q_pe, c_kv, k_pe = _oracle_inputs(wl)
    t0 = time.perf_counter()
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    t1 = time.perf_counter()
    oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"], tgt_host)
    t2 = time.perf_counter()
    total_rows = wl.B * wl.Q * wl.H
    rng = np.random.default_rng(seed)
    n, t_rows, done = min(16, total_rows), 0.0, 0
    while True:
        idx = (np.arange(total_rows) if n == total_rows
               else rng.integers(0, total_rows, size=n))
        rows = np.stack([idx // (wl.Q * wl.H), (idx // wl.H) % wl.Q, idx % wl.H], axis=1)
        ta = time.perf_counter()
        oracle.verify_attn(q_lat, q_pe, c_kv, k_pe, wl.req_to_slot, wl.prefix_len, t["n_nodes"],
                           t["vis"], wl.sm_scale, rows=rows)
        t_rows += time.perf_counter() - ta
        done += n
        if t_rows >= budget_s or n == total_rows:
            break
        n = min(2 * n, total_rows)
    per_step = (t1 - t0) + (t2 - t1) + t_rows / done * total_rows
    return {"steps_per_s": round(1.0 / per_step, 4), "rows_evaluated": done,
            "rows_per_step": total_rows, "seconds": round(t_rows + t2 - t0, 2)}


def cpu_baseline(name, wl, tgt_host, budget_s=12.0, single_budget_s=6.0):
    """The oracle on the host cores at the headline workload: whole steps on all
    the threads the oracle runs with, then on one thread."""
    import oracle
    threads = oracle.num_threads()
    full = cpu_full_steps(wl, tgt_host, budget_s)
    oracle.set_num_threads(1)
    try:
        single = cpu_full_steps(wl, tgt_host, single_budget_s)
    finally:
        oracle.set_num_threads(threads)
    return {"value": full["steps_per_s"], "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": (f"{full['steps']} full steps of {name} (tree build, attention over all "
                       f"{wl.B * wl.Q * wl.H} rows in fp64, accept) in {full['seconds']} s on "
                       f"{threads} threads; per step build {full['build_ms']} ms, attention "
                       f"{full['attn_ms']} ms, accept {full['accept_ms']} ms"),
            "cpu_model": cpu_model(),
            "single_core": {"value": single["steps_per_s"], "unit": "steps/s", "cores": 1,
                            "sample": f"{single['steps']} full steps in {single['seconds']} s"}}


def cpu_config_estimate(wl, tgt_host, budget_s=2.0):
    """Oracle steps/s of a workload on all threads and on one, each from a
    bounded row sample (cpu_sampled_step)."""
    import oracle
    threads = oracle.num_threads()
    allc = cpu_sampled_step(wl, tgt_host, budget_s)
    oracle.set_num_threads(1)
    try:
        one = cpu_sampled_step(wl, tgt_host, budget_s, seed=1)
    finally:
        oracle.set_num_threads(threads)
    return {"steps_per_s": allc["steps_per_s"], "cores": threads,
            "rows_evaluated": allc["rows_evaluated"], "rows_per_step": allc["rows_per_step"],
            "single_core_steps_per_s": one["steps_per_s"],
            "single_core_rows_evaluated": one["rows_evaluated"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="headline step replays per timed repeat (5 repeats)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only-primary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of HIP graph replays (for profilers)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for byte counters)")
    ap.add_argument("--workload", default=PRIMARY,
                    help="headline workload (default: the batch-1 configuration)")
    ap.add_argument("--ceiling", action="store_true",
                    help="run the MFMA / attention-tile ceiling microbenchmark and exit")
    ap.add_argument("--kernel-timing-only", action="store_true",
                    help="run only the live kernel timing of the workload (the attention "
                         "kernel, then the merge kernel, each launched --steps times back to "
                         "back per repeat) and print it: a profiler's trace of this command "
                         "holds exactly the launches the roofline's kernel time comes from")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="record the workload's HBM bytes per attention call from two "
                         "rocprofv3 --pmc output directories (FETCH_SIZE, WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(args.workload, *args.traffic_from)
        return
    if args.ceiling:
        run_ceiling()
        return
    if args.gpus != 1:
        print(f"bench.py: the verify step runs on one GPU; --gpus {args.gpus} is not "
              f"supported (no sharding or collectives across GPUs).", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("bench.py: --steps must be >= 1 and --warmup >= 0")

    import torch
    import tree_verify_mla_ddt_amd as ddt
    from tree_verify_mla_ddt_amd import workloads
    ddt.load_library()
    log(f"[bench] device {torch.cuda.get_device_name(0)}, {ddt.version()}")

    primary = args.workload
    runner = StepRunner(primary, torch, ddt, workloads)
    if args.kernel_timing_only:
        runner.kernel_times(args.steps, repeats=1)  # warm-up
        torch.cuda.synchronize()
        t_kern, t_merge = runner.kernel_times(args.steps)
        print(json.dumps({"workload": primary, "attn_kernel_us": t_kern.summary(),
                          "merge_kernel_us": t_merge.summary()}))
        return
    if args.copy_calibration:
        src = torch.empty((256 << 20,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.eager:
        # Eager launches only (profilers see every kernel of every step).
        t_step = runner.time_eager(runner.step, args.steps, args.warmup, repeats=1)
        t_call = runner.time_eager(runner.attn, args.steps, args.warmup, repeats=1)
        t_kern, t_merge = runner.kernel_times(args.steps, repeats=1)
        roof = runner.roofline(t_kern.ms, t_merge.ms, t_call.ms, primary)
    else:
        t_step, t_call, t_kern, t_merge, roof = runner.measure(args.steps, args.warmup)
    t_eager = runner.time_eager(runner.step, min(args.steps, MIN_REPLAYS), 5)
    log(f"[bench] {primary}: step {t_step.ms * 1e3:.1f} us (graph; repeats "
        f"{t_step.per[0] * 1e3:.1f}-{t_step.per[-1] * 1e3:.1f}), {t_eager.ms * 1e3:.1f} us "
        f"(eager), attention call {t_call.ms * 1e3:.1f} us, kernel {t_kern.ms * 1e3:.1f} us "
        f"+ merge {t_merge.ms * 1e3:.1f} us")
    wl = runner.wl
    result = {
        "metric": METRIC, "value": round(1000.0 / t_step.ms, 2), "unit": "steps/s",
        "n_gpus": 1, "steps": args.steps, "repeats": len(t_step.per), "warmup": args.warmup,
        "ms_per_step": round(t_step.ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": primary, "batch": wl.B, "heads": wl.H,
                   "prefix": int(wl.prefix_len[0]), "q_len": wl.Q, "drafter": f"{wl.D}x{wl.K}",
                   "kv": f"{wl.dtype} {wl.d_lat}+{wl.d_rope}",
                   "step": "tree_build -> verify_attn -> tree_accept, HIP graph replay"},
        "roofline": roof,
        "step_us": t_step.summary(),
        "attn_call_us": t_call.summary(),
        "attn_kernel_us": t_kern.summary(),
        "merge_kernel_us": t_merge.summary(),
        "step_eager_us": t_eager.summary(),
        # The same step four times in one graph: the replay period per step
        # without the per-launch cost of a graph (what a step embedded in a
        # larger captured loop would take).
        "step_x4_graph_us": runner.steps_in_one_graph(4).summary(),
        "kv_commit_step_ms": round(runner.commit_ms(), 5),
        "draft_topk": runner.topk_stats(),
        "accept_sampling": runner.sampling_stats(),
    }

    cpu_cfg = {}
    do_cpu = not args.no_cpu
    if do_cpu:
        log("[bench] timing the CPU oracle on the headline workload ...")
        tgt_host = runner.tgt.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(primary, wl, tgt_host)
        cpu_cfg[primary] = cpu_config_estimate(wl, tgt_host)
        log(f"[bench] oracle: {result['cpu_baseline']['value']} steps/s on "
            f"{result['cpu_baseline']['cores']} threads, "
            f"{result['cpu_baseline']['single_core']['value']} on one")

    extras = {}
    if not args.only_primary:
        del runner
        torch.cuda.empty_cache()
        for name in [n for n in [PRIMARY] + EXTRA if n != primary]:
            r = StepRunner(name, torch, ddt, workloads)
            t_s, t_c, t_k, t_m, rf = r.measure(MIN_REPLAYS, 5)
            extras[name] = {"steps_per_s": round(1000.0 / t_s.ms, 2),
                            "ms_per_step": round(t_s.ms, 5),
                            "requests_per_s": round(r.wl.B * 1000.0 / t_s.ms, 1),
                            "heads": r.wl.H, "dtype": r.wl.dtype,
                            "step_us": t_s.summary(), "attn_call_us": t_c.summary(),
                            "attn_kernel_us": t_k.summary(), "merge_kernel_us": t_m.summary(),
                            "roofline": rf,
                            "kv_commit_step_ms": round(r.commit_ms(), 5),
                            "draft_topk": r.topk_stats(),
                            "accept_sampling": r.sampling_stats()}
            log(f"[bench] {name}: step {t_s.ms * 1e3:.1f} us, attention kernel "
                f"{t_k.ms * 1e3:.1f} us = {rf['achieved']:.1f} {rf['unit']} "
                f"({100 * rf['frac']:.1f}% of {rf['peak']}), call {t_c.ms * 1e3:.1f} us "
                f"({100 * rf['call_frac']:.1f}%)")
            if do_cpu:
                cpu_cfg[name] = cpu_config_estimate(r.wl, r.tgt.cpu().numpy())
                log(f"[bench] oracle {name}: {cpu_cfg[name]['steps_per_s']} steps/s "
                    f"(estimated from {cpu_cfg[name]['rows_evaluated']} of "
                    f"{cpu_cfg[name]['rows_per_step']} rows)")
            del r
            torch.cuda.empty_cache()
        result["extra_workloads"] = extras
    if do_cpu:
        result["cpu_baseline"]["per_config"] = cpu_cfg
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
