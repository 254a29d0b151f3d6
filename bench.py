"""Benchmark: draft-verify steps/s of the tree step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = jt_topw_per_depth (draft logits) -> jt_build_tree_mask -> jt_tree_attention
-> jt_verify_greedy (target logits), all sequences, run as one jt_draft_verify_step
call (the same four steps in two or three launches; bf16 or fp32).  The tree
(parent, tokens) is an input of the step, built by the seeded workload generator, and is
not timed.  Inputs are resident in HBM before the timed region; step i reads input set
i mod n, with n sets whose total exceeds twice the 256 MB last-level cache where memory
allows (cold-cache figures).

Every figure is timed with HIP events on the stream the work runs on.  A hipGraph holds
exactly K steps (or K launches of one entry point); after W untimed steps it is replayed
R times, each replay bracketed by its own event pair, so every timed region is exactly K
steps.  The reported time per step is the median replay over K; the line also gives the
mean, p10 and p90 over the replays and the number of steps timed (R * K).

The JSON line reports the low-budget workload (B=16) as the headline; high_budget
(B=256), tiny, ragged and moe_verify each get an object of their own with the same
figures: steps/s, each entry point alone (calls[*].us, the roofline's per-launch time;
"step" is jt_draft_verify_step), the attention roofline (GB/s or TFLOP/s) and the
oracle timed on this host ("cpu_baseline": the whole step for the light workloads, a
stated sample scaled to one step for the heavy ones).  "measured_peaks" holds this
device's copy bandwidth and sustained bf16 matrix-core rate beside the nominal peaks.

Profiling modes (their output feeds the summaries kept under profiles/):
  --calls-only          time each entry point alone, nothing else (for a kernel trace)
  --traffic-run NAME    launch each entry point of workload NAME on cold input sets,
                        then a 1 GiB device-to-device copy that calibrates the
                        FETCH_SIZE / WRITE_SIZE counters (run under rocprofv3 --pmc)
  --traffic-summarize NAME FETCH_DIR WRITE_DIR
                        HBM bytes per launch from those two counter runs
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
LLC_BYTES = 256 << 20        # Infinity Cache
CALLS = ("topw", "mask", "attention", "verify")
KERNELS = {
    "topw": ["topw_partial_kernel", "topw_merge_kernel"],
    "mask": ["build_mask_kernel"],
    "attention": ["attn_bf16_kernel", "attn_combine_kernel", "attn_f32_kernel"],
    "verify": ["argmax_partial_kernel", "verify_walk_kernel"],
    "step": ["step_phase1", "step_scan_kernel", "step_phase2"],
    "tree": ["tree_build_kernel"],
    "commit": ["commit_kv_kernel"],
    "sampled": ["sample_partial_kernel", "sample_select_kernel", "verify_walk_kernel"],
}
# the kernel whose dispatches count the launches of each entry point
MARKER = {"topw": "topw_partial_kernel", "mask": "build_mask_kernel",
          "attention": ("attn_bf16_kernel", "attn_f32_kernel"),
          "verify": "argmax_partial_kernel", "step": "step_phase2", "tree": "tree_build_kernel",
          "commit": "commit_kv_kernel", "sampled": "sample_select_kernel"}


def algorithmic(w):
    """Bytes each entry point must move and the attention flops (visible keys only)."""
    c = w.cfg
    e = 4 if c.dtype == "f32" else 2
    S, B, N, W, V = c.S, c.B, c.N, c.W, c.V
    P = w.prefix_len.astype(np.int64)
    b = {}
    b["topw"] = S * N * V * e + S * N * W * 8 + S * N * 4
    b["mask"] = S * B * (4 + 32 + 4) + S * 4
    b["attention"] = (int(((P + B) * c.Hkv * c.d * 2 * e).sum()) + S * B * c.Hq * c.d * 2 * e
                      + S * B * 32 + S * B * c.Hq * 4 + S * 4 * 2
                      + (0 if w.block_table is None else int(np.ceil(P / c.block_size).sum()) * 4))
    b["verify"] = S * B * V * e + S * B * (4 + 4 + 32 + 4 + 4) + S * (N + 1 + 3) * 4
    vis = (P[:, None] + w.depth.astype(np.int64) + 1).sum()
    flops = 4 * c.Hq * c.d * int(vis)
    b["step"] = b["topw"] + b["mask"] + b["attention"] + b["verify"]
    # best-first tree from the top-W lists: ids + log-probs read; parent, tokens, score
    # and the node count written
    b["tree"] = S * N * W * 8 + S * B * 12 + S * 4
    # stochastic verification: the target rows once (the rescan of one 8192-logit piece
    # per row is not counted), the uniforms, and the outputs of greedy verification
    b["sampled"] = b["verify"] + S * B * 4
    return b, flops


class Rotation:
    """Several copies of one step's inputs (same values) so reps do not hit in cache."""

    def __init__(self, step, nsets):
        import torch
        self.steps = [step]
        names = [n for n in ("draft", "q", "k_tree", "v_tree", "k_prefix", "v_prefix", "target")
                 if hasattr(step, n)]
        for _ in range(nsets - 1):
            clone = object.__new__(type(step))
            clone.__dict__.update(step.__dict__)
            for n in names:
                setattr(clone, n, getattr(step, n).clone())
            self.steps.append(clone)
        torch.cuda.synchronize()


def footprint(step):
    tot = 0
    for n in ("draft", "q", "k_tree", "v_tree", "k_prefix", "v_prefix", "target"):
        t = getattr(step, n, None)
        if t is not None:
            tot += t.numel() * t.element_size()
    return tot


def _capture(fns):
    """One hipGraph that runs every callable in ``fns`` in order on a capture stream."""
    import torch
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for f in fns:
            f()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    torch.cuda.synchronize()
    return g


def _replays(K):
    """Replays of a K-step graph: enough for a spread, about 200 steps in all."""
    return max(5, math.ceil(200 / max(1, K)))


def _time_graph(g, K, warmup, replays=None):
    """Times replays of a graph holding K steps (or K launches) back-to-back on the current
    stream, each replay between its own pair of HIP events on that stream.  Returns the
    per-step times (us) of the replays."""
    import torch
    cur = torch.cuda.current_stream()
    for _ in range(max(1, math.ceil(warmup / max(1, K)))):
        g.replay()
    torch.cuda.synchronize()
    R = replays or _replays(K)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(R)]
    for a, b in ev:
        a.record(cur)
        g.replay()
        b.record(cur)
    torch.cuda.synchronize()
    return [1e3 * a.elapsed_time(b) / K for a, b in ev]


def _stats(per_step_us, K):
    """Median, mean and spread of per-step times from replays of K steps."""
    x = np.asarray(per_step_us, np.float64)
    return {"us_median": round(float(np.median(x)), 3), "us_mean": round(float(x.mean()), 3),
            "us_p10": round(float(np.percentile(x, 10)), 3),
            "us_p90": round(float(np.percentile(x, 90)), 3), "replays": len(x),
            "steps_per_replay": K, "steps_timed": len(x) * K}


def _k_of(rot, K, fn_name):
    """K callables, step i on cold input set i mod n."""
    return [getattr(rot.steps[i % len(rot.steps)], fn_name) for i in range(K)]


def time_workload(name, steps, warmup, seed, log=print, calls_only=False):
    import torch
    from tree_causal_draft_amd import workload as wl
    from tree_causal_draft_amd.step import DeviceStep

    t0 = time.time()
    w = wl.make(name, seed)
    log(f"[bench] {name}: inputs generated in {time.time() - t0:.1f}s")
    st = DeviceStep(w, "cuda:0")
    fp = footprint(st)
    nsets = max(1, min(64, steps, math.ceil(2 * LLC_BYTES / max(fp, 1))))
    rot = Rotation(st, nsets)
    log(f"[bench] {name}: footprint {fp / 1e6:.1f} MB per set, {nsets} sets rotated")
    cur = torch.cuda.current_stream()
    if calls_only:
        res = _time_calls(name, w, rot, st, steps, warmup, log)
        res.update(eager_us=None, step_stats=None, serial_us=None, conc_us=None,
                   fused_us=None, graph_ok=None, step_us=None)
        return res

    # ---- eager reference run (also the graph-vs-eager check)
    for i in range(max(warmup, nsets)):
        rot.steps[i % nsets].run()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for i in range(steps):
        rot.steps[i % nsets].run()
    b.record(cur)
    torch.cuda.synchronize()
    eager_us = 1e3 * a.elapsed_time(b) / steps

    def got_bufs():
        return [st.accept_len, st.bonus, st.accept_path, st.ids, st.logprob, st.attn_out, st.anc]
    ref = [t.clone() for t in got_bufs()]

    # ---- whole step: one graph holding exactly `steps` steps (step i on cold set i mod n);
    # the four calls on one stream, the four calls with their independence exposed (top-W
    # and verification on side streams), and the fused call where it applies (reported)
    def graph_step(fn_name):
        g = _capture(_k_of(rot, steps, fn_name))
        per = _time_graph(g, steps, warmup)
        for t in got_bufs():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        ok = all(torch.equal(x, y) for x, y in zip(ref, got_bufs()))
        del g
        return per, ok

    serial, serial_ok = graph_step("run")
    conc, conc_ok = graph_step("run_concurrent")
    fused, fused_ok = None, True
    if hasattr(st, "step_ws"):
        fused, fused_ok = graph_step("run_fused")
    graph_ok = serial_ok and conc_ok and fused_ok
    step_per = fused if fused is not None else conc
    med = lambda x: None if x is None else float(np.median(x))
    log(f"[bench] {name}: eager {eager_us:.2f} us/step, graph one-stream {med(serial):.2f}, "
        f"concurrent {med(conc):.2f}, fused {med(fused)} us/step (median of replays of "
        f"{steps} steps), replay == eager: {graph_ok}")

    res = _time_calls(name, w, rot, st, steps, warmup, log)
    res.update(eager_us=eager_us, step_stats=_stats(step_per, steps), serial_us=med(serial),
               conc_us=med(conc), fused_us=med(fused), graph_ok=graph_ok)
    res["step_us"] = res["step_stats"]["us_median"]
    return res


def _time_calls(name, w, rot, st, steps, warmup, log):
    import torch
    # ---- each entry point alone: one graph of exactly `steps` launches (launch i on cold
    # input set i mod n)
    per_call_us, call_stats = {}, {}
    calls_here = CALLS + (("step",) if hasattr(st, "step_ws") else ()) + \
        (("tree",) if hasattr(st, "tree_parent") else ()) + \
        (("commit",) if hasattr(st, "commit_k") else ()) + \
        (("sampled",) if hasattr(st, "smp_ws") else ())
    st.run()  # the tree call reads the top-W lists, the commit the accepted paths
    for c in calls_here:
        g = _capture(_k_of(rot, steps, "run_fused" if c == "step" else c))
        per = _time_graph(g, steps, warmup)
        del g
        call_stats[c] = _stats(per, steps)
        per_call_us[c] = call_stats[c]["us_median"]
    log(f"[bench] {name}: per call " + " ".join(f"{c}={per_call_us[c]:.2f}us" for c in calls_here))

    bytes_, flops = algorithmic(w)
    if "commit" in calls_here:
        # the accepted paths' K and V rows, read and written, plus lengths and paths
        rows = int((st.accept_len.cpu().numpy().astype(np.int64) + 1).sum())
        e = 4 if w.cfg.dtype == "f32" else 2
        bytes_["commit"] = rows * w.cfg.Hkv * w.cfg.d * e * 4 + w.cfg.S * (w.cfg.N + 1 + 4) * 4
    calls = {}
    for c in calls_here:
        us = per_call_us[c]
        calls[c] = {"us": round(us, 3), "us_p10": call_stats[c]["us_p10"],
                    "us_p90": call_stats[c]["us_p90"], "bytes": int(bytes_[c]),
                    "GBps": round(bytes_[c] / (us * 1e-6) / 1e9, 1)}
    att_us = per_call_us["attention"]
    calls["attention"]["TFLOPs"] = round(flops / (att_us * 1e-6) / 1e12, 2)
    calls["attention"]["flops"] = int(flops)
    res = dict(workload=name, w=w, calls=calls, nsets=len(rot.steps), flops=flops,
               bytes=bytes_, per_call_us=per_call_us, footprint=footprint(st))
    del rot, st
    torch.cuda.empty_cache()
    return res


def roofline(res, call, peaks=None):
    """Roofline of one entry point: the binding resource is the one whose floor (bytes at
    the HBM peak, or flops at the bf16 MFMA peak) is longer.  `frac_measured` relates the
    same rate to this device's measured ceiling (copy bandwidth or matrix-core loop)."""
    w = res["w"]
    us = res["per_call_us"][call]
    byt = res["bytes"][call]
    peaks = peaks or {}
    if call in ("attention", "step"):
        ai = res["flops"] / byt
        if ai > (MFMA_BF16_PEAK_TFS * 1e12) / (HBM_PEAK_GBS * 1e9) and w.cfg.dtype == "bf16":
            ach = res["flops"] / (us * 1e-6) / 1e12
            m = peaks.get("mfma_bf16_TFLOPs")
            return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                    "frac_measured": round(ach / m, 4) if m else None,
                    "kernel": call, "kernels": KERNELS[call], "per_launch_us": round(us, 2)}
    ach = byt / (us * 1e-6) / 1e9
    m = peaks.get("copy_GBps")
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
            "frac_measured": round(ach / m, 4) if m else None, "kernel": call,
            "kernels": KERNELS[call], "per_launch_us": round(us, 2)}


def cpu_baseline(name, seed, budget_s=20.0, log=print, w=None):
    """The CPU oracle, single-threaded, timed on the same workload's inputs, stage by stage.

    Light workloads run whole steps, repeated until `budget_s` is spent (at most 50).  For
    the heavy ones a step is timed on a stated sample and scaled: top-W on the first rows
    (scaled by the row count), the mask whole, attention on every k-th tree node of every
    sequence and head (scaled by the visible keys, i.e. the flops), and verification whole.
    """
    import oracle
    from tree_causal_draft_amd import workload as wl
    w = wl.make(name, seed) if w is None else w
    c = w.cfg
    rows = c.S * c.N
    # samples sized from the oracle's measured speed here (~35 ms per 151,936-logit row,
    # ~1 GFLOP/s of attention) so that one sampled step costs a few seconds
    rows_s = min(rows, max(1, int(64 * 151936 / max(c.V, 1))))
    P = w.prefix_len.astype(np.int64)
    vis = P[:, None] + w.depth.astype(np.int64) + 1              # keys visible per node
    flops = 4.0 * c.Hq * c.d * vis.sum()
    k = max(1, math.ceil(flops / 4e9))
    nodes = np.arange(0, c.B, k)
    sel = np.stack(np.meshgrid(np.arange(c.S), nodes, np.arange(c.Hq), indexing="ij"),
                   -1).reshape(-1, 3).astype(np.int32)
    flops_s = 4.0 * c.d * vis[:, nodes].sum() * c.Hq
    draft = w.draft_logits[:rows_s]
    kw = dict(block_table=w.block_table, block_size=c.block_size, num_blocks=w.num_blocks,
              max_prefix=w.max_prefix)
    stages = {"topw": [], "mask": [], "attention": [], "verify": []}
    t_all = time.perf_counter()
    while not stages["verify"] or (time.perf_counter() - t_all < budget_s
                                   and len(stages["verify"]) < 50):
        t = time.perf_counter()
        oracle.topw(draft, c.W)
        t1 = time.perf_counter()
        oracle.build_mask(w.parent)
        t2 = time.perf_counter()
        oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix, w.prefix_len,
                              w.parent, sel=None if k == 1 else sel, **kw)
        t3 = time.perf_counter()
        oracle.verify_greedy(w.target_logits, w.parent, w.tokens, c.N)
        t4 = time.perf_counter()
        for st_, dt in zip(stages, (t1 - t, t2 - t1, t3 - t2, t4 - t3)):
            stages[st_].append(dt)
    scale = {"topw": rows / rows_s, "mask": 1.0, "attention": flops / flops_s, "verify": 1.0}
    per = {st_: float(np.mean(v)) * scale[st_] for st_, v in stages.items()}
    sec = sum(per.values())
    n = len(stages["verify"])
    whole = rows_s == rows and k == 1
    sample = (f"{n} whole steps of {name} (seed {seed})" if whole else
              f"{n} sampled step(s) of {name} (seed {seed}): top-W on {rows_s} of {rows} rows "
              f"(x{rows / rows_s:.2f}), mask whole, attention on nodes v % {k} == 0 of every "
              f"sequence and head (x{flops / flops_s:.2f} by visible keys), verify whole")
    log(f"[bench] cpu oracle {name}: {sec:.3f} s/step ({sample})")
    return {"value": round(1.0 / sec, 5), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": sample + ", single thread",
            "stage_seconds": {k2: round(v, 4) for k2, v in per.items()},
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _kernel_hash(call):
    import hashlib
    files = {"topw": ["topw.hip"], "mask": ["mask.hip"], "attention": ["attn.hip"],
             "verify": ["verify.hip"],
             "step": ["mask.hip", "topw.hip", "verify.hip", "attn.hip", "step.hip"],
             "tree": ["tree.hip"], "commit": ["commit.hip"],
             "sampled": ["verify.hip", "sample.hip"]}[call]
    import re
    h = hashlib.sha256()
    for f in files + ["jt_internal.h"]:
        with open(os.path.join(ROOT, "tree_causal_draft_amd", "csrc", f)) as fh:
            src = fh.read()
        # the code only: comments and layout do not change what the counters measured
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def traffic(workload, call):
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel factor), or None when no summary exists or the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)["entries"][workload][call]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("src_sha") != _kernel_hash(call):
        return None
    return int(rec["bytes_per_launch"])


def roofline_line(res, call, peaks=None):
    r = roofline(res, call, peaks)
    r["traffic"] = traffic(res["workload"], call)
    return r


CALIB_BYTES = 1 << 30


def traffic_run(name, seed, reps=3, log=print):
    """Launch every entry point of one workload eagerly on cold input sets, then one
    1 GiB device-to-device copy (the counter calibration).  Meant to run under
    ``rocprofv3 --pmc FETCH_SIZE`` and, separately, ``--pmc WRITE_SIZE``."""
    import torch
    from tree_causal_draft_amd import workload as wl
    from tree_causal_draft_amd.step import DeviceStep
    w = wl.make(name, seed)
    st = DeviceStep(w, "cuda:0")
    nsets = max(1, min(64, math.ceil(2 * LLC_BYTES / max(footprint(st), 1))))
    rot = Rotation(st, nsets)
    extra = ("tree",) + (("commit",) if hasattr(st, "commit_k") else ()) + \
        (("sampled",) if hasattr(st, "smp_ws") else ())
    for c in CALLS + (("run_fused",) if hasattr(st, "step_ws") else ()) + extra:
        for i in range(reps * nsets):
            getattr(rot.steps[i % nsets], c)()
        torch.cuda.synchronize()
    del rot, st
    torch.cuda.empty_cache()
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] traffic run {name}: {reps} x {nsets} launches per entry point, "
        f"then a {CALIB_BYTES >> 20} MiB copy")


def _counter_rows(path, counter):
    """(dispatch_id, kernel_name, value summed over the dispatch) from a rocprofv3 db."""
    import glob
    import sqlite3
    dbs = sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))
    if not dbs:
        raise FileNotFoundError(f"no rocprofv3 database under {path}")
    con = sqlite3.connect(dbs[0])
    rows = con.execute("select dispatch_id, kernel_name, sum(value) from counters_collection "
                       "where counter_name = ? group by dispatch_id, kernel_name "
                       "order by dispatch_id", (counter,)).fetchall()
    con.close()
    return rows


def traffic_summarize(name, fetch_dir, write_dir):
    """Per entry point, HBM bytes per launch = (FETCH_SIZE + WRITE_SIZE) KiB over the entry
    point's dispatches, divided by its launch count, each counter scaled by (bytes the
    calibration copy moved) / (what the counter read for it).  The traffic run launches the
    entry points one after the other (top-W, mask, attention, verify, the fused step, the
    tree builder, the commit, the stochastic verifier), so dispatches are assigned in order:
    a dispatch stays with the current entry point while its kernel is one of that entry
    point's (the step's 8-wave shapes run attn_bf16_kernel, the stochastic verifier runs
    verify_walk_kernel) and moves to the next entry point it matches otherwise."""
    order = list(CALLS) + ["step", "tree", "commit", "sampled"]
    def hits(kname, call):
        return any(k in kname for k in KERNELS[call])
    def is_marker(kname, call):
        m = MARKER[call]
        return any(k in kname for k in (m if isinstance(m, tuple) else (m,)))
    out = {"counters": {}}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(path, counter)
        ours = [r for r in rows if any(hits(r[1], c) for c in order)]
        last = max(r[0] for r in ours)
        calib = [r for r in rows if r[0] > last and "copyBuffer" in r[1]]
        if not calib:
            raise RuntimeError(f"{counter}: no calibration copy after the last step kernel")
        kib = sum(r[2] for r in calib)
        factor = CALIB_BYTES / (kib * 1024.0)
        out["counters"][counter] = {"calibration_kib": kib, "scale": factor}
        cur = 0
        tot = {c: 0.0 for c in order}
        cnt = {c: 0 for c in order}
        for did, kname, val in ours:
            if not hits(kname, order[cur]):  # a kernel of a later entry point: move on
                for k in range(cur + 1, len(order)):
                    if hits(kname, order[k]):
                        cur = k
                        break
            call = order[cur]
            tot[call] += val
            cnt[call] += 1 if is_marker(kname, call) else 0
        for call in order:
            if cnt[call]:
                per.setdefault(call, {})[counter] = tot[call] * 1024.0 * factor / cnt[call]
                per[call]["launches"] = cnt[call]
    out["entries"] = {}
    for call, d in per.items():
        if "FETCH_SIZE" in d and "WRITE_SIZE" in d:
            out["entries"][call] = {
                "fetch_bytes_per_launch": int(d["FETCH_SIZE"]),
                "write_bytes_per_launch": int(d["WRITE_SIZE"]),
                "bytes_per_launch": int(d["FETCH_SIZE"] + d["WRITE_SIZE"]),
                "launches": d["launches"], "src_sha": _kernel_hash(call)}
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            allrec = json.load(fh)
    except (OSError, ValueError):
        allrec = {"entries": {}, "counters": {}}
    allrec["entries"][name] = out["entries"]
    allrec["counters"][name] = out["counters"]
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({name: out}, indent=1, sort_keys=True))


def attention_only(name, seed, reps=20, log=print):
    """The attention call alone on one workload (graph replay over cold input sets, as the
    per-call timing): for the parity configurations that are not bench lines."""
    import torch
    from tree_causal_draft_amd import workload as wl
    from tree_causal_draft_amd.step import DeviceStep
    w = wl.make(name, seed, parts=("attn",))
    st = DeviceStep(w, "cuda:0", parts=("mask", "attn"))
    st.mask()
    fp = sum(getattr(st, n).numel() * getattr(st, n).element_size()
             for n in ("q", "k_tree", "v_tree", "k_prefix", "v_prefix"))
    nsets = max(1, min(32, math.ceil(2 * LLC_BYTES / fp)))
    rot = Rotation(st, nsets)
    K = reps * nsets
    g = _capture(_k_of(rot, K, "attention"))
    us = float(np.median(_time_graph(g, K, nsets)))
    b, fl = algorithmic(w)
    tf = fl / us / 1e6
    log(f"[bench] {name}: attention {us:.2f} us/call over {nsets} cold sets")
    return {"workload": name, "attention_us": round(us, 2), "TFLOPs": round(tf, 1),
            "mfma_frac": round(tf / 2500.0, 4), "GBps": round(b["attention"] / us / 1e3, 1)}


def copy_bandwidth(nbytes=1 << 30, reps=20):
    """Device-to-device copy rate (bytes read + written per second, GB/s) of one GiB on
    this GPU: the practical HBM ceiling that the 8 TB/s peak is quoted beside."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    t1.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / us / 1e3, 1)


def mfma_rate(iters=4000, blocks=1024, reps=10, warmup=10):
    """Sustained bf16 matrix-core rate (TFLOP/s) of the library's probe kernel: 4 waves per
    SIMD, each issuing independent v_mfma_f32_32x32x16_bf16; the best of `reps` runs after
    `warmup` untimed ones (the clock settles under load)."""
    import torch
    import tree_causal_draft_amd as jt
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    flops = blocks * 4 * iters * 8 * 32768.0
    for _ in range(warmup):
        jt.probe_mfma_rate(iters, blocks, out)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        jt.probe_mfma_rate(iters, blocks, out)
        t1.record()
        t1.synchronize()
        best = max(best, flops / (t0.elapsed_time(t1) * 1e-3) / 1e12)
    return round(best, 1)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="low_budget")
    ap.add_argument("--secondary", default="high_budget,tiny,ragged,moe_verify",
                    help="comma-separated workloads reported beside the headline ('' for none)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--calls-only", action="store_true")
    ap.add_argument("--traffic-run", metavar="NAME")
    ap.add_argument("--attention-only", metavar="NAME[,NAME...]",
                    help="time the attention call alone on these workloads")
    ap.add_argument("--traffic-summarize", nargs=3, metavar=("NAME", "FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the step has no multi-GPU path here "
              "(sequences and KV groups would shard with no exchange).", file=sys.stderr)
        sys.exit(2)
    if args.traffic_summarize:
        traffic_summarize(*args.traffic_summarize)
        return

    import torch
    import tree_causal_draft_amd as jt
    from tree_causal_draft_amd import workload as wl
    jt.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    log = lambda m: print(m, file=sys.stderr, flush=True)
    seed_of = lambda n: 1000 * (wl.CONFIG_ORDER.index(n) + 1)
    if args.traffic_run:
        traffic_run(args.traffic_run, seed_of(args.traffic_run), log=log)
        return
    if args.attention_only:
        for n in args.attention_only.split(","):
            print(json.dumps(attention_only(n, seed_of(n), log=log)), flush=True)
        return

    names = [args.workload] + [n for n in args.secondary.split(",") if n and n != args.workload]
    results = [time_workload(n, args.steps, args.warmup, seed_of(n), log=log,
                             calls_only=args.calls_only) for n in names]
    peaks = {}
    if not args.calls_only:
        peaks = {"copy_GBps": copy_bandwidth(), "mfma_bf16_TFLOPs": mfma_rate(),
                 "nominal_hbm_GBps": HBM_PEAK_GBS, "nominal_mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFS}
        log(f"[bench] measured peaks: copy {peaks['copy_GBps']} GB/s, bf16 matrix cores "
            f"{peaks['mfma_bf16_TFLOPs']} TFLOP/s")
    cpu = {}
    if not args.no_cpu and not args.calls_only:
        for i, (n, r) in enumerate(zip(names, results)):
            budget = args.cpu_seconds if i == 0 else args.cpu_seconds / 2
            cpu[n] = cpu_baseline(n, seed_of(n), budget, log=log, w=r["w"])

    def summary(r):
        c = r["w"].cfg
        return f"{c.name}: S={c.S} prefix={c.prefix} B={c.B} N={c.N} W={c.W} " \
               f"heads {c.Hq}/{c.Hkv} d={c.d} V={c.V} {c.dtype}"

    def rate(us):
        return None if us is None else round(1e6 / us, 1)

    def dominant(r):
        if "step" in r["per_call_us"]:
            return "step"
        return max(CALLS, key=lambda k: r["per_call_us"][k])

    def timing(r):
        return ("hipGraph of K jt_draft_verify_step calls (step i on cold input set i mod n; "
                "two or three kernel launches each); median of the replays")

    prim = results[0]
    us = prim["step_us"]
    dom = dominant(prim)
    c = prim["w"].cfg
    line = {
        "metric": "draft-verify steps/s + tree-attn HBM GB/s / MFMA % at B=16,256 (1xMI355X)",
        "value": rate(us),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None if us is None else round(us * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c.dtype,
        "data": "synthetic (seeded; tree prebuilt, not timed)",
        "config": {"workload": summary(prim), "timing": timing(prim), "cold_sets": prim["nsets"]},
        "step_timing": prim["step_stats"],
        "eager_steps_per_s": rate(prim["eager_us"]),
        "one_stream_graph_steps_per_s": rate(prim["serial_us"]),
        "four_calls_concurrent_graph_steps_per_s": rate(prim.get("conc_us")),
        "graph_matches_eager": prim["graph_ok"],
        "calls": prim["calls"],
        "roofline": roofline_line(prim, dom, peaks),
        "attention_roofline": roofline_line(prim, "attention", peaks),
        "cpu_baseline": cpu.get(prim["workload"]),
        "measured_peaks": peaks or None,
    }
    if args.calls_only:
        line["mode"] = "calls-only (entry points timed alone; no whole-step figure)"
    for r in results[1:]:
        line[r["workload"]] = {
            "workload": summary(r),
            "timing": timing(r),
            "cold_sets": r["nsets"],
            "steps_per_s": rate(r["step_us"]),
            "step_timing": r["step_stats"],
            "eager_steps_per_s": rate(r["eager_us"]),
            "one_stream_graph_steps_per_s": rate(r["serial_us"]),
            "four_calls_concurrent_graph_steps_per_s": rate(r.get("conc_us")),
            "graph_matches_eager": r["graph_ok"],
            "calls": r["calls"],
            "attention_roofline": roofline_line(r, "attention", peaks),
            "roofline": roofline_line(r, dominant(r), peaks),
            "cpu_baseline": cpu.get(r["workload"]),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
