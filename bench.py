"""Benchmark: draft-verify steps/s of the tree step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = jt_topw_per_depth (draft logits) -> jt_build_tree_mask -> jt_tree_attention
-> jt_verify_greedy (target logits), all sequences; for bf16 it runs as one
jt_draft_verify_step call (the same four steps in two launches).  The tree (parent,
tokens) is an input of the step, built by the seeded workload generator, and is not
timed.  Inputs are resident in HBM before the timed region; input sets are rotated so
that one rotation exceeds twice the 256 MB last-level cache (cold-cache figures).

The JSON line reports the low-budget workload (B=16) as the headline and the
high-budget workload (B=256) in "high_budget".  Every figure is timed with HIP events
on the stream the work runs on, around back-to-back replays of a hipGraph that holds
one step (or one call of one entry point) per cold input set:
  value / ms_per_step   whole step (jt_draft_verify_step; the four calls with top-W and
                        verification on side streams where it does not apply)
  calls[*].us           each entry point alone (the roofline's per-launch time; "step" is
                        jt_draft_verify_step)
"cpu_baseline" times the CPU oracle (single thread) on full steps of the headline
workload.

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
    "attention": ["attn_bf16_kernel", "attn_combine_kernel", "attn_simple_kernel"],
    "verify": ["argmax_partial_kernel", "verify_walk_kernel"],
    "step": ["step_phase1", "step_scan_kernel", "step_phase2"],
    "tree": ["tree_build_kernel"],
    "commit": ["commit_kv_kernel"],
    "sampled": ["sample_partial_kernel", "sample_select_kernel", "verify_walk_kernel"],
}
# the kernel whose dispatches count the launches of each entry point
MARKER = {"topw": "topw_partial_kernel", "mask": "build_mask_kernel",
          "attention": ("attn_bf16_kernel", "attn_simple_kernel"),
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


def _time_graph(g, launches_per_replay, total_launches, warmup):
    """Average time per launch (us): the graph replayed back-to-back on the current stream,
    bracketed by HIP events on that stream."""
    import torch
    cur = torch.cuda.current_stream()
    for _ in range(max(1, warmup // max(1, launches_per_replay))):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(total_launches / launches_per_replay))
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(cur)
    for _ in range(reps):
        g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (reps * launches_per_replay), reps * launches_per_replay


def time_workload(name, steps, warmup, seed, log=print, calls_only=False):
    import torch
    from tree_causal_draft_amd import workload as wl
    from tree_causal_draft_amd.step import DeviceStep

    t0 = time.time()
    w = wl.make(name, seed)
    log(f"[bench] {name}: inputs generated in {time.time() - t0:.1f}s")
    st = DeviceStep(w, "cuda:0")
    fp = footprint(st)
    nsets = max(1, min(64, math.ceil(2 * LLC_BYTES / max(fp, 1))))
    rot = Rotation(st, nsets)
    log(f"[bench] {name}: footprint {fp / 1e6:.1f} MB per set, {nsets} sets rotated")
    cur = torch.cuda.current_stream()
    eager_us = step_us = serial_us = None
    graph_ok = None
    if calls_only:
        return _time_calls(name, w, rot, st, nsets, steps, warmup, fp, eager_us, step_us,
                           serial_us, graph_ok, log)

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
    ref = [t.clone() for t in (st.accept_len, st.bonus, st.accept_path, st.ids, st.logprob,
                               st.attn_out, st.anc)]

    # ---- whole step: one graph holding one step per input set, replayed back-to-back;
    # once with the four calls on one stream, once with their independence exposed
    # (top-W and verification on side streams), which is the reported figure
    def graph_step(fn_name):
        g = _capture([getattr(s, fn_name) for s in rot.steps])
        us, n = _time_graph(g, nsets, steps, warmup)
        for t in got_bufs():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        ok = all(torch.equal(x, y) for x, y in zip(ref, got_bufs()))
        del g
        return us, n, ok

    def got_bufs():
        return [st.accept_len, st.bonus, st.accept_path, st.ids, st.logprob, st.attn_out, st.anc]

    serial_us, nsteps, serial_ok = graph_step("run")
    conc_us, nsteps, conc_ok = graph_step("run_concurrent")
    fused_us, fused_ok = None, True
    if hasattr(st, "step_ws"):
        fused_us, nsteps, fused_ok = graph_step("run_fused")
    graph_ok = serial_ok and conc_ok and fused_ok
    step_us = fused_us if fused_us is not None else conc_us
    log(f"[bench] {name}: eager {eager_us:.1f} us/step, graph one-stream {serial_us:.1f} us/step, "
        f"graph concurrent {conc_us:.1f} us/step, fused {fused_us} us/step ({nsteps} steps), "
        f"replay == eager: {graph_ok}")

    res = _time_calls(name, w, rot, st, nsets, steps, warmup, fp, eager_us, step_us,
                      serial_us, graph_ok, log)
    res["conc_us"], res["fused_us"] = conc_us, fused_us
    return res


def _time_calls(name, w, rot, st, nsets, steps, warmup, fp, eager_us, step_us, serial_us,
                graph_ok, log):
    import torch
    # ---- each entry point alone: one graph of nsets launches (one per cold input set)
    per_call_us = {}
    calls_here = CALLS + (("step",) if hasattr(st, "step_ws") else ()) + \
        (("tree",) if hasattr(st, "tree_parent") else ()) + \
        (("commit",) if hasattr(st, "commit_k") else ()) + \
        (("sampled",) if hasattr(st, "smp_ws") else ())
    st.run()  # the tree call reads the top-W lists, the commit the accepted paths
    for c in calls_here:
        g = _capture([getattr(s, "run_fused" if c == "step" else c) for s in rot.steps])
        per_call_us[c], _ = _time_graph(g, nsets, steps, warmup)
        del g
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
        calls[c] = {"us": round(us, 3), "bytes": int(bytes_[c]),
                    "GBps": round(bytes_[c] / (us * 1e-6) / 1e9, 1)}
    att_us = per_call_us["attention"]
    calls["attention"]["TFLOPs"] = round(flops / (att_us * 1e-6) / 1e12, 2)
    calls["attention"]["flops"] = int(flops)
    res = dict(workload=name, w=w, eager_us=eager_us, step_us=step_us, serial_us=serial_us,
               graph_ok=graph_ok,
               calls=calls, nsets=nsets, flops=flops, bytes=bytes_, per_call_us=per_call_us,
               footprint=fp)
    del rot, st
    torch.cuda.empty_cache()
    return res


def roofline(res, call):
    """Roofline of one entry point: the binding resource is the one whose floor (bytes at
    the HBM peak, or flops at the bf16 MFMA peak) is longer."""
    w = res["w"]
    us = res["per_call_us"][call]
    byt = res["bytes"][call]
    if call in ("attention", "step"):
        ai = res["flops"] / byt
        if ai > (MFMA_BF16_PEAK_TFS * 1e12) / (HBM_PEAK_GBS * 1e9) and w.cfg.dtype == "bf16":
            ach = res["flops"] / (us * 1e-6) / 1e12
            return {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFS, 4), "traffic": None,
                    "kernel": call, "kernels": KERNELS[call], "per_launch_us": round(us, 2)}
    ach = byt / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": call,
            "kernels": KERNELS[call], "per_launch_us": round(us, 2)}


def cpu_baseline(name, seed, budget_s=20.0, log=print):
    """The CPU oracle, single-threaded, on full steps of the same workload."""
    import oracle
    from tree_causal_draft_amd import workload as wl
    w = wl.make(name, seed)
    c = w.cfg
    times = []
    t_all = time.perf_counter()
    while not times or (time.perf_counter() - t_all < budget_s and len(times) < 50):
        t = time.perf_counter()
        oracle.topw(w.draft_logits, c.W)
        oracle.build_mask(w.parent)
        oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix, w.prefix_len,
                              w.parent, block_table=w.block_table, block_size=c.block_size,
                              num_blocks=w.num_blocks, max_prefix=w.max_prefix)
        oracle.verify_greedy(w.target_logits, w.parent, w.tokens, c.N)
        times.append(time.perf_counter() - t)
    sec = float(np.mean(times))
    log(f"[bench] cpu oracle {name}: {sec:.2f} s/step over {len(times)} steps")
    return {"value": round(1.0 / sec, 4), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(times)} full steps of {name} (seed {seed}), single thread",
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


def roofline_line(res, call):
    r = roofline(res, call)
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
    g = _capture([s.attention for s in rot.steps])
    us, _ = _time_graph(g, nsets, reps * nsets, nsets)
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="low_budget")
    ap.add_argument("--secondary", default="high_budget", help="'' to skip")
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

    names = [args.workload] + [n for n in args.secondary.split(",") if n]
    results = [time_workload(n, args.steps, args.warmup, seed_of(n), log=log,
                             calls_only=args.calls_only) for n in names]
    cpu = None
    if not args.no_cpu and not args.calls_only:
        cpu = cpu_baseline(args.workload, seed_of(args.workload), args.cpu_seconds, log=log)
    copy_gbps = None if args.calls_only else copy_bandwidth()

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

    prim = results[0]
    us = prim["step_us"]
    dom = dominant(prim)
    c = prim["w"].cfg
    fused = prim.get("fused_us") is not None
    timing = ("hipGraph replay of one jt_draft_verify_step (two kernel launches; three when "
              "attention runs 8-wave groups) per cold input set"
              if fused else "hipGraph replay of one step per cold input set; top-W and "
              "verification on side streams")
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
        "config": {"workload": summary(prim), "timing": timing, "cold_sets": prim["nsets"]},
        "eager_steps_per_s": rate(prim["eager_us"]),
        "one_stream_graph_steps_per_s": rate(prim["serial_us"]),
        "four_calls_concurrent_graph_steps_per_s": rate(prim.get("conc_us")),
        "graph_matches_eager": prim["graph_ok"],
        "calls": prim["calls"],
        "roofline": roofline_line(prim, dom),
        "attention_roofline": roofline_line(prim, "attention"),
        "cpu_baseline": cpu,
        "copy_bandwidth_GBps": copy_gbps,
    }
    if args.calls_only:
        line["mode"] = "calls-only (entry points timed alone; no whole-step figure)"
    for r in results[1:]:
        line[r["workload"]] = {
            "workload": summary(r),
            "steps_per_s": rate(r["step_us"]),
            "eager_steps_per_s": rate(r["eager_us"]),
            "one_stream_graph_steps_per_s": rate(r["serial_us"]),
            "four_calls_concurrent_graph_steps_per_s": rate(r.get("conc_us")),
            "graph_matches_eager": r["graph_ok"],
            "calls": r["calls"],
            "attention_roofline": roofline_line(r, "attention"),
            "roofline": roofline_line(r, dominant(r)),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
