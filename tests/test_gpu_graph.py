"""Graph replays of the fused step and of the stochastic verifier.

The step is timed as a replayed hipGraph, so a replay must give the eager call's outputs
bit for bit.  Each case captures one call, then replays it several times with the
program's own eager work (the four separate calls, or the stochastic verifier) and
synchronisations in between.  Before each replay it overwrites every output, and it
checks every replay.  The shapes cover the launch schedules of the step: two launches
(4-wave attention over one 64-row tile, or over 128-row tiles of one sequence with many
rows), three (8-wave attention over several sequences, the balanced schedule), and the
fp32 step's two.
"""
import pytest
import torch

from tree_causal_draft_amd import workload as wl
from tree_causal_draft_amd.step import DeviceStep
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

STEP_OUTS = ("ids", "logprob", "row_lse", "anc", "depth", "accept_len", "accept_path",
             "bonus", "argmax", "attn_out", "lse", "err_step")
SMP_OUTS = ("smp_accept_len", "smp_accept_path", "smp_bonus", "smp_sample", "err_smp")
REPLAYS = 4


def _bits(t):
    n = t.element_size()
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}[n])


def _capture(fn):
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        fn()  # warm-up on the capture stream
    cur.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(st, fn, outs, between, what):
    fn()
    torch.cuda.synchronize()
    ref = [_bits(getattr(st, n)).clone() for n in outs]
    g = _capture(fn)
    for rep in range(REPLAYS):
        between()
        torch.cuda.synchronize()
        for n in outs:
            _bits(getattr(st, n)).fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for n, r in zip(outs, ref):
            assert torch.equal(_bits(getattr(st, n)), r), (what, rep, n)
    print(f"[graph] {what}: {REPLAYS} replays equal the eager call", flush=True)
    del g


@pytest.mark.parametrize("name,kw", [
    ("low_budget", {}),                    # two launches
    ("high_budget", dict(V=8192)),         # two: 128-row tiles beside the scans
    ("moe_verify", dict(V=8192)),          # three: balanced schedule over 32 sequences
    ("tiny", {}),                          # fp32: two launches, attention in the second
])
def test_fused_step_replays(name, kw):
    need_gpu()
    w = wl.make(name, 960, **kw)
    st = DeviceStep(w, "cuda:0")
    print(f"[graph] fused step {name} {kw}", flush=True)
    _replays_match(st, st.run_fused, STEP_OUTS, st.run, f"fused step {name}")


def test_sampled_replays():
    need_gpu()
    w = wl.make("high_budget", 961)
    st = DeviceStep(w, "cuda:0")
    st.mask()
    torch.cuda.synchronize()
    print("[graph] stochastic verifier high_budget", flush=True)
    _replays_match(st, st.sampled, SMP_OUTS, st.verify, "stochastic verifier high_budget")
