"""GPU check of jt_draft_verify_step_noalloc (the fused step with the library's static
device scratch) against jt_draft_verify_step (the same step with a caller's workspace).

Four calls in a row with shrinking inputs -- ragged at a reduced vocabulary (three
launches, balanced schedule), high_budget (two launches, 128-row attention tiles beside
the scans), a small low_budget (two
launches), then the fp32 tiny step -- so each call runs on scratch that holds the previous,
larger call's contents.
Every output must equal the workspace call's bit for bit.  The call goes through the C
ABI (ctypes) and allocates nothing: every output is passed in.
"""
import pytest
import torch

import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from tree_causal_draft_amd.step import DeviceStep
from gpu_util import need_gpu

pytestmark = pytest.mark.gpu

OUTS = ("ids", "logprob", "row_lse", "anc", "depth", "out", "lse", "accept_len",
        "accept_path", "bonus", "argmax", "err")


def _bits(t):
    return t.view(torch.uint8)


def _run(st, fn, **extra):
    w = st.w
    return fn(st.draft, st.target, st.parent, st.tokens, st.cfg.N, st.cfg.W, st.q, st.k_tree,
              st.v_tree, st.k_prefix, st.v_prefix, st.prefix_len, block_table=st.block_table,
              block_size=st.cfg.block_size, num_blocks=w.num_blocks or None,
              max_prefix=w.max_prefix, **extra)


@pytest.mark.parametrize("cases", [(("ragged", dict(V=8192)), ("high_budget", {}),
                                    ("low_budget", dict(V=20000, prefix=200)), ("tiny", {}))])
def test_noalloc_equals_workspace_call(cases):
    need_gpu()
    for name, kw in cases:
        w = wl.make(name, 931, **kw)
        c = w.cfg
        st = DeviceStep(w, "cuda:0")
        dt = jt.JT_F32 if c.dtype == "f32" else jt.JT_BF16
        need = jt.step_workspace_size(c.S, c.B, c.N, c.W, c.V, c.Hq, c.Hkv, c.d, w.max_prefix,
                                      dt, c.block_size if w.block_table is not None else 0)
        assert 0 < need <= jt.STATIC_SCRATCH_BYTES, (name, need)
        print(f"[noalloc] {name} {kw}: scratch {need / 2**20:.1f} MiB", flush=True)
        ref = _run(st, jt.draft_verify_step, workspace=st.step_ws)
        torch.cuda.synchronize()
        ref = {k: ref[k].clone() for k in OUTS}
        # outputs preset to garbage, then the static-scratch call writes them
        outs = {k: torch.empty_like(ref[k]) for k in OUTS}
        for t in outs.values():
            _bits(t).fill_(0x5A)
        torch.cuda.synchronize()
        got = _run(st, jt.draft_verify_step_noalloc,
                   **{("out" if k == "out" else ("argmax_out" if k == "argmax" else k)): outs[k]
                      for k in OUTS})
        torch.cuda.synchronize()
        for k in OUTS:
            assert got[k] is outs[k]
            assert torch.equal(_bits(outs[k]), _bits(ref[k])), (name, k)
