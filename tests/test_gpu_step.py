"""GPU parity of jt_draft_verify_step (the four steps in two or three launches).

The fused call must reproduce, bit for bit, every integer and attention output of the
four separate calls on the same inputs (those are held to the oracle by the other GPU
tests), and its err must be the OR of their flags.  Log-probs and row LSE agree to the
log-prob tolerance: the step may cut a row into pieces differently, so its sums add in
another order.  So may the attention of one bf16 sequence with more than 128 rows per KV
head: the step runs it beside the logit scans on fewer workgroups, with longer key
chunks, so there its outputs agree to the bf16 attention bounds.  The benchmark's own inputs (every configuration at full size) are also compared with the
oracle directly.  Attention outputs of
a sequence with a bad parent array are unspecified and are not compared.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_causal_draft_amd import workload as wl
from tree_causal_draft_amd.step import DeviceStep
from gpu_util import (BF16_ATOL, BF16_RTOL, LP_ATOL, LP_RTOL, assert_attention_close,
                      assert_lp_close, assert_lse_close, block_rows, host, need_gpu,
                      oracle_attention)

pytestmark = pytest.mark.gpu

OUTS = ("ids", "logprob", "row_lse", "anc", "depth", "accept_len", "accept_path", "bonus",
        "argmax", "attn_out", "lse")
ATTN = ("attn_out", "lse")
SUMS = ("logprob", "row_lse")  # float sums over a logit row


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32 if t.element_size() == 4 else torch.int64)


def _compare(w, what, tamper=None):
    need_gpu()
    c = w.cfg
    print(f"[step] {what}: S={c.S} B={c.B} N={c.N} W={c.W} V={c.V} heads {c.Hq}/{c.Hkv} "
          f"d={c.d} paged={w.block_table is not None}", flush=True)
    st = DeviceStep(w, "cuda:0")
    if tamper:
        tamper(st)
    st.run()
    torch.cuda.synchronize()
    sep = {k: getattr(st, k).clone() for k in OUTS}
    err_sep = (st.err_mask | st.err_attn | st.err_verify).clone()
    for k in OUTS:
        getattr(st, k).view(torch.uint8).fill_(0x7F)
    st.err_step.fill_(-1)
    st.run_fused()
    torch.cuda.synchronize()
    assert torch.equal(st.err_step, err_sep), (what, host(st.err_step), host(err_sep))
    bad_parent = (err_sep & 1) != 0
    own_split = c.dtype == "bf16" and c.S == 1 and (c.Hq // c.Hkv) * c.B > 128
    for k in OUTS:
        if k in SUMS:
            assert_lp_close(host(getattr(st, k)), host(sep[k]), f"{what} {k}")
            continue
        if k in ATTN and own_split:
            g, r = host(getattr(st, k)), host(sep[k])
            if bool(bad_parent.any()):  # those sequences' attention is unspecified
                keep = ~host(bad_parent).astype(bool)
                g, r = g[keep], r[keep]
            if k == "attn_out":
                assert_attention_close(g, r, c.dtype, f"{what} {k}")
            else:
                assert_lse_close(g, r, c.dtype, f"{what} {k}")
            continue
        a, b = _bits(getattr(st, k)), _bits(sep[k])
        if k in ATTN and bool(bad_parent.any()):
            keep = ~bad_parent
            a, b = a[keep], b[keep]
        assert torch.equal(a, b), (what, k)
    return st, err_sep


def _small(name, **kw):
    base = dict(V=8192)
    base.update(kw)
    return base


# the benchmark's inputs: bench.py seeds workload k (in CONFIG_ORDER) with 1000 * (k + 1)
BENCH_SEED = {n: 1000 * (k + 1) for k, n in enumerate(wl.CONFIG_ORDER)}


def _against_oracle(w, st, sel=None):
    """The fused step's outputs against the oracle on the same inputs: top-W ids and the
    verification outputs bit for bit, log-probs and row LSE within the log-prob tolerance,
    attention (every row, or the rows `sel`) and its LSE within the bf16 bounds."""
    c = w.cfg
    ids, lp, lse = oracle.topw(w.draft_logits, c.W)
    assert np.array_equal(host(st.ids), ids), "top-W ids"
    assert_lp_close(host(st.logprob), lp, "logprob")
    assert_lp_close(host(st.row_lse), lse, "row_lse")
    ref = oracle.verify_greedy(w.target_logits, w.parent, w.tokens, c.N)
    for k, t in (("accept_len", st.accept_len), ("accept_path", st.accept_path),
                 ("bonus", st.bonus), ("argmax", st.argmax)):
        assert np.array_equal(host(t), ref[k]), k
    sel, out, rlse, _ = oracle_attention(w, sel)
    got, glse = host(st.attn_out), host(st.lse)
    got = got[sel[:, 0], sel[:, 1], sel[:, 2]]
    glse = glse[sel[:, 0], sel[:, 1], sel[:, 2]]
    assert_attention_close(got, out, c.dtype, f"{c.name} attention ({len(sel)} rows)")
    e = assert_lse_close(glse, rlse, c.dtype, f"{c.name} lse")
    print(f"[step] {c.name}: oracle parity ok, {len(sel)} attention rows, "
          f"max |lse err| {e:.2e}", flush=True)


@pytest.mark.parametrize("name", ["tiny", "low_budget", "high_budget"])
def test_bench_inputs_against_oracle(name):
    """The benchmarked call on the benchmark's own inputs (its seed, full vocabulary): equal
    to the four calls bit for bit, and to the oracle on every output and attention row
    (tiny is fp32: two launches with the attention in the second)."""
    w = wl.make(name, BENCH_SEED[name])
    st, err = _compare(w, name + " bench inputs")
    assert int(err.abs().sum()) == 0
    _against_oracle(w, st)


@pytest.mark.parametrize("name", ["ragged", "moe_verify"])
def test_full_vocab_balanced_schedule(name):
    """ragged and moe_verify at full size (V = 151,936; moe_verify reads 622 MB of target
    logits) through the balanced-schedule path, on the benchmark's inputs: equal to
    the four calls bit for bit, and to the oracle on ids, acceptance and every row of one
    whole 256-row block of query rows per sequence."""
    w = wl.make(name, BENCH_SEED[name])
    st, err = _compare(w, name + " full V")
    assert int(err.abs().sum()) == 0
    _against_oracle(w, st, sel=block_rows(w))


def _small(name, **kw):
    base = dict(V=8192)
    base.update(kw)
    return base


@pytest.mark.parametrize("name", ["low_budget", "high_budget"])
def test_benchmarked_configs_full_size(name):
    w = wl.make(name, 811)
    _, err = _compare(w, name)
    assert int(err.abs().sum()) == 0


@pytest.mark.parametrize("name", ["moe_verify", "ragged"])
def test_other_configs_small_vocab(name):
    w = wl.make(name, 812, **_small(name))
    _compare(w, name + " V=8192")


@pytest.mark.parametrize("kw", [
    dict(S=3, B=1, N=1, W=2, prefix=70),                      # root only, tiny prefix
    dict(S=2, B=37, N=5, W=3, prefix=0),                      # no prefix at all
    dict(S=2, B=256, N=16, W=16, prefix=200, V=5000),         # widest W, ragged vocab tail
    dict(S=1, B=100, N=9, W=4, prefix=333, d=64),             # head dim 64, 128-row tiles
    dict(S=5, B=20, N=6, W=5, prefix=129, Hq=24, Hkv=3),      # G = 8
])
def test_shapes(kw):
    kw = dict(kw)
    V = kw.pop("V", 4096)
    w = wl.make("low_budget", 813, tree="random", V=V, **kw)
    _compare(w, f"shape {kw}")


def test_one_sequence_paged():
    """One paged sequence with more than 128 rows per KV head: the step's 4-wave attention
    runs beside the scans in its own key split, each chunk staging its block-table
    entries."""
    w = wl.make("ragged", 816, S=1, B=150, N=8, W=4, prefix=700, V=4096, tree="random")
    st, err = _compare(w, "one paged sequence")
    assert int(err.abs().sum()) == 0
    _against_oracle(w, st)


@pytest.mark.parametrize("seed", range(4))
def test_one_sequence_random_shapes(seed):
    """Seeded random single-sequence bf16 shapes with more than 128 rows per KV head through
    the fused step: against the four calls and the oracle."""
    rng = np.random.default_rng(4400 + seed)
    G = int(rng.choice([2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(128 // G + 1, 257))
    W = int(rng.integers(2, 7))
    n, cap, level = 0, 1, 1
    while cap < B:  # the least depth limit that holds B nodes of at most W children each
        level *= W
        cap += level
        n += 1
    kw = dict(S=1, B=B, N=n + int(rng.integers(0, 8)), W=W, Hq=G * Hkv, Hkv=Hkv, prefix=int(rng.integers(0, 1200)),
              d=int(rng.choice([64, 128])), V=8 * int(rng.integers(125, 750)))  # 16-byte rows
    w = wl.make("ragged", 4400 + seed, tree="random", **kw)
    st, err = _compare(w, f"one sequence {kw}")
    assert int(err.abs().sum()) == 0
    _against_oracle(w, st)


def test_flags_bad_parent_nan_bad_block():
    w = wl.make("ragged", 814, V=4096)

    def tamper(st):
        par = st.parent.clone()
        par[1, 5] = 7          # parent after the node: bad array
        st.parent.copy_(par)
        tgt = st.target.clone()
        tgt[3 * w.cfg.B + 2, 100] = float("nan")   # a NaN target logit in sequence 3
        st.target.copy_(tgt)
        bt = st.block_table.clone()
        bt[5, 0] = w.num_blocks + 3                # a block outside the pool in sequence 5
        st.block_table.copy_(bt)

    st, err = _compare(w, "flags", tamper)
    e = host(err)
    assert e[1] & 1 and e[3] & 8 and e[5] & 4, e


def test_fused_against_oracle():
    w = wl.make("low_budget", 815, V=4096, prefix=300, B=40, N=7, W=3, tree="random")
    st, _ = _compare(w, "oracle check")
    c = w.cfg
    ids, lp, lse = oracle.topw(w.draft_logits, c.W)
    assert np.array_equal(host(st.ids), ids)
    np.testing.assert_allclose(host(st.logprob), lp, rtol=LP_RTOL, atol=LP_ATOL)
    ref = oracle.verify_greedy(w.target_logits, w.parent, w.tokens, c.N)
    for k in ("accept_len", "accept_path", "bonus"):
        assert np.array_equal(host(getattr(st, k)), ref[k]), k
    out, _, _ = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                      w.prefix_len, w.parent, max_prefix=w.max_prefix)
    got = host(st.attn_out).astype(np.float64)
    assert (np.abs(got - out) <= BF16_ATOL + BF16_RTOL * np.abs(out)).all()


@pytest.mark.parametrize("kw", [
    dict(S=3, B=40, N=6, W=3, prefix=130, V=5000),            # several node blocks, G = 4
    dict(S=2, B=9, N=4, W=2, prefix=0, V=1024, d=128, Hq=8, Hkv=1),   # no prefix, G = 8
    dict(S=2, B=20, N=5, W=4, prefix=(40, 300), V=3000, Hq=6, Hkv=2,
         paged=True, block_size=16),                                      # paged, G = 3
])
def test_fp32_shapes(kw):
    """The fp32 step (two launches, attention in the second) against the four calls."""
    kw = dict(kw)
    w = wl.make("tiny", 816, tree="random", **kw)
    _compare(w, f"fp32 {kw}")


def test_rejects_misaligned_rows():
    need_gpu()
    import tree_causal_draft_amd as jt
    for name, shift in (("low_budget", 1), ("tiny", 1)):
        w = wl.make(name, 817, V=4096)
        st = DeviceStep(w, "cuda:0")
        rows, stride = st.draft.shape
        buf = torch.empty(rows * stride + shift, dtype=st.draft.dtype, device=st.draft.device)
        shifted = buf[shift:].view(rows, stride)  # contiguous, off a 16-byte boundary
        shifted.copy_(st.draft)
        with pytest.raises(jt.JTError, match="misaligned"):
            jt.draft_verify_step(shifted, st.target, st.parent, st.tokens, w.cfg.N, w.cfg.W,
                                 st.q, st.k_tree, st.v_tree, st.k_prefix, st.v_prefix,
                                 st.prefix_len, workspace=st.step_ws)


@pytest.mark.parametrize("name", ["low_budget", "high_budget"])
def test_fused_entropy_against_oracle(name):
    """row_entropy from the step's own top-W pass, against the oracle's softmax entropy."""
    need_gpu()
    import tree_causal_draft_amd as jt
    w = wl.make(name, 818, V=151936, plant=False)
    c = w.cfg
    st = DeviceStep(w, "cuda:0")
    ent = torch.empty(c.S * c.N, dtype=torch.float32, device="cuda:0")
    jt.draft_verify_step(st.draft, st.target, st.parent, st.tokens, c.N, c.W, st.q, st.k_tree,
                         st.v_tree, st.k_prefix, st.v_prefix, st.prefix_len,
                         max_prefix=w.max_prefix, workspace=st.step_ws, row_entropy=ent)
    torch.cuda.synchronize()
    *_, r_ent = oracle.topw(w.draft_logits, c.W, entropy=True)
    assert_lp_close(host(ent), r_ent, name)
