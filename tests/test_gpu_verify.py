"""GPU parity of jt_verify_greedy: bit-exact argmax, accepted length, path, bonus, flags."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from gpu_util import dev, host, need_gpu
from tree_util import enumerate_accept

pytestmark = pytest.mark.gpu


def _check(target, parent, tokens, N, V=None, what=""):
    need_gpu()
    parent = np.ascontiguousarray(parent, np.int32)
    tokens = np.ascontiguousarray(tokens, np.int32)
    S, B = parent.shape
    print(f"[verify] {what} S={S} B={B} N={N} V={V or target.shape[-1]}", flush=True)
    dp = dev(parent)
    anc, depth, _ = jt.build_tree_mask(dp)
    r = jt.verify_greedy(dev(target.reshape(S * B, -1)), dp, dev(tokens), anc, depth, N, V=V)
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(target.reshape(S * B, -1), parent, tokens, N, V=V)
    err = host(r["err"])
    assert np.array_equal(err, ref["err"]), what
    clean = (ref["err"] & (oracle.NAN)) == 0
    assert np.array_equal(host(r["argmax"])[clean], ref["argmax"][clean]), what
    for k in ("accept_len", "bonus"):
        assert np.array_equal(host(r[k])[clean], ref[k][clean]), (what, k)
    assert np.array_equal(host(r["accept_path"])[clean], ref["accept_path"][clean]), what
    return r, ref


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_config_planted(name):
    w = wl.make(name, 301, parts=("target",))
    _, ref = _check(w.target_logits, w.parent, w.tokens, w.cfg.N, what=name)
    assert (ref["err"] == 0).all()


@pytest.mark.parametrize("name", ["tiny", "low_budget", "ragged"])
def test_config_unplanted_ties(name):
    w = wl.make(name, 302, parts=("target",), plant=False)
    _check(w.target_logits, w.parent, w.tokens, w.cfg.N, what=name + " unplanted")


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6, 7])
def test_exhaustive_tiny_trees(B):
    """Every parent array with B <= 7 nodes x every accept pattern (2^(B-1)), one batched
    call per B (B = 7: 720 x 64 = 46,080 sequences).  GPU, oracle and the set-based
    enumerator must agree bit for bit.  The target argmax at node v is token 2v; the edge
    into u carries 2*parent[u] when its pattern bit is set (accepted), 2*parent[u] + 1
    otherwise, so sibling tokens may repeat (several accepted paths, lowest leaf wins)."""
    V = 2 * B + 2
    pats = np.array(list(itertools.product([0, 1], repeat=B - 1)), np.int32).reshape(2 ** (B - 1), B - 1)
    tails = list(itertools.product(*[range(i) for i in range(1, B)]))
    P = len(pats)
    par = np.empty((len(tails) * P, B), np.int32)
    tok = np.zeros((len(tails) * P, B), np.int32)
    for k, tail in enumerate(tails):
        parent = np.array([-1] + list(tail), np.int32)
        rows = slice(k * P, (k + 1) * P)
        par[rows] = parent
        if B > 1:
            tok[rows, 1:] = 2 * parent[1:] + (1 - pats)
    S = len(par)
    am = 2 * np.arange(B)
    x = np.zeros((S * B, V), np.float32)
    x[np.arange(S * B), np.tile(am, S)] = 1.0
    r, ref = _check(x, par, tok, B, what=f"exhaustive B={B}")
    got_len, got_path, got_bonus = host(r["accept_len"]), host(r["accept_path"]), host(r["bonus"])
    for s in range(S):
        ok = (1,) + tuple(int(b) for b in tok[s, 1:] == am[par[s, 1:]]) if B > 1 else (1,)
        L, path, bonus = enumerate_accept(par[s].tolist(), ok, am)
        assert got_len[s] == L and got_bonus[s] == bonus, (B, s)
        assert got_path[s, :L + 1].tolist() == path and (got_path[s, L + 1:] == -1).all(), (B, s)


def test_ties_nan_and_flags():
    V = 3000
    rng = np.random.default_rng(1)
    x = wl.to_dtype(rng.normal(0, 3, (4 * 6, V)).astype(np.float32), "bf16")
    x[0, [17, 900, 2999]] = wl.scalar_in_dtype(50.0, "bf16")   # tied maximum: id 17
    x[7, 5] = np.uint16(0x7FC0)                                   # NaN -> flagged
    par = np.array([[-1, 0, 1, 2, 3, 4]] * 4, np.int32)
    par[2, 4] = 5                                                 # bad parent
    tok = rng.integers(0, V, (4, 6)).astype(np.int32)
    _check(x, par, tok, 5, what="flags")
    _check(x, par, tok, 3, what="depth > N")


def test_all_neg_inf_rows_pick_first_id():
    x = np.full((3, 700), -np.inf, np.float32)
    par = np.array([[-1, 0, 1]], np.int32)
    _check(x, par, np.zeros((1, 3), np.int32), 2, what="-inf rows")


def test_f32_row_stride():
    rng = np.random.default_rng(3)
    w = wl.make("tiny", 5, parts=("target",))
    x = np.concatenate([w.target_logits, rng.normal(size=(16, 13)).astype(np.float32)], 1)
    _check(x, w.parent, w.tokens, w.cfg.N, V=w.cfg.V, what="stride")
