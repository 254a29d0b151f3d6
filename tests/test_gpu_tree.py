"""GPU parity of jt_build_tree_best_first: parent, tokens, n_nodes and the score bits
must equal the oracle's on the same candidate lists (the scores are float sums in one
fixed order on both sides, so they agree exactly)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from gpu_util import dev, host, need_gpu
from tree_util import check_invariants

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gpu(ids, lp, N, B, entropy=None, w_lp=1.0, w_ent=0.0, root=None):
    need_gpu()
    S = ids.shape[0] // N
    print(f"[tree] S={S} N={N} W={ids.shape[1]} B={B} w=({w_lp},{w_ent}) "
          f"entropy={entropy is not None}", flush=True)
    par, tok, sc, n = jt.build_tree_best_first(
        dev(np.ascontiguousarray(ids, np.int32)), dev(np.ascontiguousarray(lp, np.float32)), N, B,
        entropy=None if entropy is None else dev(np.ascontiguousarray(entropy, np.float32)),
        w_lp=w_lp, w_ent=w_ent, root_token=None if root is None else dev(np.asarray(root, np.int32)))
    torch.cuda.synchronize()
    return dict(parent=host(par), tokens=host(tok), score=host(sc), n_nodes=host(n))


def _same(got, want, what):
    for k in ("parent", "tokens", "n_nodes"):
        assert np.array_equal(got[k], want[k]), (what, k)
    assert np.array_equal(got["score"].view(np.uint32), want["score"].view(np.uint32)), (what, "score")


def _both(ids, lp, N, B, what, **kw):
    g = _gpu(ids, lp, N, B, entropy=kw.get("entropy"), w_lp=kw.get("w_lp", 1.0),
             w_ent=kw.get("w_ent", 0.0), root=kw.get("root_token"))
    o = oracle.build_tree(ids, lp, N, B, **kw)
    _same(g, o, what)
    return g


def test_hand_worked_cases():
    with open(os.path.join(GOLD, "bestfirst_hand.json")) as fh:
        g = json.load(fh)
    ids = np.array(g["ids"], np.int32)
    lp = np.array(g["logprob"], np.float32)
    for c in g["cases"]:
        got = _gpu(ids, lp, g["N"], c["B"], entropy=c["entropy"], w_lp=c["w_lp"],
                   w_ent=c["w_ent"], root=[g["root_token"]])
        want = [float("-inf") if x == "-inf" else x for x in c["score"]]
        assert got["parent"][0].tolist() == c["parent"], c["why"]
        assert got["tokens"][0].tolist() == c["tokens"], c["why"]
        assert got["score"][0].tolist() == want, c["why"]
        assert int(got["n_nodes"][0]) == c["n_nodes"], c["why"]


def test_float32_score_order():
    """The hand-worked case whose float32 path scores tie where the exact sums do not: the
    device must pop in the float32 order, as the oracle does."""
    with open(os.path.join(GOLD, "bestfirst_fp32.json")) as fh:
        g = json.load(fh)
    ids = np.array(g["ids"], np.int32)
    lp = np.array([[int(x, 16) for x in row] for row in g["logprob_hex"]],
                  np.uint32).view(np.float32)
    got = _both(ids, lp, g["N"], g["B"], "float32 order", root_token=[g["root_token"]])
    assert got["parent"][0].tolist() == g["expected"]["parent"]
    assert got["tokens"][0].tolist() == g["expected"]["tokens"]


@pytest.mark.parametrize("seed", range(16))
def test_random_lists(seed):
    rng = np.random.default_rng(500 + seed)
    S = int(rng.integers(1, 9))
    N = int(rng.integers(1, 20))
    W = int(rng.integers(1, 17))
    B = int(rng.integers(1, 257))
    lp = -np.sort(rng.exponential(2.0, (S * N, W)), axis=1).astype(np.float32)
    ids = rng.integers(0, 151936, (S * N, W)).astype(np.int32)
    root = rng.integers(0, 151936, S).astype(np.int32)
    _both(ids, lp, N, B, f"random {seed}", root_token=root)


@pytest.mark.parametrize("seed", range(8))
def test_tie_heavy_lists_and_scores(seed):
    rng = np.random.default_rng(600 + seed)
    S, N, W, B = 4, int(rng.integers(2, 17)), int(rng.integers(1, 17)), int(rng.integers(64, 257))
    vals = np.array([-0.0, -0.25, -0.5, -1.0], np.float32)
    lp = -np.sort(-rng.choice(vals, (S * N, W)), axis=1).astype(np.float32)
    ids = rng.integers(0, 1000, (S * N, W)).astype(np.int32)
    _both(ids, lp, N, B, "ties")
    ent = rng.choice(np.array([0.0, 0.75, 2.5], np.float32), S * N)
    _both(ids, lp, N, B, "hybrid", entropy=ent, w_lp=1.0, w_ent=0.5)
    _both(ids, lp, N, B, "entropy only", entropy=ent, w_lp=0.0, w_ent=1.0)


def test_edges():
    rng = np.random.default_rng(7)
    # budget 1: the root alone; W = 1 chains that stop at depth N and pad the rest
    ids = rng.integers(0, 50, (3 * 5, 1)).astype(np.int32)
    lp = np.full((15, 1), -0.5, np.float32)
    _both(ids, lp, 5, 1, "B=1")
    g = _both(ids, lp, 5, 40, "chain + padding")
    assert (g["n_nodes"] == 6).all()
    # the full budget at the widest lists; N = 1 (a star)
    ids = rng.integers(0, 50, (2 * 16, 16)).astype(np.int32)
    lp = -np.sort(rng.exponential(1.0, (32, 16)), axis=1).astype(np.float32)
    _both(ids, lp, 16, 256, "W=16 B=256")
    _both(ids[:2], lp[:2], 1, 256, "star, padded")
    # -inf and NaN log-probs (a -inf logit; a NaN row) rank last, NaN below -inf
    lp2 = lp.copy()
    lp2[0, 3:] = -np.inf
    lp2[17, :] = np.nan
    _both(ids, lp2, 16, 200, "-inf / NaN")
    # many sequences
    S = 300
    ids = rng.integers(0, 151936, (S * 4, 3)).astype(np.int32)
    lp = -np.sort(rng.exponential(1.0, (S * 4, 3)), axis=1).astype(np.float32)
    _both(ids, lp, 4, 37, "S=300")


@pytest.mark.parametrize("name", ["low_budget", "high_budget", "ragged", "moe_verify"])
def test_config_candidate_lists(name):
    """Each config's draft logits through the oracle's top-W; both sides build the tree
    of that config's budget from the same float32 lists."""
    w = wl.make(name, 701, parts=("draft",))
    c = w.cfg
    ids, lp, _ = oracle.topw(w.draft_logits, c.W)
    lp = lp.astype(np.float32)
    _both(ids, lp, c.N, c.B, name)


@pytest.mark.parametrize("name", ["low_budget", "high_budget", "moe_verify"])
def test_composed_with_device_topw(name):
    """The device top-W feeding the device tree: the lists must equal the oracle's ids,
    and the tree must be a valid best-first tree of the device's own log-probs."""
    need_gpu()
    w = wl.make(name, 702, parts=("draft",))
    c = w.cfg
    ids, lp, _ = jt.topw_per_depth(dev(w.draft_logits), c.W)
    par, tok, sc, n = jt.build_tree_best_first(ids, lp, c.N, c.B)
    torch.cuda.synchronize()
    r_ids, _, _ = oracle.topw(w.draft_logits, c.W)
    assert np.array_equal(host(ids), r_ids)
    out = dict(parent=host(par), tokens=host(tok), score=host(sc), n_nodes=host(n))
    check_invariants(host(ids), host(lp), c.N, c.W, c.B, out)
    assert (out["n_nodes"] == c.B).all()


@pytest.mark.parametrize("name", ["low_budget", "high_budget"])
def test_hybrid_tree_from_device_entropy(name):
    """Entropy from the device top-W pass feeding hybrid and entropy-only scoring: the
    entropy matches the oracle's, and each tree is a valid best-first tree of its score."""
    need_gpu()
    w = wl.make(name, 703, parts=("draft",), plant=False)
    c = w.cfg
    x = dev(w.draft_logits)
    ent = torch.empty(c.S * c.N, dtype=torch.float32, device=x.device)
    ids, lp, _ = jt.topw_per_depth(x, c.W, row_entropy=ent)
    *_, r_ent = oracle.topw(w.draft_logits, c.W, entropy=True)
    torch.cuda.synchronize()
    from gpu_util import assert_lp_close
    assert_lp_close(host(ent), r_ent, name)
    for w_lp, w_ent in ((1.0, 0.5), (0.0, 1.0)):
        par, tok, sc, n = jt.build_tree_best_first(ids, lp, c.N, c.B, entropy=ent, w_lp=w_lp,
                                                   w_ent=w_ent)
        torch.cuda.synchronize()
        out = dict(parent=host(par), tokens=host(tok), score=host(sc), n_nodes=host(n))
        check_invariants(host(ids), host(lp), c.N, c.W, c.B, out, host(ent), w_lp, w_ent)
