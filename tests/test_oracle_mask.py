"""Pins for the oracle's tree-causal mask and depths (CPU only).

The mask definition: M[v,u] = 0 iff u is an ancestor of v or v itself
(JetSpec review, startedourmission.github.io, 'How it works'); the verifier
works from parent indices and depths (paperlayer.ai JetSpec summary, app. E).
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from tree_causal_draft_amd import workload as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _anc_sets_recursive(parent):
    """Independent brute force: Anc*(v) = {v} union Anc*(parent(v)), by recursion."""
    memo = {}

    def rec(v):
        if v not in memo:
            memo[v] = {v} if parent[v] == -1 else ({v} | rec(int(parent[v])))
        return memo[v]
    return [rec(v) for v in range(len(parent))]


def test_hand_worked_tree7():
    g = json.load(open(os.path.join(GOLD, "tree7_hand.json")))
    vis, depth, err = oracle.build_mask(np.array([g["parent"]], np.int32))
    assert err[0] == 0
    assert depth[0].tolist() == g["depth"]
    for v, anc in enumerate(g["ancestors_incl_self"]):
        assert sorted(np.nonzero(vis[0, v])[0].tolist()) == anc


def _all_parent_arrays(B):
    return itertools.product(*[range(i) for i in range(1, B)])


@pytest.mark.parametrize("B", [1, 2, 3, 4, 5, 6])
def test_exhaustive_small_trees(B):
    """Every parent array with parent[i] < i, B <= 6: brute-force sets agree."""
    arrs = [[-1] + list(p) for p in _all_parent_arrays(B)]
    par = np.array(arrs, np.int32).reshape(len(arrs), B)
    vis, depth, err = oracle.build_mask(par)
    assert not err.any()
    for s in range(len(arrs)):
        sets = _anc_sets_recursive(par[s])
        for v in range(B):
            assert set(np.nonzero(vis[s, v])[0].tolist()) == sets[v]
            assert depth[s, v] == len(sets[v]) - 1


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_invariants_on_workload_trees(name):
    w = wl.make(name, 7, parts=())
    vis, depth, err = oracle.build_mask(w.parent)
    assert not err.any()
    S, B = w.parent.shape
    for s in range(S):
        V = vis[s].astype(bool)
        assert V.diagonal().all()                  # each node sees itself
        assert V[:, 0].all()                       # every node sees the root
        assert (V.sum(1) == depth[s] + 1).all()    # path length
        assert not np.triu(V, 1).any()             # ancestors have smaller indices
        iu, ju = np.nonzero(V)
        assert (depth[s][ju] <= depth[s][iu]).all()
        # transitivity: u visible from v  =>  Anc(u) subset of Anc(v)
        for v in range(B):
            for u in np.nonzero(V[v])[0]:
                assert not (V[u] & ~V[v]).any()
        # siblings never see each other
        ch = wl.children_lists(w.parent[s])
        for kids in ch:
            for a, b in itertools.combinations(kids, 2):
                assert not V[a, b] and not V[b, a]
        assert (depth[s] == w.depth[s]).all()


def test_chain_is_lower_triangular_and_star_is_diag_plus_root():
    B = 33
    vis, depth, _ = oracle.build_mask(wl.chain_tree(B)[0][None])
    assert (vis[0] == np.tril(np.ones((B, B), np.uint8))).all()
    assert depth[0].tolist() == list(range(B))
    vis, depth, _ = oracle.build_mask(wl.star_tree(B)[0][None])
    exp = np.eye(B, dtype=np.uint8)
    exp[:, 0] = 1
    assert (vis[0] == exp).all()
    assert depth[0].tolist() == [0] + [1] * (B - 1)


@pytest.mark.parametrize("bad", [[0, 0, 1], [-1, 1, 0], [-1, 0, 2], [-1, 0, 3], [-1, -1, 0],
                                 [-1, 0, -5]])
def test_bad_parent_arrays_flagged(bad):
    par = np.array([[-1, 0, 1], bad], np.int32)
    _, depth, err = oracle.build_mask(par)
    assert err[0] == 0 and err[1] == oracle.BAD_PARENT
    assert (depth[1] == -1).all()
