"""Properties of a best-first draft tree that hold at any size (shared by the oracle pins
and the GPU tests): parents come first; the children of a node are contiguous, in rank
order, carry their depth's candidates and add that depth's increment to the parent's
score; expansions leave the queue in (score descending, index ascending) order; and when
the budget is spent, no unexpanded node above the depth limit would have popped earlier.

enumerate_accept() is an independent set-based statement of greedy acceptance, used to
check both the oracle and the GPU walk on every tiny tree.
"""
import numpy as np


def enumerate_accept(parent, ok, am):
    """Accepted nodes grow from the root in index order (a parent precedes its children):
    u joins when its parent has joined and its edge is ok.  The deepest accepted node,
    lowest index on ties, ends the path; returns (accept_len, path, bonus)."""
    B = len(parent)
    acc = {0}
    depth = [0] * B
    for u in range(1, B):
        depth[u] = depth[parent[u]] + 1
        if parent[u] in acc and ok[u]:
            acc.add(u)
    best = min(acc, key=lambda v: (-depth[v], v))
    path = []
    u = best
    while u != -1:
        path.append(u)
        u = parent[u] if u else -1
    return depth[best], path[::-1], am[best]


def check_invariants(ids, lp, N, W, B, o, ent=None, w_lp=1.0, w_ent=0.0):
    S = o["parent"].shape[0]
    for s in range(S):
        par, tok, sc, n = o["parent"][s], o["tokens"][s], o["score"][s], int(o["n_nodes"][s])
        depth = np.zeros(B, np.int64)
        for i in range(1, n):
            assert 0 <= par[i] < i
            depth[i] = depth[par[i]] + 1
            assert depth[i] <= N
        # children of one parent are contiguous, in rank order, with that depth's candidates
        expanded = []
        i = 1
        while i < n:
            p = par[i]
            j = i
            while j < n and par[j] == p:
                j += 1
            assert p not in expanded, "a node expanded twice"
            expanded.append(p)
            row = s * N + depth[p]
            e = np.float32(0.0) if ent is None else np.float32(ent[row])
            for r in range(j - i):
                assert tok[i + r] == ids[row, r]
                inc = np.float32(np.float32(w_lp) * lp[row, r]) - np.float32(np.float32(w_ent) * e)
                assert sc[i + r] == np.float32(sc[p] + np.float32(inc))
            assert j - i == W or j == n      # only the last expansion may be cut short
            i = j
        # expansions leave the queue in (score desc, index asc) order
        keys = [(-float(sc[p]), p) for p in expanded]
        assert keys == sorted(keys)
        # nothing left unexpanded above depth N pops before the last expansion
        if n == B and expanded:
            last = keys[-1]
            for v in range(n):
                if v not in expanded and depth[v] < N:
                    assert (-float(sc[v]), v) > last
        if n < B:
            assert all(depth[v] == N or v in expanded for v in range(n))
            assert (par[n:] == 0).all() and (tok[n:] == -1).all() and np.isneginf(sc[n:]).all()
