"""GPU parity of jt_verify_sampled.  Draws, accepted lengths, paths, bonuses and flags must
equal the oracle's, except at close calls: a draw whose uniform lies within 1e-5 of its
interval's end (as a fraction of the row's weight) may go to a neighbour when fp32 sums
replace fp64 ones.  In a flat row of 151,936 logits most tokens hold less than 1e-5 of the
weight, so close calls are common there.  At a close call the device's token must still
hold the uniform in its interval widened by 1e-5 of the row's weight (checked in fp64
from the row), and the walk must agree with the device's own draws."""
import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from gpu_util import dev, host, need_gpu

pytestmark = pytest.mark.gpu
CLOSE = 1e-5


def _device(tl, parent, tokens, N, T, u, V=None):
    need_gpu()
    S, B = parent.shape
    print(f"[sampled] S={S} B={B} N={N} T={T} V={V or tl.shape[-1]} {tl.dtype}", flush=True)
    par, tok = dev(parent.astype(np.int32)), dev(tokens.astype(np.int32))
    anc, depth, _ = jt.build_tree_mask(par)
    x = dev(np.ascontiguousarray(tl.reshape(S * B, -1)))
    out = jt.verify_sampled(x, par, tok, anc, depth, N, T, dev(u.astype(np.float32)), V=V)
    torch.cuda.synchronize()
    return dict(zip(("accept_len", "accept_path", "bonus", "sample", "err"), map(host, out)))


def _walk(parent, tokens, x, N):
    """Accepted path and bonus of one sequence from its draws (validity check only)."""
    B = len(parent)
    depth = np.zeros(B, int)
    for v in range(1, B):
        depth[v] = depth[parent[v]] + 1
    ok = [True] + [tokens[v] == x[parent[v]] for v in range(1, B)]
    acc = np.zeros(B, bool)
    acc[0] = True
    for v in range(1, B):
        acc[v] = ok[v] and acc[parent[v]]
    best = max((v for v in range(B) if acc[v]), key=lambda v: (depth[v], -v))
    return depth[best], x[best]


def _holds(row, T, r, tok):
    """Does token tok's cumulative interval, widened by CLOSE of the weight, hold r * Z?"""
    x = row.astype(np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    m = x.max()
    if m == -np.inf:
        return tok == 0
    w = np.exp((x - m) / T)
    c = np.cumsum(w)
    Z = c[-1]
    return bool(w[tok] > 0 and c[tok] - w[tok] - CLOSE * Z <= r * Z <= c[tok] + CLOSE * Z)


def _compare(tl, parent, tokens, N, T, u, what, V=None):
    g = _device(tl, parent, tokens, N, T, u, V)
    o = oracle.verify_sampled(tl, parent, tokens, N, T, u, V=V)
    close = o["margin"] < CLOSE
    S, B = parent.shape
    assert np.array_equal(g["sample"][~close], o["sample"][~close]), what
    n_close = int(close.sum())
    rows = (wl.bf16_bits_to_f32(tl) if tl.dtype == np.uint16 else tl).reshape(S * B, -1)
    Vn = rows.shape[1] if V is None else V
    n_diff = int((close & (g["sample"] != o["sample"])).sum())
    print(f"[sampled] {what}: {close.size} draws, {n_close} close calls, {n_diff} differ",
          flush=True)
    for s, v in zip(*np.nonzero(close & (g["sample"] != o["sample"]))):
        assert _holds(rows[s * B + v, :Vn], T, float(u[s, v]), int(g["sample"][s, v])), (what, s, v)
    for s in range(S):
        if not close[s].any():
            for k in ("accept_len", "accept_path", "bonus", "err"):
                assert np.array_equal(g[k][s], o[k][s]), (what, s, k)
        else:
            L, bonus = _walk(parent[s], tokens[s], g["sample"][s], N)
            assert g["accept_len"][s] == L and g["bonus"][s] == bonus, (what, s)
    return g, o, n_close


def test_inverse_cdf_draws_by_hand():
    with np.errstate(divide="ignore"):
        x = np.log(np.array([[0.1, 0.2, 0.3, 0.4], [0.0, 0.5, 0.0, 0.5]])).astype(np.float32)
    x = np.tile(x, (4, 1))
    u = np.array([0.05, 0.0, 0.15, 0.49, 0.5, 0.51, 0.95, 0.999], np.float32)
    par = np.full((8, 1), -1, np.int32)
    g = _device(x.reshape(8, 1, 4), par, np.zeros((8, 1), np.int32), 0, 1.0, u.reshape(8, 1))
    assert g["sample"][:, 0].tolist() == [0, 1, 1, 1, 2, 3, 3, 3]


def test_worked_example_outcome_probabilities():
    """The pages' example (0.8 for d1; 0.5 for d2 and 0.3 for b after d1) over a grid of
    uniforms: P(1, b) = 0.24 from the device's outcomes, and every outcome equal to the
    oracle's."""
    with np.errstate(divide="ignore"):
        rows = np.log(np.array([[0.1, 0.8, 0.05, 0.05], [0.2, 0.0, 0.5, 0.3],
                                [0.25, 0.25, 0.25, 0.25]])).astype(np.float32)
    n = 40
    r = (np.arange(n) + 0.5) / n
    g0, g1, g2 = np.meshgrid(r, r, r, indexing="ij")
    u = np.stack([g0.ravel(), g1.ravel(), g2.ravel()], 1).astype(np.float32)
    S = n ** 3
    tl = np.tile(rows, (S, 1, 1))
    par = np.tile(np.array([[-1, 0, 1]], np.int32), (S, 1))
    tok = np.tile(np.array([[9, 1, 2]], np.int32), (S, 1))
    g, o, n_close = _compare(tl, par, tok, 2, 1.0, u, "worked example")
    assert n_close == 0
    assert abs(np.mean((g["accept_len"] == 1) & (g["bonus"] == 3)) - 0.24) < 1e-12


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("name", ["low_budget", "high_budget"])
def test_config_rows(name, T):
    """Full-vocabulary target rows (151,936 bf16 logits) of a config's tree, unplanted so
    that the draws spread over many tokens."""
    w = wl.make(name, 950, parts=("tree", "target"), plant=False)
    c = w.cfg
    u = np.random.default_rng(951).random((c.S, c.B)).astype(np.float32)
    _compare(w.target_logits, w.parent, w.tokens, c.N, T, u, f"{name} T={T}")


@pytest.mark.parametrize("name", ["ragged", "moe_verify"])
def test_other_configs_small_vocab(name):
    w = wl.make(name, 952, parts=("tree", "target"), V=9000, plant=False)
    c = w.cfg
    u = np.random.default_rng(953).random((c.S, c.B)).astype(np.float32)
    _compare(w.target_logits, w.parent, w.tokens, c.N, 1.0, u, name)


def test_nan_inf_rows_and_odd_vocab():
    rng = np.random.default_rng(954)
    S, B, V = 3, 5, 20001
    tl = rng.normal(0, 2, (S, B, V)).astype(np.float32)
    tl[0, 2, 100] = np.nan             # NaN weighs 0; the sequence is flagged
    tl[1, 0, :] = -np.inf              # no distribution: token 0
    tl[2, 3, :19990] = -np.inf         # all weight in the ragged tail
    par = np.tile(np.array([-1, 0, 0, 1, 2], np.int32), (S, 1))
    tok = rng.integers(0, V, (S, B)).astype(np.int32)
    u = rng.random((S, B)).astype(np.float32)
    g, o, _ = _compare(tl, par, tok, 4, 1.0, u, "nan / -inf / tail")
    assert g["err"][0] & 8 and g["sample"][1, 0] == 0 and g["sample"][2, 3] >= 19990
    bf = wl.to_dtype(tl, "bf16")
    _compare(bf, par, tok, 4, 1.3, u, "bf16")


def test_special_pieces_in_aligned_rows():
    """Rows whose length is a multiple of 8, so that whole 2048-logit pieces take the
    unmasked pass: a NaN there, a piece of -inf only, a row whose weight sits in one
    piece, a NaN in the ragged last piece, and plain rows beside them."""
    rng = np.random.default_rng(957)
    S, B, V = 2, 5, 8 * 2048 + 1000
    tl = rng.normal(0, 3, (S, B, V)).astype(np.float32)
    tl[0, 0, 3 * 2048 + 5] = np.nan
    tl[0, 1, 2048:4096] = -np.inf
    tl[0, 2, :] = -np.inf
    tl[0, 2, 4 * 2048 + 17:4 * 2048 + 900] = rng.normal(0, 1, 883)
    tl[0, 3, V - 3] = np.nan
    tl[0, 4, :2048] = -np.inf
    tl[0, 4, 5000] = 40.0
    par = np.tile(np.array([-1, 0, 0, 1, 2], np.int32), (S, 1))
    tok = rng.integers(0, V, (S, B)).astype(np.int32)
    u = rng.random((S, B)).astype(np.float32)
    for T in (1.0, 0.6):
        g, o, _ = _compare(tl, par, tok, 4, T, u, f"aligned special pieces T={T}")
        assert g["err"][0] & 8 and not g["err"][1] & 8
        assert 4 * 2048 + 17 <= g["sample"][0, 2] < 4 * 2048 + 900
        _compare(wl.to_dtype(tl, "bf16"), par, tok, 4, T, u, f"bf16 special pieces T={T}")


def test_rows_longer_than_one_chunk_of_pieces():
    """600,000-logit rows: 293 pieces, more than the 256 one pass of the piece search
    holds, with uniforms that land in the second pass."""
    rng = np.random.default_rng(958)
    S, B, V = 1, 4, 600_000
    tl = rng.normal(0, 1, (S, B, V)).astype(np.float32)
    par = np.array([[-1, 0, 0, 1]], np.int32)
    tok = rng.integers(0, V, (S, B)).astype(np.int32)
    u = np.array([[0.1, 0.9, 0.97, 0.9999]], np.float32)
    g, o, _ = _compare(tl, par, tok, 3, 1.0, u, "600k fp32")
    assert (g["sample"][0, 1:] > 256 * 2048).all()
    _compare(wl.to_dtype(tl, "bf16"), par, tok, 3, 1.0, u, "600k bf16")


def test_low_temperature_equals_device_greedy():
    w = wl.make("low_budget", 955, parts=("tree", "target"))
    c = w.cfg
    u = np.random.default_rng(956).random((c.S, c.B)).astype(np.float32)
    g = _device(w.target_logits, w.parent, w.tokens, c.N, 1e-4, u)
    par, tok = dev(w.parent), dev(w.tokens)
    anc, depth, _ = jt.build_tree_mask(par)
    r = jt.verify_greedy(dev(w.target_logits.reshape(c.S * c.B, -1)), par, tok, anc, depth, c.N)
    torch.cuda.synchronize()
    assert np.array_equal(g["sample"], host(r["argmax"]))
    for k in ("accept_len", "accept_path", "bonus"):
        assert np.array_equal(g[k], host(r[k])), k
