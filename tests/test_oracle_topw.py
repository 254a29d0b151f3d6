"""Pins for the oracle's per-depth top-W (CPU only).

The proposer takes the top-k tokens and their log-probabilities at every
future position (paperlayer.ai JetSpec summary, appendix E 'Drafting'); the
method keeps the top W candidates per depth (paper.rainbus.top summary, method
steps).  Readings: order is value descending then token id ascending, -0 == +0,
NaN ranks below -inf; log-prob = logit - logsumexp(row).
"""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
from tree_causal_draft_amd import workload as wl


def _brute(row, W):
    """Independent brute force: Python's sort on (-value, id)."""
    order = sorted(range(len(row)), key=lambda t: (-float(row[t]), t))
    return order[:W]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("W", [1, 2, 5, 16])
def test_matches_brute_force_and_scipy(dtype, W):
    rng = np.random.default_rng(W)
    x = rng.normal(0, 3, (12, 300)).astype(np.float32)
    a = wl.to_dtype(x, dtype)
    xs = wl.as_float32(a).astype(np.float64)
    ids, lp, lse = oracle.topw(a, W)
    for r in range(12):
        assert ids[r].tolist() == _brute(xs[r], W)
        np.testing.assert_allclose(lse[r], logsumexp(xs[r]), rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(lp[r], xs[r, ids[r]] - logsumexp(xs[r]), rtol=1e-13, atol=1e-13)
        assert abs(np.exp(xs[r] - lse[r]).sum() - 1.0) < 1e-12


def test_bf16_ties_lowest_id_first():
    # bf16 N(0,3) rows of a realistic width: many ties inside the top-8
    rng = np.random.default_rng(0)
    a = wl.to_dtype(rng.normal(0, 3, (6, 20000)).astype(np.float32), "bf16")
    ids, _, _ = oracle.topw(a, 8)
    xs = wl.as_float32(a)
    tied = 0
    for r in range(6):
        assert ids[r].tolist() == _brute(xs[r], 8)
        vals = xs[r, ids[r]]
        tied += int((np.diff(vals) == 0).any())
    assert tied > 0   # the case is really exercised


def test_constant_row():
    V, W = 1000, 7
    a = np.full((2, V), 0.5, np.float32)
    ids, lp, lse = oracle.topw(a, W)
    assert ids.tolist() == [list(range(W))] * 2
    np.testing.assert_allclose(lp, -np.log(V), rtol=1e-14)
    np.testing.assert_allclose(lse, 0.5 + np.log(V), rtol=1e-14)


def test_one_hot_row_and_signed_zero_and_nan():
    a = np.zeros((3, 10), np.float32)
    a[0, 6] = 50.0
    a[1] = -0.0
    a[1, 2] = 0.0          # +0 and -0 compare equal: plain id order
    a[2, 1] = np.nan       # NaN sorts after everything
    a[2, 0] = -np.inf
    ids, lp, lse = oracle.topw(a, 10)
    assert ids[0, 0] == 6 and abs(lp[0, 0]) < 1e-18
    assert ids[1].tolist() == list(range(10))
    assert ids[2].tolist() == [2, 3, 4, 5, 6, 7, 8, 9, 0, 1]
    assert np.isnan(lse[2])


def test_bf16_words_are_read_exactly():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x4049 = 3.140625, 0x0001 = smallest subnormal
    a = np.array([[0x3F80, 0xC000, 0x4049, 0x0001]], np.uint16)
    ids, lp, lse = oracle.topw(a, 4)
    assert ids[0].tolist() == [2, 0, 3, 1]
    vals = np.array([3.140625, 1.0, 2.0 ** -133, -2.0])
    np.testing.assert_allclose(lp[0], vals - logsumexp(vals), rtol=1e-15)


def test_row_stride_and_sub_vocab():
    rng = np.random.default_rng(3)
    big = rng.normal(size=(4, 50)).astype(np.float32)
    ids, lp, lse = oracle.topw(big, 3, V=40)
    for r in range(4):
        assert ids[r].tolist() == _brute(big[r, :40], 3)
        np.testing.assert_allclose(lse[r], logsumexp(big[r, :40].astype(np.float64)), rtol=1e-14)


# ---- row entropy: H = -sum p log p of the row's softmax (the per-depth entropy that
# entropy-guided and hybrid tree scoring rank by; paperlayer.ai JetSpec summary,
# appendices C and E)

def test_entropy_uniform_row_is_log_v():
    for V in (1, 7, 1000, 151936):
        x = np.full((1, V), 0.75, np.float32)
        *_, H = oracle.topw(x, 1, entropy=True)
        assert abs(H[0] - np.log(V)) <= 1e-12 * max(1.0, np.log(V))


def test_entropy_two_way_tie_and_point_mass():
    x = np.full((3, 50), -np.inf, np.float32)
    x[0, [3, 41]] = 2.0                 # two equal entries, the rest -inf: ln 2
    x[1, 17] = -5.0                     # a single finite entry: 0
    *_, H = oracle.topw(x, 1, entropy=True)
    assert abs(H[0] - np.log(2.0)) < 1e-15 and H[1] == 0.0
    assert H[2] == 0.0                  # every entry -inf: no distribution, read as a point
    y = np.zeros((1, 10), np.float32)
    y[0, 4] = np.nan
    *_, H = oracle.topw(y, 1, entropy=True)
    assert np.isnan(H[0])


def test_entropy_geometric_row_closed_form():
    """x_t = -beta t, t < V: p_t = (1-q) q^t / (1-q^V) with q = e^-beta, so
    H = -log((1-q)/(1-q^V)) + beta E[t],  E[t] = q/(1-q) - V q^V/(1-q^V)."""
    for beta, V in ((0.5, 64), (0.03125, 4096), (2.0, 11)):
        t = np.arange(V, dtype=np.float64)
        x = (-beta * t).astype(np.float32)
        assert np.array_equal(x.astype(np.float64), -beta * t)   # exact in float
        q = np.exp(-beta)
        Et = q / (1 - q) - V * q ** V / (1 - q ** V)
        want = -np.log((1 - q) / (1 - q ** V)) + beta * Et
        *_, H = oracle.topw(x[None, :], 1, entropy=True)
        assert abs(H[0] - want) <= 1e-10 * max(1.0, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_entropy_matches_scipy(dtype):
    from scipy.special import softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(41)
    x = wl.to_dtype(rng.normal(0, 3, (5, 3001)).astype(np.float32), dtype)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)
    *_, H = oracle.topw(x, 2, entropy=True)
    for r in range(5):
        assert abs(H[r] - entropy(softmax(xf[r]))) <= 1e-10
