"""GPU parity of jt_topw_per_depth: bit-exact ids, log-probs / LSE within 1e-5 + 1e-5|ref|."""
import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from gpu_util import assert_lp_close, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _check(logits, W, V=None, what=""):
    need_gpu()
    rows, stride = logits.shape
    V = stride if V is None else V
    print(f"[topw] {what} rows={rows} V={V} stride={stride} W={W} {logits.dtype}", flush=True)
    x = dev(logits)
    ids, lp, lse = jt.topw_per_depth(x, W, V=V)
    ent = torch.empty(rows, dtype=torch.float32, device=x.device)
    ids2, lp2, lse2 = jt.topw_per_depth(x, W, V=V, row_entropy=ent)
    torch.cuda.synchronize()
    r_ids, r_lp, r_lse, r_ent = oracle.topw(logits, W, V=V, entropy=True)
    assert np.array_equal(host(ids), r_ids), what
    assert_lp_close(host(lp), r_lp, what)
    assert_lp_close(host(lse), r_lse, what)
    # asking for the entropy changes nothing else, bit for bit
    for a, b in ((ids, ids2), (lp, lp2), (lse, lse2)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), what
    assert_lp_close(host(ent), r_ent, what + " entropy")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 7, 1000, 8192, 8193, 20000, 40961])
@pytest.mark.parametrize("W", [1, 2, 8, 16])
def test_random_rows(dtype, V, W):
    if W > V:
        return
    rng = np.random.default_rng(V * 31 + W)
    x = rng.normal(0, 3, (9, V)).astype(np.float32)
    _check(wl.to_dtype(x, dtype), W, what=f"{dtype}")


def test_bf16_ties_and_constant_rows():
    rng = np.random.default_rng(5)
    x = wl.to_dtype(rng.normal(0, 3, (6, 30000)).astype(np.float32), "bf16")
    x[1] = wl.scalar_in_dtype(1.5, "bf16")                     # constant row: ids 0..W-1
    x[2, ::7] = wl.scalar_in_dtype(40.0, "bf16")               # thousands of tied maxima
    x[3, 100:200] = wl.scalar_in_dtype(-0.0, "bf16")           # signed zeros
    x[3, 150:250] = wl.scalar_in_dtype(0.0, "bf16")
    for W in (1, 5, 16):
        _check(x, W, what="ties")


def test_row_stride_and_unaligned():
    rng = np.random.default_rng(9)
    x = wl.to_dtype(rng.normal(0, 3, (5, 10007)).astype(np.float32), "bf16")
    _check(x, 4, V=9001, what="odd stride, sub-vocab")
    y = rng.normal(0, 2, (3, 4099)).astype(np.float32)
    _check(y, 3, V=4097, what="f32 odd stride")


def test_neg_inf_rows():
    x = np.full((2, 5000), -np.inf, np.float32)
    x[1, 4000] = 1.0
    need_gpu()
    ent = torch.empty(2, dtype=torch.float32, device="cuda:0")
    ids, lp, lse = jt.topw_per_depth(dev(x), 3, row_entropy=ent)
    torch.cuda.synchronize()
    r_ids, _, r_lse, r_ent = oracle.topw(x, 3, entropy=True)
    assert np.array_equal(host(ids), r_ids)
    assert np.array_equal(np.isneginf(host(lse)), np.isneginf(r_lse))
    assert np.array_equal(host(ent), r_ent)  # 0 for the row of -inf, 0 for the point mass


@pytest.mark.parametrize("name", ["tiny", "low_budget", "high_budget", "ragged", "moe_verify"])
def test_config_draft_logits(name):
    w = wl.make(name, 202, parts=("draft",))
    _check(w.draft_logits, w.cfg.W, what=name)


def test_config_unplanted_ties():
    w = wl.make("moe_verify", 203, parts=("draft",), plant=False, S=4)
    _check(w.draft_logits, 8, what="unplanted")


@pytest.mark.parametrize("W", [4, 5, 9, 16])
def test_long_rows_rank_paths(W):
    """Rows of 151936 logits (75 partial lists, two list heads per lane in the merge).  A
    constant row and a heavily tied row put more than 64 keys at or above the merge's
    bound for W >= 9; a row whose largest logits all sit in one list puts the bound on
    that list's head."""
    rng = np.random.default_rng(77 + W)
    x = wl.to_dtype(rng.normal(0, 3, (4, 151936)).astype(np.float32), "bf16")
    x[1] = wl.scalar_in_dtype(1.5, "bf16")
    x[2, ::13] = wl.scalar_in_dtype(40.0, "bf16")
    x[3, 7 * 2048 + 3: 7 * 2048 + 43] = wl.scalar_in_dtype(50.0, "bf16")
    _check(x, W, what=f"long rows W={W}")


def test_entropy_nan_and_uniform_rows():
    x = np.zeros((3, 151936), np.float32)
    x[1, 77] = np.nan                    # a NaN: NaN entropy
    x[2, :5] = 30.0                      # five equal maxima far above the rest: ~ln 5
    _check(wl.to_dtype(x, "bf16"), 4, what="nan / uniform / 5-way")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [700, 151936])
def test_wth_entry_neg_inf(dtype, V):
    """Rows with fewer than W finite logits: the list ends in -inf entries (lowest ids
    first among them) whose log-probs must be exactly -inf; only -inf matches an infinite
    reference in the comparison."""
    W = 8
    rng = np.random.default_rng(V + W)
    x = np.full((4, V), -np.inf, np.float32)
    x[0, [3, V - 1]] = [1.0, 2.0]                                   # two finite
    x[1, rng.choice(V, W - 1, replace=False)] = rng.normal(0, 3, W - 1)  # the W-th is -inf
    x[2, V // 2] = 0.0                                              # one finite
    x[3] = rng.normal(0, 3, V)                                      # all finite (control)
    x[3, :: 5] = -np.inf
    r_ids, r_lp, _ = oracle.topw(wl.to_dtype(x, dtype), W)
    assert np.isneginf(r_lp[:3]).sum() == (W - 2) + 1 + (W - 1)
    _check(wl.to_dtype(x, dtype), W, what=f"W-th -inf {dtype} V={V}")
