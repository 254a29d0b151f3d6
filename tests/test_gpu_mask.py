"""GPU parity of jt_build_tree_mask against the oracle: bit-exact rows, depths, flags."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from gpu_util import anc_to_dense, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _check(parent):
    need_gpu()
    parent = np.ascontiguousarray(parent, np.int32)
    S, B = parent.shape
    print(f"[mask] S={S} B={B}", flush=True)
    anc, depth, err = jt.build_tree_mask(dev(parent))
    torch.cuda.synchronize()
    vis, d_ref, e_ref = oracle.build_mask(parent)
    e = host(err)
    assert np.array_equal(e, e_ref)
    ok = e_ref == 0
    assert np.array_equal(anc_to_dense(host(anc), B)[ok], vis[ok])
    assert np.array_equal(host(depth), d_ref)
    # bits at and beyond B stay clear
    a = host(anc).view(np.uint64)
    for u in range(B, 256):
        assert not ((a[:, :, u >> 6] >> np.uint64(u & 63)) & np.uint64(1)).any()


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_config_trees(name):
    _check(wl.make(name, 101, parts=()).parent)


@pytest.mark.parametrize("B", [1, 2, 63, 64, 65, 127, 128, 129, 255, 256])
def test_random_trees_every_size(B):
    rng = np.random.default_rng(B)
    trees = [wl.random_tree(B, 255, 256, rng)[0] for _ in range(6)]
    trees.append(wl.chain_tree(B)[0])
    trees.append(wl.star_tree(B)[0])
    _check(np.stack(trees))


def test_all_small_trees():
    arrs = [[-1] + list(p) for p in itertools.product(*[range(i) for i in range(1, 6)])]
    _check(np.array(arrs, np.int32))


def test_bad_parents_flagged():
    good = wl.random_tree(10, 5, 3, np.random.default_rng(0))[0]
    bad = [good.copy() for _ in range(4)]
    bad[0][0] = 0
    bad[1][5] = 5
    bad[2][7] = 9
    bad[3][3] = -2
    _check(np.stack([good] + bad))


def test_many_sequences():
    rng = np.random.default_rng(7)
    _check(np.stack([wl.random_tree(64, 8, 8, rng)[0] for _ in range(300)]))
