"""GPU parity of jt_tree_attention against the fp64 oracle.

bf16: |gpu - ref| <= 2e-2 + 1e-2 |ref| per element and relative L2 <= 1e-2; fp32:
1e-5 + 1e-5 |ref|.  Each bf16 case also runs with q, k ~ N(0, 1) ("sharp"), where the
softmax is peaked enough that a masking or rescaling mistake moves outputs far past the
tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from gpu_util import (assert_attention_close, assert_lse_close, block_rows, dev, host,
                      need_gpu, oracle_attention)

pytestmark = pytest.mark.gpu


def _run_gpu(w, scale=0.0):
    need_gpu()
    anc, depth, _ = jt.build_tree_mask(dev(w.parent))
    out, lse, err = jt.tree_attention(
        dev(w.q), dev(w.k_tree), dev(w.v_tree), dev(w.k_prefix), dev(w.v_prefix),
        dev(w.prefix_len), anc, block_table=None if w.block_table is None else dev(w.block_table),
        block_size=w.cfg.block_size, num_blocks=w.num_blocks or None, max_prefix=w.max_prefix,
        scale=scale)
    torch.cuda.synchronize()
    return host(out), host(lse), host(err)


def _check(w, what, sel=None, scale=0.0):
    cfg = w.cfg
    print(f"[attn] {what} S={cfg.S} B={cfg.B} P={w.prefix_len.tolist()[:4]} Hq={cfg.Hq} "
          f"Hkv={cfg.Hkv} d={cfg.d} {cfg.dtype} paged={cfg.paged}", flush=True)
    out, lse, err = _run_gpu(w, scale)
    kw = dict(block_table=w.block_table, block_size=cfg.block_size, num_blocks=w.num_blocks,
              max_prefix=w.max_prefix, scale=scale)
    if sel is None:
        ref, rlse, rerr = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                                w.prefix_len, w.parent, **kw)
        got, glse = out, lse
    else:
        ref, rlse, rerr = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                                w.prefix_len, w.parent, sel=sel, **kw)
        got = out[sel[:, 0], sel[:, 1], sel[:, 2]]
        glse = lse[sel[:, 0], sel[:, 1], sel[:, 2]]
    assert np.array_equal(err, rerr)
    assert_attention_close(got, ref, cfg.dtype, what)
    assert_lse_close(glse, rlse, cfg.dtype, what)
    return out


def _small(**kw):
    base = dict(S=2, prefix=300, B=40, N=10, W=4, Hq=8, Hkv=2, d=128, dtype="bf16", V=4096)
    base.update(kw)
    return base


def test_tiny_fp32():
    w = wl.make("tiny", 401, parts=("attn",))
    _check(w, "tiny fp32")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("sharp", [False, True])
def test_bf16_random_trees(d, G, sharp):
    w = wl.make("ragged", 410 + G, parts=("attn",), qk_std=1.0 if sharp else None,
                **_small(d=d, Hq=2 * G, Hkv=2, paged=False, prefix=(100, 300)))
    _check(w, f"bf16 d={d} G={G} sharp={sharp}")


@pytest.mark.parametrize("B,P", [(1, 0), (1, 77), (16, 0), (256, 0), (256, 130), (65, 64)])
def test_bf16_edge_shapes(B, P):
    w = wl.make("ragged", 420 + B, parts=("attn",), qk_std=1.0,
                **_small(S=1, B=B, N=255, W=256, prefix=P, paged=False))
    _check(w, f"edge B={B} P={P}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
def test_bf16_one_sequence_many_rows(d, paged):
    """One sequence with more than 128 rows per KV head: 4-wave workgroups over several
    128-row tiles (the last one 16 rows, paired where its chunks are short) and split-KV
    over a prefix that ends inside a tile; paged with the chunk's block-table entries staged
    in LDS."""
    w = wl.make("ragged", 425 + d + int(paged), parts=("attn",), qk_std=1.0,
                **_small(S=1, B=100, prefix=1000, d=d, paged=paged, N=9, W=4))
    _check(w, f"one sequence, many rows, d={d} paged={paged}")


def _min_depth(B, W):
    """The least depth limit at which a tree of at most W children per node holds B nodes."""
    n, cap, level = 0, 1, 1
    while cap < B:
        level *= W
        cap += level
        n += 1
    return n


def _one_sequence_shape(seed):
    """A seeded single-sequence shape with more than 128 rows per KV head."""
    rng = np.random.default_rng(seed)
    G = int(rng.choice([2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(128 // G + 1, 257))
    W = int(rng.integers(2, 7))
    N = _min_depth(B, W) + int(rng.integers(0, 8))
    return dict(S=1, B=B, N=N, W=W, Hq=G * Hkv, Hkv=Hkv, prefix=int(rng.integers(0, 1500)),
                d=int(rng.choice([64, 128])), paged=bool(rng.integers(0, 2)),
                block_size=int(rng.choice([4, 16])))


@pytest.mark.parametrize("seed", range(8))
def test_bf16_one_sequence_random_shapes(seed):
    """Seeded random single-sequence shapes through the 128-row-tile plan: head groups 2 to
    8, 1 to 4 KV heads, 65 to 256 nodes, prefixes from empty to 1,499 keys, both head dims,
    contiguous or paged (block size 4 or 16), sharp scores."""
    kw = _one_sequence_shape(4300 + seed)
    w = wl.make("ragged", 4300 + seed, parts=("attn",), qk_std=1.0, tree="random",
                **_small(**kw))
    _check(w, f"one sequence, random shape {kw}")


@pytest.mark.parametrize("tree", ["chain", "star"])
def test_bf16_chain_and_star(tree):
    B = 200
    t = wl.chain_tree(B) if tree == "chain" else wl.star_tree(B)
    w = wl.make("ragged", 430, parts=("attn",), qk_std=1.0, trees=[t, t],
                **_small(B=B, N=255, W=256, prefix=(50, 190), paged=False))
    _check(w, tree)


@pytest.mark.parametrize("bs", [16, 4])
def test_bf16_paged(bs):
    w = wl.make("ragged", 440 + bs, parts=("attn",), qk_std=1.0,
                **_small(S=3, prefix=(1, 500), paged=True, block_size=bs))
    _check(w, f"paged bs={bs}")


@pytest.mark.parametrize("S,B,G,prefix,paged", [
    (6, 48, 4, (0, 700), False),    # empty to long prefixes
    (5, 64, 4, (0, 1000), True),    # paged, two row tiles per KV head
    (4, 80, 2, (200, 200), False),  # equal lengths: shares may still straddle units
    (3, 136, 1, (0, 5), False),     # fewer tiles than workgroups: one-tile shares
    (40, 72, 2, (0, 300), True),    # many short sequences, shares of one or two tiles
])
def test_bf16_balanced_schedule(S, B, G, prefix, paged):
    """Several sequences with more than 128 rows per KV head: workgroups take equal shares
    of all units' key tiles, so a unit is split at arbitrary tiles and merged from the
    pieces of the workgroups it spans."""
    w = wl.make("ragged", 455 + S, parts=("attn",), qk_std=1.0,
                **_small(S=S, B=B, Hq=2 * G, Hkv=2, prefix=prefix, paged=paged,
                         N=min(10, B - 1) if B > 1 else 0, W=4))
    _check(w, f"balanced S={S} B={B} G={G} paged={paged}")


def test_fp32_paged_and_gqa():
    w = wl.make("ragged", 450, parts=("attn",), **_small(S=2, dtype="f32", d=64, Hq=8, Hkv=1,
                                                           prefix=(33, 97), paged=True, B=20))
    _check(w, "fp32 paged G=8")


def test_bad_block_flag_and_explicit_scale():
    w = wl.make("ragged", 460, parts=("attn",), **_small(S=2, prefix=(40, 80), paged=True))
    w.block_table[1, 1] = w.num_blocks + 3
    out, lse, err = _run_gpu(w)
    assert err[0] == 0 and err[1] == jt.DEV_BAD_BLOCK
    w2 = wl.make("ragged", 461, parts=("attn",), **_small(S=1, prefix=60, paged=False))
    _check(w2, "scale 0.3", scale=0.3)


def test_sibling_invariance_bitwise():
    """Perturbing K/V of nodes outside Anc(v) u {v} leaves row v bit-identical."""
    w = wl.make("ragged", 470, parts=("attn",), qk_std=1.0,
                **_small(S=1, B=96, prefix=150, paged=False, N=6, W=5))
    base, _, _ = _run_gpu(w)
    vis, _, _ = oracle.build_mask(w.parent)
    rng = np.random.default_rng(0)
    for v in (3, 40, 95):
        hidden = ~vis[0, v].astype(bool)
        w2 = wl.make("ragged", 470, parts=("attn",), qk_std=1.0,
                     **_small(S=1, B=96, prefix=150, paged=False, N=6, W=5))
        n = int(hidden.sum())
        w2.k_tree[0, hidden] = wl.to_dtype(rng.normal(0, 3, (n,) + w2.k_tree.shape[2:]), "bf16")
        w2.v_tree[0, hidden] = wl.to_dtype(rng.normal(0, 3, (n,) + w2.v_tree.shape[2:]), "bf16")
        pert, _, _ = _run_gpu(w2)
        assert np.array_equal(pert[0, v], base[0, v])
        assert not np.array_equal(pert, base)


def _sample(w, n, seed):
    rng = np.random.default_rng(seed)
    cfg = w.cfg
    sel = np.stack([rng.integers(0, cfg.S, n), rng.integers(0, cfg.B, n),
                    rng.integers(0, cfg.Hq, n)], 1).astype(np.int32)
    # always include the first and last rows and the deepest node of sequence 0
    extra = np.array([[0, 0, 0], [cfg.S - 1, cfg.B - 1, cfg.Hq - 1],
                      [0, int(w.depth[0].argmax()), 1 % cfg.Hq]], np.int32)
    return np.concatenate([sel, extra])


@pytest.mark.parametrize("name", ["low_budget", "high_budget", "ragged", "moe_verify"])
def test_config_full_size_sampled(name):
    w = wl.make(name, 480, parts=("attn",))
    _check(w, name, sel=_sample(w, 96, 1))


@pytest.mark.parametrize("name", ["ragged", "moe_verify"])
@pytest.mark.parametrize("sharp", [False, True])
def test_config_full_size_whole_blocks(name, sharp):
    """ragged (paged, shuffled table, balanced schedule) and moe_verify at full size: every
    row of one whole 256-row block of query rows per sequence (a different KV head and
    block from one sequence to the next), and the sharp variant (q, k ~ N(0, 1))."""
    w = wl.make(name, 482, parts=("attn",), qk_std=1.0 if sharp else None)
    cfg = w.cfg
    print(f"[attn] {name} sharp={sharp} whole blocks", flush=True)
    out, lse, err = _run_gpu(w)
    sel, ref, rlse, rerr = oracle_attention(w, block_rows(w))
    assert np.array_equal(err, rerr)
    got = out[sel[:, 0], sel[:, 1], sel[:, 2]]
    glse = lse[sel[:, 0], sel[:, 1], sel[:, 2]]
    assert_attention_close(got, ref, cfg.dtype, f"{name} sharp={sharp}")
    assert_lse_close(glse, rlse, cfg.dtype, f"{name} sharp={sharp}")


@pytest.mark.parametrize("name", ["low_budget", "high_budget"])
def test_config_full_size_sharp_all_rows(name):
    w = wl.make(name, 481, parts=("attn",), qk_std=1.0)
    _check(w, name + " sharp")


def test_deterministic():
    w = wl.make("high_budget", 490, parts=("attn",))
    a, _, _ = _run_gpu(w)
    b, _, _ = _run_gpu(w)
    assert np.array_equal(a, b)
