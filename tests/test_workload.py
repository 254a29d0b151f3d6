"""Seeded input generator: determinism and the structure the workloads promise."""
import numpy as np
import pytest
import torch

from tree_causal_draft_amd import workload as wl


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).normal(0, 7, 100000).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 3.0e4]   # ties to even, signed zero
    mine = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(wl.bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_same_seed_same_bytes():
    a = wl.make("ragged", 3, V=2048, prefix=(16, 200))
    b = wl.make("ragged", 3, V=2048, prefix=(16, 200))
    for f in ("parent", "tokens", "planted_next", "prefix_len", "q", "k_tree", "v_tree",
              "k_prefix", "v_prefix", "block_table", "draft_logits", "target_logits"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = wl.make("ragged", 4, V=2048, prefix=(16, 200))
    assert not np.array_equal(a.target_logits, c.target_logits)


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_tree_structure(name):
    cfg = wl.CONFIGS[name]
    w = wl.make(name, 1, parts=())
    for s in range(cfg.S):
        par = w.parent[s]
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, cfg.B))
        assert w.depth[s].max() <= cfg.N
        ch = wl.children_lists(par)
        assert max(len(c) for c in ch) <= cfg.W
        for kids in ch:   # siblings carry distinct tokens
            toks = [int(w.tokens[s, u]) for u in kids]
            assert len(set(toks)) == len(toks)
    if cfg.tree == "best_first":
        spine = wl.spine_of(w.parent[0], w.rank[0])
        assert len(spine) - 1 == w.depth[0].max()


def test_known_shapes():
    w = wl.make("low_budget", 1, parts=())
    assert w.depth[0].max() == 4           # each expansion spends W=4 nodes
    w = wl.make("high_budget", 1, parts=())
    assert w.depth[0].max() == 16
    w = wl.make("tiny", 1, parts=())
    assert w.depth[0].max() <= 4


def test_planting_makes_unique_row_maxima():
    w = wl.make("moe_verify", 2, S=3, V=5000)
    t = wl.as_float32(w.target_logits)
    top = t.max(1)
    assert ((t == top[:, None]).sum(1) == 1).all()
    assert np.array_equal(t.argmax(1), w.planted_next.reshape(-1))
    d = wl.as_float32(w.draft_logits)
    assert np.array_equal(d.argmax(1), w.extra["candidates"][:, 1:, 0].reshape(-1))


def test_spine_acceptance_rate():
    hits = tot = 0
    for seed in range(40):
        w = wl.make("moe_verify", seed, parts=(), S=8)
        for s in range(8):
            spine = wl.spine_of(w.parent[s], w.rank[s])
            for a, b in zip(spine[:-1], spine[1:]):
                tot += 1
                hits += int(w.planted_next[s, a] == w.tokens[s, b])
    assert abs(hits / tot - 0.7) < 4 * np.sqrt(0.21 / tot)


def test_prefix_poison_and_paged_table():
    w = wl.make("ragged", 6, parts=("attn",), V=64, prefix=(20, 90), block_size=16)
    bt = w.block_table
    used = np.concatenate([bt[s, : -(-int(p) // 16)] for s, p in enumerate(w.prefix_len)])
    assert sorted(used.tolist()) == list(range(w.num_blocks))   # a permutation of the pool
    kc, _ = wl.contiguous_prefix(w)
    pois = wl.scalar_in_dtype(wl.POISON, "bf16")
    for s, p in enumerate(w.prefix_len):
        assert (kc[s, p:] == pois).all() and not (kc[s, :p] == pois).any()
        last = bt[s, (int(p) - 1) // 16]
        tail = int(p) % 16
        if tail:
            assert (w.k_prefix[last, tail:] == pois).all()
