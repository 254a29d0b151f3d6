"""Pins for the oracle's tree-causal GQA attention (CPU only).

Definition pinned: node v attends to the whole prefix, its ancestors and itself
and to no sibling or descendant (JetSpec review, startedourmission.github.io,
'How it works', mask equation and branch-wise factorisation; paperlayer.ai
JetSpec summary, section 2 'Architecture').  A chain tree reproduces the
autoregressive factorisation, i.e. ordinary causal attention (same review,
factorisation of p(y_1:k | x)).  Readings: scale 1/sqrt(d), query head h uses
KV head h // (Hq/Hkv).
"""
import numpy as np
import pytest
import torch

import oracle
from tree_causal_draft_amd import workload as wl

F = torch.nn.functional


def _f64(a):
    return torch.from_numpy(wl.as_float32(a).astype(np.float64))


def _small(dtype, **kw):
    base = dict(S=2, prefix=37, B=9, N=8, W=3, Hq=4, Hkv=2, d=16, V=64, dtype=dtype)
    base.update(kw)
    return base


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2), (4, 4), (8, 1)])
def test_chain_tree_equals_causal_attention(dtype, Hq, Hkv):
    """Chain tree == textbook causal self-attention over [prefix; chain] (torch SDPA,
    fp64, enable_gqa -> repeat_interleave head mapping)."""
    B, P = 9, 37
    w = wl.make("tiny", 3, parts=("attn",), trees=[wl.chain_tree(B)] * 2,
                **_small(dtype, Hq=Hq, Hkv=Hkv, B=B, prefix=P))
    out, lse, err = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                          w.prefix_len, w.parent)
    assert not err.any()
    for s in range(2):
        k = torch.cat([_f64(w.k_prefix[s, :P]), _f64(w.k_tree[s])], 0)   # [L,Hkv,d]
        v = torch.cat([_f64(w.v_prefix[s, :P]), _f64(w.v_tree[s])], 0)
        junk = torch.randn(P, Hq, k.shape[-1], dtype=torch.float64)
        q = torch.cat([junk, _f64(w.q[s])], 0)                            # [L,Hq,d]
        ref = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                             v.transpose(0, 1)[None], is_causal=True,
                                             enable_gqa=True)[0].transpose(0, 1)[P:]
        np.testing.assert_allclose(out[s], ref.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_random_tree_equals_masked_sdpa(dtype):
    """Any tree == SDPA with the brute-force ancestor mask (prefix fully visible)."""
    B, P = 24, 21
    w = wl.make("tiny", 5, parts=("attn",), **_small(dtype, B=B, prefix=P, N=6, W=3))
    out, lse, _ = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                        w.prefix_len, w.parent)
    for s in range(2):
        par = w.parent[s]
        allowed = torch.zeros(B, P + B, dtype=torch.bool)
        allowed[:, :P] = True
        for v in range(B):
            u = v
            while u != -1:
                allowed[v, P + u] = True
                u = int(par[u])
        k = torch.cat([_f64(w.k_prefix[s, :P]), _f64(w.k_tree[s])], 0).transpose(0, 1)[None]
        vv = torch.cat([_f64(w.v_prefix[s, :P]), _f64(w.v_tree[s])], 0).transpose(0, 1)[None]
        q = _f64(w.q[s]).transpose(0, 1)[None]
        ref = F.scaled_dot_product_attention(q, k, vv, attn_mask=allowed, enable_gqa=True)
        np.testing.assert_allclose(out[s], ref[0].transpose(0, 1).numpy(), rtol=1e-12, atol=1e-12)
        # log-sum-exp of the visible scores, via torch.logsumexp on explicit scores
        G = w.q.shape[2] // w.k_tree.shape[2]
        kk = k[0].repeat_interleave(G, 0)                                  # [Hq,L,d]
        sc = torch.einsum("hvd,hjd->hvj", q[0], kk) / np.sqrt(q.shape[-1])
        sc = sc.masked_fill(~allowed[None], float("-inf"))
        np.testing.assert_allclose(lse[s], torch.logsumexp(sc, -1).transpose(0, 1).numpy(),
                                   rtol=1e-12, atol=1e-12)


def test_sibling_invariance_bitwise():
    """Perturbing every node outside Anc(v) u {v} leaves row v bit-identical."""
    B, P = 30, 19
    w = wl.make("tiny", 11, parts=("attn",), **_small("bf16", S=1, B=B, prefix=P, N=5, W=4))
    base, _, _ = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                       w.prefix_len, w.parent)
    vis, _, _ = oracle.build_mask(w.parent)
    rng = np.random.default_rng(0)
    for v in [0, 5, 17, B - 1]:
        hidden = ~vis[0, v].astype(bool)
        kt, vt, q = w.k_tree.copy(), w.v_tree.copy(), w.q.copy()
        n = int(hidden.sum())
        kt[0, hidden] = wl.to_dtype(rng.normal(0, 5, (n,) + kt.shape[2:]), "bf16")
        vt[0, hidden] = wl.to_dtype(rng.normal(0, 5, (n,) + vt.shape[2:]), "bf16")
        q[0, hidden] = wl.to_dtype(rng.normal(0, 5, (n,) + q.shape[2:]), "bf16")
        pert, _, _ = oracle.tree_attention(q, kt, vt, w.k_prefix, w.v_prefix, w.prefix_len,
                                           w.parent)
        assert np.array_equal(pert[0, v], base[0, v])
        if n:   # and the perturbation is visible elsewhere (the test has teeth)
            assert not np.array_equal(pert, base)


def test_equal_keys_closed_form():
    """All keys equal => output = mean of visible values, lse = s + log(#visible)."""
    B, P, d = 12, 7, 16
    w = wl.make("tiny", 2, parts=("attn",), **_small("f32", S=1, B=B, prefix=P, d=d))
    kvec = np.random.default_rng(1).normal(size=d).astype(np.float32)
    kt = np.broadcast_to(kvec, w.k_tree.shape).copy()
    kp = np.broadcast_to(kvec, w.k_prefix.shape).copy()
    out, lse, _ = oracle.tree_attention(w.q, kt, w.v_tree, kp, w.v_prefix, w.prefix_len,
                                        w.parent)
    vis, _, _ = oracle.build_mask(w.parent)
    G = w.q.shape[2] // w.k_tree.shape[2]
    for v in range(B):
        for h in range(w.q.shape[2]):
            g = h // G
            vals = np.concatenate([w.v_prefix[0, :P, g].astype(np.float64),
                                   w.v_tree[0, vis[0, v].astype(bool), g].astype(np.float64)])
            np.testing.assert_allclose(out[0, v, h], vals.mean(0), rtol=1e-12, atol=1e-13)
            s_ = float(np.dot(w.q[0, v, h].astype(np.float64), kvec.astype(np.float64))) / 4.0
            np.testing.assert_allclose(lse[0, v, h], s_ + np.log(len(vals)), rtol=1e-12)


def test_single_node_no_prefix():
    """B=1, P=0: the root sees only itself: out = v_root, lse = scale*<q,k_root>."""
    w = wl.make("tiny", 4, parts=("attn",), **_small("f32", S=1, B=1, prefix=0))
    out, lse, _ = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                        w.prefix_len, w.parent)
    G = 2
    for h in range(4):
        np.testing.assert_array_equal(out[0, 0, h], w.v_tree[0, 0, h // G].astype(np.float64))
        s_ = np.dot(w.q[0, 0, h].astype(np.float64), w.k_tree[0, 0, h // G].astype(np.float64)) / 4
        np.testing.assert_allclose(lse[0, 0, h], s_, rtol=1e-14)


def test_poisoned_tail_and_selected_rows():
    """Keys past prefix_len never count; selected rows equal the full computation."""
    w = wl.make("tiny", 9, parts=("attn",), prefix_len=[13, 40],
                **_small("bf16", prefix=(13, 40)))
    full, lse, _ = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                         w.prefix_len, w.parent)
    assert w.k_prefix.shape[1] == 40
    cut, _, _ = oracle.tree_attention(w.q[:1], w.k_tree[:1], w.v_tree[:1], w.k_prefix[:1, :13],
                                      w.v_prefix[:1, :13], w.prefix_len[:1], w.parent[:1])
    np.testing.assert_array_equal(full[0], cut[0])
    sel = np.array([[1, 3, 2], [0, 0, 0], [1, 8, 3]], np.int32)
    o2, l2, _ = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                      w.prefix_len, w.parent, sel=sel)
    for i, (s, v, h) in enumerate(sel):
        np.testing.assert_array_equal(o2[i], full[s, v, h])
        assert l2[i] == lse[s, v, h]


def test_paged_equals_contiguous():
    w = wl.make("ragged", 5, parts=("attn",), prefix_len=[5, 16, 33],
                **_small("bf16", S=3, prefix=(5, 33), paged=True, block_size=4))
    kc, vc = wl.contiguous_prefix(w)
    a, la, ea = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                      w.prefix_len, w.parent, block_table=w.block_table,
                                      block_size=4, max_prefix=w.max_prefix)
    b, lb, eb = oracle.tree_attention(w.q, w.k_tree, w.v_tree, kc, vc, w.prefix_len, w.parent)
    assert not ea.any() and not eb.any()
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_bad_block_and_prefix_flags():
    w = wl.make("ragged", 5, parts=("attn",), prefix_len=[8, 16],
                **_small("bf16", S=2, prefix=(8, 16), paged=True, block_size=4))
    bt = w.block_table.copy()
    bt[1, 2] = w.num_blocks          # out of range
    _, _, err = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                      w.prefix_len, w.parent, block_table=bt, block_size=4,
                                      max_prefix=w.max_prefix)
    assert err[0] == 0 and err[1] == oracle.BAD_BLOCK
    pl = w.prefix_len.copy()
    pl[0] = w.max_prefix + 1
    _, _, err = oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix, pl,
                                      w.parent, block_table=w.block_table, block_size=4,
                                      max_prefix=w.max_prefix)
    assert err[0] & oracle.BAD_PREFIX and err[1] == 0
