"""GPU parity of jt_commit_accepted_kv: the caches, new lengths and flags must equal the
oracle's bit for bit (the commit is a pure gather)."""
import numpy as np
import pytest
import torch

import oracle
import tree_causal_draft_amd as jt
from tree_causal_draft_amd import workload as wl
from tree_causal_draft_amd.step import DeviceStep
from gpu_util import dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32 if a.dtype.itemsize == 4 else np.uint16)


def _run(L, path, kt, vt, kc, vc, P, table=None, bs=16, what="", inplace=False):
    need_gpu()
    S, B, Hkv, d = kt.shape
    print(f"[commit] {what}: S={S} B={B} Hkv={Hkv} d={d} paged={table is not None} "
          f"{kt.dtype}", flush=True)
    t = lambda a: dev(np.ascontiguousarray(a))
    gk, gv, gP = t(kc), t(vc), t(np.asarray(P, np.int32))
    args = dict(block_table=None if table is None else t(np.asarray(table, np.int32)),
                block_size=bs)
    if inplace:
        newp, err = jt.commit_accepted_kv(t(np.asarray(L, np.int32)), t(np.asarray(path, np.int32)),
                                          t(kt), t(vt), gk, gv, gP, new_prefix_len=gP, **args)
    else:
        newp, err = jt.commit_accepted_kv(t(np.asarray(L, np.int32)), t(np.asarray(path, np.int32)),
                                          t(kt), t(vt), gk, gv, gP, **args)
    torch.cuda.synchronize()
    rk, rv, rP, rerr = oracle.commit_kv(L, path, path.shape[1] - 1, kt, vt, kc, vc, P,
                                        block_table=table, block_size=bs)
    got_k, got_v = host_raw(gk, kt.dtype), host_raw(gv, kt.dtype)
    assert np.array_equal(_bits(got_k), _bits(rk)), what
    assert np.array_equal(_bits(got_v), _bits(rv)), what
    assert np.array_equal(host(newp), rP), what
    assert np.array_equal(host(err), rerr), what
    return rP, rerr


def host_raw(t, dtype):
    if dtype == np.uint16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _case(seed, S, B, N, Hkv, d, dtype, cap):
    rng = np.random.default_rng(seed)
    kt = wl.to_dtype(rng.normal(0, 1, (S, B, Hkv, d)).astype(np.float32), dtype)
    vt = wl.to_dtype(rng.normal(0, 1, (S, B, Hkv, d)).astype(np.float32), dtype)
    L = rng.integers(0, N + 1, S).astype(np.int32)
    path = np.full((S, N + 1), -1, np.int32)
    for s in range(S):
        path[s, 0] = 0
        path[s, 1:L[s] + 1] = np.sort(rng.choice(np.arange(1, B), L[s], replace=False))
    P = rng.integers(0, cap - N - 1, S).astype(np.int32)
    return kt, vt, L, path, P


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_contiguous(dtype, d):
    S, B, N, Hkv, Pmax = 6, 64, 12, 4, 200
    kt, vt, L, path, P = _case(900 + d, S, B, N, Hkv, d, dtype, Pmax)
    rng = np.random.default_rng(d)
    kc = wl.to_dtype(rng.normal(0, 1, (S, Pmax, Hkv, d)).astype(np.float32), dtype)
    vc = wl.to_dtype(rng.normal(0, 1, (S, Pmax, Hkv, d)).astype(np.float32), dtype)
    _run(L, path, kt, vt, kc, vc, P, what=f"contiguous {dtype} d={d}")
    _run(L, path, kt, vt, kc, vc, P, what="in place", inplace=True)


@pytest.mark.parametrize("bs", [16, 5])
def test_paged_shuffled(bs):
    S, B, N, Hkv, d, nb = 5, 128, 12, 8, 128, 12
    kt, vt, L, path, P = _case(910 + bs, S, B, N, Hkv, d, "bf16", nb * bs)
    rng = np.random.default_rng(bs)
    table = rng.permutation(S * nb).astype(np.int32).reshape(S, nb)
    pool = wl.to_dtype(rng.normal(0, 1, (S * nb, bs, Hkv, d)).astype(np.float32), "bf16")
    _run(L, path, kt, vt, pool, pool.copy(), P, table=table, bs=bs, what=f"paged bs={bs}")


def test_flags():
    S, B, N, Hkv, d = 5, 16, 5, 2, 64
    kt, vt, L, path, P = _case(920, S, B, N, Hkv, d, "bf16", 16)
    L[0] = 6                      # accept_len > N
    P[1] = 14                     # the path would overflow the cache
    L[2] = max(L[2], 1)
    path[2, 1] = 99               # a path entry outside [0, B)
    L[3] = -1                     # negative length
    kc = np.zeros((S, 16, Hkv, d), np.uint16)
    _, err = _run(L, path, kt, vt, kc, kc.copy(), P, what="flags contiguous")
    assert err.tolist()[:4] == [2, 16, 1, 2]
    table = np.arange(S * 8, dtype=np.int32).reshape(S, 8)
    table[4, 0] = 1000            # a bad block id
    L2 = np.array([0, 0, 0, 0, 3], np.int32)
    P2 = np.zeros(S, np.int32)
    pool = np.zeros((S * 8, 2, Hkv, d), np.uint16)
    _, err = _run(L2, path, kt, vt, pool, pool.copy(), P2, table=table, bs=2, what="bad block")
    assert err[4] == 4


@pytest.mark.parametrize("name", ["low_budget", "ragged"])
def test_after_device_verify(name):
    """The device verification's accepted paths feeding the commit, on a config's tree
    K/V, into a cache with room for the path (a fresh contiguous one, or the ragged
    config's paged pool extended by the blocks the path needs)."""
    need_gpu()
    w = wl.make(name, 930)
    c = w.cfg
    st = DeviceStep(w, "cuda:0")
    st.run()
    torch.cuda.synchronize()
    L, path = host(st.accept_len), host(st.accept_path)
    kt, vt = w.k_tree, w.v_tree
    if w.block_table is None:
        cap = w.max_prefix + c.N + 1
        kc = np.zeros((c.S, cap, c.Hkv, c.d), kt.dtype)
        kc[:, :w.max_prefix] = w.k_prefix
        vc = np.zeros_like(kc)
        vc[:, :w.max_prefix] = w.v_prefix
        _run(L, path, kt, vt, kc, vc, w.prefix_len, what=name)
    else:
        bs = c.block_size
        extra = (c.N + 1 + bs - 1) // bs + 1
        nb0 = w.k_prefix.shape[0]
        table = np.concatenate([w.block_table, np.full((c.S, extra), -1, np.int32)], 1)
        for s in range(c.S):
            used = (int(w.prefix_len[s]) + bs - 1) // bs
            table[s, used:used + extra] = nb0 + s * extra + np.arange(extra)
        pad = np.zeros((c.S * extra,) + w.k_prefix.shape[1:], w.k_prefix.dtype)
        kc = np.concatenate([w.k_prefix, pad])
        vc = np.concatenate([w.v_prefix, pad])
        _, err = _run(L, path, kt, vt, kc, vc, w.prefix_len, table=table, bs=bs, what=name)
        assert not err.any()
