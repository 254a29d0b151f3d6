"""CPU checks of the C ABI: the library loads, exports what include/jt.h declares, and
rejects bad arguments on the host before anything is launched (no GPU needed)."""
import ctypes
import os
import re

import pytest

import tree_causal_draft_amd as jt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "jt.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(jt_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_the_four_steps():
    names = _declared()
    for n in ("jt_build_tree_mask", "jt_tree_attention", "jt_topw_per_depth", "jt_verify_greedy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = jt.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert set(_declared()) <= set(jt.EXPORTS)


def test_version_and_status_strings():
    L = jt.lib()
    assert L.jt_abi_version() == 2
    assert L.jt_status_string(0) == b"ok"
    assert b"NULL" in L.jt_status_string(1)
    assert L.jt_status_string(99) == b"unknown status"


def test_host_validation_returns_before_launch():
    L = jt.lib()
    nul = None
    # mask: B out of range, NULL pointers
    assert L.jt_build_tree_mask(nul, 1, 0, nul, nul, nul, nul) == 2
    assert L.jt_build_tree_mask(nul, 1, 257, nul, nul, nul, nul) == 2
    assert L.jt_build_tree_mask(nul, 1, 16, nul, nul, nul, nul) == 1
    assert L.jt_build_tree_mask(nul, 0, 16, nul, nul, nul, nul) == 0   # empty batch: no-op
    # top-W: W > 16, W > V, bad dtype, stride < V, NULLs
    args = lambda rows, V, W, dt, stride=None: (nul, stride or V, rows, V, W, dt, nul, nul, nul,
                                                 nul, nul, 0, nul)
    assert L.jt_topw_per_depth(*args(4, 100, 17, 1)) == 2
    assert L.jt_topw_per_depth(*args(4, 3, 4, 1)) == 2
    assert L.jt_topw_per_depth(*args(4, 100, 4, 7)) == 3
    assert L.jt_topw_per_depth(*args(4, 100, 4, 1, stride=50)) == 2
    assert L.jt_topw_per_depth(*args(4, 100, 4, 1)) == 1
    # attention: d = 96, Hq % Hkv, G > 8, NULLs, workspace
    def attn(S=1, B=16, Hq=32, Hkv=8, d=128, dt=1, P=64):
        return L.jt_tree_attention(nul, nul, nul, nul, nul, nul, 0, 16, 0, nul, P, nul, S, B, Hq,
                                   Hkv, d, dt, ctypes.c_float(0.0), nul, nul, nul, nul, 0, nul)
    assert attn(d=96) == 2
    assert attn(Hq=30, Hkv=8) == 2
    assert attn(Hq=32, Hkv=2) == 2
    assert attn(B=300) == 2
    assert attn(dt=5) == 3
    assert attn() == 1
    # verify: N > 255, NULLs
    def ver(N=8, B=16):
        return L.jt_verify_greedy(nul, 1000, 1000, 1, nul, nul, nul, nul, 1, B, N, nul, nul, nul,
                                  nul, nul, nul, 0, nul)
    assert ver(N=256) == 2
    assert ver() == 1
    # tree construction: W, B, N out of range, NULLs, empty batch
    def tree(S=1, N=4, W=2, B=16):
        return L.jt_build_tree_best_first(nul, nul, nul, ctypes.c_float(1.0), ctypes.c_float(0.0),
                                          nul, S, N, W, B, nul, nul, nul, nul, nul)
    assert tree(W=0) == 2 and tree(W=17) == 2
    assert tree(B=0) == 2 and tree(B=257) == 2
    assert tree(N=-1) == 2 and tree(N=256) == 2
    assert tree() == 1
    assert tree(S=0) == 0
    # accepted-path commit: d, dtype, N, NULLs
    def commit(S=1, N=4, B=16, d=128, dt=1, table=None):
        return L.jt_commit_accepted_kv(nul, nul, N, nul, nul, S, B, 8, d, dt, nul, nul, table,
                                       4, 16, 8, nul, 64, nul, nul, nul)
    assert commit(d=96) == 2 and commit(N=256) == 2 and commit(B=0) == 2
    assert commit(dt=5) == 3
    assert commit() == 1
    assert commit(S=0) == 0
    # sampled verification: temperature <= 0 or inf, N > 255, NULLs
    def smp(T=1.0, N=8):
        return L.jt_verify_sampled(nul, 1000, 1000, 1, ctypes.c_float(T), nul, nul, nul, nul,
                                   nul, 1, 16, N, nul, nul, nul, nul, nul, nul, 0, nul)
    assert smp(T=0.0) == 2 and smp(T=-1.0) == 2 and smp(T=float("inf")) == 2
    # log2(e)/T overflows fp32 below about 4.2e-39 (a subnormal T): refused, not NaN weights
    assert smp(T=1e-39) == 2 and smp(T=1e-38) != 2
    assert smp(N=256) == 2
    assert smp() == 1
    # the matrix-core rate probe
    assert L.jt_probe_mfma_rate(0, 4, nul, nul) == 2 and L.jt_probe_mfma_rate(4, 0, nul, nul) == 2
    assert L.jt_probe_mfma_rate(4, 4, nul, nul) == 1


def test_workspace_queries_are_pure():
    assert jt.topw_workspace_size(16, 151936, 4, 1) > 0
    assert jt.verify_workspace_size(1, 16, 151936, 1) > 0
    # several sequences take the balanced schedule: a table of units' share ranges and a partial
    # slot per (unit + workgroup; 256 workgroups of 8 waves here), since prefix lengths are
    # known on the device only; one short sequence is split into chunks; fp32 needs none
    units, nwg, rows, d = 32 * 4 * 2, 256, 256, 128
    slots = (units + nwg) * rows
    table = -(-units * 8 // 256) * 256  # each unit's first and last share
    assert jt.tree_attention_workspace_size(32, 64, 32, 4, 128, 4096, 1) == \
        table + slots * 8 + slots * d * 2
    assert jt.tree_attention_workspace_size(1, 16, 32, 8, 128, 1024, 1) > 0
    assert jt.tree_attention_workspace_size(1, 16, 4, 2, 64, 64, 0) == 0


def test_noalloc_step_rejects_shapes_beyond_its_scratch():
    """jt_draft_verify_step_noalloc refuses, on the host and before any device work, a shape
    whose step workspace exceeds the static scratch (JT_ERR_SCRATCH); the pointers below are
    never dereferenced."""
    L = jt.lib()
    assert L.jt_status_string(7).startswith(b"the shape needs more scratch")
    fake = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never touched

    def call(S, P, V=151936):
        return L.jt_draft_verify_step_noalloc(
            fake, V, fake, V, V, 8, fake, fake, S, 64, 8, fake, fake, fake, fake, fake, None,
            0, 16, 0, fake, P, 32, 4, 128, ctypes.c_float(0.0), 1, fake, fake, fake, None, fake,
            fake, fake, fake, fake, fake, fake, fake, fake, None)
    big = jt.step_workspace_size(128, 64, 8, 8, 151936, 32, 4, 128, 4096, 1)
    assert big > jt.STATIC_SCRATCH_BYTES
    assert call(128, 4096) == 7
    assert call(0, 4096) == 0          # nothing to do
    assert call(128, 4096, V=0) == 2   # shape errors come first
