"""Helpers for the GPU parity tests (device transfers and the comparison rules)."""
import numpy as np
import pytest
import torch

from tree_causal_draft_amd import workload as wl
from tree_causal_draft_amd.step import to_device

DEV = "cuda:0"

# attention tolerances: |gpu - ref| <= atol + rtol*|ref| elementwise, plus relative L2
BF16_ATOL, BF16_RTOL, BF16_RELL2 = 2e-2, 1e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-5, 1e-5
# log-prob / LSE tolerance (fp32 sums over up to 151,936 terms)
LP_ATOL, LP_RTOL = 1e-5, 1e-5
# attention LSE, elementwise.  bf16: the scores are fp32 sums of d exact bf16 products
# (error <= d*u*scale*sum|q_i k_i| with u = 2^-24: about 1.1e-4 for d = 128, q, k ~ N(0, 1))
# and l is an fp32 sum of at most n = 8,448 terms (relative error <= n*u = 5e-4), so the
# natural-log LSE is off by at most about 6e-4 plus rounding of its own magnitude; fp32
# keeps the stated fp32 tolerance
LSE_ATOL = {"bf16": 1e-3, "f32": 1e-5}
LSE_RTOL = {"bf16": 1e-5, "f32": 1e-5}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU (deselect with -m 'not gpu')")


def dev(a):
    return to_device(a, DEV)


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return wl.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def anc_to_dense(anc_np, B):
    """uint64 rows [S,B,4] -> dense uint8 [S,B,B] (bit u of word u>>6)."""
    a = anc_np.view(np.uint64)
    S = a.shape[0]
    out = np.zeros((S, B, B), np.uint8)
    for u in range(B):
        out[:, :, u] = ((a[:, :, u >> 6] >> np.uint64(u & 63)) & np.uint64(1)).astype(np.uint8)
    return out


def assert_attention_close(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "f32":
        bad = np.abs(got - ref) > F32_ATOL + F32_RTOL * np.abs(ref)
        assert not bad.any(), f"{what}: {bad.sum()} elements off, max err {np.abs(got-ref).max():.3e}"
        return
    bad = np.abs(got - ref) > BF16_ATOL + BF16_RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements off, max err {np.abs(got-ref).max():.3e}"
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= BF16_RELL2, f"{what}: relative L2 {rel:.3e}"


def assert_lp_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN positions differ"
    ok = ~np.isnan(ref)
    g, r = got[ok], ref[ok]
    # an infinite reference is matched only by the same infinity (|g - r| <= atol + rtol*inf
    # would accept any finite value); a finite one within the tolerance (an infinite g fails)
    inf = np.isinf(r)
    with np.errstate(invalid="ignore"):  # inf - inf where both are infinite: decided by g != r
        bad = np.where(inf, g != r, ~(np.abs(g - r) <= LP_ATOL + LP_RTOL * np.abs(r)))
    assert not bad.any(), (f"{what}: {int(bad.sum())} entries off, "
                           f"max err {np.nanmax(np.abs(g - r)) if g.size else 0:.3e}")


def assert_lse_close(got, ref, dtype, what=""):
    """Attention LSE, elementwise; an infinite reference (a row with no visible key) must be
    matched by the same infinity."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, what
    inf = np.isinf(ref)
    with np.errstate(invalid="ignore"):
        bad = np.where(inf, got != ref,
                       ~(np.abs(got - ref) <= LSE_ATOL[dtype] + LSE_RTOL[dtype] * np.abs(ref)))
    fin = ~inf
    err = np.abs(got[fin] - ref[fin]).max() if fin.any() else 0.0
    assert not bad.any(), f"{what}: {int(bad.sum())} LSE entries off, max err {err:.3e}"
    return err


def block_rows(w, rows_per_block=256):
    """(s, v, h) of every row of one whole block of query rows per sequence: the rows of KV
    head g = s % Hkv, ordered node-major (row r = node r / G, head g*G + r % G), block
    b = (s / Hkv) mod (number of blocks) of `rows_per_block` rows."""
    c = w.cfg
    G = c.Hq // c.Hkv
    R = G * c.B
    nblk = -(-R // rows_per_block)
    out = []
    for s in range(c.S):
        g = s % c.Hkv
        b = (s // c.Hkv) % nblk
        r = np.arange(b * rows_per_block, min(R, (b + 1) * rows_per_block))
        out.append(np.stack([np.full_like(r, s), r // G, g * G + r % G], 1))
    return np.concatenate(out).astype(np.int32)


def oracle_attention(w, sel=None, threads=16, **kw):
    """oracle.tree_attention over `sel` (all rows when None), the rows split over host
    threads (the oracle is single-threaded C; ctypes releases the GIL during the call)."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    c = w.cfg
    base = dict(block_table=w.block_table, block_size=c.block_size, num_blocks=w.num_blocks,
                max_prefix=w.max_prefix)
    base.update(kw)
    if sel is None:
        sel = np.stack(np.meshgrid(np.arange(c.S), np.arange(c.B), np.arange(c.Hq),
                                   indexing="ij"), -1).reshape(-1, 3).astype(np.int32)
    parts = [p for p in np.array_split(sel, max(1, min(threads, len(sel) // 64))) if len(p)]
    oracle.build_mask(np.zeros((1, 1), np.int32) - 1)  # loads the library before the threads

    def run(p):
        return oracle.tree_attention(w.q, w.k_tree, w.v_tree, w.k_prefix, w.v_prefix,
                                     w.prefix_len, w.parent, sel=p, **base)
    with ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(run, parts))
    out = np.concatenate([r[0] for r in res])
    lse = np.concatenate([r[1] for r in res])
    return sel, out, lse, res[0][2]
