"""CPU oracle for the tree draft-and-verify step -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, loads or calls anything here, and this package
imports nothing from the product.

The arithmetic lives in ``jt_oracle.c`` (plain single-threaded C11, fp64); this
module compiles it with gcc and marshals numpy arrays to it.  bfloat16 tensors
travel as raw ``uint16`` words.

Pins (tests that hold the oracle to something other than itself) are in
``tests/test_oracle_*.py``.  No oracle function is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "jt_oracle.c")
_LIB = os.path.join(_HERE, "libjt_oracle.so")

# per-sequence flags, restated from the C file
BAD_PARENT = 1
DEPTH_GT_N = 2
BAD_BLOCK = 4
NAN = 8
BAD_PREFIX = 16

_lib = None


def build(force: bool = True) -> str:
    """Compile jt_oracle.c into libjt_oracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
                        "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile jt_oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer (any report
    aborts) into ``path``; a process loads it through JT_ORACLE_LIB with the sanitizer
    runtimes preloaded (the sanitized-pins test does exactly that)."""
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-Wall",
                    "-Wextra", "-o", path, _SRC, "-lm"], check=True)
    return path


def _load():
    global _lib
    if _lib is None:
        alt = os.environ.get("JT_ORACLE_LIB")
        if alt:
            _lib = ctypes.CDLL(alt)
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or bf16-as-uint16, got {a.dtype}")


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def build_mask(parent: np.ndarray):
    """parent int32 [S,B] -> (vis uint8 [S,B,B], depth int32 [S,B], err int32 [S])."""
    parent = _c(parent, np.int32)
    S, B = parent.shape
    vis = np.zeros((S, B, B), np.uint8)
    depth = np.zeros((S, B), np.int32)
    err = np.zeros(S, np.int32)
    rc = _load().jto_build_mask(_p(parent), S, B, _p(vis), _p(depth), _p(err))
    if rc:
        raise ValueError(f"jto_build_mask rc={rc}")
    return vis, depth, err


def tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, prefix_len, parent, *,
                   block_table=None, block_size=16, num_blocks=0, max_prefix=None,
                   scale=0.0, sel=None):
    """Tree-causal GQA attention in fp64.

    q [S,B,Hq,d]; k_tree, v_tree [S,B,Hkv,d]; contiguous prefix [S,Pmax,Hkv,d] or,
    with ``block_table`` [S,maxblk], a pool [nblk,block_size,Hkv,d].
    ``sel``: optional int array [n,3] of (s, v, h) rows to compute.
    Returns (out float64, lse float64, err int32[S]); out is [S,B,Hq,d] or [n,d].
    """
    dt = _dtype_code(q)
    for a in (k_tree, v_tree, k_prefix, v_prefix):
        if a.dtype != q.dtype:
            raise TypeError("all tensors must share one dtype")
    q, k_tree, v_tree = _c(q, q.dtype), _c(k_tree, q.dtype), _c(v_tree, q.dtype)
    k_prefix, v_prefix = _c(k_prefix, q.dtype), _c(v_prefix, q.dtype)
    S, B, Hq, d = q.shape
    Hkv = k_tree.shape[2]
    prefix_len = _c(prefix_len, np.int32)
    parent = _c(parent, np.int32)
    if block_table is None:
        bt, maxblk = None, 0
        Pmax = k_prefix.shape[1] if max_prefix is None else max_prefix
        nblk = 0
    else:
        bt = _c(block_table, np.int32)
        maxblk = bt.shape[1]
        Pmax = maxblk * block_size if max_prefix is None else max_prefix
        nblk = num_blocks if num_blocks else k_prefix.shape[0]
    if sel is None:
        nsel, selp = 0, None
        out = np.zeros((S, B, Hq, d), np.float64)
        lse = np.zeros((S, B, Hq), np.float64)
    else:
        sel = _c(sel, np.int32).reshape(-1, 3)
        nsel, selp = sel.shape[0], sel
        out = np.zeros((nsel, d), np.float64)
        lse = np.zeros(nsel, np.float64)
    err = np.zeros(S, np.int32)
    lib = _load()
    lib.jto_tree_attention.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 3 + [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p] + [ctypes.c_int] * 6 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]
    rc = lib.jto_tree_attention(_p(q), _p(k_tree), _p(v_tree), _p(k_prefix), _p(v_prefix),
                                _p(bt), maxblk, block_size, nblk, _p(prefix_len), Pmax,
                                _p(parent), S, B, Hq, Hkv, d, dt, float(scale), nsel,
                                _p(selp), _p(out), _p(lse), _p(err))
    if rc:
        raise ValueError(f"jto_tree_attention rc={rc}")
    return out, lse, err


def topw(logits, W: int, rows: int | None = None, V: int | None = None, row_stride=None,
         entropy: bool = False):
    """Per-row top-W ids (value desc, id asc), fp64 log-probs and row LSE (and, with
    ``entropy=True``, the row's softmax entropy as a fourth result).

    ``logits`` is a 2-D array [rows, row_stride]; ``V`` defaults to its width.
    """
    dt = _dtype_code(logits)
    logits = np.ascontiguousarray(logits)
    R, stride = logits.shape
    rows = R if rows is None else rows
    V = stride if V is None else V
    row_stride = stride if row_stride is None else row_stride
    ids = np.zeros((rows, W), np.int32)
    lp = np.zeros((rows, W), np.float64)
    lse = np.zeros(rows, np.float64)
    ent = np.zeros(rows, np.float64) if entropy else None
    lib = _load()
    lib.jto_topw.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_void_p]
    rc = lib.jto_topw(_p(logits), row_stride, rows, V, W, dt, _p(ids), _p(lp), _p(lse),
                      _p(ent))
    if rc:
        raise ValueError(f"jto_topw rc={rc}")
    return (ids, lp, lse, ent) if entropy else (ids, lp, lse)


def verify_greedy(target_logits, parent, tokens, N: int, V=None):
    """Greedy verification.  target_logits [S*B, stride] (or [S,B,stride]); parent,
    tokens [S,B]; the first ``V`` entries of each row are the vocabulary.

    Returns dict(accept_len [S], accept_path [S,N+1], bonus [S], argmax [S,B], err [S]).
    """
    parent = _c(parent, np.int32)
    tokens = _c(tokens, np.int32)
    S, B = parent.shape
    dt = _dtype_code(target_logits)
    tl = np.ascontiguousarray(target_logits).reshape(S * B, -1)
    row_stride = tl.shape[1]
    V = row_stride if V is None else V
    out = dict(accept_len=np.zeros(S, np.int32), accept_path=np.zeros((S, N + 1), np.int32),
               bonus=np.zeros(S, np.int32), argmax=np.zeros((S, B), np.int32),
               err=np.zeros(S, np.int32))
    lib = _load()
    lib.jto_verify_greedy.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int] + \
        [ctypes.c_void_p] * 5
    rc = lib.jto_verify_greedy(_p(tl), row_stride, V, dt, _p(parent), _p(tokens), S, B, N,
                               _p(out["accept_len"]), _p(out["accept_path"]),
                               _p(out["bonus"]), _p(out["argmax"]), _p(out["err"]))
    if rc:
        raise ValueError(f"jto_verify_greedy rc={rc}")
    return out


def build_tree(ids, logprob, N: int, B: int, *, entropy=None, w_lp: float = 1.0,
               w_ent: float = 0.0, root_token=None):
    """Best-first tree construction from per-depth candidate lists.

    ``ids`` int32 and ``logprob`` float32, [S*N, W] (row s*N + d: the candidates for
    depth d + 1 of sequence s); ``entropy`` float32 [S*N] or None.  Scores are float32.
    Returns dict(parent [S,B], tokens [S,B], score [S,B] float32, n_nodes [S]).
    """
    ids = _c(ids, np.int32)
    logprob = _c(logprob, np.float32)
    rows, W = ids.shape
    if logprob.shape != ids.shape:
        raise ValueError("ids and logprob differ in shape")
    if N < 1 and rows:
        raise ValueError("rows given but N < 1")
    S = rows // N if N >= 1 else 0
    if S * N != rows:
        raise ValueError("rows is not a multiple of N")
    ent = None if entropy is None else _c(entropy, np.float32).reshape(-1)
    root = None if root_token is None else _c(root_token, np.int32).reshape(-1)
    out = dict(parent=np.zeros((S, B), np.int32), tokens=np.zeros((S, B), np.int32),
               score=np.zeros((S, B), np.float32), n_nodes=np.zeros(S, np.int32))
    lib = _load()
    lib.jto_build_tree.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int] + \
        [ctypes.c_void_p] * 4
    rc = lib.jto_build_tree(_p(ids), _p(logprob), _p(ent), w_lp, w_ent, _p(root), S, N, W, B,
                            _p(out["parent"]), _p(out["tokens"]), _p(out["score"]),
                            _p(out["n_nodes"]))
    if rc:
        raise ValueError(f"jto_build_tree rc={rc}")
    return out


def commit_kv(accept_len, accept_path, N: int, k_tree, v_tree, k_cache, v_cache, prefix_len, *,
              block_table=None, block_size: int = 16):
    """Write the accepted root path's K/V rows into copies of the prefix caches.

    ``k_tree``/``v_tree`` [S,B,Hkv,d]; caches contiguous [S,Pmax,Hkv,d] or, with
    ``block_table`` [S,max_blocks], paged [num_blocks,block_size,Hkv,d]; float32 or bf16
    words (uint16).  Returns (k_cache, v_cache, new_prefix_len [S], err [S]).
    """
    k_tree = np.ascontiguousarray(k_tree)
    v_tree = np.ascontiguousarray(v_tree)
    if k_tree.dtype not in (np.float32, np.uint16) or v_tree.dtype != k_tree.dtype:
        raise TypeError("K/V must be float32 or bf16 words")
    kc = np.array(k_cache, dtype=k_tree.dtype, copy=True, order="C")
    vc = np.array(v_cache, dtype=k_tree.dtype, copy=True, order="C")
    S, B, Hkv, d = k_tree.shape
    al = _c(accept_len, np.int32)
    ap = _c(accept_path, np.int32)
    pl = _c(prefix_len, np.int32)
    bt = None if block_table is None else _c(block_table, np.int32)
    if bt is None:
        max_prefix, max_blocks, nblk = kc.shape[1], 0, 0
    else:
        max_prefix, max_blocks, nblk = 0, bt.shape[1], kc.shape[0]
    newp = np.zeros(S, np.int32)
    err = np.zeros(S, np.int32)
    lib = _load()
    lib.jto_commit_kv.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_int] + \
        [ctypes.c_void_p] * 2
    rc = lib.jto_commit_kv(_p(al), _p(ap), N, _p(k_tree), _p(v_tree), S, B, Hkv, d,
                           k_tree.dtype.itemsize, _p(kc), _p(vc), _p(bt), max_blocks, block_size,
                           nblk, _p(pl), max_prefix, _p(newp), _p(err))
    if rc:
        raise ValueError(f"jto_commit_kv rc={rc}")
    return kc, vc, newp, err


def verify_sampled(target_logits, parent, tokens, N: int, temperature: float, uniform, V=None):
    """Stochastic verification with one inverse-CDF draw per node from softmax(logits / T).

    ``uniform`` [S,B] in [0, 1) (float32 values, widened exactly).  Returns the dict of
    verify_greedy with "sample" [S,B] in place of "argmax", plus "margin" [S,B] (each
    draw's distance from its interval's nearer end, as a fraction of the row's weight).
    """
    parent = _c(parent, np.int32)
    tokens = _c(tokens, np.int32)
    S, B = parent.shape
    dt = _dtype_code(target_logits)
    tl = np.ascontiguousarray(target_logits).reshape(S * B, -1)
    row_stride = tl.shape[1]
    V = row_stride if V is None else V
    u = np.ascontiguousarray(np.asarray(uniform, np.float32).astype(np.float64).reshape(S, B))
    out = dict(accept_len=np.zeros(S, np.int32), accept_path=np.zeros((S, N + 1), np.int32),
               bonus=np.zeros(S, np.int32), sample=np.zeros((S, B), np.int32),
               margin=np.zeros((S, B), np.float64), err=np.zeros(S, np.int32))
    lib = _load()
    lib.jto_verify_sampled.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 6
    rc = lib.jto_verify_sampled(_p(tl), row_stride, V, dt, float(temperature), _p(u), _p(parent),
                                _p(tokens), S, B, N, _p(out["accept_len"]),
                                _p(out["accept_path"]), _p(out["bonus"]), _p(out["sample"]),
                                _p(out["margin"]), _p(out["err"]))
    if rc:
        raise ValueError(f"jto_verify_sampled rc={rc}")
    return out
