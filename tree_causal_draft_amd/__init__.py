"""Python binding of libjt (tree draft-and-verify step on MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libjt.so``.  torch provides device memory and the current stream.  There is no
CPU fallback: if the library is missing or fails to load, every call raises.

Entry points (same names as the C ABI in ``include/jt.h``):
    build_tree_mask, tree_attention, topw_per_depth, verify_greedy, and
    draft_verify_step (the four steps in two launches)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjt.so")

JT_F32, JT_BF16 = 0, 1
JT_ERR_SCRATCH = 7
STATIC_SCRATCH_BYTES = 48 << 20  # JT_STATIC_SCRATCH_BYTES
DEV_BAD_PARENT, DEV_DEPTH_GT_N, DEV_BAD_BLOCK, DEV_NAN, DEV_BAD_PREFIX = 1, 2, 4, 8, 16
EXPORTS = ("jt_abi_version", "jt_status_string", "jt_build_tree_mask",
           "jt_tree_attention_workspace_size", "jt_tree_attention", "jt_topw_workspace_size",
           "jt_topw_per_depth", "jt_verify_workspace_size", "jt_verify_greedy",
           "jt_step_workspace_size", "jt_draft_verify_step", "jt_build_tree_best_first",
           "jt_commit_accepted_kv", "jt_verify_sampled_workspace_size", "jt_verify_sampled",
           "jt_probe_mfma_rate", "jt_draft_verify_step_noalloc")

_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class JTError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Loads libjt.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise JTError(f"{LIB_PATH} is missing: build it with "
                          "`python -m tree_causal_draft_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        L.jt_abi_version.restype = ctypes.c_int
        L.jt_status_string.restype = ctypes.c_char_p
        L.jt_status_string.argtypes = [ctypes.c_int]
        L.jt_build_tree_mask.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp]
        L.jt_tree_attention_workspace_size.restype = _sz
        L.jt_tree_attention_workspace_size.argtypes = [_i32] * 7 + [ctypes.c_int]
        L.jt_tree_attention.argtypes = ([_vp] * 6 + [_i32, _i32, _i32, _vp, _i32, _vp] +
                                        [_i32] * 5 + [ctypes.c_int, ctypes.c_float, _vp, _vp, _vp,
                                                      _vp, _sz, _vp])
        L.jt_topw_workspace_size.restype = _sz
        L.jt_topw_workspace_size.argtypes = [_i32, _i32, _i32, ctypes.c_int]
        L.jt_topw_per_depth.argtypes = [_vp, _i64, _i32, _i32, _i32, ctypes.c_int, _vp, _vp, _vp,
                                        _vp, _vp, _sz, _vp]
        L.jt_verify_workspace_size.restype = _sz
        L.jt_verify_workspace_size.argtypes = [_i32, _i32, _i32, ctypes.c_int]
        L.jt_verify_greedy.argtypes = ([_vp, _i64, _i32, ctypes.c_int] + [_vp] * 4 +
                                       [_i32, _i32, _i32] + [_vp] * 6 + [_sz, _vp])
        L.jt_step_workspace_size.restype = _sz
        L.jt_step_workspace_size.argtypes = [_i32] * 10 + [ctypes.c_int]
        L.jt_draft_verify_step.argtypes = (
            [_vp, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _i32] + [_vp] * 6 +
            [_i32, _i32, _i32, _vp] + [_i32] * 4 + [ctypes.c_float, ctypes.c_int] + [_vp] * 14 +
            [_sz, _vp])
        L.jt_draft_verify_step_noalloc.argtypes = L.jt_draft_verify_step.argtypes[:-3] + [_vp]
        L.jt_build_tree_best_first.argtypes = ([_vp] * 3 + [ctypes.c_float] * 2 + [_vp] +
                                               [_i32] * 4 + [_vp] * 5)
        L.jt_commit_accepted_kv.argtypes = ([_vp, _vp, _i32, _vp, _vp] + [_i32] * 4 +
                                            [ctypes.c_int, _vp, _vp, _vp] + [_i32] * 3 +
                                            [_vp, _i32, _vp, _vp, _vp])
        L.jt_verify_sampled_workspace_size.restype = _sz
        L.jt_verify_sampled_workspace_size.argtypes = [_i32, _i32, _i32, ctypes.c_int]
        L.jt_verify_sampled.argtypes = ([_vp, _i64, _i32, ctypes.c_int, ctypes.c_float] +
                                        [_vp] * 5 + [_i32] * 3 + [_vp] * 6 + [_sz, _vp])
        L.jt_probe_mfma_rate.argtypes = [_i32, _i32, _vp, _vp]
        for fn in ("jt_build_tree_mask", "jt_tree_attention", "jt_topw_per_depth",
                   "jt_verify_greedy", "jt_draft_verify_step", "jt_build_tree_best_first",
                   "jt_commit_accepted_kv", "jt_verify_sampled", "jt_probe_mfma_rate",
                   "jt_draft_verify_step_noalloc"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return JT_BF16
    if t.dtype == torch.float32:
        return JT_F32
    raise JTError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def _check(rc: int, what: str):
    if rc != 0:
        raise JTError(f"{what}: {lib().jt_status_string(rc).decode()} (status {rc})")


def _need(t, name):
    if not t.is_cuda:
        raise JTError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise JTError(f"{name} must be contiguous")
    return t


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def build_tree_mask(parent, anc=None, depth=None, err=None, stream=None):
    """parent int32 [S,B] -> (anc uint64-as-int64 [S,B,4], depth int32 [S,B], err int32 [S])."""
    _need(parent, "parent")
    S, B = parent.shape
    dev = parent.device
    anc = torch.empty((S, B, 4), dtype=torch.int64, device=dev) if anc is None else anc
    depth = torch.empty((S, B), dtype=torch.int32, device=dev) if depth is None else depth
    err = torch.empty(S, dtype=torch.int32, device=dev) if err is None else err
    _check(lib().jt_build_tree_mask(_ptr(parent), S, B, _ptr(anc), _ptr(depth), _ptr(err),
                                    _stream(stream)), "jt_build_tree_mask")
    return anc, depth, err


def tree_attention_workspace_size(S, B, Hq, Hkv, d, max_prefix, dtype, block_size=0) -> int:
    """block_size: paged pool block size, 0 for a contiguous prefix."""
    return int(lib().jt_tree_attention_workspace_size(S, B, Hq, Hkv, d, max_prefix, block_size,
                                                      dtype))


def tree_attention(q, k_tree, v_tree, k_prefix, v_prefix, prefix_len, anc, *, block_table=None,
                   block_size=16, num_blocks=None, max_prefix=None, scale=0.0, out=None,
                   lse=None, err=None, workspace=None, want_lse=True, stream=None):
    """Tree-causal GQA attention; returns (out, lse or None, err)."""
    for t, n in ((q, "q"), (k_tree, "k_tree"), (v_tree, "v_tree"), (k_prefix, "k_prefix"),
                 (v_prefix, "v_prefix"), (prefix_len, "prefix_len"), (anc, "anc")):
        _need(t, n)
    S, B, Hq, d = q.shape
    Hkv = k_tree.shape[2]
    dt = _dt(q)
    if block_table is None:
        Pmax = k_prefix.shape[1] if max_prefix is None else max_prefix
        maxblk, nblk = 0, 0
    else:
        _need(block_table, "block_table")
        maxblk = block_table.shape[1]
        Pmax = maxblk * block_size if max_prefix is None else max_prefix
        nblk = k_prefix.shape[0] if num_blocks is None else num_blocks
    dev = q.device
    out = torch.empty_like(q) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty((S, B, Hq), dtype=torch.float32, device=dev)
    err = torch.empty(S, dtype=torch.int32, device=dev) if err is None else err
    need = tree_attention_workspace_size(S, B, Hq, Hkv, d, Pmax, dt,
                                         0 if block_table is None else block_size)
    ws, wsb = _workspace(need, dev, workspace)
    _check(lib().jt_tree_attention(_ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_prefix),
                                   _ptr(v_prefix), _ptr(block_table), maxblk, block_size, nblk,
                                   _ptr(prefix_len), Pmax, _ptr(anc), S, B, Hq, Hkv, d, dt,
                                   float(scale), _ptr(out), _ptr(lse), _ptr(err), _ptr(ws), wsb,
                                   _stream(stream)), "jt_tree_attention")
    return out, lse, err


def topw_workspace_size(rows, V, W, dtype) -> int:
    return int(lib().jt_topw_workspace_size(rows, V, W, dtype))


def topw_per_depth(logits, W, *, V=None, ids=None, logprob=None, row_lse=None, workspace=None,
                   want_lse=True, row_entropy=None, stream=None):
    """logits [rows, row_stride] -> (ids int32 [rows,W], logprob fp32 [rows,W], row_lse).

    ``row_entropy``: an fp32 [rows] tensor to receive each row's softmax entropy, or None.
    """
    _need(logits, "logits")
    rows, stride = logits.shape
    V = stride if V is None else V
    dt = _dt(logits)
    dev = logits.device
    ids = torch.empty((rows, W), dtype=torch.int32, device=dev) if ids is None else ids
    logprob = torch.empty((rows, W), dtype=torch.float32, device=dev) if logprob is None else logprob
    if row_lse is None and want_lse:
        row_lse = torch.empty(rows, dtype=torch.float32, device=dev)
    ws, wsb = _workspace(topw_workspace_size(rows, V, W, dt), dev, workspace)
    _check(lib().jt_topw_per_depth(_ptr(logits), stride, rows, V, W, dt, _ptr(ids), _ptr(logprob),
                                   _ptr(row_lse), _ptr(row_entropy), _ptr(ws), wsb,
                                   _stream(stream)),
           "jt_topw_per_depth")
    return ids, logprob, row_lse


def verify_workspace_size(S, B, V, dtype) -> int:
    return int(lib().jt_verify_workspace_size(S, B, V, dtype))


def verify_greedy(target_logits, parent, tokens, anc, depth, N, *, V=None, accept_len=None,
                  accept_path=None, bonus=None, argmax_out=None, err=None, workspace=None,
                  want_argmax=True, stream=None):
    """target_logits [S*B, row_stride]; returns dict of accept_len, accept_path, bonus,
    argmax (or None) and err."""
    for t, n in ((target_logits, "target_logits"), (parent, "parent"), (tokens, "tokens"),
                 (anc, "anc"), (depth, "depth")):
        _need(t, n)
    S, B = parent.shape
    tl = target_logits
    stride = tl.shape[-1]
    V = stride if V is None else V
    dt = _dt(tl)
    dev = tl.device
    accept_len = torch.empty(S, dtype=torch.int32, device=dev) if accept_len is None else accept_len
    accept_path = (torch.empty((S, N + 1), dtype=torch.int32, device=dev)
                   if accept_path is None else accept_path)
    bonus = torch.empty(S, dtype=torch.int32, device=dev) if bonus is None else bonus
    if argmax_out is None and want_argmax:
        argmax_out = torch.empty((S, B), dtype=torch.int32, device=dev)
    err = torch.empty(S, dtype=torch.int32, device=dev) if err is None else err
    ws, wsb = _workspace(verify_workspace_size(S, B, V, dt), dev, workspace)
    _check(lib().jt_verify_greedy(_ptr(tl), stride, V, dt, _ptr(parent), _ptr(tokens), _ptr(anc),
                                  _ptr(depth), S, B, N, _ptr(accept_len), _ptr(accept_path),
                                  _ptr(bonus), _ptr(argmax_out), _ptr(err), _ptr(ws), wsb,
                                  _stream(stream)), "jt_verify_greedy")
    return dict(accept_len=accept_len, accept_path=accept_path, bonus=bonus, argmax=argmax_out,
                err=err)


def step_workspace_size(S, B, N, W, V, Hq, Hkv, d, max_prefix, dtype, block_size=0) -> int:
    """block_size: paged pool block size, 0 for a contiguous prefix."""
    return int(lib().jt_step_workspace_size(S, B, N, W, V, Hq, Hkv, d, max_prefix, block_size,
                                            dtype))


def _step_call(draft_logits, target_logits, parent, tokens, N, W, q, k_tree, v_tree,
               k_prefix, v_prefix, prefix_len, V, block_table, block_size, num_blocks,
               max_prefix, scale, out, lse, ids, logprob, row_lse, anc, depth, accept_len,
               accept_path, bonus, argmax_out, err, row_entropy):
    """Argument checks and output allocation shared by the two forms of the fused step;
    returns (C arguments up to err, outputs, workspace size)."""
    for t, n in ((draft_logits, "draft_logits"), (target_logits, "target_logits"),
                 (parent, "parent"), (tokens, "tokens"), (q, "q"), (k_tree, "k_tree"),
                 (v_tree, "v_tree"), (k_prefix, "k_prefix"), (v_prefix, "v_prefix"),
                 (prefix_len, "prefix_len")):
        _need(t, n)
    S, B = parent.shape
    _, _, Hq, d = q.shape
    Hkv = k_tree.shape[2]
    dt = _dt(q)
    dstride, tstride = draft_logits.shape[-1], target_logits.shape[-1]
    V = tstride if V is None else V
    if block_table is None:
        Pmax = k_prefix.shape[1] if max_prefix is None else max_prefix
        maxblk, nblk = 0, 0
    else:
        _need(block_table, "block_table")
        maxblk = block_table.shape[1]
        Pmax = maxblk * block_size if max_prefix is None else max_prefix
        nblk = k_prefix.shape[0] if num_blocks is None else num_blocks
    dev = q.device
    e = lambda shape, dtype: torch.empty(shape, dtype=dtype, device=dev)
    out = torch.empty_like(q) if out is None else out
    lse = e((S, B, Hq), torch.float32) if lse is None else lse
    ids = e((S * N, W), torch.int32) if ids is None else ids
    logprob = e((S * N, W), torch.float32) if logprob is None else logprob
    row_lse = e(S * N, torch.float32) if row_lse is None else row_lse
    anc = e((S, B, 4), torch.int64) if anc is None else anc
    depth = e((S, B), torch.int32) if depth is None else depth
    accept_len = e(S, torch.int32) if accept_len is None else accept_len
    accept_path = e((S, N + 1), torch.int32) if accept_path is None else accept_path
    bonus = e(S, torch.int32) if bonus is None else bonus
    argmax_out = e((S, B), torch.int32) if argmax_out is None else argmax_out
    err = e(S, torch.int32) if err is None else err
    need = step_workspace_size(S, B, N, W, V, Hq, Hkv, d, Pmax, dt,
                               0 if block_table is None else block_size)
    args = (_ptr(draft_logits), dstride, _ptr(target_logits), tstride, V, W, _ptr(parent),
            _ptr(tokens), S, B, N, _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_prefix),
            _ptr(v_prefix), _ptr(block_table), maxblk, block_size, nblk, _ptr(prefix_len), Pmax,
            Hq, Hkv, d, float(scale), dt, _ptr(ids), _ptr(logprob), _ptr(row_lse),
            _ptr(row_entropy), _ptr(anc), _ptr(depth), _ptr(out), _ptr(lse), _ptr(accept_len),
            _ptr(accept_path), _ptr(bonus), _ptr(argmax_out), _ptr(err))
    outs = dict(ids=ids, logprob=logprob, row_lse=row_lse, row_entropy=row_entropy, anc=anc,
                depth=depth, out=out, lse=lse, accept_len=accept_len, accept_path=accept_path,
                bonus=bonus, argmax=argmax_out, err=err)
    return args, outs, need


def draft_verify_step(draft_logits, target_logits, parent, tokens, N, W, q, k_tree, v_tree,
                      k_prefix, v_prefix, prefix_len, *, V=None, block_table=None, block_size=16,
                      num_blocks=None, max_prefix=None, scale=0.0, out=None, lse=None, ids=None,
                      logprob=None, row_lse=None, anc=None, depth=None, accept_len=None,
                      accept_path=None, bonus=None, argmax_out=None, err=None, workspace=None,
                      row_entropy=None, stream=None):
    """The four steps in one call (two or three launches).  draft_logits [S*N, stride] and
    target_logits [S*B, stride] bf16; the rest as for the separate calls.  Returns a dict
    of every output."""
    args, outs, need = _step_call(draft_logits, target_logits, parent, tokens, N, W, q, k_tree,
                                  v_tree, k_prefix, v_prefix, prefix_len, V, block_table,
                                  block_size, num_blocks, max_prefix, scale, out, lse, ids,
                                  logprob, row_lse, anc, depth, accept_len, accept_path, bonus,
                                  argmax_out, err, row_entropy)
    ws, wsb = _workspace(need, q.device, workspace)
    _check(lib().jt_draft_verify_step(*args, _ptr(ws), wsb, _stream(stream)),
           "jt_draft_verify_step")
    return outs


def draft_verify_step_noalloc(draft_logits, target_logits, parent, tokens, N, W, q, k_tree,
                              v_tree, k_prefix, v_prefix, prefix_len, *, V=None,
                              block_table=None, block_size=16, num_blocks=None, max_prefix=None,
                              scale=0.0, out=None, lse=None, ids=None, logprob=None,
                              row_lse=None, anc=None, depth=None, accept_len=None,
                              accept_path=None, bonus=None, argmax_out=None, err=None,
                              row_entropy=None, stream=None):
    """jt_draft_verify_step_noalloc: the fused step with the library's static device scratch
    (no workspace).  Pass every output to keep the call free of allocations."""
    args, outs, _ = _step_call(draft_logits, target_logits, parent, tokens, N, W, q, k_tree,
                               v_tree, k_prefix, v_prefix, prefix_len, V, block_table,
                               block_size, num_blocks, max_prefix, scale, out, lse, ids, logprob,
                               row_lse, anc, depth, accept_len, accept_path, bonus, argmax_out,
                               err, row_entropy)
    _check(lib().jt_draft_verify_step_noalloc(*args, _stream(stream)),
           "jt_draft_verify_step_noalloc")
    return outs


def build_tree_best_first(ids, logprob, N, B, *, entropy=None, w_lp=1.0, w_ent=0.0,
                          root_token=None, parent=None, tokens=None, score=None, n_nodes=None,
                          stream=None):
    """Best-first draft tree from the per-depth top-W lists.

    ids int32 / logprob float32 [S*N, W] (as jt_topw_per_depth returns them), entropy
    float32 [S*N] or None, root_token int32 [S] or None.  Returns (parent, tokens, score,
    n_nodes): int32 [S,B], int32 [S,B], float32 [S,B], int32 [S].
    """
    _need(ids, "ids")
    _need(logprob, "logprob")
    if ids.dtype != torch.int32 or logprob.dtype != torch.float32:
        raise JTError("ids must be int32 and logprob float32")
    rows, W = ids.shape
    if tuple(logprob.shape) != (rows, W) or N < 1 or rows % N:
        raise JTError("ids / logprob must be [S*N, W] with N >= 1")
    S = rows // N
    dev = ids.device
    for t, n in ((entropy, "entropy"), (root_token, "root_token")):
        if t is not None:
            _need(t, n)
    parent = torch.empty((S, B), dtype=torch.int32, device=dev) if parent is None else parent
    tokens = torch.empty((S, B), dtype=torch.int32, device=dev) if tokens is None else tokens
    score = torch.empty((S, B), dtype=torch.float32, device=dev) if score is None else score
    n_nodes = torch.empty(S, dtype=torch.int32, device=dev) if n_nodes is None else n_nodes
    _check(lib().jt_build_tree_best_first(_ptr(ids), _ptr(logprob), _ptr(entropy), float(w_lp),
                                          float(w_ent), _ptr(root_token), S, N, W, B,
                                          _ptr(parent), _ptr(tokens), _ptr(score),
                                          _ptr(n_nodes), _stream(stream)),
           "jt_build_tree_best_first")
    return parent, tokens, score, n_nodes


def commit_accepted_kv(accept_len, accept_path, k_tree, v_tree, k_cache, v_cache, prefix_len,
                       *, block_table=None, block_size=16, num_blocks=None, new_prefix_len=None,
                       err=None, stream=None):
    """Write the accepted root path's K/V rows into the prefix cache (in place).

    accept_len [S], accept_path [S,N+1] int32; k_tree/v_tree [S,B,Hkv,d]; caches
    contiguous [S,Pmax,Hkv,d], or paged [num_blocks,block_size,Hkv,d] with block_table
    [S,max_blocks].  new_prefix_len may be prefix_len itself.  Returns (new_prefix_len, err).
    """
    for t, n in ((accept_len, "accept_len"), (accept_path, "accept_path"), (k_tree, "k_tree"),
                 (v_tree, "v_tree"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (prefix_len, "prefix_len")):
        _need(t, n)
    S, B, Hkv, d = k_tree.shape
    N = accept_path.shape[1] - 1
    dt = _dt(k_tree)
    if block_table is None:
        maxblk, nblk, Pmax = 0, 0, k_cache.shape[1]
    else:
        _need(block_table, "block_table")
        maxblk, Pmax = block_table.shape[1], 0
        nblk = k_cache.shape[0] if num_blocks is None else num_blocks
    dev = k_tree.device
    new_prefix_len = (torch.empty(S, dtype=torch.int32, device=dev) if new_prefix_len is None
                      else new_prefix_len)
    err = torch.empty(S, dtype=torch.int32, device=dev) if err is None else err
    _check(lib().jt_commit_accepted_kv(_ptr(accept_len), _ptr(accept_path), N, _ptr(k_tree),
                                       _ptr(v_tree), S, B, Hkv, d, dt, _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_table), maxblk, block_size,
                                       nblk, _ptr(prefix_len), Pmax, _ptr(new_prefix_len),
                                       _ptr(err), _stream(stream)),
           "jt_commit_accepted_kv")
    return new_prefix_len, err


def verify_sampled_workspace_size(S, B, V, dtype) -> int:
    return int(lib().jt_verify_sampled_workspace_size(S, B, V, dtype))


def verify_sampled(target_logits, parent, tokens, anc, depth, N, temperature, uniform, *, V=None,
                   accept_len=None, accept_path=None, bonus=None, sample_out=None, err=None,
                   workspace=None, stream=None):
    """Stochastic verification: one draw per node from softmax(logits / T) at the given
    uniforms [S,B], then the greedy walk.  Returns (accept_len, accept_path, bonus,
    sample [S,B], err)."""
    for t, n in ((target_logits, "target_logits"), (parent, "parent"), (tokens, "tokens"),
                 (anc, "anc"), (depth, "depth"), (uniform, "uniform")):
        _need(t, n)
    if uniform.dtype != torch.float32:
        raise JTError("uniform must be float32")
    S, B = parent.shape
    stride = target_logits.shape[-1]
    V = stride if V is None else V
    dt = _dt(target_logits)
    dev = target_logits.device
    e = lambda shape: torch.empty(shape, dtype=torch.int32, device=dev)
    accept_len = e(S) if accept_len is None else accept_len
    accept_path = e((S, N + 1)) if accept_path is None else accept_path
    bonus = e(S) if bonus is None else bonus
    sample_out = e((S, B)) if sample_out is None else sample_out
    err = e(S) if err is None else err
    ws, wsb = _workspace(verify_sampled_workspace_size(S, B, V, dt), dev, workspace)
    _check(lib().jt_verify_sampled(_ptr(target_logits), stride, V, dt, float(temperature),
                                   _ptr(uniform), _ptr(parent), _ptr(tokens), _ptr(anc),
                                   _ptr(depth), S, B, N, _ptr(accept_len), _ptr(accept_path),
                                   _ptr(bonus), _ptr(sample_out), _ptr(err), _ptr(ws), wsb,
                                   _stream(stream)), "jt_verify_sampled")
    return accept_len, accept_path, bonus, sample_out, err



def probe_mfma_rate(iters, blocks, out=None, stream=None):
    """Launch the matrix-core rate probe (blocks * 4 * iters * 8 * 32768 bf16 flops) on the
    stream; returns the output buffer.  Time it with events on that stream."""
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    _need(out, "out")
    _check(lib().jt_probe_mfma_rate(int(iters), int(blocks), _ptr(out), _stream(stream)),
           "jt_probe_mfma_rate")
    return out
