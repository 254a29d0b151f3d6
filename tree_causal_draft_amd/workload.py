"""Seeded synthetic inputs for one draft-and-verify step over a token tree.

This module is shared by the tests and the benchmark and holds none of the
step's arithmetic: it draws random tensors, lays out trees, prefix caches and
block tables, and plants known maxima.  It never builds a mask, never sorts a
vocabulary row, never takes an argmax and never computes a softmax.

Workloads (sizes follow the JetSpec pages' draft-head shape: 32 query / 8 KV
heads, head dim 128, Qwen3 vocabulary 151,936; budgets 16 to 256):

  tiny         1 seq, prefix 64, B=16 random tree (depth <= 4, <= 2 children),
               4/2 heads, d=64, fp32 q/k/v ~ N(0,1), vocab 1024, logits N(0,2),
               W=2, ~60% of edges accept
  low_budget   1 seq, prefix 1024, B=16 best-first-shaped tree (N=16, W=4),
               32/8 heads, d=128, bf16 q/k/v ~ N(0,1)/sqrt(128), logits N(0,3),
               spine acceptance 0.8
  high_budget  as low_budget with prefix 2048, B=256 (N=16, W=8), alpha 0.85
  ragged       8 seqs, prefix ~ U{512..8192}, B=128 random trees (N=12, W=6),
               paged 16-token KV blocks with a shuffled block table, per-sequence
               alpha ~ U[0.5, 0.9]
  moe_verify   32 seqs, prefix 4096, B=64 best-first-shaped (N=8, W=8), 32/4
               heads, alpha 0.7

Trees
  random       node i picks its parent uniformly among earlier nodes that are
               shallower than N and have fewer than W children.
  best_first   priority expansion in which a child of sibling rank r costs r
               (key = sum of ranks on the path; ties by depth, then node index);
               each popped node shallower than N gets children of rank 0..W-1
               while the budget lasts.  With one dominant draft token per depth
               this is the shape best-first expansion by cumulative log-prob
               produces: one deep rank-0 spine, then a bushy second layer.
  Node tokens: every sequence draws, per depth, W distinct candidate tokens; a
  child of sibling rank r at depth k carries candidate r of depth k, so
  siblings never share a token.  Candidate 0 of depth k is also the planted
  maximum of draft-logit row k-1.

Planting (known answers, no arithmetic on the logits)
  Logit bodies are N(0, sigma) clamped to +-10 sigma; a planted entry is set
  to 12 sigma, so it is the unique row maximum.  Target row v plants the token
  the target "would emit" after node v:
    spine  (best_first): on the rank-0 spine, with probability alpha the spine
           child's token, otherwise a token that no child of v carries; every
           other node plants a non-child token.
    edge   (random): each internal node, with probability alpha, plants one
           uniformly chosen child's token, otherwise a non-child token; leaves
           plant a uniform token.
  ``plant=False`` keeps the raw bodies (frequent bf16 ties) for tie tests.

Prefix caches are poisoned past each sequence's length (value 1e4), so a key
read outside the prefix shows up in any output.

bfloat16 tensors are numpy ``uint16`` arrays of raw bf16 words (round to
nearest even from float32); fp32 tensors are ``float32``.
"""
from __future__ import annotations

import dataclasses
import heapq
import math
import zlib
from dataclasses import dataclass, field

import numpy as np

POISON = 1.0e4


@dataclass(frozen=True)
class Config:
    name: str
    S: int
    prefix: object          # int, or (lo, hi) inclusive uniform integer range
    B: int
    N: int
    W: int
    tree: str               # "random" | "best_first"
    Hq: int
    Hkv: int
    d: int
    dtype: str              # "f32" | "bf16"
    qkv_std: float
    V: int
    logit_std: float
    alpha: object           # float, or (lo, hi) uniform per sequence
    accept: str             # "spine" | "edge"
    paged: bool = False
    block_size: int = 16


CONFIGS = {
    "tiny": Config("tiny", 1, 64, 16, 4, 2, "random", 4, 2, 64, "f32", 1.0, 1024, 2.0,
                   0.6, "edge"),
    "low_budget": Config("low_budget", 1, 1024, 16, 16, 4, "best_first", 32, 8, 128, "bf16",
                         1.0 / math.sqrt(128), 151936, 3.0, 0.8, "spine"),
    "high_budget": Config("high_budget", 1, 2048, 256, 16, 8, "best_first", 32, 8, 128, "bf16",
                          1.0 / math.sqrt(128), 151936, 3.0, 0.85, "spine"),
    "ragged": Config("ragged", 8, (512, 8192), 128, 12, 6, "random", 32, 8, 128, "bf16",
                     1.0 / math.sqrt(128), 151936, 3.0, (0.5, 0.9), "edge", paged=True),
    "moe_verify": Config("moe_verify", 32, 4096, 64, 8, 8, "best_first", 32, 4, 128, "bf16",
                         1.0 / math.sqrt(128), 151936, 3.0, 0.7, "spine"),
}
CONFIG_ORDER = ["tiny", "low_budget", "high_budget", "ragged", "moe_verify"]

_STREAMS = ("tree", "cand", "plant", "alpha", "prefix", "q", "ktree", "vtree", "kpre",
            "vpre", "blocks", "draft", "target", "root")


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), zlib.crc32(stream.encode())]))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns raw uint16 words."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of raw bf16 words to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(x32, np.float32) if dtype == "f32" else f32_to_bf16_bits(x32)


def as_float32(a: np.ndarray) -> np.ndarray:
    """Values of a workload tensor as float32 (exact for both dtypes)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def scalar_in_dtype(value: float, dtype: str):
    arr = to_dtype(np.array([value], np.float32), dtype)
    return arr[0]


# --------------------------------------------------------------- trees ---

def random_tree(B: int, N: int, W: int, rng: np.random.Generator):
    """Parents, depths and sibling ranks of a random tree (see module doc)."""
    parent = [-1]
    depth = [0]
    rank = [0]
    nchild = [0]
    for i in range(1, B):
        elig = [j for j in range(i) if depth[j] < N and nchild[j] < W]
        if not elig:
            raise ValueError(f"no room for node {i} with N={N}, W={W}")
        j = elig[int(rng.integers(len(elig)))]
        parent.append(j)
        depth.append(depth[j] + 1)
        rank.append(nchild[j])
        nchild[j] += 1
        nchild.append(0)
    return np.array(parent, np.int32), np.array(depth, np.int32), np.array(rank, np.int32)


def best_first_tree(B: int, N: int, W: int):
    """Parents, depths and sibling ranks of the best-first-shaped tree."""
    parent = [-1]
    depth = [0]
    rank = [0]
    heap = [(0, 0, 0)]  # (rank cost, depth, node)
    while heap and len(parent) < B:
        key, dep, v = heapq.heappop(heap)
        if dep >= N:
            continue
        for r in range(W):
            if len(parent) >= B:
                break
            u = len(parent)
            parent.append(v)
            depth.append(dep + 1)
            rank.append(r)
            heapq.heappush(heap, (key + r, dep + 1, u))
    return np.array(parent, np.int32), np.array(depth, np.int32), np.array(rank, np.int32)


def chain_tree(B: int):
    return (np.arange(-1, B - 1, dtype=np.int32), np.arange(B, dtype=np.int32),
            np.zeros(B, np.int32))


def star_tree(B: int):
    par = np.zeros(B, np.int32)
    par[0] = -1
    dep = np.ones(B, np.int32)
    dep[0] = 0
    rank = np.maximum(np.arange(B, dtype=np.int32) - 1, 0)
    return par, dep, rank


def children_lists(parent: np.ndarray):
    ch = [[] for _ in range(len(parent))]
    for u in range(1, len(parent)):
        ch[int(parent[u])].append(u)
    return ch


def spine_of(parent: np.ndarray, rank: np.ndarray):
    """Root-to-leaf path that always follows the rank-0 child."""
    ch = children_lists(parent)
    path = [0]
    while True:
        nxt = [u for u in ch[path[-1]] if rank[u] == 0]
        if not nxt:
            return path
        path.append(nxt[0])


# ------------------------------------------------------------ workload ---

@dataclass
class Workload:
    cfg: Config
    seed: int
    parent: np.ndarray          # int32 [S,B]
    depth: np.ndarray           # int32 [S,B] (layout facts of the synthetic tree)
    rank: np.ndarray            # int32 [S,B]
    tokens: np.ndarray          # int32 [S,B]
    planted_next: np.ndarray    # int32 [S,B]  token planted as target row maximum
    alpha: np.ndarray           # float64 [S]
    prefix_len: np.ndarray      # int32 [S]
    max_prefix: int
    q: np.ndarray = None        # [S,B,Hq,d]
    k_tree: np.ndarray = None   # [S,B,Hkv,d]
    v_tree: np.ndarray = None
    k_prefix: np.ndarray = None  # contiguous [S,Pmax,Hkv,d] or pool [nblk,bs,Hkv,d]
    v_prefix: np.ndarray = None
    block_table: np.ndarray = None  # int32 [S,maxblk] (paged only, -1 = unused)
    num_blocks: int = 0
    draft_logits: np.ndarray = None   # [S*N, V]
    target_logits: np.ndarray = None  # [S*B, V]
    extra: dict = field(default_factory=dict)

    @property
    def S(self):
        return self.cfg.S

    @property
    def B(self):
        return self.cfg.B


def _draw_normal(rng, shape, std, dtype, chunk_rows=None):
    """N(0, std) in float32, converted to the dtype; generated in row chunks."""
    shape = tuple(shape)
    n_rows = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty(shape, np.float32 if dtype == "f32" else np.uint16)
    flat = out.reshape(n_rows, inner)
    step = max(1, (1 << 24) // max(inner, 1)) if chunk_rows is None else chunk_rows
    for r0 in range(0, n_rows, step):
        r1 = min(n_rows, r0 + step)
        x = rng.standard_normal((r1 - r0, inner), dtype=np.float32)
        x *= np.float32(std)
        flat[r0:r1] = to_dtype(x, dtype)
    return out


def _draw_logits(rng, rows, V, std, dtype, planted=None):
    """Logit rows N(0, std) clamped to +-10 std; row r gets 12 std at planted[r]."""
    out = np.empty((rows, V), np.float32 if dtype == "f32" else np.uint16)
    step = max(1, (1 << 24) // V)
    lim = np.float32(10.0 * std)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = rng.standard_normal((r1 - r0, V), dtype=np.float32)
        x *= np.float32(std)
        np.clip(x, -lim, lim, out=x)
        out[r0:r1] = to_dtype(x, dtype)
    if planted is not None:
        hot = scalar_in_dtype(12.0 * std, dtype)
        out[np.arange(rows), np.asarray(planted, np.int64)] = hot
    return out


def _non_child_token(rng, V, forbidden):
    while True:
        t = int(rng.integers(V))
        if t not in forbidden:
            return t


def make(cfg, seed: int, *, parts=("tree", "attn", "draft", "target"), plant: bool = True,
         qk_std: float | None = None, trees=None, prefix_len=None, **overrides) -> Workload:
    """Build one seeded workload.

    ``cfg``: a Config or the name of one; ``overrides`` replace Config fields
    (e.g. ``V=4096`` or ``prefix=100``) for smaller parity cases.
    ``parts`` selects which tensors to draw ("tree" is always built).
    ``qk_std`` draws q and k with this standard deviation instead (sharper
    softmax).  ``trees``: optional list of S (parent, depth, rank) triples.
    ``prefix_len``: optional explicit per-sequence prefix lengths.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    if overrides:
        cfg = dataclasses.replace(cfg, **overrides)
    S, B, N, W, V = cfg.S, cfg.B, cfg.N, cfg.W, cfg.V

    # ---- trees and tokens
    rt = _rng(seed, "tree")
    rc = _rng(seed, "cand")
    rp = _rng(seed, "plant")
    ra = _rng(seed, "alpha")
    rr = _rng(seed, "root")
    parent = np.zeros((S, B), np.int32)
    depth = np.zeros((S, B), np.int32)
    rank = np.zeros((S, B), np.int32)
    tokens = np.zeros((S, B), np.int32)
    planted = np.zeros((S, B), np.int32)
    if isinstance(cfg.alpha, tuple):
        alpha = ra.uniform(cfg.alpha[0], cfg.alpha[1], size=S)
    else:
        alpha = np.full(S, float(cfg.alpha))
    n_cand = max(W, 1)
    cand = np.zeros((S, N + 1, n_cand), np.int32)
    for s in range(S):
        if trees is not None:
            par, dep, rk = (np.asarray(t, np.int32) for t in trees[s])
        elif cfg.tree == "random":
            par, dep, rk = random_tree(B, N, W, rt)
        else:
            par, dep, rk = best_first_tree(B, N, W)
        parent[s], depth[s], rank[s] = par, dep, rk
        for k in range(1, N + 1):
            cand[s, k] = rc.choice(V, size=n_cand, replace=False)
        tokens[s, 0] = int(rr.integers(V))
        for u in range(1, B):
            tokens[s, u] = cand[s, min(int(dep[u]), N), int(rk[u]) % n_cand]
        ch = children_lists(par)
        spine = set(spine_of(par, rk)) if cfg.accept == "spine" else set()
        spine_list = spine_of(par, rk) if cfg.accept == "spine" else []
        for v in range(B):
            kids = ch[v]
            ktoks = {int(tokens[s, u]) for u in kids}
            if cfg.accept == "spine":
                pos = spine_list.index(v) if v in spine else -1
                if 0 <= pos < len(spine_list) - 1 and rp.random() < alpha[s]:
                    planted[s, v] = tokens[s, spine_list[pos + 1]]
                else:
                    planted[s, v] = _non_child_token(rp, V, ktoks)
            else:
                if kids and rp.random() < alpha[s]:
                    planted[s, v] = tokens[s, kids[int(rp.integers(len(kids)))]]
                elif kids:
                    planted[s, v] = _non_child_token(rp, V, ktoks)
                else:
                    planted[s, v] = int(rp.integers(V))

    # ---- prefix lengths
    if prefix_len is not None:
        plen = np.asarray(prefix_len, np.int32).reshape(S)
    elif isinstance(cfg.prefix, tuple):
        plen = _rng(seed, "prefix").integers(cfg.prefix[0], cfg.prefix[1] + 1, size=S).astype(np.int32)
    else:
        plen = np.full(S, int(cfg.prefix), np.int32)
    Pmax = int(plen.max()) if S else 0
    if not isinstance(cfg.prefix, tuple) and prefix_len is None:
        Pmax = int(cfg.prefix)
    elif isinstance(cfg.prefix, tuple) and prefix_len is None:
        Pmax = int(cfg.prefix[1])

    w = Workload(cfg, seed, parent, depth, rank, tokens, planted, alpha, plen, Pmax)
    w.extra["candidates"] = cand

    dt = cfg.dtype
    qks = cfg.qkv_std if qk_std is None else qk_std
    if "attn" in parts:
        Hq, Hkv, d = cfg.Hq, cfg.Hkv, cfg.d
        w.q = _draw_normal(_rng(seed, "q"), (S, B, Hq, d), qks, dt)
        w.k_tree = _draw_normal(_rng(seed, "ktree"), (S, B, Hkv, d), qks, dt)
        w.v_tree = _draw_normal(_rng(seed, "vtree"), (S, B, Hkv, d), cfg.qkv_std, dt)
        poison = scalar_in_dtype(POISON, dt)
        rk_, rv_ = _rng(seed, "kpre"), _rng(seed, "vpre")
        if not cfg.paged:
            kp = _draw_normal(rk_, (S, Pmax, Hkv, d), qks, dt)
            vp = _draw_normal(rv_, (S, Pmax, Hkv, d), cfg.qkv_std, dt)
            for s in range(S):
                kp[s, plen[s]:] = poison
                vp[s, plen[s]:] = poison
            w.k_prefix, w.v_prefix = kp, vp
        else:
            bs = cfg.block_size
            maxblk = max(1, -(-Pmax // bs))
            nb = [-(-int(p) // bs) for p in plen]
            total = int(sum(nb))
            perm = _rng(seed, "blocks").permutation(total).astype(np.int32)
            bt = np.full((S, maxblk), -1, np.int32)
            off = 0
            for s in range(S):
                bt[s, :nb[s]] = perm[off:off + nb[s]]
                off += nb[s]
            kpool = np.empty((max(total, 1), bs, Hkv, d), np.float32 if dt == "f32" else np.uint16)
            vpool = np.empty_like(kpool)
            kpool[...] = poison
            vpool[...] = poison
            for s in range(S):
                ks = _draw_normal(rk_, (int(plen[s]), Hkv, d), qks, dt)
                vs = _draw_normal(rv_, (int(plen[s]), Hkv, d), cfg.qkv_std, dt)
                for lb in range(nb[s]):
                    j0, j1 = lb * bs, min(int(plen[s]), (lb + 1) * bs)
                    kpool[bt[s, lb], : j1 - j0] = ks[j0:j1]
                    vpool[bt[s, lb], : j1 - j0] = vs[j0:j1]
            w.k_prefix, w.v_prefix = kpool, vpool
            w.block_table = bt
            w.num_blocks = total
    if "draft" in parts:
        planted_draft = cand[:, 1:, 0].reshape(S * N) if plant else None
        w.draft_logits = _draw_logits(_rng(seed, "draft"), S * N, V, cfg.logit_std, dt,
                                      planted_draft)
    if "target" in parts:
        w.target_logits = _draw_logits(_rng(seed, "target"), S * B, V, cfg.logit_std, dt,
                                       planted.reshape(S * B) if plant else None)
    return w


def contiguous_prefix(w: Workload):
    """Paged pool -> contiguous [S, Pmax, Hkv, d] copy (poisoned past each length)."""
    if w.block_table is None:
        return w.k_prefix, w.v_prefix
    cfg = w.cfg
    bs = cfg.block_size
    poison = scalar_in_dtype(POISON, cfg.dtype)
    kp = np.full((cfg.S, w.max_prefix, cfg.Hkv, cfg.d), poison, w.k_prefix.dtype)
    vp = np.full_like(kp, poison)
    for s in range(cfg.S):
        for j0 in range(0, int(w.prefix_len[s]), bs):
            j1 = min(int(w.prefix_len[s]), j0 + bs)
            blk = w.block_table[s, j0 // bs]
            kp[s, j0:j1] = w.k_prefix[blk, : j1 - j0]
            vp[s, j0:j1] = w.v_prefix[blk, : j1 - j0]
    return kp, vp
