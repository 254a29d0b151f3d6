"""CPU model of the attention pass's balanced schedule (index arithmetic only, no GPU).

With several sequences and 8-wave workgroups the pass does not cut each sequence's keys
into fixed chunks: the units' key tiles -- unit = (sequence, KV head, 256-row tile), in
that order, each unit holding the tiles its rows can see -- form one run of T tiles, and
workgroup w of n = min(nwg, T) takes tiles floor(w T / n) .. floor((w + 1) T / n) - 1.
Every workgroup turns the device-side prefix lengths into tile offsets and finds the unit
and tile its share starts at; it writes one partial per unit it meets into slot unit + w,
and records itself as the unit's first share (its piece starts at the unit's first tile)
or last share (its piece ends at the unit's last tile); the merge reads a unit's pieces
from slots unit + first .. unit + last.  This test restates that arithmetic in Python and
checks the invariants the kernels rely on, over random shapes and prefix lengths:
  * every (unit, tile) is covered by exactly one workgroup, and every share is nonempty;
  * the start (unit, tile) of each share is where the previous share ended;
  * partial slots unit + w are unique and inside the workspace (units + nwg slots);
  * each unit's first and last share are recorded exactly once, the range between them is
    exactly the workgroups that wrote a piece of it (the same range the tile offsets
    give), and a unit held by one workgroup (first = last) is written as output, never as
    a partial;
  * a paged share's block-table entries fit the staging area.
"""
import random

import pytest

BT_CAP = 1024  # block-table entries a workgroup stages in LDS


def unit_tiles(P, rt, rows_per_tile, B, G):
    """Key tiles (64 keys) that row tile rt of a sequence with prefix P can see."""
    v_hi = min(B - 1, (rt * rows_per_tile + rows_per_tile - 1) // G)
    return (P + v_hi + 1 + 63) // 64


def plan_nwg(S, B, G, Hkv, max_prefix, block_size, rows_per_tile=256):
    nrt = -(-(G * B) // rows_per_tile)
    tmax = S * Hkv * sum(unit_tiles(max_prefix, rt, rows_per_tile, B, G) for rt in range(nrt))
    nwg = 256
    if block_size:
        cap = max(1, (BT_CAP - 2) * block_size // 64)
        nwg = max(nwg, -(-tmax // cap))
    return max(1, min(nwg, tmax)), nrt


def schedule(S, B, G, Hkv, Ps, nwg, nrt, rows_per_tile=256):
    """Tile offsets per sequence and each workgroup's start, as each workgroup finds them."""
    tab, c = [], 0
    for s in range(S):
        tab.append(c)
        c += Hkv * sum(unit_tiles(Ps[s], rt, rows_per_tile, B, G) for rt in range(nrt))
    tab.append(c)
    T = c
    nw = min(nwg, T)
    starts = []
    for w in range(nwg):
        if w >= nw:
            starts.append((-1, 0))
            continue
        a0 = w * T // nw
        # the sequence whose tile range holds a0 (ranges are nonempty and partition [0, T))
        holders = [s for s in range(S) if tab[s] <= a0 < tab[s + 1]]
        assert len(holders) == 1
        lo = holders[0]
        rel = a0 - tab[lo]
        ts = (tab[lo + 1] - tab[lo]) // Hkv
        g = rel // ts
        rel -= g * ts
        rt = 0
        while rt < nrt - 1:
            t = unit_tiles(Ps[lo], rt, rows_per_tile, B, G)
            if rel < t:
                break
            rel -= t
            rt += 1
        starts.append(((lo * Hkv + g) * nrt + rt, rel))
    return tab, T, starts


def check(S, B, G, Hkv, Ps, max_prefix, block_size):
    rows_per_tile = 256
    nwg, nrt = plan_nwg(S, B, G, Hkv, max_prefix, block_size)
    U = S * Hkv * nrt
    tab, T, starts = schedule(S, B, G, Hkv, Ps, nwg, nrt)
    nw = min(nwg, T)
    covered, slots, finals, writers = {}, set(), set(), {}
    first, last = {}, {}  # the shares each unit records
    per_seq = Hkv * nrt
    prev_end = (0, 0)
    for w in range(nwg):
        u, off = starts[w]
        if u < 0:
            assert w >= nw
            continue
        assert (u, off) == prev_end or (off == 0 and prev_end == (u, 0)), (w, u, off, prev_end)
        left = (w + 1) * T // nw - w * T // nw
        assert left >= 1, "empty share"
        while left > 0:
            s, rt = u // per_seq, u % nrt
            tu = unit_tiles(Ps[s], rt, rows_per_tile, B, G)
            n = min(tu - off, left)
            assert n >= 1
            if block_size:
                assert n * 64 <= (BT_CAP - 2) * block_size + 64
            for t in range(off, off + n):
                assert (u, t) not in covered
                covered[(u, t)] = w
            if off == 0:
                assert u not in first
                first[u] = w
            if off + n == tu:
                assert u not in last
                last[u] = w
            if off == 0 and n == tu:
                finals.add(u)
            else:
                slot = u + w
                assert slot not in slots and 0 <= slot < U + nwg
                slots.add(slot)
                writers.setdefault(u, []).append(w)
            left -= n
            prev_end = (u, off + n) if off + n < tu else (u + 1, 0)
            off = 0
            u += 1
    for u in range(U):
        s, rt = u // per_seq, u % nrt
        for t in range(unit_tiles(Ps[s], rt, rows_per_tile, B, G)):
            assert (u, t) in covered, (u, t)
    # the merge's view of each unit
    wg_of = lambda x: ((x + 1) * nw + T - 1) // T - 1
    for u in range(U):
        s, rt, g = u // per_seq, u % nrt, (u // nrt) % Hkv
        ts = (tab[s + 1] - tab[s]) // Hkv
        A = tab[s] + g * ts + sum(unit_tiles(Ps[s], r2, rows_per_tile, B, G) for r2 in range(rt))
        tu = unit_tiles(Ps[s], rt, rows_per_tile, B, G)
        wf, wl = wg_of(A), wg_of(A + tu - 1)
        assert (first[u], last[u]) == (wf, wl), (u, first[u], last[u], wf, wl)
        if wf == wl:
            assert u in finals and u not in writers
        else:
            assert u not in finals
            assert writers[u] == list(range(wf, wl + 1)), (u, writers[u], wf, wl)
    return T, nwg


@pytest.mark.parametrize("seed", range(8))
def test_balanced_schedule_invariants(seed):
    rng = random.Random(seed)
    n = 0
    while n < 40:
        S = rng.choice([2, 3, 5, 8, 17, 32, 100, 300])
        B = rng.choice([1, 2, 16, 64, 128, 200, 256])
        G = rng.choice([1, 2, 4, 8])
        if G * B <= 128:
            continue          # 4-wave workgroups keep the chunked schedule
        Hkv = rng.choice([1, 2, 4, 8])
        mp = rng.choice([0, 1, 63, 64, 65, 512, 4096, 8192, 20000])
        bs = rng.choice([0, 16, 128, 256])
        Ps = [min(max(rng.choice([0, mp, rng.randint(0, mp), rng.randint(-5, mp + 5)]), 0), mp)
              for _ in range(S)]
        check(S, B, G, Hkv, Ps, mp, bs)
        n += 1


def test_configs():
    """The two benchmark configurations that take the balanced schedule, and many short
    sequences (shares spanning several units)."""
    rng = random.Random(4000)
    check(1000, 72, 2, 2, [rng.randint(0, 300) for _ in range(1000)], 300, 16)
    check(8, 128, 4, 8, [rng.randint(512, 8192) for _ in range(8)], 8192, 16)   # ragged
    check(32, 64, 8, 4, [4096] * 32, 4096, 0)                                 # moe_verify
