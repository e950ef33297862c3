"""Host models of the attention kernels' work schedules (test infrastructure).

Unit kernel (static CHUNK_CAUSAL and DENSE plans):

It replays, in plain Python, how each of the G workgroups of the unit kernel picks its work
from a plan: query tiles with equal span lists paired into units, rounds of whole units, then
either one more round of whole units (when that bound is close to the balanced share) or the
left-over units' key iterations laid end to end and cut into G equal contiguous shares, each
share visited as: the segment of its last unit, the whole units in between (each started at
the share's elapsed iteration count and wrapped), the segment of its first unit.  Split units
are merged by the last of their segments to arrive; the model counts those segments the way
the kernel does.  Tests use it to check that every key iteration of every unit is computed
exactly once, and to know which path a geometry takes on a device with a given CU count.

Tile kernel on a dynamic plan (`tile_work_list`): each query tile's key steps n_t, the chunk
length L = max(8, ceil(W / 512)) with W = heads * sum(n_t), tiles with n_t > L cut into
ceil(n_t / L) chunks of near-equal length (the first n_t mod c one step longer), each chunk of
a split tile with its partial-result slot (split tiles numbered in tile order); the list is
ordered longest first.  The GPU tests compare the device's list with it.
"""
from __future__ import annotations

from dataclasses import dataclass, field

KBN = 64  # keys per iteration


def units_from_plan(qtiles, row_ptr, spans):
    """Units of one head: (first tile, has partner, iterations), from the plan's words."""
    nq = len(qtiles)
    it = [sum((int(kl) + KBN - 1) // KBN for _, kl in spans[row_ptr[q]:row_ptr[q + 1]]) for q in range(nq)]
    same = [q > 0 and [tuple(x) for x in spans[row_ptr[q - 1]:row_ptr[q]]] ==
            [tuple(x) for x in spans[row_ptr[q]:row_ptr[q + 1]]] for q in range(nq)]
    units, run_start = [], 0
    for q in range(nq):
        if not same[q]:
            run_start = q
        if (q - run_start) % 2 == 0:
            partner = q + 1 < nq and same[q + 1]
            units.append((q, partner, it[q]))
    return units


@dataclass
class Schedule:
    whole: bool
    rounds: int
    sk_base: int
    total: int
    # per workgroup (logical index w): list of (h, k, first, end) iteration ranges of units,
    # and whether the range came from the stream
    work: list = field(default_factory=list)
    nseg: dict = field(default_factory=dict)  # (h, k) of each split unit -> its segment count


def schedule(unit_iters, heads, G, lds_rounds=24576):
    n_units = len(unit_iters)
    u_pre = [0]
    for n in unit_iters:
        u_pre.append(u_pre[-1] + n)
    t_head = u_pre[-1]
    total = t_head * heads
    n_all = n_units * heads
    R = (n_all + G - 1) // G
    whole = False
    if n_all % G != 0 and R <= lds_rounds:
        rmax = [0] * R
        for j in range(n_all):
            rmax[j // G] = max(rmax[j // G], unit_iters[j % n_units])
        share = (total + G - 1) // G
        whole = sum(rmax) <= share + min(share * 3 // 16, 40)
    rounds = R if whole else n_all // G
    sk_base = total if whole else (rounds * G // n_units) * t_head + u_pre[(rounds * G) % n_units]
    sk_len = total - sk_base

    def wg_begin(u):
        return sk_base + u * sk_len // G

    def wg_of(x):
        u = (x - sk_base) * G // sk_len
        while u + 1 < G and wg_begin(u + 1) <= x:
            u += 1
        return u

    def locate(r):  # the unit holding iteration r of a head (a unit with iterations)
        lo, hi = 0, n_units - 1
        while lo < hi:
            mid = (lo + hi + 1) >> 1
            if u_pre[mid] <= r:
                lo = mid
            else:
                hi = mid - 1
        return lo, r - u_pre[lo]

    sch = Schedule(whole, rounds, sk_base, total, [[] for _ in range(G)])
    for bid in range(G):
        w = (bid % 8) * (G // 8) + bid // 8  # XCD-contiguous logical index
        out = sch.work[w]
        for rnd in range(rounds):  # rounds of whole units
            j = rnd * G + w
            if whole and rnd == rounds - 1:
                L = n_all - rnd * G
                q, r = L // 8, L % 8
                xcd, idx = bid % 8, bid // 8
                j = rnd * G + xcd * q + min(xcd, r) + idx if idx < q + (1 if xcd < r else 0) else n_all
            if j < n_all and unit_iters[j % n_units] > 0:
                out.append((j // n_units, j % n_units, 0, unit_iters[j % n_units], False))
        B, E = wg_begin(w), wg_begin(w + 1)
        if B == E:
            continue
        h_b, (k_b, ib_b) = B // t_head, locate(B % t_head)
        h_l, (k_l, ie_l) = (E - 1) // t_head, locate((E - 1) % t_head)
        ie_l += 1
        if (h_b, k_b) == (h_l, k_l):
            out.append((h_b, k_b, ib_b, ie_l, True))
            continue
        out.append((h_l, k_l, 0, ie_l, True))  # last unit's segment first
        mh, mk = h_b, k_b
        while True:  # whole units in between
            mk += 1
            if mk == n_units:
                mk, mh = 0, mh + 1
            if (mh, mk) == (h_l, k_l):
                break
            if unit_iters[mk] > 0:
                out.append((mh, mk, 0, unit_iters[mk], True))
        out.append((h_b, k_b, ib_b, unit_iters[k_b], True))
    # split units: the segments the kernel counts (non-empty shares meeting the unit)
    for w in range(G):
        for h, k, a, b, stream in sch.work[w]:
            n = unit_iters[k]
            if stream and not (a == 0 and b == n):
                ut = h * t_head + u_pre[k]
                u0, u1 = wg_of(ut), wg_of(ut + n - 1)
                sch.nseg[(h, k)] = sum(1 for u in range(u0, u1 + 1) if wg_begin(u + 1) > wg_begin(u))
    return sch


def cover_counts(sch, unit_iters, heads):
    """How many times every (head, unit, iteration) is computed, and the segments per unit."""
    cnt = {}
    segs = {}
    for w, items in enumerate(sch.work):
        for h, k, a, b, stream in items:
            segs[(h, k)] = segs.get((h, k), 0) + 1
            for i in range(a, b):
                cnt[(h, k, i)] = cnt.get((h, k, i), 0) + 1
    return cnt, segs


TILE_SLOTS = 512       # balancing target: tile workgroups resident at once
SPLIT_CAP = 2 * TILE_SLOTS
SPLIT_MIN = 8


def tile_steps_from_plan(qtiles, row_ptr, spans):
    """Key steps (KBN keys each) of every query tile of a plan."""
    return [sum((int(kl) + KBN - 1) // KBN for _, kl in spans[row_ptr[q]:row_ptr[q + 1]]) for q in range(len(qtiles))]


def tile_work_list(steps, heads):
    """(items, chunk length) of the tile kernel's work list: items are (tile, begin, end,
    slot, chunk, chunks) in the device's order up to ties (equal lengths in any order; lengths
    of 1023 steps and more count as equal)."""
    W = heads * sum(steps)
    L = max(SPLIT_MIN, -(-W // TILE_SLOTS))
    chunks = [-(-n // L) if n > L else 1 for n in steps]
    if sum(c for c in chunks if c > 1) * heads > SPLIT_CAP:  # the kernel's guard; never taken
        chunks = [1] * len(steps)
    items, first = [], 0
    for t, (n, c) in enumerate(zip(steps, chunks)):
        beg = 0
        for k in range(c):
            ln = n // c + (1 if k < n % c else 0)
            items.append((t, beg, beg + ln, first + k if c > 1 else -1, k, c))
            beg += ln
        if c > 1:
            first += c
    items.sort(key=lambda it: -min(it[2] - it[1], 1023))
    return items, L


def item_start(row_ptr, spans, tile, begin):
    """(span, skip): the plan span that holds key step `begin` of `tile`, and the steps before
    it inside that span."""
    left = begin
    for sp in range(row_ptr[tile], row_ptr[tile + 1]):
        n = (int(spans[sp][1]) + KBN - 1) // KBN
        if left < n:
            return sp, left
        left -= n
    return row_ptr[tile], 0  # an empty item
