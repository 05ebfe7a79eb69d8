"""Pure-Python brute force for tiny inputs, written independently of the
oracle with a different formulation of each step, so that the oracle can be
pinned against something other than itself.

* selection: an expert is chosen iff fewer than k experts beat it, where e'
  beats e when L[e'] > L[e], or L[e'] == L[e] and e' < e; its position in the
  output is the number of experts that beat it;
* capacity: a slot (t, j) is kept iff fewer than cap earlier slots (in
  (t, j) order) went to the same expert; its row is the number of kept slots
  of lower experts plus that count.
"""
from __future__ import annotations

from typing import List, Sequence


def beats(Lrow: Sequence[float], a: int, b: int) -> bool:
    return Lrow[a] > Lrow[b] or (Lrow[a] == Lrow[b] and a < b)


def select(Lrow: Sequence[float], k: int) -> List[int]:
    E = len(Lrow)
    rank = [sum(1 for o in range(E) if o != e and beats(Lrow, o, e)) for e in range(E)]
    out = [-1] * k
    for e in range(E):
        if rank[e] < k:
            out[rank[e]] = e
    return out


def dispatch(idx: Sequence[Sequence[int]], E: int, cap: int):
    T = len(idx)
    k = len(idx[0]) if T else 0
    flat = [(t, j, idx[t][j]) for t in range(T) for j in range(k)]
    before = []
    for n, (t, j, e) in enumerate(flat):
        before.append(sum(1 for (_, _, e2) in flat[:n] if e2 == e))
    kept = [b < cap for b in before]
    counts = [sum(1 for n, (_, _, e2) in enumerate(flat) if e2 == e and kept[n]) for e in range(E)]
    routed = [sum(1 for (_, _, e2) in flat if e2 == e) for e in range(E)]
    offsets = [sum(counts[:e]) for e in range(E + 1)]
    smax = min(T * k, E * cap)
    perm = [-1] * smax
    slot = [[-1] * k for _ in range(T)]
    for n, (t, j, e) in enumerate(flat):
        if kept[n]:
            row = offsets[e] + before[n]
            perm[row] = t
            slot[t][j] = row
    return dict(routed=routed, counts=counts, offsets=offsets, perm=perm, slot=slot)


def coactivation(idx: Sequence[Sequence[int]], E: int):
    """H[i][j] = number of tokens whose list holds both i and j with i at the
    earlier position, found by looking both experts up in every list."""
    H = [[0] * E for _ in range(E)]
    for i in range(E):
        for j in range(E):
            n = 0
            for row in idx:
                row = list(row)
                if i in row and j in row and row.index(i) < row.index(j):
                    n += 1
            H[i][j] = n
    routed = [sum(list(row).count(e) for row in idx) for e in range(E)]
    return H, routed
