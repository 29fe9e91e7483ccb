"""Oracle of the width planners and the routing-mass accumulator.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): plain Python loops over
Python floats (IEEE fp64), written from the description of the
quality-aware runtime planner in "Technical summary: PagedWeight", Core
components 2: the planner scores each possible width reduction by its
damage and, when a memory target must be met, greedily takes the reductions
with the lowest damage per byte saved; frequently routed ("hot") experts get
a higher width floor and a damage multiplier; the routing mass of an expert
counts how often and how strongly it is selected.  The pages' Hessian
sensitivity is an input here and their prompt residuals are left out (both
need trained models).  Readings (stated in the library header too):
routing mass = sum of gate weights, per call summed in ascending assignment
order; damage of lowering q -> q - 1 = weight * 3 * 4^(8 - q); a block's
bytes at width q are its q bit-planes plus LUT_q: R * K * q / 8 + R * 2^q * 2.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple


def block_bytes(R: int, K: int, q: int) -> int:
    """Bytes of one R x K linear block at width q: its q bit-planes, one bit
    per weight each (R * K * q / 8), plus LUT_q, 2^q fp16 entries per row
    (R * 2^q * 2)."""
    return R * K * q // 8 + R * (1 << q) * 2


def block_shape(module: int, H: int, I: int) -> Tuple[int, int]:
    return (2 * I, H) if module == 0 else (H, I)


def routing_mass_add(mass_row: List[float], idx: Sequence[Sequence[int]], w: Sequence[Sequence[float]]) -> None:
    """One call's routing mass: for each expert, the gate weights of its
    assignments a = t * k + j in ascending a, summed from 0.0, then added to
    the running total."""
    T = len(idx)
    k = len(idx[0]) if T else 0
    per = {}
    for a in range(T * k):
        t, j = divmod(a, k)
        e = int(idx[t][j])
        per[e] = per.get(e, 0.0) + float(w[t][j])
    for e, s in per.items():
        mass_row[e] += s


def plan_widths(L: int, E: int, H: int, I: int, q_cur, mass, sens, q_min: int, q_max: int, hot_floor: int,
                hot_share: float, hot_mult: float, mass_eps: float, target: int):
    """Greedy planner; q_cur, sens: [L][E][2]; mass: [L][E].  Returns
    (q [L][E][2] as nested lists, total bytes of the routed blocks)."""
    blocks = []  # (layer, expert, module, weight, floor)
    for l in range(L):
        tot = 0.0
        for e in range(E):
            tot += float(mass[l][e])
        for e in range(E):
            share = float(mass[l][e]) / tot if tot > 0.0 else 0.0
            hot = hot_share > 0.0 and share >= hot_share
            for m in range(2):
                weight = float(sens[l][e][m]) * (share + mass_eps) * (hot_mult if hot else 1.0)
                floor = max(q_min, hot_floor) if hot else q_min
                blocks.append((l, e, m, weight, floor))
    q = []
    for (l, e, m, weight, floor) in blocks:
        q.append(min(max(int(q_cur[l][e][m]), floor), q_max))

    def nbytes(b, qq):
        R, K = block_shape(blocks[b][2], H, I)
        return block_bytes(R, K, qq)

    def drop(b, qq):  # damage added by lowering from qq to qq - 1
        return blocks[b][3] * (3.0 * float(4 ** (8 - qq)))

    total = sum(nbytes(b, q[b]) for b in range(len(blocks)))
    if total > target:
        while total > target:
            best, best_key = -1, 0.0
            for b in range(len(blocks)):
                if q[b] > blocks[b][4]:
                    key = drop(b, q[b]) / float(nbytes(b, q[b]) - nbytes(b, q[b] - 1))
                    if best < 0 or key < best_key:
                        best, best_key = b, key
            if best < 0:
                break
            total -= nbytes(best, q[best]) - nbytes(best, q[best] - 1)
            q[best] -= 1
    else:
        while True:
            best, best_key = -1, 0.0
            for b in range(len(blocks)):
                if q[b] < q_max:
                    add = nbytes(b, q[b] + 1) - nbytes(b, q[b])
                    if total + add > target:
                        continue
                    key = drop(b, q[b] + 1) / float(add)
                    if best < 0 or key > best_key:
                        best, best_key = b, key
            if best < 0:
                break
            total += nbytes(best, q[best] + 1) - nbytes(best, q[best])
            q[best] += 1
    out = [[[0, 0] for _ in range(E)] for _ in range(L)]
    for b, (l, e, m, _, _) in enumerate(blocks):
        out[l][e][m] = q[b]
    return out, total


def plan_event(mass, q, lower: bool, n_change: int, skip=None):
    """One commit event of the fixed-fraction schedule: every routed block
    (layer l, expert e, module m) not skipped and not at the bound (q > 3 when
    lowering, q < 8 when raising) is a candidate; candidates are taken in
    order of their expert's routing mass, then of their block id
    (l * (E + 1) + e) * 2 + m, and the first n_change move one bit.  Returns
    (block ids, new widths) in that order."""
    L = len(q)
    E = len(q[0]) if L else 0
    cands = []
    for l in range(L):
        for e in range(E):
            for m in range(2):
                if skip is not None and skip[l][e][m]:
                    continue
                qq = int(q[l][e][m])
                if (lower and qq <= 3) or (not lower and qq >= 8):
                    continue
                cands.append((float(mass[l][e]), (l * (E + 1) + e) * 2 + m, qq))
    cands.sort()
    chosen = cands[:max(0, n_change)]
    return [c[1] for c in chosen], [c[2] + (-1 if lower else 1) for c in chosen]
