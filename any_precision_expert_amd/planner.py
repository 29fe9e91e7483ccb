"""Host-side width planner used by the multi-layer decode driver.

The PagedWeight pages ("Technical summary: PagedWeight", Core components 2)
describe a planner that, under memory pressure, lowers the widths of the
linear blocks whose reduction costs least, protecting frequently routed
("hot") experts via their routing mass (selection frequency x gate weight).
Their damage score also uses offline Hessian sensitivities and prompt
residuals, which need trained weights; this stand-in ranks blocks by routing
mass alone:

* routing mass of (layer, expert) = sum of the gate weights it received;
* an event changes `fraction` of the routed blocks by one bit, lowering
  (or raising) the blocks with the least routing mass first, ties broken by
  block id, skipping blocks already at the bound (3 when lowering, 8 when
  raising); both blocks of an expert share its mass; shared experts are not
  touched.

Block ids follow the library's (layer * (E + 1) + slot) * 2 + module.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

QMIN, QMAX = 3, 8


class RoutingMass:
    """Accumulated gate weight per (layer, routed expert)."""

    def __init__(self, layers: int, experts: int):
        self.E = experts
        self.m = np.zeros((layers, experts), dtype=np.float64)

    def add(self, layer: int, topk_idx: np.ndarray, topk_w: np.ndarray) -> None:
        np.add.at(self.m[layer], np.asarray(topk_idx).ravel(), np.asarray(topk_w, dtype=np.float64).ravel())


def block_id(layer: int, expert: int, module: int, E: int) -> int:
    return (layer * (E + 1) + expert) * 2 + module


def plan_event(mass: np.ndarray, q: np.ndarray, lower: bool, n_change: int) -> Tuple[np.ndarray, np.ndarray]:
    """Choose blocks for one commit event.

    mass: [L][E] routing mass; q: int [L][E][2] committed widths (routed
    blocks).  Returns (block_ids int32, new widths uint8), ordered by
    (mass ascending, block id ascending)."""
    L, E, _ = q.shape
    lay, exp, mod = np.meshgrid(np.arange(L), np.arange(E), np.arange(2), indexing="ij")
    lay, exp, mod = lay.ravel(), exp.ravel(), mod.ravel()
    qv = q.reshape(-1)
    ok = qv > QMIN if lower else qv < QMAX
    bid = (lay * (E + 1) + exp) * 2 + mod
    ms = mass[lay, exp]
    cand = np.nonzero(ok)[0]
    order = cand[np.lexsort((bid[cand], ms[cand]))]
    pick = order[:n_change]
    newq = qv[pick] + (-1 if lower else 1)
    return bid[pick].astype(np.int32), newq.astype(np.uint8)


def apply_event(q: np.ndarray, ids: np.ndarray, newq: np.ndarray, E: int) -> None:
    """Update the host copy q [L][E][2] with an event's widths."""
    for b, v in zip(ids.tolist(), newq.tolist()):
        module = b & 1
        slot = (b >> 1) % (E + 1)
        layer = (b >> 1) // (E + 1)
        q[layer, slot, module] = v
