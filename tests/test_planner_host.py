"""The fixed-fraction commit-event planner (host, no GPU).

The oracle (oracle/plan.py plan_event) is pinned by hand-worked events
(ordering by routing mass then block id, the width bounds, the cap at the
number of candidates) and by consequences of its definition on random
instances (every skipped or unchosen candidate ranks after every chosen one);
the library's pw_plan_event must then return exactly the oracle's blocks and
widths, ties and skip masks included.  Quality-aware planner and commit
events: "Technical summary: PagedWeight", Core components 2 and 3.
"""
import numpy as np
import pytest

import oracle.plan as op


def bid(l, e, m, E):
    return (l * (E + 1) + e) * 2 + m


def test_lowering_picks_least_mass_first_and_skips_the_bound():
    L, E = 2, 3
    q = np.full((L, E, 2), 6)
    q[0, 0, :] = 3                       # at the lower bound: never lowered
    mass = np.array([[0.0, 5.0, 1.0], [1.0, 0.5, 9.0]])
    ids, nq = op.plan_event(mass, q, lower=True, n_change=5)
    # candidates by (mass, id), ids = (l * 4 + e) * 2 + m: (1,1) mass 0.5 -> ids 10, 11;
    # (0,2) mass 1.0 -> 4, 5; (1,0) mass 1.0 -> 8, 9 (after 4, 5: higher ids)
    assert ids == [bid(1, 1, 0, E), bid(1, 1, 1, E), bid(0, 2, 0, E), bid(0, 2, 1, E), bid(1, 0, 0, E)]
    assert ids == [10, 11, 4, 5, 8]
    assert nq == [5] * 5


def test_raising_skips_width_eight():
    E = 4
    q = np.array([[[8, 8], [3, 4], [7, 8], [5, 5]]])
    mass = np.array([[0.0, 2.0, 1.0, 3.0]])
    ids, nq = op.plan_event(mass, q, lower=False, n_change=3)
    assert ids == [bid(0, 2, 0, E), bid(0, 1, 0, E), bid(0, 1, 1, E)] == [4, 2, 3]
    assert nq == [8, 4, 5]


def test_event_size_is_capped_by_candidates_and_skip_removes_blocks():
    q = np.full((1, 2, 2), 3)
    assert op.plan_event(np.zeros((1, 2)), q, lower=True, n_change=10) == ([], [])
    q = np.full((1, 2, 2), 5)
    skip = np.zeros((1, 2, 2), np.uint8)
    skip[0, 0, 1] = 1
    ids, nq = op.plan_event(np.zeros((1, 2)), q, lower=False, n_change=10, skip=skip)
    assert ids == [0, 2, 3] and nq == [6, 6, 6]


def _random_instance(rng, L, E):
    q = rng.integers(3, 9, size=(L, E, 2))
    mass = rng.integers(0, 4, size=(L, E)).astype(np.float64) * 0.25  # many exact ties
    skip = (rng.random((L, E, 2)) < 0.15).astype(np.uint8)
    return q, mass, skip


@pytest.mark.parametrize("seed", range(12))
def test_oracle_choice_ranks_before_every_other_candidate(seed):
    rng = np.random.default_rng(seed)
    L, E = int(rng.integers(1, 4)), int(rng.integers(1, 9))
    q, mass, skip = _random_instance(rng, L, E)
    lower = bool(seed % 2)
    n = int(rng.integers(0, 2 * L * E + 2))
    ids, nq = op.plan_event(mass, q, lower, n, skip)
    key = {}
    for l in range(L):
        for e in range(E):
            for m in range(2):
                ok = not skip[l, e, m] and (q[l, e, m] > 3 if lower else q[l, e, m] < 8)
                if ok:
                    key[bid(l, e, m, E)] = (mass[l, e], bid(l, e, m, E), int(q[l, e, m]))
    assert len(ids) == min(n, len(key)) and len(set(ids)) == len(ids)
    assert all(b in key for b in ids)
    worst_chosen = max((key[b] for b in ids), default=None)
    for b, k in key.items():
        if b not in ids:
            assert worst_chosen is None or k > worst_chosen
    for b, v in zip(ids, nq):
        assert v == key[b][2] + (-1 if lower else 1)


@pytest.mark.parametrize("seed", range(12))
def test_library_event_planner_equals_the_oracle(seed):
    import any_precision_expert_amd as pw
    rng = np.random.default_rng(100 + seed)
    L, E = int(rng.integers(1, 5)), int(rng.integers(1, 61))
    q, mass, skip = _random_instance(rng, L, E)
    for lower in (True, False):
        n = int(rng.integers(0, 2 * L * E + 2))
        use_skip = skip if seed % 3 else None
        want = op.plan_event(mass, q, lower, n, use_skip)
        ids, nq = pw.plan_event(q, mass, lower, n, use_skip)
        assert ids.tolist() == want[0] and nq.tolist() == want[1]
