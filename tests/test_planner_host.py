"""Host logic of the width planner stand-in (no GPU): ordering by routing
mass then block id, bounds, event size, and the host width bookkeeping."""
import numpy as np

from any_precision_expert_amd.planner import RoutingMass, apply_event, block_id, plan_event


def test_routing_mass_accumulates_gate_weights():
    m = RoutingMass(2, 4)
    m.add(1, np.array([[0, 3], [3, 2]]), np.array([[0.75, 0.25], [0.5, 0.5]]))
    m.add(1, np.array([[3, 0]]), np.array([[1.0, 0.0]]))
    assert np.array_equal(m.m[0], np.zeros(4))
    assert np.allclose(m.m[1], [0.75, 0.0, 0.5, 1.75])


def test_lowering_picks_least_mass_first_and_skips_the_bound():
    L, E = 2, 3
    q = np.full((L, E, 2), 6)
    q[0, 0, :] = 3                       # at the lower bound: never lowered
    mass = np.array([[0.0, 5.0, 1.0], [1.0, 0.5, 9.0]])
    ids, nq = plan_event(mass, q, lower=True, n_change=5)
    # candidates by (mass, id): (1,1)=0.5 -> ids 18,19; (0,2)=1.0 -> 4,5; (1,0)=1.0 -> 16,17
    assert ids.tolist() == [block_id(1, 1, 0, E), block_id(1, 1, 1, E), block_id(0, 2, 0, E),
                            block_id(0, 2, 1, E), block_id(1, 0, 0, E)]
    assert np.all(nq == 5)


def test_raising_skips_width_eight_and_apply_updates_host_copy():
    L, E = 1, 4
    q = np.array([[[8, 8], [3, 4], [7, 8], [5, 5]]])
    mass = np.array([[0.0, 2.0, 1.0, 3.0]])
    ids, nq = plan_event(mass, q, lower=False, n_change=3)
    assert ids.tolist() == [block_id(0, 2, 0, E), block_id(0, 1, 0, E), block_id(0, 1, 1, E)]
    assert nq.tolist() == [8, 4, 5]
    apply_event(q, ids, nq, E)
    assert q[0].tolist() == [[8, 8], [4, 5], [8, 8], [5, 5]]


def test_event_size_is_capped_by_candidates():
    q = np.full((1, 2, 2), 3)
    ids, nq = plan_event(np.zeros((1, 2)), q, lower=True, n_change=10)
    assert ids.size == 0 and nq.size == 0
