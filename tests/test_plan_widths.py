"""Width planner and routing-mass accumulator (host, no GPU).

The oracle (oracle/plan.py) is pinned by consequences of its definition
(targets that fit everything or nothing, hot-expert floors, zero-damage
reductions first, the raise direction, monotonicity in the target, the
routing mass of a softmax summing to the token count).  The library's host
planner (pw_plan_widths) must then return exactly the oracle's widths and
byte total on seeded random instances.  Quality-aware runtime planner:
"Technical summary: PagedWeight", Core components 2.
"""
import numpy as np
import pytest

import oracle.plan as op

P = dict(q_min=3, q_max=8, hot_floor=6, hot_share=0.1, hot_mult=4.0, mass_eps=1e-3)


def run_oracle(H, I, q, mass, sens, target, **kw):
    prm = dict(P, **kw)
    L, E = len(q), len(q[0])
    out, total = op.plan_widths(L, E, H, I, q, mass, sens, prm["q_min"], prm["q_max"], prm["hot_floor"],
                                prm["hot_share"], prm["hot_mult"], prm["mass_eps"], target)
    return np.array(out), total


def total_bytes(H, I, q):
    L, E = q.shape[0], q.shape[1]
    s = 0
    for l in range(L):
        for e in range(E):
            for m in range(2):
                R, K = op.block_shape(m, H, I)
                s += op.block_bytes(R, K, int(q[l, e, m]))
    return s


def test_block_bytes_hand_computed():
    # 64 x 256 block at q = 3: 3 planes of 64 * 256 bits = 3 * 2048 bytes, plus
    # 64 rows x 8 fp16 entries = 1024 bytes
    assert op.block_bytes(64, 256, 3) == 6144 + 1024
    # q = 8: one byte per weight (16384) plus 64 rows x 256 entries x 2 bytes (32768)
    assert op.block_bytes(64, 256, 8) == 16384 + 32768
    # a Qwen1.5-MoE-shaped gate_up block (2 x 1408 rows, K = 2048) at q = 5:
    # 2816 * 2048 * 5 / 8 = 3604480 plus 2816 * 32 * 2 = 180224
    assert op.block_bytes(*op.block_shape(0, 2048, 1408), 5) == 3604480 + 180224
    # down block of the same expert (2048 x 1408) at q = 4
    assert op.block_bytes(*op.block_shape(1, 2048, 1408), 4) == 1441792 + 65536


def test_target_that_fits_everything_raises_all_to_q_max():
    H, I = 128, 256
    q = np.full((2, 3, 2), 3)
    mass = np.ones((2, 3))
    sens = np.ones((2, 3, 2))
    out, total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), 10 ** 12)
    assert np.all(out == 8)
    assert total == total_bytes(H, I, out)


def test_target_zero_leaves_every_block_at_its_floor():
    H, I = 128, 256
    q = np.full((1, 4, 2), 8)
    mass = np.array([[10.0, 0.0, 0.0, 0.0]])  # expert 0 hot (share 1), the rest cold
    sens = np.ones((1, 4, 2))
    out, total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), 0)
    assert np.all(out[0, 0] == P["hot_floor"]) and np.all(out[0, 1:] == P["q_min"])
    assert total == total_bytes(H, I, out)


def test_zero_damage_reduction_is_taken_first_lowest_block_first():
    H, I = 128, 128
    q = np.full((1, 2, 2), 8)
    mass = np.ones((1, 2))
    sens = np.zeros((1, 2, 2))
    sens[0, 0, 0] = 1.0  # only block 0 costs damage
    full = total_bytes(H, I, q)
    out, total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), full - 1)
    changed = np.argwhere(out != q)
    assert changed.tolist() == [[0, 0, 1]] and out[0, 0, 1] == 7  # block 1 = (expert 0, down), one bit
    assert total < full


def test_heavier_expert_is_lowered_only_after_the_light_one_reaches_its_floor():
    H, I = 128, 128
    q = np.full((1, 2, 2), 8)
    mass = np.ones((1, 2))
    sens = np.ones((1, 2, 2))
    sens[0, 1] = 1e6
    floors_light = total_bytes(H, I, np.array([[[3, 3], [8, 8]]]))
    out, total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), floors_light - 1, hot_share=0.0)
    assert np.all(out[0, 0] == 3)
    assert int(np.sum(8 - out[0, 1])) == 1 and total <= floors_light - 1


def test_raise_takes_the_block_with_most_damage_removed_per_byte():
    H, I = 128, 128
    q = np.full((1, 3, 2), 3)
    mass = np.ones((1, 3))
    sens = np.ones((1, 3, 2))
    sens[0, 2, 1] = 1e4  # block 5 dominates
    base = total_bytes(H, I, q)
    R, K = op.block_shape(1, H, I)
    step = op.block_bytes(R, K, 4) - op.block_bytes(R, K, 3)
    out, total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), base + step, hot_share=0.0)
    assert np.argwhere(out != q).tolist() == [[0, 2, 1]] and out[0, 2, 1] == 4
    assert total == base + step


def test_total_is_monotone_in_the_target_and_fits_it():
    rng = np.random.default_rng(5)
    H, I = 96, 160
    q = rng.integers(3, 9, size=(2, 4, 2))
    mass = rng.random((2, 4))
    sens = rng.random((2, 4, 2))
    floor_total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), 0)[1]
    last = -1
    for target in np.linspace(floor_total, total_bytes(H, I, np.full((2, 4, 2), 8)), 9).astype(int):
        _, total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.tolist(), int(target))
        assert total <= target and total >= last
        last = total


def test_routing_mass_of_softmax_weights_sums_to_the_tokens():
    rng = np.random.default_rng(2)
    E, k, T = 6, 2, 5
    row = [0.0] * E
    for _ in range(3):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        w = rng.random((T, k))
        w /= w.sum(1, keepdims=True)
        op.routing_mass_add(row, idx.tolist(), w.tolist())
    assert abs(sum(row) - 3 * T) < 1e-12 and min(row) >= 0.0
    row2 = [0.0] * E
    op.routing_mass_add(row2, [[1, 3]], [[0.25, 0.75]])
    assert row2 == [0.0, 0.25, 0.0, 0.75, 0.0, 0.0]


@pytest.mark.parametrize("seed", range(24))
def test_library_planner_equals_oracle(seed):
    import any_precision_expert_amd as pw
    rng = np.random.default_rng(100 + seed)
    L, E = int(rng.integers(1, 4)), int(rng.integers(2, 9))
    H, I = int(rng.choice([64, 96, 128, 256])), int(rng.choice([64, 160, 352]))
    q = rng.integers(3, 9, size=(L, E, 2)).astype(np.uint8)
    mass = rng.random((L, E)) * (rng.random((L, E)) < 0.7)
    if seed % 5 == 0:
        mass[0] = 0.0
    sens = (rng.random((L, E, 2)) * (rng.random((L, E, 2)) < 0.9)).astype(np.float32)
    kw = dict(q_min=int(rng.integers(3, 5)), q_max=int(rng.integers(6, 9)), hot_floor=int(rng.integers(3, 9)),
              hot_share=float(rng.choice([0.0, 0.05, 0.2])), hot_mult=float(rng.choice([1.0, 4.0])), mass_eps=1e-3)
    kw["hot_floor"] = min(kw["hot_floor"], kw["q_max"])
    lo = run_oracle(H, I, q.tolist(), mass.tolist(), sens.astype(np.float64).tolist(), 0, **kw)[1]
    hi = total_bytes(H, I, np.full((L, E, 2), kw["q_max"]))
    for target in (0, lo, int(lo + (hi - lo) * rng.random()), total_bytes(H, I, q), hi, 10 ** 12):
        want, want_total = run_oracle(H, I, q.tolist(), mass.tolist(), sens.astype(np.float64).tolist(), target, **kw)
        got, got_total = pw.plan_widths(H, I, q, mass, sens, target, **kw)
        assert np.array_equal(got, want) and got_total == want_total, (seed, target)
