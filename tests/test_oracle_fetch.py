"""Pins of the oracle's cold-pool fetch (O10).

The pages move every entry scoring >= 0.5 from the CPU cold pool into GPU
memory ([SUMMARY] 2.1 dynamic-fetch bullet; [REVIEW] section 2).  The
resident set after a fetch must therefore hold exactly the survivors, each
with its own cold-pool row.  The slot each new row takes (the i-th new
survivor in entry order takes the i-th free slot in slot order) and the rule
that rows already resident are not copied again are this library's reading;
they are pinned here by hand-worked cases and by invariants."""
import numpy as np
import pytest

from oracle import oracle


def _state(N, S, rb):
    return (np.full(N, -1, np.int32), np.full(S, -1, np.int32), np.zeros((S, rb), np.uint8))


def _cold(N, rb, seed=0):
    return np.random.default_rng(seed).integers(0, 256, (N, rb), dtype=np.uint8)


def test_hand_worked_sequence():
    # N = 8 entries, S = 4 slots, 2-byte rows holding (2s, 2s+1).
    N, S, rb = 8, 4, 2
    cold = np.arange(N * rb, dtype=np.uint8).reshape(N, rb)
    so, eo, rows = _state(N, S, rb)
    # survivors {1, 3, 6} into the empty set: slots 0, 1, 2 in entry order
    assert oracle.fetch(cold, [1, 3, 6], so, eo, rows) == 3
    assert eo.tolist() == [1, 3, 6, -1]
    assert so.tolist() == [-1, 0, -1, 1, -1, -1, 2, -1]
    assert rows.ravel().tolist() == [2, 3, 6, 7, 12, 13, 0, 0]
    # survivors {0, 3, 5, 7}: 1 and 6 leave slots 0 and 2; 3 stays in slot 1;
    # the new 0, 5, 7 take the free slots 0, 2, 3
    assert oracle.fetch(cold, [0, 3, 5, 7], so, eo, rows) == 3
    assert eo.tolist() == [0, 3, 5, 7]
    assert so.tolist() == [0, -1, -1, 1, -1, 2, -1, 3]
    assert rows.ravel().tolist() == [0, 1, 6, 7, 10, 11, 14, 15]
    # the same survivors again: nothing to copy, nothing moves
    assert oracle.fetch(cold, [0, 3, 5, 7], so, eo, rows) == 0
    assert eo.tolist() == [0, 3, 5, 7]
    # no survivors: every slot is freed, the bytes stay where they were
    assert oracle.fetch(cold, [], so, eo, rows) == 0
    assert eo.tolist() == [-1] * 4 and so.tolist() == [-1] * 8
    assert rows.ravel().tolist() == [0, 1, 6, 7, 10, 11, 14, 15]


def test_capacity_shortfall_leaves_the_tables_alone():
    N, S, rb = 10, 3, 4
    cold = _cold(N, rb)
    so, eo, rows = _state(N, S, rb)
    assert oracle.fetch(cold, [2, 5], so, eo, rows) == 2
    before = (so.copy(), eo.copy(), rows.copy())
    assert oracle.fetch(cold, [1, 2, 5, 9], so, eo, rows) == -1
    assert all(np.array_equal(a, b) for a, b in zip(before, (so, eo, rows)))
    # exactly S survivors fit, whatever was resident before
    assert oracle.fetch(cold, [0, 1, 9], so, eo, rows) == 3
    assert sorted(eo.tolist()) == [0, 1, 9]


@pytest.mark.parametrize("S_extra", [0, 7])
def test_invariants_over_a_trigger_sequence(S_extra):
    rng = np.random.default_rng(5)
    N, rb = 300, 16
    cold = _cold(N, rb, 1)
    sets = []
    cur = set(rng.choice(N, 60, replace=False).tolist())
    for _ in range(8):
        # each trigger keeps about 70% of the previous survivors, adds others
        keep = {s for s in cur if rng.random() < 0.7}
        add = set(rng.choice(N, 40, replace=False).tolist())
        cur = keep | add
        sets.append(sorted(cur))
    S = max(len(s) for s in sets) + S_extra
    so, eo, rows = _state(N, S, rb)
    prev = set()
    for surv in sets:
        slot_before = so.copy()
        kept = set(surv) & prev
        # change the cold rows of resident survivors: a reused row is not
        # read again, so the resident bytes must keep their old value
        old_rows = {s: rows[so[s]].copy() for s in kept}
        cold_mod = cold.copy()
        for s in kept:
            cold_mod[s] ^= 0xFF
        got = oracle.fetch(cold_mod, surv, so, eo, rows)
        assert got == len(set(surv) - prev)
        resident = {int(e) for e in eo if e >= 0}
        assert resident == set(surv)
        for j, e in enumerate(eo):
            if e >= 0:
                assert so[e] == j
        assert int((so >= 0).sum()) == len(surv)
        for s in surv:
            if s in kept:
                assert so[s] == slot_before[s]
                assert np.array_equal(rows[so[s]], old_rows[s])
            else:
                assert np.array_equal(rows[so[s]], cold_mod[s])
        # placement: new survivors in entry order take the free slots in
        # slot order (free = not held by a kept survivor)
        held = {int(slot_before[s]) for s in kept}
        free = [j for j in range(S) if j not in held]
        new = sorted(set(surv) - prev)
        assert [int(so[s]) for s in new] == free[:len(new)]
        prev = set(surv)


def test_gather_resident_follows_the_slot_table():
    N, S, rb = 50, 20, 8
    cold = _cold(N, rb, 3)
    so, eo, rows = _state(N, S, rb)
    surv = [3, 4, 17, 20, 33, 48]
    oracle.fetch(cold, surv, so, eo, rows)
    idx = np.array([48, 3, -1, 20, 5], np.int32)          # 5 is not resident
    hot = oracle.gather_resident(rows, so, idx)
    assert np.array_equal(hot[0], cold[48]) and np.array_equal(hot[1], cold[3])
    assert np.array_equal(hot[3], cold[20])
    assert not hot[2].any() and not hot[4].any()
