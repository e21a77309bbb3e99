"""Pins of the oracle's expert slot plan (expert paging): a worked example
derived by hand from the rule, and invariants that hold for any sequence of
steps (the maps stay inverse, needed experts end up resident, nothing needed
or protected is evicted, a plan that does not fit moves nothing)."""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O


def test_worked_example():
    st = O.SlotState(6, 3)
    # step 1: experts 1 and 4 take the empty slots 0 and 1 (ascending expert
    # order, slots from the hand at 0); the hand moves to 2
    sid, fetch, n = O.expert_slot_plan(st, [[4, 1]], 1, 1)
    assert n == 2 and fetch == [(1, 0), (4, 1)]
    assert sid.tolist() == [[1, 0]]
    assert st.slot_of == [-1, 0, -1, -1, 1, -1] and st.expert_of == [1, 4, -1]
    assert st.last_use == [1, 1, 0] and st.hand == 2
    # step 2: expert 1 is a hit (stamp 2); expert 5 takes slot 2, the first
    # free slot from the hand (slot 1, expert 4 unused since step 1, is free
    # too but comes later); the hand wraps to 0
    sid, fetch, n = O.expert_slot_plan(st, [[1, 5]], 2, 2)
    assert n == 1 and fetch == [(5, 2)]
    assert sid.tolist() == [[0, 2]]
    assert st.expert_of == [1, 4, 5] and st.last_use == [2, 1, 2] and st.hand == 0
    # step 3 while step 2 may still run (protect_from = 2): only slot 1 is
    # free for two missing experts, so nothing moves and both pairs get slot
    # -1 (dropped by the later calls)
    before = st.copy()
    sid, fetch, n = O.expert_slot_plan(st, [[0, 2]], 3, 2)
    assert n == -1 and fetch == [] and sid.tolist() == [[-1, -1]]
    assert (st.slot_of, st.expert_of, st.last_use, st.hand) == \
        (before.slot_of, before.expert_of, before.last_use, before.hand)
    # the same step once step 2 is done (protect_from = 3): experts 0 and 2
    # evict experts 1 and 4 from slots 0 and 1
    sid, fetch, n = O.expert_slot_plan(st, [[0, 2]], 3, 3)
    assert n == 2 and fetch == [(0, 0), (2, 1)]
    assert sid.tolist() == [[0, 1]]
    assert st.slot_of == [0, -1, 1, -1, -1, 2] and st.expert_of == [0, 2, 5]
    assert st.last_use == [3, 3, 2] and st.hand == 2
    # step 4: experts 1 (a miss), 5 (a hit) and 3 (a miss) with room for
    # two fetches but a fetch limit of one: nothing moves, the hit keeps
    # slot 2 (stamp 4) and the misses get -1; with a limit of two, experts 1
    # and 3 take slots 0 and 1 (neither holds a needed expert: 0 and 2 are
    # not needed, and their stamps 3 are below protect_from 4)
    before = st.copy()
    sid, fetch, n = O.expert_slot_plan(st, [[1, 5], [3, 5]], 4, 4, max_fetch=1)
    assert n == -1 and fetch == [] and sid.tolist() == [[-1, 2], [-1, 2]]
    assert st.slot_of == before.slot_of and st.hand == before.hand
    assert st.last_use == [3, 3, 4]
    sid, fetch, n = O.expert_slot_plan(st, [[1, 5], [3, 5]], 4, 4, max_fetch=2)
    assert n == 2 and fetch == [(1, 0), (3, 1)]
    assert sid.tolist() == [[0, 2], [1, 2]] and st.expert_of == [1, 3, 5]


def test_ids_outside_the_experts_are_ignored():
    st = O.SlotState(4, 2)
    sid, fetch, n = O.expert_slot_plan(st, [[-1, 3], [4, 3]], 1, 1)
    assert n == 1 and fetch == [(3, 0)]
    assert sid.tolist() == [[-1, 0], [-1, 0]] and st.slot_of == [-1, -1, -1, 0]


@pytest.mark.parametrize("E,S,k,steps,seed", [(12, 4, 2, 300, 0), (40, 16, 4, 300, 1),
                                              (8, 8, 3, 200, 2), (3, 1, 1, 100, 3),
                                              (64, 10, 8, 200, 4)])
def test_invariants_over_random_steps(E, S, k, steps, seed):
    rng = np.random.default_rng(seed)
    st = O.SlotState(E, S)
    fits = fails = 0
    for step in range(1, steps + 1):
        T = int(rng.integers(1, 5))
        ids = np.stack([rng.choice(E, size=min(k, E), replace=False) for _ in range(T)])
        protect = int(rng.choice([step, step - 1, max(step - 3, 0)]))
        max_fetch = int(rng.choice([S, S, max(1, S // 2)]))
        before = st.copy()
        needed = set(int(e) for e in ids.ravel())
        sid, fetch, n = O.expert_slot_plan(st, ids, step, protect, max_fetch)
        # the maps stay inverse to each other
        assert all(st.expert_of[s] == e for e, s in enumerate(st.slot_of) if s >= 0)
        assert all(st.slot_of[e] == s for s, e in enumerate(st.expert_of) if e >= 0)
        hits = {e for e in needed if before.slot_of[e] >= 0}
        if n < 0:
            fails += 1
            # nothing moves; only the hits' stamps change; the hits' pairs
            # read their slots and every other pair is dropped (-1)
            assert st.slot_of == before.slot_of and st.expert_of == before.expert_of
            assert st.hand == before.hand
            for s in range(S):
                want = step if before.expert_of[s] in hits else before.last_use[s]
                assert st.last_use[s] == want
            want_sid = np.array([[before.slot_of[e] if e in hits else -1 for e in row]
                                 for row in ids])
            assert np.array_equal(sid, want_sid)
            assert len(needed - hits) > min(max_fetch, S)  or \
                sum(1 for s in range(S) if before.expert_of[s] < 0 or
                    (before.expert_of[s] not in needed and before.last_use[s] < protect)) \
                < len(needed - hits)
            continue
        assert n <= max_fetch
        fits += 1
        # every needed expert is resident and every pair reads its expert
        assert all(st.slot_of[e] >= 0 for e in needed)
        assert np.array_equal(np.array(st.expert_of)[sid], ids)
        # exactly the missing experts are fetched, in ascending order, into
        # distinct slots that held nothing needed or protected
        assert [e for e, _ in fetch] == sorted(needed - hits) and n == len(fetch)
        slots = [s for _, s in fetch]
        assert len(set(slots)) == len(slots)
        for e, s in fetch:
            old = before.expert_of[s]
            assert old < 0 or (old not in needed and before.last_use[s] < protect)
        # resident experts keep their slots; evictions only in fetched slots
        for e in hits:
            assert st.slot_of[e] == before.slot_of[e]
        for s in range(S):
            if s not in slots:
                assert st.expert_of[s] == before.expert_of[s]
        for e in needed:
            assert st.last_use[st.slot_of[e]] == step
        if fetch:
            assert st.hand == (slots[-1] + 1) % S
    assert fits > 0
