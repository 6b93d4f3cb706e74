"""Pins of the two-tier cache's placement model (oracle/hot_cache.py): a
hand-worked sequence, and, on random sequences, properties that a mistake in
the construction would break -- checked here from first principles, not by
re-running the model's own sort."""
import random

import pytest

from oracle.hot_cache import MAX_AGE, HotCacheModel


def test_hand_worked_sequence():
    m = HotCacheModel(4)
    # step 1: three misses fill the three lowest never-used slots
    assert m.step([(0, 2), (0, 0), (0, 1)]) == ([(0, 0), (0, 1), (0, 2)], [0, 1, 2], [])
    # step 2: token 1 hits (slot 1); token 3 takes the never-used slot 3
    assert m.step([(0, 1), (0, 3)]) == ([(0, 3)], [3], [])
    # step 3: token 0 hits; ages now: slot 1 -> 1, slot 2 -> 2, slot 3 -> 1.
    # Two misses: slot 2 (oldest) first, then slot 1 (age 1, lower than slot 3)
    misses, victims, evicted = m.step([(0, 4), (0, 0), (0, 5)])
    assert misses == [(0, 4), (0, 5)]
    assert victims == [2, 1]
    assert evicted == [(0, 2), (0, 1)]
    assert m.slot_of == {(0, 0): 0, (0, 5): 1, (0, 4): 2, (0, 3): 3}
    assert m.last_use == [3, 3, 3, 2]
    assert m.clock == 3


def test_victim_order_older_first_then_ties_by_slot():
    m = HotCacheModel(5)
    m.step([(0, 0), (0, 1), (0, 2), (0, 3), (0, 4)])          # all slots used at step 1
    m.step([(0, 1), (0, 3)])                                  # slots 1, 3 at step 2
    m.step([(0, 3)])                                          # slot 3 at step 3
    # step 4: ages 0 -> 3, 1 -> 2, 2 -> 3, 3 -> used, 4 -> 3; three misses take
    # the age-3 slots; the next oldest (slot 1) stays
    _, victims, _ = m.step([(0, 3), (1, 7), (1, 8), (1, 9)])
    assert victims == [0, 2, 4]
    # step 5: slot 1 -> age 3, every other slot -> age 1 (used at step 4): the
    # older victim (slot 1) first, then the lowest of the age-1 slots
    _, victims, _ = m.step([(2, 0), (2, 1)])
    assert victims == [1, 0]
    # step 6: slot 2 and 3 and 4 -> age 2, slots 0 and 1 -> used; three of
    # age 2 by slot
    _, victims, _ = m.step([(2, 0), (2, 1), (3, 0), (3, 1), (3, 2)])
    assert victims == [2, 3, 4]


def test_age_saturates_and_never_used_is_oldest():
    m = HotCacheModel(2)
    m.step([(0, 0)])
    m.clock = MAX_AGE + 10                                    # slot 0 last used long ago
    assert m.age(0, m.clock + 1) == MAX_AGE
    assert m.age(1, m.clock + 1) == MAX_AGE                   # never used
    _, victims, _ = m.step([(0, 5)])
    assert victims == [0]                                     # tie at the cap: lower slot


@pytest.mark.parametrize("seed", range(6))
def test_properties_on_random_sequences(seed):
    rnd = random.Random(seed)
    cap = rnd.choice([8, 16, 33])
    m = HotCacheModel(cap)
    last_use = {}                                             # token -> step it was last selected
    for step in range(1, 40):
        sel = {(rnd.randrange(3), rnd.randrange(40)) for _ in range(rnd.randrange(1, cap + 1))}
        sel = set(list(sel)[:cap])
        before = dict(m.slot_of)
        ages_before = {v: m.age(v, step) for v in range(cap)}
        misses, victims, evicted = m.step(sel)
        for rs in sel:
            last_use[rs] = step
        # every selected token is resident; the maps are mutually inverse
        assert all(rs in m.slot_of for rs in sel)
        assert len(m.slot_of) <= cap
        for rs, v in m.slot_of.items():
            assert m.owner[v] == rs
        # misses: exactly the selected tokens not resident before, in order
        assert misses == sorted(rs for rs in sel if rs not in before)
        # victims: distinct, never a slot holding a selected token
        assert len(set(victims)) == len(victims) == len(misses)
        used = {before[rs] for rs in sel if rs in before}
        assert not used & set(victims)
        # LRU: no kept, unused slot is older than an evicted one; equal ages
        # go to the lower slot first
        kept = [v for v in range(cap) if v not in used and v not in victims]
        if victims:
            youngest = min(ages_before[v] for v in victims)
            assert all(ages_before[v] <= youngest for v in kept)
            tie_kept = [v for v in kept if ages_before[v] == youngest]
            tie_taken = [v for v in victims if ages_before[v] == youngest]
            assert not tie_kept or max(tie_taken) < min(tie_kept)
        # a slot's last use is the last step its token was selected
        for rs, v in m.slot_of.items():
            assert m.last_use[v] == last_use[rs]
        assert set(evicted) == {before_rs for before_rs, v in before.items() if v in victims}
