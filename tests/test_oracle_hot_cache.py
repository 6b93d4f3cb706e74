"""Pins of the two-tier cache's LRU model (oracle/hot_cache.py): hand-worked
sequences, and, on random sequences, least-recently-used properties that a
mistake in the model would break -- checked here from first principles
(pairwise comparisons of last uses), not by re-running the model's ranking."""
import random

import pytest

from oracle.hot_cache import HotCacheModel


def test_hand_worked_sequence():
    m = HotCacheModel(4)
    # step 1: three misses fill the three lowest never-used slots
    assert m.step([(0, 2), (0, 0), (0, 1)]) == ([(0, 0), (0, 1), (0, 2)], [0, 1, 2], [])
    # step 2: token 1 hits (slot 1); token 3 takes the never-used slot 3
    assert m.step([(0, 1), (0, 3)]) == ([(0, 3)], [3], [])
    # step 3: token 0 hits (slot 0).  Last uses: slot 1 -> 2, slot 2 -> 1,
    # slot 3 -> 2.  Two misses: slot 2 (used longest ago) ranks first, then
    # slot 1 (last use 2, lower than slot 3)
    misses, victims, evicted = m.step([(0, 4), (0, 0), (0, 5)])
    assert misses == [(0, 4), (0, 5)]
    assert victims == [2, 1]
    assert evicted == [(0, 2), (0, 1)]
    assert m.slot_of == {(0, 0): 0, (0, 5): 1, (0, 4): 2, (0, 3): 3}
    assert m.last_use == [3, 3, 3, 2]
    assert m.clock == 3


def test_ranking_oldest_first_then_lower_slot():
    m = HotCacheModel(5)
    m.step([(0, 0), (0, 1), (0, 2), (0, 3), (0, 4)])          # all slots used at step 1
    m.step([(0, 1), (0, 3)])                                  # slots 1, 3 at step 2
    m.step([(0, 3)])                                          # slot 3 at step 3
    # step 4: last uses 0 -> 1, 1 -> 2, 2 -> 1, 3 -> this step, 4 -> 1: three
    # misses take the slots last used at step 1; slot 1 (step 2) stays
    _, victims, _ = m.step([(0, 3), (1, 7), (1, 8), (1, 9)])
    assert victims == [0, 2, 4]
    # step 5: slot 1 -> step 2, the others -> step 4: slot 1 first, then slot 0
    _, victims, _ = m.step([(2, 0), (2, 1)])
    assert victims == [1, 0]
    # step 6: slots 0, 1 used now; 2, 3, 4 last used at step 4, by slot
    _, victims, _ = m.step([(2, 0), (2, 1), (3, 0), (3, 1), (3, 2)])
    assert victims == [2, 3, 4]


def test_ages_are_not_capped():
    """A slot last used 70000 steps ago is older than one used 60000 steps
    ago: no age limit makes them tie (where a 16-bit age would)."""
    m = HotCacheModel(3)
    m.step([(0, 0), (0, 1), (0, 2)])                          # step 1: slots 0, 1, 2
    m.clock = 9
    m.step([(0, 2)])                                          # step 10: slot 2
    m.clock = 70000
    m.step([(0, 1)])                                          # step 70001: slot 1
    m.clock = 130000
    # step 130001: ages 130000 (slot 0), 60000 (slot 1), 129991 (slot 2)
    _, victims, evicted = m.step([(5, 5), (5, 6)])
    assert victims == [0, 2]
    assert evicted == [(0, 0), (0, 2)]


def test_never_used_ranks_before_any_used_slot():
    m = HotCacheModel(4)
    m.step([(0, 9)])                                          # slot 0 used at step 1
    m.clock = 10 ** 6                                         # ... a million steps ago
    _, victims, _ = m.step([(1, 0), (1, 1), (1, 2)])
    assert victims == [1, 2, 3]                               # the never-used slots, by slot


def test_supplied_assignment_is_checked_and_used():
    m = HotCacheModel(4)
    m.step([(0, 0), (0, 1)])
    # misses (0, 5), (0, 6) go to the never-used slots 2 and 3, in either order
    misses, victims, _ = m.step([(0, 5), (0, 6)], assign={(0, 5): 3, (0, 6): 2})
    assert victims == [2, 3]
    assert m.slot_of[(0, 5)] == 3 and m.slot_of[(0, 6)] == 2
    with pytest.raises(AssertionError):                       # slot 1 is not a victim here
        HotCacheModel(2).step([(0, 1)], assign={(0, 1): 1})
    with pytest.raises(AssertionError):                       # two misses into one slot
        HotCacheModel(3).step([(0, 1), (0, 2)], assign={(0, 1): 0, (0, 2): 0})


def test_capacity_below_selection_is_an_error():
    with pytest.raises(ValueError):
        HotCacheModel(2).step([(0, 0), (0, 1), (0, 2)])


@pytest.mark.parametrize("seed", range(6))
def test_lru_properties_on_random_sequences(seed):
    rnd = random.Random(seed)
    cap = rnd.choice([8, 16, 33])
    m = HotCacheModel(cap)
    last_sel = {}                                             # token -> step it was last selected
    for _ in range(40):
        if rnd.random() < 0.2:                                # jump the clock now and then
            m.clock += rnd.choice([1, 100, 70000])
        step = m.clock + 1
        sel = {(rnd.randrange(3), rnd.randrange(40)) for _ in range(rnd.randrange(1, cap + 1))}
        sel = set(list(sel)[:cap])
        before = dict(m.slot_of)
        lu0 = list(m.last_use)
        used = {before[rs] for rs in sel if rs in before}
        misses_pred = sorted(rs for rs in sel if rs not in before)
        # a random one-to-one assignment onto the victims half of the time
        assign = None
        if rnd.random() < 0.5:
            slots = [v for v in m.rank(step) if v not in used][:len(misses_pred)]
            rnd.shuffle(slots)
            assign = dict(zip(misses_pred, slots))
        misses, victims, evicted = m.step(sel, assign=assign)
        for rs in sel:
            last_sel[rs] = step
        # every selected token is resident; the maps are mutually inverse
        assert all(rs in m.slot_of for rs in sel)
        assert len(m.slot_of) <= cap
        for rs, v in m.slot_of.items():
            assert m.owner[v] == rs
        # misses: exactly the selected tokens not resident before, in order
        assert misses == misses_pred
        # victims: distinct, never a slot holding a selected token
        assert len(set(victims)) == len(victims) == len(misses)
        assert not used & set(victims)
        # LRU, pairwise: every slot kept (not used now, not a victim) was used
        # no earlier than every victim (never used = -1 counts as earliest),
        # and at equal last uses the victim has the lower slot number
        kept = [v for v in range(cap) if v not in used and v not in victims]
        for v in victims:
            for w in kept:
                assert lu0[v] <= lu0[w]
                if lu0[v] == lu0[w]:
                    assert v < w
        # a slot's last use is the last step its token was selected
        for rs, v in m.slot_of.items():
            assert m.last_use[v] == last_sel[rs]
        assert set(evicted) == {rs for rs, v in before.items() if v in victims}
