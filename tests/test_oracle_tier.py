"""Pins for the placement oracle (oracle/tier.py), from what the pages state about
the tier rules: 'Colibrì 深度解析' section 三 (a saturated heat must stay sticky, not
wrap the threshold; one count is worth 256 points of score and recency at most 255,
so a merely recent expert never displaces a hotter one; the page's worked ranking
of a 256-count expert idle 300 ticks over a 50-count expert used 5 ticks ago;
promotion needs 25 % + 4), and the REPIN page (the logged swap 'evict 4021 (heat 3)
- admit 118 (heat 57)', heat halving, at most four swaps per check)."""
import random

import pytest

from oracle import tier as T

U32 = 0xFFFFFFFF


def test_page_ranking_example():
    clock = 10_000
    assert T.lfru_score(256, clock - 300, clock) > T.lfru_score(50, clock - 5, clock)


def test_one_count_outweighs_any_recency():
    clock = 777
    for h in (0, 1, 5, 1000):
        assert T.lfru_score(h + 1, clock - 10_000, clock) > T.lfru_score(h, clock, clock)
    assert T.lfru_score(3, 777, 777) == 3 * 256 + 255  # just routed: full recency
    assert T.lfru_score(3, 777 - 255, 777) == 3 * 256  # 255 ticks old: none left
    assert T.lfru_score(3, 777 - 254, 777) == 3 * 256 + 1


def test_recency_age_wraps_with_the_clock():
    # the tick counter is 32-bit: an expert routed just before the wrap is recent
    assert T.lfru_score(1, U32 - 1, 3) == 256 + (255 - 5)


def test_hysteresis_25_percent_plus_4():
    assert not T.should_promote(129, 100) and T.should_promote(130, 100)
    assert not T.should_promote(4, 0) and T.should_promote(5, 0)
    assert T.should_promote(57, 3)  # the page's logged swap: heat 57 replaces heat 3
    assert not T.should_promote(7, 3) and T.should_promote(8, 3)


def test_saturated_heat_is_sticky():
    # widened arithmetic: the threshold of a saturated cold counter is above 2^32
    assert not T.should_promote(U32, U32)
    assert not T.should_promote(U32, U32 - 10)
    # (a 32-bit threshold would have wrapped to a small number and admitted it)
    wrapped = (U32 + (U32 >> 2) + 4) & U32
    assert U32 > wrapped


def test_decay_halves_heat():
    c = T.Cache(4, 2)
    c.heat = [0, 1, 7, U32]
    c.decay()
    assert c.heat == [0, 0, 3, U32 >> 1]


def test_admit_fills_free_slots_then_evicts_the_coldest_unneeded():
    c = T.Cache(6, 3)
    assert c.admit([4, 1]) == [(4, 0), (1, 1)]
    assert c.admit([1, 2]) == [(2, 2)]  # 1 already resident
    # full: 5 needs a slot; the residents this batch does not need are 4 (heat 1)
    # and 1 (heat 2): the colder one, 4, goes
    assert c.admit([5, 2]) == [(5, 0)]
    assert c.slot_of[4] == -1 and c.expert_of == [5, 1, 2]
    # heat breaks recency: make 1 hot, then a newcomer evicts the colder of 5, 2
    for _ in range(5):
        c.admit([1])
    assert c.admit([0, 1]) == [(0, 0)]  # 5 (heat 1, older) goes before 2 (heat 2)
    with pytest.raises(ValueError):
        c.admit([0, 1, 2, 3])


def test_repin_swaps_at_most_four_past_the_hysteresis():
    c = T.Cache(20, 6)
    c.admit(list(range(6)))            # residents 0..5, heat 1
    for _ in range(20):                # experts 10..16 grow hot while not resident
        for e in range(10, 17):
            c.heat[e] += 1
    swaps = c.repin()
    assert len(swaps) == 4             # seven candidates pass, four may swap
    assert [h for h, _, _ in swaps] == [10, 11, 12, 13]
    assert all(c.slot_of[h] == s for h, s, _ in swaps)
    # a candidate under the hysteresis stays out
    c2 = T.Cache(4, 1)
    c2.admit([0])
    c2.heat[0] = 100
    c2.heat[3] = 129
    assert c2.repin() == []
    c2.heat[3] = 130
    assert c2.repin() == [(3, 0, 0)]


def test_admit_invariants_random():
    rng = random.Random(1)
    c = T.Cache(50, 12)
    for _ in range(300):
        need = rng.sample(range(50), rng.randint(1, 12))
        loads = c.admit(need)
        assert all(c.slot_of[e] >= 0 for e in need)
        assert all(c.expert_of[c.slot_of[e]] == e for e in range(50) if c.slot_of[e] >= 0)
        assert len({s for _, s in loads}) == len(loads)
        if rng.random() < 0.1:
            c.decay()
        if rng.random() < 0.2:
            c.repin()
