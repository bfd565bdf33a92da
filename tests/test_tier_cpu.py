"""The library's expert placement (coli_tier_*, coli_cache_*) against the placement
oracle on seeded traces, host only.  The plans (loads, swaps, evictions) and the
whole cache state must match exactly after every call.

The traces follow the routing of the Zipf workloads: each batch needs the experts
of T tokens x K draws from a Zipf(1.1) popularity over a seeded expert order, with
a decay every few batches and a REPIN check after others."""
import ctypes

import numpy as np
import pytest

import int4_grouped_expert_amd as coli
from oracle import tier as T

U32 = 0xFFFFFFFF


def same_state(lib_cache, ora):
    assert lib_cache.clock == ora.clock
    assert lib_cache.heat.tolist() == ora.heat
    assert lib_cache.last.tolist() == ora.last
    assert lib_cache.slot_of.tolist() == ora.slot_of
    assert lib_cache.expert_of.tolist() == ora.expert_of


def test_rules_match_the_oracle():
    rng = np.random.default_rng(5)
    vals = [0, 1, 3, 4, 5, 7, 8, 100, 129, 130, 254, 255, 256, U32 - 10, U32 - 1, U32]
    vals += [int(v) for v in rng.integers(0, U32 + 1, 200, dtype=np.uint64)]
    for h in vals:
        for c in vals[:40]:
            assert coli.coli_tier_should_promote(h, c) == T.should_promote(h, c), (h, c)
    for heat in vals[:40]:
        for last in vals[:30]:
            for clock in (0, 3, 255, 777, U32):
                assert coli.coli_tier_lfru_score(heat, last, clock) == \
                    T.lfru_score(heat, last, clock), (heat, last, clock)


def zipf_batches(E, T_tok, K, n, seed):
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    order = rng.permutation(E)
    for _ in range(n):
        picks = []
        for _t in range(T_tok):
            # K distinct experts per token, drawn by popularity
            picks.extend(order[rng.choice(E, size=K, replace=False, p=p)].tolist())
        yield picks


@pytest.mark.parametrize("E,S,T_tok,K,seed", [(16, 6, 1, 4, 1), (64, 24, 2, 8, 2),
                                              (256, 64, 4, 8, 3), (256, 200, 8, 8, 4),
                                              (40, 40, 3, 6, 5)])
def test_traces_match_the_oracle(E, S, T_tok, K, seed):
    lib_cache = coli.Cache(E, S)
    ora = T.Cache(E, S)
    same_state(lib_cache, ora)
    for i, need in enumerate(zipf_batches(E, T_tok, K, 300, seed)):
        if len(set(need)) > S:
            need = list(dict.fromkeys(need))[:S]
        assert lib_cache.admit(need) == ora.admit(need)
        same_state(lib_cache, ora)
        if i % 17 == 16:
            lib_cache.decay()
            ora.decay()
        if i % 5 == 4:
            ms = (4, 1, 0, 7)[i % 4]
            assert lib_cache.repin(ms) == ora.repin(ms)
        same_state(lib_cache, ora)
    # every resident maps back to its slot
    for s, e in enumerate(lib_cache.expert_of.tolist()):
        if e >= 0:
            assert lib_cache.slot_of[e] == s


def test_repin_swaps_hot_experts_in():
    # a cache whose residents went cold while outsiders stayed hot
    E, S = 12, 3
    lib_cache, ora = coli.Cache(E, S), T.Cache(E, S)
    for c in (lib_cache, ora):
        c.admit([0, 1, 2])
    for _ in range(40):
        for c in (lib_cache, ora):
            c.heat[5] += 1
            c.heat[7] += 2
    sw = lib_cache.repin(4)
    assert sw == ora.repin(4)
    assert {h for h, _, _ in sw} == {5, 7}
    same_state(lib_cache, ora)


def test_saturated_heat_stays():
    lib_cache, ora = coli.Cache(4, 2), T.Cache(4, 2)
    for c in (lib_cache, ora):
        c.admit([0, 1])
        c.heat[0] = U32
        c.heat[1] = U32
        c.heat[2] = U32
        c.heat[3] = U32
    assert lib_cache.repin(4) == ora.repin(4) == []
    assert lib_cache.admit([0]) == ora.admit([0])
    assert int(lib_cache.heat[0]) == U32  # saturates, does not wrap
    same_state(lib_cache, ora)


def test_errors_leave_the_state_unchanged():
    L = coli.lib
    c = coli.Cache(8, 3)
    c.admit([1, 2])
    before = (c.clock, c.heat.copy(), c.last.copy(), c.slot_of.copy(), c.expert_of.copy())

    def unchanged():
        assert c.clock == before[0]
        for a, b in zip((c.heat, c.last, c.slot_of, c.expert_of), before[1:]):
            assert (a == b).all()
    with pytest.raises(coli.ColiError) as ei:
        c.admit([0, 1, 2, 3])  # four experts, three slots
    assert ei.value.status == coli.COLI_ESHAPE
    unchanged()
    for bad in ([8], [-1], [0, 9]):
        with pytest.raises(coli.ColiError) as ei:
            c.admit(bad)
        assert ei.value.status == coli.COLI_EINVAL
        unchanged()
    buf = np.zeros(8, dtype=np.int32)
    n = ctypes.c_int(0)
    assert L.coli_cache_admit(None, buf.ctypes.data, 1, buf.ctypes.data, buf.ctypes.data,
                              ctypes.byref(n)) == coli.COLI_EINVAL
    assert L.coli_cache_repin(ctypes.byref(c.c), -1, buf.ctypes.data, buf.ctypes.data,
                              buf.ctypes.data, ctypes.byref(n)) == coli.COLI_ESHAPE
    unchanged()
    # an empty batch still ticks the clock and loads nothing
    assert c.admit([]) == []
    assert c.clock == before[0] + 1


def test_bad_shapes_rejected():
    L = coli.lib
    h = np.zeros(4, dtype=np.uint32)
    s = np.zeros(4, dtype=np.int32)
    for E, S in ((0, 0), (4, 0), (4, 5), (2000, 3)):
        st = coli.coli_cache(E, S, 0, h.ctypes.data, h.ctypes.data, s.ctypes.data, s.ctypes.data)
        assert L.coli_cache_init(ctypes.byref(st)) == coli.COLI_ESHAPE
        assert L.coli_cache_decay(ctypes.byref(st)) == coli.COLI_ESHAPE
    st = coli.coli_cache(4, 2, 0, h.ctypes.data, None, s.ctypes.data, s.ctypes.data)
    assert L.coli_cache_init(ctypes.byref(st)) == coli.COLI_ESHAPE
    assert L.coli_cache_init(None) == coli.COLI_EINVAL
    # staging: argument errors before any copy (pointers here are not device memory)
    one = np.zeros(1, dtype=np.int32)
    assert L.coli_cache_stage(None, None, 64, one.ctypes.data, one.ctypes.data, 1,
                              None) == coli.COLI_EINVAL
    assert L.coli_cache_stage(None, None, 64, None, None, 0, None) == coli.COLI_OK
    neg = np.full(1, -1, dtype=np.int32)
    assert L.coli_cache_stage(1 << 20, 1 << 21, 64, neg.ctypes.data, one.ctypes.data, 1,
                              None) == coli.COLI_EINVAL
    assert L.coli_cache_stage(1 << 20, 1 << 21, 0, one.ctypes.data, one.ctypes.data, 1,
                              None) == coli.COLI_ESHAPE
    assert L.coli_cache_slot_map(None, None, None) == coli.COLI_EINVAL
