"""The oracle of expert placement: the tier admission and ranking rules and an HBM
expert cache that follows them.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

Sources (page titles and sections):
* "Colibrì 深度解析:用 12 万行纯 C 把 744B MoE 塞进 25GB 笔记本", section 三
  (JIT for Weights): the shared admission rule and the LFRU score of every
  adaptive resident tier, and the two-level LFRU it describes: each expert has a
  heat (routing count) and a last-routed tick; eviction ranks by frequency first,
  recency only breaks close calls; promotion needs a hysteresis of 25 % + 4.
* "为什么Colibrì越用越快：路由热度学习缓存与专家自动固定机制深度解析", section 实时重固定
  REPIN: every n tokens, at a safe point, heat halves over time (tier_decay), the
  candidates are ranked by LFRU score, a hot expert replaces a cold one only past
  the 25 % + 4 hysteresis, and at most 4 replacements happen per check.

Restated here in plain Python:
* should_promote(hot, cold): hot > cold + floor(cold / 4) + 4, computed in wide
  integers so that a saturated 32-bit heat stays put instead of wrapping the
  threshold;
* lfru_score(heat, last, clock): 256 * heat + recent, recent = 255 - age when the
  age (clock - last, modulo 2^32) is below 255, else 0;
* decay: every heat halves (integer halving);
* the cache (the HBM tier over host memory, the readings of this build): S slots;
  `admit(needed)` advances the clock by one, adds one to the heat of every needed
  expert (saturating at 2^32 - 1) and stamps its last tick, then gives each needed
  expert that is not resident a slot: a free slot (lowest index first), else the
  slot of the resident expert with the lowest LFRU score among those the batch
  does not need (ties: the lower expert id goes first);
* `repin(max_swaps=4)`: the non-resident experts ranked by LFRU score (highest
  first, ties to the lower id) against the residents ranked lowest first; pair
  them in order and swap while should_promote(hot heat, cold heat) holds, at
  most max_swaps times.
"""
from __future__ import annotations

U32 = 0xFFFFFFFF


def should_promote(hot: int, cold: int) -> bool:
    threshold = cold + cold // 4 + 4
    return hot > threshold


def lfru_score(heat: int, last: int, clock: int) -> int:
    age = (clock - last) & U32
    recent = 255 - age if age < 255 else 0
    return (heat << 8) | recent


class Cache:
    def __init__(self, E: int, S: int):
        self.E, self.S = E, S
        self.clock = 0
        self.heat = [0] * E
        self.last = [0] * E
        self.slot_of = [-1] * E
        self.expert_of = [-1] * S

    def score(self, e: int) -> int:
        return lfru_score(self.heat[e], self.last[e], self.clock)

    def decay(self) -> None:
        self.heat = [h >> 1 for h in self.heat]

    def _place(self, e: int, s: int) -> None:
        old = self.expert_of[s]
        if old >= 0:
            self.slot_of[old] = -1
        self.expert_of[s] = e
        self.slot_of[e] = s

    def admit(self, needed) -> list:
        """-> [(expert, slot)] loads, in the order the needed list names them."""
        needed = list(dict.fromkeys(int(e) for e in needed))  # unique, first order
        if len(needed) > self.S:
            raise ValueError("batch needs more experts than the cache holds")
        self.clock = (self.clock + 1) & U32
        for e in needed:
            self.heat[e] = min(U32, self.heat[e] + 1)
            self.last[e] = self.clock
        need = set(needed)
        loads = []
        for e in needed:
            if self.slot_of[e] >= 0:
                continue
            free = [s for s in range(self.S) if self.expert_of[s] < 0]
            if free:
                s = free[0]
            else:
                victims = [self.expert_of[s] for s in range(self.S)
                           if self.expert_of[s] not in need]
                v = min(victims, key=lambda x: (self.score(x), x))
                s = self.slot_of[v]
            self._place(e, s)
            loads.append((e, s))
        return loads

    def repin(self, max_swaps: int = 4) -> list:
        """-> [(admitted expert, slot, evicted expert)]."""
        hot = sorted((e for e in range(self.E) if self.slot_of[e] < 0),
                     key=lambda e: (-self.score(e), e))
        cold = sorted((self.expert_of[s] for s in range(self.S) if self.expert_of[s] >= 0),
                      key=lambda e: (self.score(e), e))
        swaps = []
        for h, c in zip(hot, cold):
            if len(swaps) >= max_swaps or not should_promote(self.heat[h], self.heat[c]):
                break
            s = self.slot_of[c]
            self._place(h, s)
            swaps.append((h, s, c))
        return swaps
