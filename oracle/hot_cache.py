"""Reference model of the two-tier latent cache's placement policy.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the product library
never imports it, and it imports nothing from the product library.

Sources: SemiAnalysis, "Sparse Savings, Persistent Demand: inside GLM-5.3",
section "How Sparse Attention Affects DRAM/NAND Memory", and remio.ai, section
"HiSparse Move o Histórico Completo para Fora da GPU" -- a bounded device
cache in front of the full history in host memory that behaves like an LRU
cache: tokens a top-K selection misses are loaded from host memory, the least
recently used entries are evicted.  The pages fix no tie rule, age unit or
order of placement; the readings taken here (also the library's contract):

* a step is one selection; selected resident tokens are hits and their
  slot's last use becomes the step;
* the misses are the distinct selected tokens that are not resident, in
  (request, token) order;
* the victims are the slots not used in the step with the greatest age
  (step - last use, saturated at 65535; a never-used slot has age 65535),
  ties to the lower slot, one per miss; miss i moves into the i-th victim of
  the order "victims older than the last one's age, by slot; then those of
  that age, by slot";
* the victim's previous token stops being resident.

Plain Python over dicts and lists, one selection at a time, for the small
cases the tests use.  Pins: ``tests/test_oracle_hot_cache.py`` (a hand-worked
sequence, and LRU / consistency properties checked independently of this
construction on random sequences).
"""
from __future__ import annotations

MAX_AGE = 65535


class HotCacheModel:
    def __init__(self, capacity: int):
        self.capacity = capacity
        self.slot_of = {}                      # (r, s) -> slot
        self.owner = [None] * capacity         # slot -> (r, s) or None
        self.last_use = [-1] * capacity        # slot -> step, -1 never
        self.clock = 0

    def age(self, slot: int, step: int) -> int:
        lu = self.last_use[slot]
        return MAX_AGE if lu < 0 else min(step - lu, MAX_AGE)

    def step(self, selected):
        """selected: iterable of (request, token).  Returns (misses, victims,
        evicted) of this step, each in placement order."""
        step = self.clock + 1
        sel = set(selected)
        for rs in sel:
            if rs in self.slot_of:
                self.last_use[self.slot_of[rs]] = step
        misses = sorted(rs for rs in sel if rs not in self.slot_of)
        eligible = [v for v in range(self.capacity) if self.last_use[v] != step]
        if len(misses) > len(eligible):
            raise ValueError("capacity below the step's distinct selected tokens")
        ranked = sorted(eligible, key=lambda v: (-self.age(v, step), v))[:len(misses)]
        victims = []
        if ranked:
            a_star = self.age(ranked[-1], step)
            victims = sorted(v for v in ranked if self.age(v, step) > a_star)
            victims += sorted(v for v in ranked if self.age(v, step) == a_star)
        evicted = []
        for rs, v in zip(misses, victims):
            old = self.owner[v]
            if old is not None:
                del self.slot_of[old]
                evicted.append(old)
            self.owner[v] = rs
            self.slot_of[rs] = v
            self.last_use[v] = step
        self.clock = step
        return misses, victims, evicted
