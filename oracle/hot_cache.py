"""Reference model of the two-tier latent cache's placement policy.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the product library
never imports it, and it imports nothing from the product library.

Sources: SemiAnalysis, "Sparse Savings, Persistent Demand: inside GLM-5.3",
section "How Sparse Attention Affects DRAM/NAND Memory", and remio.ai, section
"HiSparse Move o Histórico Completo para Fora da GPU": a bounded device cache
in front of the full history in host memory; the tokens a top-K selection
misses are loaded from host memory and the least recently used entries are
evicted to make room.

Plain least-recently-used replacement, written from those words:

* a step is one selection; selected tokens already resident are hits, and
  their slot counts as used in this step;
* the misses are the distinct selected tokens that are not resident;
* the slots that may be reused are those not used in this step; they are
  ranked least recently used first: a slot never used comes before any used
  one, otherwise the earlier last use comes first (ages are unbounded step
  counts), and equal ranks go to the lower slot number;
* as many slots as there are misses are taken from the front of that ranking
  (the victims); each victim's previous token stops being resident, and each
  miss moves into one victim.

Which miss moves into which victim is a placement detail the pages do not fix:
any one-to-one assignment of the misses onto the victims gives the same
resident set and the same slot ages.  ``step`` assigns them in order (the
i-th miss in (request, token) order to the i-th ranked victim) unless the
caller supplies an assignment, which is then checked to be such a one-to-one
map and used.

Plain Python over dicts and lists, one selection at a time, for the small
cases the tests use.  Pins: ``tests/test_oracle_hot_cache.py`` (hand-worked
sequences, and LRU properties checked on random sequences without the
model's own ranking).
"""
from __future__ import annotations


class HotCacheModel:
    def __init__(self, capacity: int):
        self.capacity = capacity
        self.slot_of = {}                      # (r, s) -> slot
        self.owner = [None] * capacity         # slot -> (r, s) or None
        self.last_use = [-1] * capacity        # slot -> step of last use, -1 never
        self.clock = 0                         # the last step taken

    def rank(self, step: int):
        """Slots that may be reused at `step`, least recently used first."""
        free = [v for v in range(self.capacity) if self.last_use[v] != step]
        never = [v for v in free if self.last_use[v] < 0]
        used = sorted((v for v in free if self.last_use[v] >= 0), key=lambda v: (self.last_use[v], v))
        return never + used

    def step(self, selected, assign=None):
        """selected: iterable of (request, token).  assign: optional dict
        miss -> victim slot.  Returns (misses, victims, evicted): the misses
        in (request, token) order, the victims in ranking order, and the
        evicted tokens in miss order."""
        step = self.clock + 1
        sel = set(selected)
        for rs in sel:
            if rs in self.slot_of:
                self.last_use[self.slot_of[rs]] = step
        misses = sorted(rs for rs in sel if rs not in self.slot_of)
        ranked = self.rank(step)
        if len(misses) > len(ranked):
            raise ValueError("capacity below the step's distinct selected tokens")
        victims = ranked[:len(misses)]
        if assign is None:
            assign = dict(zip(misses, victims))
        else:
            if set(assign) != set(misses) or sorted(assign.values()) != sorted(victims):
                raise AssertionError("assignment is not a one-to-one map of the misses onto the victims")
        evicted = []
        for rs in misses:
            v = assign[rs]
            old = self.owner[v]
            if old is not None:
                del self.slot_of[old]
                evicted.append(old)
            self.owner[v] = rs
            self.slot_of[rs] = v
            self.last_use[v] = step
        self.clock = step
        return misses, victims, evicted
