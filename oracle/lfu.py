"""LFU expert-slot cache simulator (one instance per layer).

The pages fix a per-layer expert cache of 16 slots managed by an LFU policy
("Como executar um modelo de 26 bilhões de parâmetros ...", section "Qual é
o principal truque da arquitetura"; "Show HN: mecanismo de código aberto
executando Gemma 4 26B em 2 GB de RAM", section "Abordagem técnica", which
adds that more slots use more memory and that the hit rate is ~60-70 %).
They do not fix tie-breaks. Reading taken (so that a trace is unique):

* state per slot: (expert or EMPTY, freq, last);
* a token's ids are looked up in rank order; a resident id is a hit:
  freq += 1, last = tick;
* a missing id takes the lowest-index EMPTY slot if there is one, else the
  slot minimising (freq, last, slot index) among slots that hold none of this
  token's ids; the new entry starts at freq 1, last = tick;
* frequencies count token-steps while resident and restart on eviction; no
  ageing; the cache starts empty; the tick is the step number;
* hits are settled before misses, but events are reported in rank order.

Policy variant for comparisons (not the pages' policy): with policy="lru" the
victim minimises (last, slot index) instead; everything else is unchanged.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

EMPTY = -1


class LFUCache:
    def __init__(self, n_slots: int, n_experts: int, policy: str = "lfu"):
        if n_slots < 1:
            raise ValueError("need at least one slot")
        if policy not in ("lfu", "lru"):
            raise ValueError("policy must be 'lfu' or 'lru'")
        self.policy = policy
        self.n_slots = n_slots
        self.n_experts = n_experts
        self.expert = [EMPTY] * n_slots
        self.freq = [0] * n_slots
        self.last = [-1] * n_slots
        self.tick = 0
        self.hits = 0
        self.misses = 0

    def slot_of(self, e: int) -> int:
        for s in range(self.n_slots):
            if self.expert[s] == e:
                return s
        return -1

    def step(self, ids):
        """Process one token's expert ids (rank order).

        Returns one event per id, in rank order: (expert, slot, hit, evicted),
        with evicted = -1 when the slot was empty or on a hit.
        """
        ids = [int(i) for i in ids]
        if len(set(ids)) != len(ids):
            raise ValueError("duplicate expert id in one token")
        if len(ids) > self.n_slots:
            raise ValueError("more ids than slots")
        if any(i < 0 or i >= self.n_experts for i in ids):
            raise ValueError("expert id out of range")
        t = self.tick
        events = [None] * len(ids)
        for j, e in enumerate(ids):
            s = self.slot_of(e)
            if s >= 0:
                self.freq[s] += 1
                self.last[s] = t
                events[j] = (e, s, 1, -1)
                self.hits += 1
        wanted = set(ids)
        for j, e in enumerate(ids):
            if events[j] is not None:
                continue
            empties = [s for s in range(self.n_slots) if self.expert[s] == EMPTY]
            if empties:
                victim = empties[0]
            else:
                cands = [s for s in range(self.n_slots) if self.expert[s] not in wanted]
                if self.policy == "lru":
                    victim = min(cands, key=lambda s: (self.last[s], s))
                else:
                    victim = min(cands, key=lambda s: (self.freq[s], self.last[s], s))
            old = self.expert[victim]
            self.expert[victim] = e
            self.freq[victim] = 1
            self.last[victim] = t
            events[j] = (e, victim, 0, old)
            self.misses += 1
        self.tick += 1
        return events


def simulate(id_rows, n_slots: int, n_experts: int, policy: str = "lfu"):
    """Run a whole id trace; returns (events per step, cache)."""
    c = LFUCache(n_slots, n_experts, policy)
    return [c.step(r) for r in id_rows], c
