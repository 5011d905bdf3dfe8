"""Reference of the device expert cache's policy, for tests.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.  Written from
"Run Kimi 3.1 locally on one GPU" (argonautlabs.ai): "One GPU, three storage
tiers" (a device expert cache in front of a pinned host pool) and "A drafter
that leaves the answer unchanged" (LRU alone never hits once a block needs
more experts than the cache has room for; admitting only experts with a
minimum row count per block reduces the reads).  The pages give no
slot-level rules; the ones below are this library's, stated in its header.

Per call (one layer, its routed experts ascending, each with its row count):
  1. cached experts are hits and are stamped with the call's tick;
  2. with admission on (r > 0), misses used by fewer than r rows take the
     transient slots 0, 1, ... in order while there are any;
  3. every other miss is admitted into a cached slot: the lowest free one,
     else the one least recently used (lowest index on equal ticks) that no
     expert of this call holds; with none left it takes the next transient
     slot.
A call that does not fit raises ValueError and changes nothing.  Cached slot
c is reported as n_transient + c.
"""
from __future__ import annotations


class CachePolicyRef:
    def __init__(self, n_layers: int, n_routed: int, n_cache: int, n_transient: int, admit_min_rows: int):
        self.n_layers, self.n_routed = n_layers, n_routed
        self.n_cache, self.n_transient, self.admit = n_cache, n_transient, admit_min_rows
        self.where = {}                      # (layer, expert) -> cached slot
        self.holder = [None] * n_cache       # cached slot -> (layer, expert)
        self.last = [0] * n_cache            # cached slot -> tick of last use
        self.tick = 0

    def plan(self, layer: int, experts, rows):
        experts, rows = list(experts), list(rows)
        held = [e for e in experts if (layer, e) in self.where]
        missing = [(e, r) for e, r in zip(experts, rows) if (layer, e) not in self.where]
        n_bypass = 0
        if self.admit > 0:
            n_bypass = min(sum(1 for _, r in missing if r < self.admit), self.n_transient)
        if len(missing) - n_bypass > (self.n_cache - len(held)) + (self.n_transient - n_bypass):
            raise ValueError("the call's experts do not fit the cache")
        self.tick += 1
        this_call = set()
        slot, hit, admitted = {}, {}, {}
        for e in held:
            c = self.where[(layer, e)]
            self.last[c] = self.tick
            this_call.add(c)
            slot[e], hit[e], admitted[e] = self.n_transient + c, 1, 0
        t = 0
        if self.admit > 0:
            for e, r in missing:
                if r < self.admit and t < self.n_transient:
                    slot[e], hit[e], admitted[e] = t, 0, 0
                    t += 1
        for e, r in missing:
            if e in slot:
                continue
            free = [c for c in range(self.n_cache) if self.holder[c] is None]
            if free:
                c = free[0]
            else:
                old = [c for c in range(self.n_cache) if c not in this_call]
                c = min(old, key=lambda c: (self.last[c], c)) if old else None
            if c is None:
                slot[e], hit[e], admitted[e] = t, 0, 0
                t += 1
                continue
            if self.holder[c] is not None:
                del self.where[self.holder[c]]
            self.holder[c] = (layer, e)
            self.where[(layer, e)] = c
            self.last[c] = self.tick
            this_call.add(c)
            slot[e], hit[e], admitted[e] = self.n_transient + c, 0, 1
        return ([slot[e] for e in experts], [hit[e] for e in experts], [admitted[e] for e in experts])
