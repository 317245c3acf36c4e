"""Per-layer VRAM expert-slot cache with least-recently-used replacement.

[39TOK] section "设计核心": a global LRU cache of experts in VRAM catches the
routing overlap of adjacent tokens; what misses is filled into the GPU cache.
[753B] section "按带宽动态分配参数存储": frequently used experts stay resident,
the rest are fetched on demand.  The pages give no further policy detail; the
batch-aware rule below is a stated reading (one pool per layer, cold start):

* One pool of S slots per layer over E experts; it starts cold (all empty).
* A step presents T*k accesses in pair order q = t*k + j.
* Hits are classified against the state at the start of the step.
* Each distinct missed expert (in order of first appearance) takes one victim
  slot.  Victims come only from slots whose expert is not requested in this
  step: first the empty slots in ascending index, then occupied slots in
  ascending last-use stamp.  Too few candidates -> capacity error, state kept.
* Every access, in pair order, advances the clock by one and stamps its slot.
* Hit rate = (accesses - distinct misses) / accesses: a repeated access to an
  expert filled earlier in the same step counts as a hit.

Elastic resize ([39TOK] section "设计核心", the third mechanism: at a scheduler
safe point the GPU expert cache is resized to the memory at hand and rebuilt,
with no restart and no reload of the host-resident expert pool).  The pages
give no rule for which experts survive or where they go; the stated reading:

* Between steps, the pool goes from S to S' slots.  The min(S', resident)
  experts with the latest last use are kept; the others leave the cache.
* A kept expert whose slot is below S' keeps it.  The other kept experts take
  the lowest free slots below S', in ascending order of their old slot.
* Stamps and the clock are unchanged; slots added by growing start empty.
* The blob copies this implies: every kept blob into a new pool, or, rebuilding
  the same pool in place, only the blobs that change slot (from slots >= S'
  into free slots < S', so no copy reads what another writes).

``StampLRU`` is the form the GPU kernel implements (four arrays).  ``ListLRU``
is an independent move-to-MRU list simulation of the same policy; the tests
require both to give identical slot tables at every step.
"""

import numpy as np

OK = 0
E_CAPACITY = -3


def _unique_in_order(seq):
    seen, out = set(), []
    for e in seq:
        if e not in seen:
            seen.add(e)
            out.append(e)
    return out


class StampLRU:
    def __init__(self, E: int, S: int):
        self.E, self.S = E, S
        self.slot_expert = np.full(S, -1, dtype=np.int32)
        self.expert_slot = np.full(E, -1, dtype=np.int32)
        self.slot_stamp = np.zeros(S, dtype=np.int64)
        self.clock = 0

    def state(self):
        return (self.slot_expert.copy(), self.expert_slot.copy(),
                self.slot_stamp.copy(), int(self.clock))

    def step(self, pair_experts):
        pair_experts = [int(e) for e in np.asarray(pair_experts).ravel()]
        n = len(pair_experts)
        requested = set(pair_experts)
        uniq = _unique_in_order(pair_experts)
        resident_at_start = {e for e in uniq if self.expert_slot[e] >= 0}
        misses = [e for e in uniq if e not in resident_at_start]
        cand = [s for s in range(self.S)
                if self.slot_expert[s] < 0 or int(self.slot_expert[s]) not in requested]
        cand.sort(key=lambda s: (0 if self.slot_expert[s] < 0 else 1,
                                 int(self.slot_stamp[s]), s))
        if len(cand) < len(misses):
            return dict(status=E_CAPACITY, n_miss=len(misses))
        victims = cand[:len(misses)]
        for e, s in zip(misses, victims):
            old = int(self.slot_expert[s])
            if old >= 0:
                self.expert_slot[old] = -1
            self.slot_expert[s] = e
            self.expert_slot[e] = s
        for e in pair_experts:
            self.clock += 1
            self.slot_stamp[self.expert_slot[e]] = self.clock
        pair_slot = np.array([self.expert_slot[e] for e in pair_experts], dtype=np.int32)
        hit_pairs = [q for q, e in enumerate(pair_experts) if e in resident_at_start]
        miss_pairs = [q for q, e in enumerate(pair_experts) if e not in resident_at_start]
        return dict(status=OK, pair_slot=pair_slot,
                    pair_order=np.array(hit_pairs + miss_pairs, dtype=np.int32),
                    n_hit_pairs=len(hit_pairs), n_miss=len(misses),
                    miss_expert=np.array(misses, dtype=np.int32),
                    miss_slot=np.array(victims, dtype=np.int32),
                    n_hits=n - len(misses), n_access=n)


def _placement(kept_slots, S_new):
    """Old slot -> new slot for the kept slots (the placement rule above)."""
    stay = sorted(s for s in kept_slots if s < S_new)
    movers = sorted(s for s in kept_slots if s >= S_new)
    taken = set(stay)
    free = [t for t in range(S_new) if t not in taken]
    new_of = {s: s for s in stay}
    new_of.update(zip(movers, free))
    return new_of, movers


def stamp_resize(lru, S_new):
    """Resize a StampLRU to S_new slots; returns the copy plans as lists of
    (old slot, new slot): ``all`` for a new pool, ``in_place`` for the same pool."""
    occupied = [s for s in range(lru.S) if lru.slot_expert[s] >= 0]
    # latest stamp first; equal stamps (not produced by step) take the lower slot first
    kept = sorted(occupied, key=lambda s: (-int(lru.slot_stamp[s]), s))[:S_new]
    new_of, movers = _placement(kept, S_new)
    se = np.full(S_new, -1, dtype=np.int32)
    st = np.zeros(S_new, dtype=np.int64)
    es = np.full(lru.E, -1, dtype=np.int32)
    for s, t in new_of.items():
        e = int(lru.slot_expert[s])
        se[t], st[t], es[e] = e, lru.slot_stamp[s], t
    plan_all = [(s, new_of[s]) for s in sorted(new_of)]
    plan_in_place = [(s, new_of[s]) for s in movers]
    lru.S, lru.slot_expert, lru.slot_stamp, lru.expert_slot = S_new, se, st, es
    return dict(all=plan_all, in_place=plan_in_place)


StampLRU.resize = stamp_resize


class ListLRU:
    """Move-to-MRU list form of the same policy (independent formulation)."""

    def __init__(self, E: int, S: int):
        self.E, self.S = E, S
        self.recency = []            # resident experts, least recent first
        self.slot_of = {}            # expert -> slot

    def slot_table(self):
        se = np.full(self.S, -1, dtype=np.int32)
        for e, s in self.slot_of.items():
            se[s] = e
        return se

    def step(self, pair_experts):
        pair_experts = [int(e) for e in np.asarray(pair_experts).ravel()]
        requested = set(pair_experts)
        uniq = _unique_in_order(pair_experts)
        misses = [e for e in uniq if e not in self.slot_of]
        used = set(self.slot_of.values())
        victims = [s for s in range(self.S) if s not in used][:len(misses)]
        evict = []
        if len(victims) < len(misses):
            for e in self.recency:               # from the least-recent end
                if len(victims) + len(evict) == len(misses):
                    break
                if e not in requested:
                    evict.append(e)
            if len(victims) + len(evict) < len(misses):
                return dict(status=E_CAPACITY)
        for e in evict:
            victims.append(self.slot_of.pop(e))
            self.recency.remove(e)
        for e, s in zip(misses, victims):
            self.slot_of[e] = s
        for e in pair_experts:                   # each access moves to MRU
            if e in self.recency:
                self.recency.remove(e)
            self.recency.append(e)
        return dict(status=OK,
                    pair_slot=np.array([self.slot_of[e] for e in pair_experts], dtype=np.int32),
                    n_miss=len(misses), miss_expert=np.array(misses, dtype=np.int32),
                    miss_slot=np.array(victims, dtype=np.int32))


def _list_resize(lru, S_new):
    """The same resize on the move-to-MRU list: the last S_new entries of the
    recency list survive, and placement follows the same stated rule."""
    kept = lru.recency[max(0, len(lru.recency) - S_new):]
    keep = set(kept)
    old = {e: s for e, s in lru.slot_of.items() if e in keep}
    order = sorted(old.items(), key=lambda es: es[1])          # by old slot
    new = {e: s for e, s in order if s < S_new}
    used = set(new.values())
    holes = (t for t in range(S_new) if t not in used)
    for e, s in order:
        if s >= S_new:
            new[e] = next(holes)
    lru.recency = list(kept)
    lru.slot_of = new
    lru.S = S_new


ListLRU.resize = _list_resize


class LayerView:
    """One layer's view of a cache shared by several layers ([39TOK] section
    "设计核心": the expert cache is one global LRU; the stated reading of its
    cross-layer form).  The shared state is keyed by (layer, expert): layer j's
    expert e is key key_base + e, with key_base = j * experts; each layer's
    lookup is one step of the shared policy on its own keys, so victims may be
    any slot the step does not request, whichever layer filled it.  Records
    name the layer's experts, not keys.  ``lru`` is a StampLRU or a ListLRU over
    all the keys (E = layers * experts)."""

    def __init__(self, lru, key_base: int):
        self.lru, self.key_base = lru, key_base

    def step(self, pair_experts):
        keys = [self.key_base + int(e) for e in np.asarray(pair_experts).ravel()]
        r = self.lru.step(keys)
        if r["status"] == OK:
            r["miss_expert"] = np.asarray(r["miss_expert"], dtype=np.int32) - self.key_base
        return r


def prefetch_step(lru, ranked):
    """Predictive prefetch after a layer's routed step ([753B] section
    "按带宽动态分配参数存储": copies guided by the gate's routing run ahead of
    use; the pages give no predictor, so the stated reading takes the token's
    runner-up experts).  ``ranked`` is the token's top-(k+m) experts in rank
    order, the first k being the ones just routed.  The rule is one more step
    of the same policy over that list: the routed experts are hits and are
    restamped in rank order, each runner-up that misses takes a victim by the
    usual rule (so never a slot of this list) and is stamped after them.  The
    step's misses are the prefetched experts; ``lru`` is a StampLRU or a
    ListLRU."""
    return lru.step(list(ranked))


def simulate_hit_rate(steps, E: int, S: int, skip: int = 0):
    """Hit rate of a sequence of per-step access lists (steps >= skip counted)."""
    lru = StampLRU(E, S)
    hits = acc = 0
    for i, s in enumerate(steps):
        r = lru.step(s)
        if r["status"] != OK:
            raise RuntimeError("capacity")
        if i >= skip:
            hits += r["n_hits"]
            acc += r["n_access"]
    return hits / max(acc, 1)
