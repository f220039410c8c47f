"""Fixed-size HBM page cache over a host-resident KV tier -- TEST INFRASTRUCTURE ONLY.

Oracle of the in-graph cache resolver described on [P2] "HiSparse: Scaling
Sparse Attention Decoding with Hierarchical KV Cache" (abstract, sentence on the
fused resolver, which finds hits, replaces least recently used entries and
fetches misses from the host inside the decode graph; and the sentence on
outputs staying the same because only where KV lives changes).  The pages give no slot or tie rules; the ones below
are this library's reading, stated once here:

* A cache unit is one (logical page, KV head) of one request: its K tile and V
  tile.  unit id = h * max_pages + p.
* Per request and step, the requested set R is the union of that request's
  per-KV-head page lists.  Units of R already resident are hits; they get the
  step number as their stamp.
* Misses, in ascending unit id, take slots in ascending slot index from the
  available set.  If the free slots suffice, the available set is the lowest
  free slots; otherwise it is every free slot plus the r least recently used
  resident units outside R, ordered by (stamp ascending, unit id ascending),
  r = |misses| - |free|.  (This is exact LRU eviction with ties broken by the
  lower unit id; which slot a miss lands in is placement only.)
* If fewer slots can be made available than there are misses, the step sets
  the overflow flag, the misses that got no slot keep slot -1, and the step's
  outputs are not meaningful.

Bucketed LRU ([P3] "Unifying Sparse Attention with Hierarchical Memory for
Scalable Long-Context LLM Serving", the SPIN abstract, technique (2): a
GPU-friendly bucketed LRU policy in the KV cache manager; no bucket rule is
given, so this is this library's reading): with recency shift s, stamps are compared only in
buckets of 2**s steps -- victims are ordered by (stamp >> s, unit id), so
within one bucket the lower unit id goes first.  s = 0 is exact LRU.
"""

from collections import OrderedDict

import numpy as np


class LRUState:
    """Cache state of one request: capacity slots, their unit tags and stamps."""

    def __init__(self, capacity, n_units):
        self.capacity = int(capacity)
        self.tag = np.full(self.capacity, -1, dtype=np.int64)
        self.stamp = np.full(self.capacity, -1, dtype=np.int64)
        self.slot_of = np.full(int(n_units), -1, dtype=np.int64)

    def copy(self):
        c = LRUState(self.capacity, self.slot_of.shape[0])
        c.tag[:] = self.tag
        c.stamp[:] = self.stamp
        c.slot_of[:] = self.slot_of
        return c


def resolve_step(state, requested_units, step, recency_shift=0):
    """Apply one step to ``state`` in place.

    requested_units: iterable of unit ids (duplicates allowed); recency_shift:
    victims are ordered by (stamp >> recency_shift, unit id).  Returns a dict
    with 'hits', 'misses', 'evictions', 'overflow' and 'placed' (list of
    (unit, slot) for the misses, ascending unit id; slot -1 if unplaced).
    """
    R = np.unique(np.asarray(list(requested_units), dtype=np.int64))
    resident = state.slot_of[R] >= 0
    hits = R[resident]
    misses = R[~resident]
    state.stamp[state.slot_of[hits]] = step

    free = np.nonzero(state.tag < 0)[0]
    if misses.size <= free.size:
        avail = free[:misses.size]
    else:
        r = misses.size - free.size
        inR = np.zeros(state.slot_of.shape[0], dtype=bool)
        inR[R] = True
        cand = np.nonzero((state.tag >= 0) & ~inR[np.maximum(state.tag, 0)])[0]
        order = np.lexsort((state.tag[cand], state.stamp[cand] >> int(recency_shift)))
        victims = cand[order[:r]]
        avail = np.sort(np.concatenate([free, victims]))

    evictions = 0
    placed = []
    evicting = []
    for i, u in enumerate(misses):
        if i >= avail.size:
            placed.append((int(u), -1))
            continue
        s = int(avail[i])
        old = state.tag[s]
        if old >= 0:
            state.slot_of[old] = -1
            evictions += 1
            evicting.append(int(u))
        state.tag[s] = u
        state.stamp[s] = step
        state.slot_of[u] = s
        placed.append((int(u), s))
    overflow = int(misses.size > avail.size)
    return {"hits": int(hits.size), "misses": int(misses.size),
            "evictions": evictions, "overflow": overflow, "placed": placed,
            "hit_units": hits, "evicting_units": evicting}


def pooled_unit(b, h, p, kv_heads, max_pages):
    """Unit id in a pool shared by every request: (b * Hkv + h) * max_pages + p."""
    return (b * kv_heads + h) * max_pages + p


def resolve_pooled_step(state, units_per_request, step, units_per_req_space, recency_shift=0):
    """One step of a cache pool shared by all requests ([P3], the SPIN
    abstract, technique (2): per-request HBM budgets sized dynamically -- here
    a request holds as many slots as the pool-wide replacement leaves it).
    The rule is resolve_step's over pooled unit ids (ascending pooled id
    places the misses, so request b's misses precede request b+1's).
    units_per_request[b]: pooled ids requested by request b;
    units_per_req_space = Hkv * max_pages.  Returns resolve_step's dict plus
    'per_request': [B][4] hits, misses, evictions (slots taken from resident
    units by that request's misses), overflow (a miss of that request got no
    slot)."""
    allu = [u for us in units_per_request for u in us]
    r = resolve_step(state, allu, step, recency_shift)
    B = len(units_per_request)
    per = np.zeros((B, 4), dtype=np.int64)
    for u in r["hit_units"]:
        per[int(u) // units_per_req_space, 0] += 1
    for u, s in r["placed"]:
        b = u // units_per_req_space
        per[b, 1] += 1
        if s < 0:
            per[b, 3] = 1
    for u in r["evicting_units"]:
        per[u // units_per_req_space, 2] += 1
    r["per_request"] = per
    return r


def textbook_lru_trace(capacity, steps_units):
    """Plain LRU over an OrderedDict, one step at a time.

    Within a step every requested unit counts as used at that step; units used
    at the same step are ordered by ascending unit id.  Eviction only happens
    when the cache is full and takes the least recently used unit that the
    step does not request.  Returns per step (hits, misses, evictions,
    resident set).
    """
    lru = OrderedDict()
    out = []
    for units in steps_units:
        R = sorted(set(int(u) for u in units))
        Rset = set(R)
        hits = [u for u in R if u in lru]
        misses = [u for u in R if u not in lru]
        ev = 0
        for u in misses:
            if len(lru) >= capacity:
                victim = next((k for k in lru if k not in Rset), None)
                if victim is None:
                    raise OverflowError("more distinct units in one step than slots")
                del lru[victim]
                ev += 1
            lru[u] = True
        for u in R:            # re-insert the step's units in ascending id
            del lru[u]
        for u in R:
            lru[u] = True
        out.append((len(hits), len(misses), ev, frozenset(lru.keys())))
    return out


def textbook_bucketed_trace(capacity, steps_units, shift):
    """Bucketed LRU kept as recency buckets: bucket k holds the resident units
    last used in steps [k * 2**shift, (k + 1) * 2**shift).  A miss in a full
    cache evicts the lowest unit id of the oldest non-empty bucket, among the
    units the step does not request.  Returns per step (hits, misses,
    evictions, resident set)."""
    buckets = {}          # bucket -> set of units
    where = {}            # unit -> bucket
    out = []
    for t, units in enumerate(steps_units):
        R = sorted(set(int(u) for u in units))
        Rset = set(R)
        hits = [u for u in R if u in where]
        misses = [u for u in R if u not in where]
        ev = 0
        for u in misses:
            if len(where) >= capacity:
                victim = None
                for k in sorted(buckets):
                    cands = [v for v in buckets[k] if v not in Rset]
                    if cands:
                        victim = min(cands)
                        break
                if victim is None:
                    raise OverflowError("more distinct units in one step than slots")
                buckets[where.pop(victim)].discard(victim)
                ev += 1
            where[u] = None
        now = t >> shift
        for u in R:
            if where[u] is not None:
                buckets[where[u]].discard(u)
            where[u] = now
            buckets.setdefault(now, set()).add(u)
        out.append((len(hits), len(misses), ev, frozenset(where)))
    return out
