"""Delta-cache policy oracle: which variant's packed delta lives in which
device slot, what a request does, which variant is evicted.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain Python, one
request at a time, no arithmetic beyond integer counts.

Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
"Altyapı ayrıntıları" (infrastructure details), the cold-start, eviction and
routing paragraphs:

* a variant whose delta is not resident pays one load from host storage into
  device memory on its first request; afterwards it stays resident until the
  eviction policy removes it;
* eviction is least-recently-used, weighted by request rate: the variants
  with the highest request rate are pinned (the page keeps the top 6 of 14
  resident at all times), the others share the remaining slots under LRU;
* the router tracks in-flight loads per variant: while a variant's delta is
  loading, further requests for it queue behind that load instead of each
  starting a load of its own.

Readings taken where the page leaves the rule open:

* Request rate is an integer request count per variant that is halved
  (shift right by one, all variants at once) after every `halve_every`-th
  request; `halve_every = 0` never halves, which makes it the traffic volume
  so far.  The request being served is counted first, then the halving (if
  due) applies, then the pinned set is formed.
* The pinned set is the `n_pinned` variants with the highest rate, ties to
  the lower variant id.  Being pinned protects a resident variant from
  eviction; it does not reserve a slot for a variant that is not resident.
* A miss takes the lowest-numbered free slot; with none free it evicts the
  least recently requested variant among those that are resident, not
  pinned, not in use (every request that returned it has been released) and
  not the requested one.  A variant still loading is never evicted.
* If nothing can be evicted the request is refused (FULL) and changes no
  state at all: the caller retries it later and only the retry is counted.
* "Recently" is the logical time of the variant's latest counted request.
"""

from __future__ import annotations

HIT = 0      # resident and loaded: use the slot now
QUEUED = 1   # a load of this variant is in flight: wait for it, start none
LOAD = 2     # this request starts the load into the returned slot
FULL = 3     # no slot can be freed now; nothing changed

ABSENT = 0
LOADING = 1
RESIDENT = 2


class CachePolicy:
    """State of one cache of `n_slots` slots serving `n_variants` variants."""

    def __init__(self, n_variants: int, n_slots: int, n_pinned: int, halve_every: int = 0):
        if not (n_variants >= 1 and n_slots >= 1 and 0 <= n_pinned < n_slots
                and halve_every >= 0):
            raise ValueError("need n_variants >= 1, n_slots >= 1, 0 <= n_pinned < n_slots")
        self.V, self.S, self.P, self.H = n_variants, n_slots, n_pinned, halve_every
        self.time = 0
        self.rate = [0] * n_variants
        self.last = [-1] * n_variants
        self.state = [ABSENT] * n_variants
        self.slot = [-1] * n_variants
        self.users = [0] * n_variants
        self.owner = [-1] * n_slots

    def pinned(self) -> set:
        order = sorted(range(self.V), key=lambda u: (-self.rate[u], u))
        return set(order[:self.P])

    def request(self, v: int):
        """One request for variant v: (action, slot, evicted variant or -1)."""
        if not 0 <= v < self.V:
            raise ValueError("variant out of range")
        if self.state[v] == ABSENT and -1 not in self.owner:
            # would the request find a victim once it is counted?
            if self._victim(v, self._rates_after(v)) is None:
                return FULL, -1, -1
        self._count(v)
        if self.state[v] == RESIDENT:
            self.users[v] += 1
            return HIT, self.slot[v], -1
        if self.state[v] == LOADING:
            self.users[v] += 1
            return QUEUED, self.slot[v], -1
        evicted = -1
        if -1 in self.owner:
            s = self.owner.index(-1)
        else:
            evicted = self._victim(v, self.rate)
            s = self.slot[evicted]
            self.state[evicted] = ABSENT
            self.slot[evicted] = -1
        self.owner[s] = v
        self.slot[v] = s
        self.state[v] = LOADING
        self.users[v] += 1
        return LOAD, s, evicted

    def loaded(self, v: int) -> None:
        if self.state[v] != LOADING:
            raise ValueError("variant is not loading")
        self.state[v] = RESIDENT

    def release(self, v: int) -> None:
        if self.users[v] <= 0:
            raise ValueError("variant is not in use")
        self.users[v] -= 1

    # ------------------------------------------------------------------ helpers
    def _rates_after(self, v):
        rate = list(self.rate)
        rate[v] += 1
        if self.H and (self.time + 1) % self.H == 0:
            rate = [r >> 1 for r in rate]
        return rate

    def _count(self, v):
        self.rate = self._rates_after(v)
        self.time += 1
        self.last[v] = self.time

    def _victim(self, v, rate):
        order = sorted(range(self.V), key=lambda u: (-rate[u], u))
        pinned = set(order[:self.P])
        best = None
        for u in range(self.V):
            if (u != v and self.state[u] == RESIDENT and self.users[u] == 0
                    and u not in pinned):
                if best is None or self.last[u] < self.last[best]:
                    best = u
        return best


class Router:
    """Decode batches fed from a request queue over a CachePolicy.

    Page section "Altyapı ayrıntıları", the routing paragraph: the router
    keeps track of the requests in flight per variant and avoids head-of-line
    blocking; requests for a variant whose delta is loading wait for that one
    load.  Reading taken:

    * a request registers with the cache once, the first time a batch is
      formed after it arrived (so the cache counts it once); a FULL refusal
      leaves it unregistered, to be tried again at the next batch;
    * a registered request is ready once its variant is resident; a request
      for the base model alone (variant -1) is ready at once and never
      touches the cache;
    * a batch takes the ready requests in arrival order, at most max_batch:
      a later request whose variant is resident does not wait behind an
      earlier one whose variant is still loading;
    * completing a batch releases each served request's variant.
    """

    NEW, WAITING, READY = 0, 1, 2

    def __init__(self, cache: CachePolicy):
        self.cache = cache
        self.queue = []          # [request id, variant, state, slot] in arrival order

    def submit(self, rid: int, variant: int) -> None:
        if not -1 <= variant < self.cache.V:
            raise ValueError("variant out of range")
        self.queue.append([rid, variant, self.READY if variant < 0 else self.NEW, -1])

    def next_batch(self, max_batch: int):
        """[(request id, variant, slot)] of the next batch, slot -1 for the base."""
        if max_batch < 1:
            raise ValueError("max_batch must be positive")
        for r in self.queue:
            if r[2] == self.NEW:
                act, slot, _ = self.cache.request(r[1])
                if act != FULL:
                    r[2] = self.READY if act == HIT else self.WAITING
                    r[3] = slot
        for r in self.queue:
            if r[2] == self.WAITING and self.cache.state[r[1]] == RESIDENT:
                r[2] = self.READY
        batch, rest = [], []
        for r in self.queue:
            if r[2] == self.READY and len(batch) < max_batch:
                batch.append((r[0], r[1], r[3]))
            else:
                rest.append(r)
        self.queue = rest
        return batch

    def complete(self, batch) -> None:
        for _, v, _ in batch:
            if v >= 0:
                self.cache.release(v)
