"""Delta-cache policy: the oracle pinned against hand-derived traces and a
textbook LRU, then the library's native policy (C ABI, host only, no GPU)
checked against the oracle decision by decision on synthetic Zipf traces."""

import collections
import ctypes
import os

import numpy as np
import pytest

from oracle import cache_policy as CP

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_traces.txt")
ACTIONS = {"HIT": CP.HIT, "QUEUED": CP.QUEUED, "LOAD": CP.LOAD, "FULL": CP.FULL}


def read_traces():
    """The policy traces ("trace" blocks; "router" blocks are skipped)."""
    traces, cur, skip = [], None, False
    for raw in open(GOLDEN):
        line = raw.split("#", 1)[0].split()
        if not line:
            continue
        if line[0] == "router":
            skip = True
        elif skip:
            skip = line[0] != "end"
        elif line[0] == "trace":
            cur = (tuple(int(t) for t in line[1:5]), [])
        elif line[0] == "end":
            traces.append(cur)
            cur = None
        elif line[0] == "req":
            cur[1].append(("req", int(line[1]), ACTIONS[line[2]], int(line[3]), int(line[4])))
        else:
            cur[1].append((line[0], int(line[1])))
    return traces


def zipf_trace(n, n_variants, seed, a=1.1):
    rng = np.random.default_rng(seed)
    p = np.arange(1, n_variants + 1, dtype=np.float64) ** -a
    return rng.choice(n_variants, size=n, p=p / p.sum())


# ---------------------------------------------------------------- oracle pins
def test_oracle_golden_traces():
    traces = read_traces()
    assert len(traces) == 3
    for (V, S, P, H), steps in traces:
        c = CP.CachePolicy(V, S, P, H)
        for st in steps:
            if st[0] == "req":
                assert c.request(st[1]) == st[2:], (V, S, P, H, st)
            elif st[0] == "loaded":
                c.loaded(st[1])
            else:
                c.release(st[1])


@pytest.mark.parametrize("S", [1, 2, 3, 5])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_without_pinning_is_textbook_lru(S, seed):
    """No pinned variants, loads that finish at once, every request released
    at once: hits, misses and victims are those of an LRU cache of S entries
    (collections.OrderedDict)."""
    V = 8
    c = CP.CachePolicy(V, S, 0, 0)
    lru = collections.OrderedDict()
    for v in zipf_trace(400, V, seed):
        v = int(v)
        act, slot, ev = c.request(v)
        if v in lru:
            lru.move_to_end(v)
            assert (act, ev) == (CP.HIT, -1)
        else:
            want_ev = -1
            if len(lru) == S:
                want_ev, _ = lru.popitem(last=False)
            lru[v] = True
            assert (act, ev) == (CP.LOAD, want_ev)
            c.loaded(v)
        c.release(v)


@pytest.mark.parametrize("P", [0, 3, 6])
def test_oracle_room_for_all_loads_each_variant_once(P):
    """With a slot for every variant only the first request of each loads."""
    V = 14
    c = CP.CachePolicy(V, V, P, 16)
    seen = set()
    for v in zipf_trace(500, V, 5):
        v = int(v)
        act, slot, ev = c.request(v)
        assert ev == -1
        if v in seen:
            assert act in (CP.HIT, CP.QUEUED)
        else:
            assert act == CP.LOAD and slot == len(seen)
            seen.add(v)
        if act == CP.LOAD:
            c.loaded(v)
        c.release(v)


def test_oracle_requests_queue_behind_one_load():
    c = CP.CachePolicy(4, 2, 1, 0)
    assert c.request(3) == (CP.LOAD, 0, -1)
    for _ in range(5):
        assert c.request(3) == (CP.QUEUED, 0, -1)
    c.loaded(3)
    assert c.request(3) == (CP.HIT, 0, -1)


def test_oracle_full_changes_nothing():
    c = CP.CachePolicy(3, 1, 0, 0)
    assert c.request(0) == (CP.LOAD, 0, -1)
    c.loaded(0)
    before = (c.time, list(c.rate), list(c.last))
    assert c.request(1) == (CP.FULL, -1, -1)   # variant 0 still in use
    assert (c.time, c.rate, c.last) == before
    c.release(0)
    assert c.request(1) == (CP.LOAD, 0, 0)


def test_oracle_pinned_top_variants_never_evicted():
    """Zipf traffic over 14 variants with 8 slots and the top 6 pinned (the
    page's split): every victim is outside the top 6 by the request counts
    kept here independently of the oracle."""
    V, S, P = 14, 8, 6
    c = CP.CachePolicy(V, S, P, 0)
    counts = [0] * V
    last = [0] * V
    for t, v in enumerate(zipf_trace(3000, V, 11), start=1):
        v = int(v)
        act, slot, ev = c.request(v)
        counts[v] += 1
        last[v] = t
        if ev >= 0:
            top = sorted(range(V), key=lambda u: (-counts[u], u))[:P]
            assert ev not in top
            # the victim is the least recently requested resident outsider
            others = [u for u in range(V) if c.state[u] == CP.RESIDENT and u not in top
                      and u != v]
            assert all(last[ev] < last[u] for u in others)
        if act == CP.LOAD:
            c.loaded(v)
        c.release(v)
    top = sorted(range(V), key=lambda u: (-counts[u], u))[:P]
    assert all(c.state[u] == CP.RESIDENT for u in top)


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        CP.CachePolicy(4, 2, 2, 0)
    c = CP.CachePolicy(4, 2, 1, 0)
    with pytest.raises(ValueError):
        c.request(4)
    with pytest.raises(ValueError):
        c.loaded(0)
    with pytest.raises(ValueError):
        c.release(0)


# ------------------------------------------------- library policy vs the oracle
def _lib_cache(V, S, P, H):
    import tenant_linear_layers_amd as T
    return T.DeltaCache(V, S, P, H)


def test_library_golden_traces():
    for (V, S, P, H), steps in read_traces():
        c = _lib_cache(V, S, P, H)
        for st in steps:
            if st[0] == "req":
                assert c.request(st[1]) == st[2:], (V, S, P, H, st)
            elif st[0] == "loaded":
                c.loaded(st[1])
            else:
                c.release(st[1])


@pytest.mark.parametrize("V,S,P,H", [(14, 8, 6, 0), (14, 8, 6, 64), (14, 4, 2, 7),
                                     (5, 1, 0, 0), (30, 10, 3, 100), (3, 5, 4, 1)])
@pytest.mark.parametrize("seed", [0, 1])
def test_library_matches_oracle_on_zipf_traffic(V, S, P, H, seed):
    """Every decision of the native policy equals the oracle's on Zipf(1.1)
    traffic with loads that finish out of order after random delays and
    uses released in random order (FULL refusals included)."""
    rng = np.random.default_rng(1000 * seed + V)
    lib_c = _lib_cache(V, S, P, H)
    orc = CP.CachePolicy(V, S, P, H)
    loading, in_use = [], []
    seen = collections.Counter()
    for v in zipf_trace(1500, V, seed):
        v = int(v)
        got = lib_c.request(v)
        want = orc.request(v)
        assert got == want, (v, got, want)
        seen[want[0]] += 1
        if want[0] != CP.FULL:
            in_use.append(v)
            if want[0] == CP.LOAD:
                loading.append(v)
        # finish some loads, end some uses, in random order
        for _ in range(int(rng.integers(0, 3))):
            if loading:
                u = loading.pop(int(rng.integers(len(loading))))
                lib_c.loaded(u)
                orc.loaded(u)
        for _ in range(int(rng.integers(0, 3))):
            if in_use:
                u = in_use.pop(int(rng.integers(len(in_use))))
                lib_c.release(u)
                orc.release(u)
        if rng.random() < 0.05:
            u = int(rng.integers(V))
            assert lib_c.state(u) == (orc.state[u], orc.slot[u], orc.rate[u])
    print(dict(seen))
    assert seen[CP.LOAD] and seen[CP.HIT] and seen[CP.QUEUED]
    if S < V:
        assert seen[CP.FULL]   # refusals were exercised too


def test_library_rejects_bad_calls():
    import tenant_linear_layers_amd as T
    for args in [(0, 2, 0, 0), (4, 0, 0, 0), (4, 2, 2, 0), (4, 2, -1, 0), (4, 2, 1, -1)]:
        with pytest.raises(T.BitDeltaError) as e:
            T.DeltaCache(*args)
        assert e.value.status == 10
    c = T.DeltaCache(4, 2, 1, 0)
    for call in (lambda: c.request(4), lambda: c.request(-1), lambda: c.loaded(0),
                 lambda: c.release(0), lambda: c.state(9)):
        with pytest.raises(T.BitDeltaError) as e:
            call()
        assert e.value.status == 10
    with pytest.raises(RuntimeError):
        c.acquire(0, None)


def test_library_attach_argument_checks():
    """attach validates its arguments before any HIP call (these addresses
    are never dereferenced)."""
    import tenant_linear_layers_amd as T
    L = T.lib()
    c = T.DeltaCache(2, 2, 0, 0)
    slots = (ctypes.c_void_p * 2)(0x100000, 0x200000)
    srcs = (ctypes.c_void_p * 2)(0x300000, 0x400000)
    small = (ctypes.c_size_t * 2)(64, 64)
    big = (ctypes.c_size_t * 2)(64, 4096)
    cast = lambda a: ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    assert L.bitdelta_cache_attach(c._h, cast(slots), 1024, cast(srcs), cast(big)) == 10
    bad = (ctypes.c_void_p * 2)(0x100008, 0x200000)
    assert L.bitdelta_cache_attach(c._h, cast(bad), 1024, cast(srcs), cast(small)) == 3
    over = (ctypes.c_void_p * 2)(0x100000, 0x100200)
    assert L.bitdelta_cache_attach(c._h, cast(over), 1024, cast(srcs), cast(small)) == 9
    nul = (ctypes.c_void_p * 2)(0x100000, None)
    assert L.bitdelta_cache_attach(c._h, cast(nul), 1024, cast(srcs), cast(small)) == 1
    c.request(0)   # a request was made: attaching afterwards is refused
    assert L.bitdelta_cache_attach(c._h, cast(slots), 1024, cast(srcs), cast(small)) == 10
    assert L.bitdelta_cache_poll(c._h, None) == 10


def test_delta_layout_offsets():
    import tenant_linear_layers_amd as T
    offs, total = T.delta_layout([(10240, 8192), (8192, 8192), (28672, 8192), (28672, 8192),
                                  (8192, 28672)], T.ALPHA_PER_ROW)
    packed = sum(a * b // 8 for a, b in [(10240, 8192), (8192, 8192), (28672, 8192),
                                         (28672, 8192), (8192, 28672)])
    assert packed == 106_954_752            # one 70B-shaped layer, n/8 bytes
    assert all(p % 256 == 0 and a % 256 == 0 for p, a in offs)
    assert packed < total <= packed + 4 * 83968 + 10 * 256
    import torch
    buf = torch.zeros(total, dtype=torch.uint8)
    views = T.delta_views(buf, [(10240, 8192), (8192, 8192), (28672, 8192), (28672, 8192),
                                (8192, 28672)], T.ALPHA_PER_ROW)
    assert [tuple(p.shape) for p, _ in views][0] == (10240, 128)
    assert [a.numel() for _, a in views] == [10240, 8192, 28672, 28672, 8192]


# ------------------------------------------------------------------ router
def read_router_traces():
    traces, cur = [], None
    for raw in open(GOLDEN):
        line = raw.split("#", 1)[0].split()
        if not line:
            continue
        if line[0] == "router":
            cur = (tuple(int(t) for t in line[1:5]), [])
        elif line[0] == "trace":
            cur = None
        elif cur is None:
            continue
        elif line[0] == "end":
            traces.append(cur)
            cur = None
        elif line[0] == "batch":
            want = [tuple(int(f) for f in item.split(":")) for item in line[3:]]
            cur[1].append(("batch", int(line[1]), want))
        elif line[0] == "submit":
            cur[1].append(("submit", int(line[1]), int(line[2])))
        elif line[0] == "loaded":
            cur[1].append(("loaded", int(line[1])))
        else:
            cur[1].append(("complete",))
    return traces


def run_router_trace(make, steps):
    cache, router = make()
    open_batches = []
    for st in steps:
        if st[0] == "submit":
            router.submit(st[1], st[2])
        elif st[0] == "loaded":
            cache.loaded(st[1])
        elif st[0] == "batch":
            got = router.next_batch(st[1])
            assert [tuple(b) for b in got] == st[2], (st, got)
            open_batches.append(got)
        else:
            router.complete(open_batches.pop())


def test_router_oracle_golden_traces():
    traces = read_router_traces()
    assert len(traces) == 2
    for (V, S, P, H), steps in traces:
        def make():
            c = CP.CachePolicy(V, S, P, H)
            return c, CP.Router(c)
        run_router_trace(make, steps)


def test_router_oracle_properties_on_zipf_traffic():
    """Every request is served exactly once, only when its variant is
    resident, ready requests leave in arrival order, each request is counted
    by the cache once, and with room for every variant and instant loads the
    batches are plain arrival-order chunks."""
    V = 14
    rng = np.random.default_rng(21)
    for S_, P in ((14, 6), (8, 6), (4, 2)):
        c = CP.CachePolicy(V, S_, P, 0)
        r = CP.Router(c)
        served, submitted, counted = [], [], [0] * V
        rid = 0
        for step in range(400):
            for _ in range(int(rng.integers(0, 4))):
                v = int(zipf_trace(1, V, 1000 * step + rid)[0]) if rng.random() > 0.1 else -1
                r.submit(rid, v)
                submitted.append((rid, v))
                rid += 1
            for u in range(V):          # loads finish at random
                if c.state[u] == CP.LOADING and rng.random() < 0.5:
                    c.loaded(u)
            batch = r.next_batch(int(rng.integers(1, 9)))
            order = [b[0] for b in batch]
            assert order == sorted(order)
            for b_rid, v, slot in batch:
                if v >= 0:
                    assert c.state[v] == CP.RESIDENT and c.slot[v] == slot
            served.extend(order)
            r.complete(batch)
        assert len(served) == len(set(served))
        assert set(served) <= {i for i, _ in submitted}
        for i, v in submitted:
            if v >= 0 and (i in served or any(q[0] == i and q[2] != CP.Router.NEW
                                               for q in r.queue)):
                counted[v] += 1
        assert counted == c.rate            # no halving: rate = registered requests
    # room for all and instant loads: arrival-order chunks
    c = CP.CachePolicy(V, V, 0, 0)
    r = CP.Router(c)
    for i in range(37):
        r.submit(i, i % V)
    served = []
    for _ in range(20):
        b = r.next_batch(8)          # the first call registers everything and serves nothing
        for u in range(V):
            if c.state[u] == CP.LOADING:
                c.loaded(u)
        if b:
            served.append([x[0] for x in b])
            r.complete(b)
    flat = [i for chunk in served for i in chunk]
    assert flat == list(range(37)) and all(len(ch) == 8 for ch in served[:-1])


def test_router_library_golden_traces():
    import tenant_linear_layers_amd as T
    for (V, S, P, H), steps in read_router_traces():
        def make():
            c = T.DeltaCache(V, S, P, H)
            return c, T.Router(c)
        run_router_trace(make, steps)


@pytest.mark.parametrize("V,S,P,H", [(14, 8, 6, 0), (14, 4, 2, 16), (6, 2, 0, 0), (30, 10, 3, 50)])
def test_router_library_matches_oracle(V, S, P, H):
    """Batch by batch, the native router equals the oracle's on Zipf(1.1)
    traffic with base-only requests, random batch sizes, loads that finish
    at random and batches completed out of order."""
    import tenant_linear_layers_amd as T
    rng = np.random.default_rng(V * 100 + S)
    lc = T.DeltaCache(V, S, P, H)
    lr = T.Router(lc)
    oc = CP.CachePolicy(V, S, P, H)
    orr = CP.Router(oc)
    open_b = []
    rid = 0
    for step in range(600):
        for _ in range(int(rng.integers(0, 4))):
            v = int(zipf_trace(1, V, 7 * step + rid)[0]) if rng.random() > 0.1 else -1
            lr.submit(rid, v)
            orr.submit(rid, v)
            rid += 1
        for u in range(V):
            if oc.state[u] == CP.LOADING and rng.random() < 0.4:
                lc.loaded(u)
                oc.loaded(u)
        mb = int(rng.integers(1, 9))
        got = lr.next_batch(mb)
        want = orr.next_batch(mb)
        assert got == [tuple(w) for w in want], step
        open_b.append(got)
        while open_b and rng.random() < 0.6:
            b = open_b.pop(int(rng.integers(len(open_b))))
            lr.complete(b)
            orr.complete(b)
        assert lr.pending() == len(orr.queue)
    for u in range(V):
        assert lc.state(u) == (oc.state[u], oc.slot[u], oc.rate[u])


def test_router_library_rejects_bad_calls():
    import tenant_linear_layers_amd as T
    c = T.DeltaCache(4, 2, 0, 0)
    r = T.Router(c)
    for call in (lambda: r.submit(0, 4), lambda: r.submit(0, -2), lambda: r.next_batch(0),
                 lambda: r.complete([(0, 1, 0)])):
        with pytest.raises(T.BitDeltaError) as e:
            call()
        assert e.value.status == 10
