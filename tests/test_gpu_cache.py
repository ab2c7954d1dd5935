"""GPU tests of the delta cache: variants' packed signs and alpha loaded from
page-locked host memory into device slots by bitdelta_cache_acquire, and the
fused linears run on the slots' bytes.

Parity: the slot bytes equal the host bytes; every linear through a slot is
bit-identical to the same call on the variant's own tensors and within the
output tolerance of the oracle; the policy's decisions equal the oracle
policy's when every load has finished before the next request.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
import tenant_linear_layers_amd as T
from helpers import assert_y_close, bits16, packed_u64
from oracle import cache_policy as CP

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T.lib()


def make_variants(shapes, n_variants, mode, seed):
    """Base matrices and n_variants compressed fine-tunes of each, on the GPU;
    each variant's delta also as one page-locked host blob (delta_layout)."""
    g = S.generator(seed, DEV)
    bases = [S.draw_base(d_out, d_in, 0.02, g, DEV) for d_out, d_in in shapes]
    packs, alphas, blobs = [], [], []
    for v in range(n_variants):
        pv, av = [], []
        for wb in bases:
            wf = S.draw_finetuned(wb, 2e-4 * (v + 1), g)
            p, a = T.compress(wf, wb, mode)
            pv.append(p)
            av.append(a)
            del wf
        _, total = T.delta_layout(shapes, mode)
        blob = torch.zeros(total, dtype=torch.uint8, pin_memory=True)
        for (hp, ha), p, a in zip(T.delta_views(blob, shapes, mode), pv, av):
            hp.copy_(p.cpu())
            ha.copy_(a.cpu())
        packs.append(pv)
        alphas.append(av)
        blobs.append(blob)
    torch.cuda.synchronize()
    return bases, packs, alphas, blobs


def make_cache(n_variants, n_slots, n_pinned, halve_every, blobs):
    c = T.DeltaCache(n_variants, n_slots, n_pinned, halve_every)
    nbytes = max(b.numel() for b in blobs)
    slots = [torch.zeros(nbytes, dtype=torch.uint8, device=DEV) for _ in range(n_slots)]
    c.attach(slots, blobs)
    return c, slots


def test_cache_loads_and_policy_match_oracle():
    """Loads finish before each request (synchronised), so the native policy
    must take the oracle's decisions; every linear through a slot equals the
    direct call bit for bit, and the oracle within tolerance."""
    shapes = [(192, 512), (320, 1024)]
    mode = T.ALPHA_PER_ROW
    V, Sl, P = 6, 3, 1
    bases, packs, alphas, blobs = make_variants(shapes, V, mode, 41)
    cache, slots = make_cache(V, Sl, P, 0, blobs)
    orc = CP.CachePolicy(V, Sl, P, 0)
    copy = torch.cuda.Stream()
    g = S.generator(42)
    xs = [S.draw_activations(4, d_in, g).to(DEV) for _, d_in in shapes]
    trace = S.zipf_ids(48, V, 43)
    loads = 0
    for step, v in enumerate(trace):
        v = int(v)
        torch.cuda.synchronize()
        for u in range(V):
            if orc.state[u] == CP.LOADING:
                orc.loaded(u)
        act, slot, ev = cache.acquire(v, copy)
        want = orc.request(v)
        assert (act, ev) == (want[0], want[2]), (step, v)
        assert slot is slots[want[1]]
        loads += act == T.CACHE_LOAD
        views = T.delta_views(slot, shapes, mode)
        for i, (p, a) in enumerate(views):
            y = T.linear(xs[i], bases[i], p, a, mode)
            y_direct = T.linear(xs[i], bases[i], packs[v][i], alphas[v][i], mode)
            assert torch.equal(y.view(torch.int16), y_direct.view(torch.int16)), (step, v, i)
            if step % 8 == 0:
                ref = O.linear(bits16(xs[i]), bits16(bases[i]), packed_u64(packs[v][i]),
                               alphas[v][i].cpu().numpy(), mode)
                assert_y_close(y, ref, f"cached variant {v} matrix {i}")
        cache.release(v)
        orc.release(v)
    assert loads > V // 2 and loads < len(trace)
    torch.cuda.synchronize()
    for v in range(V):
        st, s, _ = cache.state(v)
        if st != T.CACHE_ABSENT:
            n = blobs[v].numel()
            assert torch.equal(slots[s][:n].cpu(), blobs[v]), v


def test_cache_from_delta_files(tmp_path):
    """Variants written to delta files and read back into page-locked blobs
    (tenant_linear_layers_amd.deltafile) serve the cache exactly as the blobs
    they were written from: the blob built from the device tensors equals
    the test's own, the read-back blob equals it byte for byte, and every
    linear through a slot loaded from it equals the direct call."""
    shapes = [(192, 512), (320, 1024)]
    mode = T.ALPHA_PER_ROW
    V = 3
    bases, packs, alphas, blobs = make_variants(shapes, V, mode, 61)
    loaded = []
    for v in range(V):
        built = T.delta_blob(list(zip(packs[v], alphas[v])), shapes, mode)
        assert torch.equal(built, blobs[v]), v
        path = tmp_path / f"variant{v}.bdlt"
        T.save_delta(path, built, shapes, mode)
        blob, shp, m = T.load_delta(path)
        assert shp == shapes and m == mode and blob.is_pinned()
        assert torch.equal(blob, blobs[v]), v
        loaded.append(blob)
    cache, slots = make_cache(V, 2, 0, 0, loaded)
    copy = torch.cuda.Stream()
    g = S.generator(62)
    xs = [S.draw_activations(4, d_in, g).to(DEV) for _, d_in in shapes]
    for v in [2, 0, 1, 2, 1]:
        act, slot, _ = cache.acquire(v, copy)
        assert act != T.CACHE_FULL and slot is not None
        for i, (p, a) in enumerate(T.delta_views(slot, shapes, mode)):
            y = T.linear(xs[i], bases[i], p, a, mode)
            y_direct = T.linear(xs[i], bases[i], packs[v][i], alphas[v][i], mode)
            assert torch.equal(y.view(torch.int16), y_direct.view(torch.int16)), (v, i)
        cache.release(v)
    torch.cuda.synchronize()


def test_cache_mixed_batches_without_synchronisation():
    """Batches hold several variants at once and nothing waits on the host:
    loads overlap earlier batches' kernels; each mixed-variant output equals
    the direct call on the variants' own tensors bit for bit."""
    shapes = [(256, 1024)]
    mode = T.ALPHA_PER_ROW
    V, Sl, P = 7, 4, 2
    bases, packs, alphas, blobs = make_variants(shapes, V, mode, 51)
    cache, slots = make_cache(V, Sl, P, 16, blobs)
    copy = torch.cuda.Stream()
    g = S.generator(52)
    rng = np.random.default_rng(53)
    outs = []
    fulls = 0
    for step in range(30):
        want = sorted(set(int(u) for u in S.zipf_ids(3, V, 100 + step)))
        held, views = [], []
        for v in want:
            act, slot, ev = cache.acquire(v, copy)
            if act == T.CACHE_FULL:
                fulls += 1
                continue
            held.append(v)
            views.append(T.delta_views(slot, shapes, mode)[0])
        if not held:   # every slot busy loading or pinned: a legitimate refusal
            continue
        x = S.draw_activations(8, shapes[0][1], g).to(DEV)
        ids_np = rng.integers(-1, len(held), size=8).astype(np.int32)
        ids = torch.from_numpy(ids_np).to(DEV)
        y = T.linear_multi(x, ids, bases[0], [p for p, _ in views], [a for _, a in views], mode)
        y_direct = T.linear_multi(x, ids, bases[0], [packs[v][0] for v in held],
                                  [alphas[v][0] for v in held], mode)
        outs.append((y, y_direct, step))
        for v in held:
            cache.release(v)
    torch.cuda.synchronize()
    for y, y_direct, step in outs:
        assert torch.equal(y.view(torch.int16), y_direct.view(torch.int16)), step
    assert cache.poll() >= 0


def test_cache_queued_request_waits_for_the_load():
    """A second request while a large load is in flight queues behind it
    (QUEUED, same slot, no second load); a kernel enqueued after either
    request reads the loaded bytes."""
    shapes = [(8192, 8192)]
    mode = T.ALPHA_PER_ROW
    bases, packs, alphas, blobs = make_variants(shapes, 2, mode, 61)
    cache, slots = make_cache(2, 1, 0, 0, blobs)
    copy = torch.cuda.Stream()
    x = S.draw_activations(4, 8192, S.generator(62)).to(DEV)
    y_want = T.linear(x, bases[0], packs[1][0], alphas[1][0], mode)
    torch.cuda.synchronize()
    act1, slot1, _ = cache.acquire(1, copy)
    act2, slot2, _ = cache.acquire(1, copy)
    assert act1 == T.CACHE_LOAD
    assert act2 in (T.CACHE_QUEUED, T.CACHE_HIT) and slot2 is slot1
    p, a = T.delta_views(slot2, shapes, mode)[0]
    y = T.linear(x, bases[0], p, a, mode)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_want.view(torch.int16))
    cache.release(1)
    cache.release(1)
    assert cache.state(1)[0] in (T.CACHE_LOADING, T.CACHE_RESIDENT)
    cache.poll()
    assert cache.state(1)[0] == T.CACHE_RESIDENT


def test_cache_eviction_waits_for_released_work():
    """Kernels still queued on the use stream when their variant is released
    read the old bytes: the load that evicts it into the same slot waits for
    the release's event."""
    shapes = [(8192, 8192)]
    mode = T.ALPHA_PER_ROW
    bases, packs, alphas, blobs = make_variants(shapes, 2, mode, 71)
    cache, slots = make_cache(2, 1, 0, 0, blobs)
    copy = torch.cuda.Stream()
    x = S.draw_activations(16, 8192, S.generator(72)).to(DEV)
    want = [T.linear(x, bases[0], packs[v][0], alphas[v][0], mode) for v in range(2)]
    torch.cuda.synchronize()
    act, slot, _ = cache.acquire(0, copy)
    assert act == T.CACHE_LOAD
    p, a = T.delta_views(slot, shapes, mode)[0]
    ys0 = [T.linear(x, bases[0], p, a, mode) for _ in range(24)]   # queued work on slot 0
    cache.release(0)
    act, slot_b, ev = cache.acquire(1, copy)
    assert (act, ev) == (T.CACHE_LOAD, 0) and slot_b is slot
    pb, ab = T.delta_views(slot_b, shapes, mode)[0]
    y1 = T.linear(x, bases[0], pb, ab, mode)
    cache.release(1)
    torch.cuda.synchronize()
    for k, y in enumerate(ys0):
        assert torch.equal(y.view(torch.int16), want[0].view(torch.int16)), k
    assert torch.equal(y1.view(torch.int16), want[1].view(torch.int16))


def test_router_feeds_mixed_batches():
    """Requests over 8 variants (Zipf, one in ten base-only) through the
    router and a 3-slot cache into bitdelta_linear_multi: every request is
    served once, each batch's output equals the same call on the variants'
    own tensors bit for bit (and the oracle on some batches); nothing waits
    on the host except when no request is ready."""
    shapes = [(256, 1024)]
    mode = T.ALPHA_PER_ROW
    V, Sl, P = 8, 3, 1
    bases, packs, alphas, blobs = make_variants(shapes, V, mode, 81)
    cache, slots = make_cache(V, Sl, P, 0, blobs)
    router = T.Router(cache)
    copy = torch.cuda.Stream()
    g = S.generator(82)
    rng = np.random.default_rng(83)
    n_req = 120
    xs = S.draw_activations(n_req, shapes[0][1], g).to(DEV)
    variant_of = [int(v) if rng.random() > 0.1 else -1 for v in S.zipf_ids(n_req, V, 84)]
    submitted, served, outs = 0, [], []
    for it in range(2000):
        for _ in range(int(rng.integers(0, 6))):
            if submitted < n_req:
                router.submit(submitted, variant_of[submitted])
                submitted += 1
        batch = router.next_batch(16, copy)
        if not batch:
            if submitted == n_req and router.pending() == 0:
                break
            copy.synchronize()   # only loads are outstanding
            continue
        rids = [b[0] for b in batch]
        local = sorted({b[1] for b in batch if b[1] >= 0})
        slot_of = {b[1]: b[2] for b in batch if b[1] >= 0}
        ids = torch.tensor([local.index(b[1]) if b[1] >= 0 else -1 for b in batch],
                           dtype=torch.int32, device=DEV)
        x = xs[torch.as_tensor(rids, device=DEV)].contiguous()
        if local:
            views = [T.delta_views(slots[slot_of[v]], shapes, mode)[0] for v in local]
            y = T.linear_multi(x, ids, bases[0], [p for p, _ in views], [a for _, a in views], mode)
            y_direct = T.linear_multi(x, ids, bases[0], [packs[v][0] for v in local],
                                      [alphas[v][0] for v in local], mode)
        else:
            y = y_direct = T.linear_multi(x, ids, bases[0], [packs[0][0]], [alphas[0][0]], mode)
        outs.append((y, y_direct, x, ids, local))
        served.extend(rids)
        router.complete(batch)
    torch.cuda.synchronize()
    assert sorted(served) == list(range(n_req))
    for k, (y, y_direct, x, ids, local) in enumerate(outs):
        assert torch.equal(y.view(torch.int16), y_direct.view(torch.int16)), k
        if k % 10 == 0 and local:
            ref = O.linear_multi(bits16(x), ids.cpu().numpy(), bits16(bases[0]),
                                 [packed_u64(packs[v][0]) for v in local],
                                 [alphas[v][0].cpu().numpy() for v in local], mode)
            assert_y_close(y, ref, f"router batch {k}")
