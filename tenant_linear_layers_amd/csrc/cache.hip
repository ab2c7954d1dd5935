// Delta cache: which variant's packed delta (signs + alpha) is resident in
// which device slot, and the host-to-device loads that fill the slots.
//
// Page "BitDelta: Tek bir GPU kümesinden 14 Zen modeli sunmak", section
// "Altyapı ayrıntıları": a variant's delta that is not resident is loaded
// into device memory on its first request (the cold-start paragraph), and
// stays until evicted; eviction is least-recently-used weighted by request
// rate, the highest-rate variants pinned (the eviction paragraph); while a
// variant's delta is loading, further requests for it wait for that load
// instead of starting their own (the routing paragraph).
//
// Policy (host only, no device work): rate = request count per variant,
// halved for all variants after every halve_every-th counted request (0:
// never); the n_pinned variants of highest rate (ties to the lower id) are
// never evicted; a miss takes the lowest free slot, else evicts the least
// recently requested variant that is resident, unpinned, released and not the
// one requested; if there is none the request is refused (FULL) and changes
// nothing.
//
// Loads: bitdelta_cache_acquire copies the variant's host bytes into its slot
// with hipMemcpyAsync on the caller's copy stream, records the variant's load
// event there and makes the caller's use stream wait on it; requests that
// find the load in flight make their stream wait on the same event.  A slot
// is overwritten only after the copy stream has waited for the event that
// the slot's last release recorded on its use stream, so work enqueued
// before the release still reads the old delta.  Load completion is observed
// by polling the events; a load counts as finished once its event has
// completed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <deque>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>

#include "bitdelta.h"

#define BD_EXPORT extern "C" __attribute__((visibility("default")))

struct bitdelta_cache {
  std::mutex mu;
  int V = 0, S = 0, P = 0;
  int64_t H = 0;
  int64_t time = 0;
  std::vector<int64_t> rate, last;
  std::vector<int32_t> state, slot, users, owner;
  // device memory, once attached
  bool attached = false;
  int device = -1;
  size_t slot_bytes = 0;
  std::vector<void*> slot_dev;
  std::vector<const void*> src;
  std::vector<size_t> src_bytes;
  std::vector<hipEvent_t> load_ev;   // per variant: its last load
  std::vector<hipEvent_t> free_ev;   // per slot: its last release
  std::vector<char> free_recorded;
};

namespace {

constexpr int kMaxCacheVariants = 1 << 16;

bool valid_variant(const bitdelta_cache* c, int32_t v) { return v >= 0 && v < c->V; }

// Rates after counting one request for v at the next logical time.
std::vector<int64_t> rates_after(const bitdelta_cache* c, int32_t v) {
  std::vector<int64_t> r = c->rate;
  r[v] += 1;
  if (c->H > 0 && (c->time + 1) % c->H == 0)
    for (auto& x : r) x >>= 1;
  return r;
}

// The variant to evict for a request of v under the given rates, or -1.
int32_t victim(const bitdelta_cache* c, int32_t v, const std::vector<int64_t>& r) {
  std::vector<int32_t> order(c->V);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return r[a] > r[b]; });
  std::vector<char> pinned(c->V, 0);
  for (int i = 0; i < c->P && i < c->V; ++i) pinned[order[i]] = 1;
  int32_t best = -1;
  for (int32_t u = 0; u < c->V; ++u) {
    if (u == v || c->state[u] != BITDELTA_CACHE_RESIDENT || c->users[u] != 0 || pinned[u])
      continue;
    if (best < 0 || c->last[u] < c->last[best]) best = u;
  }
  return best;
}

int32_t free_slot(const bitdelta_cache* c) {
  for (int32_t s = 0; s < c->S; ++s)
    if (c->owner[s] < 0) return s;
  return -1;
}

// One request (caller holds the lock).
void request_locked(bitdelta_cache* c, int32_t v, int32_t* action, int32_t* slot,
                    int32_t* evicted) {
  *slot = -1;
  *evicted = -1;
  if (c->state[v] == BITDELTA_CACHE_ABSENT && free_slot(c) < 0 &&
      victim(c, v, rates_after(c, v)) < 0) {
    *action = BITDELTA_CACHE_FULL;
    return;
  }
  c->rate = rates_after(c, v);
  c->time += 1;
  c->last[v] = c->time;
  if (c->state[v] != BITDELTA_CACHE_ABSENT) {
    c->users[v] += 1;
    *action = c->state[v] == BITDELTA_CACHE_RESIDENT ? BITDELTA_CACHE_HIT : BITDELTA_CACHE_QUEUED;
    *slot = c->slot[v];
    return;
  }
  int32_t s = free_slot(c);
  if (s < 0) {
    const int32_t u = victim(c, v, c->rate);
    s = c->slot[u];
    c->state[u] = BITDELTA_CACHE_ABSENT;
    c->slot[u] = -1;
    *evicted = u;
  }
  c->owner[s] = v;
  c->slot[v] = s;
  c->state[v] = BITDELTA_CACHE_LOADING;
  c->users[v] += 1;
  *action = BITDELTA_CACHE_LOAD;
  *slot = s;
}

// Mark finished loads resident (caller holds the lock).
int poll_locked(bitdelta_cache* c, int32_t* n_loaded) {
  int n = 0;
  for (int32_t u = 0; u < c->V; ++u) {
    if (c->state[u] != BITDELTA_CACHE_LOADING) continue;
    const hipError_t e = hipEventQuery(c->load_ev[u]);
    if (e == hipSuccess) {
      c->state[u] = BITDELTA_CACHE_RESIDENT;
      ++n;
    } else if (e != hipErrorNotReady) {
      return BITDELTA_ERR_HIP;
    }
  }
  if (n_loaded) *n_loaded = n;
  return BITDELTA_OK;
}

// One use of v ends (caller holds the lock; v is in use).
int release_locked(bitdelta_cache* c, int32_t v, hipStream_t stream) {
  if (c->attached) {
    const int32_t s = c->slot[v];
    if (hipEventRecord(c->free_ev[s], stream) != hipSuccess) return BITDELTA_ERR_HIP;
    c->free_recorded[s] = 1;
  }
  c->users[v] -= 1;
  return BITDELTA_OK;
}

// One request that moves the bytes (caller holds the lock, memory attached):
// on a LOAD, the copy into the slot after the slot's last release; with a
// use stream, LOAD and QUEUED make it wait for the load.
int acquire_locked(bitdelta_cache* c, int32_t v, hipStream_t cs, bool wait_use, hipStream_t us,
                   int32_t* action, int32_t* slot, int32_t* evicted) {
  request_locked(c, v, action, slot, evicted);
  if (*action == BITDELTA_CACHE_FULL) return BITDELTA_OK;
  const int32_t s = *slot;
  if (*action == BITDELTA_CACHE_LOAD) {
    hipError_t e = hipSuccess;
    if (c->free_recorded[s]) e = hipStreamWaitEvent(cs, c->free_ev[s], 0);
    if (e == hipSuccess)
      e = hipMemcpyAsync(c->slot_dev[s], c->src[v], c->src_bytes[v], hipMemcpyHostToDevice, cs);
    if (e == hipSuccess) e = hipEventRecord(c->load_ev[v], cs);
    if (e != hipSuccess) {
      // the variant is not loading after all; the evicted one stays evicted
      c->state[v] = BITDELTA_CACHE_ABSENT;
      c->slot[v] = -1;
      c->owner[s] = -1;
      c->users[v] -= 1;
      return BITDELTA_ERR_HIP;
    }
  }
  if (wait_use && *action != BITDELTA_CACHE_HIT &&
      hipStreamWaitEvent(us, c->load_ev[v], 0) != hipSuccess) {
    c->users[v] -= 1;  // the caller gets no slot and releases nothing
    return BITDELTA_ERR_HIP;
  }
  return BITDELTA_OK;
}

void destroy_events(bitdelta_cache* c) {
  for (auto& e : c->load_ev)
    if (e) (void)hipEventDestroy(e);
  for (auto& e : c->free_ev)
    if (e) (void)hipEventDestroy(e);
  c->load_ev.clear();
  c->free_ev.clear();
}

}  // namespace

BD_EXPORT int bitdelta_cache_create(int32_t n_variants, int32_t n_slots, int32_t n_pinned,
                                    int64_t halve_every, bitdelta_cache** out) {
  if (!out) return BITDELTA_ERR_NULL;
  *out = nullptr;
  if (n_variants < 1 || n_variants > kMaxCacheVariants || n_slots < 1 ||
      n_slots > kMaxCacheVariants || n_pinned < 0 || n_pinned >= n_slots || halve_every < 0)
    return BITDELTA_ERR_CACHE;
  bitdelta_cache* c = new (std::nothrow) bitdelta_cache;
  if (!c) return BITDELTA_ERR_CACHE;
  c->V = n_variants;
  c->S = n_slots;
  c->P = n_pinned;
  c->H = halve_every;
  c->rate.assign(n_variants, 0);
  c->last.assign(n_variants, -1);
  c->state.assign(n_variants, BITDELTA_CACHE_ABSENT);
  c->slot.assign(n_variants, -1);
  c->users.assign(n_variants, 0);
  c->owner.assign(n_slots, -1);
  *out = c;
  return BITDELTA_OK;
}

BD_EXPORT void bitdelta_cache_destroy(bitdelta_cache* c) {
  if (!c) return;
  destroy_events(c);
  delete c;
}

BD_EXPORT int bitdelta_cache_request(bitdelta_cache* c, int32_t variant, int32_t* action,
                                     int32_t* slot, int32_t* evicted) {
  if (!c || !action || !slot || !evicted) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  if (c->attached || !valid_variant(c, variant)) return BITDELTA_ERR_CACHE;
  request_locked(c, variant, action, slot, evicted);
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_cache_loaded(bitdelta_cache* c, int32_t variant) {
  if (!c) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  if (c->attached || !valid_variant(c, variant) ||
      c->state[variant] != BITDELTA_CACHE_LOADING)
    return BITDELTA_ERR_CACHE;
  c->state[variant] = BITDELTA_CACHE_RESIDENT;
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_cache_release(bitdelta_cache* c, int32_t variant, void* stream) {
  if (!c) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  if (!valid_variant(c, variant) || c->users[variant] <= 0) return BITDELTA_ERR_CACHE;
  return release_locked(c, variant, static_cast<hipStream_t>(stream));
}

BD_EXPORT int bitdelta_cache_state(bitdelta_cache* c, int32_t variant, int32_t* state,
                                   int32_t* slot, int64_t* rate) {
  if (!c || !state || !slot || !rate) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  if (!valid_variant(c, variant)) return BITDELTA_ERR_CACHE;
  *state = c->state[variant];
  *slot = c->slot[variant];
  *rate = c->rate[variant];
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_cache_attach(bitdelta_cache* c, void* const* slots, size_t slot_bytes,
                                    const void* const* sources, const size_t* source_bytes) {
  if (!c || !slots || !sources || !source_bytes) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  if (c->attached || c->time != 0) return BITDELTA_ERR_CACHE;
  for (int s = 0; s < c->S; ++s) {
    if (!slots[s]) return BITDELTA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(slots[s]) & 15u) return BITDELTA_ERR_ALIGN;
  }
  for (int s = 0; s < c->S; ++s)
    for (int t = s + 1; t < c->S; ++t) {
      const uintptr_t a = reinterpret_cast<uintptr_t>(slots[s]);
      const uintptr_t b = reinterpret_cast<uintptr_t>(slots[t]);
      if (a < b + slot_bytes && b < a + slot_bytes) return BITDELTA_ERR_OVERLAP;
    }
  for (int v = 0; v < c->V; ++v) {
    if (!sources[v]) return BITDELTA_ERR_NULL;
    if (source_bytes[v] > slot_bytes) return BITDELTA_ERR_CACHE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BITDELTA_ERR_HIP;
  c->load_ev.assign(c->V, nullptr);
  c->free_ev.assign(c->S, nullptr);
  for (auto& e : c->load_ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      destroy_events(c);
      return BITDELTA_ERR_HIP;
    }
  for (auto& e : c->free_ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      destroy_events(c);
      return BITDELTA_ERR_HIP;
    }
  c->free_recorded.assign(c->S, 0);
  c->slot_dev.assign(slots, slots + c->S);
  c->src.assign(sources, sources + c->V);
  c->src_bytes.assign(source_bytes, source_bytes + c->V);
  c->slot_bytes = slot_bytes;
  c->device = dev;
  c->attached = true;
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_cache_poll(bitdelta_cache* c, int32_t* n_loaded) {
  if (!c) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  if (!c->attached) return BITDELTA_ERR_CACHE;
  return poll_locked(c, n_loaded);
}

BD_EXPORT int bitdelta_cache_acquire(bitdelta_cache* c, int32_t variant, void* copy_stream,
                                     void* use_stream, int32_t* action, void** slot_ptr,
                                     int32_t* evicted) {
  if (!c || !action || !slot_ptr || !evicted) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(c->mu);
  *slot_ptr = nullptr;
  if (!c->attached || !valid_variant(c, variant)) return BITDELTA_ERR_CACHE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BITDELTA_ERR_HIP;
  if (dev != c->device) return BITDELTA_ERR_DEVICE;
  int st = poll_locked(c, nullptr);
  if (st != BITDELTA_OK) return st;
  int32_t s = -1;
  st = acquire_locked(c, variant, static_cast<hipStream_t>(copy_stream), true,
                      static_cast<hipStream_t>(use_stream), action, &s, evicted);
  if (st != BITDELTA_OK || *action == BITDELTA_CACHE_FULL) return st;
  *slot_ptr = c->slot_dev[s];
  return BITDELTA_OK;
}

// ------------------------------------------------------------------ router
// Decode batches fed from a request queue over a cache (section "Altyapı
// ayrıntıları", the routing paragraph: requests are tracked per variant and
// nothing is blocked behind a variant whose delta is loading).  A request
// registers with the cache once, at the first batch formed after it arrived
// (a FULL refusal leaves it unregistered until the next batch); it is ready
// once its variant is resident (a base-only request at once); a batch takes
// ready requests in arrival order.  With memory attached the registration
// starts the loads on the copy stream and no stream waits on them: a request
// joins a batch only after its load has completed.

struct bitdelta_router {
  std::mutex mu;
  bitdelta_cache* cache = nullptr;
  struct Req {
    int64_t id;
    int32_t v, state, slot;
  };
  std::deque<Req> q;
};

namespace {
constexpr int32_t kReqNew = 0, kReqWaiting = 1, kReqReady = 2;
}

BD_EXPORT int bitdelta_router_create(bitdelta_cache* cache, bitdelta_router** out) {
  if (!cache || !out) return BITDELTA_ERR_NULL;
  *out = nullptr;
  bitdelta_router* r = new (std::nothrow) bitdelta_router;
  if (!r) return BITDELTA_ERR_CACHE;
  r->cache = cache;
  *out = r;
  return BITDELTA_OK;
}

BD_EXPORT void bitdelta_router_destroy(bitdelta_router* r) { delete r; }

BD_EXPORT int bitdelta_router_submit(bitdelta_router* r, int64_t request_id, int32_t variant) {
  if (!r) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(r->mu);
  if (variant < -1 || variant >= r->cache->V) return BITDELTA_ERR_CACHE;
  r->q.push_back({request_id, variant, variant < 0 ? kReqReady : kReqNew, -1});
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_router_next_batch(bitdelta_router* r, int32_t max_batch, void* copy_stream,
                                         int64_t* ids, int32_t* variants, int32_t* slots,
                                         int32_t* n) {
  if (!r || !ids || !variants || !slots || !n) return BITDELTA_ERR_NULL;
  *n = 0;
  if (max_batch < 1) return BITDELTA_ERR_CACHE;
  std::lock_guard<std::mutex> lock(r->mu);
  bitdelta_cache* c = r->cache;
  std::lock_guard<std::mutex> clock(c->mu);
  if (c->attached) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return BITDELTA_ERR_HIP;
    if (dev != c->device) return BITDELTA_ERR_DEVICE;
    const int st = poll_locked(c, nullptr);
    if (st != BITDELTA_OK) return st;
  }
  for (auto& q : r->q) {
    if (q.state != kReqNew) continue;
    int32_t act = 0, slot = -1, ev = -1;
    if (c->attached) {
      const int st = acquire_locked(c, q.v, static_cast<hipStream_t>(copy_stream), false,
                                    nullptr, &act, &slot, &ev);
      if (st != BITDELTA_OK) return st;
    } else {
      request_locked(c, q.v, &act, &slot, &ev);
    }
    if (act == BITDELTA_CACHE_FULL) continue;
    q.state = act == BITDELTA_CACHE_HIT ? kReqReady : kReqWaiting;
    q.slot = slot;
  }
  for (auto& q : r->q)
    if (q.state == kReqWaiting && c->state[q.v] == BITDELTA_CACHE_RESIDENT) q.state = kReqReady;
  std::deque<bitdelta_router::Req> rest;
  int32_t k = 0;
  for (const auto& q : r->q) {
    if (q.state == kReqReady && k < max_batch) {
      ids[k] = q.id;
      variants[k] = q.v;
      slots[k] = q.slot;
      ++k;
    } else {
      rest.push_back(q);
    }
  }
  r->q.swap(rest);
  *n = k;
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_router_complete(bitdelta_router* r, int32_t n, const int32_t* variants,
                                       void* use_stream) {
  if (!r || (n > 0 && !variants)) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(r->mu);
  bitdelta_cache* c = r->cache;
  std::lock_guard<std::mutex> clock(c->mu);
  for (int32_t i = 0; i < n; ++i)
    if (variants[i] >= c->V || variants[i] < -1 ||
        (variants[i] >= 0 && c->users[variants[i]] <= 0))
      return BITDELTA_ERR_CACHE;
  for (int32_t i = 0; i < n; ++i) {
    if (variants[i] < 0) continue;
    const int st = release_locked(c, variants[i], static_cast<hipStream_t>(use_stream));
    if (st != BITDELTA_OK) return st;
  }
  return BITDELTA_OK;
}

BD_EXPORT int bitdelta_router_pending(bitdelta_router* r, int32_t* n) {
  if (!r || !n) return BITDELTA_ERR_NULL;
  std::lock_guard<std::mutex> lock(r->mu);
  *n = (int32_t)r->q.size();
  return BITDELTA_OK;
}
