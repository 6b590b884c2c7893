// Expert staging: one bounded pool of HBM slots shared by every layer,
// filled from pinned host bundles with LRU replacement.
//
// [Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction": Figure 1 (bounded streaming pool, LRU,
// staged fixed-slot double buffer), §3.1 "Executor paths" (bundles copied
// into slots, kernels index them through the slot table), §3.2
// "Motivation" (the next token's sets are known one token ahead), Table 1
// caption (one LRU of bundles shared by all layers).  [Cacheable] =
// "Cacheable by Design?", App. E (LRU replay).
//
// Policy (edge0_lru, host only): a request pins its (layer, id) keys until
// its release; its ids are then taken in order - a resident key is a hit, a
// missing key takes the lowest free slot, else the unpinned resident slot
// with the oldest stamp; every touched key takes the next value of one
// global clock.  The stager adds the data movement: per request, the misses'
// bundles are copied host-to-device into their slots and the slot table is
// patched by one small kernel on the staging stream, then a ready event is
// recorded there.  Cross-stream hazards are ordered with events only:
//   - a copy into a slot that some layer read waits for the release event
//     recorded on the compute stream after that layer's kernels;
//   - a hit on a slot whose fill ran on another stream waits for that fill's
//     ready event;
//   - the compute stream waits for a set's ready event before the layer
//     (edge0_stager_wait).
// Events are per (layer, step parity): at most two sets of a layer are
// pending, and waiting on a later record of the same event only delays.
#include <map>
#include <new>
#include <set>
#include <utility>
#include <vector>

#include "moe_internal.h"

namespace e0 {

struct Lru {
  int n_slots = 0, n_layers = 0, n_experts = 0;
  std::vector<int32_t> owner;   // slot -> key L*E + e, or -1
  std::vector<uint64_t> stamp;  // slot -> clock of its last touch
  std::vector<int32_t> slot_of; // key -> slot, or -1
  std::vector<int32_t> pins;    // key -> number of pending sets holding it
  std::set<std::pair<uint64_t, int>> by_stamp;  // resident slots, oldest first
  std::set<int> free_slots;
  std::map<std::pair<int, int>, std::vector<int32_t>> pending;  // (L, t) -> keys
  uint64_t clock = 0;
  edge0_stage_stats stats{};

  int init(int slots, int layers, int experts) {
    if (slots < 1 || layers < 1 || experts < 1) return EDGE0_EINVAL;
    if ((int64_t)layers * experts > (int64_t)1 << 30) return EDGE0_EINVAL;
    n_slots = slots;
    n_layers = layers;
    n_experts = experts;
    owner.assign(slots, -1);
    stamp.assign(slots, 0);
    slot_of.assign((size_t)layers * experts, -1);
    pins.assign((size_t)layers * experts, 0);
    for (int s = 0; s < slots; ++s) free_slots.insert(s);
    return EDGE0_OK;
  }

  // Checks a request; returns EDGE0_OK and fills keys, or an error with the
  // state unchanged.
  int check(int L, int t, const int32_t* ids, int n, std::vector<int32_t>& keys) const {
    if (L < 0 || L >= n_layers || t < 0 || !ids || n < 1 || n > 16) return EDGE0_EINVAL;
    if (pending.count({L, t})) return EDGE0_EINVAL;
    keys.resize(n);
    int misses = 0;
    for (int i = 0; i < n; ++i) {
      if (ids[i] < 0 || ids[i] >= n_experts) return EDGE0_EINVAL;
      for (int j = 0; j < i; ++j)
        if (ids[j] == ids[i]) return EDGE0_EINVAL;
      keys[i] = L * n_experts + ids[i];
      if (slot_of[keys[i]] < 0) ++misses;
    }
    const int n_free = (int)free_slots.size();
    if (misses <= n_free) return EDGE0_OK;
    // evictable: resident, unpinned, and not a key of this request
    int need = misses - n_free;
    for (const auto& ps : by_stamp) {
      const int key = owner[ps.second];
      bool mine = false;
      for (int i = 0; i < n; ++i) mine |= keys[i] == key;
      if (pins[key] == 0 && !mine && --need == 0) return EDGE0_OK;
    }
    return EDGE0_ENOSLOT;
  }

  // Applies a checked request.  evicted[i] = key replaced by miss i, or -1.
  void apply(int L, int t, const std::vector<int32_t>& keys, int32_t* slots, int32_t* hit,
             int32_t* evicted) {
    const int n = (int)keys.size();
    pending[{L, t}] = keys;
    for (int i = 0; i < n; ++i) ++pins[keys[i]];
    ++stats.requests;
    for (int i = 0; i < n; ++i) {
      const int key = keys[i];
      ++clock;
      ++stats.touches;
      int s = slot_of[key];
      int ev = -1;
      if (s >= 0) {
        ++stats.hits;
        by_stamp.erase({stamp[s], s});
        if (hit) hit[i] = 1;
      } else {
        ++stats.misses;
        if (!free_slots.empty()) {
          s = *free_slots.begin();
          free_slots.erase(free_slots.begin());
        } else {
          auto it = by_stamp.begin();
          while (pins[owner[it->second]] != 0) ++it;  // check() guarantees one
          s = it->second;
          by_stamp.erase(it);
          ev = owner[s];
          slot_of[ev] = -1;
          ++stats.evictions;
        }
        owner[s] = key;
        slot_of[key] = s;
        if (hit) hit[i] = 0;
      }
      stamp[s] = clock;
      by_stamp.insert({clock, s});
      slots[i] = s;
      if (evicted) evicted[i] = ev;
    }
  }

  int release(int L, int t, std::vector<int32_t>* keys_out = nullptr) {
    auto it = pending.find({L, t});
    if (it == pending.end()) return EDGE0_EINVAL;
    for (int key : it->second) --pins[key];
    if (keys_out) *keys_out = std::move(it->second);
    pending.erase(it);
    return EDGE0_OK;
  }
};

// slot-table entries to set, passed by value (captured at launch)
constexpr int kMaxPatch = 32;
struct TablePatch {
  int n;
  int32_t idx[kMaxPatch];
  int32_t val[kMaxPatch];
};
__global__ void k_patch_table(int32_t* __restrict__ table, TablePatch p) {
  const int i = threadIdx.x;
  if (i < p.n) table[p.idx[i]] = p.val[i];
}

}  // namespace e0

using namespace e0;

struct edge0_lru {
  Lru lru;
};

struct edge0_stager {
  Lru lru;
  edge0_moe_shape shape;
  edge0_slot_pool pool;
  int64_t bundle_bytes = 0;
  std::vector<const void*> host;  // [L * E]
  int32_t* table = nullptr;
  std::vector<hipEvent_t> ev_ready, ev_rel;  // [L][2]
  // per slot: the event index (L*2 + parity) and stream of its last fill
  // and of the last release of a set that read it (-1: none)
  std::vector<int32_t> fill_ev, rel_ev;
  std::vector<hipStream_t> fill_stream, rel_stream;
  std::map<std::pair<int, int>, hipStream_t> staged_on;  // pending (L, t) -> stream
};

extern "C" int edge0_lru_create(edge0_lru** out, int32_t n_slots, int32_t n_layers,
                                int32_t n_experts) {
  if (!out) return EDGE0_EINVAL;
  edge0_lru* h = new (std::nothrow) edge0_lru();
  if (!h) return EDGE0_ENOMEM;
  const int rc = h->lru.init(n_slots, n_layers, n_experts);
  if (rc != EDGE0_OK) {
    delete h;
    return rc;
  }
  *out = h;
  return EDGE0_OK;
}

extern "C" int edge0_lru_request(edge0_lru* h, int32_t layer, int32_t step, const int32_t* ids,
                                 int32_t n, int32_t* slots_out, int32_t* hit_out,
                                 int32_t* evicted_out) {
  if (!h || !slots_out) return EDGE0_EINVAL;
  std::vector<int32_t> keys;
  const int rc = h->lru.check(layer, step, ids, n, keys);
  if (rc != EDGE0_OK) return rc;
  h->lru.apply(layer, step, keys, slots_out, hit_out, evicted_out);
  return EDGE0_OK;
}

extern "C" int edge0_lru_release(edge0_lru* h, int32_t layer, int32_t step) {
  if (!h) return EDGE0_EINVAL;
  return h->lru.release(layer, step);
}

extern "C" int edge0_lru_stats(const edge0_lru* h, edge0_stage_stats* out) {
  if (!h || !out) return EDGE0_EINVAL;
  *out = h->lru.stats;
  return EDGE0_OK;
}

extern "C" void edge0_lru_destroy(edge0_lru* h) { delete h; }

extern "C" void edge0_stager_destroy(edge0_stager* sg) {
  if (!sg) return;
  for (auto e : sg->ev_ready)
    if (e) (void)hipEventDestroy(e);
  for (auto e : sg->ev_rel)
    if (e) (void)hipEventDestroy(e);
  delete sg;
}

extern "C" int edge0_stager_create(edge0_stager** out, const edge0_moe_shape* shape,
                                   const edge0_slot_pool* pool, int32_t n_layers,
                                   const void* const* host_bundles, int32_t* slot_table) {
  if (!out || !shape || !shape_ok(shape) || !pool || !pool->base || pool->n_slots < 1 ||
      !host_bundles || !slot_table || n_layers < 1)
    return EDGE0_EINVAL;
  edge0_bundle_layout lay;
  if (bundle_layout(shape, &lay) != EDGE0_OK) return EDGE0_EINVAL;
  if (pool->slot_bytes < lay.bytes || pool->slot_bytes % 256 != 0) return EDGE0_EINVAL;
  const int E = shape->n_experts;
  for (int64_t i = 0; i < (int64_t)n_layers * E; ++i)
    if (!host_bundles[i]) return EDGE0_EINVAL;
  edge0_stager* sg = new (std::nothrow) edge0_stager();
  if (!sg) return EDGE0_ENOMEM;
  int rc = sg->lru.init(pool->n_slots, n_layers, E);
  if (rc != EDGE0_OK) {
    delete sg;
    return rc;
  }
  sg->shape = *shape;
  sg->pool = *pool;
  sg->bundle_bytes = lay.bytes;
  sg->host.assign(host_bundles, host_bundles + (size_t)n_layers * E);
  sg->table = slot_table;
  sg->ev_ready.assign((size_t)n_layers * 2, nullptr);
  sg->ev_rel.assign((size_t)n_layers * 2, nullptr);
  bool ok = true;
  for (size_t i = 0; i < sg->ev_ready.size() && ok; ++i)
    ok = hipEventCreateWithFlags(&sg->ev_ready[i], hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&sg->ev_rel[i], hipEventDisableTiming) == hipSuccess;
  sg->fill_ev.assign(pool->n_slots, -1);
  sg->rel_ev.assign(pool->n_slots, -1);
  sg->fill_stream.assign(pool->n_slots, nullptr);
  sg->rel_stream.assign(pool->n_slots, nullptr);
  ok = ok && hipMemset(slot_table, 0xFF, (size_t)n_layers * E * 4) == hipSuccess &&
       hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    edge0_stager_destroy(sg);
    return EDGE0_EHIP;
  }
  *out = sg;
  return EDGE0_OK;
}

extern "C" int edge0_stage_experts(edge0_stager* sg, int32_t layer, int32_t step,
                                   const int32_t* ids, int32_t n, int32_t* slots_out,
                                   hipStream_t stream) {
  if (!sg) return EDGE0_EINVAL;
  std::vector<int32_t> keys;
  int rc = sg->lru.check(layer, step, ids, n, keys);
  if (rc != EDGE0_OK) return rc;
  int32_t slots[16], hit[16], evicted[16];
  sg->lru.apply(layer, step, keys, slots, hit, evicted);
  sg->staged_on[{layer, step}] = stream;
  const int E = sg->shape.n_experts;
  const int my_ev = layer * 2 + (step & 1);
  // hazards first: every wait this request needs, each event once
  int waits[2 * 16];
  int n_waits = 0;
  auto add_wait = [&](int ev) {
    for (int j = 0; j < n_waits; ++j)
      if (waits[j] == ev * 2 + 0) return;
    waits[n_waits++] = ev * 2 + 0;
  };
  auto add_rel = [&](int ev) {
    for (int j = 0; j < n_waits; ++j)
      if (waits[j] == ev * 2 + 1) return;
    waits[n_waits++] = ev * 2 + 1;
  };
  for (int i = 0; i < n; ++i) {
    const int s = slots[i];
    if (hit[i]) {
      if (sg->fill_ev[s] >= 0 && sg->fill_stream[s] != stream) add_wait(sg->fill_ev[s]);
    } else {
      if (sg->rel_ev[s] >= 0 && sg->rel_stream[s] != stream) add_rel(sg->rel_ev[s]);
      if (sg->fill_ev[s] >= 0 && sg->fill_stream[s] != stream) add_wait(sg->fill_ev[s]);
    }
  }
  for (int j = 0; j < n_waits; ++j) {
    hipEvent_t e = (waits[j] & 1) ? sg->ev_rel[waits[j] >> 1] : sg->ev_ready[waits[j] >> 1];
    if (hipStreamWaitEvent(stream, e, 0) != hipSuccess) return EDGE0_EHIP;
  }
  TablePatch p{};
  uint8_t* base = static_cast<uint8_t*>(sg->pool.base);
  for (int i = 0; i < n; ++i) {
    if (hit[i]) continue;
    const int s = slots[i];
    if (hipMemcpyAsync(base + (size_t)s * sg->pool.slot_bytes, sg->host[keys[i]],
                       (size_t)sg->bundle_bytes, hipMemcpyHostToDevice, stream) != hipSuccess)
      return EDGE0_EHIP;
    sg->lru.stats.bytes_staged += sg->bundle_bytes;
    if (evicted[i] >= 0) {
      p.idx[p.n] = evicted[i];
      p.val[p.n++] = -1;
    }
    p.idx[p.n] = keys[i];
    p.val[p.n++] = s;
    sg->fill_ev[s] = my_ev;
    sg->fill_stream[s] = stream;
    sg->rel_ev[s] = -1;
    sg->rel_stream[s] = nullptr;
  }
  if (p.n > 0) {
    k_patch_table<<<1, 64, 0, stream>>>(sg->table, p);
    E0_CHECK_LAUNCH();
  }
  if (hipEventRecord(sg->ev_ready[my_ev], stream) != hipSuccess) return EDGE0_EHIP;
  if (slots_out)
    for (int i = 0; i < n; ++i) slots_out[i] = slots[i];
  (void)E;
  return EDGE0_OK;
}

extern "C" int edge0_stager_wait(edge0_stager* sg, int32_t layer, int32_t step,
                                 hipStream_t compute_stream) {
  if (!sg) return EDGE0_EINVAL;
  auto it = sg->staged_on.find({layer, step});
  if (it == sg->staged_on.end()) return EDGE0_EINVAL;
  if (it->second == compute_stream) return EDGE0_OK;
  return hipStreamWaitEvent(compute_stream, sg->ev_ready[layer * 2 + (step & 1)], 0) == hipSuccess
             ? EDGE0_OK
             : EDGE0_EHIP;
}

extern "C" int edge0_stager_release(edge0_stager* sg, int32_t layer, int32_t step,
                                    hipStream_t compute_stream) {
  if (!sg) return EDGE0_EINVAL;
  if (!sg->lru.pending.count({layer, step})) return EDGE0_EINVAL;
  const int ev = layer * 2 + (step & 1);
  if (hipEventRecord(sg->ev_rel[ev], compute_stream) != hipSuccess) return EDGE0_EHIP;
  std::vector<int32_t> keys;
  const int rc = sg->lru.release(layer, step, &keys);
  if (rc != EDGE0_OK) return rc;
  for (int key : keys) {
    const int s = sg->lru.slot_of[key];
    if (s < 0) continue;
    sg->rel_ev[s] = ev;
    sg->rel_stream[s] = compute_stream;
  }
  sg->staged_on.erase({layer, step});
  return EDGE0_OK;
}

extern "C" int edge0_stager_stats(const edge0_stager* sg, edge0_stage_stats* out) {
  if (!sg || !out) return EDGE0_EINVAL;
  *out = sg->lru.stats;
  return EDGE0_OK;
}

namespace e0 {
edge0_slot_pool stager_pool(const edge0_stager* sg) { return sg->pool; }
const int32_t* stager_table(const edge0_stager* sg) { return sg->table; }
int stager_layers(const edge0_stager* sg) { return sg->lru.n_layers; }
}  // namespace e0
