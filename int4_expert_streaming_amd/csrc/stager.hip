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
// global clock.  The stager adds the data movement: per request, one kernel
// copies the misses' bundles from pinned host memory into their slots on the
// staging stream, then a ready event is recorded.  Cross-stream hazards are ordered with events only:
//   - a copy into a slot that some layer read waits for the release event
//     recorded on the compute stream after that layer's kernels;
//   - a hit on a slot whose fill ran on another stream waits for that fill's
//     ready event;
//   - the compute stream waits for a set's ready event before the layer
//     (edge0_stager_wait).
// Each record has a serial, so a wait targets exactly the record it needs
// and is dropped once that record has completed.  The slot table is written
// on the compute stream only: a request's updates (its new keys, -1 for the
// keys it evicted) are queued and applied, coalesced in request order, by
// the next edge0_stager_wait or edge0_stager_flush.  A new key's entry may
// land before its copy finishes; only a set holding that key reads it, and
// such a set is ordered after the copy.
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

// Slot-table entries to set, passed by value (captured at launch); the
// entries of one launch have distinct indices.
constexpr int kMaxPatch = 384;
struct TablePatch {
  int n;
  int32_t idx[kMaxPatch];
  int32_t val[kMaxPatch];
};
__global__ void k_patch_table(int32_t* __restrict__ table, TablePatch p) {
  for (int i = threadIdx.x; i < p.n; i += blockDim.x) table[p.idx[i]] = p.val[i];
}

// One request's fills: bundle b of the list is copied from pinned host
// memory (read by the kernel over the host link) into its slot.  A kernel
// rather than the DMA engine: the copy then orders with the layer kernels on
// the compute stream without an engine switch, and 32 workgroups per bundle
// already saturate the link.
constexpr int kCopyWGs = 32;
struct CopyList {
  const uint4* src[16];
  uint4* dst[16];
};
__global__ __launch_bounds__(256) void k_stage_copy(CopyList c, int64_t n16) {
  const uint4* __restrict__ src = c.src[blockIdx.y];
  uint4* __restrict__ dst = c.dst[blockIdx.y];
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// A ring of events whose records carry serial numbers.  An entry is reused
// only after its previous record completed (a host wait, which also bounds
// how far the host runs ahead), so a serial that is no longer in the ring has
// completed and needs no wait.
struct EventRing {
  std::vector<hipEvent_t> ev;
  std::vector<uint64_t> serial;  // serial held by each entry, 0 = none
  std::vector<hipStream_t> stream;
  uint64_t last = 0;

  bool init(int n) {
    ev.assign(n, nullptr);
    serial.assign(n, 0);
    stream.assign(n, nullptr);
    for (int i = 0; i < n; ++i)
      if (hipEventCreateWithFlags(&ev[i], hipEventDisableTiming) != hipSuccess) return false;
    return true;
  }
  void destroy() {
    for (auto e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  // records the next serial on s; 0 on a HIP error
  uint64_t record(hipStream_t s) {
    const uint64_t q = last + 1;
    const size_t i = q % ev.size();
    if (serial[i] != 0 && hipEventSynchronize(ev[i]) != hipSuccess) return 0;
    if (hipEventRecord(ev[i], s) != hipSuccess) return 0;
    last = q;
    serial[i] = q;
    stream[i] = s;
    return q;
  }
  // the event a stream s must wait on to be ordered after record q, or
  // nullptr when no wait is needed (none, recycled, same stream, complete)
  hipEvent_t pending(uint64_t q, hipStream_t s) const {
    if (q == 0) return nullptr;
    const size_t i = q % ev.size();
    if (serial[i] != q || stream[i] == s) return nullptr;
    if (hipEventQuery(ev[i]) == hipSuccess) return nullptr;
    return ev[i];
  }
};
constexpr int kRing = 1024;

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
  std::vector<const void*> host;  // [L * E] device addresses of the pinned host bundles
  edge0_filetier* files = nullptr;  // or: misses are read from the layer files
  int32_t* table = nullptr;
  EventRing ready;  // recorded after each request's copies, on its stream
  EventRing rel;    // recorded at each release, on the compute stream
  // per slot: serial of the request that last filled it and of the last
  // release of a set that read it
  std::vector<uint64_t> fill_q, rel_q;
  struct Staged {
    hipStream_t stream;
    uint64_t q;
  };
  std::map<std::pair<int, int>, Staged> staged;  // pending (L, t)
  std::vector<std::pair<int32_t, int32_t>> patches;  // table updates not yet applied, in order
  int copy_mode = EDGE0_COPY_KERNEL;
};

// Applies the pending slot-table updates on `stream`, in request order (a
// later update of an entry replaces an earlier one).
static int flush_patches(edge0_stager* sg, hipStream_t stream) {
  if (sg->patches.empty()) return EDGE0_OK;
  std::map<int32_t, int32_t> last;
  for (const auto& pv : sg->patches) last[pv.first] = pv.second;
  sg->patches.clear();
  TablePatch p{};
  for (auto it = last.begin(); it != last.end();) {
    p.n = 0;
    for (; it != last.end() && p.n < kMaxPatch; ++it) {
      p.idx[p.n] = it->first;
      p.val[p.n++] = it->second;
    }
    k_patch_table<<<1, 256, 0, stream>>>(sg->table, p);
    E0_CHECK_LAUNCH();
  }
  return EDGE0_OK;
}

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
  (void)hipDeviceSynchronize();
  sg->ready.destroy();
  sg->rel.destroy();
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
  // every bundle must be pinned host memory the device can read, 16-byte
  // aligned; the kernels use its device address
  std::vector<const void*> dev_ptrs((size_t)n_layers * E);
  for (int64_t i = 0; i < (int64_t)n_layers * E; ++i) {
    if (!host_bundles[i] || reinterpret_cast<uintptr_t>(host_bundles[i]) % 16 != 0)
      return EDGE0_EINVAL;
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, host_bundles[i]) != hipSuccess) {
      (void)hipGetLastError();  // clear the sticky error of the failed query
      return EDGE0_EINVAL;
    }
    if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) return EDGE0_EINVAL;
    dev_ptrs[i] = attr.devicePointer;
  }
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
  sg->host = std::move(dev_ptrs);
  sg->table = slot_table;
  sg->fill_q.assign(pool->n_slots, 0);
  sg->rel_q.assign(pool->n_slots, 0);
  const bool ok = sg->ready.init(kRing) && sg->rel.init(kRing) &&
                  hipMemset(slot_table, 0xFF, (size_t)n_layers * E * 4) == hipSuccess &&
                  hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    edge0_stager_destroy(sg);
    return EDGE0_EHIP;
  }
  *out = sg;
  return EDGE0_OK;
}

extern "C" int edge0_stager_create_files(edge0_stager** out, const edge0_moe_shape* shape,
                                         const edge0_slot_pool* pool, int32_t n_layers,
                                         edge0_filetier* files, int32_t* slot_table) {
  if (!out || !shape || !shape_ok(shape) || !pool || !pool->base || pool->n_slots < 1 || !files ||
      !slot_table || n_layers < 1 || !filetier_matches(files, *shape, n_layers))
    return EDGE0_EINVAL;
  edge0_bundle_layout lay;
  if (bundle_layout(shape, &lay) != EDGE0_OK) return EDGE0_EINVAL;
  if (pool->slot_bytes < lay.bytes || pool->slot_bytes % 256 != 0) return EDGE0_EINVAL;
  edge0_stager* sg = new (std::nothrow) edge0_stager();
  if (!sg) return EDGE0_ENOMEM;
  int rc = sg->lru.init(pool->n_slots, n_layers, shape->n_experts);
  if (rc != EDGE0_OK) {
    delete sg;
    return rc;
  }
  sg->shape = *shape;
  sg->pool = *pool;
  sg->bundle_bytes = lay.bytes;
  sg->files = files;
  sg->table = slot_table;
  sg->fill_q.assign(pool->n_slots, 0);
  sg->rel_q.assign(pool->n_slots, 0);
  const bool ok = sg->ready.init(kRing) && sg->rel.init(kRing) &&
                  hipMemset(slot_table, 0xFF, (size_t)n_layers * shape->n_experts * 4) ==
                      hipSuccess &&
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
  // hazards: a hit on a slot filled on another stream waits for that fill; a
  // copy into a slot waits for the last release of a set that read it
  hipEvent_t waits[32];
  int n_waits = 0;
  auto add = [&](hipEvent_t e) {
    if (!e) return;
    for (int j = 0; j < n_waits; ++j)
      if (waits[j] == e) return;
    waits[n_waits++] = e;
  };
  for (int i = 0; i < n; ++i) {
    const int s = slots[i];
    add(sg->ready.pending(sg->fill_q[s], stream));
    if (!hit[i]) add(sg->rel.pending(sg->rel_q[s], stream));
  }
  for (int j = 0; j < n_waits; ++j)
    if (hipStreamWaitEvent(stream, waits[j], 0) != hipSuccess) return EDGE0_EHIP;
  uint8_t* base = static_cast<uint8_t*>(sg->pool.base);
  // file tier: the misses' records read into staging buffers first
  const void* staged_src[16];
  int staged_buf[16];
  int n_miss = 0;
  if (sg->files) {
    int32_t miss_keys[16];
    for (int i = 0; i < n; ++i)
      if (!hit[i]) miss_keys[n_miss++] = keys[i];
    if (n_miss > 0 && (rc = filetier_read(sg->files, miss_keys, n_miss, staged_src, staged_buf)) !=
                          EDGE0_OK)
      return rc;
  }
  CopyList cl{};
  int n_copy = 0;
  for (int i = 0; i < n; ++i) {
    if (hit[i]) continue;
    const int s = slots[i];
    cl.src[n_copy] = static_cast<const uint4*>(sg->files ? staged_src[n_copy] : sg->host[keys[i]]);
    cl.dst[n_copy++] = reinterpret_cast<uint4*>(base + (size_t)s * sg->pool.slot_bytes);
    sg->lru.stats.bytes_staged += sg->bundle_bytes;
    if (evicted[i] >= 0) sg->patches.emplace_back(evicted[i], -1);
    sg->patches.emplace_back(keys[i], s);
  }
  if (n_copy > 0 && sg->copy_mode == EDGE0_COPY_KERNEL) {
    k_stage_copy<<<dim3(kCopyWGs, n_copy), 256, 0, stream>>>(cl, sg->bundle_bytes / 16);
    E0_CHECK_LAUNCH();
  }
  for (int i = 0; i < n_copy && sg->copy_mode == EDGE0_COPY_DMA; ++i)
    if (hipMemcpyAsync(cl.dst[i], cl.src[i], (size_t)sg->bundle_bytes, hipMemcpyHostToDevice,
                       stream) != hipSuccess)
      return EDGE0_EHIP;
  if (sg->files && n_miss > 0 && (rc = filetier_mark(sg->files, staged_buf, n_miss, stream)) != EDGE0_OK)
    return rc;
  const uint64_t q = sg->ready.record(stream);
  if (q == 0) return EDGE0_EHIP;
  for (int i = 0; i < n; ++i)
    if (!hit[i]) {
      sg->fill_q[slots[i]] = q;
      sg->rel_q[slots[i]] = 0;
    }
  sg->staged[{layer, step}] = {stream, q};
  if (slots_out)
    for (int i = 0; i < n; ++i) slots_out[i] = slots[i];
  return EDGE0_OK;
}

extern "C" int edge0_stager_wait(edge0_stager* sg, int32_t layer, int32_t step,
                                 hipStream_t compute_stream) {
  if (!sg) return EDGE0_EINVAL;
  auto it = sg->staged.find({layer, step});
  if (it == sg->staged.end()) return EDGE0_EINVAL;
  int rc = flush_patches(sg, compute_stream);
  if (rc != EDGE0_OK) return rc;
  hipEvent_t e = sg->ready.pending(it->second.q, compute_stream);
  if (e && hipStreamWaitEvent(compute_stream, e, 0) != hipSuccess) return EDGE0_EHIP;
  return EDGE0_OK;
}

extern "C" int edge0_stager_release(edge0_stager* sg, int32_t layer, int32_t step,
                                    hipStream_t compute_stream) {
  if (!sg) return EDGE0_EINVAL;
  if (!sg->lru.pending.count({layer, step})) return EDGE0_EINVAL;
  const uint64_t q = sg->rel.record(compute_stream);
  if (q == 0) return EDGE0_EHIP;
  std::vector<int32_t> keys;
  const int rc = sg->lru.release(layer, step, &keys);
  if (rc != EDGE0_OK) return rc;
  for (int key : keys) {
    const int s = sg->lru.slot_of[key];
    if (s >= 0) sg->rel_q[s] = q;
  }
  sg->staged.erase({layer, step});
  return EDGE0_OK;
}

extern "C" int edge0_stager_flush(edge0_stager* sg, hipStream_t compute_stream) {
  if (!sg) return EDGE0_EINVAL;
  return flush_patches(sg, compute_stream);
}

extern "C" int edge0_stager_set_copy_mode(edge0_stager* sg, int32_t mode) {
  if (!sg || (mode != EDGE0_COPY_KERNEL && mode != EDGE0_COPY_DMA)) return EDGE0_EINVAL;
  sg->copy_mode = mode;
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
