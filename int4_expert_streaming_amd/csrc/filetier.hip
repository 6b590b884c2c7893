// Expert files under the pinned host tier: the weights' home is the SSD
// ([Edge0] = "The Other Half of the Memory Wall: Serving 35B MoEs from SSD
// with Trained Routing Prediction", §3.1 "Problem" and Figure 1: SSD, page
// cache, staged slots; the checkpoint stacked per layer so a layer's experts
// are direct reads).  Host code only.
//
// A layer file is a 4096-byte header (magic, version, layer, expert count,
// bundle and record sizes, the shape) followed by one record per expert: the
// bundle in the device layout, zero-padded to a multiple of 4096 bytes, so
// with O_DIRECT every read is aligned and bypasses the page cache.
//
// The file tier owns the open files, a ring of pinned staging buffers (one
// record each) and a pool of I/O threads (with O_DIRECT each reads into an
// aligned buffer of its own, then copies into the pinned one).  A stager created on it reads a
// request's misses in parallel into staging buffers (pread; a buffer is
// reused once the copy that last read it has completed: an event per
// buffer) and then copies them into their slots as it copies host bundles.
#include <fcntl.h>
#include <unistd.h>

#include <chrono>
#include <condition_variable>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <thread>

#include "moe_internal.h"

namespace e0 {

constexpr int64_t kFileAlign = 4096;
constexpr char kFileMagic[8] = {'E', '0', 'L', 'A', 'Y', 'E', 'R', '1'};

struct FileHeader {
  char magic[8];
  int32_t version, layer, n_experts, pad0;
  int64_t bundle_bytes, record_bytes;
  edge0_moe_shape shape;
};
static_assert(sizeof(FileHeader) <= kFileAlign, "header exceeds its block");

static int64_t record_bytes_of(int64_t bundle_bytes) {
  return (bundle_bytes + kFileAlign - 1) / kFileAlign * kFileAlign;
}

// whole-range pread (partial reads and interrupts retried); false on error
static bool pread_all(int fd, void* dst, int64_t bytes, int64_t off) {
  uint8_t* p = static_cast<uint8_t*>(dst);
  while (bytes > 0) {
    const ssize_t n = ::pread(fd, p, (size_t)bytes, (off_t)off);
    if (n < 0 && errno == EINTR) continue;
    if (n <= 0) return false;
    p += n;
    off += n;
    bytes -= n;
  }
  return true;
}

}  // namespace e0

using namespace e0;

struct edge0_filetier {
  edge0_moe_shape shape;
  int n_layers = 0, E = 0, flags = 0;
  int64_t bundle_bytes = 0, record_bytes = 0;
  std::vector<int> fds;
  // staging ring
  std::vector<void*> buf;       // pinned host, record_bytes each
  std::vector<void*> buf_dev;   // their device addresses
  std::vector<hipEvent_t> buf_ev;
  std::vector<char> buf_used;   // an event has been recorded for the buffer
  int next = 0;
  // I/O pool
  struct Task {
    int fd;
    int64_t off;
    void* dst;
  };
  std::vector<std::thread> threads;
  std::mutex m;
  std::condition_variable cv_task, cv_done;
  std::deque<Task> tasks;
  int outstanding = 0;
  bool failed = false, stop = false;
  edge0_file_stats stats{};

  // A direct read cannot target the pinned staging memory (the kernel
  // refuses to pin those pages for I/O: EFAULT), so with O_DIRECT each I/O
  // thread reads into its own aligned bounce buffer and copies from there.
  void worker() {
    void* bounce = nullptr;
    if ((flags & EDGE0_FILE_DIRECT) && posix_memalign(&bounce, kFileAlign, (size_t)record_bytes) != 0)
      bounce = nullptr;
    for (;;) {
      Task t;
      {
        std::unique_lock<std::mutex> lk(m);
        cv_task.wait(lk, [&] { return stop || !tasks.empty(); });
        if (stop && tasks.empty()) break;
        t = tasks.front();
        tasks.pop_front();
      }
      bool ok;
      if (flags & EDGE0_FILE_DIRECT) {
        ok = bounce != nullptr && pread_all(t.fd, bounce, record_bytes, t.off);
        if (ok) std::memcpy(t.dst, bounce, (size_t)record_bytes);
      } else {
        ok = pread_all(t.fd, t.dst, record_bytes, t.off);
      }
      {
        std::lock_guard<std::mutex> lk(m);
        if (!ok) failed = true;
        if (--outstanding == 0) cv_done.notify_all();
      }
    }
    free(bounce);
  }
};

extern "C" int64_t edge0_layer_file_record_bytes(const edge0_moe_shape* shape) {
  edge0_bundle_layout lay;
  if (!shape || bundle_layout(shape, &lay) != EDGE0_OK) return 0;
  return record_bytes_of(lay.bytes);
}

extern "C" int edge0_layer_file_write(const char* path, const edge0_moe_shape* shape,
                                      int32_t layer, const void* const* bundles) {
  edge0_bundle_layout lay;
  if (!path || !shape || !bundles || layer < 0 || bundle_layout(shape, &lay) != EDGE0_OK)
    return EDGE0_EINVAL;
  const int E = shape->n_experts;
  for (int e = 0; e < E; ++e)
    if (!bundles[e]) return EDGE0_EINVAL;
  const int fd = ::open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644);
  if (fd < 0) return EDGE0_EINVAL;
  const int64_t rec = record_bytes_of(lay.bytes);
  std::vector<uint8_t> block((size_t)std::max<int64_t>(rec, kFileAlign), 0);
  FileHeader h{};
  std::memcpy(h.magic, kFileMagic, 8);
  h.version = 1;
  h.layer = layer;
  h.n_experts = E;
  h.bundle_bytes = lay.bytes;
  h.record_bytes = rec;
  h.shape = *shape;
  std::memcpy(block.data(), &h, sizeof h);
  auto write_all = [&](const void* p, int64_t n) {
    const uint8_t* q = static_cast<const uint8_t*>(p);
    while (n > 0) {
      const ssize_t w = ::write(fd, q, (size_t)n);
      if (w < 0 && errno == EINTR) continue;
      if (w <= 0) return false;
      q += w;
      n -= w;
    }
    return true;
  };
  bool ok = write_all(block.data(), kFileAlign);
  for (int e = 0; ok && e < E; ++e) {
    std::memcpy(block.data(), bundles[e], (size_t)lay.bytes);
    std::memset(block.data() + lay.bytes, 0, (size_t)(rec - lay.bytes));
    ok = write_all(block.data(), rec);
  }
  ok = ::close(fd) == 0 && ok;
  return ok ? EDGE0_OK : EDGE0_EINVAL;
}

extern "C" void edge0_filetier_destroy(edge0_filetier* ft) {
  if (!ft) return;
  {
    std::lock_guard<std::mutex> lk(ft->m);
    ft->stop = true;
  }
  ft->cv_task.notify_all();
  for (auto& t : ft->threads) t.join();
  (void)hipDeviceSynchronize();  // copies from the staging buffers have ended
  for (auto e : ft->buf_ev)
    if (e) (void)hipEventDestroy(e);
  for (auto p : ft->buf)
    if (p) (void)hipHostFree(p);
  for (int fd : ft->fds)
    if (fd >= 0) ::close(fd);
  delete ft;
}

extern "C" int edge0_filetier_create(edge0_filetier** out, const edge0_moe_shape* shape,
                                     int32_t n_layers, const char* const* paths,
                                     int32_t n_buffers, int32_t n_threads, int32_t flags) {
  edge0_bundle_layout lay;
  if (!out || !shape || !shape_ok(shape) || !paths || n_layers < 1 || n_buffers < 16 ||
      n_buffers > 4096 || n_threads < 1 || n_threads > 64 || (flags & ~EDGE0_FILE_DIRECT) != 0 ||
      bundle_layout(shape, &lay) != EDGE0_OK)
    return EDGE0_EINVAL;
  edge0_filetier* ft = new (std::nothrow) edge0_filetier();
  if (!ft) return EDGE0_ENOMEM;
  ft->shape = *shape;
  ft->n_layers = n_layers;
  ft->E = shape->n_experts;
  ft->flags = flags;
  ft->bundle_bytes = lay.bytes;
  ft->record_bytes = record_bytes_of(lay.bytes);
  ft->fds.assign(n_layers, -1);
  // every file: readable, its header this layer's and this shape's, long enough
  for (int L = 0; L < n_layers; ++L) {
    if (!paths[L]) {
      edge0_filetier_destroy(ft);
      return EDGE0_EINVAL;
    }
    const int fd = ::open(paths[L], O_RDONLY | ((flags & EDGE0_FILE_DIRECT) ? O_DIRECT : 0));
    ft->fds[L] = fd;
    FileHeader h{};
    void* hb = nullptr;
    bool ok = fd >= 0 && posix_memalign(&hb, kFileAlign, kFileAlign) == 0 &&
              pread_all(fd, hb, kFileAlign, 0);
    if (ok) std::memcpy(&h, hb, sizeof h);
    free(hb);
    const off_t end = ok ? ::lseek(fd, 0, SEEK_END) : 0;
    ok = ok && std::memcmp(h.magic, kFileMagic, 8) == 0 && h.version == 1 && h.layer == L &&
         h.n_experts == ft->E && h.bundle_bytes == lay.bytes && h.record_bytes == ft->record_bytes &&
         std::memcmp(&h.shape, shape, sizeof(edge0_moe_shape)) == 0 &&
         (int64_t)end >= kFileAlign + (int64_t)ft->E * ft->record_bytes;
    if (!ok) {
      edge0_filetier_destroy(ft);
      return EDGE0_EINVAL;
    }
  }
  ft->buf.assign(n_buffers, nullptr);
  ft->buf_dev.assign(n_buffers, nullptr);
  ft->buf_ev.assign(n_buffers, nullptr);
  ft->buf_used.assign(n_buffers, 0);
  for (int b = 0; b < n_buffers; ++b) {
    hipPointerAttribute_t attr{};
    if (hipHostMalloc(&ft->buf[b], (size_t)ft->record_bytes, hipHostMallocDefault) != hipSuccess ||
        hipPointerGetAttributes(&attr, ft->buf[b]) != hipSuccess || !attr.devicePointer ||
        hipEventCreateWithFlags(&ft->buf_ev[b], hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      edge0_filetier_destroy(ft);
      return EDGE0_ENOMEM;
    }
    ft->buf_dev[b] = attr.devicePointer;
  }
  for (int t = 0; t < n_threads; ++t) ft->threads.emplace_back([ft] { ft->worker(); });
  *out = ft;
  return EDGE0_OK;
}

extern "C" int edge0_filetier_stats(const edge0_filetier* ft, edge0_file_stats* out) {
  if (!ft || !out) return EDGE0_EINVAL;
  *out = ft->stats;
  return EDGE0_OK;
}

namespace e0 {
// Reads the bundles of keys[0..n) (key = layer * E + expert) into staging
// buffers and returns their device addresses; the buffers' events are
// recorded on `stream` by filetier_mark once their copies are enqueued.
int filetier_read(edge0_filetier* ft, const int32_t* keys, int n, const void** dev_out,
                  int* buf_out) {
  if (n > (int)ft->buf.size()) return EDGE0_EINVAL;
  const auto t0 = std::chrono::steady_clock::now();
  {
    std::unique_lock<std::mutex> lk(ft->m);
    ft->failed = false;
  }
  for (int i = 0; i < n; ++i) {
    const int b = ft->next;
    ft->next = (ft->next + 1) % (int)ft->buf.size();
    if (ft->buf_used[b] && hipEventSynchronize(ft->buf_ev[b]) != hipSuccess) return EDGE0_EHIP;
    buf_out[i] = b;
    dev_out[i] = ft->buf_dev[b];
    const int L = keys[i] / ft->E, e = keys[i] % ft->E;
    std::lock_guard<std::mutex> lk(ft->m);
    ft->tasks.push_back({ft->fds[L], kFileAlign + (int64_t)e * ft->record_bytes, ft->buf[b]});
    ++ft->outstanding;
  }
  ft->cv_task.notify_all();
  bool failed;
  {
    std::unique_lock<std::mutex> lk(ft->m);
    ft->cv_done.wait(lk, [&] { return ft->outstanding == 0; });
    failed = ft->failed;
  }
  ft->stats.reads += n;
  ft->stats.bytes += (int64_t)n * ft->record_bytes;
  ft->stats.read_ns +=
      std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0)
          .count();
  return failed ? EDGE0_EINVAL : EDGE0_OK;
}
int filetier_mark(edge0_filetier* ft, const int* bufs, int n, hipStream_t stream) {
  for (int i = 0; i < n; ++i) {
    if (hipEventRecord(ft->buf_ev[bufs[i]], stream) != hipSuccess) return EDGE0_EHIP;
    ft->buf_used[bufs[i]] = 1;
  }
  return EDGE0_OK;
}
bool filetier_matches(const edge0_filetier* ft, const edge0_moe_shape& s, int n_layers) {
  return std::memcmp(&ft->shape, &s, sizeof s) == 0 && ft->n_layers >= n_layers;
}
}  // namespace e0
