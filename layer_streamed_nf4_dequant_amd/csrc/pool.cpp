// The layer pool: K device slots, a copy stream, and events that order each slot's refill
// after the compute that last read it.
//
// "Can You Fine-Tune a 27B Model on a Laptop? (I Did the Math)", transcript @7:11-7:32: the
// frozen base sits in host RAM; one decoder layer at a time is copied into a small on-card
// buffer on a separate stream, so the copy lands while the previous layer computes; each
// layer crosses the host link two times in a step (forward, and the backward's recompute). "An 8B Fine-Tune Now
// Fits in 4 GB of VRAM": the buffers are pre-allocated. "Exact Layer Streaming", Abstract:
// the silent wrong-gradient defect at large layer sizes was aliasing, not a race; the audit
// below checks that every visit reads exactly its own layer's bytes.
//
// State of a slot: FREE (may be refilled once its release event has fired), PENDING (a copy
// for `layer` has been enqueued, ready event recorded), ACQUIRED (compute is using it).
// Two backends share the state machine: HIP (device slots, hipMemcpyAsync on the copy stream,
// hipEvents) and HOST_SIM (host slots, memcpy, no events) for tests without a GPU.
//
// Memory: the slots, the audit's checksum array and the file tier's two pinned bounce buffers
// are the caller's (lsn_pool_buffers); the pool owns only its host state, its events and the
// I/O thread, and allocates no device or pinned memory.
//
// File tier (LSN_POOL_FILE_TIER; "Soup v0.73.0 benchmarks README", record index: the disk tier,
// and "An 8B Fine-Tune Now Fits in 4 GB of VRAM": the frozen base stays in host RAM, or on NVMe
// when RAM is short): a layer registered from a file is read by the pool's I/O thread, split
// over kReaders reader threads, into one of two pinned bounce buffers, and copied from there on
// the copy stream. The bounce buffers alternate, so the next layer is read while the last one
// crosses the link; a bounce buffer is reused only after its copy's event. prefetch() posts the
// fill and returns; acquire() waits (on the host) until the I/O thread has enqueued that fill's
// copy and recorded its ready event, then makes the compute stream wait for the event.
// With LSN_POOL_FILE_DIRECT the reads bypass the page cache (O_DIRECT): every read is a read
// of the storage device, in 4096-byte aligned pieces (the image's file region padded to whole
// 4 KiB blocks), so the tier's rate is the disk's, not RAM's. Direct I/O cannot target the
// driver's pinned host memory (the kernel refuses to map it for the transfer), so each reader
// reads its piece into a plain host staging buffer and copies it into the pinned bounce buffer.

#include <fcntl.h>
#include <unistd.h>

#include <atomic>
#include <cerrno>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "common.h"
#include "pool_checksum.h"

namespace lsn {
lsn_status require_gfx950();
}

using namespace lsn;

namespace {

enum SlotState { FREE = 0, PENDING = 1, ACQUIRED = 2 };

struct Slot {
  void *mem = nullptr;
  int layer = -1;          // layer whose image the slot holds or is receiving
  bool valid = false;      // holds an intact copy of `layer` (poisoned slots are not valid)
  SlotState state = FREE;
  uint64_t fill_ticket = 0;  // file tier: the I/O job filling the slot (0: none)
  uint64_t gen = 0;        // number of fills
  uint64_t acquired_gen = 0;
  uint64_t released_tick = 0;
  bool release_recorded = false;
  hipEvent_t ready = nullptr;
  hipEvent_t released = nullptr;
};

struct LayerInfo {
  const void *host = nullptr;
  int fd = -1;              // file tier: the image is bytes at file_off of this file
  uint64_t file_off = 0;
  size_t bytes = 0;
  size_t span = 0;          // file tier: bytes read per fill (bytes, or rounded up to 4 KiB with O_DIRECT)
  uint64_t checksum = 0;
  int visits = 0;           // prefetches so far (a layer's first visit is 1)
};

struct FillJob {
  uint64_t ticket;
  int slot;
  int layer;
  bool skip;                // a planted stale re-fetch: no read, no copy
};

constexpr int kReaders = 8;
constexpr size_t kDirectAlign = 4096;       // O_DIRECT: offset, length and buffer alignment

struct AuditRecord {
  int layer;
  int visit;
  int at_release;           // 0 = taken at acquire, 1 = at release
};

}  // namespace

struct lsn_pool {
  int n_slots = 0;
  size_t slot_bytes = 0;
  int n_layers = 0;
  hipStream_t copy = nullptr;
  uint32_t flags = 0;
  bool sim = false;
  std::vector<Slot> slots;
  std::vector<LayerInfo> layers;
  lsn_pool_stats stats{};
  uint64_t tick = 0;
  // audit
  unsigned long long *sums = nullptr;        // caller's checksum array (device; host under HOST_SIM)
  size_t audit_capacity = 0;
  std::vector<AuditRecord> records;
  // file tier
  bool file_tier = false;
  void *bounce[2] = {nullptr, nullptr};      // caller's pinned (host-sim: plain) read buffers
  void *stage[2] = {nullptr, nullptr};       // caller's plain host buffers for O_DIRECT reads
  hipEvent_t bounce_free[2] = {nullptr, nullptr};
  bool bounce_used[2] = {false, false};
  int next_bounce = 0;
  std::thread io;
  std::mutex mu;
  std::condition_variable cv_job, cv_done;
  std::deque<FillJob> jobs;
  uint64_t tickets = 0;                      // last ticket handed out
  uint64_t done = 0;                         // every ticket <= done has been enqueued (in order)
  bool stop = false;
  std::string io_error;                      // first I/O-thread failure, reported by acquire
};

namespace {

bool audit_on(const lsn_pool *p) { return (p->flags & LSN_POOL_AUDIT) != 0; }

lsn_status check_pool(const lsn_pool *p, const char *what) {
  if (!p) return fail(LSN_E_ARG, "%s: null pool", what);
  return LSN_OK;
}

lsn_status check_layer(const lsn_pool *p, int layer, const char *what) {
  if (layer < 0 || layer >= p->n_layers)
    return fail(LSN_E_ARG, "%s: layer %d out of range [0, %d)", what, layer, p->n_layers);
  if (!p->layers[layer].host && p->layers[layer].fd < 0)
    return fail(LSN_E_STATE, "%s: layer %d not registered", what, layer);
  return LSN_OK;
}

int find_slot(const lsn_pool *p, int layer, SlotState st) {
  for (int i = 0; i < p->n_slots; ++i)
    if (p->slots[i].layer == layer && p->slots[i].state == st) return i;
  return -1;
}

// A layer registered anew: a free slot still holding its old bytes must not serve it again
// (KEEP_AT_TURN reuse would skip the copy).
void forget_copies(lsn_pool *p, int layer) {
  for (Slot &s : p->slots)
    if (s.layer == layer && s.state == FREE) s.valid = false;
}

lsn_status record_checksum(lsn_pool *p, const void *mem, size_t bytes, int layer, int at_release,
                           hipStream_t s) {
  if (p->records.size() >= p->audit_capacity)
    return fail(LSN_E_STATE, "audit capacity (%zu checksums) exhausted: call layer_pool_audit",
                p->audit_capacity);
  const size_t idx = p->records.size();
  p->records.push_back({layer, p->layers[layer].visits, at_release});
  if (p->sim) {
    p->sums[idx] = checksum_host(mem, bytes);
    return LSN_OK;
  }
  return check_hip(launch_checksum(mem, bytes, p->sums + idx, s), "audit checksum launch");
}

lsn_status do_prefetch(lsn_pool *p, int layer) {
  if (find_slot(p, layer, PENDING) >= 0) return LSN_OK;   // already in flight
  if (find_slot(p, layer, ACQUIRED) >= 0)
    return fail(LSN_E_STATE, "layer_pool_prefetch: layer %d is acquired; release it first", layer);
  LayerInfo &L = p->layers[layer];
  // reuse a free slot that still holds this layer intact (KEEP_AT_TURN only)
  if (p->flags & LSN_POOL_KEEP_AT_TURN) {
    for (int i = 0; i < p->n_slots; ++i) {
      Slot &s = p->slots[i];
      if (s.state == FREE && s.layer == layer && s.valid) {
        s.state = PENDING;
        ++p->stats.hits;
        ++L.visits;
        return LSN_OK;
      }
    }
  }
  // victim: a free slot, never-used first, else the one released longest ago
  int victim = -1;
  for (int i = 0; i < p->n_slots; ++i) {
    const Slot &s = p->slots[i];
    if (s.state != FREE) continue;
    if (victim < 0) { victim = i; continue; }
    const Slot &v = p->slots[victim];
    const bool s_unused = s.layer < 0, v_unused = v.layer < 0;
    if ((s_unused && !v_unused) || (s_unused == v_unused && s.released_tick < v.released_tick)) victim = i;
  }
  if (victim < 0)
    return fail(LSN_E_STATE, "layer_pool_prefetch: all %d slots are acquired or pending", p->n_slots);
  Slot &s = p->slots[victim];
  ++L.visits;
  const bool refetch = L.visits >= 2;
  const bool skip_copy = refetch && (p->flags & LSN_FAULT_STALE_REFETCH);
  s.fill_ticket = 0;
  if (L.fd >= 0) {
    // file tier: the I/O thread reads and copies; the slot's events are its from here on
    std::lock_guard<std::mutex> g(p->mu);
    s.fill_ticket = ++p->tickets;
    p->jobs.push_back({s.fill_ticket, victim, layer, skip_copy});
    p->cv_job.notify_one();
  } else if (p->sim) {
    if (!skip_copy) std::memcpy(s.mem, L.host, L.bytes);
  } else {
    hipError_t e = hipSuccess;
    if (s.release_recorded) e = hipStreamWaitEvent(p->copy, s.released, 0);
    if (e == hipSuccess && !skip_copy)
      e = hipMemcpyAsync(s.mem, L.host, L.bytes, hipMemcpyHostToDevice, p->copy);
    if (e == hipSuccess) e = hipEventRecord(s.ready, p->copy);
    if (e != hipSuccess) return check_hip(e, "layer_pool_prefetch copy");
  }
  s.layer = layer;
  s.valid = !skip_copy;
  s.state = PENDING;
  ++s.gen;
  if (!skip_copy) {
    ++p->stats.copies;
    p->stats.bytes_copied += L.bytes;
  }
  return LSN_OK;
}

// Reads bytes at off of fd into dst, split over kReaders threads in pieces that are multiples of
// `align` (for O_DIRECT); with `stage`, each piece is read into the same place of stage and then
// copied to dst. False (with errno text in err) on a short or failed read.
bool read_parallel(int fd, uint64_t off, size_t bytes, void *dst, std::string &err, size_t align = 1,
                   void *stage = nullptr) {
  std::atomic<bool> ok{true};
  std::string first_err;
  std::mutex emu;
  auto part = [&](int k) {
    const size_t chunk = ((bytes + kReaders - 1) / kReaders + align - 1) / align * align;
    size_t a = (size_t)k * chunk, b = a + chunk < bytes ? a + chunk : bytes;
    char *into = static_cast<char *>(stage ? stage : dst);
    const size_t a0 = a;
    while (a < b) {
      const ssize_t n = pread(fd, into + a, b - a, (off_t)(off + a));
      if (n <= 0) {
        std::lock_guard<std::mutex> g(emu);
        if (first_err.empty()) first_err = n == 0 ? "unexpected end of file" : std::strerror(errno);
        ok = false;
        return;
      }
      a += (size_t)n;
    }
    if (stage && b > a0) std::memcpy(static_cast<char *>(dst) + a0, into + a0, b - a0);
  };
  std::vector<std::thread> th;
  for (int k = 1; k < kReaders; ++k) th.emplace_back(part, k);
  part(0);
  for (auto &t : th) t.join();
  if (!ok) err = first_err;
  return ok;
}

// The I/O thread: takes fill jobs in order, reads each layer into the next bounce buffer, and
// enqueues its copy into the job's slot on the copy stream (after the slot's release event).
void io_loop(lsn_pool *p) {
  for (;;) {
    FillJob job;
    {
      std::unique_lock<std::mutex> g(p->mu);
      p->cv_job.wait(g, [&] { return p->stop || !p->jobs.empty(); });
      if (p->jobs.empty()) return;           // stop requested and nothing left
      job = p->jobs.front();
      p->jobs.pop_front();
    }
    Slot &s = p->slots[job.slot];
    const LayerInfo &L = p->layers[job.layer];
    std::string err;
    hipError_t e = hipSuccess;
    if (!job.skip) {
      const int b = p->next_bounce;
      p->next_bounce ^= 1;
      if (!p->sim && p->bounce_used[b]) e = hipEventSynchronize(p->bounce_free[b]);
      const bool direct = (p->flags & LSN_POOL_FILE_DIRECT) != 0;
      if (e == hipSuccess && !read_parallel(L.fd, L.file_off, L.span, p->bounce[b], err, direct ? kDirectAlign : 1,
                                            direct ? p->stage[b] : nullptr))
        err = "read: " + err;
      if (err.empty() && e == hipSuccess) {
        if (p->sim) {
          std::memcpy(s.mem, p->bounce[b], L.bytes);
        } else {
          if (s.release_recorded) e = hipStreamWaitEvent(p->copy, s.released, 0);
          if (e == hipSuccess) e = hipMemcpyAsync(s.mem, p->bounce[b], L.bytes, hipMemcpyHostToDevice, p->copy);
          if (e == hipSuccess) e = hipEventRecord(p->bounce_free[b], p->copy);
          p->bounce_used[b] = true;
        }
      }
    }
    if (err.empty() && e == hipSuccess && !p->sim) e = hipEventRecord(s.ready, p->copy);
    if (e != hipSuccess) err = std::string("HIP: ") + hipGetErrorString(e);
    {
      std::lock_guard<std::mutex> g(p->mu);
      if (!err.empty() && p->io_error.empty()) p->io_error = err;
      p->done = job.ticket;
    }
    p->cv_done.notify_all();
  }
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

bool is_pinned_host(const void *ptr) {
  hipPointerAttribute_t attr;
  const hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeHost;
}

}  // namespace

extern "C" {

lsn_status layer_pool_create(int32_t n_slots, size_t slot_bytes, void *const *slots, int32_t n_layers,
                             void *copy_stream, uint32_t flags, const lsn_pool_buffers *bufs, lsn_pool **out) {
  if (!out) return fail(LSN_E_ARG, "layer_pool_create: null out");
  *out = nullptr;
  if (n_slots < 1 || n_layers < 1 || slot_bytes == 0 || !slots)
    return fail(LSN_E_ARG, "layer_pool_create: need n_slots >= 1, n_layers >= 1, slot_bytes > 0, slots");
  if (slot_bytes % 256 != 0) return fail(LSN_E_ARG, "layer_pool_create: slot_bytes must be a multiple of 256");
  for (int i = 0; i < n_slots; ++i) {
    if (!slots[i] || ((uintptr_t)slots[i] & 255))
      return fail(LSN_E_ARG, "layer_pool_create: slot %d is null or not 256-byte aligned", i);
    for (int j = 0; j < i; ++j)
      if (overlaps(slots[i], slot_bytes, slots[j], slot_bytes))
        return fail(LSN_E_ARG, "layer_pool_create: slots %d and %d overlap", j, i);
  }
  const bool sim = (flags & LSN_POOL_HOST_SIM) != 0;
  const bool audit = (flags & LSN_POOL_AUDIT) != 0, file_tier = (flags & LSN_POOL_FILE_TIER) != 0;
  if (!sim) {
    lsn_status st = require_gfx950();
    if (st != LSN_OK) return st;
    if (!copy_stream) return fail(LSN_E_ARG, "layer_pool_create: the copy stream must be a created stream");
  }
  if ((audit || file_tier) && !bufs)
    return fail(LSN_E_ARG, "layer_pool_create: LSN_POOL_AUDIT and LSN_POOL_FILE_TIER need the caller's buffers");
  if (audit) {
    if (!bufs->audit_sums || bufs->audit_capacity < 1 || ((uintptr_t)bufs->audit_sums & 7))
      return fail(LSN_E_ARG, "layer_pool_create: LSN_POOL_AUDIT needs an 8-byte aligned checksum array "
                  "of audit_capacity >= 1 entries");
    for (int i = 0; i < n_slots; ++i)
      if (overlaps(bufs->audit_sums, bufs->audit_capacity * 8, slots[i], slot_bytes))
        return fail(LSN_E_ARG, "layer_pool_create: the checksum array overlaps slot %d", i);
  }
  if (file_tier) {
    for (int b = 0; b < 2; ++b) {
      if (!bufs->bounce[b])
        return fail(LSN_E_ARG, "layer_pool_create: LSN_POOL_FILE_TIER needs two bounce buffers of slot_bytes");
      if (!sim && !is_pinned_host(bufs->bounce[b]))
        return fail(LSN_E_ARG, "layer_pool_create: bounce buffer %d is not pinned host memory", b);
    }
    if (overlaps(bufs->bounce[0], slot_bytes, bufs->bounce[1], slot_bytes))
      return fail(LSN_E_ARG, "layer_pool_create: the two bounce buffers overlap");
  }
  if (flags & LSN_POOL_FILE_DIRECT) {
    if (!file_tier) return fail(LSN_E_ARG, "layer_pool_create: LSN_POOL_FILE_DIRECT needs LSN_POOL_FILE_TIER");
    if (slot_bytes % kDirectAlign || !bufs->direct_stage[0] || !bufs->direct_stage[1] ||
        ((uintptr_t)bufs->direct_stage[0] % kDirectAlign) || ((uintptr_t)bufs->direct_stage[1] % kDirectAlign))
      return fail(LSN_E_ARG, "layer_pool_create: LSN_POOL_FILE_DIRECT needs slot_bytes a multiple of %zu and "
                  "two staging buffers of slot_bytes aligned to it", kDirectAlign);
    if (overlaps(bufs->direct_stage[0], slot_bytes, bufs->direct_stage[1], slot_bytes))
      return fail(LSN_E_ARG, "layer_pool_create: the two staging buffers overlap");
  }
  lsn_pool *p = new lsn_pool();
  p->file_tier = (flags & LSN_POOL_FILE_TIER) != 0;
  p->n_slots = n_slots;
  p->slot_bytes = slot_bytes;
  p->n_layers = n_layers;
  p->copy = (hipStream_t)copy_stream;
  p->flags = flags;
  p->sim = sim;
  p->slots.resize(n_slots);
  p->layers.resize(n_layers);
  for (int i = 0; i < n_slots; ++i) p->slots[i].mem = slots[i];
  if (audit) {
    p->sums = bufs->audit_sums;
    p->audit_capacity = bufs->audit_capacity;
  }
  if (file_tier) p->bounce[0] = bufs->bounce[0], p->bounce[1] = bufs->bounce[1];
  if (flags & LSN_POOL_FILE_DIRECT) p->stage[0] = bufs->direct_stage[0], p->stage[1] = bufs->direct_stage[1];
  hipError_t e = hipSuccess;
  if (!sim) {
    for (int i = 0; i < n_slots && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&p->slots[i].ready, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&p->slots[i].released, hipEventDisableTiming);
    }
    // the checksums are added into with integer atomics: they start at zero
    if (e == hipSuccess && audit) e = hipMemset(p->sums, 0, p->audit_capacity * sizeof(unsigned long long));
    for (int b = 0; b < 2 && e == hipSuccess && file_tier; ++b)
      e = hipEventCreateWithFlags(&p->bounce_free[b], hipEventDisableTiming);
  } else if (audit) {
    std::memset(p->sums, 0, p->audit_capacity * sizeof(unsigned long long));
  }
  if (e == hipSuccess && file_tier) p->io = std::thread(io_loop, p);
  if (e != hipSuccess) {
    lsn_status st = check_hip(e, "layer_pool_create");
    layer_pool_destroy(p);
    return st;
  }
  *out = p;
  return LSN_OK;
}

lsn_status layer_pool_register(lsn_pool *p, int32_t layer, const void *host_image, size_t bytes) {
  lsn_status st = check_pool(p, "layer_pool_register");
  if (st != LSN_OK) return st;
  if (layer < 0 || layer >= p->n_layers)
    return fail(LSN_E_ARG, "layer_pool_register: layer %d out of range [0, %d)", layer, p->n_layers);
  if (!host_image || bytes == 0) return fail(LSN_E_ARG, "layer_pool_register: empty image");
  if (bytes % 256 != 0) return fail(LSN_E_ARG, "layer_pool_register: image bytes must be a multiple of 256");
  if (bytes > p->slot_bytes)
    return fail(LSN_E_NOFIT, "layer_pool_register: layer %d image (%zu B) does not fit a slot (%zu B)",
                layer, bytes, p->slot_bytes);
  if (!p->sim) {
    hipPointerAttribute_t attr;
    const hipError_t e = hipPointerGetAttributes(&attr, host_image);
    if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return fail(LSN_E_ARG, "layer_pool_register: layer %d image is not pinned host memory", layer);
    }
  }
  if (find_slot(p, layer, PENDING) >= 0 || find_slot(p, layer, ACQUIRED) >= 0)
    return fail(LSN_E_STATE, "layer_pool_register: layer %d is in flight", layer);
  forget_copies(p, layer);
  LayerInfo &L = p->layers[layer];
  if (L.fd >= 0) {
    close(L.fd);
    L.fd = -1;
  }
  L.host = host_image;
  L.bytes = bytes;
  L.visits = 0;
  L.checksum = audit_on(p) ? checksum_host(host_image, bytes) : 0;
  return LSN_OK;
}

lsn_status layer_pool_register_file(lsn_pool *p, int32_t layer, const char *path, uint64_t offset, size_t bytes) {
  lsn_status st = check_pool(p, "layer_pool_register_file");
  if (st != LSN_OK) return st;
  if (!p->file_tier) return fail(LSN_E_STATE, "layer_pool_register_file: pool created without LSN_POOL_FILE_TIER");
  if (layer < 0 || layer >= p->n_layers)
    return fail(LSN_E_ARG, "layer_pool_register_file: layer %d out of range [0, %d)", layer, p->n_layers);
  if (!path || bytes == 0) return fail(LSN_E_ARG, "layer_pool_register_file: empty image");
  if (bytes % 256 != 0) return fail(LSN_E_ARG, "layer_pool_register_file: image bytes must be a multiple of 256");
  if (bytes > p->slot_bytes)
    return fail(LSN_E_NOFIT, "layer_pool_register_file: layer %d image (%zu B) does not fit a slot (%zu B)",
                layer, bytes, p->slot_bytes);
  if (find_slot(p, layer, PENDING) >= 0 || find_slot(p, layer, ACQUIRED) >= 0)
    return fail(LSN_E_STATE, "layer_pool_register_file: layer %d is in flight", layer);
  const bool direct = (p->flags & LSN_POOL_FILE_DIRECT) != 0;
  if (direct && offset % kDirectAlign)
    return fail(LSN_E_ARG, "layer_pool_register_file: LSN_POOL_FILE_DIRECT needs the offset aligned to %zu",
                kDirectAlign);
  const size_t span = direct ? (bytes + kDirectAlign - 1) / kDirectAlign * kDirectAlign : bytes;
  const int fd = open(path, O_RDONLY | O_CLOEXEC | (direct ? O_DIRECT : 0));
  if (fd < 0)
    return fail(LSN_E_ARG, "layer_pool_register_file: cannot open %s%s: %s", path, direct ? " with O_DIRECT" : "",
                std::strerror(errno));
  const off_t end = lseek(fd, 0, SEEK_END);
  if (end < 0 || (uint64_t)end < offset + span) {
    close(fd);
    return fail(LSN_E_ARG, "layer_pool_register_file: %s holds %lld B, the image needs %llu B at offset %llu",
                path, (long long)end, (unsigned long long)span, (unsigned long long)offset);
  }
  uint64_t checksum = 0;
  if (audit_on(p)) {
    // (through the page cache, into plain host memory: the checksum read is not a fill)
    const int cfd = open(path, O_RDONLY | O_CLOEXEC);
    std::vector<uint64_t> tmp(bytes / 8);
    std::string err;
    if (cfd < 0 || !read_parallel(cfd, offset, bytes, tmp.data(), err)) {
      if (cfd >= 0) close(cfd);
      close(fd);                             // the layer keeps its previous registration
      return fail(LSN_E_ARG, "layer_pool_register_file: reading %s: %s", path,
                  cfd < 0 ? std::strerror(errno) : err.c_str());
    }
    close(cfd);
    checksum = checksum_host(tmp.data(), bytes);
  }
  forget_copies(p, layer);
  LayerInfo &L = p->layers[layer];
  if (L.fd >= 0) close(L.fd);
  L.host = nullptr;
  L.fd = fd;
  L.file_off = offset;
  L.bytes = bytes;
  L.span = span;
  L.visits = 0;
  L.checksum = checksum;
  return LSN_OK;
}

lsn_status layer_pool_prefetch(lsn_pool *p, int32_t layer) {
  lsn_status st = check_pool(p, "layer_pool_prefetch");
  if (st != LSN_OK) return st;
  if ((st = check_layer(p, layer, "layer_pool_prefetch")) != LSN_OK) return st;
  return do_prefetch(p, layer);
}

lsn_status layer_pool_acquire(lsn_pool *p, int32_t layer, void *compute_stream, const void **dev_image) {
  lsn_status st = check_pool(p, "layer_pool_acquire");
  if (st != LSN_OK) return st;
  if ((st = check_layer(p, layer, "layer_pool_acquire")) != LSN_OK) return st;
  if (!dev_image) return fail(LSN_E_ARG, "layer_pool_acquire: null dev_image");
  if (!p->sim && compute_stream == (void *)p->copy)
    return fail(LSN_E_ARG, "layer_pool_acquire: the compute stream must differ from the copy stream");
  if (find_slot(p, layer, ACQUIRED) >= 0)
    return fail(LSN_E_STATE, "layer_pool_acquire: layer %d is already acquired", layer);
  int i = find_slot(p, layer, PENDING);
  if (i < 0) {
    ++p->stats.misses;
    if ((st = do_prefetch(p, layer)) != LSN_OK) return st;
    i = find_slot(p, layer, PENDING);
  }
  Slot &s = p->slots[i];
  if (s.fill_ticket) {
    std::unique_lock<std::mutex> g(p->mu);
    p->cv_done.wait(g, [&] { return p->done >= s.fill_ticket || !p->io_error.empty(); });
    if (!p->io_error.empty()) return fail(LSN_E_HIP, "layer_pool_acquire: file tier: %s", p->io_error.c_str());
  }
  if (!p->sim) {
    const hipError_t e = hipStreamWaitEvent((hipStream_t)compute_stream, s.ready, 0);
    if (e != hipSuccess) return check_hip(e, "layer_pool_acquire wait");
  }
  s.state = ACQUIRED;
  s.acquired_gen = s.gen;
  ++p->stats.acquires;
  void *mem = s.mem;
  if ((p->flags & LSN_FAULT_WRONG_SLOT) && p->layers[layer].visits >= 2 && p->n_slots >= 2)
    mem = p->slots[(i + 1) % p->n_slots].mem;
  if (audit_on(p) &&
      (st = record_checksum(p, mem, p->layers[layer].bytes, layer, 0, (hipStream_t)compute_stream)) != LSN_OK)
    return st;
  *dev_image = mem;
  return LSN_OK;
}

lsn_status layer_pool_release(lsn_pool *p, int32_t layer, void *compute_stream) {
  lsn_status st = check_pool(p, "layer_pool_release");
  if (st != LSN_OK) return st;
  if (layer < 0 || layer >= p->n_layers)
    return fail(LSN_E_ARG, "layer_pool_release: layer %d out of range", layer);
  const int i = find_slot(p, layer, ACQUIRED);
  if (i < 0) return fail(LSN_E_STATE, "layer_pool_release: layer %d is not acquired", layer);
  Slot &s = p->slots[i];
  if (s.gen != s.acquired_gen)
    return fail(LSN_E_AUDIT, "layer_pool_release: slot %d was refilled while layer %d held it", i, layer);
  hipStream_t cs = (hipStream_t)compute_stream;
  if (audit_on(p)) {
    void *mem = s.mem;
    if ((p->flags & LSN_FAULT_WRONG_SLOT) && p->layers[layer].visits >= 2 && p->n_slots >= 2)
      mem = p->slots[(i + 1) % p->n_slots].mem;
    if ((st = record_checksum(p, mem, p->layers[layer].bytes, layer, 1, cs)) != LSN_OK) return st;
    if (!(p->flags & LSN_POOL_KEEP_AT_TURN)) {
      if (p->sim) std::memset(s.mem, 0xFF, p->slot_bytes);
      else if ((st = check_hip(launch_poison(s.mem, p->slot_bytes, cs), "poison launch")) != LSN_OK) return st;
      s.valid = false;
    }
  }
  if (!p->sim) {
    const hipError_t e = hipEventRecord(s.released, cs);
    if (e != hipSuccess) return check_hip(e, "layer_pool_release record");
    s.release_recorded = true;
  }
  s.state = FREE;
  s.released_tick = ++p->tick;
  ++p->stats.releases;
  return LSN_OK;
}

lsn_status layer_pool_stats(const lsn_pool *p, lsn_pool_stats *out) {
  lsn_status st = check_pool(p, "layer_pool_stats");
  if (st != LSN_OK) return st;
  if (!out) return fail(LSN_E_ARG, "layer_pool_stats: null out");
  *out = p->stats;
  return LSN_OK;
}

lsn_status layer_pool_audit(lsn_pool *p) {
  lsn_status st = check_pool(p, "layer_pool_audit");
  if (st != LSN_OK) return st;
  if (!audit_on(p)) return fail(LSN_E_STATE, "layer_pool_audit: pool created without LSN_POOL_AUDIT");
  const size_t n = p->records.size();
  std::vector<uint64_t> sums(n);
  if (p->sim) {
    for (size_t i = 0; i < n; ++i) sums[i] = p->sums[i];
    std::memset(p->sums, 0, n * 8);
  } else if (n > 0) {
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(sums.data(), p->sums, n * 8, hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemset(p->sums, 0, n * 8);
    if (e != hipSuccess) return check_hip(e, "layer_pool_audit");
  }
  uint64_t failures = 0;
  std::string first;
  for (size_t i = 0; i < n; ++i) {
    const AuditRecord &r = p->records[i];
    if (sums[i] != p->layers[r.layer].checksum) {
      if (failures == 0)
        first = "layer " + std::to_string(r.layer) + " visit " + std::to_string(r.visit) +
                (r.at_release ? " at release" : " at acquire");
      ++failures;
    }
  }
  p->stats.audit_checks += n;
  p->stats.audit_failures += failures;
  p->records.clear();
  if (failures)
    return fail(LSN_E_AUDIT, "layer_pool_audit: %llu of %zu slot checksums differ from their layer's "
                "image (first: %s)", (unsigned long long)failures, n, first.c_str());
  return LSN_OK;
}

lsn_status layer_pool_destroy(lsn_pool *p) {
  if (!p) return LSN_OK;
  hipError_t e = hipSuccess;
  if (p->io.joinable()) {
    {
      std::lock_guard<std::mutex> g(p->mu);
      p->stop = true;
    }
    p->cv_job.notify_all();
    p->io.join();                            // finishes the jobs already posted
  }
  for (LayerInfo &L : p->layers)
    if (L.fd >= 0) close(L.fd);
  if (!p->sim) {
    if (p->copy) e = hipStreamSynchronize(p->copy);
    for (Slot &s : p->slots) {
      if (s.ready) (void)hipEventDestroy(s.ready);
      if (s.released) (void)hipEventDestroy(s.released);
    }
    for (int b = 0; b < 2; ++b)
      if (p->bounce_free[b]) (void)hipEventDestroy(p->bounce_free[b]);
  }
  delete p;
  return check_hip(e, "layer_pool_destroy");
}

}  // extern "C"
