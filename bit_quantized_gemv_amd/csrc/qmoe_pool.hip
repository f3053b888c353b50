// qmoe_pool.hip -- host-resident expert pool: per layer, a fixed number of
// device slots (16 for the model) caches routed-expert blobs; the blobs
// themselves live in pinned host memory.  Replacement is least frequently
// used over the whole history of the layer (devtrends.cc "Come eseguire un
// modello da 26 miliardi…", section "Qual è il trucco principale
// dell'architettura"; remio.ai "TurboFieldfare esegue Mac Gemma 4 26B in
// 2 GB…", section "Mac Gemma 4 26B entra nello spazio disponibile…"): misses
// are copied host -> device on a side stream while the shared expert runs.
//
// Policy (one layer; a step is one acquire for that layer):
//   - every needed expert's use count goes up by one and its last use is the
//     current step, before anything is placed;
//   - needed experts already in a slot are hits;
//   - misses, in rank order, take the lowest free slot, else evict the
//     resident expert that is not needed in this step with the smallest
//     (use count, last use, expert id).
// Counts persist across evictions.  Only host bookkeeping and
// hipMemcpyAsync: no kernels, no device allocation.
#include <errno.h>
#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include <chrono>
#include <condition_variable>
#include <mutex>
#include <thread>
#include <vector>

#include "qmoe.h"

struct qmoe_pool {
  int32_t layers, experts, slots;
  size_t blob_bytes;
  std::vector<const void*> host_blobs;  // [layers * experts] (empty: planning only)
  std::vector<void*> arena;             // [layers] device slot arenas
  struct Layer {
    std::vector<int64_t> uses, last;    // [experts]
    std::vector<int32_t> slot_of;       // [experts]: slot or -1
    std::vector<int32_t> held;          // [slots]: expert or -1
    int64_t step = 0;
    int32_t* map_host[2] = {nullptr, nullptr};  // pinned expert -> slot staging
    hipEvent_t map_done[2] = {nullptr, nullptr};  // its last copy has completed
    int flip = 0;
  };
  std::vector<Layer> L;
  qmoe_pool_stats st;
};

namespace {

// One LFU step of layer `ly` for the needed experts `need[0..k)`.
qmoe_status lfu_step(qmoe_pool* p, int32_t ly, const int32_t* need, int32_t k, int32_t* slot_out,
                     int32_t* hit_out, int32_t* victim_out) {
  qmoe_pool::Layer& S = p->L[ly];
  const int64_t now = S.step++;
  std::vector<char> wanted(p->experts, 0);
  for (int32_t j = 0; j < k; ++j) {
    if (need[j] < 0 || need[j] >= p->experts) return QMOE_ERR_BAD_SHAPE;
    if (wanted[need[j]]) return QMOE_ERR_BAD_SHAPE;  // ids of one step are distinct
    wanted[need[j]] = 1;
  }
  for (int32_t j = 0; j < k; ++j) {
    S.uses[need[j]] += 1;
    S.last[need[j]] = now;
  }
  for (int32_t j = 0; j < k; ++j) {
    const int32_t e = need[j];
    int32_t victim = -1, s = S.slot_of[e];
    const bool hit = s >= 0;
    if (!hit) {
      for (int32_t i = 0; i < p->slots && s < 0; ++i)
        if (S.held[i] < 0) s = i;
      if (s < 0) {
        // evict: smallest (uses, last, id) among residents not needed now
        for (int32_t i = 0; i < p->slots; ++i) {
          const int32_t c = S.held[i];
          if (wanted[c]) continue;
          if (s < 0) {
            s = i;
            continue;
          }
          const int32_t b = S.held[s];
          const bool less = S.uses[c] != S.uses[b]  ? S.uses[c] < S.uses[b]
                            : S.last[c] != S.last[b] ? S.last[c] < S.last[b]
                                                     : c < b;
          if (less) s = i;
        }
        if (s < 0) return QMOE_ERR_UNSUPPORTED;  // unreachable with k <= slots
        victim = S.held[s];
        S.slot_of[victim] = -1;
      }
      S.held[s] = e;
      S.slot_of[e] = s;
    }
    if (slot_out) slot_out[j] = s;
    if (hit_out) hit_out[j] = hit ? 1 : 0;
    if (victim_out) victim_out[j] = victim;
  }
  return QMOE_OK;
}

// The end of an acquire: the layer's expert -> slot map to the device
// (non-resident experts map to slot 0, a valid address; the kernels only look
// up the routed experts), `ready` after it, the statistics.  The map's pinned
// staging buffer is rewritten only after its previous copy has completed.
qmoe_status finish_acquire(qmoe_pool* p, int32_t layer, int32_t nh, int32_t nm,
                           int32_t* dev_expert_slot, hipStream_t cs, void* ready,
                           qmoe_pool_stats* st) {
  qmoe_pool::Layer& S = p->L[layer];
  const int f = S.flip;
  S.flip ^= 1;
  if (hipEventSynchronize(S.map_done[f]) != hipSuccess) return QMOE_ERR_HIP;
  int32_t* m = S.map_host[f];
  for (int32_t e = 0; e < p->experts; ++e) m[e] = S.slot_of[e] >= 0 ? S.slot_of[e] : 0;
  if (hipMemcpyAsync(dev_expert_slot, m, sizeof(int32_t) * p->experts, hipMemcpyHostToDevice, cs) !=
      hipSuccess)
    return QMOE_ERR_HIP;
  if (hipEventRecord(S.map_done[f], cs) != hipSuccess) return QMOE_ERR_HIP;
  if (ready && hipEventRecord(reinterpret_cast<hipEvent_t>(ready), cs) != hipSuccess)
    return QMOE_ERR_HIP;
  p->st.hits += nh;
  p->st.misses += nm;
  p->st.h2d_bytes += (int64_t)nm * (int64_t)p->blob_bytes;
  p->st.last_hits = nh;
  p->st.last_misses = nm;
  if (st) *st = p->st;
  return QMOE_OK;
}

}  // namespace

// ------------------------------------------------------------ file tier
// The routed experts on storage: an expert-major file, the blob of (layer,
// e) at byte (layer * experts + e) * stride (devtrends.cc "Come eseguire un
// modello da 26 miliardi…", section "Qual è il trucco principale
// dell'architettura": the CPU compares the router's choice with the cache
// and issues bounded parallel reads for the missing experts; remio.ai
// "TurboFieldfare esegue Mac Gemma 4 26B in 2 GB…", section "L'affermazione
// dei 2 GB trasforma la larghezza di banda dell'SSD nel nuovo vincolo").
// A fixed set of worker threads preads whole strides into pinned staging
// buffers (two sets, used in turn: a set is rewritten only after the copies
// out of it have completed), then the blobs go host -> device on the copy
// stream.  With `direct` the file is opened O_DIRECT (reads bypass the page
// cache; stride and staging are 4096-aligned).
struct qmoe_file_tier {
  int fd = -1;
  int32_t layers = 0, experts = 0, max_misses = 0;
  size_t blob_bytes = 0, stride = 0;
  void* staging[2] = {nullptr, nullptr};
  hipEvent_t staged_free[2] = {nullptr, nullptr};
  int flip = 0;
  // workers
  struct Job {
    void* dst;
    size_t bytes;
    off_t off;
  };
  std::vector<std::thread> workers;
  std::mutex mu;
  std::condition_variable cv_job, cv_done;
  std::vector<Job> jobs;
  size_t next = 0;
  int pending = 0, err = 0;
  bool stop = false;
  qmoe_file_tier_stats st{};

  void work() {
    std::unique_lock<std::mutex> lk(mu);
    for (;;) {
      cv_job.wait(lk, [&] { return stop || next < jobs.size(); });
      if (stop) return;
      const Job j = jobs[next++];
      lk.unlock();
      size_t got = 0;
      int e = 0;
      while (got < j.bytes) {
        const ssize_t r = pread(fd, static_cast<uint8_t*>(j.dst) + got, j.bytes - got,
                                j.off + (off_t)got);
        if (r <= 0) {
          e = r == 0 ? -1 : 1;
          break;
        }
        got += (size_t)r;
      }
      const int saved = errno;
      lk.lock();
      if (e) {
        err = 1;
        st.last_errno = e > 0 ? saved : -1;
      }
      if (--pending == 0) cv_done.notify_all();
    }
  }
};

extern "C" {

qmoe_status qmoe_file_tier_open(const char* path, int32_t layers, int32_t experts,
                                size_t blob_bytes, size_t stride, int32_t threads,
                                int32_t max_misses, int32_t direct, qmoe_file_tier** out) {
  if (!path || !out) return QMOE_ERR_NULL_ARG;
  *out = nullptr;
  if (layers <= 0 || experts <= 0 || blob_bytes == 0 || stride < blob_bytes || threads < 1 ||
      threads > 64 || max_misses < 1 || max_misses > QMOE_MAX_TOP_K)
    return QMOE_ERR_BAD_SHAPE;
  if (stride % 4096) return QMOE_ERR_ALIGN;
  qmoe_file_tier* t = new qmoe_file_tier();
  t->fd = open(path, O_RDONLY | (direct ? O_DIRECT : 0));
  if (t->fd < 0) {
    delete t;
    return QMOE_ERR_BAD_SHAPE;
  }
  const off_t need = (off_t)layers * experts * (off_t)stride;
  if (lseek(t->fd, 0, SEEK_END) < need) {
    close(t->fd);
    delete t;
    return QMOE_ERR_BAD_SHAPE;
  }
  t->layers = layers;
  t->experts = experts;
  t->blob_bytes = blob_bytes;
  t->stride = stride;
  t->max_misses = max_misses;
  for (int i = 0; i < 2; ++i) {
    if (hipHostMalloc(&t->staging[i], stride * (size_t)max_misses, hipHostMallocDefault) !=
            hipSuccess ||
        hipEventCreateWithFlags(&t->staged_free[i], hipEventDisableTiming) != hipSuccess) {
      qmoe_file_tier_close(t);
      return QMOE_ERR_HIP;
    }
  }
  if (direct) {
    // some file systems open with O_DIRECT and refuse the reads: try one
    if (pread(t->fd, t->staging[0], stride, 0) != (ssize_t)stride) {
      qmoe_file_tier_close(t);
      return QMOE_ERR_UNSUPPORTED;
    }
  }
  for (int32_t i = 0; i < threads; ++i) t->workers.emplace_back([t] { t->work(); });
  *out = t;
  return QMOE_OK;
}

qmoe_status qmoe_pool_acquire_file(qmoe_pool* p, qmoe_file_tier* t, int32_t layer,
                                   const int32_t* host_idx, int32_t k, int32_t* dev_expert_slot,
                                   void* copy_stream, void* ready, qmoe_pool_stats* st) {
  if (!p || !t || !host_idx || !dev_expert_slot) return QMOE_ERR_NULL_ARG;
  if (p->arena.empty()) return QMOE_ERR_UNSUPPORTED;  // planning-only pool
  if (layer < 0 || layer >= p->layers || k <= 0 || k > QMOE_MAX_TOP_K || k > p->slots ||
      k > t->max_misses || t->layers != p->layers || t->experts != p->experts ||
      t->blob_bytes != p->blob_bytes)
    return QMOE_ERR_BAD_SHAPE;
  int32_t slot[QMOE_MAX_TOP_K], hit[QMOE_MAX_TOP_K], victim[QMOE_MAX_TOP_K];
  qmoe_status s = lfu_step(p, layer, host_idx, k, slot, hit, victim);
  if (s != QMOE_OK) return s;
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  // the staging set of this acquire: free once its previous copies are done
  const int f = t->flip;
  t->flip ^= 1;
  if (hipEventSynchronize(t->staged_free[f]) != hipSuccess) return QMOE_ERR_HIP;
  uint8_t* stage = static_cast<uint8_t*>(t->staging[f]);
  int32_t nh = 0, nm = 0, miss[QMOE_MAX_TOP_K];
  for (int32_t j = 0; j < k; ++j) {
    if (hit[j])
      ++nh;
    else
      miss[nm++] = j;
  }
  if (nm) {
    const auto t0 = std::chrono::steady_clock::now();
    {
      std::lock_guard<std::mutex> lk(t->mu);
      t->jobs.clear();
      t->next = 0;
      t->err = 0;
      for (int32_t i = 0; i < nm; ++i) {
        const int64_t blob = (int64_t)layer * t->experts + host_idx[miss[i]];
        t->jobs.push_back({stage + (size_t)i * t->stride, t->stride, (off_t)(blob * (int64_t)t->stride)});
      }
      t->pending = nm;
    }
    t->cv_job.notify_all();
    {
      std::unique_lock<std::mutex> lk(t->mu);
      t->cv_done.wait(lk, [&] { return t->pending == 0; });
      if (t->err) return QMOE_ERR_HIP;  // a read failed (I/O error or short file)
    }
    const auto t1 = std::chrono::steady_clock::now();
    t->st.reads += nm;
    t->st.read_bytes += (int64_t)nm * (int64_t)t->stride;
    t->st.read_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(t1 - t0).count();
    for (int32_t i = 0; i < nm; ++i) {
      void* dst = static_cast<uint8_t*>(p->arena[layer]) + (size_t)slot[miss[i]] * p->blob_bytes;
      if (hipMemcpyAsync(dst, stage + (size_t)i * t->stride, p->blob_bytes, hipMemcpyHostToDevice,
                         cs) != hipSuccess)
        return QMOE_ERR_HIP;
    }
    if (hipEventRecord(t->staged_free[f], cs) != hipSuccess) return QMOE_ERR_HIP;
  }
  return finish_acquire(p, layer, nh, nm, dev_expert_slot, cs, ready, st);
}

qmoe_status qmoe_file_tier_stats_get(const qmoe_file_tier* t, qmoe_file_tier_stats* st) {
  if (!t || !st) return QMOE_ERR_NULL_ARG;
  *st = t->st;
  return QMOE_OK;
}

void qmoe_file_tier_close(qmoe_file_tier* t) {
  if (!t) return;
  {
    std::lock_guard<std::mutex> lk(t->mu);
    t->stop = true;
  }
  t->cv_job.notify_all();
  for (auto& w : t->workers) w.join();
  for (int i = 0; i < 2; ++i) {
    if (t->staged_free[i]) {
      (void)hipEventSynchronize(t->staged_free[i]);
      (void)hipEventDestroy(t->staged_free[i]);
    }
    if (t->staging[i]) (void)hipHostFree(t->staging[i]);
  }
  if (t->fd >= 0) close(t->fd);
  delete t;
}

}  // extern "C"

extern "C" {

qmoe_status qmoe_pool_create(int32_t layers, int32_t experts, int32_t slots, size_t blob_bytes,
                             const void* const* host_blobs, void* const* dev_slot_arena,
                             qmoe_pool** out) {
  if (!out) return QMOE_ERR_NULL_ARG;
  *out = nullptr;
  if (layers <= 0 || experts <= 0 || slots <= 0 || slots > experts) return QMOE_ERR_BAD_SHAPE;
  if (host_blobs && !dev_slot_arena) return QMOE_ERR_NULL_ARG;
  if (dev_slot_arena && (blob_bytes == 0 || blob_bytes % 256)) return QMOE_ERR_ALIGN;
  qmoe_pool* p = new qmoe_pool();
  p->layers = layers;
  p->experts = experts;
  p->slots = slots;
  p->blob_bytes = blob_bytes;
  memset(&p->st, 0, sizeof(p->st));
  p->L.resize(layers);
  for (auto& S : p->L) {
    S.uses.assign(experts, 0);
    S.last.assign(experts, -1);
    S.slot_of.assign(experts, -1);
    S.held.assign(slots, -1);
  }
  if (dev_slot_arena) {
    if (host_blobs) p->host_blobs.assign(host_blobs, host_blobs + (size_t)layers * experts);
    p->arena.assign(dev_slot_arena, dev_slot_arena + layers);
    for (auto& S : p->L)
      for (int i = 0; i < 2; ++i) {
        void* m = nullptr;
        if (hipHostMalloc(&m, sizeof(int32_t) * experts, hipHostMallocDefault) != hipSuccess) {
          qmoe_pool_destroy(p);
          return QMOE_ERR_HIP;
        }
        S.map_host[i] = static_cast<int32_t*>(m);
        if (hipEventCreateWithFlags(&S.map_done[i], hipEventDisableTiming) != hipSuccess) {
          qmoe_pool_destroy(p);
          return QMOE_ERR_HIP;
        }
      }
  }
  *out = p;
  return QMOE_OK;
}

qmoe_status qmoe_pool_plan(qmoe_pool* p, int32_t layer, const int32_t* host_idx, int32_t k,
                           int32_t* slot_out, int32_t* hit_out, int32_t* victim_out) {
  if (!p || !host_idx) return QMOE_ERR_NULL_ARG;
  if (layer < 0 || layer >= p->layers || k <= 0 || k > p->slots) return QMOE_ERR_BAD_SHAPE;
  return lfu_step(p, layer, host_idx, k, slot_out, hit_out, victim_out);
}

qmoe_status qmoe_pool_acquire(qmoe_pool* p, int32_t layer, const int32_t* host_idx, int32_t k,
                              int32_t* dev_expert_slot, void* copy_stream, void* ready,
                              qmoe_pool_stats* st) {
  if (!p || !host_idx || !dev_expert_slot) return QMOE_ERR_NULL_ARG;
  if (p->host_blobs.empty()) return QMOE_ERR_UNSUPPORTED;  // planning-only or file-backed
  if (layer < 0 || layer >= p->layers || k <= 0 || k > QMOE_MAX_TOP_K || k > p->slots)
    return QMOE_ERR_BAD_SHAPE;
  int32_t slot[QMOE_MAX_TOP_K], hit[QMOE_MAX_TOP_K], victim[QMOE_MAX_TOP_K];
  qmoe_status s = lfu_step(p, layer, host_idx, k, slot, hit, victim);
  if (s != QMOE_OK) return s;
  hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  int32_t nh = 0, nm = 0;
  for (int32_t j = 0; j < k; ++j) {
    if (hit[j]) {
      ++nh;
      continue;
    }
    ++nm;
    const void* src = p->host_blobs[(size_t)layer * p->experts + host_idx[j]];
    void* dst = static_cast<uint8_t*>(p->arena[layer]) + (size_t)slot[j] * p->blob_bytes;
    if (hipMemcpyAsync(dst, src, p->blob_bytes, hipMemcpyHostToDevice, cs) != hipSuccess)
      return QMOE_ERR_HIP;
  }
  return finish_acquire(p, layer, nh, nm, dev_expert_slot, cs, ready, st);
}

qmoe_status qmoe_pool_stats_get(const qmoe_pool* p, qmoe_pool_stats* st) {
  if (!p || !st) return QMOE_ERR_NULL_ARG;
  *st = p->st;
  return QMOE_OK;
}

void qmoe_pool_destroy(qmoe_pool* p) {
  if (!p) return;
  for (auto& S : p->L)
    for (int i = 0; i < 2; ++i) {
      if (S.map_done[i]) (void)hipEventDestroy(S.map_done[i]);
      if (S.map_host[i]) (void)hipHostFree(S.map_host[i]);
    }
  delete p;
}

}  // extern "C"
