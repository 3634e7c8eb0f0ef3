// Host-tiered exact-token attention: the token K/V live in pinned host RAM,
// the chunk / group summary tables in HBM.
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3, tiered K/V store: summaries and routing stay on the device, the
// full token K/V history sits in host RAM and only what the router selects
// is moved to the device for the exact-token attention.
//
// Pipeline (one call = one prefill over [q_pos0, q_pos0 + n_q)):
//   1. route every unit on the device (summaries in HBM);
//   2. one device-to-host copy of the granule lists and counts;
//   3. windows of consecutive query chunks: the union of the granules their
//      units attend to (fixed windows + routed groups or chunks, each granule
//      once per (sequence, KV head)) is gathered by host threads from the
//      granule-major store into pinned staging, moved with one
//      hipMemcpyAsync on the copy stream, and an event gates the window's
//      attention on the compute stream;
//   4. two window buffers alternate, so window w+1 is packed and copied
//      while window w is attended.
// With a warm tier (cache_slots > 0) the device keeps a cache of granules
// across the windows of the call (least recently used evicted first):
// a window copies only the granules the cache lacks, into a landing buffer,
// and a gather kernel on the compute stream moves them to their cache slots
// before the window's attention; stream order makes every slot that the
// window does not use safe to evict.
// The call returns after the last attention launch is enqueued.
#include <algorithm>
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "hga_internal.h"

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of every buffer carved from the caller's staging memory.
struct Layout {
  int64_t units = 0, wunits = 0, slots = 0, cache_slots = 0;
  size_t granule_bytes = 0;
  size_t cidx = 0, gidx = 0, gran = 0, gcnt = 0, rws = 0, cache = 0, win[2] = {0, 0}, dev_total = 0;
  // inside one window buffer: the pool (no cache) or the landing buffer of
  // the window's misses (cache), then its index arrays
  size_t pool_bytes = 0, wgran = 0, wslot = 0, wcnt = 0, wdst = 0, win_bytes = 0;
  size_t hgran = 0, hcnt = 0, hwin[2] = {0, 0}, host_total = 0;
};

Layout make_layout(const hga::Geometry& g, int32_t wmax, int64_t slots, int64_t cache_slots) {
  Layout L;
  const size_t elem = g.bf16 ? 2 : 4;
  L.units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  L.wunits = static_cast<int64_t>(g.B) * g.Hkv * wmax;
  L.slots = slots;
  L.cache_slots = cache_slots;
  L.granule_bytes = static_cast<size_t>(2) * g.gs * g.d * elem;
  const size_t u = static_cast<size_t>(L.units);
  size_t off = 0;
  L.cidx = off; off = align_up(off + u * std::max(g.Kc, 1) * 4);
  L.gidx = off; off = align_up(off + u * std::max(g.Kg, 1) * 4);
  L.gran = off; off = align_up(off + u * g.gmax * 4);
  L.gcnt = off; off = align_up(off + u * 4);
  L.rws = off; off = align_up(off + hga::route_workspace(g));
  L.cache = off; off = align_up(off + static_cast<size_t>(cache_slots) * L.granule_bytes);
  L.pool_bytes = align_up(static_cast<size_t>(slots) * L.granule_bytes);
  L.wgran = L.pool_bytes;
  L.wslot = align_up(L.wgran + static_cast<size_t>(L.wunits) * g.gmax * 4);
  L.wcnt = align_up(L.wslot + static_cast<size_t>(L.wunits) * g.gmax * 4);
  L.wdst = align_up(L.wcnt + static_cast<size_t>(L.wunits) * 4);
  L.win_bytes = align_up(L.wdst + (cache_slots > 0 ? static_cast<size_t>(slots) * 4 : 0));
  L.win[0] = off; off += L.win_bytes;
  L.win[1] = off; off += L.win_bytes;
  L.dev_total = off;
  size_t h = 0;
  L.hgran = h; h = align_up(h + u * g.gmax * 4);
  L.hcnt = h; h = align_up(h + u * 4);
  L.hwin[0] = h; h += L.win_bytes;
  L.hwin[1] = h; h += L.win_bytes;
  L.host_total = h;
  return L;
}

// A fixed set of host threads that run one job (thread i of n) per run().
class Packer {
 public:
  explicit Packer(int n) {
    for (int i = 0; i < n; ++i) th_.emplace_back([this, i, n] { loop(i, n); });
  }
  ~Packer() {
    {
      std::lock_guard<std::mutex> l(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  void run(const std::function<void(int, int)>& job) {
    if (th_.empty()) {
      job(0, 1);
      return;
    }
    std::unique_lock<std::mutex> l(mu_);
    job_ = &job;
    pending_ = static_cast<int>(th_.size());
    ++gen_;
    cv_.notify_all();
    done_.wait(l, [this] { return pending_ == 0; });
    job_ = nullptr;
  }

 private:
  void loop(int i, int n) {
    int64_t seen = 0;
    for (;;) {
      const std::function<void(int, int)>* job;
      {
        std::unique_lock<std::mutex> l(mu_);
        cv_.wait(l, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
        job = job_;
      }
      (*job)(i, n);
      {
        std::lock_guard<std::mutex> l(mu_);
        if (--pending_ == 0) done_.notify_one();
      }
    }
  }
  std::vector<std::thread> th_;
  std::mutex mu_;
  std::condition_variable cv_, done_;
  const std::function<void(int, int)>* job_ = nullptr;
  int pending_ = 0;
  int64_t gen_ = 0;
  bool stop_ = false;
};

bool pinned_host(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // a failed query must not poison later launches
    return false;
  }
  return a.type == hipMemoryTypeHost;
}

struct Events {
  hipEvent_t e[4] = {nullptr, nullptr, nullptr, nullptr};
  ~Events() {
    for (hipEvent_t x : e)
      if (x != nullptr) (void)hipEventDestroy(x);
  }
};

hga_status tier_geometry(const hga_config* cfg, hga_dtype dtype, int32_t batch, int64_t q_pos0,
                         int64_t n_q, int64_t kv_cap, int32_t wmax, int64_t slots,
                         int64_t cache_slots, hga::Geometry& g) {
  hga_status st = hga::make_geometry(cfg, dtype, batch, kv_cap, q_pos0, n_q, g);
  if (st != HGA_OK) return st;
  if (n_q <= 0 || wmax <= 0 || cache_slots < 0) return HGA_ERR_INVALID_ARGUMENT;
  // one query chunk of every (sequence, KV head) must fit a window (and the cache)
  const int64_t chunk_need = static_cast<int64_t>(g.B) * g.Hkv * g.gmax;
  if (slots < chunk_need) return HGA_ERR_INVALID_ARGUMENT;
  if (cache_slots > 0 && cache_slots < chunk_need) return HGA_ERR_INVALID_ARGUMENT;
  if (!hga::route_supported(g) || !hga::attend_supported(g)) return HGA_ERR_UNSUPPORTED;
  // the pool (or cache) is read through 32-bit buffer offsets, every list by one work item
  const int64_t pool = std::max(slots, cache_slots) * 2 * g.gs * g.d * (g.bf16 ? 2 : 4);
  if (g.bf16 && (pool >= (int64_t{1} << 31) || g.gmax > hga::kAttendTable)) return HGA_ERR_UNSUPPORTED;
  return HGA_OK;
}

// Copies granule j of the landing buffer to cache slot dst[j] (one
// workgroup per granule, 16-byte words).
__global__ __launch_bounds__(256) void land_granules(const uint4* landing, uint4* cache,
                                                     const int32_t* dst, int64_t words) {
  const uint4* src = landing + static_cast<int64_t>(blockIdx.x) * words;
  uint4* out = cache + static_cast<int64_t>(dst[blockIdx.x]) * words;
  for (int64_t i = threadIdx.x; i < words; i += blockDim.x) out[i] = src[i];
}

// Least-recently-used order of the cache slots (a doubly linked list; the
// front is the most recent).  Slot owners are (sequence, KV head, granule)
// keys, -1 when free.
class Lru {
 public:
  explicit Lru(int64_t n) : prev_(n), next_(n), owner_(n, -1) {
    for (int64_t i = 0; i < n; ++i) {
      prev_[i] = i - 1;
      next_[i] = i + 1 < n ? i + 1 : -1;
    }
    head_ = n > 0 ? 0 : -1;
    tail_ = n - 1;
  }
  void touch(int64_t s) {  // move to the front
    if (s == head_) return;
    unlink(s);
    prev_[s] = -1;
    next_[s] = head_;
    if (head_ >= 0) prev_[head_] = s;
    head_ = s;
    if (tail_ < 0) tail_ = s;
  }
  int64_t victim() const { return tail_; }
  int64_t owner(int64_t s) const { return owner_[s]; }
  void set_owner(int64_t s, int64_t key) { owner_[s] = key; }

 private:
  void unlink(int64_t s) {
    if (prev_[s] >= 0) next_[prev_[s]] = next_[s]; else head_ = next_[s];
    if (next_[s] >= 0) prev_[next_[s]] = prev_[s]; else tail_ = prev_[s];
  }
  std::vector<int64_t> prev_, next_, owner_;
  int64_t head_ = -1, tail_ = -1;
};

// The window loop with a warm tier (see the file comment): L.cache holds
// cache_slots granules; a window holds at most cache_slots distinct granules
// and at most slots_per_window misses.
hga_status tiered_cached(const hga::Geometry& g, const Layout& L, const void* q_raw,
                         const void* kv_host, void* out, float* lse, char* dev, char* host,
                         const int32_t* h_gran, const int32_t* h_gcnt, int32_t wmax,
                         int64_t slots_per_window, int64_t cache_slots, int32_t n_threads,
                         hipStream_t cs, hipStream_t xs, hipEvent_t* copied, hipEvent_t* attended,
                         hga_tier_stats* stats, std::chrono::steady_clock::time_point t_start) {
  const int64_t ngran = g.kv_cap / g.gs;
  const int64_t bh = static_cast<int64_t>(g.B) * g.Hkv;
  const size_t gb = L.granule_bytes;
  char* cache = dev + L.cache;
  Lru lru(cache_slots);
  std::vector<int64_t> slot_of(static_cast<size_t>(bh * ngran), -1);
  std::vector<int32_t> stamp(static_cast<size_t>(bh * ngran), -1);
  std::vector<std::pair<const char*, char*>> jobs;
  jobs.reserve(static_cast<size_t>(slots_per_window));
  const char* store = static_cast<const char*>(kv_host);
  Packer packer(n_threads);
  double pack_s = 0.0;
  int64_t copied_granules = 0, hits = 0, bytes_h2d = 0;
  const int64_t t_end = g.t0 + g.nqc;
  hipError_t e = hipSuccess;
  int32_t w = 0;
  for (int64_t ta = g.t0; ta < t_end; ++w) {
    const int buf = w & 1;
    char* hw = host + L.hwin[buf];
    char* dw = dev + L.win[buf];
    if (w >= 2) {  // the copy that last read this host buffer must be done
      e = hipEventSynchronize(copied[buf]);
      if (e != hipSuccess) return hga::hip_fail(e);
    }
    int32_t* wdst = reinterpret_cast<int32_t*>(hw + L.wdst);
    // Grow the window one query chunk at a time while its distinct granules
    // fit the cache and its misses the landing buffer; hits move to the
    // front of the LRU order, misses take the least recently used slots.
    int64_t need = 0, miss = 0, tb = ta;
    jobs.clear();
    while (tb < t_end && tb - ta < wmax) {
      int64_t add_need = 0, add_miss = 0;
      for (int64_t x = 0; x < bh; ++x) {
        const int64_t u = x * g.nqc + (tb - g.t0);
        for (int32_t i = 0; i < h_gcnt[u]; ++i) {
          const size_t k = static_cast<size_t>(x * ngran + h_gran[u * g.gmax + i]);
          if (stamp[k] != w) {
            ++add_need;
            add_miss += slot_of[k] < 0;
          }
        }
      }
      if (need + add_need > cache_slots || miss + add_miss > slots_per_window) break;
      for (int64_t x = 0; x < bh; ++x) {
        const int64_t u = x * g.nqc + (tb - g.t0);
        for (int32_t i = 0; i < h_gcnt[u]; ++i) {
          const int64_t k = x * ngran + h_gran[u * g.gmax + i];
          if (stamp[static_cast<size_t>(k)] == w) continue;
          stamp[static_cast<size_t>(k)] = w;
          int64_t sl = slot_of[static_cast<size_t>(k)];
          if (sl >= 0) {
            ++hits;
          } else {
            sl = lru.victim();  // untouched in this window (need <= cache_slots)
            const int64_t prev = lru.owner(sl);
            if (prev >= 0) slot_of[static_cast<size_t>(prev)] = -1;
            lru.set_owner(sl, k);
            slot_of[static_cast<size_t>(k)] = sl;
            wdst[miss] = static_cast<int32_t>(sl);
            jobs.emplace_back(store + k * gb, hw + miss * gb);
            ++miss;
          }
          lru.touch(sl);
        }
      }
      need += add_need;
      ++tb;
    }
    const int64_t nw = tb - ta;
    int32_t* wgran = reinterpret_cast<int32_t*>(hw + L.wgran);
    int32_t* wslot = reinterpret_cast<int32_t*>(hw + L.wslot);
    int32_t* wcnt = reinterpret_cast<int32_t*>(hw + L.wcnt);
    for (int64_t x = 0; x < bh; ++x) {
      for (int64_t t = ta; t < tb; ++t) {
        const int64_t u = x * g.nqc + (t - g.t0);
        const int64_t wu = x * nw + (t - ta);
        wcnt[wu] = h_gcnt[u];
        for (int32_t i = 0; i < g.gmax; ++i) {
          const int32_t gid = i < h_gcnt[u] ? h_gran[u * g.gmax + i] : -1;
          wgran[wu * g.gmax + i] = gid;
          wslot[wu * g.gmax + i] =
              gid >= 0 ? static_cast<int32_t>(slot_of[static_cast<size_t>(x * ngran + gid)]) : -1;
        }
      }
    }
    const auto p0 = std::chrono::steady_clock::now();
    const size_t nj = jobs.size();
    packer.run([&](int i, int n) {
      const size_t lo = nj * i / n, hi = nj * (i + 1) / n;
      for (size_t j = lo; j < hi; ++j) std::memcpy(jobs[j].second, jobs[j].first, gb);
    });
    pack_s += std::chrono::duration<double>(std::chrono::steady_clock::now() - p0).count();
    // the landing buffer and index arrays of this window buffer were last
    // read by window w-2's gather and attention on the compute stream
    if (w >= 2) {
      e = hipStreamWaitEvent(xs, attended[buf], 0);
      if (e != hipSuccess) return hga::hip_fail(e);
    }
    const size_t idx_bytes = L.win_bytes - L.wgran;
    if (miss > 0) e = hipMemcpyAsync(dw, hw, static_cast<size_t>(miss) * gb, hipMemcpyHostToDevice, xs);
    if (e == hipSuccess) e = hipMemcpyAsync(dw + L.wgran, hw + L.wgran, idx_bytes, hipMemcpyHostToDevice, xs);
    if (e == hipSuccess) e = hipEventRecord(copied[buf], xs);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, copied[buf], 0);
    if (e != hipSuccess) return hga::hip_fail(e);
    if (miss > 0) {
      hipLaunchKernelGGL(land_granules, dim3(static_cast<unsigned>(miss)), dim3(256), 0, cs,
                         reinterpret_cast<const uint4*>(dw), reinterpret_cast<uint4*>(cache),
                         reinterpret_cast<const int32_t*>(dw + L.wdst), static_cast<int64_t>(gb / 16));
      e = hipGetLastError();
      if (e != hipSuccess) return hga::hip_fail(e);
    }
    copied_granules += miss;
    bytes_h2d += static_cast<int64_t>(static_cast<size_t>(miss) * gb + idx_bytes);
    hga::Geometry gw = g;
    gw.q_pos0 = std::max(ta * g.C, g.q_pos0);
    gw.n_q = std::min(tb * g.C, g.q_pos0 + g.n_q) - gw.q_pos0;
    gw.t0 = ta;
    gw.nqc = nw;
    hga::AttendExtra ex;
    ex.pool_slot = reinterpret_cast<const int32_t*>(dw + L.wslot);
    ex.pool_slots = cache_slots;
    ex.allow_split = false;
    ex.q_stride = g.n_q;
    ex.q_row0 = g.q_pos0;
    e = hga::launch_attend(gw, q_raw, cache, cache, reinterpret_cast<const int32_t*>(dw + L.wgran),
                           reinterpret_cast<const int32_t*>(dw + L.wcnt), false, out, lse, nullptr, cs, &ex);
    if (e == hipSuccess) e = hipEventRecord(attended[buf], cs);
    if (e != hipSuccess) return hga::hip_fail(e);
    ta = tb;
  }
  if (stats != nullptr) {
    stats->windows = w;
    stats->granules_copied = copied_granules;
    stats->bytes_h2d = bytes_h2d;
    stats->pack_seconds = pack_s;
    stats->host_seconds =
        std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
    stats->granules_hit = hits;
  }
  return HGA_OK;
}

// The largest n in [lo, hi] with fits(n) (fits is monotone: true up to
// some n), or lo - 1 when fits(lo) fails.
template <typename Fits>
int64_t largest_fitting(int64_t lo, int64_t hi, Fits fits) {
  if (hi < lo || !fits(lo)) return lo - 1;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (fits(mid)) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Device memory that can be given to a warm tier while `headroom` bytes of
// the current device's free memory stay unused.
hga_status free_budget(size_t headroom, size_t& budget) {
  size_t free_b = 0, total_b = 0;
  const hipError_t e = hipMemGetInfo(&free_b, &total_b);
  if (e != hipSuccess) return hga::hip_fail(e);
  budget = free_b > headroom ? free_b - headroom : 0;
  return HGA_OK;
}

}  // namespace

extern "C" {

hga_status hga_host_tiered_buffer_bytes(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                        int64_t q_pos0, int64_t n_q, int32_t max_window_chunks,
                                        int64_t slots_per_window, int64_t cache_slots,
                                        size_t* device_bytes, size_t* host_bytes) {
  if (device_bytes == nullptr || host_bytes == nullptr || cfg == nullptr || cfg->chunk_size <= 0)
    return HGA_ERR_INVALID_ARGUMENT;
  const int64_t cap = ((q_pos0 + n_q + cfg->chunk_size - 1) / cfg->chunk_size) * cfg->chunk_size;
  hga::Geometry g;
  hga_status st = tier_geometry(cfg, dtype, batch, q_pos0, n_q, cap > 0 ? cap : cfg->chunk_size,
                                max_window_chunks, slots_per_window, cache_slots, g);
  if (st != HGA_OK) return st;
  const Layout L = make_layout(g, max_window_chunks, slots_per_window, cache_slots);
  *device_bytes = L.dev_total;
  *host_bytes = L.host_total;
  return HGA_OK;
}

hga_status hga_host_tiered_cache_slots(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                       int64_t q_pos0, int64_t n_q, int32_t max_window_chunks,
                                       int64_t slots_per_window, size_t headroom_bytes,
                                       int64_t* cache_slots) {
  if (cfg == nullptr || cache_slots == nullptr || cfg->chunk_size <= 0 || cfg->group_size <= 0)
    return HGA_ERR_INVALID_ARGUMENT;
  const int64_t cap = ((q_pos0 + n_q + cfg->chunk_size - 1) / cfg->chunk_size) * cfg->chunk_size;
  hga::Geometry g;
  hga_status st = tier_geometry(cfg, dtype, batch, q_pos0, n_q, cap > 0 ? cap : cfg->chunk_size,
                                max_window_chunks, slots_per_window, 0, g);
  if (st != HGA_OK) return st;
  size_t budget = 0;
  st = free_budget(headroom_bytes, budget);
  if (st != HGA_OK) return st;
  const int64_t lo = static_cast<int64_t>(g.B) * g.Hkv * g.gmax;         // a window's granules
  const int64_t hi = static_cast<int64_t>(g.B) * g.Hkv * (g.kv_cap / g.gs);  // all of the call's
  auto fits = [&](int64_t n) {
    hga::Geometry gc;
    if (tier_geometry(cfg, dtype, batch, q_pos0, n_q, g.kv_cap, max_window_chunks, slots_per_window, n, gc) !=
        HGA_OK)
      return false;
    return make_layout(gc, max_window_chunks, slots_per_window, n).dev_total <= budget;
  };
  const int64_t n = largest_fitting(lo, std::max(lo, hi), fits);
  *cache_slots = n >= lo ? n : 0;
  return HGA_OK;
}

hga_status hga_attend_host_tiered(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                  const void* q_raw, int64_t q_pos0, int64_t n_q,
                                  const void* kv_host, int64_t kv_cap, const float* chunk_sum,
                                  const float* group_sum, void* out, float* lse,
                                  void* dev_staging, size_t dev_bytes, void* host_staging,
                                  size_t host_bytes, int32_t max_window_chunks,
                                  int64_t slots_per_window, int64_t cache_slots,
                                  int32_t n_threads, void* compute_stream, void* copy_stream,
                                  hga_tier_stats* stats) {
  const auto t_start = std::chrono::steady_clock::now();
  hga::Geometry g;
  hga_status st = tier_geometry(cfg, dtype, batch, q_pos0, n_q, kv_cap, max_window_chunks,
                                slots_per_window, cache_slots, g);
  if (st != HGA_OK) return st;
  if (q_raw == nullptr || kv_host == nullptr || out == nullptr || chunk_sum == nullptr ||
      dev_staging == nullptr || host_staging == nullptr || n_threads < 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if (g.Kg > 0 && group_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(dev_staging) | reinterpret_cast<uintptr_t>(host_staging)) % kAlign)
    return HGA_ERR_INVALID_ARGUMENT;
  if (!pinned_host(kv_host) || !pinned_host(host_staging)) return HGA_ERR_INVALID_ARGUMENT;
  const Layout L = make_layout(g, max_window_chunks, slots_per_window, cache_slots);
  if (dev_bytes < L.dev_total || host_bytes < L.host_total) return HGA_ERR_WORKSPACE_TOO_SMALL;

  hipStream_t cs = static_cast<hipStream_t>(compute_stream);
  hipStream_t xs = static_cast<hipStream_t>(copy_stream);
  char* dev = static_cast<char*>(dev_staging);
  char* host = static_cast<char*>(host_staging);
  int32_t* d_cidx = reinterpret_cast<int32_t*>(dev + L.cidx);
  int32_t* d_gidx = reinterpret_cast<int32_t*>(dev + L.gidx);
  int32_t* d_gran = reinterpret_cast<int32_t*>(dev + L.gran);
  int32_t* d_gcnt = reinterpret_cast<int32_t*>(dev + L.gcnt);
  const int32_t* h_gran = reinterpret_cast<const int32_t*>(host + L.hgran);
  const int32_t* h_gcnt = reinterpret_cast<const int32_t*>(host + L.hcnt);

  // 1-2. route on the device, bring the granule lists to the host
  hipError_t e = hga::launch_route(g, q_raw, chunk_sum, group_sum, d_cidx, g.Kg > 0 ? d_gidx : nullptr,
                                   d_gran, d_gcnt, dev + L.rws, cs);
  if (e != hipSuccess) return hga::hip_fail(e);
  e = hipMemcpyAsync(host + L.hgran, d_gran, static_cast<size_t>(L.units) * g.gmax * 4,
                     hipMemcpyDeviceToHost, cs);
  if (e == hipSuccess)
    e = hipMemcpyAsync(host + L.hcnt, d_gcnt, static_cast<size_t>(L.units) * 4, hipMemcpyDeviceToHost, cs);
  if (e == hipSuccess) e = hipStreamSynchronize(cs);
  if (e != hipSuccess) return hga::hip_fail(e);

  Events ev;  // copied[0..1], attended[0..1]
  for (auto& x : ev.e) {
    e = hipEventCreateWithFlags(&x, hipEventDisableTiming);
    if (e != hipSuccess) return hga::hip_fail(e);
  }
  hipEvent_t* copied = ev.e;
  hipEvent_t* attended = ev.e + 2;

  const int64_t ngran = g.kv_cap / g.gs;
  const int64_t bh = static_cast<int64_t>(g.B) * g.Hkv;
  if (cache_slots > 0)
    return tiered_cached(g, L, q_raw, kv_host, out, lse, dev, host, h_gran, h_gcnt,
                         max_window_chunks, slots_per_window, cache_slots, n_threads, cs, xs,
                         copied, attended, stats, t_start);
  std::vector<int32_t> stamp(static_cast<size_t>(bh * ngran), -1);
  std::vector<int32_t> slotmap(static_cast<size_t>(bh * ngran), 0);
  std::vector<std::pair<const char*, char*>> jobs;
  jobs.reserve(static_cast<size_t>(slots_per_window));
  const char* store = static_cast<const char*>(kv_host);
  Packer packer(n_threads);
  double pack_s = 0.0;
  int64_t copied_granules = 0, bytes_h2d = 0;
  const int64_t t_end = g.t0 + g.nqc;
  int32_t w = 0;
  for (int64_t ta = g.t0; ta < t_end; ++w) {
    const int buf = w & 1;
    char* hw = host + L.hwin[buf];
    char* dw = dev + L.win[buf];
    if (w >= 2) {  // the copy that last read this host buffer must be done
      e = hipEventSynchronize(copied[buf]);
      if (e != hipSuccess) return hga::hip_fail(e);
    }
    // Grow the window one query chunk at a time while its granule union fits.
    int64_t next = 0, tb = ta;
    jobs.clear();
    while (tb < t_end && tb - ta < max_window_chunks) {
      int64_t add = 0;
      for (int64_t x = 0; x < bh; ++x) {
        const int64_t u = x * g.nqc + (tb - g.t0);
        for (int32_t i = 0; i < h_gcnt[u]; ++i) {
          const int64_t gid = h_gran[u * g.gmax + i];
          add += stamp[static_cast<size_t>(x * ngran + gid)] != w;
        }
      }
      if (next + add > slots_per_window) break;
      for (int64_t x = 0; x < bh; ++x) {
        const int64_t u = x * g.nqc + (tb - g.t0);
        for (int32_t i = 0; i < h_gcnt[u]; ++i) {
          const int64_t gid = h_gran[u * g.gmax + i];
          const size_t k = static_cast<size_t>(x * ngran + gid);
          if (stamp[k] != w) {
            stamp[k] = w;
            slotmap[k] = static_cast<int32_t>(next);
            jobs.emplace_back(store + (x * ngran + gid) * L.granule_bytes, hw + next * L.granule_bytes);
            ++next;
          }
        }
      }
      ++tb;
    }
    const int64_t nw = tb - ta;
    int32_t* wgran = reinterpret_cast<int32_t*>(hw + L.wgran);
    int32_t* wslot = reinterpret_cast<int32_t*>(hw + L.wslot);
    int32_t* wcnt = reinterpret_cast<int32_t*>(hw + L.wcnt);
    for (int64_t x = 0; x < bh; ++x) {
      for (int64_t t = ta; t < tb; ++t) {
        const int64_t u = x * g.nqc + (t - g.t0);
        const int64_t wu = x * nw + (t - ta);
        wcnt[wu] = h_gcnt[u];
        for (int32_t i = 0; i < g.gmax; ++i) {
          const int32_t gid = i < h_gcnt[u] ? h_gran[u * g.gmax + i] : -1;
          wgran[wu * g.gmax + i] = gid;
          wslot[wu * g.gmax + i] = gid >= 0 ? slotmap[static_cast<size_t>(x * ngran + gid)] : -1;
        }
      }
    }
    // 3. pack on the host threads
    const auto p0 = std::chrono::steady_clock::now();
    const size_t nj = jobs.size();
    const size_t gb = L.granule_bytes;
    packer.run([&](int i, int n) {
      const size_t lo = nj * i / n, hi = nj * (i + 1) / n;
      for (size_t j = lo; j < hi; ++j) std::memcpy(jobs[j].second, jobs[j].first, gb);
    });
    pack_s += std::chrono::duration<double>(std::chrono::steady_clock::now() - p0).count();
    // H2D on the copy stream once the attention that last read this device buffer is done
    if (w >= 2) {
      e = hipStreamWaitEvent(xs, attended[buf], 0);
      if (e != hipSuccess) return hga::hip_fail(e);
    }
    const size_t pool_used = static_cast<size_t>(next) * L.granule_bytes;
    const size_t idx_bytes = L.win_bytes - L.wgran;
    e = hipMemcpyAsync(dw, hw, pool_used, hipMemcpyHostToDevice, xs);
    if (e == hipSuccess) e = hipMemcpyAsync(dw + L.wgran, hw + L.wgran, idx_bytes, hipMemcpyHostToDevice, xs);
    if (e == hipSuccess) e = hipEventRecord(copied[buf], xs);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, copied[buf], 0);
    if (e != hipSuccess) return hga::hip_fail(e);
    copied_granules += next;
    bytes_h2d += static_cast<int64_t>(pool_used + idx_bytes);
    // attention of the window's units over the staged pool
    hga::Geometry gw = g;
    gw.q_pos0 = std::max(ta * g.C, g.q_pos0);
    gw.n_q = std::min(tb * g.C, g.q_pos0 + g.n_q) - gw.q_pos0;
    gw.t0 = ta;
    gw.nqc = nw;
    hga::AttendExtra ex;
    ex.pool_slot = reinterpret_cast<const int32_t*>(dw + L.wslot);
    ex.pool_slots = slots_per_window;
    ex.allow_split = false;
    ex.q_stride = g.n_q;
    ex.q_row0 = g.q_pos0;
    e = hga::launch_attend(gw, q_raw, dw, dw, reinterpret_cast<const int32_t*>(dw + L.wgran),
                           reinterpret_cast<const int32_t*>(dw + L.wcnt), false, out, lse, nullptr, cs, &ex);
    if (e == hipSuccess) e = hipEventRecord(attended[buf], cs);
    if (e != hipSuccess) return hga::hip_fail(e);
    ta = tb;
  }
  if (stats != nullptr) {
    stats->windows = w;
    stats->granules_copied = copied_granules;
    stats->bytes_h2d = bytes_h2d;
    stats->pack_seconds = pack_s;
    stats->host_seconds =
        std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
    stats->granules_hit = 0;
  }
  return HGA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Streaming decode from the host tier.
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3, tiered K/V store (RAM-cached decode): the token K/V history
// stays in host RAM, summaries and routing on the device, and each decode
// step moves only the granules its routes need; a device cache keeps
// granules across steps (consecutive steps re-route mostly the same ones).
//
// A session carves the caller's device / host buffers:
//   device: route outputs, route and attention workspaces, the granule
//           cache and its directory (slot of every (sequence, KV head,
//           granule), owner, token count and last-use step of every slot,
//           a replacement hand), the per-entry cache slots and one step's
//           miss list, and the raw and rotated keys of the current chunk;
//   host:   the step's hit / miss counts, read back only when asked.
// append() rotates a new token's key on the device (and builds the chunk /
// group summaries a token closes, from the current chunk's raw keys), then
// copies its rotated key and value into the host store.  step() enqueues,
// with no host wait: the routing of the step's queries; one workgroup that
// looks every listed granule up in the directory (a granule cached while
// it held fewer tokens than the step needs, i.e. the granule being filled,
// counts as a miss), gives each granule without a slot a victim slot (the
// next slots from the hand that this step does not use, in ring order) and
// writes the miss list; a gather kernel that reads the missing granules
// straight from the pinned store over the host link (no host-side packing)
// into their cache slots; then the decode attention over the cache.
// ---------------------------------------------------------------------------
namespace {

struct SessionLayout {
  int64_t units = 0, per_step = 0, keys = 0;
  size_t granule_bytes = 0, row_bytes = 0;
  size_t cidx = 0, gidx = 0, gran = 0, gcnt = 0, rws = 0, aws = 0, cache = 0, idx = 0,
         win_raw = 0, win_rot = 0, dir = 0, dev_total = 0;
  size_t hstate = 0, host_total = 0;
  size_t rws_bytes = 0, aws_bytes = 0, idx_bytes = 0, slots_off = 0, src_off = 0, dst_off = 0;
  // directory block: slot_of [keys], owner / fill / stamp [cache_slots],
  // victim [per_step] (int32 each), state [16] int32 (hand, misses, hits)
  size_t slot_of_off = 0, owner_off = 0, fill_off = 0, stamp_off = 0, victim_off = 0, state_off = 0,
         dir_bytes = 0;
};

constexpr int kDirThreads = 1024;

struct DirParams {
  const int32_t* gran;   // [units][gmax] the step's granule lists
  const int32_t* gcnt;   // [units]
  int32_t* slot_of;      // [units * ngran] cache slot of a (unit, granule) or -1
  int32_t* owner;        // [cache_slots] key held by a slot or -1
  int32_t* fill;         // [cache_slots] tokens of the slot's granule copy
  int32_t* stamp;        // [cache_slots] last step that used the slot (-1: never)
  int32_t* victim;       // [per_step] scratch: the step's victim slots
  int32_t* slots;        // [units][gmax] out: cache slot per list entry, -1 past the count
  int64_t* src;          // [per_step] out: store granule of each miss
  int32_t* dst;          // [per_step] out: its cache slot
  int32_t* state;        // [0] hand, [1] misses, [2] hits, [3] slots missing (0 unless a bug)
  int64_t units, gmax, ngran, cache_slots, pos;
  int32_t gs, step;
};

constexpr int kDirPer = 4;  // list entries per thread per pass

// Exclusive prefix, in thread order, of every thread's count c over the
// workgroup, and their total; every thread of the workgroup calls it.
__device__ int block_scan(int c, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = c;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    incl += lane >= o ? t : 0;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0, tot = 0;
  for (int w = 0; w < kDirThreads / 64; ++w) {
    const int x = wave_tot[w];
    before += w < wv ? x : 0;
    tot += x;
  }
  __syncthreads();  // wave_tot is rewritten by the next call
  total = tot;
  return before + incl - c;
}

// The decode session's cache directory, one workgroup per step: entries
// whose granule has a slot mark it used in this step; the entries without
// one take, in pass / thread / entry order, the next slots from the hand
// (ring order) that this step does not use, evicting their owners; an
// entry is a miss when its slot is new or holds fewer tokens than the step
// needs.  Slots used in the step (every fixed-window granule, every step)
// are never victims, and one step's entries fit the cache (cache_slots >=
// per_step), so the victim search ends within one pass over the slots.
// Each thread takes kDirPer entries per pass (entry e0 + j * kDirThreads +
// tid) so that their loads are in flight together.
__global__ __launch_bounds__(kDirThreads) void directory_kernel(DirParams p) {
  __shared__ int wave_tot[kDirThreads / 64];
  __shared__ int s_need, s_hits;
  __shared__ long long s_hand;
  const int tid = threadIdx.x;
  const int64_t n = p.units * p.gmax;
  const int64_t pass = static_cast<int64_t>(kDirPer) * kDirThreads;
  if (tid == 0) {
    s_need = 0;
    s_hits = 0;
    s_hand = p.state[0];
  }
  __syncthreads();
  // 1. lookups; a found slot is marked used in this step
  int need = 0;
  for (int64_t e0 = 0; e0 < n; e0 += pass) {
    int64_t key[kDirPer];
    int32_t sl[kDirPer];
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      const int64_t e = e0 + j * kDirThreads + tid;
      key[j] = -1;
      if (e < n) {
        const int64_t x = e / p.gmax, gid = p.gran[e];
        if (e - x * p.gmax < p.gcnt[x] && gid >= 0 && gid < p.ngran) key[j] = x * p.ngran + gid;
      }
    }
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) sl[j] = key[j] >= 0 ? p.slot_of[key[j]] : -2;
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      const int64_t e = e0 + j * kDirThreads + tid;
      if (sl[j] >= 0) p.stamp[sl[j]] = p.step;
      need += sl[j] == -1 ? 1 : 0;
      if (e < n) p.slots[e] = sl[j];
    }
  }
  atomicAdd(&s_need, need);
  __syncthreads();
  const int R = s_need;
  const int64_t hand = s_hand;
  // 2. R victims: the slots this step does not use, from the hand on
  int found = 0;
  for (int64_t base = 0; found < R && base < p.cache_slots; base += kDirThreads) {
    const int64_t j = base + tid;
    int32_t slot = -1;
    bool fr = false;
    if (j < p.cache_slots) {
      slot = static_cast<int32_t>((hand + j) % p.cache_slots);
      fr = p.stamp[slot] != p.step;
    }
    int tot = 0;
    const int r = found + block_scan(fr ? 1 : 0, wave_tot, tot);
    if (fr && r < R) {
      p.victim[r] = slot;
      if (r == R - 1) s_hand = (slot + 1) % p.cache_slots;
    }
    found += tot;
  }
  const int have = found < R ? found : R;
  // 3. new slots, misses, the per-entry slots
  int new_base = 0, miss_base = 0, hits = 0;
  for (int64_t e0 = 0; e0 < n; e0 += pass) {
    int32_t sl[kDirPer], last[kDirPer], fill[kDirPer];
    int64_t key[kDirPer];
    int fresh = 0;
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      const int64_t e = e0 + j * kDirThreads + tid;
      sl[j] = e < n ? p.slots[e] : -2;
    }
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      const int64_t e = e0 + j * kDirThreads + tid;
      key[j] = 0;
      last[j] = 0;
      if (sl[j] != -2) {
        const int64_t x = e / p.gmax, gid = p.gran[e];
        key[j] = x * p.ngran + gid;
        const int64_t left = p.pos + 1 - gid * p.gs;  // tokens this step needs
        last[j] = static_cast<int32_t>(left < p.gs ? left : p.gs);
      }
      fresh += sl[j] == -1 ? 1 : 0;
    }
    int tot = 0;
    int r = new_base + block_scan(fresh, wave_tot, tot);
    new_base += tot;
    int32_t prev[kDirPer];
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      fill[j] = 0;
      prev[j] = -1;
      if (sl[j] == -1) {
        if (r < have) {
          sl[j] = p.victim[r];
          key[j] = ~key[j];  // marks a new slot (keys are >= 0)
        } else {
          sl[j] = -2;  // unreachable while cache_slots >= per_step
        }
        ++r;
      } else if (sl[j] >= 0) {
        fill[j] = p.fill[sl[j]];
      }
    }
#pragma unroll
    for (int j = 0; j < kDirPer; ++j)
      if (key[j] < 0) prev[j] = p.owner[sl[j]];
    int misses = 0;
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      if (key[j] < 0) {
        key[j] = ~key[j];
        if (prev[j] >= 0) p.slot_of[prev[j]] = -1;
        p.owner[sl[j]] = static_cast<int32_t>(key[j]);
        p.slot_of[key[j]] = sl[j];
        p.stamp[sl[j]] = p.step;
        fill[j] = -1;  // a new slot is a miss
      }
      misses += (sl[j] >= 0 && fill[j] < last[j]) ? 1 : 0;
    }
    int m = miss_base + block_scan(misses, wave_tot, tot);
    miss_base += tot;
#pragma unroll
    for (int j = 0; j < kDirPer; ++j) {
      const int64_t e = e0 + j * kDirThreads + tid;
      if (sl[j] >= 0 && fill[j] < last[j]) {
        p.fill[sl[j]] = last[j];
        p.src[m] = key[j];
        p.dst[m] = sl[j];
        ++m;
      } else if (sl[j] >= 0) {
        ++hits;
      }
      if (e < n) p.slots[e] = sl[j] >= 0 ? sl[j] : -1;
    }
  }
  atomicAdd(&s_hits, hits);
  __syncthreads();
  if (tid == 0) {
    p.state[0] = static_cast<int32_t>(s_hand);
    p.state[1] = miss_base;
    p.state[2] = s_hits;
    p.state[3] = R - have;
  }
}

// Empty directory: no granule has a slot, no slot an owner or a use.
__global__ __launch_bounds__(256) void directory_init(int32_t* slot_of, int64_t keys, int32_t* owner,
                                                      int32_t* fill, int32_t* stamp, int64_t slots,
                                                      int32_t* state) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < keys; i += stride) slot_of[i] = -1;
  for (int64_t i = i0; i < slots; i += stride) {
    owner[i] = -1;
    fill[i] = 0;
    stamp[i] = -1;
  }
  if (i0 < 16) state[i0] = 0;
}

// Reads granule src[j] of the pinned host store (through its device
// mapping, over the host link) into cache slot dst[j] for j < *count (the
// directory's miss count); workgroups stride over the misses, 16-byte words.
__global__ __launch_bounds__(256) void fetch_granules(const uint4* store, const int64_t* src,
                                                      const int32_t* dst, const int32_t* count,
                                                      uint4* cache, int64_t words) {
  const int32_t n = *count;
  for (int32_t j = blockIdx.x; j < n; j += gridDim.x) {
    const uint4* in = store + src[j] * words;
    uint4* out = cache + static_cast<int64_t>(dst[j]) * words;
    for (int64_t i = threadIdx.x; i < words; i += blockDim.x) out[i] = in[i];
  }
}

// Geometry of a decode call at position pos (one query per sequence).
hga_status session_geometry(const hga_config* cfg, hga_dtype dtype, int32_t batch, int64_t kv_cap,
                            int64_t pos, hga::Geometry& g) {
  return hga::make_geometry(cfg, dtype, batch, kv_cap, pos, 1, g);
}

hga_status session_layout(const hga_config* cfg, hga_dtype dtype, int32_t batch, int64_t kv_cap,
                          int64_t cache_slots, SessionLayout& L) {
  hga::Geometry g;
  // sizes at the last position: route and attention workspaces only grow
  // with the context
  hga_status st = session_geometry(cfg, dtype, batch, kv_cap, kv_cap - 1, g);
  if (st != HGA_OK) return st;
  if (dtype != HGA_BF16 || g.G > 16) return HGA_ERR_UNSUPPORTED;  // decode attention kernel
  if (!hga::route_supported(g) || !hga::attend_supported(g)) return HGA_ERR_UNSUPPORTED;
  L.units = static_cast<int64_t>(g.B) * g.Hkv;
  L.per_step = L.units * g.gmax;
  if (cache_slots < L.per_step) return HGA_ERR_INVALID_ARGUMENT;
  L.granule_bytes = static_cast<size_t>(2) * g.gs * g.d * 2;
  L.row_bytes = static_cast<size_t>(g.d) * 2;
  if (static_cast<double>(cache_slots) * 2 * g.gs >= 2147483647.0) return HGA_ERR_UNSUPPORTED;
  L.rws_bytes = hga::route_workspace(g);
  L.aws_bytes = hga::attend_workspace(g, false, true);
  const size_t u = static_cast<size_t>(L.units);
  size_t off = 0;
  L.cidx = off; off = align_up(off + u * std::max(g.Kc, 1) * 4);
  L.gidx = off; off = align_up(off + u * std::max(g.Kg, 1) * 4);
  L.gran = off; off = align_up(off + u * g.gmax * 4);
  L.gcnt = off; off = align_up(off + u * 4);
  L.rws = off; off = align_up(off + L.rws_bytes);
  L.aws = off; off = align_up(off + L.aws_bytes);
  L.cache = off; off = align_up(off + static_cast<size_t>(cache_slots) * L.granule_bytes);
  // index block: slots [per_step] int32, src [per_step] int64, dst [per_step] int32
  L.slots_off = 0;
  L.src_off = align_up(static_cast<size_t>(L.per_step) * 4);
  L.dst_off = align_up(L.src_off + static_cast<size_t>(L.per_step) * 8);
  L.idx_bytes = align_up(L.dst_off + static_cast<size_t>(L.per_step) * 4);
  L.idx = off; off = align_up(off + L.idx_bytes);
  L.win_raw = off; off = align_up(off + u * g.C * L.row_bytes);
  L.win_rot = off; off = align_up(off + u * g.C * L.row_bytes);
  // the directory keys (unit, granule) and slots as int32
  L.keys = L.units * (kv_cap / g.gs);
  if (L.keys >= 2147483647 || cache_slots >= 2147483647) return HGA_ERR_UNSUPPORTED;
  L.slot_of_off = 0;
  L.owner_off = align_up(static_cast<size_t>(L.keys) * 4);
  L.fill_off = align_up(L.owner_off + static_cast<size_t>(cache_slots) * 4);
  L.stamp_off = align_up(L.fill_off + static_cast<size_t>(cache_slots) * 4);
  L.victim_off = align_up(L.stamp_off + static_cast<size_t>(cache_slots) * 4);
  L.state_off = align_up(L.victim_off + static_cast<size_t>(L.per_step) * 4);
  L.dir_bytes = align_up(L.state_off + 16 * 4);
  L.dir = off; off = align_up(off + L.dir_bytes);
  L.dev_total = off;
  L.hstate = 0;
  L.host_total = align_up(16 * 4);
  return HGA_OK;
}

}  // namespace

struct hga_decode_session {
  hga_config cfg;
  hga_dtype dtype;
  int32_t batch;
  int64_t kv_cap, cache_slots, ngran;
  SessionLayout L;
  char* dev;
  char* host;
  char* store;
  const uint4* store_dev;        // the store's device mapping
  int32_t steps = 0;             // steps enqueued (the directory's use stamps)
  bool dir_ready = false;        // directory cleared on the device
  int64_t next_pos;              // position append() expects next
};

extern "C" {

hga_status hga_decode_session_cache_slots(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                          int64_t kv_cap, size_t headroom_bytes, int64_t* cache_slots) {
  if (cfg == nullptr || cache_slots == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  hga::Geometry g;
  hga_status st = session_geometry(cfg, dtype, batch, kv_cap, kv_cap - 1, g);
  if (st != HGA_OK) return st;
  size_t budget = 0;
  st = free_budget(headroom_bytes, budget);
  if (st != HGA_OK) return st;
  const int64_t lo = static_cast<int64_t>(g.B) * g.Hkv * g.gmax;         // one step's granules
  const int64_t hi = static_cast<int64_t>(g.B) * g.Hkv * (kv_cap / g.gs);  // the whole store
  auto fits = [&](int64_t n) {
    SessionLayout L;
    return session_layout(cfg, dtype, batch, kv_cap, n, L) == HGA_OK && L.dev_total <= budget;
  };
  const int64_t n = largest_fitting(lo, std::max(lo, hi), fits);
  if (n < lo) return HGA_ERR_WORKSPACE_TOO_SMALL;  // a session needs one step's granules
  *cache_slots = n;
  return HGA_OK;
}

hga_status hga_decode_session_buffer_bytes(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                           int64_t kv_cap, int64_t cache_slots,
                                           size_t* device_bytes, size_t* host_bytes) {
  if (cfg == nullptr || device_bytes == nullptr || host_bytes == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  SessionLayout L;
  hga_status st = session_layout(cfg, dtype, batch, kv_cap, cache_slots, L);
  if (st != HGA_OK) return st;
  *device_bytes = L.dev_total;
  *host_bytes = L.host_total;
  return HGA_OK;
}

hga_status hga_decode_session_create(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                     int64_t kv_cap, int64_t first_pos, int64_t cache_slots,
                                     void* kv_host, void* dev_buffer, size_t dev_bytes,
                                     void* host_buffer, size_t host_bytes,
                                     hga_decode_session** session) {
  if (session == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  *session = nullptr;
  if (cfg == nullptr || kv_host == nullptr || dev_buffer == nullptr || host_buffer == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  SessionLayout L;
  hga_status st = session_layout(cfg, dtype, batch, kv_cap, cache_slots, L);
  if (st != HGA_OK) return st;
  if (first_pos < 0 || first_pos >= kv_cap || first_pos % cfg->chunk_size != 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(dev_buffer) | reinterpret_cast<uintptr_t>(host_buffer)) % kAlign)
    return HGA_ERR_INVALID_ARGUMENT;
  if (!pinned_host(kv_host) || !pinned_host(host_buffer)) return HGA_ERR_INVALID_ARGUMENT;
  if (dev_bytes < L.dev_total || host_bytes < L.host_total) return HGA_ERR_WORKSPACE_TOO_SMALL;
  void* store_dev = nullptr;
  hipError_t e = hipHostGetDevicePointer(&store_dev, kv_host, 0);
  if (e != hipSuccess || store_dev == nullptr) {
    (void)hipGetLastError();
    return HGA_ERR_UNSUPPORTED;  // the store must be mapped into the device's address space
  }
  hga_decode_session* s = nullptr;
  try {
    s = new hga_decode_session();
    s->cfg = *cfg;
    s->dtype = dtype;
    s->batch = batch;
    s->kv_cap = kv_cap;
    s->cache_slots = cache_slots;
    s->ngran = kv_cap / cfg->group_size;
    s->L = L;
    s->dev = static_cast<char*>(dev_buffer);
    s->host = static_cast<char*>(host_buffer);
    s->store = static_cast<char*>(kv_host);
    s->store_dev = static_cast<const uint4*>(store_dev);
    s->next_pos = first_pos;
  } catch (...) {
    delete s;
    return HGA_ERR_INVALID_ARGUMENT;
  }
  *session = s;
  return HGA_OK;
}

void hga_decode_session_destroy(hga_decode_session* session) { delete session; }

hga_status hga_decode_session_append(hga_decode_session* s, const void* k_raw_new, const void* v_new,
                                     int64_t pos, float* chunk_sum, float* group_sum,
                                     void* compute_stream) {
  if (s == nullptr || k_raw_new == nullptr || v_new == nullptr || chunk_sum == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  if (s->cfg.top_groups > 0 && group_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if (pos != s->next_pos || pos >= s->kv_cap) return HGA_ERR_INVALID_ARGUMENT;
  hga::Geometry g;
  hga_status st = session_geometry(&s->cfg, s->dtype, s->batch, s->kv_cap, pos, g);
  if (st != HGA_OK) return st;
  hipStream_t cs = static_cast<hipStream_t>(compute_stream);
  const SessionLayout& L = s->L;
  const int64_t w0 = pos / g.C * g.C;
  const size_t row = static_cast<size_t>(pos - w0);
  const size_t rb = L.row_bytes;
  char* win_raw = s->dev + L.win_raw;
  char* win_rot = s->dev + L.win_rot;
  // raw key into the current chunk's window, then rotation (and the
  // summaries of the blocks this token closes) on the device
  hipError_t e = hipMemcpy2DAsync(win_raw + row * rb, g.C * rb, k_raw_new, rb, rb,
                                  static_cast<size_t>(L.units), hipMemcpyDeviceToDevice, cs);
  if (e == hipSuccess)
    e = hga::launch_summarize(g, win_raw, pos, pos + 1, win_rot, chunk_sum, group_sum, cs, w0, g.C);
  // rotated key and value into the granule-major host store
  const size_t gb = L.granule_bytes;
  const int64_t gid = pos / g.gs;
  const size_t in_gran = static_cast<size_t>(pos % g.gs) * rb;
  char* dst = s->store + static_cast<size_t>(gid) * gb + in_gran;
  if (e == hipSuccess)
    e = hipMemcpy2DAsync(dst, static_cast<size_t>(s->ngran) * gb, win_rot + row * rb, g.C * rb, rb,
                         static_cast<size_t>(L.units), hipMemcpyDeviceToHost, cs);
  if (e == hipSuccess)
    e = hipMemcpy2DAsync(dst + static_cast<size_t>(g.gs) * rb, static_cast<size_t>(s->ngran) * gb,
                         v_new, rb, rb, static_cast<size_t>(L.units), hipMemcpyDeviceToHost, cs);
  if (e != hipSuccess) return hga::hip_fail(e);
  s->next_pos = pos + 1;
  return HGA_OK;
}

hga_status hga_decode_session_step(hga_decode_session* s, const void* q_raw, int64_t pos,
                                   const float* chunk_sum, const float* group_sum, void* out,
                                   float* lse, void* compute_stream, hga_tier_stats* stats) {
  const auto t_start = std::chrono::steady_clock::now();
  if (s == nullptr || q_raw == nullptr || chunk_sum == nullptr || out == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  if (s->cfg.top_groups > 0 && group_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if (pos < 0 || pos >= s->next_pos) return HGA_ERR_INVALID_ARGUMENT;  // its token must be stored
  hga::Geometry g;
  hga_status st = session_geometry(&s->cfg, s->dtype, s->batch, s->kv_cap, pos, g);
  if (st != HGA_OK) return st;
  hipStream_t cs = static_cast<hipStream_t>(compute_stream);
  const SessionLayout& L = s->L;
  char* dev = s->dev;
  char* host = s->host;
  int32_t* d_gran = reinterpret_cast<int32_t*>(dev + L.gran);
  int32_t* d_gcnt = reinterpret_cast<int32_t*>(dev + L.gcnt);
  char* dir = dev + L.dir;
  int32_t* d_state = reinterpret_cast<int32_t*>(dir + L.state_off);
  hipError_t e = hipSuccess;
  if (s->steps == 2147483647) {
    // use stamps would repeat: start again from an empty cache
    s->steps = 0;
    s->dir_ready = false;
  }
  if (!s->dir_ready) {
    hipLaunchKernelGGL(directory_init, dim3(256), dim3(256), 0, cs,
                       reinterpret_cast<int32_t*>(dir + L.slot_of_off), L.keys,
                       reinterpret_cast<int32_t*>(dir + L.owner_off), reinterpret_cast<int32_t*>(dir + L.fill_off),
                       reinterpret_cast<int32_t*>(dir + L.stamp_off), s->cache_slots, d_state);
    e = hipGetLastError();
    if (e != hipSuccess) return hga::hip_fail(e);
    s->dir_ready = true;
  }
  e = hga::launch_route(g, q_raw, chunk_sum, group_sum, reinterpret_cast<int32_t*>(dev + L.cidx),
                        g.Kg > 0 ? reinterpret_cast<int32_t*>(dev + L.gidx) : nullptr, d_gran, d_gcnt,
                        dev + L.rws, cs);
  if (e != hipSuccess) return hga::hip_fail(e);
  int32_t* d_slots = reinterpret_cast<int32_t*>(dev + L.idx + L.slots_off);
  int64_t* d_src = reinterpret_cast<int64_t*>(dev + L.idx + L.src_off);
  int32_t* d_dst = reinterpret_cast<int32_t*>(dev + L.idx + L.dst_off);
  DirParams dp;
  dp.gran = d_gran;
  dp.gcnt = d_gcnt;
  dp.slot_of = reinterpret_cast<int32_t*>(dir + L.slot_of_off);
  dp.owner = reinterpret_cast<int32_t*>(dir + L.owner_off);
  dp.fill = reinterpret_cast<int32_t*>(dir + L.fill_off);
  dp.stamp = reinterpret_cast<int32_t*>(dir + L.stamp_off);
  dp.victim = reinterpret_cast<int32_t*>(dir + L.victim_off);
  dp.slots = d_slots;
  dp.src = d_src;
  dp.dst = d_dst;
  dp.state = d_state;
  dp.units = L.units;
  dp.gmax = g.gmax;
  dp.ngran = s->ngran;
  dp.cache_slots = s->cache_slots;
  dp.pos = pos;
  dp.gs = static_cast<int32_t>(g.gs);
  dp.step = s->steps++;
  hipLaunchKernelGGL(directory_kernel, dim3(1), dim3(kDirThreads), 0, cs, dp);
  e = hipGetLastError();
  if (e != hipSuccess) return hga::hip_fail(e);
  const size_t gb = L.granule_bytes;
  char* cache = dev + L.cache;
  const unsigned fetch_groups = static_cast<unsigned>(std::min<int64_t>(L.per_step, 1024));
  hipLaunchKernelGGL(fetch_granules, dim3(fetch_groups), dim3(256), 0, cs, s->store_dev, d_src, d_dst,
                     d_state + 1, reinterpret_cast<uint4*>(cache), static_cast<int64_t>(gb / 16));
  e = hipGetLastError();
  if (e != hipSuccess) return hga::hip_fail(e);
  hga::AttendExtra ex;
  ex.pool_slot = d_slots;
  ex.pool_slots = s->cache_slots;
  ex.allow_split = true;
  e = hga::launch_attend(g, q_raw, cache, cache, d_gran, d_gcnt, false, out, lse, dev + L.aws, cs, &ex);
  if (e != hipSuccess) return hga::hip_fail(e);
  if (stats != nullptr) {
    // the only wait of a step, and only when its counts are asked for
    int32_t* h_state = reinterpret_cast<int32_t*>(host + L.hstate);
    e = hipMemcpyAsync(h_state, d_state, 16 * 4, hipMemcpyDeviceToHost, cs);
    if (e == hipSuccess) e = hipStreamSynchronize(cs);
    if (e != hipSuccess) return hga::hip_fail(e);
    stats->windows = 1;
    stats->granules_copied = h_state[1];
    stats->bytes_h2d = static_cast<int64_t>(static_cast<size_t>(h_state[1]) * gb);
    stats->pack_seconds = 0.0;
    stats->host_seconds =
        std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
    stats->granules_hit = h_state[2];
  }
  return HGA_OK;
}

}  // extern "C"
