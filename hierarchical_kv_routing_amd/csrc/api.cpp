// C ABI of the routed exact-token attention library: argument validation,
// call geometry, workspace sizing and kernel dispatch.  Every check runs on
// the host before anything is enqueued; on an error nothing is enqueued.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "hga_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

}  // namespace

int hga::current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  return dev;
}

// Compute units of the current device, queried once per device (the cache
// entries are atomics, so concurrent first calls agree).
int64_t hga::device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus[kMaxDevices];
  const int dev = current_device();
  if (dev >= kMaxDevices) {
    int n = 0;
    (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    return n > 0 ? n : 256;
  }
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    v = n > 0 ? n : 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hga_status hga::hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return HGA_ERR_HIP;
}

namespace {
using hga::hip_fail;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

hga_status check_config(const hga_config* c) {
  if (c == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if (c->chunk_size <= 0 || c->group_size <= 0 || c->chunk_size % c->group_size != 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads != 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if (c->n_sink_chunks < 0 || c->n_recent_chunks < 0 || c->top_chunks < 0 || c->top_groups < 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if (c->head_dim <= 0 || (c->head_dim & 1) != 0) return HGA_ERR_INVALID_ARGUMENT;
  if (c->n_hf_pairs < 0 || c->n_hf_pairs > c->head_dim / 2) return HGA_ERR_INVALID_ARGUMENT;
  if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta)) return HGA_ERR_INVALID_ARGUMENT;
  if (!(c->softmax_scale >= 0.f) || !std::isfinite(c->softmax_scale)) return HGA_ERR_INVALID_ARGUMENT;
  if (c->rope_period < 0 || c->rope_period % c->chunk_size != 0) return HGA_ERR_INVALID_ARGUMENT;
  if (c->head_dim != 64 && c->head_dim != 128) return HGA_ERR_UNSUPPORTED;
  if (c->chunk_size > 64) return HGA_ERR_UNSUPPORTED;
  return HGA_OK;
}

int32_t max_granules(const hga_config* c) {
  const int32_t r = c->chunk_size / c->group_size;
  const int32_t lp = c->n_recent_chunks > 1 ? c->n_recent_chunks : 1;
  const int32_t routed = c->top_groups > 0 ? c->top_groups : c->top_chunks * r;
  return r * (1 + c->n_sink_chunks + lp) + routed;
}

}  // namespace

hga_status hga::make_geometry(const hga_config* c, hga_dtype dt, int32_t batch, int64_t kv_cap,
                              int64_t q_pos0, int64_t n_q, hga::Geometry& g) {
  hga_status st = check_config(c);
  if (st != HGA_OK) return st;
  if (dt != HGA_F32 && dt != HGA_BF16) return HGA_ERR_INVALID_ARGUMENT;
  if (batch <= 0 || kv_cap <= 0 || kv_cap % c->chunk_size != 0) return HGA_ERR_INVALID_ARGUMENT;
  if (kv_cap > (int64_t{1} << 30)) return HGA_ERR_UNSUPPORTED;
  if (q_pos0 < 0 || n_q < 0 || q_pos0 + n_q > kv_cap) return HGA_ERR_INVALID_ARGUMENT;
  g.B = batch;
  g.Hq = c->n_q_heads;
  g.Hkv = c->n_kv_heads;
  g.G = g.Hq / g.Hkv;
  g.d = c->head_dim;
  g.C = c->chunk_size;
  g.gs = c->group_size;
  g.r = g.C / g.gs;
  g.F = c->n_sink_chunks;
  g.L = c->n_recent_chunks;
  g.Kc = c->top_chunks;
  g.Kg = c->top_groups;
  g.n_hf = c->n_hf_pairs;
  g.kv_cap = kv_cap;
  g.q_pos0 = q_pos0;
  g.n_q = n_q;
  g.t0 = n_q > 0 ? q_pos0 / g.C : 0;
  g.nqc = n_q > 0 ? (q_pos0 + n_q - 1) / g.C - g.t0 + 1 : 0;
  g.gmax = max_granules(c);
  g.scale = c->softmax_scale > 0.f ? c->softmax_scale : 1.0f / std::sqrt(static_cast<float>(g.d));
  g.bf16 = dt == HGA_BF16;
  for (int b = 0; b < 6; ++b) g.rope.step[b] = std::pow(c->rope_theta, -2.0 * (1 << b) / g.d);
  g.rope.period = c->rope_period;
  const int64_t units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  if (units * 64 > (int64_t{1} << 31) - 1) return HGA_ERR_UNSUPPORTED;
  return HGA_OK;
}

namespace {
using hga::make_geometry;
}  // namespace

extern "C" {

const char* hga_status_string(hga_status s) {
  switch (s) {
    case HGA_OK: return "HGA_OK";
    case HGA_ERR_INVALID_ARGUMENT: return "HGA_ERR_INVALID_ARGUMENT";
    case HGA_ERR_UNSUPPORTED: return "HGA_ERR_UNSUPPORTED";
    case HGA_ERR_WORKSPACE_TOO_SMALL: return "HGA_ERR_WORKSPACE_TOO_SMALL";
    case HGA_ERR_HIP: return "HGA_ERR_HIP";
  }
  return "HGA_ERR_UNKNOWN";
}

int hga_last_hip_error(void) { return g_last_hip_error; }

int32_t hga_max_granules(const hga_config* cfg) {
  if (check_config(cfg) != HGA_OK) return -1;
  return max_granules(cfg);
}

hga_status hga_build_summaries(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                               const void* k_raw, int64_t kv_cap, int64_t tok_begin,
                               int64_t tok_end, void* k_rot, float* chunk_sum, float* group_sum,
                               void* stream) {
  hga::Geometry g;
  hga_status st = make_geometry(cfg, dtype, batch, kv_cap, 0, 0, g);
  if (st != HGA_OK) return st;
  if (tok_begin < 0 || tok_end <= tok_begin || tok_end > kv_cap) return HGA_ERR_INVALID_ARGUMENT;
  if (k_raw == nullptr || chunk_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if (cfg->top_groups > 0 && group_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if (!aligned16(k_raw) || !aligned16(chunk_sum) || !aligned16(k_rot) || !aligned16(group_sum))
    return HGA_ERR_INVALID_ARGUMENT;
  hipError_t e = hga::launch_summarize(g, k_raw, tok_begin, tok_end, k_rot, chunk_sum, group_sum,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HGA_OK : hip_fail(e);
}

size_t hga_route_workspace_bytes(const hga_config* cfg, int32_t batch, int64_t q_pos0, int64_t n_q) {
  hga::Geometry g;
  if (cfg == nullptr || cfg->chunk_size <= 0) return 0;
  const int64_t capc = ((q_pos0 + n_q + cfg->chunk_size - 1) / cfg->chunk_size) * cfg->chunk_size;
  if (make_geometry(cfg, HGA_BF16, batch, capc > 0 ? capc : cfg->chunk_size, q_pos0, n_q, g) != HGA_OK)
    return 0;
  return hga::route_workspace(g);
}

hga_status hga_route(const hga_config* cfg, hga_dtype dtype, int32_t batch, const void* q_raw,
                     int64_t q_pos0, int64_t n_q, const float* chunk_sum, const float* group_sum,
                     int64_t kv_cap, int32_t* chunk_idx, int32_t* group_idx, int32_t* granules,
                     int32_t* granule_count, void* workspace, size_t workspace_bytes,
                     void* stream) {
  hga::Geometry g;
  hga_status st = make_geometry(cfg, dtype, batch, kv_cap, q_pos0, n_q, g);
  if (st != HGA_OK) return st;
  if (n_q == 0) return HGA_OK;  // nothing to route
  if (!hga::route_supported(g)) return HGA_ERR_UNSUPPORTED;
  if (q_raw == nullptr || granules == nullptr || granule_count == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  if (g.Kc > 0 && (chunk_sum == nullptr || chunk_idx == nullptr)) return HGA_ERR_INVALID_ARGUMENT;
  if (g.Kg > 0 && (group_sum == nullptr || group_idx == nullptr)) return HGA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_raw) || !aligned16(chunk_sum) || !aligned16(group_sum) || !aligned16(workspace))
    return HGA_ERR_INVALID_ARGUMENT;
  const size_t need = hga::route_workspace(g);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return HGA_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = hga::launch_route(g, q_raw, chunk_sum, group_sum, chunk_idx, group_idx, granules,
                                   granule_count, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HGA_OK : hip_fail(e);
}

size_t hga_attend_workspace_bytes(const hga_config* cfg, int32_t batch, int64_t q_pos0, int64_t n_q) {
  hga::Geometry g;
  if (cfg == nullptr || cfg->chunk_size <= 0) return 0;
  const int64_t capc = ((q_pos0 + n_q + cfg->chunk_size - 1) / cfg->chunk_size) * cfg->chunk_size;
  size_t need = 0;
  for (hga_dtype dt : {HGA_BF16, HGA_F32}) {
    if (make_geometry(cfg, dt, batch, capc > 0 ? capc : cfg->chunk_size, q_pos0, n_q, g) != HGA_OK)
      return 0;
    for (bool dense : {false, true}) {
      const size_t w = hga::attend_workspace(g, dense);
      if (w > need) need = w;
    }
  }
  return need;
}

static hga_status attend_common(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                const void* q_raw, int64_t q_pos0, int64_t n_q, const void* k_rot,
                                const void* v, int64_t kv_cap, const int32_t* granules,
                                const int32_t* granule_count, bool dense, void* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream,
                                bool static_scratch = false) {
  hga::Geometry g;
  hga_status st = make_geometry(cfg, dtype, batch, kv_cap, q_pos0, n_q, g);
  if (st != HGA_OK) return st;
  if (n_q == 0) return HGA_OK;  // no queries
  if (!hga::attend_supported(g)) return HGA_ERR_UNSUPPORTED;
  if (q_raw == nullptr || k_rot == nullptr || v == nullptr || out == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  if (!dense && (granules == nullptr || granule_count == nullptr)) return HGA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_raw) || !aligned16(k_rot) || !aligned16(v) || !aligned16(out) ||
      !aligned16(workspace))
    return HGA_ERR_INVALID_ARGUMENT;
  const size_t need = hga::attend_workspace(g, dense);
  if (static_scratch) {
    // the library's static scratch replaces the caller's workspace
    if (need > hga::kNoAllocScratchBytes) return HGA_ERR_WORKSPACE_TOO_SMALL;
    workspace = nullptr;
    if (need > 0) {
      const hipError_t e = hga::attend_noalloc_scratch(&workspace);
      if (e != hipSuccess) return hip_fail(e);
    }
  } else if (need > 0 && (workspace == nullptr || workspace_bytes < need)) {
    return HGA_ERR_WORKSPACE_TOO_SMALL;
  }
  hipError_t e = hga::launch_attend(g, q_raw, k_rot, v, granules, granule_count, dense, out, lse,
                                    workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HGA_OK : hip_fail(e);
}

hga_status hga_attend_noalloc(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                              const void* q_raw, int64_t q_pos0, int64_t n_q, const void* k_rot,
                              const void* v, int64_t kv_cap, const int32_t* granules,
                              const int32_t* granule_count, void* out, float* lse, void* stream) {
  return attend_common(cfg, dtype, batch, q_raw, q_pos0, n_q, k_rot, v, kv_cap, granules,
                       granule_count, false, out, lse, nullptr, 0, stream, true);
}

size_t hga_attend_noalloc_max_scratch_bytes(void) { return hga::kNoAllocScratchBytes; }

size_t hga_decode_step_workspace_bytes(const hga_config* cfg, int32_t batch, int64_t pos) {
  hga::Geometry g;
  if (cfg == nullptr || cfg->chunk_size <= 0 || pos < 0) return 0;
  const int64_t cap = (pos / cfg->chunk_size + 1) * cfg->chunk_size;
  if (make_geometry(cfg, HGA_BF16, batch, cap, pos, 1, g) != HGA_OK) return 0;
  return hga::decode_step_workspace(g);
}

hga_status hga_decode_step(const hga_config* cfg, hga_dtype dtype, int32_t batch, const void* q_raw,
                           int64_t pos, const void* k_rot, const void* v, int64_t kv_cap,
                           const float* chunk_sum, const float* group_sum, int32_t* chunk_idx,
                           int32_t* group_idx, int32_t* granules, int32_t* granule_count,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           void* stream) {
  hga::Geometry g;
  hga_status st = make_geometry(cfg, dtype, batch, kv_cap, pos, 1, g);
  if (st != HGA_OK) return st;
  if (!hga::decode_step_supported(g)) return HGA_ERR_UNSUPPORTED;
  if (q_raw == nullptr || k_rot == nullptr || v == nullptr || out == nullptr || workspace == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  if (g.Kc > 0 && chunk_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  if (g.Kg > 0 && group_sum == nullptr) return HGA_ERR_INVALID_ARGUMENT;
  // the lists: all or none (group_idx only with group routing)
  const bool lists = granules != nullptr;
  if (lists != (granule_count != nullptr) || (lists && g.Kc > 0 && chunk_idx == nullptr) ||
      (lists && g.Kg > 0 && group_idx == nullptr))
    return HGA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_raw) || !aligned16(k_rot) || !aligned16(v) || !aligned16(out) ||
      !aligned16(chunk_sum) || !aligned16(group_sum) || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return HGA_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < hga::decode_step_workspace(g)) return HGA_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = hga::launch_decode_step(g, q_raw, k_rot, v, chunk_sum, group_sum,
                                         lists ? chunk_idx : nullptr, lists ? group_idx : nullptr,
                                         granules, granule_count, out, lse, workspace,
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HGA_OK : hip_fail(e);
}

hga_status hga_attend(const hga_config* cfg, hga_dtype dtype, int32_t batch, const void* q_raw,
                      int64_t q_pos0, int64_t n_q, const void* k_rot, const void* v, int64_t kv_cap,
                      const int32_t* granules, const int32_t* granule_count, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return attend_common(cfg, dtype, batch, q_raw, q_pos0, n_q, k_rot, v, kv_cap, granules,
                       granule_count, false, out, lse, workspace, workspace_bytes, stream);
}

hga_status hga_dense_causal(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                            const void* q_raw, int64_t q_pos0, int64_t n_q, const void* k_rot,
                            const void* v, int64_t kv_cap, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return attend_common(cfg, dtype, batch, q_raw, q_pos0, n_q, k_rot, v, kv_cap, nullptr, nullptr,
                       true, out, lse, workspace, workspace_bytes, stream);
}

size_t hga_attend_backward_workspace_bytes(const hga_config* cfg, int32_t batch, int64_t q_pos0,
                                           int64_t n_q) {
  hga::Geometry g;
  if (cfg == nullptr || cfg->chunk_size <= 0) return 0;
  const int64_t capc = ((q_pos0 + n_q + cfg->chunk_size - 1) / cfg->chunk_size) * cfg->chunk_size;
  if (make_geometry(cfg, HGA_BF16, batch, capc > 0 ? capc : cfg->chunk_size, q_pos0, n_q, g) != HGA_OK)
    return 0;
  return hga::backward_workspace(g);
}

hga_status hga_attend_backward(const hga_config* cfg, hga_dtype dtype, int32_t batch, const void* q_raw,
                               int64_t q_pos0, int64_t n_q, const void* k_rot, const void* v,
                               int64_t kv_cap, const int32_t* granules, const int32_t* granule_count,
                               const void* out, const float* lse, const void* d_out, float* dq,
                               float* dk, float* dv, void* workspace, size_t workspace_bytes,
                               void* stream) {
  hga::Geometry g;
  hga_status st = make_geometry(cfg, dtype, batch, kv_cap, q_pos0, n_q, g);
  if (st != HGA_OK) return st;
  if (n_q == 0) return HGA_OK;
  if (q_raw == nullptr || k_rot == nullptr || v == nullptr || granules == nullptr ||
      granule_count == nullptr || out == nullptr || lse == nullptr || d_out == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return HGA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_raw) || !aligned16(k_rot) || !aligned16(v) || !aligned16(out) ||
      !aligned16(d_out) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return HGA_ERR_INVALID_ARGUMENT;
  if (!hga::backward_supported(g) || !hga::attend_supported(g)) return HGA_ERR_UNSUPPORTED;
  const size_t need = hga::backward_workspace(g);
  if (workspace == nullptr || workspace_bytes < need) return HGA_ERR_WORKSPACE_TOO_SMALL;
  hipError_t e = hga::launch_backward(g, q_raw, k_rot, v, granules, granule_count, out, lse, d_out, dq,
                                      dk, dv, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HGA_OK : hip_fail(e);
}

}  // extern "C"
