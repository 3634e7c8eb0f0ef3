// Internal interface between the C ABI layer (api.cpp) and the kernel
// translation units.  Not installed; the public interface is include/hga.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hga.h"

namespace hga {

constexpr int kMaxHalfDim = 64;  // d <= 128

// RoPE frequencies theta_i = rope_theta^(-2i/d) for i < d/2 <= 64, kept as
// the six factors step[b] = rope_theta^(-2^(b+1)/d) (host, double): a lane
// forms theta_i as the product of the factors of the set bits of i, with no
// memory access.  period: positions wrap modulo it before rotation (0 = no).
struct RopeFreqs {
  double step[6];
  int64_t period;
};

// A validated call shape.  Built by api.cpp, read by the launchers.
struct Geometry {
  int B, Hq, Hkv, G, d, C, gs, r;  // r = C / gs granules per chunk
  int F, L, Kc, Kg, n_hf;
  int64_t kv_cap, q_pos0, n_q;
  int64_t t0, nqc;  // first query chunk, number of query chunks
  int gmax;         // granules per unit at most
  float scale;      // softmax scale
  bool bf16;
  RopeFreqs rope;
};

// Validates a config and call shape and fills the geometry (api.cpp).
hga_status make_geometry(const hga_config* cfg, hga_dtype dtype, int32_t batch, int64_t kv_cap,
                         int64_t q_pos0, int64_t n_q, Geometry& g);
// Records a failed HIP call as this thread's last error; returns HGA_ERR_HIP.
hga_status hip_fail(hipError_t e);
// The current HIP device, and its compute units (cached per device).
int current_device();
int64_t device_cus();

// k_raw / k_rot hold tokens [k_first, k_first + k_rows) per (sequence, KV
// head) (k_rows <= 0: the whole cache); every token the call reads or writes
// must lie in that range.
hipError_t launch_summarize(const Geometry& g, const void* k_raw, int64_t tok_begin,
                            int64_t tok_end, void* k_rot, float* chunk_sum,
                            float* group_sum, hipStream_t stream, int64_t k_first = 0,
                            int64_t k_rows = 0);

size_t route_workspace(const Geometry& g);
bool route_supported(const Geometry& g);
hipError_t launch_route(const Geometry& g, const void* q, const float* chunk_sum,
                        const float* group_sum, int32_t* chunk_idx, int32_t* group_idx,
                        int32_t* granules, int32_t* granule_count, void* ws,
                        hipStream_t stream);

// Options of the host tier: K/V read from a granule-major staging pool
// ([slot][2][g_s][d], K then V) through per-entry pool slots, and no key
// splitting (so no workspace).
struct AttendExtra {
  const int32_t* pool_slot = nullptr;
  int64_t pool_slots = 0;
  bool allow_split = true;
  int64_t q_stride = -1;  // rows per (sequence, head) of q/out/lse; -1 = n_q
  int64_t q_row0 = -1;    // position of row 0; -1 = q_pos0
};

// Granules one bf16 attention work item can read (an LDS table); longer
// lists are split over several work items, which the host tier (no
// splitting) cannot do, so it requires G_max <= kAttendTable.
constexpr int kAttendTable = 2048;

bool attend_supported(const Geometry& g);
// Bytes of the static device scratch of hga_attend_noalloc, and its address
// on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
hipError_t attend_noalloc_scratch(void** ptr);
size_t attend_workspace(const Geometry& g, bool dense, bool allow_split = true);
hipError_t launch_attend(const Geometry& g, const void* q, const void* k_rot, const void* v,
                         const int32_t* granules, const int32_t* granule_count, bool dense,
                         void* out, float* lse, void* ws, hipStream_t stream,
                         const AttendExtra* extra = nullptr);

// One decode step (n_q = 1 at position q_pos0) in two launches (decode.hip).
bool decode_step_supported(const Geometry& g);
size_t decode_step_workspace(const Geometry& g);
hipError_t launch_decode_step(const Geometry& g, const void* q, const void* k_rot, const void* v,
                              const float* chunk_sum, const float* group_sum, int32_t* chunk_idx,
                              int32_t* group_idx, int32_t* granules, int32_t* granule_count, void* out,
                              float* lse, void* ws, hipStream_t stream);

// Backward of routed exact-token attention (bf16): dq (raw queries), dk (raw
// keys) and dv, all f32; dk and dv are overwritten.  Workspace: one f32 per
// query row.
bool backward_supported(const Geometry& g);
size_t backward_workspace(const Geometry& g);
hipError_t launch_backward(const Geometry& g, const void* q, const void* k_rot, const void* v,
                           const int32_t* granules, const int32_t* granule_count, const void* out,
                           const float* lse, const void* d_out, float* dq, float* dk, float* dv,
                           void* ws, hipStream_t stream);

}  // namespace hga
