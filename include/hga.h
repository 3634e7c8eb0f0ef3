/*
 * hga.h -- C ABI of the MI355X (gfx950) routed exact-token attention library
 * (Hierarchical Global Attention, arXiv:2606.30709).
 *
 * The pages that define the method (the xllm-io paper-review page, section 3
 * "technical architecture") describe a key/value store with four operations:
 * append a closed chunk, read the chunk summaries for routing, fetch the group
 * summaries for the second routing level, and gather the exact token K/V of
 * the selected chunks or groups; routing is kept apart from storage.  The
 * entry points below map onto them:
 *
 *   append               -> hga_build_summaries
 *   read + fetch (route) -> hga_route
 *   gather + attend      -> hga_attend, hga_attend_host_tiered
 *   one decode step      -> hga_decode_step (route + gather + attend, two launches)
 *   Eq. (1) reference    -> hga_dense_causal
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Positions are absolute token indices starting at 0.  Chunk m covers tokens
 * [m*C, (m+1)*C); group (granule) g covers tokens [g*g_s, (g+1)*g_s).  Query
 * chunk t covers query positions [t*C, (t+1)*C).
 *
 * Layouts (row-major, innermost last):
 *   k_raw, k_rot, v : [B][Hkv][kv_cap][d]   element dtype (f32 or bf16);
 *                     slot j holds the token at position j.
 *   q_raw, out      : [B][Hq][n_q][d]       query qi sits at q_pos0 + qi.
 *   lse             : [B][Hq][n_q]          f32, natural-log sum-exp.
 *   chunk_sum       : [B][Hkv][kv_cap/C][d]   f32
 *   group_sum       : [B][Hkv][kv_cap/g_s][d] f32
 *   NQC (query chunks of a call) = (q_pos0+n_q-1)/C - q_pos0/C + 1; unit
 *   (b, kvh, t) is stored at index [b][kvh][t - q_pos0/C].
 *   chunk_idx       : [B][Hkv][NQC][K_c]    int32 ascending, -1 padded
 *   group_idx       : [B][Hkv][NQC][K_g]    int32 ascending, -1 padded
 *   granules        : [B][Hkv][NQC][G_max]  int32 ascending unique, -1 padded
 *   granule_count   : [B][Hkv][NQC]         int32
 *
 * RoPE: theta_i = rope_theta^(-2i/d) for pair i < d/2; pair i is the
 * elements (i, i + d/2) (half-split layout); R_p turns a pair by p*theta_i.
 * Angles are formed in double precision and reduced before an f32 sincos.
 * With rope_period = P > 0 (the wrapped-position variant of the xllm-io
 * page, Sec. 5.5, P = 65536 there) every rotation uses p mod P instead of p:
 * queries, keys and the middle positions of summaries.  P must be a multiple
 * of C, so no chunk or group straddles a wrap.  Causality, chunk indices and
 * routing keep absolute positions.
 *
 * Ownership: the caller owns every buffer and allocates it; the library never
 * allocates device memory.  Its global state is a per-thread last-HIP-error
 * code, device properties cached once per device, and the static device
 * scratch of hga_attend_noalloc (allocated with the code object, one copy
 * per device).  All device pointers must be 16-byte aligned device (or
 * managed) memory.
 *
 * Asynchrony: every entry point enqueues work on `stream` (a hipStream_t,
 * NULL = the default stream) and returns without synchronising, except
 * hga_attend_host_tiered which is documented as host-blocking.
 *
 * Errors: all arguments are validated on the host before anything is
 * enqueued; on an error nothing is enqueued and the outputs are untouched.
 * No C++ exception crosses the ABI.  HGA_ERR_HIP means a HIP launch or
 * runtime call failed; hga_last_hip_error() returns its hipError_t code.
 *
 * Thread safety: the entry points are re-entrant given distinct workspaces.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HGA_OK = 0,
  HGA_ERR_INVALID_ARGUMENT = 1,
  HGA_ERR_UNSUPPORTED = 2,
  HGA_ERR_WORKSPACE_TOO_SMALL = 3,
  HGA_ERR_HIP = 4
} hga_status;

/* q, k, v and out share one element type. */
typedef enum { HGA_F32 = 0, HGA_BF16 = 1 } hga_dtype;

typedef struct hga_config {
  int32_t chunk_size;      /* C: tokens per chunk (framework paragraph), <= 64    */
  int32_t group_size;      /* g_s: tokens per group; C % g_s == 0                 */
  int32_t n_sink_chunks;   /* F: first chunks always visible (routing policy)    */
  int32_t n_recent_chunks; /* L: last closed chunks always visible               */
  int32_t top_chunks;      /* K_c: routed middle chunks (selection equation)     */
  int32_t top_groups;      /* K_g: routed groups; 0 = routed chunks open whole   */
  int32_t n_hf_pairs;      /* RoPE pairs [0, n_hf) are high frequency (Mixed-RoPE) */
  int32_t head_dim;        /* d in {64, 128}                                      */
  int32_t n_q_heads;       /* Hq; Hq % Hkv == 0, query head h reads KV head h/(Hq/Hkv) */
  int32_t n_kv_heads;      /* Hkv                                                 */
  double rope_theta;       /* RoPE base, > 0                                      */
  float softmax_scale;     /* 0 => 1/sqrt(d) (Eq. 1)                              */
  int64_t rope_period;     /* 0, or P: RoPE sees positions mod P (Sec. 5.5); P % C == 0 */
} hga_config;

/*
 * hga_build_summaries -- "append closed chunk".
 *
 * Mixed-RoPE summary equation (xllm-io page, section 3): for a closed chunk
 * (or group) G with first token f and middle position p_mid = f + (|G|-1)/2,
 *   pairs i <  n_hf : (1/|G|) sum_{j in G} R_j k_j        (rotate, then mean)
 *   pairs i >= n_hf : R_{p_mid}((1/|G|) sum_{j in G} k_j)  (mean, then rotate)
 *
 * Rotates the raw keys of tokens [tok_begin, tok_end) into k_rot (when k_rot
 * is not NULL; stored in the input dtype, round-to-nearest-even for bf16) and
 * writes the summary of every chunk and group whose last token lies in
 * [tok_begin, tok_end).  Summaries read every token of their block from
 * k_raw, so k_raw must already hold the earlier tokens of a block that
 * completes in the range.  Used both for prefill (0, n) and for the decode
 * append of one token (p, p+1).
 *
 * group_sum may be NULL iff top_groups == 0.  Requires kv_cap % C == 0 and
 * 0 <= tok_begin < tok_end <= kv_cap.
 */
hga_status hga_build_summaries(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                               const void* k_raw, int64_t kv_cap,
                               int64_t tok_begin, int64_t tok_end,
                               void* k_rot, float* chunk_sum, float* group_sum,
                               void* stream);

/* Granules one unit can attend to at most:
 * (C/g_s)(1 + F + max(L,1)) + (K_g if K_g > 0 else K_c C/g_s).  -1 on a bad config. */
int32_t hga_max_granules(const hga_config* cfg);

/* Workspace bytes hga_route needs for this call shape (may be 0): the
 * segment winners of decode-shaped calls, or, for calls whose units have
 * more than 64 (query, head) rows, the summary rows the call can read split
 * into bf16 hi / lo halves (chunks up to the last query chunk and their
 * groups, 4 * d bytes per row) and the norms of those chunk rows (4 bytes
 * each). */
size_t hga_route_workspace_bytes(const hga_config* cfg, int32_t batch,
                                 int64_t q_pos0, int64_t n_q);

/*
 * hga_route -- "read chunk summaries" and "fetch group summaries".
 *
 * Routing policy and selection equation (xllm-io page, section 3).  For each
 * unit (sequence b, KV head kvh, query chunk t):
 *   Fixed(t)  = first min(F,t) chunks  U  last L closed chunks  U  {t-1}
 *   Middle(t) = closed chunks m < t not in Fixed(t)
 *   s[m]      = max over the unit's query rows (queries of chunk t inside
 *               [q_pos0, q_pos0+n_q) x the G query heads of kvh) of q~ . c_m
 *               (q~ = RoPE-rotated query, no 1/sqrt(d))
 *   M_sel     = first min(K_c, |Middle|) of Middle by (s descending, m ascending)
 *   G_sel     = when K_g > 0: the same over the C/g_s groups of each chunk in
 *               M_sel (global id m*C/g_s + g), scored against group_sum
 *   granules  = Fixed(t) granules U routed groups (or the granules of the
 *               chunks in M_sel when K_g == 0) U the granules of chunk t whose
 *               first token is <= the unit's last query (sorted, unique)
 * Scores are evaluated with split-bf16 matrix-core products (hi*hi + hi*lo +
 * lo*hi, f32 accumulation), about 1e-5 relative to an f64 evaluation; exact
 * ties go to the lowest index.  Units with more than 64 rows and 64 middle
 * chunks screen the chunks with hi*hi alone first and take the split
 * products only of the chunks that a proven bound on the difference leaves
 * in contention: the selection is the same as scoring every chunk.
 *
 * chunk_sum must hold every chunk < the last query chunk; group_sum every
 * group of those chunks (group_sum / group_idx may be NULL iff K_g == 0).
 * Requires kv_cap % C == 0 and q_pos0 + n_q <= kv_cap.  HGA_ERR_UNSUPPORTED
 * when K_c or K_g exceeds 256, a unit has more than 512 (query, head) rows
 * (C * G), more than 4096 middle chunks, or K_c * C/g_s exceeds 4096.
 */
hga_status hga_route(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                     const void* q_raw, int64_t q_pos0, int64_t n_q,
                     const float* chunk_sum, const float* group_sum, int64_t kv_cap,
                     int32_t* chunk_idx, int32_t* group_idx,
                     int32_t* granules, int32_t* granule_count,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes hga_attend / hga_dense_causal need for this call shape. */
size_t hga_attend_workspace_bytes(const hga_config* cfg, int32_t batch,
                                  int64_t q_pos0, int64_t n_q);

/*
 * hga_attend -- "gather exact token K/V" + exact-token softmax attention.
 *
 * Exact-token output paragraph and Eq. (1) (xllm-io page, section 3): the
 * query at position i with head h attends, with softmax over exactly these
 * tokens, to every token j of its unit's granule list with j < t*C or
 * j <= i (causal inside the current chunk):
 *   out[i,h] = sum_j softmax_j(scale * q~_{i,h} . k~_j) v_j
 * granules / granule_count are those written by hga_route (or any ascending
 * list of granules inside [0, kv_cap/g_s) with count <= G_max; lists must
 * not repeat a granule).  k_rot holds RoPE-rotated keys (hga_build_summaries).
 * Rows of k_rot and v at or after the call's last query (q_pos0 + n_q) are
 * never read into a result and may hold anything (a cache filled up to the
 * current token).  bf16 runs QK^T and PV on bf16 matrix cores (P rounded
 * to bf16) with f32 online softmax; f32 runs on f32 vector ALUs.  lse may
 * be NULL.  HGA_ERR_UNSUPPORTED when g_s is not a power of two, or (bf16)
 * when one (sequence, KV head) slab of k_rot or v reaches 2^31 bytes.
 */
hga_status hga_attend(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                      const void* q_raw, int64_t q_pos0, int64_t n_q,
                      const void* k_rot, const void* v, int64_t kv_cap,
                      const int32_t* granules, const int32_t* granule_count,
                      void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * hga_attend_noalloc -- hga_attend without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments (minus
 * the workspace), checks, kernels and outputs (bitwise) as hga_attend.
 * The scratch hga_attend would take from its workspace (the split-key
 * partials of calls with few units, e.g. decode) lives instead in a static
 * device array of hga_attend_noalloc_max_scratch_bytes() bytes (16 MiB) that
 * the library holds on each device it runs on until the process ends.  A
 * call that needs more (hga_attend_workspace_bytes above that) returns
 * HGA_ERR_WORKSPACE_TOO_SMALL and enqueues nothing.  The call allocates
 * nothing.  Every call on a device shares that device's array: calls that
 * overlap on one device (other streams, other threads) race and must be
 * serialised by the caller; nothing in the array needs clearing between
 * calls.
 */
hga_status hga_attend_noalloc(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                              const void* q_raw, int64_t q_pos0, int64_t n_q,
                              const void* k_rot, const void* v, int64_t kv_cap,
                              const int32_t* granules, const int32_t* granule_count,
                              void* out, float* lse, void* stream);

size_t hga_attend_noalloc_max_scratch_bytes(void);

/*
 * hga_decode_step -- one decode step (one new query per sequence at
 * position pos, n_q = 1) of hga_route + hga_attend in two launches.
 *
 * Routing policy, selection equation and exact-token output (xllm-io page,
 * section 3) for the query of every (sequence, KV head) unit: the same
 * selections, lists and attention as hga_route followed by hga_attend with
 * q_pos0 = pos, n_q = 1, except that chunk and group scores are evaluated
 * with f32 matrix-core products (about 1e-7 relative to an f64 evaluation;
 * ties still go to the lowest index) and the attention sums its keys in
 * another order (outputs agree to rounding, not bitwise).  The first launch
 * scans the middle chunks and, at the same time, attends the fixed windows
 * (sink and recent chunks, the current chunk up to pos), which routing does
 * not change; the second selects, writes the lists, attends the routed
 * tokens and merges.
 *   q_raw [B][Hq][1][d], out [B][Hq][1][d], lse [B][Hq][1] (may be NULL);
 *   k_rot, v, chunk_sum, group_sum as for hga_route / hga_attend (every chunk
 *   and group before pos's chunk summarised; rows after pos may hold
 *   anything);
 *   chunk_idx [B][Hkv][K_c], group_idx [B][Hkv][K_g], granules
 *   [B][Hkv][G_max], granule_count [B][Hkv]: the lists hga_route would write;
 *   pass NULL for all four to skip them (group_idx may be NULL iff K_g == 0).
 * workspace: device memory of hga_decode_step_workspace_bytes, 256-byte
 * aligned, no initial contents needed; calls sharing one workspace must not
 * overlap.
 * bf16 only; d in {64, 128}; at most 16 query heads per KV head; K_c, K_g
 * <= 256; at most 1024 routed granules per unit; g_s a power of two; the
 * fixed windows and current chunk in W = ceil(keys / 128) blocks with
 * W * R * (d + 2) <= 16384 floats (d = 128) or 8448 (d = 64), R the query
 * heads per KV head rounded up to 4, 8 or 16 (896 keys at 16 heads and
 * d = 128).  Other shapes return HGA_ERR_UNSUPPORTED (hga_route +
 * hga_attend cover them).
 */
size_t hga_decode_step_workspace_bytes(const hga_config* cfg, int32_t batch, int64_t pos);
hga_status hga_decode_step(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                           const void* q_raw, int64_t pos,
                           const void* k_rot, const void* v, int64_t kv_cap,
                           const float* chunk_sum, const float* group_sum,
                           int32_t* chunk_idx, int32_t* group_idx,
                           int32_t* granules, int32_t* granule_count,
                           void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * hga_dense_causal -- Eq. (1): every query i attends to all keys j <= i.
 * The reference the routed path reduces to when the budgets cover every
 * middle chunk.  Same layouts and numerics as hga_attend.
 */
hga_status hga_dense_causal(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                            const void* q_raw, int64_t q_pos0, int64_t n_q,
                            const void* k_rot, const void* v, int64_t kv_cap,
                            void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Host tier -- tiered K/V store of the xllm-io page, section 3: summaries
 * and routing stay on the device; the full token K/V history lives in host
 * RAM and only the routed working set is moved to the device.
 *
 * kv_host (pinned host memory, e.g. hipHostMalloc) holds the RoPE-rotated
 * keys and the values granule-major: [B][Hkv][kv_cap/g_s][2][g_s][d] in the
 * call dtype, K block then V block of each granule (g_s * d elements each).
 *
 * hga_attend_host_tiered computes the same outputs as hga_route followed by
 * hga_attend on device-resident K/V, for queries [q_pos0, q_pos0 + n_q):
 * the same granules in the same order, and bitwise the same values whenever
 * hga_attend plans one work item per unit row slice with units of more than
 * 16 rows; for few-unit calls hga_attend instead splits each unit's keys
 * over workgroups or takes its decode kernel (units of at most 16 rows),
 * which sum in another order and agree to rounding.  The outputs do not
 * depend on max_window_chunks, slots_per_window or cache_slots (bitwise).
 *   1. routes every unit on compute_stream (chunk_sum / group_sum in HBM);
 *   2. copies the granule lists to the host (the call blocks for this);
 *   3. walks windows of at most max_window_chunks query chunks whose union
 *      of needed granules (one copy per granule per (sequence, KV head))
 *      fits slots_per_window; n_threads host threads pack each union from
 *      kv_host into pinned staging, one hipMemcpyAsync per window moves it
 *      on copy_stream, and an event gates the window's attention on
 *      compute_stream;
 *   4. two window buffers alternate, so window w+1 is packed and copied
 *      while window w is attended.
 * It returns once the last attention is enqueued on compute_stream.
 *
 * Warm tier (the tiered store's VRAM cache, xllm-io page, section 3):
 * with cache_slots > 0 the device keeps up to cache_slots granules across
 * the windows of the call, evicting the least recently used; a window then
 * holds at most cache_slots distinct granules and copies only its misses
 * (at most slots_per_window), which a device gather moves into their cache
 * slots before the window's attention.  Outputs are unchanged (bitwise);
 * stats->granules_hit counts the reuses.  cache_slots = 0: no warm tier;
 * otherwise cache_slots >= B * Hkv * hga_max_granules(cfg).
 *
 * dev_staging (device) and host_staging (pinned host) are caller-owned,
 * 256-byte aligned, at least the sizes hga_host_tiered_buffer_bytes returns;
 * slots_per_window >= B * Hkv * hga_max_granules(cfg).  Both streams must
 * be distinct from work that uses the staging buffers concurrently.
 * Returns HGA_ERR_INVALID_ARGUMENT when kv_host or host_staging is not
 * pinned host memory.  stats may be NULL.
 */
typedef struct hga_tier_stats {
  int64_t windows;          /* attention launches (windows)                       */
  int64_t granules_copied;  /* granules moved host -> device (K and V together)    */
  int64_t bytes_h2d;        /* bytes of all host -> device copies of the call      */
  double pack_seconds;      /* host time spent packing granules into staging       */
  double host_seconds;      /* host time of the whole call                         */
  int64_t granules_hit;     /* granules a window found in the warm tier (cache)    */
} hga_tier_stats;

hga_status hga_host_tiered_buffer_bytes(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                        int64_t q_pos0, int64_t n_q, int32_t max_window_chunks,
                                        int64_t slots_per_window, int64_t cache_slots,
                                        size_t* device_bytes, size_t* host_bytes);

/*
 * Warm-tier size under a VRAM headroom (the tiered store of the xllm-io
 * page, section 3: the warm tier is bounded so that a configurable amount of
 * device memory stays free).  The library allocates nothing, so the policy
 * is a sizing call: *cache_slots receives the largest cache_slots whose
 * dev_staging (hga_host_tiered_buffer_bytes with these arguments) leaves at
 * least headroom_bytes of the current device's free memory (hipMemGetInfo,
 * read now) unused, at most one slot per granule of the call's context, or 0
 * when even the smallest warm tier (B * Hkv * hga_max_granules(cfg) slots)
 * does not fit: the call then runs on the cold tier alone.  Recomputing it
 * before a call shrinks or grows the tier with the memory other work holds.
 * HGA_ERR_HIP when the device cannot be queried.
 */
hga_status hga_host_tiered_cache_slots(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                       int64_t q_pos0, int64_t n_q, int32_t max_window_chunks,
                                       int64_t slots_per_window, size_t headroom_bytes,
                                       int64_t* cache_slots);

hga_status hga_attend_host_tiered(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                  const void* q_raw, int64_t q_pos0, int64_t n_q,
                                  const void* kv_host, int64_t kv_cap,
                                  const float* chunk_sum, const float* group_sum,
                                  void* out, float* lse,
                                  void* dev_staging, size_t dev_bytes,
                                  void* host_staging, size_t host_bytes,
                                  int32_t max_window_chunks, int64_t slots_per_window,
                                  int64_t cache_slots, int32_t n_threads,
                                  void* compute_stream, void* copy_stream,
                                  hga_tier_stats* stats);

/*
 * hga_attend_backward -- gradients of exact-token attention (the training
 * path; xllm-io page, section 3, exact-token output, Eq. 1 restricted to the
 * visible tokens) with the routes of a forward hga_route held fixed: no
 * gradient flows through summaries or selection.
 *   q_raw, out, d_out : [B][Hq][n_q][d] (dtype; out and lse from hga_attend
 *                       on the same inputs, d_out = dL/d out)
 *   k_rot, v          : [B][Hkv][kv_cap][d] (dtype)
 *   granules, granule_count : the forward's lists
 *   dq                : [B][Hq][n_q][d] f32, dL/d q_raw (through R^T)
 *   dk, dv            : [B][Hkv][kv_cap][d] f32, dL/d k_raw (through R^T) and
 *                       dL/d v; overwritten (zero where no query looks)
 * With P = exp(s q~.k~ - lse): dP = dO.v, D = dO.O, dS = P (dP - D),
 * dq~ = s dS k~, dk~ = s dS^T q~, dv = P^T dO.  bf16 only; granules of at
 * least 4 tokens.  dq is bitwise repeatable; dk and dv sum per-(unit, key)
 * partials in an order that can change between calls (f32 rounding only).
 * As in hga_attend, rows of k_rot and v from q_pos0 + n_q on may hold
 * anything; dk and dv are zero there.  Workspace:
 * hga_attend_backward_workspace_bytes (it depends on q_pos0 + n_q, not on
 * kv_cap) -- per query row D (f32) and Q' (bf16); granule lists; and two
 * f32 partial rows of d per (unit, list key),
 * units * gmax * g_s * d * 8 bytes, the largest piece (2.5 GB for 32768
 * queries, 32 query and 4 KV heads, d = 128, 76 granules per list).  Errors: HGA_ERR_UNSUPPORTED for
 * other dtypes or shapes, HGA_ERR_WORKSPACE when workspace_bytes is short;
 * nothing is launched then.
 */
size_t hga_attend_backward_workspace_bytes(const hga_config* cfg, int32_t batch, int64_t q_pos0,
                                           int64_t n_q);

hga_status hga_attend_backward(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                               const void* q_raw, int64_t q_pos0, int64_t n_q,
                               const void* k_rot, const void* v, int64_t kv_cap,
                               const int32_t* granules, const int32_t* granule_count,
                               const void* out, const float* lse, const void* d_out,
                               float* dq, float* dk, float* dv,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Streaming decode from the host tier (xllm-io page, section 3, tiered K/V
 * store, RAM-cached decode): the token K/V history stays in the pinned
 * granule-major host store (layout of hga_attend_host_tiered), summaries and
 * routing on the device, and a device cache of cache_slots granules keeps
 * what earlier steps brought over.  Its directory lives on the device: a
 * granule without a slot takes the next slot, in ring order from a
 * replacement hand, that the step does not use (so the always-visible
 * windows, used every step, stay cached; the oldest-filled routed granules
 * go first).
 *
 * A session (host object) owns the cache bookkeeping; the caller owns and
 * allocates every buffer: kv_host (pinned, hipHostMalloc, mapped into the
 * device's address space: the device reads missing granules from it
 * directly over the host link), dev_buffer
 * (device, 256-byte aligned, hga_decode_session_buffer_bytes), host_buffer
 * (pinned, 256-byte aligned) and the summary tables chunk_sum / group_sum of
 * hga_build_summaries.  bf16 only, at most 16 query heads per KV head,
 * cache_slots >= batch * n_kv_heads * hga_max_granules(cfg).
 *
 * hga_decode_session_create: the store holds tokens [0, first_pos) and the
 *   summary tables every chunk below first_pos; first_pos % C == 0.
 * hga_decode_session_append: token pos (pos = the previous append + 1, the
 *   first one first_pos) of every sequence: k_raw_new / v_new
 *   [B][Hkv][1][d] device rows (raw key, value).  Rotates the key on the
 *   device, writes the chunk and group summaries the token closes, and
 *   copies the rotated key and the value into the host store (asynchronous on
 *   compute_stream).  Unwritten store rows must hold finite values.
 * hga_decode_session_step: one query per sequence at position pos (<= the
 *   last appended position): q_raw [B][Hq][1][d], out [B][Hq][1][d], lse
 *   [B][Hq][1] (may be NULL).  Same outputs as hga_route + hga_attend with
 *   q_pos0 = pos, n_q = 1 over the device-resident cache.  Asynchronous:
 *   it enqueues on compute_stream the route, the cache lookup (one
 *   workgroup), the gather of the misses from the store and the attention,
 *   and returns without waiting.  A granule cached while it held fewer
 *   tokens than the step needs is fetched again.  stats (may be NULL; then
 *   the call waits for the step to finish): granules fetched
 *   (granules_copied) / found (granules_hit), bytes over the host link,
 *   pack_seconds = 0 (no host lookup), host_seconds = whole call.
 *   The device buffer holds the cache and its directory between calls:
 *   leave it untouched while the session lives.
 * Calls on one session must not overlap.
 */
typedef struct hga_decode_session hga_decode_session;

/* The same sizing for a decode session's cache: the largest cache_slots
 * whose dev_buffer (hga_decode_session_buffer_bytes) leaves headroom_bytes
 * of the device's free memory unused, at most one slot per granule of
 * kv_cap; HGA_ERR_WORKSPACE_TOO_SMALL when one step's granules do not fit. */
hga_status hga_decode_session_cache_slots(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                          int64_t kv_cap, size_t headroom_bytes, int64_t* cache_slots);

hga_status hga_decode_session_buffer_bytes(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                           int64_t kv_cap, int64_t cache_slots,
                                           size_t* device_bytes, size_t* host_bytes);

hga_status hga_decode_session_create(const hga_config* cfg, hga_dtype dtype, int32_t batch,
                                     int64_t kv_cap, int64_t first_pos, int64_t cache_slots,
                                     void* kv_host, void* dev_buffer, size_t dev_bytes,
                                     void* host_buffer, size_t host_bytes,
                                     hga_decode_session** session);

void hga_decode_session_destroy(hga_decode_session* session);

hga_status hga_decode_session_append(hga_decode_session* session, const void* k_raw_new,
                                     const void* v_new, int64_t pos, float* chunk_sum,
                                     float* group_sum, void* compute_stream);

hga_status hga_decode_session_step(hga_decode_session* session, const void* q_raw, int64_t pos,
                                   const float* chunk_sum, const float* group_sum, void* out,
                                   float* lse, void* compute_stream, hga_tier_stats* stats);

const char* hga_status_string(hga_status status);

/* hipError_t of the last failed HIP call made by this thread (0 if none). */
int hga_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */
