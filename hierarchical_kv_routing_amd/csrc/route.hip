// Two-level content routing: chunk scores, top-K_c, group scores inside the
// selected chunks, top-K_g, and the visible-granule list of every unit.
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3: routing policy (fixed sink / recent / previous-chunk windows,
// middle context competes), score_m = q^T c_m, the selection equation
// M_sel = topK_c, G_sel = topK_g over the groups of M_sel, and the exact-token
// output paragraph (which tokens are opened).  Scores of a unit are the max
// over its query rows (query chunk x GQA group of the KV head).
//
// Scoring is a small dense contraction (rows x d) . (d x candidates) done on
// bf16 matrix cores with both operands split hi + lo (hi*hi + hi*lo + lo*hi,
// f32 accumulation), about 1e-5 relative to f64, so routing decisions agree
// with an f64 evaluation except at near-ties.  Selection is an exact block
// radix select on order-preserving 32-bit keys; equal keys go to the lowest
// index.
//
// Two launch shapes:
//  * fused: one workgroup per unit (sequence, KV head, query chunk) scores
//    every middle chunk, selects, scores the groups and writes the lists.
//    Units run longest (largest t) first.
//  * segmented (few units with long middle contexts, e.g. a decode step):
//    score_kernel spreads each unit's middle chunks over many workgroups;
//    each scores its segment, keeps the segment's own top-K_c (same order:
//    score, then lower index) and scores those chunks' groups, and writes
//    all of it to the workspace.  merge_kernel then selects the unit's
//    top-K_c among the segments' winners (every chunk of the unit's top-K_c
//    is in its segment's top-K_c, so the result is the same set), the top-K_g
//    among their groups, and writes the lists.
#include "hga_device.h"
#include "hga_select.h"

namespace hga {
namespace {

constexpr int kRouteThreads = 512;      // 8 waves
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kScoreThreads = 256;      // segmented scoring: 4 waves
constexpr int kRowsPerWave = 64;        // 4 row blocks of 16
constexpr int kMaxRows = kRowsPerWave * kRouteWaves;
constexpr int kMaxCand = 4096;          // middle chunks per unit held in LDS
constexpr int kMaxSel = 256;            // K_c, K_g upper bound
constexpr int kMaxTableQ = 64;          // queries per unit (C <= 64)
constexpr int kScreenMin = 64;          // middle chunks above which chunk scoring is screened

// Screening bound.  With x = hi + lo + e (hi = bf16(x), lo = bf16(x - hi),
// u = 2^-8: |hi| <= (1+u)|x|, |lo| <= u(1+u)|x|), the split score
// hi.hi + hi.lo + lo.hi of a query row q and a chunk summary c differs from
// hi.hi alone by at most 2u(1+u)^2 sum_d |q_d c_d| <= 2u(1+u)^2 |q| |c|
// (Cauchy-Schwarz), plus the f32 accumulation of both (at most 384 terms,
// 2^-24 each, of a sum of magnitudes <= (1+u)^2 |q| |c|): in all below
// 1.014 * 2^-7 |q| |c|.  The max over a unit's rows moves by at most the
// same with |q| -> Q, the largest row norm.  kScreenEps adds headroom for
// the f32 rounding of the norms and of s -/+ E; kScreenAbs keeps E > 0.
constexpr float kScreenEps = 1.03f / 128.f;
constexpr float kScreenAbs = 1e-30f;

struct RouteParams {
  const void* q;
  const float* csum;
  const float* gsum;
  int32_t* cidx;
  int32_t* gidx;
  int32_t* gran;
  int32_t* gcnt;
  // segmented: per unit, nseg*Kc segment winners' keys, their middle chunk
  // offsets, and (group routing) nseg*Kc*r group keys, all 32-bit words
  uint32_t* ws;
  int64_t ws_stride;
  // unsegmented calls with several row groups per unit: the summary tables
  // split into bf16 hi / lo rows (split_kernel), [slab][row][hi d, lo d]
  const uint16_t* csplit;
  const uint16_t* gsplit;
  const float* cnorm;                // |c_m| of every split chunk row, [slab][row]
  int64_t csplit_rows, gsplit_rows;  // rows per (sequence, KV head) table
  int64_t q_pos0, n_q, t0, nqc, nchunk_cap, ngroup_cap;
  int B, Hq, Hkv, G, d, C, gs, r, F, L, Kc, Kg, gmax;
  int seg_chunks, nseg;
  RopeFreqs rope;
};

struct Unit {
  int b, kvh;
  int64_t t, qlo, mid_lo, mid_hi, sink_hi, rec_lo, slot;
  int nq, R;
};

// Unit u in [0, B*Hkv*nqc): largest query chunk first; (b, kvh) fastest so
// that units sharing a summary table stay on the same XCD's L2.
__device__ __forceinline__ Unit make_unit(const RouteParams& p, int64_t u) {
  Unit w;
  // units < 2^31 (checked on the host): 32-bit division
  const uint32_t bh = static_cast<uint32_t>(p.B) * static_cast<uint32_t>(p.Hkv);
  const uint32_t u32 = static_cast<uint32_t>(u);
  const uint32_t q = u32 / bh;
  const uint32_t rem = u32 - q * bh;
  const int64_t trel = p.nqc - 1 - static_cast<int64_t>(q);
  const uint32_t bq = rem / static_cast<uint32_t>(p.Hkv);
  w.b = static_cast<int>(bq);
  w.kvh = static_cast<int>(rem - bq * static_cast<uint32_t>(p.Hkv));
  w.t = p.t0 + trel;
  const int64_t c0 = w.t * p.C;
  w.qlo = c0 > p.q_pos0 ? c0 : p.q_pos0;
  const int64_t qend = p.q_pos0 + p.n_q;
  const int64_t qhi = (c0 + p.C) < qend ? (c0 + p.C) : qend;
  w.nq = static_cast<int>(qhi - w.qlo);
  w.R = w.nq * p.G;
  const int64_t lp = p.L > 1 ? p.L : 1;
  w.sink_hi = w.t < p.F ? w.t : p.F;
  const int64_t rl = w.t - lp;
  w.rec_lo = rl > w.sink_hi ? rl : w.sink_hi;
  w.mid_lo = w.sink_hi;
  w.mid_hi = w.rec_lo;
  w.slot = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.nqc + trel;
  return w;
}

// cos/sin of every (query of the unit, pair) into LDS (block-wide; scratch:
// 16 * d/2 float2, free for the call).
template <int KS>
__device__ __forceinline__ void fill_rope_table(const RouteParams& p, const Unit& w, float2* cs,
                                                float2* scratch) {
  // a unit's queries share one chunk, so one wrap of its first position;
  // d/2 = 16 KS is a constant here, so the table's index arithmetic is shifts
  rope_table(p.rope, rope_base(p.rope, w.qlo), w.nq, 16 * KS, cs, scratch);
}

// The wave's NB row blocks of 16 rotated query rows as split-bf16 A operands
// (16x16x32 layout: lane -> row lane%16, d slots ks*32 + 8*(lane/16) + i).
// Rows past the unit's last row repeat the last row, which leaves every max
// unchanged.  Row r of a unit is (query r / G, head r % G).
__device__ __forceinline__ int row_of_lane(const Unit& w, int rbase, int blk) {
  const int r = rbase + blk * 16 + (threadIdx.x & 15);
  return r < w.R ? r : w.R - 1;
}

// Raw query elements of one row block (issued early, rotated later).
template <bool BF16, int KS>
__device__ __forceinline__ void load_row_raw(const RouteParams& p, const Unit& w, int r,
                                             float (&x)[KS][8]) {
  const int sub = (threadIdx.x & 63) >> 4;
  const int qi = r / p.G;
  const int hl = r - qi * p.G;
  const int64_t base =
      ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.n_q + (w.qlo + qi - p.q_pos0)) * p.d;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) load8<BF16>(p.q, base + ks * 32 + sub * 8, x[ks]);
}

// Rotates one row block's raw elements with the unit's RoPE table and splits
// them into the bf16 hi / lo A operands; ss receives the sum of squares of
// the lane's rotated elements (a quarter of its row).
template <int KS>
__device__ __forceinline__ void rotate_split(const RouteParams& p, int r, const float2* cs,
                                             float (&x)[KS][8], Pack8 (&ahi)[KS], Pack8 (&alo)[KS],
                                             float& ss) {
  const int sub = (threadIdx.x & 63) >> 4;
  const int h = p.d >> 1;
  const int qi = r / p.G;
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 t = cs[qi * h + ks * 32 + sub * 8 + i];
      const float a = x[ks][i], b = x[ks + KS / 2][i];
      x[ks][i] = a * t.x - b * t.y;
      x[ks + KS / 2][i] = a * t.y + b * t.x;
    }
  }
  ss = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      split_bf16x2(x[ks][2 * i], x[ks][2 * i + 1], ahi[ks].u[i], alo[ks].u[i]);
      ss += x[ks][2 * i] * x[ks][2 * i] + x[ks][2 * i + 1] * x[ks][2 * i + 1];
    }
  }
}

// bf16 queries: the raw 16-byte slices of the wave's NB row blocks, issued
// together (before the RoPE table is built) and held as packed bf16.
template <int KS, int NB>
__device__ __forceinline__ void issue_rows16(const RouteParams& p, const Unit& w, int rbase,
                                             uint4 (&raw)[NB][KS]) {
  const int sub = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int r = row_of_lane(w, rbase, blk);
    const int qi = r / p.G;
    const int hl = r - qi * p.G;
    const int64_t base =
        ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.n_q + (w.qlo + qi - p.q_pos0)) * p.d;
    const uint16_t* src = static_cast<const uint16_t*>(p.q) + base + sub * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[blk][ks] = *reinterpret_cast<const uint4*>(src + ks * 32);
  }
}

// Rotates and splits the rows issue_rows16 loaded; returns the largest
// squared norm of the wave's rotated rows (the same value in every lane).
template <int KS, int NB>
__device__ __forceinline__ float rotate_rows16(const RouteParams& p, const Unit& w, int rbase,
                                               const float2* cs, const uint4 (&raw)[NB][KS],
                                               Pack8 (&ahi)[NB][KS], Pack8 (&alo)[NB][KS]) {
  float n2 = 0.f;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    float x[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t u[4] = {raw[blk][ks].x, raw[blk][ks].y, raw[blk][ks].z, raw[blk][ks].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[ks][2 * i] = __uint_as_float(u[i] << 16);
        x[ks][2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    }
    float ss;
    rotate_split<KS>(p, row_of_lane(w, rbase, blk), cs, x, ahi[blk], alo[blk], ss);
    ss += __shfl_xor(ss, 16);  // the four lanes of a row
    ss += __shfl_xor(ss, 32);
    n2 = fmaxf(n2, ss);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) n2 = fmaxf(n2, __shfl_xor(n2, m));
  return n2;
}

// The wave's rows as split operands; returns the largest squared norm of
// the wave's rotated rows (the same value in every lane).
template <bool BF16, int KS, int NB>
__device__ __forceinline__ float load_rows(const RouteParams& p, const Unit& w, int rbase,
                                           const float2* cs, Pack8 (&ahi)[NB][KS],
                                           Pack8 (&alo)[NB][KS]) {
  float n2 = 0.f;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    const int r = row_of_lane(w, rbase, blk);
    float x[KS][8];
    load_row_raw<BF16, KS>(p, w, r, x);
    float ss;
    rotate_split<KS>(p, r, cs, x, ahi[blk], alo[blk], ss);
    ss += __shfl_xor(ss, 16);  // the four lanes of a row
    ss += __shfl_xor(ss, 32);
    n2 = fmaxf(n2, ss);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) n2 = fmaxf(n2, __shfl_xor(n2, m));
  return n2;
}

// Summary rows staged in LDS, split into bf16 hi and lo halves, so that the
// waves of a block that score the same rows for different query rows share
// one load.  The split is made once per call into the workspace (split_kernel:
// row = d hi values then d lo values), so a stage is a plain copy: direct
// global -> LDS loads (a wave's lane l lands at 16*l of the wave's 1 KB
// block) into unpadded rows of 2*d bytes with XOR-swizzled 16-byte chunks
// (rswz), two stages in separate buffers so that the next stage's loads
// overlap the current stage's products.
constexpr int kStageRows = 64;

// Score tiles of one staged 64-row block: tile `tile` (16 rows), the max
// over the wave's row blocks of q . row: the split products hi.hi + hi.lo +
// lo.hi (FULL), or hi.hi alone (the screening pass, no lo rows staged).
// Returns the lane's part of the max: candidate lane%16 over the rows
// 4*(lane/16) + j of each row block (the caller combines the four lanes of
// a candidate with an LDS atomic max).
template <int KS, int NB, bool FULL>
__device__ __forceinline__ float score16_staged(const char* shi, const char* slo, int tile,
                                                const Pack8 (&ahi)[NB][KS],
                                                const Pack8 (&alo)[NB][KS]) {
  constexpr int D = 32 * KS;
  const int lane = threadIdx.x & 63;
  const int row = tile * 16 + (lane & 15), sub = lane >> 4;
  Pack8 bhi[KS], blo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int off = row * (2 * D) + 16 * ((4 * ks + sub) ^ rswz<D>(row));
    bhi[ks].q = *reinterpret_cast<const uint4*>(shi + off);
    if constexpr (FULL) blo[ks].q = *reinterpret_cast<const uint4*>(slo + off);
  }
  float best = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mfma16x16x32(ahi[blk][ks].v, bhi[ks].v, acc);
      if constexpr (FULL) {
        acc = mfma16x16x32(ahi[blk][ks].v, blo[ks].v, acc);
        acc = mfma16x16x32(alo[blk][ks].v, bhi[ks].v, acc);
      }
    }
    best = fmaxf(best, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
  }
  return best;
}

// hi.hi scores of two staged tiles (t0, t1) at once: both tiles' operands
// are read before the products, so the LDS reads of the second overlap the
// products of the first.  Lane parts of the max, as score16_staged.
template <int KS, int NB>
__device__ __forceinline__ void score16x2_hh(const char* shi, int t0, int t1, const Pack8 (&ahi)[NB][KS],
                                             float& v0, float& v1) {
  constexpr int D = 32 * KS;
  const int lane = threadIdx.x & 63;
  const int sub = lane >> 4;
  Pack8 b0[KS], b1[KS];
  const int r0 = t0 * 16 + (lane & 15), r1 = t1 * 16 + (lane & 15);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    b0[ks].q = *reinterpret_cast<const uint4*>(shi + r0 * (2 * D) + 16 * ((4 * ks + sub) ^ rswz<D>(r0)));
    b1[ks].q = *reinterpret_cast<const uint4*>(shi + r1 * (2 * D) + 16 * ((4 * ks + sub) ^ rswz<D>(r1)));
  }
  v0 = -INFINITY;
  v1 = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      a0 = mfma16x16x32(ahi[blk][ks].v, b0[ks].v, a0);
      a1 = mfma16x16x32(ahi[blk][ks].v, b1[ks].v, a1);
    }
    v0 = fmaxf(v0, fmaxf(fmaxf(a0[0], a0[1]), fmaxf(a0[2], a0[3])));
    v1 = fmaxf(v1, fmaxf(fmaxf(a1[0], a1[1]), fmaxf(a1[2], a1[3])));
  }
}

// Max-scores of n candidates into keys[0..n) (atomic max: several row
// groups share the tiles); row(i) is the split row of candidate i.  Stages
// of 64 rows alternate between buffers (h0, l0) and (h1, l1); rows at or
// past n repeat row n-1.  FULL = false: hi.hi products only, and only the hi
// halves are staged.  Block-wide.
template <int KS, int NB, bool FULL, typename RowPtr>
__device__ __forceinline__ void score_staged(int n, RowPtr row, bool has_rows, int tg, int TG,
                                             const Pack8 (&ahi)[NB][KS],
                                             const Pack8 (&alo)[NB][KS], char* h0, char* l0,
                                             char* h1, char* l1, uint32_t* keys) {
  constexpr int D = 32 * KS;
  constexpr int ROW = 2 * D;
  constexpr int NBLK = kStageRows * ROW / 1024;  // 1 KB blocks per tile
  static_assert(NBLK % kRouteWaves == 0, "stage blocks spread evenly over the waves");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nst = (n + kStageRows - 1) / kStageRows;
  auto issue = [&](int s, char* hs, char* ls) {
    int ln = lane;
    asm volatile("" : "+v"(ln));  // addresses formed here, not hoisted into registers
#pragma unroll
    for (int j = 0; j < NBLK / kRouteWaves; ++j) {
      const int blk = (wave + j * kRouteWaves) * 1024;
      const int o = blk + 16 * ln;
      const int m = o / ROW;
      const int c = ((o % ROW) / 16) ^ rswz<D>(m);
      int i = s * kStageRows + m;
      i = i < n ? i : n - 1;
      const char* src = reinterpret_cast<const char*>(row(i)) + 16 * c;
      load_lds16(src, hs + blk);
      if constexpr (FULL) load_lds16(src + ROW, ls + blk);
    }
  };
  auto step = [&](int s, const char* hs, const char* ls, char* hn, char* ln_) {
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nst) issue(s + 1, hn, ln_);
    if (has_rows) {
      const int nb = n - s * kStageRows < kStageRows ? n - s * kStageRows : kStageRows;
      for (int tile = tg; tile * 16 < nb; tile += TG) {
        const float v = score16_staged<KS, NB, FULL>(hs, ls, tile, ahi, alo);
        const int c = s * kStageRows + tile * 16 + (lane & 15);
        if (c < n) atomicMax(&keys[c], order_key(v));
      }
    }
    wait_vm_barrier<0>();
  };
  if (nst > 0) issue(0, h0, l0);
  wait_vm_barrier<0>();
  for (int s = 0; s < nst; s += 2) {
    step(s, h0, l0, h1, l1);
    if (s + 1 >= nst) break;
    step(s + 1, h1, l1, h0, l0);
  }
}

// hi.hi max-scores of n candidates into keys[0..n) (atomic max), the
// screening pass: only the hi halves of the split rows are staged, through
// a ring of four 64-row buffers with three stages in flight (the loop is
// unrolled by four so that every stage names its buffers statically, and
// the LDS reads of one buffer need not wait for the loads into the others).
// Rows at or past n repeat row n-1.  Block-wide.
template <int KS, int NB, typename RowPtr>
__device__ __forceinline__ void screen_staged(int n, RowPtr row, bool has_rows, int tg, int TG,
                                              const Pack8 (&ahi)[NB][KS], const Pack8 (&alo)[NB][KS],
                                              char* b0, char* b1, char* b2, char* b3, uint32_t* keys) {
  constexpr int D = 32 * KS;
  constexpr int ROW = 2 * D;
  constexpr int NBLK = kStageRows * ROW / 1024;  // 1 KB blocks per stage
  constexpr int LPS = NBLK / kRouteWaves;        // loads per wave per stage
  static_assert(NBLK % kRouteWaves == 0, "stage blocks spread evenly over the waves");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nst = (n + kStageRows - 1) / kStageRows;
  auto issue = [&](int s, char* hs) {
    if (s >= nst) return;  // uniform
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < LPS; ++j) {
      const int blk = (wave + j * kRouteWaves) * 1024;
      const int o = blk + 16 * ln;
      const int m = o / ROW;
      const int c = ((o % ROW) / 16) ^ rswz<D>(m);
      int i = s * kStageRows + m;
      i = i < n ? i : n - 1;
      load_lds16(reinterpret_cast<const char*>(row(i)) + 16 * c, hs + blk);
    }
  };
  auto step = [&](int s, const char* hs, char* nxt) {
    // stage s landed (later stages may stay in flight), in every wave
    if (s + 2 < nst) wait_vm_barrier<2 * LPS>();
    else if (s + 1 < nst) wait_vm_barrier<LPS>();
    else wait_vm_barrier<0>();
    __builtin_amdgcn_sched_barrier(0);
    issue(s + 3, nxt);  // into the buffer stage s-1 used
    if (has_rows) {
      const int nb = n - s * kStageRows < kStageRows ? n - s * kStageRows : kStageRows;
      for (int tile = tg; tile * 16 < nb; tile += 2 * TG) {
        const int t1 = (tile + TG) * 16 < nb ? tile + TG : tile;  // a lone last tile is scored twice
        float v0, v1;
        score16x2_hh<KS, NB>(hs, tile, t1, ahi, v0, v1);
        const int c0 = s * kStageRows + tile * 16 + (lane & 15);
        const int c1 = s * kStageRows + t1 * 16 + (lane & 15);
        if (c0 < n) atomicMax(&keys[c0], order_key(v0));
        if (c1 < n) atomicMax(&keys[c1], order_key(v1));
      }
    }
  };
  issue(0, b0);
  issue(1, b1);
  issue(2, b2);
  for (int s = 0; s < nst; s += 4) {
    step(s, b0, b3);
    if (s + 1 >= nst) break;
    step(s + 1, b1, b0);
    if (s + 2 >= nst) break;
    step(s + 2, b2, b1);
    if (s + 3 >= nst) break;
    step(s + 3, b3, b2);
  }
  __syncthreads();  // every wave's reads of the ring are done
}

// Summary rows (f32) -> split rows (d bf16 hi values, then d lo values), for
// the first `rows` rows of every (sequence, KV head) table of cap rows, into
// tables of `rows` rows; one thread per 8 values.  norms (may be null):
// the f32 norm of every row, [slab][row].  The d/8 threads of a row are
// consecutive lanes of one wave (d/8 divides 64), and a row is either
// wholly inside the grid's range or wholly outside.
__global__ __launch_bounds__(256) void split_kernel(const float* src, uint16_t* dst, float* norms, int64_t cap,
                                                    int64_t rows, int64_t slabs, int d) {
  const int64_t segs = d / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const bool in = i < slabs * rows * segs;
  const int64_t ii = in ? i : 0;
  const int64_t sg = ii % segs, r = (ii / segs) % rows, x = ii / (segs * rows);
  float v[8];
  load8<false>(src + (x * cap + r) * d, sg * 8, v);
  Pack8 h, l;
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    split_bf16(v[k], h.h[k], l.h[k]);
    ss += v[k] * v[k];
  }
  if (in) {
    uint16_t* o = dst + (x * rows + r) * 2 * d;
    *reinterpret_cast<uint4*>(o + sg * 8) = h.q;
    *reinterpret_cast<uint4*>(o + d + sg * 8) = l.q;
  }
  if (norms != nullptr) {  // uniform
    for (int m = 1; m < segs; m <<= 1) ss += __shfl_xor(ss, m);
    if (in && sg == 0) norms[x * rows + r] = sqrtf(ss);
  }
}

// Exact top-k selection (lowest index wins ties): hga_select.h.

// Max over NB row blocks of q~ . s for the 16 summary rows whose f32 slices
// (d slots ks*32 + 8*(lane/16) + i of row lane%16) a lane holds in x.
template <int KS, int NB>
__device__ __forceinline__ float score16_regs(const float (&x)[KS][8], const Pack8 (&ahi)[NB][KS],
                                              const Pack8 (&alo)[NB][KS]) {
  Pack8 bhi[KS], blo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) split_bf16(x[ks][i], bhi[ks].h[i], blo[ks].h[i]);
  float best = -INFINITY;
#pragma unroll
  for (int blk = 0; blk < NB; ++blk) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      acc = mfma16x16x32(ahi[blk][ks].v, bhi[ks].v, acc);
      acc = mfma16x16x32(ahi[blk][ks].v, blo[ks].v, acc);
      acc = mfma16x16x32(alo[blk][ks].v, bhi[ks].v, acc);
    }
    best = fmaxf(best, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
  }
  best = fmaxf(best, __shfl_xor(best, 16));
  best = fmaxf(best, __shfl_xor(best, 32));
  return best;
}

// Max-scores of tiles tile0, tile0 + step, ... (16 candidates each) of n
// candidates given by row(i), streamed by one wave with DEPTH-1 tiles of
// summary rows in flight ahead of the one being multiplied; emit(tile, v)
// receives each tile's scores (lane%16 = candidate within the tile).  pro()
// runs after the first tiles' loads are issued and before the first product
// (it may fill ahi / alo; the wave must reach it even with no tiles).
template <int KS, int NB, typename RowPtr, typename Emit, typename Pro>
__device__ __forceinline__ void score_stream(int n, int tile0, int step, RowPtr row,
                                             const Pack8 (&ahi)[NB][KS],
                                             const Pack8 (&alo)[NB][KS], Emit emit, Pro pro) {
  constexpr int DEPTH = NB <= 2 ? 3 : 2;
  const int lane = threadIdx.x & 63;
  const int ntile = (n + 15) / 16;
  auto fetch = [&](int tile, float (&x)[KS][8]) {
    int c = tile * 16 + (lane & 15);
    if (c >= n) c = n - 1;
    const float* src = row(c);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load8<false>(src, ks * 32 + (lane >> 4) * 8, x[ks]);
  };
  float x[DEPTH][KS][8];
#pragma unroll
  for (int j = 0; j < DEPTH - 1; ++j)
    if (tile0 + j * step < ntile) fetch(tile0 + j * step, x[j]);
  pro();
  for (int base = 0;; base += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int tile = tile0 + (base + j) * step;
      if (tile >= ntile) return;
      const int ahead = tile + (DEPTH - 1) * step;
      if (ahead < ntile) fetch(ahead, x[(j + DEPTH - 1) % DEPTH]);
      emit(tile, score16_regs<KS, NB>(x[j], ahi, alo));
    }
  }
}

template <int KS, int NB, typename RowPtr, typename Emit>
__device__ __forceinline__ void score_stream(int n, int tile0, int step, RowPtr row,
                                             const Pack8 (&ahi)[NB][KS],
                                             const Pack8 (&alo)[NB][KS], Emit emit) {
  score_stream<KS, NB>(n, tile0, step, row, ahi, alo, emit, [] {});
}

// Segmented routing, first kernel: one segment of a unit's middle chunks,
// reduced to the segment's own top-K_c (keys and chunk offsets, ascending
// chunk order, key 0 for missing entries: real keys are never 0) and, with
// group routing, the scores of all groups of those K_c chunks (each
// segment scores its winners' groups, so the merge needs no query rows).
// NB row blocks of 16 rows cover the unit's rows; each wave streams every
// fourth tile of 16 rows, loading the next tiles while the current one is
// multiplied.  Workspace per unit: [nseg][K_c] keys, [nseg][K_c] offsets,
// [nseg][K_c][C/g_s] group keys (32-bit words).
template <bool BF16, int KS, int NB>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(RouteParams p) {
  __shared__ float2 cs[kMaxTableQ * kMaxHalfDim];
  __shared__ __align__(16) uint32_t keys[kMaxCand];  // also the RoPE table scratch
  __shared__ int sel[kMaxSel];
  __shared__ SelScratch scr;
  if (p.Kc <= 0) return;  // uniform: the merge does not route either
  const int64_t u = blockIdx.x / p.nseg;
  const int sg = blockIdx.x - static_cast<int>(u * p.nseg);
  const Unit w = make_unit(p, u);
  const int64_t m0 = w.mid_lo + static_cast<int64_t>(sg) * p.seg_chunks;
  int64_t m1 = m0 + p.seg_chunks;
  if (m1 > w.mid_hi) m1 = w.mid_hi;
  const int n = m1 > m0 && w.R > 0 ? static_cast<int>(m1 - m0) : 0;  // uniform
  const int64_t ncand = static_cast<int64_t>(p.nseg) * p.Kc;
  uint32_t* dk = p.ws + w.slot * p.ws_stride + static_cast<int64_t>(sg) * p.Kc;
  uint32_t* di = dk + ncand;
  uint32_t* dg = p.ws + w.slot * p.ws_stride + 2 * ncand + static_cast<int64_t>(sg) * p.Kc * p.r;
  const int ng = p.Kg > 0 ? p.Kc * p.r : 0;  // group keys this segment writes
  int nl = 0;
  if (n > 0) {
    Pack8 ahi[NB][KS], alo[NB][KS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float* base = p.csum + ((static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.nchunk_cap + m0) * p.d;
    auto rowp = [&](int c) { return base + static_cast<int64_t>(c) * p.d; };
    auto emit = [&](int tile, float v) {
      const int c = tile * 16 + (lane & 15);
      if (lane < 16 && c < n) keys[c] = order_key(v);
    };
    if constexpr (NB <= 2) {
      // the raw query rows and the first summary tiles are loaded while the
      // RoPE table is computed
      float xq[NB][KS][8];
#pragma unroll
      for (int blk = 0; blk < NB; ++blk) load_row_raw<BF16, KS>(p, w, row_of_lane(w, 0, blk), xq[blk]);
      score_stream<KS, NB>(n, wave, kScoreThreads / 64, rowp, ahi, alo, emit, [&] {
        fill_rope_table<KS>(p, w, cs, reinterpret_cast<float2*>(keys));
        __syncthreads();
#pragma unroll
        for (int blk = 0; blk < NB; ++blk)
        {
          float ss;
          rotate_split<KS>(p, row_of_lane(w, 0, blk), cs, xq[blk], ahi[blk], alo[blk], ss);
        }
      });
    } else {
      fill_rope_table<KS>(p, w, cs, reinterpret_cast<float2*>(keys));
      __syncthreads();
      load_rows<BF16, KS, NB>(p, w, 0, cs, ahi, alo);
      score_stream<KS, NB>(n, wave, kScoreThreads / 64, rowp, ahi, alo, emit);
    }
    __syncthreads();
    nl = block_select(keys, n, p.Kc, sel, scr);
    if (p.Kg > 0) {
      // groups of the segment's winners: candidate c = i * r + g is group g
      // of winner i (global id (m0 + sel[i]) * r + g)
      const int nc = nl * p.r;
      const float* g0 = p.gsum + (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.ngroup_cap * p.d;
      score_stream<KS, NB>(nc, wave, kScoreThreads / 64,
                           [&](int c) {
                             const int i = c / p.r;
                             return g0 + ((m0 + sel[i]) * p.r + (c - i * p.r)) * p.d;
                           },
                           ahi, alo, [&](int tile, float v) {
                             const int c = tile * 16 + (lane & 15);
                             if (lane < 16 && c < nc) dg[c] = order_key(v);
                           });
    }
  }
  const uint32_t off = static_cast<uint32_t>(m0 - w.mid_lo);
  for (int i = threadIdx.x; i < p.Kc; i += blockDim.x) {
    dk[i] = i < nl ? keys[sel[i]] : 0u;
    di[i] = i < nl ? off + static_cast<uint32_t>(sel[i]) : 0u;
  }
  for (int c = nl * p.r + threadIdx.x; c < ng; c += blockDim.x) dg[c] = 0u;
}

// Outputs of a unit.  The visible list is: sink granules, routed granules,
// recent granules, current-chunk granules up to the last query; the routed
// ones lie in [sink_hi, rec_lo) so the concatenation is ascending and
// unique.  selc: chosen chunks (ascending); selg: chosen groups (ascending
// global ids).  Block-wide.
__device__ __forceinline__ void write_lists(const RouteParams& p, const Unit& w, const int* selc,
                                            int nselc, const int* selg, int nselg) {
  const int tid = threadIdx.x, nt = blockDim.x;
  int32_t* ci = p.cidx + w.slot * p.Kc;
  for (int i = tid; i < p.Kc; i += nt) ci[i] = i < nselc ? selc[i] : -1;
  if (p.Kg > 0 && p.gidx != nullptr) {
    int32_t* gi = p.gidx + w.slot * p.Kg;
    for (int i = tid; i < p.Kg; i += nt) gi[i] = i < nselg ? selg[i] : -1;
  }
  const int r = p.r;
  const int n1 = static_cast<int>(w.sink_hi) * r;
  const int n2 = p.Kg > 0 ? nselg : nselc * r;
  const int64_t rec0 = w.rec_lo * r;
  const int n3 = static_cast<int>(w.t - w.rec_lo) * r;
  const int64_t cur0 = w.t * r;
  const int64_t qlast = w.qlo + w.nq - 1;
  const int n4 = static_cast<int>(qlast / p.gs - cur0 + 1);
  const int total = n1 + n2 + n3 + n4;
  int32_t* gl = p.gran + w.slot * p.gmax;
  for (int i = tid; i < p.gmax; i += nt) {
    int32_t v = -1;
    if (i < n1) {
      v = i;
    } else if (i < n1 + n2) {
      const int j = i - n1;
      v = p.Kg > 0 ? selg[j] : selc[j / r] * r + (j - (j / r) * r);
    } else if (i < n1 + n2 + n3) {
      v = static_cast<int32_t>(rec0 + (i - n1 - n2));
    } else if (i < total) {
      v = static_cast<int32_t>(cur0 + (i - n1 - n2 - n3));
    }
    gl[i] = v;
  }
  if (tid == 0) p.gcnt[w.slot] = total;
}

// Segmented routing, second kernel: one workgroup per unit.
constexpr int kMergeThreads = 256;
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(RouteParams p) {
  __shared__ uint32_t keys[kMaxCand];
  __shared__ int offs[kMaxCand];
  __shared__ uint32_t gks[kMaxCand];
  __shared__ int pos[kMaxSel];
  __shared__ int selc[kMaxSel];
  __shared__ int selg[kMaxSel];
  __shared__ SelScratch scr;
  const Unit w = make_unit(p, blockIdx.x);
  const int n_mid = static_cast<int>(w.mid_hi - w.mid_lo);
  int nselc = 0, nselg = 0;
  if (p.Kc > 0 && n_mid > 0 && w.R > 0) {  // uniform
    const int ncand = p.nseg * p.Kc;
    const int ngk = p.Kg > 0 ? ncand * p.r : 0;
    const uint32_t* src = p.ws + w.slot * p.ws_stride;
    for (int i = threadIdx.x; i < ncand; i += blockDim.x) {
      keys[i] = src[i];
      offs[i] = static_cast<int>(src[ncand + i]);
    }
    for (int i = threadIdx.x; i < ngk; i += blockDim.x) gks[i] = src[2 * ncand + i];
    __syncthreads();
    nselc = block_select(keys, ncand, p.Kc < n_mid ? p.Kc : n_mid, pos, scr);
    for (int i = threadIdx.x; i < nselc; i += blockDim.x) selc[i] = offs[pos[i]] + static_cast<int>(w.mid_lo);
    if (p.Kg > 0) {
      // candidate c = i * r + g: group g of the i-th chosen chunk (ascending
      // global group ids)
      const int nc = nselc * p.r;
      for (int c = threadIdx.x; c < nc; c += blockDim.x) {
        const int i = c / p.r;
        keys[c] = gks[pos[i] * p.r + (c - i * p.r)];
      }
      __syncthreads();
      nselg = block_select(keys, nc, p.Kg, selg, scr);
      for (int j = threadIdx.x; j < nselg; j += blockDim.x) {
        const int c = selg[j];
        const int i = c / p.r;
        selg[j] = selc[i] * p.r + (c - i * p.r);
      }
    }
    __syncthreads();
  }
  write_lists(p, w, selc, nselc, selg, nselg);
}

template <bool BF16, int KS, int NB>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteParams p) {
  __shared__ float2 cs[kMaxTableQ * kMaxHalfDim];
  __shared__ __align__(16) uint32_t keys[kMaxCand];  // also the RoPE table scratch
  __shared__ int selc[kMaxSel];
  __shared__ int selg[kMaxSel];
  __shared__ SelScratch scr;
  __shared__ uint32_t qmax2;  // largest squared norm of the unit's rotated rows (f32 bits)
  // staged split rows, two stages (the stage buffers are separate arrays so
  // that the compiler sees that reading one need not wait for loads into
  // the other)
  __shared__ __align__(1024) char sh0[kStageRows * 4 * kMaxHalfDim];
  __shared__ __align__(1024) char sl0[kStageRows * 4 * kMaxHalfDim];
  __shared__ __align__(1024) char sh1[kStageRows * 4 * kMaxHalfDim];
  __shared__ __align__(1024) char sl1[kStageRows * 4 * kMaxHalfDim];

  const Unit w = make_unit(p, blockIdx.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_mid = static_cast<int>(w.mid_hi - w.mid_lo);
  const bool route = p.Kc > 0 && n_mid > 0 && w.R > 0;

  // Work split inside the block: RG row groups (16*NB rows per wave) x TG
  // tile groups.
  constexpr int kRows = 16 * NB;
  const int RG = (w.R + kRows - 1) / kRows;
  const int TG = RG > 0 ? kRouteWaves / RG : 1;
  const int rg = RG > 0 ? wave % RG : 0;
  const int tg = RG > 0 ? wave / RG : kRouteWaves;
  const bool has_rows = route && tg < TG;

  Pack8 ahi[NB][KS], alo[NB][KS];
  int nselc = 0;
  if (route && n_mid <= p.Kc) {
    // every middle chunk is chosen: no scores needed
    nselc = n_mid;
    for (int i = threadIdx.x; i < n_mid; i += blockDim.x) selc[i] = static_cast<int>(w.mid_lo) + i;
    __syncthreads();
    if (p.Kg > 0) {  // the group phase needs the query rows
      fill_rope_table<KS>(p, w, cs, reinterpret_cast<float2*>(keys));
      __syncthreads();
      if (has_rows) load_rows<BF16, KS, NB>(p, w, rg * kRows, cs, ahi, alo);
      __syncthreads();
    }
  } else if (route) {
    {
      if (threadIdx.x == 0) qmax2 = 0u;
      float n2 = 0.f;
      if constexpr (BF16) {
        // the raw rows are in flight while the RoPE table is built
        uint4 raw[NB][KS];
        if (has_rows) issue_rows16<KS, NB>(p, w, rg * kRows, raw);
        fill_rope_table<KS>(p, w, cs, reinterpret_cast<float2*>(keys));
        __syncthreads();
        if (has_rows) n2 = rotate_rows16<KS, NB>(p, w, rg * kRows, cs, raw, ahi, alo);
      } else {
        fill_rope_table<KS>(p, w, cs, reinterpret_cast<float2*>(keys));
        __syncthreads();
        if (has_rows) n2 = load_rows<BF16, KS, NB>(p, w, rg * kRows, cs, ahi, alo);
      }
      if (has_rows && lane == 0) atomicMax(&qmax2, __float_as_uint(n2));  // n2 >= 0: bit order is value order
      for (int i = threadIdx.x; i < n_mid; i += blockDim.x) keys[i] = 0u;
      __syncthreads();
      const int64_t cbase = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.nchunk_cap;
      const int64_t slab = static_cast<int64_t>(w.b) * p.Hkv + w.kvh;
      const uint16_t* c0 = p.csplit + (slab * p.csplit_rows + w.mid_lo) * 2 * p.d;
      if (RG > 1 && n_mid > kScreenMin) {
        // Screened chunk scoring.  hi.hi scores s of every middle chunk
        // bound the split scores to s -/+ E_m (E_m = kScreenEps Q |c_m|);
        // lam = the K_c-th largest lower end; a chunk whose upper end is
        // below lam is beaten by at least K_c chunks, so the split scores
        // of the others (S, ascending) decide the same selection as
        // scoring them all.  cs (the RoPE table, no longer needed) holds
        // the upper ends and S.
        screen_staged<KS, NB>(n_mid, [&](int c) { return c0 + static_cast<int64_t>(c) * 2 * p.d; },
                              has_rows, tg, TG, ahi, alo, sh0, sl0, sh1, sl1, keys);
        uint32_t* hik = reinterpret_cast<uint32_t*>(cs);
        int* sidx = reinterpret_cast<int*>(cs) + kMaxCand;
        const float qn = sqrtf(__uint_as_float(qmax2));
        const float* cn = p.cnorm + slab * p.csplit_rows + w.mid_lo;
        for (int i = threadIdx.x; i < n_mid; i += blockDim.x) {
          const float sc = key_float(keys[i]);
          const float e = kScreenEps * qn * cn[i] + kScreenAbs;
          keys[i] = order_key(plus_zero(sc - e));
          hik[i] = order_key(plus_zero(sc + e));
        }
        __syncthreads();
        const uint32_t lam = block_kth(keys, n_mid, p.Kc, scr);
        const int ns = block_compact_ge(hik, n_mid, lam, sidx, scr);
        for (int i = threadIdx.x; i < ns; i += blockDim.x) keys[i] = 0u;
        __syncthreads();
        score_staged<KS, NB, true>(ns, [&](int i) { return c0 + static_cast<int64_t>(sidx[i]) * 2 * p.d; },
                                   has_rows, tg, TG, ahi, alo, sh0, sl0, sh1, sl1, keys);
        __syncthreads();
        nselc = block_select(keys, ns, p.Kc, selc, scr);
        for (int i = threadIdx.x; i < nselc; i += blockDim.x) selc[i] = sidx[selc[i]] + static_cast<int>(w.mid_lo);
        __syncthreads();
      } else {
      if (RG > 1) {
        score_staged<KS, NB, true>(n_mid, [&](int c) { return c0 + static_cast<int64_t>(c) * 2 * p.d; },
                             has_rows, tg, TG, ahi, alo, sh0, sl0, sh1, sl1, keys);
      } else if (has_rows) {
        const float* c0 = p.csum + (cbase + w.mid_lo) * p.d;
        score_stream<KS, NB>(n_mid, tg, TG, [&](int c) { return c0 + static_cast<int64_t>(c) * p.d; },
                             ahi, alo, [&](int tile, float v) {
                               const int c = tile * 16 + (lane & 15);
                               if (lane < 16 && c < n_mid) keys[c] = order_key(v);
                             });
      }
      __syncthreads();
      nselc = block_select(keys, n_mid, p.Kc, selc, scr);
      for (int i = threadIdx.x; i < nselc; i += blockDim.x) selc[i] += static_cast<int>(w.mid_lo);
      __syncthreads();
      }
    }
  }

  int nselg = 0;
  if (p.Kg > 0 && nselc > 0) {
    const int nc = nselc * p.r;
    for (int i = threadIdx.x; i < nc; i += blockDim.x) keys[i] = 0u;
    __syncthreads();
    const int64_t gbase = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.ngroup_cap;
    const float* g0 = p.gsum + gbase * p.d;
    auto grow = [&](int c) {
      const int cr = c / p.r;
      return g0 + (static_cast<int64_t>(selc[cr]) * p.r + (c - cr * p.r)) * p.d;
    };
    if (RG > 1) {
      const uint16_t* gs0 = p.gsplit + (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.gsplit_rows * 2 * p.d;
      score_staged<KS, NB, true>(nc, [&](int c) {
                             const int cr = c / p.r;
                             return gs0 + (static_cast<int64_t>(selc[cr]) * p.r + (c - cr * p.r)) * 2 * p.d;
                           },
                           has_rows, tg, TG, ahi, alo, sh0, sl0, sh1, sl1, keys);
    } else if (has_rows) {
      score_stream<KS, NB>(nc, tg, TG, grow, ahi, alo, [&](int tile, float v) {
        const int c = tile * 16 + (lane & 15);
        if (lane < 16 && c < nc) keys[c] = order_key(v);
      });
    }
    __syncthreads();
    nselg = block_select(keys, nc, p.Kg, selg, scr);
    for (int i = threadIdx.x; i < nselg; i += blockDim.x) {
      const int c = selg[i];
      const int cr = c / p.r;
      selg[i] = selc[cr] * p.r + (c - cr * p.r);
    }
    __syncthreads();
  }

  write_lists(p, w, selc, nselc, selg, nselg);
}


template <bool BF16, int KS, int NB>
hipError_t launch_route_nb(const RouteParams& p, int64_t units, bool segmented, hipStream_t stream) {
  if (segmented) {
    hipLaunchKernelGGL((score_kernel<BF16, KS, NB>), dim3(static_cast<unsigned>(units * p.nseg)),
                       dim3(kScoreThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(units)), dim3(kMergeThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((route_kernel<BF16, KS, NB>), dim3(static_cast<unsigned>(units)),
                       dim3(kRouteThreads), 0, stream, p);
  }
  return hipGetLastError();
}

// Row blocks of 16 per wave: enough for the rows of one unit up to 64 (then
// several waves split the rows).
template <bool BF16, int KS>
hipError_t launch_route_t(const RouteParams& p, int64_t units, bool segmented, hipStream_t stream) {
  const int64_t rows = (p.C < p.n_q ? p.C : p.n_q) * static_cast<int64_t>(p.G);
  if (rows <= 16) return launch_route_nb<BF16, KS, 1>(p, units, segmented, stream);
  if (rows <= 32) return launch_route_nb<BF16, KS, 2>(p, units, segmented, stream);
  return launch_route_nb<BF16, KS, 4>(p, units, segmented, stream);
}

int64_t max_middle(const Geometry& g) {
  const int64_t t = g.t0 + g.nqc - 1;
  const int64_t lp = g.L > 1 ? g.L : 1;
  const int64_t sink = t < g.F ? t : g.F;
  const int64_t rec = t - lp > sink ? t - lp : sink;
  return rec - sink;
}

// Few units with long middle contexts (decode-shaped calls): spread each
// unit's chunk scoring over several workgroups.
constexpr int64_t kSegUnits = 512;
bool use_segmented(const Geometry& g) {
  const int64_t units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  return units < kSegUnits && max_middle(g) > 256 && g.nqc == 1 &&
         g.n_q * static_cast<int64_t>(g.G) <= kRowsPerWave;
}

// Segments of a segmented call: about kSegBlocks scoring workgroups, each
// a multiple of kSegChunks chunks, and at most kMaxCand winners per unit.
constexpr int kSegChunks = 64;
constexpr int64_t kSegBlocks = 512;
struct SegPlan {
  int seg_chunks, nseg;
};
SegPlan seg_plan(const Geometry& g) {
  const int64_t units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  const int64_t mm = max_middle(g);
  int64_t nseg = (kSegBlocks + units - 1) / units;
  const int64_t most = (mm + kSegChunks - 1) / kSegChunks;
  if (nseg > most) nseg = most;
  // winners (and their groups) of all segments fit the merge's LDS
  const int64_t per = static_cast<int64_t>(g.Kc) * (g.Kg > 0 ? g.r : 1);
  if (per > 0 && nseg > kMaxCand / per) nseg = kMaxCand / per;
  if (nseg < 1) nseg = 1;
  SegPlan sp;
  sp.seg_chunks = static_cast<int>(((mm + nseg - 1) / nseg + kSegChunks - 1) / kSegChunks * kSegChunks);
  if (sp.seg_chunks < kSegChunks) sp.seg_chunks = kSegChunks;
  sp.nseg = static_cast<int>((mm + sp.seg_chunks - 1) / sp.seg_chunks);
  if (sp.nseg < 1) sp.nseg = 1;
  return sp;
}

// Unsegmented calls whose units have more rows than one wave holds score
// staged split rows (split_kernel); the split tables live in the workspace:
// [slab][chunk][2d] then [slab][group][2d] bf16.
bool use_split(const Geometry& g) {
  const int64_t rows = (g.C < g.n_q ? g.C : g.n_q) * static_cast<int64_t>(g.G);
  return !use_segmented(g) && g.Kc > 0 && rows > kRowsPerWave;
}
// Rows split: chunks [0, t_last] (a unit reads middle chunks before its own)
// and their groups; independent of kv_cap (the sizing call has none).  After
// the two split tables, the norms of the chunk rows (f32).
int64_t split_chunks(const Geometry& g) { return g.t0 + g.nqc; }
size_t split_bytes(const Geometry& g, size_t& gsplit_off, size_t& norm_off) {
  const size_t slabs = static_cast<size_t>(g.B) * g.Hkv;
  const size_t row = static_cast<size_t>(g.d) * 2 * 2;
  const size_t rc = static_cast<size_t>(split_chunks(g));
  const size_t c = slabs * rc * row;
  gsplit_off = (c + 255) / 256 * 256;
  const size_t gend = gsplit_off + (g.Kg > 0 ? slabs * rc * static_cast<size_t>(g.r) * row : 0);
  norm_off = (gend + 255) / 256 * 256;
  return norm_off + slabs * rc * sizeof(float);
}

}  // namespace

bool route_supported(const Geometry& g) {
  return (g.d == 64 || g.d == 128) && g.C <= kMaxTableQ && g.C * g.G <= kMaxRows &&
         max_middle(g) <= kMaxCand && g.Kc <= kMaxSel && g.Kg <= kMaxSel &&
         static_cast<int64_t>(g.Kc) * g.r <= kMaxCand;
}


size_t route_workspace(const Geometry& g) {
  if (use_split(g)) {
    size_t goff = 0, noff = 0;
    return split_bytes(g, goff, noff);
  }
  if (!use_segmented(g) || g.Kc <= 0) return 0;
  const SegPlan sp = seg_plan(g);
  return static_cast<size_t>(g.B) * g.Hkv * g.nqc * static_cast<size_t>(sp.nseg) * g.Kc *
         (2 + (g.Kg > 0 ? g.r : 0)) * sizeof(uint32_t);
}

hipError_t launch_route(const Geometry& g, const void* q, const float* chunk_sum,
                        const float* group_sum, int32_t* chunk_idx, int32_t* group_idx,
                        int32_t* granules, int32_t* granule_count, void* ws,
                        hipStream_t stream) {
  RouteParams p;
  p.q = q;
  p.csum = chunk_sum;
  p.gsum = group_sum;
  p.cidx = chunk_idx;
  p.gidx = group_idx;
  p.gran = granules;
  p.gcnt = granule_count;
  p.ws = static_cast<uint32_t*>(ws);
  p.q_pos0 = g.q_pos0;
  p.n_q = g.n_q;
  p.t0 = g.t0;
  p.nqc = g.nqc;
  p.nchunk_cap = g.kv_cap / g.C;
  p.ngroup_cap = g.kv_cap / g.gs;
  p.B = g.B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.d = g.d;
  p.C = g.C;
  p.gs = g.gs;
  p.r = g.r;
  p.F = g.F;
  p.L = g.L;
  p.Kc = g.Kc;
  p.Kg = g.Kg;
  p.gmax = g.gmax;
  p.rope = g.rope;
  const bool seg = use_segmented(g) && g.Kc > 0;
  const int64_t units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  const SegPlan sp = seg_plan(g);
  p.seg_chunks = sp.seg_chunks;
  p.nseg = sp.nseg;
  p.ws_stride = static_cast<int64_t>(sp.nseg) * g.Kc * (2 + (g.Kg > 0 ? g.r : 0));
  p.csplit = nullptr;
  p.gsplit = nullptr;
  p.cnorm = nullptr;
  p.csplit_rows = p.gsplit_rows = 0;
  if (use_split(g)) {
    // split the summary rows the call can read: chunks before the last
    // query chunk and their groups
    size_t goff = 0, noff = 0;
    split_bytes(g, goff, noff);
    uint16_t* cs = static_cast<uint16_t*>(ws);
    uint16_t* gsp = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + goff);
    float* cn = reinterpret_cast<float*>(static_cast<char*>(ws) + noff);
    const int64_t slabs = static_cast<int64_t>(g.B) * g.Hkv;
    const int64_t rc = split_chunks(g);  // <= nchunk_cap (q_pos0 + n_q <= kv_cap)
    const int64_t n8 = slabs * rc * (g.d / 8);
    hipLaunchKernelGGL(split_kernel, dim3(static_cast<unsigned>((n8 + 255) / 256)), dim3(256), 0, stream,
                       chunk_sum, cs, cn, p.nchunk_cap, rc, slabs, g.d);
    p.csplit_rows = rc;
    p.gsplit_rows = rc * g.r;
    if (g.Kg > 0) {
      const int64_t g8 = slabs * rc * g.r * (g.d / 8);
      hipLaunchKernelGGL(split_kernel, dim3(static_cast<unsigned>((g8 + 255) / 256)), dim3(256), 0, stream,
                         group_sum, gsp, nullptr, p.ngroup_cap, rc * g.r, slabs, g.d);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    p.csplit = cs;
    p.gsplit = gsp;
    p.cnorm = cn;
  }
  if (g.bf16) {
    return g.d == 128 ? launch_route_t<true, 4>(p, units, seg, stream)
                      : launch_route_t<true, 2>(p, units, seg, stream);
  }
  return g.d == 128 ? launch_route_t<false, 4>(p, units, seg, stream)
                    : launch_route_t<false, 2>(p, units, seg, stream);
}

}  // namespace hga
