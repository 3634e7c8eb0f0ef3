// One decode step of routed exact-token attention: one new query per
// sequence at position pos; chunk scan, top-K_c, group scores and top-K_g,
// the visible lists, exact-token attention and the merge of its partials,
// in two launches.
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3: routing policy (the sink, recent and previous-chunk windows are
// visible whatever routing picks; the middle context competes), the score
// q^T c_m, the selection equation (top-K_c chunks, then top-K_g of their
// groups) and the exact-token output paragraph.  The pages name the
// exhaustive scan of the routing table as the step's cost (section 8); the
// fixed windows, which do not depend on it, are attended while it runs.
//
// Launch 1 (decode_scan_kernel, 256 threads per item), two kinds of items
// per unit (sequence, KV head), all independent:
//  * scan items, one per segment of the unit's middle chunks: score the
//    segment's chunk summaries on f32 matrix cores (max over the unit's
//    query rows, i.e. the G heads of the KV head), keep the segment's
//    top-K_c (a unit's top-K_c is a subset of the union of its segments'
//    top-K_c, in the same order and tie-break) and score those chunks'
//    groups; write both to the workspace;
//  * window items, one per 128 keys of the fixed windows and the current
//    chunk up to pos: attend them and write an (m, l, O) partial.
// Launch 2 (decode_finish_kernel, one item of 8 waves per unit): select the
// unit's top-K_c among the segments' winners and its top-K_g among their
// groups, write the lists, attend the routed tokens (256 keys per round) and
// merge that with the window partials into the output and the LSE.  The
// launch boundary orders the two; nothing waits on a counter.
//
// Attention of 32 keys per wave: K rows from HBM into the A operands of
// 16x16x32 bf16 products (S^T = K Q^T, query rows on N), softmax in
// registers (base 2), P and V through the wave's LDS rows for O = P V on
// the same products; the waves' (m, l, O) are merged in LDS.
#include <algorithm>

#include "hga_device.h"
#include "hga_select.h"

namespace hga {
namespace {

constexpr int kScanThreads = 256;              // launch 1: 4 waves
constexpr int kFinishThreads = 512;            // launch 2: 8 waves
constexpr int kDsWaveKeys = 32;
constexpr int kDsWinKeys = 4 * kDsWaveKeys;    // keys per window item
constexpr int kDsMaxRows = 16;                 // query rows per unit (G)
constexpr int kDsMaxSeg = 1024;                // chunks per scan item
constexpr int kDsMaxCand = 1024;               // segment winners per unit (merge)
constexpr int kDsMaxGroupCand = 4096;          // their groups
constexpr int kDsMaxRouted = 1024;             // routed granules per unit
constexpr int kDsWinRegs = 32;                 // window partial floats per launch-2 thread
constexpr int kDsMinSeg = 32;                  // chunks per scan item, at least
constexpr int kDsItemsPerCU = 3;               // launch-1 items resident per CU
constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.6931471805599453f;
constexpr float kNegBigD = -1.0e30f;

struct DecodeParams {
  const void* q;        // [B][Hq][1][D] raw queries
  const void* k;        // [B][Hkv][kv_cap][D] rotated keys
  const void* v;        // [B][Hkv][kv_cap][D]
  const float* csum;    // [B][Hkv][kv_cap/C][D]
  const float* gsum;    // [B][Hkv][kv_cap/g_s][D]
  int32_t* cidx;        // [B][Hkv][K_c] (with gidx, gran, gcnt: NULL = lists not written)
  int32_t* gidx;        // [B][Hkv][K_g]
  int32_t* gran;        // [B][Hkv][gmax]
  int32_t* gcnt;        // [B][Hkv]
  void* out;            // [B][Hq][1][D]
  float* lse;           // [B][Hq][1] or NULL
  uint32_t* seg;        // per unit: [nseg][K_c] keys, [nseg][K_c] offsets, [nseg][K_c][r] group keys
  float* part;          // per unit: nwin window partials of RP rows: O [RP][D], then (m, l) [RP][2]
  int64_t pos, kv_cap, nchunk_cap, ngroup_cap, units;
  int64_t t, sink_hi, rec_lo, n_sink_tok, win_keys;
  int64_t seg_stride;   // words per unit in seg
  int B, Hq, Hkv, G, C, gs, lg_gs, r, Kc, Kg, gmax;
  int nseg, seg_chunks, nwin;
  float scale_log2;
  RopeFreqs rope;
};

// LDS of the attention of NW waves (32 keys each) for up to 16 rows.
template <int D, int NW>
struct AttnSmem {
  char vbuf[NW * kDsWaveKeys * (2 * D + 32)];  // V tiles; also the wave merge buffer [NW][16][D]
  float wm[NW][kDsMaxRows], wl[NW][kDsMaxRows];
  float run_o[kDsMaxRows][D];
  float run_m[kDsMaxRows], run_l[kDsMaxRows];
  float new_m[kDsMaxRows], new_l[kDsMaxRows];
};
static_assert(sizeof(float) * kDsMaxRows * 128 <= kDsWaveKeys * (2 * 128 + 32), "merge buffer fits vbuf");
static_assert(sizeof(float) * kDsMaxRows * 64 <= kDsWaveKeys * (2 * 64 + 32), "merge buffer fits vbuf");
// Window partial floats per unit launch 2 can hold: kDsWinRegs per thread,
// parked in the 8-wave V buffer once the routed rounds are done.
constexpr int64_t win_floats(int d) {
  return std::min<int64_t>(kDsWinRegs * 512, 8 * kDsWaveKeys * (2 * d + 32) / 4);
}

// Barrier for LDS traffic: waits for this wave's LDS operations only, not
// for vector-memory loads still in flight (the fence of __syncthreads would
// wait for those too, stalling every prefetch issued before it).
__device__ __forceinline__ void lds_barrier() { wait_vm_barrier<63>(); }

// Row r (< 16) of the unit reads query head kvh * G + min(r, G - 1): padded
// rows repeat the last one, which leaves every max unchanged.
__device__ __forceinline__ int head_of_row(const DecodeParams& p, int kvh, int r) {
  const int rr = r < p.G ? r : p.G - 1;
  return kvh * p.G + rr;
}

template <int D>
__device__ __forceinline__ void fill_cs(const DecodeParams& p, float2* cs) {
  for (int j = threadIdx.x; j < D / 2; j += blockDim.x) {
    float c, s;
    rope_cs(static_cast<double>(rope_base(p.rope, p.pos)), rope_freq(p.rope, j), c, s);
    cs[j] = make_float2(c, s);
  }
}

__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Scores of n summary rows (row(c) -> its D floats) against the unit's
// rotated query rows, on f32 matrix cores (16x16x4: A = 16 summary rows x 4
// dims, B = 4 dims x 16 query rows, f32 products and sums): in tile t of 16
// rows, lane l loads float4 s of row 16t + l%16 at dims 16s + 4(l/16); the
// j-th element of that float4 and q~[l%16][16s + 4(l/16) + j] (qv[s][j]) are
// the lane's A and B values of product (s, j).  Wave w takes tiles w, w+4,
// ...: the loads of its first two tiles go out before prologue() (which
// fills qv), and each later tile's loads go out while the previous tile is
// multiplied.  The max over the query rows (lanes l%16) gives emit(c, score)
// on lanes l%16 == 0.
template <int D, typename RowPtr, typename Prologue, typename Emit>
__device__ __forceinline__ void score_rows(int n, RowPtr row, const float (&qv)[D / 16][4], Prologue prologue,
                                           Emit emit) {
  constexpr int S = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int ntile = (n + 15) >> 4;
  auto fetch = [&](int tile, float4 (&x)[S]) {
    const int c = tile * 16 + m;
    const float* rp = row(c < n ? c : 0);
#pragma unroll
    for (int s = 0; s < S; ++s)
      x[s] = c < n ? *reinterpret_cast<const float4*>(rp + 16 * s + 4 * kg) : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  auto reduce_emit = [&](int tile, const float4 (&x)[S]) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < S; s += 2) {
      a0 = mfma16x16x4f32(x[s].x, qv[s][0], a0);
      a1 = mfma16x16x4f32(x[s + 1].x, qv[s + 1][0], a1);
      a0 = mfma16x16x4f32(x[s].y, qv[s][1], a0);
      a1 = mfma16x16x4f32(x[s + 1].y, qv[s + 1][1], a1);
      a0 = mfma16x16x4f32(x[s].z, qv[s][2], a0);
      a1 = mfma16x16x4f32(x[s + 1].z, qv[s + 1][2], a1);
      a0 = mfma16x16x4f32(x[s].w, qv[s][3], a0);
      a1 = mfma16x16x4f32(x[s + 1].w, qv[s + 1][3], a1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = row16_max(a0[i] + a1[i]);  // row 4 kg + i of the tile, max over query rows l%16
      const int c = tile * 16 + 4 * kg + i;
      if (m == 0 && c < n) emit(c, plus_zero(v));
    }
  };
  float4 x0[S], x1[S];
  if (wave < ntile) fetch(wave, x0);
  if (wave + 4 < ntile) fetch(wave + 4, x1);
  prologue();
  for (int t = wave; t < ntile; t += 8) {
    reduce_emit(t, x0);
    if (t + 8 < ntile) fetch(t + 8, x0);
    if (t + 4 < ntile) {
      reduce_emit(t + 4, x1);
      if (t + 12 < ntile) fetch(t + 12, x1);
    }
  }
}

// K and V of the wave's 32 keys (lane l and l + 32 name key l of the wave
// through tok: a token <= pos, or -1).  K rows go to registers as the A
// operands of two 16-key tiles (key lane % 16, d slots ks*32 + 8*(lane/16) +
// i); V rows are loaded 16 bytes per lane (CPR lanes per row, 64 / CPR rows
// per load) for the wave's row-major LDS tile.  Absent keys read row 0 of K
// (their score is masked) and zeros for V (their P is zero, and 0 * NaN
// would not be).
template <int D>
struct WaveKV {
  static constexpr int CPR = D / 8;        // 16-byte chunks per V row
  static constexpr int RPI = 64 / CPR;     // V rows per load
  static constexpr int NI = kDsWaveKeys / RPI;
  Pack8 ka[2][D / 32];
  uint4 vq[NI];
  int tok;
};

// V rows of the wave in LDS: row-major, 2d + 32 bytes apart (the
// transposing reads of a 16-lane group then touch disjoint banks).
template <int D>
constexpr int vpitch() { return 2 * D + 32; }

template <int D>
__device__ __forceinline__ void load_wave_kv(const DecodeParams& p, int64_t slab, int tok, WaveKV<D>& kv) {
  constexpr int KS = D / 32;
  using KV = WaveKV<D>;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, sub = lane >> 4;
  kv.tok = tok;
  const int row = tok >= 0 ? tok : 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kr = __shfl(row, t * 16 + n);
    const int64_t e = (slab + kr) * D + sub * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kv.ka[t][ks].q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + e + ks * 32);
  }
#pragma unroll
  for (int j = 0; j < KV::NI; ++j) {
    const int vt = __shfl(tok, j * KV::RPI + lane / KV::CPR);
    const int64_t e = (slab + (vt >= 0 ? vt : 0)) * D + (lane % KV::CPR) * 8;
    kv.vq[j] = vt >= 0 ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + e)
                       : make_uint4(0u, 0u, 0u, 0u);
  }
}

// The wave's keys against the unit's rows: (m, l) per row and the row's O
// tile in ot (16x16x32 accumulator layout: column n = lane % 16 is the row,
// the four values are output columns 4*(lane/16)+i of each tile).
// S^T = K Q^T on two 16x16x32 bf16 products leaves lane (n, sub) the scores
// of keys 4 sub + i and 16 + 4 sub + i of row n; those are exactly the keys
// of its eight k slots in O = P V when V's B operand comes from the
// transposing LDS read (ds_read_b64_tr_b16: lane j of a 16-lane group reads
// 8 bytes of row 16 h + 4 sub + j/4 at columns 4 (j%4) .. +3 of the tile,
// lane i receives column i of the 4 rows), so P goes from the softmax
// registers straight into the A operand.
template <int D, int NW>
__device__ __forceinline__ void attend_wave(const Pack8 (&qb)[D / 32], const WaveKV<D>& kv,
                                            AttnSmem<D, NW>& sa, float& mx, float& ls,
                                            f32x4 (&ot)[D / 16]) {
  constexpr int KS = D / 32;
  constexpr int NT = D / 16;
  constexpr int VP = vpitch<D>();
  using KV = WaveKV<D>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, sub = lane >> 4;
  // V rows into the wave's LDS tile (read back after the softmax)
  char* vw = sa.vbuf + wave * kDsWaveKeys * VP;
#pragma unroll
  for (int j = 0; j < KV::NI; ++j)
    *reinterpret_cast<uint4*>(vw + (j * KV::RPI + lane / KV::CPR) * VP + (lane % KV::CPR) * 16) = kv.vq[j];
  float sv[2][4];
  mx = kNegBigD;
  // key k of the wave is present iff bit k of the ballot is set (lane k names it)
  const uint64_t present = __ballot(kv.tok >= 0);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(kv.ka[t][ks].v, qb[ks].v, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool on = (present >> (t * 16 + sub * 4 + i)) & 1ull;
      sv[t][i] = on ? acc[i] : -INFINITY;
      mx = fmaxf(mx, sv[t][i]);
    }
  }
  mx = xor32_max(xor16_max(mx));
  Pack8 pa;
  ls = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float e0 = exp2f(sv[t][0] - mx), e1 = exp2f(sv[t][1] - mx);
    const float e2 = exp2f(sv[t][2] - mx), e3 = exp2f(sv[t][3] - mx);  // 0 for masked keys
    ls += (e0 + e1) + (e2 + e3);
    pa.u[2 * t] = pack_bf16x2(e0, e1);
    pa.u[2 * t + 1] = pack_bf16x2(e2, e3);
  }
  ls = xor32_sum(xor16_sum(ls));
  // the wave's own LDS rows: a wave-local wait suffices
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    Pack8 vb;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint2 v2 = lds_read_tr16(vw + (16 * h + 4 * sub + (n >> 2)) * VP + (16 * c + 4 * (n & 3)) * 2);
      vb.u[2 * h] = v2.x;
      vb.u[2 * h + 1] = v2.y;
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    ot[c] = mfma16x16x32(pa.v, vb.v, z);
  }
}

template <int D, int NW>
__device__ __forceinline__ void reset_running(AttnSmem<D, NW>& sa) {
  for (int i = threadIdx.x; i < kDsMaxRows; i += NW * 64) {
    sa.run_m[i] = kNegBigD;
    sa.run_l[i] = 0.f;
  }
  for (int i = threadIdx.x; i < kDsMaxRows * D; i += NW * 64) (&sa.run_o[0][0])[i] = 0.f;
}

// One round of NW * 32 keys already loaded (kv): the waves' results folded
// into the running (m, l, O) of the unit's R rows in sa.run_*.
template <int D, int NW>
__device__ __forceinline__ void fold_round(const Pack8 (&qb)[D / 32], const WaveKV<D>& kv, int R,
                                           AttnSmem<D, NW>& sa) {
  constexpr int NT = D / 16;
  constexpr int NTH = NW * 64;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, sub = lane >> 4;
  float mx, ls;
  f32x4 ot[NT];
  __syncthreads();  // the previous round's fold has read vbuf / pw
  attend_wave<D, NW>(qb, kv, sa, mx, ls, ot);
  __syncthreads();
  float* wo = reinterpret_cast<float*>(sa.vbuf);  // [NW][16][D]
  if (sub == 0) {
    sa.wm[wave][n] = mx;
    sa.wl[wave][n] = ls;
  }
#pragma unroll
  for (int c = 0; c < NT; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = sub * 4 + i;
      if (rr < R) wo[(wave * kDsMaxRows + rr) * D + c * 16 + n] = ot[c][i];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R * D; i += NTH) {
    const int rr = i / D, d = i - rr * D;
    float m = sa.run_m[rr];
#pragma unroll
    for (int x = 0; x < NW; ++x) m = fmaxf(m, sa.wm[x][rr]);
    const float s0 = exp2f(sa.run_m[rr] - m);
    float l = sa.run_l[rr] * s0, acc = sa.run_o[rr][d] * s0;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      const float sc = exp2f(sa.wm[x][rr] - m);
      l += sa.wl[x][rr] * sc;
      acc += wo[(x * kDsMaxRows + rr) * D + d] * sc;
    }
    sa.run_o[rr][d] = acc;
    if (d == 0) {
      sa.new_m[rr] = m;
      sa.new_l[rr] = l;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R; i += NTH) {
    sa.run_m[i] = sa.new_m[i];
    sa.run_l[i] = sa.new_l[i];
  }
  __syncthreads();
}

// The rotated, scaled query rows as bf16 B operands (row n = lane % 16,
// d slots ks*32 + 8*(lane/16) + i; pairs (j, j + D/2)): the raw elements
// first (load_query_raw), the rotation once cs is filled (rotate_query).
template <int D>
__device__ __forceinline__ void load_query_raw(const DecodeParams& p, int b, int kvh, float (&xq)[D / 32][8]) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, sub = lane >> 4;
  const int64_t base = (static_cast<int64_t>(b) * p.Hq + head_of_row(p, kvh, n)) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) load8<true>(p.q, base + ks * 32 + sub * 8, xq[ks]);
}

template <int D>
__device__ __forceinline__ void rotate_query(const DecodeParams& p, const float2* cs, const float (&xq)[D / 32][8],
                                             Pack8 (&qb)[D / 32]) {
  constexpr int KS = D / 32;
  const int sub = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 t = cs[ks * 32 + sub * 8 + i];
      const float a = xq[ks][i], c = xq[ks + KS / 2][i];
      qb[ks].h[i] = f32_to_bf16((a * t.x - c * t.y) * p.scale_log2);
      qb[ks + KS / 2].h[i] = f32_to_bf16((a * t.y + c * t.x) * p.scale_log2);
    }
  }
}

// Write the unit's lists: chunk / group selections and the visible granules
// (sink, routed, recent, current up to pos: four ascending runs).
__device__ __forceinline__ void write_lists(const DecodeParams& p, int64_t u, const int* selc, int nselc,
                                            const int* selg, int nselg) {
  const int tid = threadIdx.x;
  if (p.Kc > 0) {
    int32_t* ci = p.cidx + u * p.Kc;
    for (int i = tid; i < p.Kc; i += static_cast<int>(blockDim.x)) ci[i] = i < nselc ? selc[i] : -1;
  }
  if (p.Kg > 0) {
    int32_t* gi = p.gidx + u * p.Kg;
    for (int i = tid; i < p.Kg; i += static_cast<int>(blockDim.x)) gi[i] = i < nselg ? selg[i] : -1;
  }
  const int r = p.r;
  const int n1 = static_cast<int>(p.sink_hi) * r;
  const int n2 = p.Kg > 0 ? nselg : nselc * r;
  const int64_t rec0 = p.rec_lo * r;
  const int n3 = static_cast<int>(p.t - p.rec_lo) * r;
  const int64_t cur0 = p.t * r;
  const int n4 = static_cast<int>(p.pos / p.gs - cur0 + 1);
  const int total = n1 + n2 + n3 + n4;
  int32_t* gl = p.gran + u * p.gmax;
  for (int i = tid; i < p.gmax; i += static_cast<int>(blockDim.x)) {
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
  if (tid == 0) p.gcnt[u] = total;
}

// ---------------------------------------------------------------- launch 1

template <int D>
union ScanSmem {
  struct {
    float qs[kDsMaxRows][D];  // rotated query rows (f32)
    uint32_t keys[kDsMaxSeg];
    int sel[256];
    SelScratch scr;
  } scan;
  AttnSmem<D, 4> attn;
};

template <int D, int RP>
__global__ __launch_bounds__(kScanThreads) void decode_scan_kernel(DecodeParams p) {
  __shared__ ScanSmem<D> sm;
  __shared__ float2 cs[D / 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t nscan = p.units * p.nseg;
  const bool scan = static_cast<int64_t>(blockIdx.x) < nscan;
  const int64_t item = scan ? blockIdx.x : blockIdx.x - nscan;
  const int64_t u = item % p.units;
  const int idx = static_cast<int>(item / p.units);  // segment or window block
  const int b = static_cast<int>(u / p.Hkv), kvh = static_cast<int>(u - static_cast<int64_t>(b) * p.Hkv);
  const int64_t slab = (static_cast<int64_t>(b) * p.Hkv + kvh) * p.kv_cap;

  if (!scan) {
    // window block: keys [idx*128, (idx+1)*128) of the sink tokens followed
    // by the recent chunks and the current chunk up to pos
    const int64_t kk = static_cast<int64_t>(idx) * kDsWinKeys + (tid >> 6) * kDsWaveKeys + (lane & 31);
    const int tok = kk < p.win_keys
                        ? static_cast<int>(kk < p.n_sink_tok ? kk : p.rec_lo * p.C + (kk - p.n_sink_tok))
                        : -1;
    float xq[D / 32][8];
    load_query_raw<D>(p, b, kvh, xq);  // first: the rotation waits on these alone
    WaveKV<D> kv;
    load_wave_kv<D>(p, slab, tok, kv);
    fill_cs<D>(p, cs);
    reset_running<D, 4>(sm.attn);
    lds_barrier();  // K and V stay in flight while the query is rotated
    Pack8 qb[D / 32];
    rotate_query<D>(p, cs, xq, qb);
    fold_round<D, 4>(qb, kv, p.G, sm.attn);
    float* dst = p.part + (u * p.nwin + idx) * static_cast<int64_t>(RP) * (D + 2);
    for (int i = tid; i < p.G * D; i += kScanThreads) dst[i] = (&sm.attn.run_o[0][0])[i];
    for (int i = tid; i < p.G; i += kScanThreads) {
      dst[RP * D + 2 * i] = sm.attn.run_m[i];
      dst[RP * D + 2 * i + 1] = sm.attn.run_l[i];
    }
    return;
  }

  // scan item: one segment of the middle chunks
  if (p.Kc <= 0) return;
  const int64_t m0 = p.sink_hi + static_cast<int64_t>(idx) * p.seg_chunks;
  const int n = static_cast<int>(std::max<int64_t>(0, std::min<int64_t>(m0 + p.seg_chunks, p.rec_lo) - m0));
  const int64_t ncand = static_cast<int64_t>(p.nseg) * p.Kc;
  uint32_t* useg = p.seg + u * p.seg_stride;
  auto& ss = sm.scan;
  // the query setup runs while the first summary tiles are loading
  constexpr int PER = kDsMaxRows * (D / 2) / kScanThreads;
  float xa[PER], xc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid + k * kScanThreads;
    const int rr = i / (D / 2), j = i - rr * (D / 2);
    const int64_t qb0 = (static_cast<int64_t>(b) * p.Hq + head_of_row(p, kvh, rr)) * D;
    xa[k] = load1<true>(p.q, qb0 + j);
    xc[k] = load1<true>(p.q, qb0 + j + D / 2);
  }
  float qv[D / 16][4];
  auto setup = [&] {  // the summary tiles stay in flight across its barriers
    fill_cs<D>(p, cs);
    lds_barrier();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int i = tid + k * kScanThreads;
      const int rr = i / (D / 2), j = i - rr * (D / 2);
      const float2 t = cs[j];
      ss.qs[rr][j] = xa[k] * t.x - xc[k] * t.y;
      ss.qs[rr][j + D / 2] = xa[k] * t.y + xc[k] * t.x;
    }
    lds_barrier();
    const int qn = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) {
      const float4 x = *reinterpret_cast<const float4*>(&ss.qs[qn][16 * s2 + 4 * kg]);
      qv[s2][0] = x.x; qv[s2][1] = x.y; qv[s2][2] = x.z; qv[s2][3] = x.w;
    }
  };
  const float* cbase = p.csum + ((static_cast<int64_t>(b) * p.Hkv + kvh) * p.nchunk_cap + m0) * D;
  score_rows<D>(n, [&](int c) { return cbase + static_cast<int64_t>(c) * D; }, qv, setup,
                [&](int c, float s) { ss.keys[c] = order_key(s); });
  __syncthreads();
  int nl;
  if (p.Kc < n && n <= 256) {  // one wave selects (ballot radix), no block-wide passes
    if (tid < 64) {
      auto key = [&](int i) { return ss.keys[i]; };
      if (n <= 64) wave_select<1>(key, n, p.Kc, ss.sel);
      else if (n <= 128) wave_select<2>(key, n, p.Kc, ss.sel);
      else if (n <= 192) wave_select<3>(key, n, p.Kc, ss.sel);
      else wave_select<4>(key, n, p.Kc, ss.sel);
    }
    __syncthreads();
    nl = p.Kc;
  } else {
    nl = block_select(ss.keys, n, p.Kc, ss.sel, ss.scr);
  }
  uint32_t* dk = useg + static_cast<int64_t>(idx) * p.Kc;
  uint32_t* di = dk + ncand;
  if (p.Kg > 0) {
    uint32_t* dg = useg + 2 * ncand + static_cast<int64_t>(idx) * p.Kc * p.r;
    const int nc = nl * p.r;
    const float* g0 = p.gsum + (static_cast<int64_t>(b) * p.Hkv + kvh) * p.ngroup_cap * D;
    score_rows<D>(nc,
                  [&](int c) {
                    const int i = c / p.r;
                    return g0 + ((m0 + ss.sel[i]) * p.r + (c - i * p.r)) * D;
                  },
                  qv, [] {}, [&](int c, float s) { dg[c] = order_key(s); });
    for (int c = nc + tid; c < p.Kc * p.r; c += kScanThreads) dg[c] = 0u;
  }
  const uint32_t off = static_cast<uint32_t>(m0 - p.sink_hi);
  for (int i = tid; i < p.Kc; i += kScanThreads) {
    dk[i] = i < nl ? ss.keys[ss.sel[i]] : 0u;  // 0: no entry (real keys are never 0)
    di[i] = i < nl ? off + static_cast<uint32_t>(ss.sel[i]) : 0u;
  }
}

// ---------------------------------------------------------------- launch 2

template <int D>
struct FinishSmem {
  union {
    struct {
      uint32_t keys[kDsMaxGroupCand];
      int offs[kDsMaxCand];
      uint32_t gks[kDsMaxGroupCand];
      int pos[256];
      SelScratch scr;
    } merge;
    AttnSmem<D, 8> attn;
  } u;
  float2 cs[D / 2];
  int selc[256], selg[256];
  int nselc, nselg;
  float wpart[win_floats(D)];  // the window partials, parked once the selection is done
};

template <int D, int RP>
__global__ __launch_bounds__(kFinishThreads) void decode_finish_kernel(DecodeParams p) {
  __shared__ FinishSmem<D> sm;
  constexpr int NTH = kFinishThreads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t u = blockIdx.x;
  const int b = static_cast<int>(u / p.Hkv), kvh = static_cast<int>(u - static_cast<int64_t>(b) * p.Hkv);
  const int R = p.G;
  const int64_t slab = (static_cast<int64_t>(b) * p.Hkv + kvh) * p.kv_cap;
  const int64_t n_mid = p.rec_lo - p.sink_hi;
  const bool routing = p.Kc > 0 && n_mid > 0;
  const int ncand = p.nseg * p.Kc;
  const int ngk = p.Kg > 0 ? ncand * p.r : 0;
  const uint32_t* useg = p.seg + u * p.seg_stride;
  // everything this item reads first, in the order it is needed: the
  // segments' winners (into registers, so that their LDS stores wait for
  // them alone), the query, then the window partials (held in registers
  // until the routed attention is done: nwin slots of RP rows, O then (m, l))
  constexpr int WPT = (kDsMaxCand + NTH - 1) / NTH;        // winners per thread
  constexpr int GPT = (kDsMaxGroupCand + NTH - 1) / NTH;   // group keys per thread
  uint32_t wk[WPT], wo[WPT], wg[GPT];
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int i = tid + k * NTH;
    const bool in = routing && i < ncand;
    wk[k] = in ? useg[i] : 0u;
    wo[k] = in ? useg[ncand + i] : 0u;
  }
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int i = tid + k * NTH;
    wg[k] = routing && i < ngk ? useg[2 * ncand + i] : 0u;
  }
  float xq[D / 32][8];
  load_query_raw<D>(p, b, kvh, xq);
  const int64_t nwf = static_cast<int64_t>(p.nwin) * RP * (D + 2);
  const float* wp = p.part + u * nwf;
  float wreg[kDsWinRegs];
#pragma unroll
  for (int k = 0; k < kDsWinRegs; ++k) {
    const int64_t i = tid + static_cast<int64_t>(k) * NTH;
    wreg[k] = i < nwf ? wp[i] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < WPT; ++k) {
    const int i = tid + k * NTH;
    if (routing && i < ncand) {
      sm.u.merge.keys[i] = wk[k];
      sm.u.merge.offs[i] = static_cast<int>(wo[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int i = tid + k * NTH;
    if (routing && i < ngk) sm.u.merge.gks[i] = wg[k];
  }
  fill_cs<D>(p, sm.cs);
  if (tid == 0) sm.nselc = sm.nselg = 0;
  lds_barrier();
  const int want = routing ? static_cast<int>(std::min<int64_t>(p.Kc, n_mid)) : 0;
  if (routing && ncand <= 64 && (p.Kg <= 0 || std::min(want, ncand) * p.r <= 64)) {
    // wave 0 makes both selections (ballot radix select, no block-wide
    // passes): at most 64 segment winners and 64 groups of the chosen chunks
    auto& ms = sm.u.merge;
    if (wave == 0) {
      const int nselc = want < ncand ? want : ncand;
      if (want < ncand) {
        wave_select<1>([&](int i) { return ms.keys[i]; }, ncand, want, ms.pos);
      } else if (lane < ncand) {
        ms.pos[lane] = lane;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's own LDS writes
      __builtin_amdgcn_wave_barrier();
      if (lane < nselc) sm.selc[lane] = ms.offs[ms.pos[lane]] + static_cast<int>(p.sink_hi);
      int nselg = 0;
      if (p.Kg > 0) {
        const int nc = nselc * p.r;
        auto gkey = [&](int c) {
          const int i = c / p.r;
          return ms.gks[ms.pos[i] * p.r + (c - i * p.r)];
        };
        nselg = p.Kg < nc ? p.Kg : nc;
        if (p.Kg < nc) {
          wave_select<1>(gkey, nc, p.Kg, sm.selg);
        } else if (lane < nc) {
          sm.selg[lane] = lane;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        if (lane < nselg) {
          const int c = sm.selg[lane];
          const int i = c / p.r;
          sm.selg[lane] = sm.selc[i] * p.r + (c - i * p.r);
        }
      }
      if (lane == 0) {
        sm.nselc = nselc;
        sm.nselg = nselg;
      }
    }
  } else if (routing) {
    auto& ms = sm.u.merge;
    const int nselc = block_select(ms.keys, ncand, want, ms.pos, ms.scr);
    for (int i = tid; i < nselc; i += NTH) sm.selc[i] = ms.offs[ms.pos[i]] + static_cast<int>(p.sink_hi);
    int nselg = 0;
    if (p.Kg > 0) {
      const int nc = nselc * p.r;
      __syncthreads();  // ms.keys is rewritten with the group keys
      for (int c = tid; c < nc; c += NTH) {
        const int i = c / p.r;
        ms.keys[c] = ms.gks[ms.pos[i] * p.r + (c - i * p.r)];
      }
      __syncthreads();
      nselg = block_select(ms.keys, nc, p.Kg, sm.selg, ms.scr);
      __syncthreads();
      for (int j = tid; j < nselg; j += NTH) {
        const int c = sm.selg[j];
        const int i = c / p.r;
        sm.selg[j] = sm.selc[i] * p.r + (c - i * p.r);
      }
    }
    if (tid == 0) {
      sm.nselc = nselc;
      sm.nselg = nselg;
    }
  }
  __syncthreads();
  const int nselc = sm.nselc, nselg = sm.nselg;
  const int nrouted = p.Kg > 0 ? nselg : nselc * p.r;
  // routed tokens, 256 keys per round: token of routed key k, from the
  // selections in LDS; the first round's K/V loads go out before the lists
  // are written and the query is rotated
  const int64_t nkeys = static_cast<int64_t>(nrouted) * p.gs;
  // the window partials (loaded first, in registers since) into their LDS region
#pragma unroll
  for (int k = 0; k < kDsWinRegs; ++k) {
    const int64_t i = tid + static_cast<int64_t>(k) * NTH;
    if (i < nwf) sm.wpart[i] = wreg[k];
  }
  auto tok_of = [&](int64_t k) -> int {
    if (k >= nkeys) return -1;
    const int j = static_cast<int>(k >> p.lg_gs);
    const int g = p.Kg > 0 ? sm.selg[j] : sm.selc[j / p.r] * p.r + (j - (j / p.r) * p.r);
    return g * p.gs + static_cast<int>(k & (p.gs - 1));
  };
  WaveKV<D> kv;
  load_wave_kv<D>(p, slab, tok_of(wave * kDsWaveKeys + (lane & 31)), kv);
  if (p.gran != nullptr) write_lists(p, u, sm.selc, nselc, sm.selg, nselg);
  Pack8 qb[D / 32];
  rotate_query<D>(p, sm.cs, xq, qb);
  auto& sa = sm.u.attn;
  constexpr int SS = RP * (D + 2);  // floats per window partial
  if (nkeys <= 8 * kDsWaveKeys) {
    // One round: the eight waves' partials and the window partials are
    // merged in one pass; each wave's O rows overwrite its own V tile once
    // its products have read it.
    float mx, ls;
    f32x4 ot[D / 16];
    attend_wave<D, 8>(qb, kv, sa, mx, ls, ot);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's V reads are done
    __builtin_amdgcn_wave_barrier();
    float* wo = reinterpret_cast<float*>(sa.vbuf + wave * kDsWaveKeys * vpitch<D>());  // [16][D]
    const int n = lane & 15, sub = lane >> 4;
    if (sub == 0) {
      sa.wm[wave][n] = mx;
      sa.wl[wave][n] = ls;
    }
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = sub * 4 + i;
        if (rr < R) wo[rr * D + c * 16 + n] = ot[c][i];
      }
    __syncthreads();
    for (int i = tid; i < R * D; i += NTH) {
      const int rr = i / D, d = i - rr * D;
      float m = kNegBigD;
#pragma unroll
      for (int x = 0; x < 8; ++x) m = fmaxf(m, sa.wm[x][rr]);
      for (int s = 0; s < p.nwin; ++s) m = fmaxf(m, sm.wpart[s * SS + RP * D + 2 * rr]);
      float l = 0.f, acc = 0.f;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const float sc = exp2f(sa.wm[x][rr] - m);
        l += sa.wl[x][rr] * sc;
        acc += reinterpret_cast<const float*>(sa.vbuf + x * kDsWaveKeys * vpitch<D>())[rr * D + d] * sc;
      }
      for (int s = 0; s < p.nwin; ++s) {
        const float sc = exp2f(sm.wpart[s * SS + RP * D + 2 * rr] - m);
        l += sm.wpart[s * SS + RP * D + 2 * rr + 1] * sc;
        acc += sm.wpart[s * SS + rr * D + d] * sc;
      }
      const int64_t orow = static_cast<int64_t>(b) * p.Hq + kvh * p.G + rr;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      store1<true>(p.out, orow * D + d, acc * inv);
      if (p.lse != nullptr && d == 0) p.lse[orow] = (m + log2f(l)) * kLn2D;
    }
    return;
  }
  reset_running<D, 8>(sa);  // fold_round's first barrier orders it before any read
  for (int64_t k0 = 0; k0 < nkeys; k0 += 8 * kDsWaveKeys) {
    if (k0 > 0) load_wave_kv<D>(p, slab, tok_of(k0 + wave * kDsWaveKeys + (lane & 31)), kv);
    fold_round<D, 8>(qb, kv, R, sa);
  }
  // merge with the window partials: output rows and LSE (fold_round ended
  // with a barrier, which also made the parked partials visible)
  const float* win = sm.wpart;
  for (int i = tid; i < R * D; i += NTH) {
    const int rr = i / D, d = i - rr * D;
    float m = sa.run_m[rr];
    for (int s = 0; s < p.nwin; ++s) m = fmaxf(m, win[s * SS + RP * D + 2 * rr]);
    const float s0 = exp2f(sa.run_m[rr] - m);
    float l = sa.run_l[rr] * s0, acc = sa.run_o[rr][d] * s0;
    for (int s = 0; s < p.nwin; ++s) {
      const float sc = exp2f(win[s * SS + RP * D + 2 * rr] - m);
      l += win[s * SS + RP * D + 2 * rr + 1] * sc;
      acc += win[s * SS + rr * D + d] * sc;
    }
    const int64_t orow = static_cast<int64_t>(b) * p.Hq + kvh * p.G + rr;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    store1<true>(p.out, orow * D + d, acc * inv);
    if (p.lse != nullptr && d == 0) p.lse[orow] = (m + log2f(l)) * kLn2D;
  }
}

struct DecodePlan {
  int64_t units, t, sink_hi, rec_lo, n_mid, n_sink_tok, win_keys;
  int nseg, seg_chunks, nwin, rp;
  size_t seg_off, part_off, total;
  bool ok;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

DecodePlan decode_plan(const Geometry& g, int64_t cus) {
  DecodePlan pl{};
  pl.units = static_cast<int64_t>(g.B) * g.Hkv;
  const int64_t pos = g.q_pos0;
  pl.t = pos / g.C;
  const int64_t lp = g.L > 1 ? g.L : 1;
  pl.sink_hi = pl.t < g.F ? pl.t : g.F;
  pl.rec_lo = std::max<int64_t>(pl.sink_hi, pl.t - lp);
  pl.n_mid = pl.rec_lo - pl.sink_hi;
  pl.n_sink_tok = pl.sink_hi * g.C;
  pl.win_keys = pl.n_sink_tok + (pos + 1 - pl.rec_lo * g.C);
  pl.nwin = static_cast<int>((pl.win_keys + kDsWinKeys - 1) / kDsWinKeys);
  pl.rp = g.G <= 4 ? 4 : (g.G <= 8 ? 8 : 16);
  // scan items: the launch's items fill the resident slots once (window
  // items included), each at least kDsMinSeg chunks, the winners of all
  // segments within the merge's LDS
  const int64_t slots = kDsItemsPerCU * cus;
  int64_t nseg = (slots - pl.units * pl.nwin) / pl.units;
  nseg = std::min<int64_t>(std::max<int64_t>(nseg, 1), std::max<int64_t>(1, (pl.n_mid + kDsMinSeg - 1) / kDsMinSeg));
  if (g.Kc > 0) {
    nseg = std::min<int64_t>(nseg, kDsMaxCand / g.Kc);
    if (g.Kg > 0) nseg = std::min<int64_t>(nseg, kDsMaxGroupCand / (static_cast<int64_t>(g.Kc) * g.r));
  }
  nseg = std::max<int64_t>(nseg, 1);
  const int64_t seg = pl.n_mid > 0 ? (pl.n_mid + nseg - 1) / nseg : 1;
  pl.seg_chunks = static_cast<int>(seg);
  pl.nseg = pl.n_mid > 0 ? static_cast<int>((pl.n_mid + seg - 1) / seg) : 1;
  const int64_t routed = g.Kg > 0 ? g.Kg : static_cast<int64_t>(g.Kc) * g.r;
  pl.ok = g.bf16 && (g.d == 64 || g.d == 128) && g.n_q == 1 && g.G <= kDsMaxRows &&
          g.Kc <= 256 && g.Kg <= 256 && seg <= kDsMaxSeg && routed <= kDsMaxRouted &&
          (g.Kc == 0 || static_cast<int64_t>(pl.nseg) * g.Kc <= kDsMaxCand) &&
          (g.Kg == 0 || static_cast<int64_t>(pl.nseg) * g.Kc * g.r <= kDsMaxGroupCand) &&
          static_cast<int64_t>(pl.nwin) * pl.rp * (g.d + 2) <= win_floats(g.d) && (g.gs & (g.gs - 1)) == 0;
  const size_t words = static_cast<size_t>(pl.nseg) * g.Kc * (2 + (g.Kg > 0 ? g.r : 0));
  pl.seg_off = 0;
  pl.part_off = round256(static_cast<size_t>(pl.units) * words * sizeof(uint32_t));
  pl.total = pl.part_off + static_cast<size_t>(pl.units) * pl.nwin * pl.rp * (g.d + 2) * sizeof(float);
  return pl;
}

template <int D, int RP>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int64_t grid = p.units * (p.nseg + p.nwin);
  hipLaunchKernelGGL((decode_scan_kernel<D, RP>), dim3(static_cast<unsigned>(grid)), dim3(kScanThreads), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_finish_kernel<D, RP>), dim3(static_cast<unsigned>(p.units)), dim3(kFinishThreads),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace

// The plan depends on the device's compute units only through the number of
// scan items (how the scan is split, not what it computes), so sizing and
// support use 256 CUs (MI355X) and the launch uses the same plan.
constexpr int64_t kPlanCUs = 256;

bool decode_step_supported(const Geometry& g) { return decode_plan(g, kPlanCUs).ok; }

size_t decode_step_workspace(const Geometry& g) { return decode_plan(g, kPlanCUs).total; }

hipError_t launch_decode_step(const Geometry& g, const void* q, const void* k_rot, const void* v,
                              const float* chunk_sum, const float* group_sum, int32_t* chunk_idx,
                              int32_t* group_idx, int32_t* granules, int32_t* granule_count, void* out,
                              float* lse, void* ws, hipStream_t stream) {
  const DecodePlan pl = decode_plan(g, kPlanCUs);
  DecodeParams p;
  p.q = q;
  p.k = k_rot;
  p.v = v;
  p.csum = chunk_sum;
  p.gsum = group_sum;
  p.cidx = chunk_idx;
  p.gidx = group_idx;
  p.gran = granules;
  p.gcnt = granule_count;
  p.out = out;
  p.lse = lse;
  char* w = static_cast<char*>(ws);
  p.seg = reinterpret_cast<uint32_t*>(w + pl.seg_off);
  p.part = reinterpret_cast<float*>(w + pl.part_off);
  p.pos = g.q_pos0;
  p.kv_cap = g.kv_cap;
  p.nchunk_cap = g.kv_cap / g.C;
  p.ngroup_cap = g.kv_cap / g.gs;
  p.units = pl.units;
  p.t = pl.t;
  p.sink_hi = pl.sink_hi;
  p.rec_lo = pl.rec_lo;
  p.n_sink_tok = pl.n_sink_tok;
  p.win_keys = pl.win_keys;
  p.seg_stride = static_cast<int64_t>(pl.nseg) * g.Kc * (2 + (g.Kg > 0 ? g.r : 0));
  p.B = g.B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.C = g.C;
  p.gs = g.gs;
  p.lg_gs = 0;
  while ((1 << p.lg_gs) < g.gs) ++p.lg_gs;
  p.r = g.r;
  p.Kc = g.Kc;
  p.Kg = g.Kg;
  p.gmax = g.gmax;
  p.nseg = pl.nseg;
  p.seg_chunks = pl.seg_chunks;
  p.nwin = pl.nwin;
  p.scale_log2 = g.scale * kLog2eD;
  p.rope = g.rope;
  if (g.d == 128) {
    if (pl.rp == 4) return launch_t<128, 4>(p, stream);
    if (pl.rp == 8) return launch_t<128, 8>(p, stream);
    return launch_t<128, 16>(p, stream);
  }
  if (pl.rp == 4) return launch_t<64, 4>(p, stream);
  if (pl.rp == 8) return launch_t<64, 8>(p, stream);
  return launch_t<64, 16>(p, stream);
}

}  // namespace hga
