// Exact-token attention over each unit's visible granules (routed) or over
// every key j <= i (dense causal, Eq. 1).
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3: exact-token output (softmax over the real token K/V of the
// current chunk's causal part, the fixed windows and the routed groups or
// chunks, with no summary tokens) and Eq. (1) (dense causal attention).
//
// bf16 path (attend_mfma_kernel): one workgroup holds NW waves x 32 query
// rows of one unit (sequence, KV head, query chunk); a row is (query, head)
// with the G query heads of the KV head interleaved, so all GQA heads share
// every K/V tile.  K/V tiles of 32 gathered tokens are staged in LDS (K
// row-major, V transposed) and double-buffered; each wave computes
//   S^T = K Q^T      (32x32x16 bf16 MFMA, keys on M, query rows on N)
//   online softmax   (f32, base 2, Q pre-scaled by scale*log2(e))
//   O^T += V^T P^T   (32x32x16 bf16 MFMA, P rounded to bf16)
// With rows on N each lane owns one row, so row max / sum need one lane
// exchange.  K rows are read into the MFMA in the order pi(m) (bits 2 and 3
// of m swapped), which makes the S^T accumulator registers of a lane cover
// exactly the 8 consecutive keys the PV product wants from it: P never goes
// through LDS.  Few-unit calls (decode) split each unit's keys over several
// workgroups and merge (m, l, O) partials in combine_kernel.
//
// f32 path (attend_f32_kernel): one wave per 64 rows, one lane per row,
// K/V tiles in LDS, f32 vector ALU; exact to f32 rounding.
#include <algorithm>

#include "hga_device.h"

namespace hga {
namespace {

constexpr int kTK = 32;           // keys per tile
constexpr int kVPitch = kTK * 2 + 16;  // bytes per transposed V row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;

struct AttendParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* gran;
  const int32_t* gcnt;
  // Pool mode (host tier): K and V of granule-list entry i of a unit live in
  // a granule-major staging pool [slot][2][g_s][D] at slot pool_slot[i];
  // k and v then both point at the pool.
  const int32_t* pool_slot;
  int64_t pool_slots;
  float* ws_o;   // [slot][split][Rcap][D]
  float* ws_ml;  // [slot][split][Rcap][2]
  int64_t q_pos0, n_q, kv_cap, t0, nqc;
  // q / out / lse rows: row r of a (sequence, head) holds position q_row0 + r
  // and rows are q_stride apart (a window call covers part of the array).
  int64_t q_stride, q_row0;
  int B, Hq, Hkv, G, d, C, gs, gmax, Rcap;
  int nw, slices, splits, keys_per_split;
  int dense;
  float scale_log2;
  RopeFreqs rope;
};

struct AUnit {
  int b, kvh;
  int64_t t, qlo, slot;
  int nq, R, nkeys;
};

__device__ __forceinline__ AUnit make_aunit(const AttendParams& p, int64_t u) {
  AUnit w;
  const int64_t bh = static_cast<int64_t>(p.B) * p.Hkv;
  const int64_t trel = p.nqc - 1 - u / bh;
  const int64_t rem = u % bh;
  w.b = static_cast<int>(rem / p.Hkv);
  w.kvh = static_cast<int>(rem % p.Hkv);
  w.t = p.t0 + trel;
  const int64_t c0 = w.t * p.C;
  w.qlo = c0 > p.q_pos0 ? c0 : p.q_pos0;
  const int64_t qend = p.q_pos0 + p.n_q;
  const int64_t qhi = (c0 + p.C) < qend ? (c0 + p.C) : qend;
  w.nq = static_cast<int>(qhi - w.qlo);
  w.R = w.nq * p.G;
  w.slot = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.nqc + trel;
  if (p.dense) {
    w.nkeys = static_cast<int>(((qhi - 1) / p.gs + 1) * p.gs);
  } else {
    w.nkeys = p.gcnt[w.slot] * p.gs;
  }
  return w;
}

// Token held by key slot s of a unit (slot order = ascending granules), or
// -1 when a caller-supplied granule id lies outside [0, kv_cap / g_s) (or,
// in pool mode, its pool slot lies outside the pool).
__device__ __forceinline__ int64_t slot_token(const AttendParams& p, const AUnit& w, int s) {
  if (p.dense) return s;
  const int gi = s / p.gs;
  const int64_t tok = static_cast<int64_t>(p.gran[w.slot * p.gmax + gi]) * p.gs + (s - gi * p.gs);
  if (p.pool_slot != nullptr) {
    const int64_t ps = p.pool_slot[w.slot * p.gmax + gi];
    if (ps < 0 || ps >= p.pool_slots) return -1;
  }
  return (tok >= 0 && tok < p.kv_cap) ? tok : -1;
}

// Element offsets (from p.k and p.v) of the K and V rows of key slot s
// holding token tok.
template <int D>
__device__ __forceinline__ void kv_offsets(const AttendParams& p, const AUnit& w, int s, int64_t tok,
                                           int64_t slab, int64_t& ko, int64_t& vo) {
  if (p.pool_slot != nullptr) {
    const int gi = s / p.gs;
    const int64_t ps = p.pool_slot[w.slot * p.gmax + gi];
    ko = (ps * 2 * p.gs + (s - gi * p.gs)) * D;
    vo = ko + static_cast<int64_t>(p.gs) * D;
  } else {
    ko = vo = (slab + tok) * D;
  }
}

// K row index read by MFMA row m: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D, int NW>
struct TileRegs {
  static constexpr int kSlots = kTK * (D / 8);
  static constexpr int kPer = (kSlots + NW * 64 - 1) / (NW * 64);
  uint4 k[kPer];
  uint4 v[kPer];
  int tok;  // token of key slot threadIdx.x (threads < kTK), -1 = none
};

template <int D, int NW>
__device__ __forceinline__ void load_tile(const AttendParams& p, const AUnit& w, int kbase,
                                          int kend, int64_t slab, TileRegs<D, NW>& tr) {
  constexpr int SL = D / 8;
#pragma unroll
  for (int i = 0; i < TileRegs<D, NW>::kPer; ++i) {
    const int idx = threadIdx.x + i * NW * 64;
    uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (idx < TileRegs<D, NW>::kSlots) {
      const int s = idx / SL, sl = idx - s * SL;
      const int gs = kbase + s;
      const int64_t tok = gs < kend ? slot_token(p, w, gs) : -1;
      if (tok >= 0) {
        int64_t ko, vo;
        kv_offsets<D>(p, w, gs, tok, slab, ko, vo);
        kk = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + ko + sl * 8);
        vv = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + vo + sl * 8);
      }
    }
    tr.k[i] = kk;
    tr.v[i] = vv;
  }
  tr.tok = -1;
  if (threadIdx.x < kTK) {
    const int gs = kbase + threadIdx.x;
    if (gs < kend) tr.tok = static_cast<int>(slot_token(p, w, gs));
  }
}

template <int D, int NW>
__device__ __forceinline__ void store_tile(const TileRegs<D, NW>& tr, char* kl, char* vl, int* tl) {
  constexpr int SL = D / 8;
  constexpr int KP = D * 2 + 16;
#pragma unroll
  for (int i = 0; i < TileRegs<D, NW>::kPer; ++i) {
    const int idx = threadIdx.x + i * NW * 64;
    if (idx < TileRegs<D, NW>::kSlots) {
      const int s = idx / SL, sl = idx - s * SL;
      *reinterpret_cast<uint4*>(kl + s * KP + sl * 16) = tr.k[i];
      const uint32_t u[4] = {tr.v[i].x, tr.v[i].y, tr.v[i].z, tr.v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint16_t*>(vl + (sl * 8 + 2 * e) * kVPitch + s * 2) =
            static_cast<uint16_t>(u[e] & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(vl + (sl * 8 + 2 * e + 1) * kVPitch + s * 2) =
            static_cast<uint16_t>(u[e] >> 16);
      }
    }
  }
  if (threadIdx.x < kTK) tl[threadIdx.x] = tr.tok;
}

template <int D>
constexpr int tile_bytes() {
  return kTK * (D * 2 + 16) + D * kVPitch + kTK * 4;
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attend_mfma_kernel(AttendParams p) {
  constexpr int KS = D / 16;    // k-steps of S^T over d
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int KP = D * 2 + 16;
  constexpr int TB = tile_bytes<D>();
  constexpr int H = D / 2;
  constexpr int kTable = 64 * H * 8;
  constexpr int kSmem = (2 * TB) > kTable ? (2 * TB) : kTable;
  __shared__ __align__(16) char smem[kSmem];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int per_unit = p.slices * p.splits;
  const int64_t u = blockIdx.x / per_unit;
  const int rem = static_cast<int>(blockIdx.x - u * per_unit);
  const int slice = rem / p.splits;
  const int split = rem - slice * p.splits;
  const AUnit w = make_aunit(p, u);
  const int r0 = slice * NW * 32;
  if (r0 >= w.R) return;  // uniform
  const int kbeg = split * p.keys_per_split;
  int kend = kbeg + p.keys_per_split;
  if (kend > w.nkeys) kend = w.nkeys;

  // RoPE table for the queries of this workgroup's rows.
  const int rend = (r0 + NW * 32) < w.R ? (r0 + NW * 32) : w.R;
  const int q_first = r0 / p.G;
  const int nqt = (rend - 1) / p.G - q_first + 1;
  float2* cs = reinterpret_cast<float2*>(smem);
  for (int i = threadIdx.x; i < nqt * H; i += NW * 64) {
    const int qi = i / H, pr = i - qi * H;
    float c, s;
    rope_cs(static_cast<double>(w.qlo + q_first + qi), p.rope.f[pr], c, s);
    cs[i] = make_float2(c, s);
  }
  __syncthreads();

  // Query rows: lane -> row n = lane % 32, d slots ks*16 + 8*(lane/32) + i.
  const int n = lane & 31, hsub = lane >> 5;
  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < w.R;
  const int qloc = row_ok ? row / p.G : q_first;
  const int hl = row_ok ? row - qloc * p.G : 0;
  const int64_t qpos = w.qlo + qloc;
  Pack8 qb[KS];
  {
    float x[KS][8];
    const int64_t base =
        ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (qpos - p.q_row0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row_ok) {
        load8<true>(p.q, base + ks * 16 + hsub * 8, x[ks]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[ks][i] = 0.f;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float2 t = cs[(qloc - q_first) * H + ks * 16 + hsub * 8 + i];
        const float a = x[ks][i], b = x[ks + KS / 2][i];
        x[ks][i] = a * t.x - b * t.y;
        x[ks + KS / 2][i] = a * t.y + b * t.x;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) qb[ks].h[i] = f32_to_bf16(x[ks][i] * p.scale_log2);
    }
  }
  __syncthreads();  // the table space becomes K/V tile buffers

  const bool wave_rows = (r0 + wave * 32) < w.R;
  const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap;
  const int64_t cur0 = w.t * p.C;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.f;
  float m_run = kNegBig, l_run = 0.f;

  const int ntiles = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;
  TileRegs<D, NW> tr;
  if (ntiles > 0) load_tile<D, NW>(p, w, kbeg, kend, slab, tr);
  const int prow = perm_row(n);
  for (int tile = 0; tile < ntiles; ++tile) {
    char* kl = smem + (tile & 1) * TB;
    char* vl = kl + kTK * KP;
    int* tl = reinterpret_cast<int*>(vl + D * kVPitch);
    store_tile<D, NW>(tr, kl, vl, tl);
    __syncthreads();
    if (tile + 1 < ntiles) load_tile<D, NW>(p, w, kbeg + (tile + 1) * kTK, kend, slab, tr);
    if (wave_rows) {
      f32x16 s;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + prow * KP + (ks * 16 + hsub * 8) * 2);
        s = mfma32x32x16(a, qb[ks].v, s);
      }
      // s[j] holds key slot 16*(j/8) + 8*hsub + (j%8) of the tile for row n.
      float mx = kNegBig;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int ks_ = 16 * (j >> 3) + 8 * hsub + (j & 7);
        const int tok = tl[ks_];
        const bool ok = tok >= 0 && (tok < cur0 || tok <= qpos);
        s[j] = ok ? s[j] : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      float psum = 0.f;
      Pack8 pb[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = __builtin_amdgcn_exp2f(s[j] - m_new);
        psum += e;
        pb[j >> 3].h[j & 7] = f32_to_bf16(e);
      }
      psum += __shfl_xor(psum, 32);
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(vl + (db * 32 + n) * kVPitch + (kk * 16 + hsub * 8) * 2);
          o[db] = mfma32x32x16(a, pb[kk].v, o[db]);
        }
      }
    }
  }

  if (!row_ok) return;
  // O^T register j of block db is d = db*32 + 8*(j/4) + 4*hsub + (j%4).
  const int64_t orow = (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (qpos - p.q_row0);
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* out = static_cast<uint16_t*>(p.out) + orow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hsub;
        uint2 pk;
        pk.x = pack_bf16x2(o[db][4 * g4 + 0] * inv, o[db][4 * g4 + 1] * inv);
        pk.y = pack_bf16x2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
        *reinterpret_cast<uint2*>(out + d0) = pk;
      }
    }
    if (p.lse != nullptr && hsub == 0) p.lse[orow] = (m_run + log2f(l_run)) * kLn2;
  } else {
    const int64_t prow_i = (w.slot * p.splits + split) * p.Rcap + row;
    float* wo = p.ws_o + prow_i * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * hsub;
        *reinterpret_cast<float4*>(wo + d0) =
            make_float4(o[db][4 * g4], o[db][4 * g4 + 1], o[db][4 * g4 + 2], o[db][4 * g4 + 3]);
      }
    }
    if (hsub == 0) {
      p.ws_ml[prow_i * 2] = m_run;
      p.ws_ml[prow_i * 2 + 1] = l_run;
    }
  }
}

// f32 inputs: one wave per 64 rows, one lane per row.
template <int D>
__global__ __launch_bounds__(64) void attend_f32_kernel(AttendParams p) {
  constexpr int TK = 32;
  constexpr int H = D / 2;
  __shared__ __align__(16) float kt[TK][D];
  __shared__ __align__(16) float vt[TK][D];
  __shared__ int tk[TK];
  const int lane = threadIdx.x;
  const int per_unit = p.slices * p.splits;
  const int64_t u = blockIdx.x / per_unit;
  const int rem = static_cast<int>(blockIdx.x - u * per_unit);
  const int slice = rem / p.splits;
  const int split = rem - slice * p.splits;
  const AUnit w = make_aunit(p, u);
  const int r0 = slice * 64;
  if (r0 >= w.R) return;
  const int kbeg = split * p.keys_per_split;
  int kend = kbeg + p.keys_per_split;
  if (kend > w.nkeys) kend = w.nkeys;

  const int row = r0 + lane;
  const bool row_ok = row < w.R;
  const int qloc = row_ok ? row / p.G : 0;
  const int hl = row_ok ? row - qloc * p.G : 0;
  const int64_t qpos = w.qlo + qloc;
  float q[D];
  {
    const float* src = static_cast<const float*>(p.q) +
        ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (qpos - p.q_row0)) * D;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float a = row_ok ? src[i] : 0.f, b = row_ok ? src[i + H] : 0.f;
      float c, s;
      rope_cs(static_cast<double>(qpos), p.rope.f[i], c, s);
      q[i] = (a * c - b * s) * p.scale_log2;
      q[i + H] = (a * s + b * c) * p.scale_log2;
    }
  }
  float o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap;
  const int64_t cur0 = w.t * p.C;
  for (int kb = kbeg; kb < kend; kb += TK) {
    __syncthreads();
    for (int idx = lane; idx < TK * D / 4; idx += 64) {
      const int s = idx / (D / 4), c4 = idx - s * (D / 4);
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      const int64_t tok = kb + s < kend ? slot_token(p, w, kb + s) : -1;
      if (tok >= 0) {
        int64_t ko, vo;
        kv_offsets<D>(p, w, kb + s, tok, slab, ko, vo);
        kk = reinterpret_cast<const float4*>(static_cast<const float*>(p.k) + ko)[c4];
        vv = reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + vo)[c4];
      }
      reinterpret_cast<float4*>(&kt[s][0])[c4] = kk;
      reinterpret_cast<float4*>(&vt[s][0])[c4] = vv;
    }
    if (lane < TK) tk[lane] = (kb + lane < kend) ? static_cast<int>(slot_token(p, w, kb + lane)) : -1;
    __syncthreads();
    float sc[TK];
    float mx = kNegBig;
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) acc = fmaf(q[i], kt[s][i], acc);
      const int tok = tk[s];
      const bool ok = tok >= 0 && (tok < cur0 || tok <= qpos);
      sc[s] = ok ? acc : -INFINITY;
      mx = fmaxf(mx, sc[s]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] *= alpha;
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      const float e = exp2f(sc[s] - m_new);
      l_run += e;
#pragma unroll
      for (int i = 0; i < D; ++i) o[i] = fmaf(e, vt[s][i], o[i]);
    }
    m_run = m_new;
  }
  if (!row_ok) return;
  const int64_t orow = (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (qpos - p.q_row0);
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = static_cast<float*>(p.out) + orow * D;
#pragma unroll
    for (int i = 0; i < D; ++i) out[i] = o[i] * inv;
    if (p.lse != nullptr) p.lse[orow] = (m_run + log2f(l_run)) * kLn2;
  } else {
    const int64_t prow_i = (w.slot * p.splits + split) * p.Rcap + row;
#pragma unroll
    for (int i = 0; i < D; ++i) p.ws_o[prow_i * D + i] = o[i];
    p.ws_ml[prow_i * 2] = m_run;
    p.ws_ml[prow_i * 2 + 1] = l_run;
  }
}

// Merge split-key partials: m = max m_s, l = sum l_s 2^(m_s - m),
// O = sum O_s 2^(m_s - m) / l.  One wave per row.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttendParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 4 + wave;  // (unit, row)
  const int64_t units = static_cast<int64_t>(p.B) * p.Hkv * p.nqc;
  if (gr >= units * p.Rcap) return;
  const int64_t u = gr / p.Rcap;
  const int row = static_cast<int>(gr - u * p.Rcap);
  const AUnit w = make_aunit(p, u);
  if (row >= w.R) return;
  float m = kNegBig;
  for (int s = 0; s < p.splits; ++s) {
    if (s * p.keys_per_split >= w.nkeys) break;
    m = fmaxf(m, p.ws_ml[((w.slot * p.splits + s) * p.Rcap + row) * 2]);
  }
  float l = 0.f;
  float acc[D / 64 > 0 ? D / 64 : 1];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    if (s * p.keys_per_split >= w.nkeys) break;
    const int64_t pr = (w.slot * p.splits + s) * p.Rcap + row;
    const float sc = exp2f(p.ws_ml[pr * 2] - m);
    l += p.ws_ml[pr * 2 + 1] * sc;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] += p.ws_o[pr * D + lane + 64 * i] * sc;
  }
  const int qloc = row / p.G, hl = row - qloc * p.G;
  const int64_t orow =
      (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (w.qlo + qloc - p.q_row0);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) store1<BF16>(p.out, orow * D + lane + 64 * i, acc[i] * inv);
  if (p.lse != nullptr && lane == 0) p.lse[orow] = (m + log2f(l)) * kLn2;
}

struct Plan {
  int nw, slices, splits, kps, rcap;
  int64_t units;
};

// Keys of the largest unit: every key up to the last query (dense), or the
// granule budget, which can never exceed that count (routed).
int64_t max_keys(const Geometry& g, bool dense) {
  const int64_t qlast = g.q_pos0 + g.n_q - 1;
  const int64_t causal = (qlast / g.gs + 1) * g.gs;
  if (dense) return causal;
  return std::min<int64_t>(static_cast<int64_t>(g.gmax) * g.gs, causal);
}

Plan make_plan(const Geometry& g, bool dense, bool allow_split) {
  Plan pl;
  pl.units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  // Rows of the largest unit: a query chunk holds at most min(C, n_q) queries.
  const int64_t rows = std::min<int64_t>(g.C, g.n_q) * static_cast<int64_t>(g.G);
  pl.rcap = static_cast<int>(rows);
  if (g.bf16) {
    const int64_t blocks = (rows + 31) / 32;
    pl.nw = blocks >= 8 ? 8 : (blocks >= 4 ? 4 : (blocks >= 2 ? 2 : 1));
    pl.slices = static_cast<int>((blocks + pl.nw - 1) / pl.nw);
  } else {
    pl.nw = 1;
    pl.slices = static_cast<int>((rows + 63) / 64);
  }
  const int64_t wgs = pl.units * pl.slices;
  const int64_t keys = max_keys(g, dense);
  pl.splits = 1;
  pl.kps = static_cast<int>(keys);
  if (allow_split && wgs < 512 && keys > 256) {
    int64_t sp = (keys + 127) / 128;
    const int64_t want = (1024 + wgs - 1) / wgs;
    if (sp > want) sp = want;
    if (sp > 1) {
      pl.splits = static_cast<int>(sp);
      pl.kps = static_cast<int>(((keys + sp - 1) / sp + kTK - 1) / kTK * kTK);
      pl.splits = static_cast<int>((keys + pl.kps - 1) / pl.kps);
    }
  }
  return pl;
}

template <int D>
hipError_t launch_attend_d(const Geometry& g, AttendParams& p, const Plan& pl, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(pl.units * pl.slices * pl.splits);
  if (g.bf16) {
    switch (pl.nw) {
      case 8: hipLaunchKernelGGL((attend_mfma_kernel<D, 8>), dim3(grid), dim3(512), 0, stream, p); break;
      case 4: hipLaunchKernelGGL((attend_mfma_kernel<D, 4>), dim3(grid), dim3(256), 0, stream, p); break;
      case 2: hipLaunchKernelGGL((attend_mfma_kernel<D, 2>), dim3(grid), dim3(128), 0, stream, p); break;
      default: hipLaunchKernelGGL((attend_mfma_kernel<D, 1>), dim3(grid), dim3(64), 0, stream, p); break;
    }
  } else {
    hipLaunchKernelGGL((attend_f32_kernel<D>), dim3(grid), dim3(64), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  const unsigned cgrid = static_cast<unsigned>((pl.units * pl.rcap + 3) / 4);
  if (g.bf16)
    hipLaunchKernelGGL((combine_kernel<true, D>), dim3(cgrid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((combine_kernel<false, D>), dim3(cgrid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t attend_workspace(const Geometry& g, bool dense, bool allow_split) {
  const Plan pl = make_plan(g, dense, allow_split);
  if (pl.splits == 1) return 0;
  const size_t rows = static_cast<size_t>(pl.units) * pl.splits * pl.rcap;
  return rows * (static_cast<size_t>(g.d) + 2) * sizeof(float);
}

hipError_t launch_attend(const Geometry& g, const void* q, const void* k_rot, const void* v,
                         const int32_t* granules, const int32_t* granule_count, bool dense,
                         void* out, float* lse, void* ws, hipStream_t stream,
                         const AttendExtra* extra) {
  const AttendExtra none;
  const AttendExtra& ex = extra != nullptr ? *extra : none;
  const Plan pl = make_plan(g, dense, ex.allow_split);
  AttendParams p;
  p.q = q;
  p.k = k_rot;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.gran = granules;
  p.gcnt = granule_count;
  p.pool_slot = ex.pool_slot;
  p.pool_slots = ex.pool_slots;
  const size_t rows = static_cast<size_t>(pl.units) * pl.splits * pl.rcap;
  p.ws_o = static_cast<float*>(ws);
  p.ws_ml = pl.splits > 1 ? static_cast<float*>(ws) + rows * g.d : nullptr;
  p.q_pos0 = g.q_pos0;
  p.n_q = g.n_q;
  p.q_stride = ex.q_stride >= 0 ? ex.q_stride : g.n_q;
  p.q_row0 = ex.q_row0 >= 0 ? ex.q_row0 : g.q_pos0;
  p.kv_cap = g.kv_cap;
  p.t0 = g.t0;
  p.nqc = g.nqc;
  p.B = g.B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.d = g.d;
  p.C = g.C;
  p.gs = g.gs;
  p.gmax = g.gmax;
  p.Rcap = pl.rcap;
  p.nw = pl.nw;
  p.slices = pl.slices;
  p.splits = pl.splits;
  p.keys_per_split = pl.kps;
  p.dense = dense ? 1 : 0;
  p.scale_log2 = g.scale * kLog2e;
  p.rope = g.rope;
  return g.d == 128 ? launch_attend_d<128>(g, p, pl, stream) : launch_attend_d<64>(g, p, pl, stream);
}

}  // namespace hga
