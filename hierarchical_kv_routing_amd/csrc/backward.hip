// Backward of routed exact-token attention: gradients of the output with
// respect to the raw queries, the raw keys and the values, with the routes
// (granule lists) held fixed.
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3, exact-token output (softmax over the visible tokens only,
// Eq. (1) restricted to them); the pages train through this attention
// (Tab. 8 "Train ms").  With scale s, rotated q~_i, k~_j and the forward's
// row log-sum-exp:
//   P_ij = exp(s q~_i . k~_j - lse_i),  dP_ij = dO_i . v_j,
//   D_i = dO_i . O_i,  dS_ij = P_ij (dP_ij - D_i),
//   dq~_i = s sum_j dS_ij k~_j,  dk~_j = s sum_i dS_ij q~_i,  dv_j = sum_i P_ij dO_i,
// and dq = R_i^T dq~, dk = R_j^T dk~ (transposed RoPE turns).
//
// Kernels (bf16 operands on 16x16x32 matrix cores, f32 accumulation):
//  * delta_kernel: D_i for every row.
//  * dq_kernel: one workgroup per (unit, 128 rows), four waves of 32 rows,
//    loops over the unit's visible keys 32 at a time.  S^T = K Q'^T and
//    dP^T = V dO^T take K and V rows straight from HBM as A operands (query
//    rows on N); dS stays in registers and is directly the B operand of
//    dQ^T += K^T dS^T, whose A operand reads the wave's K rows back from
//    LDS transposed.  The epilogue applies R^T and writes dq.
//  * dkv_kernel: one workgroup per (unit, 128 keys), four waves of 32 keys,
//    loops over the unit's rows 32 at a time: the same S^T and dP^T, then P,
//    dS, the scaled queries and dO go through LDS and are read back
//    transposed for dV^T += dO^T P and dK^T += Q'^T dS (contraction over
//    rows).  The workgroup adds its keys' dk~, dv into f32 outputs with
//    atomics (a key is visible to several units).
//  * unrotate_kernel: dk = R^T dk~ in place.
// Q' = q~ * s * log2(e) rounded to bf16 (the forward's query operand), so
// P = exp2(S' - lse * log2(e)) and dk~ = ln(2) * sum_i dS_ij Q'_i.
#include "hga_device.h"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBwdRows = 32;        // rows per wave (two 16-row blocks)
constexpr int kBwdKeys = 32;        // keys per wave (two 16-key tiles)
constexpr int kBwdMaxQ = 64;        // queries per unit (C <= 64)

struct BwdParams {
  const void* q;        // [B][Hq][n_q][D] raw queries
  const void* k;        // [B][Hkv][kv_cap][D] rotated keys
  const void* v;        // [B][Hkv][kv_cap][D]
  const void* out;      // [B][Hq][n_q][D] forward output
  const float* lse;     // [B][Hq][n_q] forward log-sum-exp (natural log)
  const void* dout;     // [B][Hq][n_q][D]
  const int32_t* gran;  // [units][gmax]
  const int32_t* gcnt;  // [units]
  float* dq;            // [B][Hq][n_q][D]
  float* dk;            // [B][Hkv][kv_cap][D] (accumulated, then turned back)
  float* dv;            // [B][Hkv][kv_cap][D] (accumulated)
  float* delta;         // [B][Hq][n_q]
  int64_t q_pos0, n_q, kv_cap, t0, nqc, units, rows_total;
  int B, Hq, Hkv, G, C, gs, lg_gs, gmax;
  float scale, scale_log2;
  RopeFreqs rope;
};

struct BUnit {
  int b, kvh;
  int64_t t, qlo, slot;
  int nq, R, nkeys;
};

__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint64_t v = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Unit u (units < 2^31): (sequence, KV head) fastest, largest query chunk first.
__device__ __forceinline__ BUnit make_bunit(const BwdParams& p, int64_t u) {
  BUnit w;
  const uint32_t bh = static_cast<uint32_t>(p.B) * static_cast<uint32_t>(p.Hkv);
  const uint32_t u32 = static_cast<uint32_t>(u);
  const uint32_t q = u32 / bh;
  const uint32_t rem = u32 - q * bh;
  const int64_t trel = p.nqc - 1 - static_cast<int64_t>(q);
  const uint32_t bq = rem / static_cast<uint32_t>(p.Hkv);
  w.b = __builtin_amdgcn_readfirstlane(static_cast<int>(bq));
  w.kvh = __builtin_amdgcn_readfirstlane(static_cast<int>(rem - bq * static_cast<uint32_t>(p.Hkv)));
  w.t = uni64(p.t0 + trel);
  const int64_t c0 = w.t * p.C;
  w.qlo = uni64(c0 > p.q_pos0 ? c0 : p.q_pos0);
  const int64_t qend = p.q_pos0 + p.n_q;
  const int64_t qhi = (c0 + p.C) < qend ? (c0 + p.C) : qend;
  w.nq = __builtin_amdgcn_readfirstlane(static_cast<int>(qhi - w.qlo));
  w.R = w.nq * p.G;
  w.slot = uni64((static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.nqc + trel);
  w.nkeys = __builtin_amdgcn_readfirstlane(p.gcnt[w.slot] * p.gs);
  return w;
}

// Element offset of row r's first element in a [B][Hq][n_q][D] tensor, and
// its index in [B][Hq][n_q].
__device__ __forceinline__ int64_t row_index(const BwdParams& p, const BUnit& w, int r) {
  const int qi = r / p.G, hl = r - qi * p.G;
  return (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.n_q + (w.qlo + qi - p.q_pos0);
}

// cos / sin of the unit's queries for every pair, in LDS.
template <int H>
__device__ __forceinline__ void fill_cs(const BwdParams& p, const BUnit& w, float2* cs) {
  const int64_t q0 = rope_base(p.rope, w.qlo);
  for (int i = threadIdx.x; i < w.nq * H; i += blockDim.x) {
    const int qi = i / H, pr = i - qi * H;
    float c, s;
    rope_cs(static_cast<double>(q0 + qi), rope_freq(p.rope, pr), c, s);
    cs[i] = make_float2(c, s);
  }
}

// The B operands of a 16-row block for the S and dP products: the rotated
// queries scaled by s*log2(e) (bf16) and dO (bf16), d slots
// ks*32 + 8*(lane/16) + i of row (lane % 16); plus the row's lse*log2(e) and
// D.  Rows past R repeat row R-1 (their products are masked).
template <int D>
__device__ __forceinline__ void load_row_block(const BwdParams& p, const BUnit& w, int r0,
                                               const float2* cs, Pack8 (&qb)[D / 32],
                                               Pack8 (&gb)[D / 32], float& lse2, float& dl) {
  constexpr int KS = D / 32, H = D / 2;
  const int lane = threadIdx.x & 63, n = lane & 15, sub = lane >> 4;
  int r = r0 + n;
  if (r >= w.R) r = w.R - 1;
  const int64_t ri = row_index(p, w, r);
  float x[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    load8<true>(p.q, ri * D + ks * 32 + sub * 8, x[ks]);
    gb[ks].q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.dout) + ri * D + ks * 32 + sub * 8);
  }
  lse2 = p.lse[ri] * kLog2e;
  dl = p.delta[ri];
  const int qi = r / p.G;
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 t = cs[qi * H + ks * 32 + sub * 8 + i];
      const float a = x[ks][i], b = x[ks + KS / 2][i];
      qb[ks].h[i] = f32_to_bf16((a * t.x - b * t.y) * p.scale_log2);
      qb[ks + KS / 2].h[i] = f32_to_bf16((a * t.y + b * t.x) * p.scale_log2);
    }
  }
}

// Key kb + (lane % 32) of the unit: its token (or -1 past the list) and the
// A operands (key lane % 16 of tile t, d slots ks*32 + 8*(lane/16) + i) of K
// and V for the two 16-key tiles.
template <int D>
__device__ __forceinline__ int load_key_block(const BwdParams& p, const BUnit& w, int64_t kb,
                                              Pack8 (&ka)[2][D / 32], Pack8 (&va)[2][D / 32]) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, n = lane & 15, sub = lane >> 4;
  const int64_t k = kb + (lane & 31);
  int tok = -1;
  if (k < w.nkeys) {
    const int g = p.gran[w.slot * p.gmax + (k >> p.lg_gs)];
    tok = g >= 0 ? g * p.gs + static_cast<int>(k & (p.gs - 1)) : -1;
  }
  const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kt = __shfl(tok, t * 16 + n);
    const int64_t e = (slab + (kt >= 0 ? kt : 0)) * D + sub * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ka[t][ks].q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + e + ks * 32);
      va[t][ks].q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + e + ks * 32);
    }
  }
  return tok;
}

// P and dS of one 16-row block against the two key tiles: lane holds row
// r0 + lane%16 and keys 16t + 4*(lane/16) + i.
template <int D>
__device__ __forceinline__ void probs(const BwdParams& p, const BUnit& w, int r0, int tok,
                                      const Pack8 (&ka)[2][D / 32], const Pack8 (&va)[2][D / 32],
                                      const Pack8 (&qb)[D / 32], const Pack8 (&gb)[D / 32],
                                      float lse2, float dl, float (&pr)[2][4], float (&ds)[2][4]) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, n = lane & 15, sub = lane >> 4;
  const int r = r0 + n;
  const bool row_ok = r < w.R;
  const int64_t qpos = w.qlo + (row_ok ? r / p.G : 0);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma16x16x32(ka[t][ks].v, qb[ks].v, s);
      dp = mfma16x16x32(va[t][ks].v, gb[ks].v, dp);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kt = __shfl(tok, t * 16 + sub * 4 + i);
      const bool ok = row_ok && kt >= 0 && kt <= qpos;
      const float e = ok ? exp2f(s[i] - lse2) : 0.f;
      pr[t][i] = e;
      ds[t][i] = e * (dp[i] - dl);
    }
  }
}

// D_i = dO_i . O_i, one wave per row.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(BwdParams p) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.rows_total) return;
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const int64_t e = row * D + lane + 64 * i;
    acc += load1<true>(p.dout, e) * load1<true>(p.out, e);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) p.delta[row] = acc;
}

template <int D>
__global__ __launch_bounds__(256) void dq_kernel(BwdParams p) {
  constexpr int KS = D / 32, H = D / 2, NT = D / 16;
  constexpr int RP = D * 2 + 8;  // K row pitch in LDS (bytes)
  __shared__ float2 cs[kBwdMaxQ * H];
  __shared__ __align__(16) char kl[4][kBwdKeys * RP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, sub = lane >> 4;
  const int per = (p.C * p.G + 4 * kBwdRows - 1) / (4 * kBwdRows);  // row blocks of 128 per unit
  const int64_t u = blockIdx.x / per;
  const int blk = static_cast<int>(blockIdx.x - u * per);
  const BUnit w = make_bunit(p, u);
  const int rbase = blk * 4 * kBwdRows;
  if (rbase >= w.R) return;  // uniform
  fill_cs<H>(p, w, cs);
  __syncthreads();
  const int r0 = rbase + wave * kBwdRows;
  if (r0 >= w.R) return;  // uniform per wave; no barrier follows
  Pack8 qb[2][KS], gb[2][KS];
  float lse2[2], dl[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) load_row_block<D>(p, w, r0 + sb * 16, cs, qb[sb], gb[sb], lse2[sb], dl[sb]);
  f32x4 acc[NT][2];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) acc[c][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
  char* myk = kl[wave];
  for (int64_t kb = 0; kb < w.nkeys; kb += kBwdKeys) {
    Pack8 ka[2][KS], va[2][KS];
    const int tok = load_key_block<D>(p, w, kb, ka, va);
    // the K rows for the transposed reads (wave-local LDS)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        char* dst = myk + (t * 16 + n) * RP + (ks * 32 + sub * 8) * 2;
        *reinterpret_cast<uint2*>(dst) = make_uint2(ka[t][ks].u[0], ka[t][ks].u[1]);
        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(ka[t][ks].u[2], ka[t][ks].u[3]);
      }
    Pack8 dsb[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      float pr[2][4], ds[2][4];
      probs<D>(p, w, r0 + sb * 16, tok, ka, va, qb[sb], gb[sb], lse2[sb], dl[sb], pr, ds);
      // k slots: keys 4*sub + i (tile 0), then 16 + 4*sub + i (tile 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dsb[sb].h[i] = f32_to_bf16(ds[0][i]);
        dsb[sb].h[4 + i] = f32_to_bf16(ds[1][i]);
      }
    }
    // dQ^T[d][rows] += K^T[d][keys] dS^T[keys][rows]
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      Pack8 kt;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kt.h[i] = *reinterpret_cast<const uint16_t*>(myk + (sub * 4 + i) * RP + (c * 16 + n) * 2);
        kt.h[4 + i] = *reinterpret_cast<const uint16_t*>(myk + (16 + sub * 4 + i) * RP + (c * 16 + n) * 2);
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) acc[c][sb] = mfma16x16x32(kt.v, dsb[sb].v, acc[c][sb]);
    }
  }
  // dq = R^T (s * dq~): lane holds d = c*16 + 4*(lane/16) + i of row r0 + sb*16 + n
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int r = r0 + sb * 16 + n;
    if (r >= w.R) continue;
    const int64_t ri = row_index(p, w, r);
    const int qi = r / p.G;
#pragma unroll
    for (int c = 0; c < NT / 2; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = c * 16 + sub * 4 + i;
        const float2 t = cs[qi * H + d];
        const float a = acc[c][sb][i] * p.scale, b = acc[c + NT / 2][sb][i] * p.scale;
        p.dq[ri * D + d] = a * t.x + b * t.y;
        p.dq[ri * D + d + H] = b * t.x - a * t.y;
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void dkv_kernel(BwdParams p) {
  constexpr int KS = D / 32, H = D / 2, NT = D / 16;
  constexpr int RP = D * 2 + 8;              // q' / dO row pitch in LDS (bytes)
  constexpr int PP = kBwdKeys * 2 + 8;       // P / dS row pitch in LDS (bytes)
  __shared__ float2 cs[kBwdMaxQ * H];
  __shared__ __align__(16) char ql[4][kBwdRows * RP];
  __shared__ __align__(16) char gl[4][kBwdRows * RP];
  __shared__ __align__(16) char pl[4][kBwdRows * PP];
  __shared__ __align__(16) char sl[4][kBwdRows * PP];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, sub = lane >> 4;
  const int per = (p.gmax * p.gs + 4 * kBwdKeys - 1) / (4 * kBwdKeys);  // key blocks of 128 per unit
  const int64_t u = blockIdx.x / per;
  const int blk = static_cast<int>(blockIdx.x - u * per);
  const BUnit w = make_bunit(p, u);
  const int64_t kbase = static_cast<int64_t>(blk) * 4 * kBwdKeys;
  if (kbase >= w.nkeys) return;  // uniform
  fill_cs<H>(p, w, cs);
  __syncthreads();
  const int64_t kb = kbase + wave * kBwdKeys;
  if (kb >= w.nkeys) return;  // uniform per wave; no barrier follows
  Pack8 ka[2][KS], va[2][KS];
  const int tok = load_key_block<D>(p, w, kb, ka, va);
  f32x4 dka[NT][2], dva[NT][2];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      dka[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
      dva[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  char* myq = ql[wave];
  char* myg = gl[wave];
  char* myp = pl[wave];
  char* mys = sl[wave];
  for (int r0 = 0; r0 < w.R; r0 += kBwdRows) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      Pack8 qb[KS], gb[KS];
      float lse2, dl;
      load_row_block<D>(p, w, r0 + sb * 16, cs, qb, gb, lse2, dl);
      float pr[2][4], ds[2][4];
      probs<D>(p, w, r0 + sb * 16, tok, ka, va, qb, gb, lse2, dl, pr, ds);
      // rows sb*16 + n of the wave's LDS tiles
      const int row = sb * 16 + n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        char* dq_ = myq + row * RP + (ks * 32 + sub * 8) * 2;
        char* dg_ = myg + row * RP + (ks * 32 + sub * 8) * 2;
        *reinterpret_cast<uint2*>(dq_) = make_uint2(qb[ks].u[0], qb[ks].u[1]);
        *reinterpret_cast<uint2*>(dq_ + 8) = make_uint2(qb[ks].u[2], qb[ks].u[3]);
        *reinterpret_cast<uint2*>(dg_) = make_uint2(gb[ks].u[0], gb[ks].u[1]);
        *reinterpret_cast<uint2*>(dg_ + 8) = make_uint2(gb[ks].u[2], gb[ks].u[3]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        Pack8 pk, sk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk.h[i] = f32_to_bf16(pr[t][i]);
          sk.h[i] = f32_to_bf16(ds[t][i]);
        }
        *reinterpret_cast<uint2*>(myp + row * PP + (t * 16 + sub * 4) * 2) = make_uint2(pk.u[0], pk.u[1]);
        *reinterpret_cast<uint2*>(mys + row * PP + (t * 16 + sub * 4) * 2) = make_uint2(sk.u[0], sk.u[1]);
      }
    }
    // dV^T[d][keys] += dO^T[d][rows] P[rows][keys]; dK^T likewise with Q', dS
    // (k slots: rows 8*(lane/16) + i of the 32)
    Pack8 pb[2], sbk[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = sub * 8 + i;
        pb[t].h[i] = *reinterpret_cast<const uint16_t*>(myp + row * PP + (t * 16 + n) * 2);
        sbk[t].h[i] = *reinterpret_cast<const uint16_t*>(mys + row * PP + (t * 16 + n) * 2);
      }
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      Pack8 ga, qa;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = sub * 8 + i;
        ga.h[i] = *reinterpret_cast<const uint16_t*>(myg + row * RP + (c * 16 + n) * 2);
        qa.h[i] = *reinterpret_cast<const uint16_t*>(myq + row * RP + (c * 16 + n) * 2);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        dva[c][t] = mfma16x16x32(ga.v, pb[t].v, dva[c][t]);
        dka[c][t] = mfma16x16x32(qa.v, sbk[t].v, dka[c][t]);
      }
    }
  }
  // lane holds key kb + 16t + n and d = c*16 + 4*(lane/16) + i
  const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kt = __shfl(tok, t * 16 + n);
    if (kt < 0) continue;
    float* dkr = p.dk + (slab + kt) * D;
    float* dvr = p.dv + (slab + kt) * D;
#pragma unroll
    for (int c = 0; c < NT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = c * 16 + sub * 4 + i;
        unsafeAtomicAdd(dkr + d, dka[c][t][i] * kLn2);
        unsafeAtomicAdd(dvr + d, dva[c][t][i]);
      }
  }
}

// dk = R_j^T dk~ in place for tokens [0, n_tok) of every (sequence, KV head).
template <int D>
__global__ __launch_bounds__(256) void unrotate_kernel(BwdParams p, int64_t n_tok) {
  constexpr int H = D / 2;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (slab row, pair)
  const int64_t total = static_cast<int64_t>(p.B) * p.Hkv * n_tok * H;
  if (i >= total) return;
  const int pr = static_cast<int>(i % H);
  const int64_t rowi = i / H;
  const int64_t j = rowi % n_tok;
  const int64_t bh = rowi / n_tok;
  float* x = p.dk + (bh * p.kv_cap + j) * D;
  float c, s;
  rope_cs(static_cast<double>(rope_base(p.rope, j)), rope_freq(p.rope, pr), c, s);
  const float a = x[pr], b = x[pr + H];
  x[pr] = a * c + b * s;
  x[pr + H] = b * c - a * s;
}

__global__ __launch_bounds__(256) void zero_kernel(float4* x, int64_t n4) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<int64_t>(gridDim.x) * 256)
    x[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int D>
hipError_t launch_backward_d(const Geometry& g, BwdParams& p, hipStream_t stream) {
  // dk and dv are accumulated (hardware f32 atomics on device memory): clear
  // them first (a kernel, not a memset)
  const int64_t n4 = static_cast<int64_t>(g.B) * g.Hkv * g.kv_cap * D / 4;
  hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dk), n4);
  hipLaunchKernelGGL(zero_kernel, dim3(2048), dim3(256), 0, stream, reinterpret_cast<float4*>(p.dv), n4);
  hipLaunchKernelGGL((delta_kernel<D>), dim3(static_cast<unsigned>((p.rows_total + 3) / 4)), dim3(256), 0,
                     stream, p);
  const int per_q = (g.C * g.G + 4 * kBwdRows - 1) / (4 * kBwdRows);
  hipLaunchKernelGGL((dq_kernel<D>), dim3(static_cast<unsigned>(p.units * per_q)), dim3(256), 0, stream, p);
  const int per_k = (g.gmax * g.gs + 4 * kBwdKeys - 1) / (4 * kBwdKeys);
  hipLaunchKernelGGL((dkv_kernel<D>), dim3(static_cast<unsigned>(p.units * per_k)), dim3(256), 0, stream, p);
  const int64_t n_tok = std::min<int64_t>(g.kv_cap, g.q_pos0 + g.n_q);
  const int64_t total = static_cast<int64_t>(g.B) * g.Hkv * n_tok * (D / 2);
  hipLaunchKernelGGL((unrotate_kernel<D>), dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                     stream, p, n_tok);
  return hipGetLastError();
}

}  // namespace

bool backward_supported(const Geometry& g) {
  return g.bf16 && (g.d == 64 || g.d == 128) && g.C <= kBwdMaxQ && (g.gs & (g.gs - 1)) == 0 &&
         g.gs >= 1;
}

size_t backward_workspace(const Geometry& g) {
  return static_cast<size_t>(g.B) * g.Hq * g.n_q * sizeof(float);
}

hipError_t launch_backward(const Geometry& g, const void* q, const void* k_rot, const void* v,
                           const int32_t* granules, const int32_t* granule_count, const void* out,
                           const float* lse, const void* d_out, float* dq, float* dk, float* dv,
                           void* ws, hipStream_t stream) {
  BwdParams p;
  p.q = q;
  p.k = k_rot;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.dout = d_out;
  p.gran = granules;
  p.gcnt = granule_count;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = static_cast<float*>(ws);
  p.q_pos0 = g.q_pos0;
  p.n_q = g.n_q;
  p.kv_cap = g.kv_cap;
  p.t0 = g.t0;
  p.nqc = g.nqc;
  p.units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  p.rows_total = static_cast<int64_t>(g.B) * g.Hq * g.n_q;
  p.B = g.B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.C = g.C;
  p.gs = g.gs;
  p.lg_gs = 0;
  while ((1 << p.lg_gs) < g.gs) ++p.lg_gs;
  p.gmax = g.gmax;
  p.scale = g.scale;
  p.scale_log2 = g.scale * kLog2e;
  p.rope = g.rope;
  return g.d == 128 ? launch_backward_d<128>(g, p, stream) : launch_backward_d<64>(g, p, stream);
}

}  // namespace hga
