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
//  * prep_kernel: D_i for every row, and Q'_i = R_i q_i * s * log2(e) as bf16
//    (the forward's query operand), row-major, into the workspace; one
//    workgroup per (sequence, query position), its RoPE table shared by the
//    query heads.
//  * dq_kernel: one workgroup per (unit, 128 rows), four waves of 32 rows,
//    over the unit's keys 32 at a time: the workgroup stages K and V of the
//    32 keys in LDS by direct global -> LDS loads; each wave forms
//    S^T = K Q'^T and dP^T = V dO^T (query rows on N, Q' and dO held in
//    registers), dS^T in registers as the B operand of dQ^T += K^T dS^T,
//    whose K^T operand comes from the K rows through the transposing LDS
//    read.  The epilogue applies R^T and writes dq.
//  * dkv_kernel: one workgroup per (unit, 128 keys of its list), eight waves
//    of 16 keys (K and V held in registers), over the unit's rows 64 at a
//    time: the workgroup stages Q' and dO of the rows in LDS by direct
//    global -> LDS loads; each wave forms S = Q' K^T and dP = dO V^T (keys on
//    N), so P and dS sit in registers as the A operands of dV += P^T dO and
//    dK~ += dS^T Q', whose B operands come from the same tiles through the
//    transposing LDS read.  A unit's sums go to a partial buffer, one row per
//    (unit, list key).
//  * list kernels: for every (sequence, KV head) and granule, the (unit,
//    list entry) pairs that hold it (counted, scanned and scattered).
//  * reduce_kernel: per 16 tokens, the sum of their partial rows (each list
//    split four ways inside the workgroup), turned by R^T for dk; tokens in
//    no list get zeros.
// P = exp2(S' - lse * log2(e)) with S' = Q' . k~, and dk~ = ln(2) sum_i dS_ij Q'_i.
#include "hga_device.h"

namespace hga {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowsWave = 32;   // rows per wave in dq_kernel (two 16-row blocks)
constexpr int kStage = 32;      // keys (dq_kernel) or rows (dkv_kernel) per LDS stage
constexpr int kKeysWG = 128;    // keys per dkv_kernel workgroup (four waves of 32)
constexpr int kDkvKT = 1;        // 16-key tiles per dkv_kernel wave
constexpr int kNoRow = -0x7fffffff - 1;  // query offset of a stage row that is not the unit's

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
  float* dk;            // [B][Hkv][kv_cap][D]
  float* dv;            // [B][Hkv][kv_cap][D]
  // workspace
  float* delta;         // [rows_total]
  uint16_t* qr;         // [rows_total][D] Q' (bf16)
  int32_t* cnt;         // [slabs][ngran] entries per granule, then scatter cursors
  int32_t* off;         // [slabs][ngran + 1] list offsets
  int32_t* list;        // [slabs][nqc * gmax] entries slot * gmax + i
  float* pk;            // [units * gmax * gs][D] dk~ per (unit, list key)
  float* pv;            // [units * gmax * gs][D] dv likewise
  int64_t q_pos0, n_q, kv_cap, t0, nqc, units, rows_total, n_tok;
  int B, Hq, Hkv, G, C, gs, lg_gs, gmax, ngran, nkb, nslice;
  float scale, scale_log2;
  RopeFreqs rope;
};

struct BUnit {
  int b, kvh, trel;
  int64_t t, qlo, slot;
  int nq, R, nkeys;
};

__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint64_t v = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The unit of (sequence, KV head) slab x and relative query chunk trel.
__device__ __forceinline__ BUnit unit_of(const BwdParams& p, int64_t x, int trel) {
  BUnit w;
  w.b = __builtin_amdgcn_readfirstlane(static_cast<int>(x / p.Hkv));
  w.kvh = __builtin_amdgcn_readfirstlane(static_cast<int>(x - static_cast<int64_t>(w.b) * p.Hkv));
  w.trel = trel;
  w.t = uni64(p.t0 + trel);
  const int64_t c0 = w.t * p.C;
  w.qlo = uni64(c0 > p.q_pos0 ? c0 : p.q_pos0);
  const int64_t qend = p.q_pos0 + p.n_q;
  const int64_t qhi = (c0 + p.C) < qend ? (c0 + p.C) : qend;
  w.nq = __builtin_amdgcn_readfirstlane(static_cast<int>(qhi - w.qlo));
  w.R = w.nq * p.G;
  w.slot = uni64(x * p.nqc + trel);
  w.nkeys = __builtin_amdgcn_readfirstlane(p.gcnt[w.slot] * p.gs);
  return w;
}

// Workgroup -> (unit, part) with all parts of a unit on one XCD (workgroups
// are dealt to the eight XCDs in turn), units largest query chunk first and
// (sequence, KV head) fastest.  Returns false past the last unit.
__device__ __forceinline__ bool map_block(const BwdParams& p, int parts, BUnit& w, int& part) {
  const uint32_t i = blockIdx.x, xcd = i & 7, j = i >> 3;
  const uint32_t v = (j / parts) * 8 + xcd;
  part = static_cast<int>(j % parts);
  if (v >= static_cast<uint64_t>(p.units)) return false;
  const uint32_t bh = static_cast<uint32_t>(p.B) * static_cast<uint32_t>(p.Hkv);
  const uint32_t q = v / bh;
  w = unit_of(p, v - q * bh, static_cast<int>(p.nqc - 1 - q));
  return true;
}

// Index of row r (counted from the unit's first query) in [B][Hq][n_q].
__device__ __forceinline__ int64_t row_index(const BwdParams& p, const BUnit& w, int r) {
  const int qi = r / p.G, hl = r - qi * p.G;
  return (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.n_q + (w.qlo + qi - p.q_pos0);
}

// D_i = dO_i . O_i and Q'_i (bf16) for every query head of one (sequence,
// query position): the position's cos/sin table is formed once in LDS, then
// each wave takes heads wave, wave + 4, ...; lane owns the pairs
// (j, j + D/2) for j = lane, lane + 64, ...
template <int D>
__global__ __launch_bounds__(256) void prep_kernel(BwdParams p) {
  constexpr int H = D / 2;
  __shared__ float2 cs[H];
  const int64_t bq = blockIdx.x;  // b * n_q + query index
  const int64_t b = bq / p.n_q, qi = bq - b * p.n_q;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const double pos = static_cast<double>(rope_base(p.rope, p.q_pos0 + qi));
  for (int j = threadIdx.x; j < H; j += 256) {
    float c, sn;
    rope_cs(pos, rope_freq(p.rope, j), c, sn);
    cs[j] = make_float2(c, sn);
  }
  __syncthreads();
  for (int h = wave; h < p.Hq; h += 4) {
    const int64_t row = (b * p.Hq + h) * p.n_q + qi;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int64_t e = row * D + lane + 64 * i;
      acc += load1<true>(p.dout, e) * load1<true>(p.out, e);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (lane == 0) p.delta[row] = acc;
    for (int j = lane; j < H; j += 64) {
      const float2 t = cs[j];
      const float a = load1<true>(p.q, row * D + j), c2 = load1<true>(p.q, row * D + j + H);
      p.qr[row * D + j] = f32_to_bf16((a * t.x - c2 * t.y) * p.scale_log2);
      p.qr[row * D + j + H] = f32_to_bf16((a * t.y + c2 * t.x) * p.scale_log2);
    }
  }
}

// Token of unit list key k (per lane), or -1 past the list.  With at most
// 128 granules per list, the list sits in two registers per lane (entries
// lane and lane + 64) and is read with lane shuffles; longer lists are read
// from memory.  Every lane must call it (a shuffle reads other lanes'
// registers, and a lane that is switched off gives no data).
struct GranList {
  int lo = -1, hi = -1;
  bool regs = false;
};

__device__ __forceinline__ GranList load_glist(const BwdParams& p, const BUnit& w) {
  GranList gl;
  gl.regs = p.gmax <= 128;
  if (gl.regs) {
    const int lane = threadIdx.x & 63;
    const int32_t* src = p.gran + w.slot * p.gmax;
    gl.lo = lane < p.gmax ? src[lane] : -1;
    gl.hi = lane + 64 < p.gmax ? src[lane + 64] : -1;
  }
  return gl;
}

__device__ __forceinline__ int token_of(const BwdParams& p, const BUnit& w, const GranList& gl, int64_t k) {
  const bool in = k < w.nkeys;
  const int gi = in ? static_cast<int>(k >> p.lg_gs) : 0;
  int g;
  if (gl.regs) {  // uniform
    const int a = __shfl(gl.lo, gi & 63), b = __shfl(gl.hi, gi & 63);
    g = gi < 64 ? a : b;
  } else {
    g = in ? p.gran[w.slot * p.gmax + gi] : -1;
  }
  return in && g >= 0 ? g * p.gs + static_cast<int>(k & (p.gs - 1)) : -1;
}

// k slots of a contraction over 32 rows of the stage (half h; slot
// 8*(lane/16) + j <-> row 32h + 16*(j/4) + 4*(lane/16) + j%4) for column
// 16c + lane%16 of a swizzled row-major tile, by two transposing LDS reads
// (ds_read_b64_tr_b16): in each group of 16 lanes, lane j reads 8 bytes of
// row base + j/4 at columns 4*(j%4) .. +3 of the 16, and lane i receives
// column i of the 4 rows.
template <int D>
__device__ __forceinline__ Pack8 ld_rowslots(const char* tile, int c, int h, int n, int sub) {
  Pack8 r;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int row = 32 * h + 16 * half + 4 * sub + (n >> 2);
    const int col = 16 * c + 4 * (n & 3);           // element column of this lane's 8 bytes
    const int off = row * (2 * D) + 16 * ((col >> 3) ^ rswz<D>(row)) + 2 * (col & 7);
    const uint2 v = lds_read_tr16(tile + off);
    r.u[2 * half] = v.x;
    r.u[2 * half + 1] = v.y;
  }
  return r;
}

// dq: stage of 32 keys in LDS, filled by direct global -> LDS loads: K and
// V rows (unswizzled order, XOR-swizzled chunks as rswz); the keys' tokens
// in a separate array.  The dQ product's K^T operand (keys in the k slots)
// comes from the K rows through the transposing LDS read.
template <int D>
struct DqStage {
  static constexpr int ROW = 2 * D;
  static constexpr int TILE = kStage * ROW;
  static constexpr int K = 0, V = TILE, BYTES = 2 * TILE;
  static constexpr int NBLK = TILE / 1024;
};

// Source of absent keys' K and V rows (their products are selected out or
// multiplied by zero, so the row must hold finite values: zeros).
__device__ __align__(16) uint4 g_zero_row[16];

template <int D>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdParams p) {
  using S = DqStage<D>;
  constexpr int KS = D / 32, H = D / 2, NT = D / 16, NW = 4;
  static_assert(S::NBLK % NW == 0, "tile blocks spread evenly over the waves");
  __shared__ __align__(1024) char b0[S::BYTES];
  __shared__ __align__(1024) char b1[S::BYTES];
  __shared__ int tok0[kStage], tok1[kStage];
  BUnit w;
  int slice;
  if (!map_block(p, p.nslice, w, slice)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, sub = lane >> 4;
  const int r0 = slice * 4 * kRowsWave + wave * kRowsWave;  // this wave's rows
  if (slice * 4 * kRowsWave >= w.R) return;  // uniform over the workgroup
  const int64_t x = static_cast<int64_t>(w.b) * p.Hkv + w.kvh;
  const char* kg = static_cast<const char*>(p.k) + x * p.kv_cap * S::ROW;
  const char* vg = static_cast<const char*>(p.v) + x * p.kv_cap * S::ROW;
  const char* zrow = reinterpret_cast<const char*>(g_zero_row);
  const GranList gl = load_glist(p, w);
  // B operands of the wave's two 16-row blocks (rows past the unit repeat
  // its last row and are dropped at the end): Q' and dO at d slots
  // ks*32 + 8*(lane/16) + i of row lane % 16, and lse*log2(e), D
  Pack8 qb[2][KS], gb[2][KS];
  float lse2[2], dl[2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    int r = r0 + sb * 16 + n;
    if (r >= w.R) r = w.R - 1;
    const int64_t ri = row_index(p, w, r);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qb[sb][ks].q = *reinterpret_cast<const uint4*>(p.qr + ri * D + ks * 32 + sub * 8);
      gb[sb][ks].q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.dout) + ri * D + ks * 32 + sub * 8);
    }
    lse2[sb] = p.lse[ri] * kLog2e;
    dl[sb] = p.delta[ri];
  }
  f32x4 acc[NT][2];
#pragma unroll
  for (int c = 0; c < NT; ++c)
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) acc[c][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Stage of list keys kb .. kb+31 into st: each wave issues its 1 KB blocks
  // of the K and V tiles (block row m = key m); a key past the list, or at
  // or after n_tok (no query sees it, and its memory may be unwritten),
  // reads the zero row and gets token -1.
  auto issue_stage = [&](int64_t kb, char* st, int* tok) {
    const int tk = token_of(p, w, gl, kb + (lane & 31));  // token of key kb + lane % 32
    const int tkv = tk < p.n_tok ? tk : -1;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // addresses formed here, not hoisted out of the loop
#pragma unroll
    for (int j = 0; j < S::NBLK / NW; ++j) {
      const int blk = (wave + j * NW) * 1024;
      const int o = blk + 16 * ln;
      const int m = o / S::ROW;
      const int c = ((o % S::ROW) / 16) ^ rswz<D>(m);
      const int t = __shfl(tkv, m);
      const int64_t e = static_cast<int64_t>(t) * S::ROW + 16 * c;
      load_lds16(t >= 0 ? kg + e : zrow + 16 * c, st + S::K + blk);
      load_lds16(t >= 0 ? vg + e : zrow + 16 * c, st + S::V + blk);
    }
    if (tid < kStage) tok[tid] = tkv;
  };
  // One stage: the next stage's loads into nxt, then S^T, dP^T, dS^T and
  // dQ^T from cur, then wait for the next stage and meet at the barrier.
  const int nst = (w.nkeys + kStage - 1) / kStage;
  auto step = [&](int s, const char* cur, const int* toks, char* nxt, int* ntok) {
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nst) issue_stage(static_cast<int64_t>(s + 1) * kStage, nxt, ntok);
    // S^T and dP^T: lane holds row lane % 16 of block sb and keys 16t + 4*(lane/16) + i
    f32x4 sv[2][2], dp[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        sv[t][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[t][sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int m = t * 16 + n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = m * S::ROW + 16 * ((ks * 4 + sub) ^ rswz<D>(m));
        Pack8 ka, va;
        ka.q = *reinterpret_cast<const uint4*>(cur + S::K + off);
        va.q = *reinterpret_cast<const uint4*>(cur + S::V + off);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          sv[t][sb] = mfma16x16x32(ka.v, qb[sb][ks].v, sv[t][sb]);
          dp[t][sb] = mfma16x16x32(va.v, gb[sb][ks].v, dp[t][sb]);
        }
      }
    }
    Pack8 dsb[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int r = r0 + sb * 16 + n;
      const bool row_ok = r < w.R;
      const int64_t qpos = w.qlo + (row_ok ? r / p.G : 0);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tk = toks[t * 16 + sub * 4 + i];
          const bool ok = row_ok && tk >= 0 && tk <= qpos;
          // selects, not products with a zero P (0 * NaN is NaN)
          const float e = ok ? exp2f(sv[t][sb][i] - lse2[sb]) : 0.f;
          dsb[sb].h[t * 4 + i] = f32_to_bf16(ok ? e * (dp[t][sb][i] - dl[sb]) : 0.f);
        }
    }
    // dQ^T[d][rows] += K^T[d][keys] dS^T[keys][rows]: A = K^T through the
    // transposing read (k slots: keys 4*(lane/16) + i, then 16 + 4*(lane/16) + i)
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const Pack8 kt_ = ld_rowslots<D>(cur + S::K, c, 0, n, sub);
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) acc[c][sb] = mfma16x16x32(kt_.v, dsb[sb].v, acc[c][sb]);
    }
    wait_vm_barrier<0>();
  };
  if (nst > 0) issue_stage(0, b0, tok0);
  wait_vm_barrier<0>();
  for (int s = 0; s < nst; s += 2) {
    step(s, b0, tok0, b1, tok1);
    if (s + 1 >= nst) break;
    step(s + 1, b1, tok1, b0, tok0);
  }
  // dq = R^T (s * dq~): lane holds d = c*16 + 4*(lane/16) + i of row r0 + sb*16 + n
  const int64_t q0 = rope_base(p.rope, w.qlo);
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int r = r0 + sb * 16 + n;
    if (r >= w.R) continue;
    const int64_t ri = row_index(p, w, r);
    const double pos = static_cast<double>(q0 + r / p.G);
#pragma unroll
    for (int c = 0; c < NT / 2; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = c * 16 + sub * 4 + i;
        float cs, sn;
        rope_cs(pos, rope_freq(p.rope, d), cs, sn);
        const float a = acc[c][sb][i] * p.scale, b = acc[c + NT / 2][sb][i] * p.scale;
        p.dq[ri * D + d] = a * cs + b * sn;
        p.dq[ri * D + d + H] = b * cs - a * sn;
      }
    }
  }
}

// dkv: stage of 64 chunk rows in LDS, filled by direct global -> LDS loads
// (a wave's lane l lands at 16*l, or 4*l, of the wave's block), so the
// tiles are unpadded and their 16-byte chunks XOR-swizzled against bank
// conflicts: Q' and dO rows (row j: 2*D bytes, chunk c at c ^ rswz(j));
// then the rows' lse, D and query offsets (RV).  The products that
// contract over rows read them with the transposing LDS read.
constexpr int kDkvRows = 64;
template <int D>
struct DkvStage {
  static constexpr int TILE = kDkvRows * D * 2;  // bytes of one tensor's tile
  static constexpr int NBLK = TILE / 1024;       // 1 KB blocks per tile
  static constexpr int QA = 0, GA = TILE, RV = 2 * TILE;
  static constexpr int BYTES = RV + 3 * 4 * kDkvRows;
};

// KT key tiles of 16 per wave, 128 / (16 KT) waves per workgroup; two stage
// buffers.
constexpr int kDkvThreads = kKeysWG / (16 * kDkvKT) * 64;
template <int D, int KT>
__global__ __launch_bounds__(kDkvThreads) void dkv_kernel(BwdParams p) {
  using S = DkvStage<D>;
  constexpr int KS = D / 32, NT = D / 16, NW = kKeysWG / (16 * KT);
  static_assert(S::NBLK % NW == 0, "tile blocks spread evenly over the waves");
  __shared__ __align__(1024) char b0[S::BYTES];
  __shared__ __align__(1024) char b1[S::BYTES];
  BUnit w;
  int kblk;
  if (!map_block(p, p.nkb, w, kblk)) return;
  if (kblk * kKeysWG >= w.nkeys || w.R == 0) return;  // uniform over the workgroup
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, sub = lane >> 4;
  const int64_t x = static_cast<int64_t>(w.b) * p.Hkv + w.kvh;
  const int64_t kw0 = static_cast<int64_t>(kblk) * kKeysWG + wave * 16 * KT;  // this wave's first list key
  const GranList gl = load_glist(p, w);
  // the wave's 16 KT keys: K and V operands (key lane % 16 of tile t, d
  // slots ks*32 + 8*(lane/16) + i) and the token of key 16t + lane % 16
  Pack8 kb[KT][KS], vb[KT][KS];
  int krel[KT];
  {
    const int tok = token_of(p, w, gl, kw0 + (lane & (16 * KT - 1)));
    const uint16_t* kg = static_cast<const uint16_t*>(p.k) + x * p.kv_cap * D;
    const uint16_t* vg = static_cast<const uint16_t*>(p.v) + x * p.kv_cap * D;
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int kt_ = __shfl(tok, t * 16 + n);
      // token relative to the chunk start (absent keys: a large value), so
      // a key is seen iff krel <= the row's query offset
      krel[t] = kt_ >= 0 ? static_cast<int>(kt_ - w.t * p.C) : (1 << 30);
      const int64_t e = static_cast<int64_t>(kt_ >= 0 ? kt_ : 0) * D + sub * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kb[t][ks].q = *reinterpret_cast<const uint4*>(kg + e + ks * 32);
        vb[t][ks].q = *reinterpret_cast<const uint4*>(vg + e + ks * 32);
      }
    }
  }
  f32x4 dka[KT][NT], dva[KT][NT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      dka[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
      dva[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // the unit's rows in its chunk-row space: row rr is query t*C + rr/G,
  // head rr % G; valid rows [lo, hi); stages of 64 from a multiple of 64
  const int lo = static_cast<int>(w.qlo - w.t * p.C) * p.G;
  const int hi = lo + w.R;
  const int rb0 = lo / kDkvRows * kDkvRows;
  const int nst = (hi - rb0 + kDkvRows - 1) / kDkvRows;
  const uint16_t* dog = static_cast<const uint16_t*>(p.dout);
  // Stage rb into st: every wave issues NBLK/NW loads per tile (blocks
  // wave + k*NW; rows that are not the unit's read row lo instead, their P
  // and dS being zero) and the loads of the rows' lse and D (all waves
  // write the same values); wave 0 writes the query offsets.
  auto issue_stage = [&](int rb, char* st) {
    // the lane index made opaque here, so that the address arithmetic is
    // redone per stage rather than hoisted out of the loop and held in
    // registers
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < S::NBLK / NW; ++k) {
      const int blk = (wave + k * NW) * 1024;
      const int o = blk + 16 * ln;
      {
        const int r = o / (2 * D), c = ((o % (2 * D)) / 16) ^ rswz<D>(r);
        int rr = rb + r;
        if (rr < lo || rr >= hi) rr = lo;
        const int64_t e = row_index(p, w, rr - lo) * D + 8 * c;
        load_lds16(p.qr + e, st + S::QA + blk);
        load_lds16(dog + e, st + S::GA + blk);
      }
    }
    {
      int rr = rb + ln;
      if (rr < lo || rr >= hi) rr = lo;
      const int64_t ri = row_index(p, w, rr - lo);
      load_lds4(p.lse + ri, st + S::RV);
      load_lds4(p.delta + ri, st + S::RV + 4 * kDkvRows);
    }
    if (tid < kDkvRows) {
      const int rr = rb + tid;
      reinterpret_cast<int*>(st + S::RV + 8 * kDkvRows)[tid] = rr >= lo && rr < hi ? rr / p.G : kNoRow;
    }
  };
  // 32 rows (half h of the stage)
  auto compute = [&](const char* st, int h) {
    // S and dP of the two 16-row blocks: lane holds key lane % 16 of tile t
    // and rows 32h + 16*sb + 4*(lane/16) + i; P and dS into the A-operand
    // slots.  The lane's row and column indices are made opaque so that the
    // LDS addresses are formed here, not hoisted (one set per buffer).
    int n = lane & 15, sub = lane >> 4;
    asm volatile("" : "+v"(n), "+v"(sub));
    Pack8 pb[KT], sk[KT];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x4 sv[KT], dp[KT];
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        sv[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const int row = 32 * h + sb * 16 + n;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = row * (2 * D) + 16 * ((ks * 4 + sub) ^ rswz<D>(row));
        Pack8 qa, ga;
        qa.q = *reinterpret_cast<const uint4*>(st + S::QA + off);
        ga.q = *reinterpret_cast<const uint4*>(st + S::GA + off);
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          sv[t] = mfma16x16x32(qa.v, kb[t][ks].v, sv[t]);
          dp[t] = mfma16x16x32(ga.v, vb[t][ks].v, dp[t]);
        }
      }
      const int r4 = 32 * h + sb * 16 + sub * 4;
      const float4 l4 = *reinterpret_cast<const float4*>(st + S::RV + 4 * r4);
      const float4 d4 = *reinterpret_cast<const float4*>(st + S::RV + 4 * (kDkvRows + r4));
      const int4 q4 = *reinterpret_cast<const int4*>(st + S::RV + 4 * (2 * kDkvRows + r4));
      const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
      const int qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const bool ok = krel[t] <= qv[i];  // rows that are not the unit's have kNoRow, below all
          // selects, not products with a zero P: a masked key's V may be
          // unwritten memory (a NaN there would survive 0 * NaN)
          const float e = ok ? exp2f(sv[t][i] - lv[i]) : 0.f;
          pb[t].h[sb * 4 + i] = f32_to_bf16(e);
          sk[t].h[sb * 4 + i] = f32_to_bf16(ok ? e * (dp[t][i] - dv4[i]) : 0.f);
        }
    }
    // dV[keys][d] += P^T[keys][rows] dO[rows][d], dK~ likewise with dS and Q'
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      const Pack8 g_ = ld_rowslots<D>(st + S::GA, c, h, n, sub);
      const Pack8 q_ = ld_rowslots<D>(st + S::QA, c, h, n, sub);
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        dva[t][c] = mfma16x16x32(pb[t].v, g_.v, dva[t][c]);
        dka[t][c] = mfma16x16x32(sk[t].v, q_.v, dka[t][c]);
      }
    }
  };
  // One stage: issue stage s + 1 into the other buffer, compute stage s,
  // wait for stage s + 1 and meet at the barrier.  The two buffers are
  // separate arrays, so the compiler sees that the reads of one do not wait
  // for the loads into the other.
  auto step = [&](int s, const char* cur, char* next) {
    __builtin_amdgcn_sched_barrier(0);  // no interleaving of one stage's work with the next
    if (s + 1 < nst) issue_stage(rb0 + (s + 1) * kDkvRows, next);
    compute(cur, 0);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur, 1);
    wait_vm_barrier<0>();
  };
  issue_stage(rb0, b0);
  wait_vm_barrier<0>();
  for (int s = 0; s < nst; s += 2) {
    step(s, b0, b1);
    if (s + 1 >= nst) break;
    step(s + 1, b1, b0);
  }
  // partial rows: lane holds d = c*16 + lane % 16 of list keys kw0 + 16t + 4*(lane/16) + i
  const int64_t prow0 = w.slot * p.gmax * p.gs;
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t k = kw0 + t * 16 + sub * 4 + i;
      if (k >= w.nkeys) continue;
      float* dkr = p.pk + (prow0 + k) * D;
      float* dvr = p.pv + (prow0 + k) * D;
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        dkr[c * 16 + n] = dka[t][c][i] * kLn2;
        dvr[c * 16 + n] = dva[t][c][i];
      }
    }
}

// Entries per granule: one count per (unit, list entry).
__global__ __launch_bounds__(256) void count_kernel(BwdParams p) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // slot * gmax + i
  if (e >= p.units * p.gmax) return;
  const int64_t slot = e / p.gmax;
  const int i = static_cast<int>(e - slot * p.gmax);
  if (i >= p.gcnt[slot]) return;
  const int g = p.gran[e];
  if (g < 0 || g >= p.ngran) return;
  const int64_t x = slot / p.nqc;
  atomicAdd(&p.cnt[x * p.ngran + g], 1);
}

// Block-wide inclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  __syncthreads();  // wsum is free
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int pre = 0;
  for (int i = 0; i < wave; ++i) pre += wsum[i];
  return v + pre;
}

// One workgroup per slab: list offsets (exclusive scan of the counts), and
// the counts cleared again to serve as scatter cursors.
__global__ __launch_bounds__(1024) void scan_kernel(BwdParams p) {
  __shared__ int wsum[16];
  __shared__ int carry;
  const int64_t x = blockIdx.x;
  int32_t* cnt = p.cnt + x * p.ngran;
  int32_t* off = p.off + x * (p.ngran + 1);
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < p.ngran; base += 1024) {
    const int g = base + tid;
    const int c = g < p.ngran ? cnt[g] : 0;
    const int c0 = carry;
    const int ex = block_scan(c, wsum) - c + c0;
    if (g < p.ngran) {
      off[g] = ex;
      cnt[g] = 0;
    }
    __syncthreads();  // every thread has read carry
    if (tid == 1023) carry = ex + c;
    __syncthreads();
  }
  if (tid == 0) off[p.ngran] = carry;
}

// Scatter: every list entry (slot * gmax + i) into its granule's list (the
// order within a list is arbitrary).
__global__ __launch_bounds__(256) void scatter_kernel(BwdParams p) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= p.units * p.gmax) return;
  const int64_t slot = e / p.gmax;
  const int i = static_cast<int>(e - slot * p.gmax);
  if (i >= p.gcnt[slot]) return;
  const int g = p.gran[e];
  if (g < 0 || g >= p.ngran) return;
  const int64_t x = slot / p.nqc;
  const int pos = atomicAdd(&p.cnt[x * p.ngran + g], 1);
  p.list[x * p.nqc * p.gmax + p.off[x * (p.ngran + 1) + g] + pos] = static_cast<int32_t>(e);
}

// dk and dv of 16 tokens of one slab, four quarters of 256 threads: thread
// (quarter, token, pair columns ((tid % 256) % 16) * PW .. + PW - 1 and their
// partners + D/2) sums every fourth partial row of its granule's list (a
// sink granule's list holds every unit of the slab); the quarters meet in
// LDS, then dk = R^T (sum).  Tokens in no list get zeros.
template <int D>
__global__ __launch_bounds__(1024) void reduce_kernel(BwdParams p) {
  constexpr int H = D / 2, PW = H / 16;
  __shared__ float4 part[3][256][PW];  // quarters 1..3: (dk lo, dk hi, dv lo, dv hi) per column
  const int64_t slabs = static_cast<int64_t>(p.B) * p.Hkv;
  const int64_t x = blockIdx.x % slabs, tb = blockIdx.x / slabs;
  const int quarter = threadIdx.x >> 8, t = threadIdx.x & 255;
  const int64_t tok = tb * 16 + (t >> 4);
  const bool tok_ok = tok < p.kv_cap;
  const int col = (t & 15) * PW;
  const int64_t g = tok >> p.lg_gs;
  int l0 = 0, l1 = 0;
  if (tok_ok && g < p.ngran) {
    l0 = p.off[x * (p.ngran + 1) + g];
    l1 = p.off[x * (p.ngran + 1) + g + 1];
  }
  const int32_t* lst = p.list + x * p.nqc * p.gmax;
  const int64_t kin = tok & (p.gs - 1);
  float ka[PW] = {}, kb_[PW] = {}, va[PW] = {}, vb_[PW] = {};
  auto add_row = [&](int32_t e) {
    const int64_t r = (static_cast<int64_t>(e) * p.gs + kin) * D + col;
#pragma unroll
    for (int j = 0; j < PW; j += 2) {
      const float2 a = *reinterpret_cast<const float2*>(p.pk + r + j);
      const float2 b = *reinterpret_cast<const float2*>(p.pk + r + H + j);
      const float2 c = *reinterpret_cast<const float2*>(p.pv + r + j);
      const float2 d = *reinterpret_cast<const float2*>(p.pv + r + H + j);
      ka[j] += a.x; ka[j + 1] += a.y;
      kb_[j] += b.x; kb_[j + 1] += b.y;
      va[j] += c.x; va[j + 1] += c.y;
      vb_[j] += d.x; vb_[j + 1] += d.y;
    }
  };
  int l = l0 + quarter;
  for (; l + 12 < l1; l += 16) {
    const int32_t e0 = lst[l], e1 = lst[l + 4], e2 = lst[l + 8], e3 = lst[l + 12];
    add_row(e0);
    add_row(e1);
    add_row(e2);
    add_row(e3);
  }
  for (; l < l1; l += 4) add_row(lst[l]);
  if (quarter > 0) {
#pragma unroll
    for (int j = 0; j < PW; ++j) part[quarter - 1][t][j] = make_float4(ka[j], kb_[j], va[j], vb_[j]);
  }
  __syncthreads();
  if (quarter > 0 || !tok_ok) return;
#pragma unroll
  for (int qq = 0; qq < 3; ++qq)
#pragma unroll
    for (int j = 0; j < PW; ++j) {
      const float4 v = part[qq][t][j];
      ka[j] += v.x;
      kb_[j] += v.y;
      va[j] += v.z;
      vb_[j] += v.w;
    }
  const double pos = static_cast<double>(rope_base(p.rope, tok));
  float* dkr = p.dk + (x * p.kv_cap + tok) * D;
  float* dvr = p.dv + (x * p.kv_cap + tok) * D;
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    float c, s;
    rope_cs(pos, rope_freq(p.rope, col + j), c, s);
    dkr[col + j] = ka[j] * c + kb_[j] * s;
    dkr[col + j + H] = kb_[j] * c - ka[j] * s;
    dvr[col + j] = va[j];
    dvr[col + j + H] = vb_[j];
  }
}

__global__ __launch_bounds__(256) void zero_i32(int32_t* x, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * 256)
    x[i] = 0;
}

// Workspace carve-up (256-byte aligned pieces).
struct BwdLayout {
  size_t delta, qr, cnt, off, list, pk, pv, total;
  int ngran;
};

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(const Geometry& g) {
  BwdLayout L;
  const size_t rows = static_cast<size_t>(g.B) * g.Hq * g.n_q;
  const size_t slabs = static_cast<size_t>(g.B) * g.Hkv;
  const size_t units = slabs * g.nqc;
  // only tokens before the last query's end are in any list (granules
  // holding a visible token), so the per-token pieces cover those: the
  // workspace depends on q_pos0 + n_q, not on kv_cap
  const int64_t n_tok = std::min<int64_t>(g.kv_cap, g.q_pos0 + g.n_q);
  L.ngran = static_cast<int>((n_tok + g.gs - 1) / g.gs);
  const size_t prow = units * g.gmax * g.gs;  // partial rows
  size_t off = 0;
  L.delta = off; off = al256(off + rows * 4);
  L.qr = off; off = al256(off + rows * g.d * 2);
  L.cnt = off; off = al256(off + slabs * L.ngran * 4);
  L.off = off; off = al256(off + slabs * (L.ngran + 1) * 4);
  L.list = off; off = al256(off + slabs * g.nqc * g.gmax * 4);
  L.pk = off; off = al256(off + prow * g.d * 4);
  L.pv = off; off = al256(off + prow * g.d * 4);
  L.total = off;
  return L;
}

template <int D>
hipError_t launch_backward_d(const Geometry& g, BwdParams& p, hipStream_t stream) {
  const int64_t slabs = static_cast<int64_t>(g.B) * g.Hkv;
  hipLaunchKernelGGL(zero_i32, dim3(256), dim3(256), 0, stream, p.cnt, slabs * p.ngran);
  hipLaunchKernelGGL((prep_kernel<D>), dim3(static_cast<unsigned>(static_cast<int64_t>(p.B) * p.n_q)), dim3(256), 0,
                     stream, p);
  const int64_t entries = p.units * p.gmax;
  const unsigned eg = static_cast<unsigned>((entries + 255) / 256);
  hipLaunchKernelGGL(count_kernel, dim3(eg), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(scan_kernel, dim3(static_cast<unsigned>(slabs)), dim3(1024), 0, stream, p);
  hipLaunchKernelGGL(scatter_kernel, dim3(eg), dim3(256), 0, stream, p);
  const int64_t units8 = (p.units + 7) / 8 * 8;
  hipLaunchKernelGGL((dq_kernel<D>), dim3(static_cast<unsigned>(units8 * p.nslice)), dim3(256), 0, stream, p);
  hipLaunchKernelGGL((dkv_kernel<D, kDkvKT>), dim3(static_cast<unsigned>(units8 * p.nkb)),
                     dim3(kDkvThreads), 0, stream, p);
  const int64_t tblocks = (p.kv_cap + 15) / 16;
  hipLaunchKernelGGL((reduce_kernel<D>), dim3(static_cast<unsigned>(slabs * tblocks)), dim3(1024), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool backward_supported(const Geometry& g) {
  // granules of at least 4 tokens (runs of 4 consecutive tokens per key
  // group of a 32-key stage); list entries (slot * gmax + i) and grid sizes
  // fit 32 bits
  const int64_t units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  const int64_t units8 = (units + 7) / 8 * 8;
  const int64_t nkb = (static_cast<int64_t>(g.gmax) * g.gs + kKeysWG - 1) / kKeysWG;
  const int64_t nslice = (static_cast<int64_t>(g.C) * g.G + 4 * kRowsWave - 1) / (4 * kRowsWave);
  const int64_t tblocks = static_cast<int64_t>(g.B) * g.Hkv * ((g.kv_cap + 15) / 16);
  const bool gs_ok = (g.gs & (g.gs - 1)) == 0 && g.gs >= 4;
  return g.bf16 && (g.d == 64 || g.d == 128) && gs_ok && units * g.gmax < (int64_t{1} << 31) &&
         units8 * nkb < (int64_t{1} << 31) && units8 * nslice < (int64_t{1} << 31) &&
         tblocks < (int64_t{1} << 31) && static_cast<int64_t>(g.B) * g.n_q < (int64_t{1} << 31);
}

size_t backward_workspace(const Geometry& g) { return bwd_layout(g).total; }

hipError_t launch_backward(const Geometry& g, const void* q, const void* k_rot, const void* v,
                           const int32_t* granules, const int32_t* granule_count, const void* out,
                           const float* lse, const void* d_out, float* dq, float* dk, float* dv,
                           void* ws, hipStream_t stream) {
  const BwdLayout L = bwd_layout(g);
  char* w = static_cast<char*>(ws);
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
  p.delta = reinterpret_cast<float*>(w + L.delta);
  p.qr = reinterpret_cast<uint16_t*>(w + L.qr);
  p.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
  p.off = reinterpret_cast<int32_t*>(w + L.off);
  p.list = reinterpret_cast<int32_t*>(w + L.list);
  p.pk = reinterpret_cast<float*>(w + L.pk);
  p.pv = reinterpret_cast<float*>(w + L.pv);
  p.q_pos0 = g.q_pos0;
  p.n_q = g.n_q;
  p.kv_cap = g.kv_cap;
  p.t0 = g.t0;
  p.nqc = g.nqc;
  p.units = static_cast<int64_t>(g.B) * g.Hkv * g.nqc;
  p.rows_total = static_cast<int64_t>(g.B) * g.Hq * g.n_q;
  p.n_tok = std::min<int64_t>(g.kv_cap, g.q_pos0 + g.n_q);
  p.B = g.B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.C = g.C;
  p.gs = g.gs;
  p.lg_gs = 0;
  while ((1 << p.lg_gs) < g.gs) ++p.lg_gs;
  p.gmax = g.gmax;
  p.ngran = L.ngran;
  p.nkb = static_cast<int>((static_cast<int64_t>(g.gmax) * g.gs + kKeysWG - 1) / kKeysWG);
  p.nslice = (g.C * g.G + 4 * kRowsWave - 1) / (4 * kRowsWave);
  p.scale = g.scale;
  p.scale_log2 = g.scale * kLog2e;
  p.rope = g.rope;
  return g.d == 128 ? launch_backward_d<128>(g, p, stream) : launch_backward_d<64>(g, p, stream);
}

}  // namespace hga
