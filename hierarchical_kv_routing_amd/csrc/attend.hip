// Exact-token attention over each unit's visible granules (routed) or over
// every key j <= i (dense causal, Eq. 1).
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3: exact-token output (softmax over the real token K/V of the
// current chunk's causal part, the fixed windows and the routed groups or
// chunks, with no summary tokens) and Eq. (1) (dense causal attention).
//
// bf16 path (attend_mfma_kernel): a workgroup holds NW waves, each with RB
// (= 1) blocks of 32 query rows of one unit (sequence, KV head, query chunk); a
// row is (query, head) with the G query heads of the KV head interleaved, so
// all GQA heads share every K/V stage.  Stages of 64 gathered tokens are
// staged in LDS (K row-major, V transposed, written as packed key pairs) and
// double-buffered from registers.  Per 32-key sub-tile each wave computes
//   S^T = K Q^T      (32x32x16 bf16 MFMA, keys on M, query rows on N)
//   softmax          (f32, base 2, Q pre-scaled by scale*log2(e))
//   O^T += V^T P^T   (32x32x16 bf16 MFMA, P rounded to bf16)
// With rows on N each lane owns one row.  MFMA row m of K is key pi(m)
// (bits 2 and 3 of m swapped), which makes the S^T accumulator registers of
// a lane cover exactly the 8 consecutive keys the PV product wants from it:
// P never goes through LDS.  The permutation is applied when K is stored
// (LDS row pi(s) holds key s), so the MFMA reads consecutive LDS rows and
// both LDS reads and writes are free of bank conflicts.
//
// Softmax keeps a per-row reference r and accumulates 2^(s - r): r moves
// only when a stage's scores exceed it by more than 2^8 (a wave-uniform
// branch), so the common stage does one subtraction, one exp2, one max and
// one add per score.  Row sums stay lane-local until the end.  Causal /
// validity masks are evaluated only in stages that hold current-chunk or
// out-of-range keys.  Few-unit calls (decode) split each unit's keys over
// several workgroups and merge (m, l, O) partials in combine_kernel.
//
// f32 path (attend_f32_kernel): four waves per 64 rows, four lanes per row
// (each owns a quarter of d), K/V tiles in LDS, f32 vector ALU; a score is
// the sum of the row's four lane partials; exact to f32 rounding.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include <type_traits>

#include "hga_device.h"

// Scratch of hga_attend_noalloc (the split-key partials of few-unit calls),
// for callers that cannot allocate device memory.  Each device the library
// runs on holds its own copy until the process ends; host code reaches it
// only through the address hipGetSymbolAddress returns for the current
// device (attend_noalloc_scratch), never through the name.
static __device__ __align__(256) char scratch[hga::kNoAllocScratchBytes];

namespace hga {
namespace {


constexpr int kTK = 64;                // keys per LDS stage (bf16 path)
constexpr int kTab = kAttendTable;     // granule-table entries per work item (bf16 path)
constexpr int kVP = kTK * 2 + 16;      // bytes per transposed V row in LDS
constexpr int kTKf = 32;               // keys per LDS tile (f32 path)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSum = 4096.0f;
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f}; // move the reference when a lane's half sum exceeds 2^12

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
  int64_t q_pos0, n_q, kv_cap, t0, nqc, units;
  // q / out / lse rows: row r of a (sequence, head) holds position q_row0 + r
  // and rows are q_stride apart (a window call covers part of the array).
  int64_t q_stride, q_row0;
  int B, Hq, Hkv, G, d, C, gs, lg_gs, gmax, Rcap;
  int slices, splits, keys_per_split, per_unit;
  int64_t nblocks;  // work items (bx) of the launch; a workgroup takes bx = blockIdx.x + k*gridDim.x
  int dense;
  int all_splits;   // every split wrote its partial (decode kernel)
  float scale_log2;
  RopeFreqs rope;
};

struct AUnit {
  int b, kvh;
  int64_t t, qlo, slot;
  int nq, R, nkeys;
};

__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t v = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The unit's fields as scalars (the same on every lane of the block).
__device__ __forceinline__ AUnit uniform_unit(const AUnit& a) {
  AUnit w;
  w.b = __builtin_amdgcn_readfirstlane(a.b);
  w.kvh = __builtin_amdgcn_readfirstlane(a.kvh);
  w.t = uniform64(a.t);
  w.qlo = uniform64(a.qlo);
  w.slot = uniform64(a.slot);
  w.nq = __builtin_amdgcn_readfirstlane(a.nq);
  w.R = __builtin_amdgcn_readfirstlane(a.R);
  w.nkeys = __builtin_amdgcn_readfirstlane(a.nkeys);
  return w;
}

// Unit u (largest query chunk first, (sequence, KV head) fastest).  With
// count = false the routed key count is left unread (nkeys = 0).
__device__ __forceinline__ AUnit make_aunit(const AttendParams& p, int64_t u, bool count = true) {
  AUnit w;
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
  w.slot = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.nqc + trel;
  if (p.dense) {
    w.nkeys = static_cast<int>(((qhi - 1) / p.gs + 1) * p.gs);
  } else {
    w.nkeys = count ? p.gcnt[w.slot] * p.gs : 0;
  }
  return w;
}

// Work item of this block.  Units are taken 8 at a time, one per XCD
// (consecutive blocks go to consecutive XCDs), and every item (row slice x
// key split) of a unit lands on the same XCD, whose L2 then serves the
// unit's K/V to all of them.
__device__ __forceinline__ bool block_item(const AttendParams& p, int64_t bx, int64_t& u, int& item) {
  const int64_t per = 8 * static_cast<int64_t>(p.per_unit);
  const int64_t grp = bx / per;
  const int rem = static_cast<int>(bx - grp * per);
  item = rem >> 3;
  u = grp * 8 + (rem & 7);
  return u < p.units;
}

// Token held by key slot s of a unit (slot order = ascending granules), or
// -1 when a caller-supplied granule id lies outside [0, kv_cap / g_s) (or,
// in pool mode, its pool slot lies outside the pool).
__device__ __forceinline__ int slot_token(const AttendParams& p, const AUnit& w, int s) {
  if (p.dense) return s;
  const int gi = s >> p.lg_gs;
  const int64_t g = p.gran[w.slot * p.gmax + gi];
  if (p.pool_slot != nullptr) {
    const int64_t ps = p.pool_slot[w.slot * p.gmax + gi];
    if (ps < 0 || ps >= p.pool_slots) return -1;
  }
  const int64_t tok = (g << p.lg_gs) + (s & ((1 << p.lg_gs) - 1));
  return (tok >= 0 && tok < p.kv_cap) ? static_cast<int>(tok) : -1;
}

// Element offsets (from p.k and p.v) of the K and V rows of key slot s
// holding token tok.
template <int D>
__device__ __forceinline__ void kv_offsets(const AttendParams& p, const AUnit& w, int s, int tok,
                                           int64_t slab, int64_t& ko, int64_t& vo) {
  if (p.pool_slot != nullptr) {
    const int gi = s >> p.lg_gs;
    const int64_t ps = p.pool_slot[w.slot * p.gmax + gi];
    ko = ((ps << (p.lg_gs + 1)) + (s & ((1 << p.lg_gs) - 1))) * D;
    vo = ko + (static_cast<int64_t>(1) << p.lg_gs) * D;
  } else {
    ko = vo = (slab + tok) * D;
  }
}

// K row index read by MFMA row m: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int perm_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// One 64-key stage in registers: thread item = (key pair, 16-byte d slice).
template <int D, int NW>
struct StageRegs {
  static constexpr int SL = D / 8;
  static constexpr int kItems = (kTK / 2) * SL;
  static constexpr int kPer = (kItems + NW * 64 - 1) / (NW * 64);
  uint4 k0[kPer], k1[kPer], v0[kPer], v1[kPer];
  int t0[kPer], t1[kPer];
};

// Buffer resource over `bytes` bytes from `base`: a load whose offset is
// at or beyond `bytes` returns zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}
constexpr uint32_t kNoRow = 0x80000000u;  // beyond every K/V buffer (their sizes stay below 2^31)

// 16 bytes at byte offset off of a K or V buffer resource (zero when off is
// kNoRow).
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Item i of a stage covers one key pair and one 16-byte d slice.  K items
// run slice-fastest (a half wave reads whole 256-byte rows); V items run
// key-pair-fastest so that the transposed LDS stores of a wave land in 64
// distinct banks.  gtab holds the work item's granules from granule gfirst on
// (entry: row of the granule's first key in the K/V resource, its first
// token; -1 when invalid).  A key past kend or in an invalid granule gets
// offset kNoRow (zeros) and token -1.  No branches: the stage's first key kb
// is a multiple of g_s, so a key's table entry is the stage's first entry
// plus a per-thread constant.
//
// fast (a uniform flag): every key of the stage is valid and before the
// current chunk, and g_s >= 2, so the two keys of a pair share a granule.
// Then a thread reads one table entry for its K pair and one for its V
// pair, forms the offsets without any validity test, and leaves the token
// slots unset (only masked stages read tokens, and those are never fast).
template <int D, int NW>
__device__ __forceinline__ void load_stage(const AttendParams& p, __amdgpu_buffer_rsrc_t kr,
                                           __amdgpu_buffer_rsrc_t vr, const int2* gtab, int gfirst,
                                           int kb, int kend, int qend, bool fast, StageRegs<D, NW>& r) {
  constexpr int SL = StageRegs<D, NW>::SL;
  const int lg = p.lg_gs, gm = (1 << lg) - 1;
  const int gbase = (kb >> lg) - gfirst;
  if (fast) {
    const int* gx = reinterpret_cast<const int*>(gtab) + 2 * gbase;
#pragma unroll
    for (int i = 0; i < StageRegs<D, NW>::kPer; ++i) {
      const int idx = threadIdx.x + i * NW * 64;
      if (idx < StageRegs<D, NW>::kItems) {
        const int kpk = idx / SL, slk = idx - kpk * SL;
        const int kpv = idx & 31, slv = idx >> 5;
        const int ek = gx[2 * ((2 * kpk) >> lg)];
        const int ev = gx[2 * ((2 * kpv) >> lg)];
        const uint32_t ok = static_cast<uint32_t>(ek + ((2 * kpk) & gm)) * (D * 2) + slk * 16;
        const uint32_t ov = static_cast<uint32_t>(ev + ((2 * kpv) & gm)) * (D * 2) + slv * 16;
        r.k0[i] = load16(kr, ok);
        r.k1[i] = load16(kr, ok + D * 2);
        r.v0[i] = load16(vr, ov);
        r.v1[i] = load16(vr, ov + D * 2);
        r.t0[i] = r.t1[i] = 0;
      }
    }
    return;
  }
  const int rem = kend - kb;  // keys of the stage before kend
  // Table entries as single 64-bit LDS reads, all issued before any is used.
  auto entry = [&](int s) {
    int gi = gbase + (s >> lg);
    gi = gi < kTab - 1 ? gi : kTab - 1;  // keys past kend may point past the table
    return *reinterpret_cast<const unsigned long long*>(gtab + gi);
  };
  // A key is absent (zeros, token -1) past the list, in an empty entry, or
  // at or past qend (after the unit's last query: no row sees it, and its
  // memory need not have been written).
  auto key = [&](int s, unsigned long long ev, int sl, uint32_t& off, int& tok) {
    const int ex = static_cast<int>(static_cast<uint32_t>(ev));
    const int ey = static_cast<int>(static_cast<uint32_t>(ev >> 32));
    const int t = ey + (s & gm);
    const bool ok = (s < rem) & (ex >= 0) & (t < qend);
    off = ok ? static_cast<uint32_t>(ex + (s & gm)) * (D * 2) + sl * 16 : kNoRow;
    tok = ok ? t : -1;
  };
#pragma unroll
  for (int i = 0; i < StageRegs<D, NW>::kPer; ++i) {
    const int idx = threadIdx.x + i * NW * 64;
    if (idx < StageRegs<D, NW>::kItems) {
      const int kpk = idx / SL, slk = idx - kpk * SL;
      const int kpv = idx & 31, slv = idx >> 5;
      const unsigned long long k0 = entry(2 * kpk), k1 = entry(2 * kpk + 1);
      const unsigned long long v0 = entry(2 * kpv), v1 = entry(2 * kpv + 1);
      uint32_t o0, o1;
      key(2 * kpk, k0, slk, o0, r.t0[i]);
      key(2 * kpk + 1, k1, slk, o1, r.t1[i]);
      r.k0[i] = load16(kr, o0);
      r.k1[i] = load16(kr, o1);
      int u0, u1;
      key(2 * kpv, v0, slv, o0, u0);
      key(2 * kpv + 1, v1, slv, o1, u1);
      r.v0[i] = load16(vr, o0);
      r.v1[i] = load16(vr, o1);
    }
  }
}

template <int D, int NW>
__device__ __forceinline__ void store_stage(const StageRegs<D, NW>& r, char* kl, char* vl, int* tl) {
  constexpr int SL = StageRegs<D, NW>::SL;
  constexpr int KP = D * 2 + 16;
#pragma unroll
  for (int i = 0; i < StageRegs<D, NW>::kPer; ++i) {
    const int idx = threadIdx.x + i * NW * 64;
    if (idx < StageRegs<D, NW>::kItems) {
      int kp = idx / SL, sl = idx - kp * SL;
      // K row of key s goes to LDS row pi(s), so MFMA row m reads LDS row m
      *reinterpret_cast<uint4*>(kl + perm_row(2 * kp) * KP + sl * 16) = r.k0[i];
      *reinterpret_cast<uint4*>(kl + perm_row(2 * kp + 1) * KP + sl * 16) = r.k1[i];
      if (sl == 0) {
        tl[2 * kp] = r.t0[i];
        tl[2 * kp + 1] = r.t1[i];
      }
      kp = idx & 31;
      sl = idx >> 5;
      const uint32_t x[4] = {r.v0[i].x, r.v0[i].y, r.v0[i].z, r.v0[i].w};
      const uint32_t y[4] = {r.v1[i].x, r.v1[i].y, r.v1[i].z, r.v1[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // element d of keys (2kp, 2kp+1) packed as one 32-bit LDS word
        const uint32_t lo = __builtin_amdgcn_perm(y[e], x[e], 0x05040100u);  // low halves
        const uint32_t hi = __builtin_amdgcn_perm(y[e], x[e], 0x07060302u);  // high halves
        *reinterpret_cast<uint32_t*>(vl + (sl * 8 + 2 * e) * kVP + kp * 4) = lo;
        *reinterpret_cast<uint32_t*>(vl + (sl * 8 + 2 * e + 1) * kVP + kp * 4) = hi;
      }
    }
  }
}

template <int D>
constexpr int stage_bytes() {
  return kTK * (D * 2 + 16) + D * kVP + kTK * 4;
}

// 2^x of the 16 scores of a half (x already relative to the reference):
// P as bf16 MFMA operands (pb[0]: keys 0..15, pb[1]: keys 16..31) and the
// lane's partial row sum of those bf16 values.
__device__ __forceinline__ float exp_pack(const f32x16& s, Pack8 (&pb)[2]) {
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const float e0 = __builtin_amdgcn_exp2f(s[j]);
    const float e1 = __builtin_amdgcn_exp2f(s[j + 1]);
    const f32x2 f = {e0, e1};
    const bf16x2 pk = __builtin_convertvector(f, bf16x2);
    pb[j >> 3].u[(j & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
    ps = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes2, ps, false);
  }
  return ps;
}

// Softmax of one 32-key half for one row, in pieces that sit between
// matrix-core products: s[j] holds the score of key 16*(j/8) + 8*hsub + (j%8)
// of the half (tokens tl[] when masked).  sm_pair handles elements j and
// j+1 (j even): the mask, s - ref, 2^x, the pair's bf16 P operand and the
// lane's partial row sum (a dot product of the bf16 pair with (1, 1), so the
// sum is the one of the P the products use).  sm_post: the reference moves
// (and o, lsum are rescaled) only when a lane's sum of the half's terms
// exceeds 2^12 (every term is then bounded by 2^12), a wave-uniform branch
// taken rarely; the common case costs one compare per half instead of a
// running maximum.  Then the half's sum joins the row sum.
template <bool MASKED>
__device__ __forceinline__ void sm_pair(f32x16& s, int j, const int* tl, int hsub, int cur0, int qpos,
                                        float ref, float& ps, Pack8 (&pb)[2]) {
  float x0 = s[j], x1 = s[j + 1];
  if constexpr (MASKED) {
    const int t0 = tl[16 * (j >> 3) + 8 * hsub + (j & 7)];
    const int t1 = tl[16 * ((j + 1) >> 3) + 8 * hsub + ((j + 1) & 7)];
    x0 = ((t0 >= 0) & ((t0 < cur0) | (t0 <= qpos))) ? x0 - ref : -INFINITY;
    x1 = ((t1 >= 0) & ((t1 < cur0) | (t1 <= qpos))) ? x1 - ref : -INFINITY;
  } else {
    x0 -= ref;
    x1 -= ref;
  }
  s[j] = x0;
  s[j + 1] = x1;
  const float e0 = __builtin_amdgcn_exp2f(x0);
  const float e1 = __builtin_amdgcn_exp2f(x1);
  const f32x2 f = {e0, e1};
  const bf16x2 pk = __builtin_convertvector(f, bf16x2);
  pb[j >> 3].u[(j & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
  ps = __builtin_amdgcn_fdot2_f32_bf16(pk, kOnes2, ps, false);
}

template <int DB>
__device__ __forceinline__ void sm_post(f32x16& s, float ps, float& ref, float& lsum, bool& started,
                                        f32x16 (&o)[DB], Pack8 (&pb)[2]) {
  if (__builtin_amdgcn_ballot_w64(!started || ps > kRescaleSum) != 0) {  // wave-uniform, rare
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[j]);
    const float mrow = fmaxf(mx, __shfl_xor(mx, 32));
    float delta = 0.f;
    if (!started) {
      if (mrow > -INFINITY) {
        delta = mrow;
        started = true;
      }
    } else if (mrow > 0.f) {
      delta = mrow;
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
    }
    if (delta != 0.f) {
      ref += delta;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] -= delta;
      ps = exp_pack(s, pb);
    }
  }
  lsum += ps;
}

template <int D>
constexpr int attend_main_bytes() {
  return (2 * stage_bytes<D>()) > (64 * (D / 2) * 8) ? (2 * stage_bytes<D>()) : (64 * (D / 2) * 8);
}

// One work item bx: a row slice and key split of one unit.
template <int D, int NW, int RB, bool POOL>
__device__ __forceinline__ void attend_item(const AttendParams& p, int64_t bx, char* smem) {
  constexpr int KS = D / 16;    // k-steps of S^T over d
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int KP = D * 2 + 16;
  constexpr int SB = stage_bytes<D>();
  constexpr int H = D / 2;
  constexpr int kMain = attend_main_bytes<D>();
  constexpr int kRows = NW * 32 * RB;

  int64_t u;
  int item;
  if (!block_item(p, bx, u, item)) return;  // uniform
  const int slice = item / p.splits;
  const int split = item - slice * p.splits;
  const AUnit w = uniform_unit(make_aunit(p, u));
  const int r0 = slice * kRows;
  if (r0 >= w.R) return;  // uniform
  const int kbeg = split * p.keys_per_split;
  int kend = kbeg + p.keys_per_split;
  if (kend > w.nkeys) kend = w.nkeys;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;

  // Query rows: lane -> row n = lane % 32 of each row block, d slots
  // ks*16 + 8*(lane/32) + i.  Their loads are issued first, so that they are
  // in flight while the granule and RoPE tables are built.
  const int n = lane & 31, hsub = lane >> 5;
  const int cur0 = static_cast<int>(w.t * p.C);
  const int qend = static_cast<int>(w.qlo + w.nq);  // past the unit's last query
  const int q_first = r0 / p.G;
  Pack8 qraw[RB][KS];
  int qpos[RB], hl[RB], row[RB];
  bool rb_on[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    row[rb] = r0 + (wave * RB + rb) * 32 + n;
    rb_on[rb] = (r0 + (wave * RB + rb) * 32) < w.R;
    const bool ok = row[rb] < w.R;
    const int qloc = ok ? row[rb] / p.G : q_first;
    hl[rb] = ok ? row[rb] - qloc * p.G : 0;
    qpos[rb] = static_cast<int>(w.qlo) + qloc;
    const int64_t base =
        ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl[rb]) * p.q_stride + (qpos[rb] - p.q_row0)) * D;
    const uint16_t* qsrc = static_cast<const uint16_t*>(p.q) + base + hsub * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[rb][ks].q = ok ? *reinterpret_cast<const uint4*>(qsrc + ks * 16) : make_uint4(0, 0, 0, 0);
  }

  // Granule table of the item's key range (rows and tokens of each granule's
  // first key), read once so that stage loads need no dependent global load.
  // Each wave also finds its first table entry that is absent or in the
  // current chunk (wfb[wave]): tokens ascend along a list, so every key
  // before the first such entry (and before kend) is valid and unmasked.
  int2* gtab = reinterpret_cast<int2*>(smem + kMain);
  int* wfb = reinterpret_cast<int*>(smem + kMain + kTab * 8);
  const int gfirst = kbeg >> p.lg_gs;
  int fb = kTab;
  if (kend > kbeg) {
    const int ng = ((kend - 1) >> p.lg_gs) - gfirst + 1;  // <= kTab (make_plan)
    const int64_t gcap = p.kv_cap >> p.lg_gs;
    for (int i = threadIdx.x; i < ng; i += NW * 64) {
      const int64_t e = w.slot * p.gmax + gfirst + i;
      const int64_t g = p.dense ? gfirst + i : p.gran[e];  // dense: every granule in order
      int2 t = make_int2(-1, -1);
      if (g >= 0 && g < gcap) {
        const int tok = static_cast<int>(g << p.lg_gs);
        if constexpr (POOL) {
          const int64_t ps = p.pool_slot[e];
          if (ps >= 0 && ps < p.pool_slots) t = make_int2(static_cast<int>(ps << (p.lg_gs + 1)), tok);
        } else {
          t = make_int2(tok, tok);
        }
      }
      gtab[i] = t;
      if ((t.x < 0 || t.y >= cur0) && i < fb) fb = i;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) fb = min(fb, __shfl_xor(fb, m));
  if (lane == 0) wfb[wave] = fb;

  // RoPE table for the queries of this workgroup's rows.
  const int rend = (r0 + kRows) < w.R ? (r0 + kRows) : w.R;
  const int nqt = (rend - 1) / p.G - q_first + 1;
  float2* cs = reinterpret_cast<float2*>(smem);
  const int64_t q0 = rope_base(p.rope, w.qlo) + q_first;  // the unit's queries share one chunk
  static_assert(80 * H * 8 <= kMain, "RoPE table and its scratch fit the stage space");
  rope_table(p.rope, q0, nqt, H, cs, reinterpret_cast<float2*>(smem + 64 * H * 8));
  __syncthreads();

  // K and V buffer resources: the (sequence, KV head) slab, or the staging
  // pool whose slot holds K then V of one granule.
  __amdgpu_buffer_rsrc_t kr, vr;
  if constexpr (POOL) {
    const int64_t gbytes = static_cast<int64_t>(p.gs) * D * 2;
    const uint32_t bytes = static_cast<uint32_t>(p.pool_slots * 2 * gbytes);
    kr = buffer_rsrc(p.k, bytes);
    vr = buffer_rsrc(static_cast<const char*>(p.v) + gbytes, bytes - static_cast<uint32_t>(gbytes));
  } else {
    const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap * D * 2;
    const uint32_t bytes = static_cast<uint32_t>(p.kv_cap * D * 2);
    kr = buffer_rsrc(static_cast<const char*>(p.k) + slab, bytes);
    vr = buffer_rsrc(static_cast<const char*>(p.v) + slab, bytes);
  }
  // Stages [0, nu) hold only valid keys before the current chunk (no masks);
  // their loads take the fast path when g_s >= 2 (nfast).
  const int nstages = kend > kbeg ? (kend - kbeg + kTK - 1) / kTK : 0;
  int nu;
  {
    int f = wfb[0];
#pragma unroll
    for (int x = 1; x < NW; ++x) f = min(f, wfb[x]);
    const int good = min(f << p.lg_gs, kend - kbeg);
    nu = __builtin_amdgcn_readfirstlane(good > 0 ? good / kTK : 0);
  }
  const int nfast = p.lg_gs >= 1 ? nu : 0;
  // The first stage's loads go out before the query rows are rotated.
  StageRegs<D, NW> sr;
  if (nstages > 0) load_stage<D, NW>(p, kr, vr, gtab, gfirst, kbeg, kend, qend, nfast > 0, sr);

  // Rotate, scale by softmax_scale * log2(e) and round the query rows to
  // bf16 MFMA operands.
  Pack8 qb[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int qloc = qpos[rb] - static_cast<int>(w.qlo);
    float x[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) x[ks][i] = bf16_to_f32(qraw[rb][ks].h[i]);
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
      for (int i = 0; i < 4; ++i) {
        const f32x2 f = {x[ks][2 * i] * p.scale_log2, x[ks][2 * i + 1] * p.scale_log2};
        qb[rb][ks].u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
      }
    }
  }
  __syncthreads();  // the table space becomes the K/V stage buffers

  f32x16 o[RB][DB];
  float ref[RB], lsum[RB];
  bool started[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    ref[rb] = 0.f;
    lsum[rb] = 0.f;
    started[rb] = false;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[rb][db][j] = 0.f;
  }

  // One stage, with its matrix-core products and the other work of the
  // stage interleaved in a fixed order (scheduling barriers): S of the first
  // key half beside the next stage's loads, S of the second half beside the
  // softmax of the first, PV of the first beside the softmax of the second,
  // PV of the second beside the next stage's LDS stores (into the buffer the
  // previous stage used).  Operands are read three products ahead.
  constexpr int NS = 2 * KS;      // S products: i -> half i / KS, slice i % KS
  constexpr int NP = 2 * DB;      // PV products of a half: i -> kk = i / DB, db = i % DB
  constexpr int AH = 3;
  auto kop = [&](const char* kl, int i) {
    return *reinterpret_cast<const bf16x8*>(kl + ((i / KS) * 32 + n) * KP + ((i % KS) * 16 + hsub * 8) * 2);
  };
  auto vop = [&](const char* vl, int h, int i) {
    return *reinterpret_cast<const bf16x8*>(vl + ((i % DB) * 32 + n) * kVP + ((2 * h + i / DB) * 16 + hsub * 8) * 2);
  };
  auto step = [&](int st, auto mtag, auto ftag) {
    constexpr bool masked = decltype(mtag)::value;
    constexpr bool fast = decltype(ftag)::value;  // the next stage's loads take the fast path
    const char* kl = smem + (st & 1) * SB;
    const char* vl = kl + kTK * KP;
    const int* tl = reinterpret_cast<const int*>(vl + D * kVP);
    char* kn = smem + ((st + 1) & 1) * SB;
    char* vn = kn + kTK * KP;
    int* tn = reinterpret_cast<int*>(vn + D * kVP);
    const int knext = kbeg + (st + 1) * kTK;
    if (!rb_on[0]) {  // wave-uniform: this wave has no rows, only loads and stores
      load_stage<D, NW>(p, kr, vr, gtab, gfirst, knext, kend, qend, fast, sr);
      store_stage<D, NW>(sr, kn, vn, tn);
      return;
    }
    f32x16 s[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) s[rb][h][j] = 0.f;
    bf16x8 a[AH];
#pragma unroll
    for (int i = 0; i < AH; ++i) a[i] = kop(kl, i);
    __builtin_amdgcn_sched_barrier(0);
    // S of the first half, the next stage's loads after two products
#pragma unroll
    for (int i = 0; i < KS; ++i) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb_on[rb]) s[rb][0] = mfma32x32x16(a[i % AH], qb[rb][i].v, s[rb][0]);
      if (i + AH < NS) a[i % AH] = kop(kl, i + AH);
      if (i == 1) load_stage<D, NW>(p, kr, vr, gtab, gfirst, knext, kend, qend, fast, sr);
      __builtin_amdgcn_sched_barrier(0);
    }
    // S of the second half, the softmax terms of the first
    Pack8 pb[RB][2][2];
    float ps[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ps[rb][0] = ps[rb][1] = 0.f;
    constexpr int PPS = 8 / KS;  // element pairs per product
#pragma unroll
    for (int i = KS; i < NS; ++i) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb_on[rb]) s[rb][1] = mfma32x32x16(a[i % AH], qb[rb][i - KS].v, s[rb][1]);
      if (i + AH < NS) a[i % AH] = kop(kl, i + AH);
#pragma unroll
      for (int q = 0; q < PPS; ++q)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (rb_on[rb])
            sm_pair<masked>(s[rb][0], 2 * ((i - KS) * PPS + q), tl, hsub, cur0, qpos[rb], ref[rb], ps[rb][0],
                            pb[rb][0]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (rb_on[rb]) sm_post<DB>(s[rb][0], ps[rb][0], ref[rb], lsum[rb], started[rb], o[rb], pb[rb][0]);
    // PV of the first half, the softmax terms of the second
    constexpr int PPP = 8 / NP;
#pragma unroll
    for (int i = 0; i < AH; ++i) a[i] = vop(vl, 0, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb_on[rb]) o[rb][i % DB] = mfma32x32x16(a[i % AH], pb[rb][0][i / DB].v, o[rb][i % DB]);
      if (i + AH < NP) a[i % AH] = vop(vl, 0, i + AH);
#pragma unroll
      for (int q = 0; q < PPP; ++q)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          if (rb_on[rb])
            sm_pair<masked>(s[rb][1], 2 * (i * PPP + q), tl + 32, hsub, cur0, qpos[rb], ref[rb], ps[rb][1],
                            pb[rb][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      if (rb_on[rb]) sm_post<DB>(s[rb][1], ps[rb][1], ref[rb], lsum[rb], started[rb], o[rb], pb[rb][1]);
    // PV of the second half, the next stage's LDS stores after two products
#pragma unroll
    for (int i = 0; i < AH; ++i) a[i] = vop(vl, 1, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb_on[rb]) o[rb][i % DB] = mfma32x32x16(a[i % AH], pb[rb][1][i / DB].v, o[rb][i % DB]);
      if (i + AH < NP) a[i % AH] = vop(vl, 1, i + AH);
      if (i == 1) store_stage<D, NW>(sr, kn, vn, tn);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (nstages > 0) {
    store_stage<D, NW>(sr, smem, smem + kTK * KP, reinterpret_cast<int*>(smem + kTK * KP + D * kVP));
    __syncthreads();
  }
  // Masked stages (past the key range, absent keys, current-chunk keys) form
  // a suffix of an item's stages, since tokens ascend along a list: a loop
  // over the unmasked stages, then one over the rest (two stage bodies in
  // sequence rather than a choice inside one loop, which the register
  // allocator handles without spills).
  // The unmasked stages whose successor is also fast-loaded run a body with
  // only the fast load path (a body with both paths would merge their load
  // registers, which makes the loads wait).
  int st = 0;
  for (; st + 1 < nfast; ++st) {
    step(st, std::false_type{}, std::true_type{});
    __syncthreads();  // stage st + 1 is in LDS; every read of stage st is done
  }
  for (; st < nu; ++st) {
    step(st, std::false_type{}, std::false_type{});
    __syncthreads();
  }
  for (; st < nstages; ++st) {
    step(st, std::true_type{}, std::false_type{});
    __syncthreads();
  }

  // O^T register j of block db is d = db*32 + 8*(j/4) + 4*hsub + (j%4).
  // Unsplit items stage their bf16 rows in LDS (the stage buffers are free
  // once the last stage's barrier has passed) and write whole rows, 16 bytes
  // per lane: a lane's own pieces of a row are 8 bytes at 16-byte strides,
  // which would touch 32 rows' cache lines per store instruction.
  constexpr int OP = D * 2 + 16;  // bytes per staged output row
  static_assert(kRows * OP <= kMain, "the output tile fits the stage buffers");
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!rb_on[rb]) continue;
    const float lrow = lsum[rb] + __shfl_xor(lsum[rb], 32);
    if (row[rb] >= w.R) continue;
    const int64_t orow =
        (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl[rb]) * p.q_stride + (qpos[rb] - p.q_row0);
    if (p.splits == 1) {
      const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
      char* ot = smem + (row[rb] - r0) * OP;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * hsub;
          const f32x2 f0 = {o[rb][db][4 * g4 + 0] * inv, o[rb][db][4 * g4 + 1] * inv};
          const f32x2 f1 = {o[rb][db][4 * g4 + 2] * inv, o[rb][db][4 * g4 + 3] * inv};
          uint2 pk;
          pk.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f0, bf16x2));
          pk.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f1, bf16x2));
          *reinterpret_cast<uint2*>(ot + d0 * 2) = pk;
        }
      }
      if (p.lse != nullptr && hsub == 0)
        p.lse[orow] = started[rb] ? (ref[rb] + log2f(lrow)) * kLn2 : -INFINITY;
    } else {
      const int64_t pr = (w.slot * p.splits + split) * p.Rcap + row[rb];
      float* wo = p.ws_o + pr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * hsub;
          *reinterpret_cast<float4*>(wo + d0) =
              make_float4(o[rb][db][4 * g4], o[rb][db][4 * g4 + 1], o[rb][db][4 * g4 + 2], o[rb][db][4 * g4 + 3]);
        }
      }
      if (hsub == 0) {
        p.ws_ml[pr * 2] = started[rb] ? ref[rb] : kNegBig;
        p.ws_ml[pr * 2 + 1] = lrow;
      }
    }
  }
  if (p.splits == 1) {  // uniform
    __syncthreads();
    constexpr int CPR = D / 8;  // 16-byte pieces per row
    const int nrows = (w.R - r0) < kRows ? (w.R - r0) : kRows;
    for (int i = threadIdx.x; i < nrows * CPR; i += NW * 64) {
      const int lr = i / CPR, c = i - lr * CPR;
      const int r = r0 + lr;
      const int qi = r / p.G;
      const int64_t orow = (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + (r - qi * p.G)) * p.q_stride +
                           (w.qlo + qi - p.q_row0);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow * D + c * 8) =
          *reinterpret_cast<const uint4*>(smem + lr * OP + c * 16);
    }
  }
}

// Persistent launch: one resident workgroup per slot walks the work items
// bx = blockIdx.x, blockIdx.x + gridDim.x, ...; the grid is a multiple of 8,
// so every item stays on the XCD that block_item intends for it, and no
// workgroup dispatch separates one item from the next.
template <int D, int NW, int RB, bool POOL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void attend_mfma_kernel(AttendParams p) {
  __shared__ __align__(16) char smem[attend_main_bytes<D>() + kTab * 8 + 64];
  for (int64_t bx = blockIdx.x; bx < p.nblocks; bx += gridDim.x) {
    attend_item<D, NW, RB, POOL>(p, bx, smem);
    __syncthreads();  // the next item rewrites the LDS tables
  }
}

// f32 inputs: 64 rows per workgroup, four consecutive lanes per row.  Lane
// part q of a row owns the 16-byte chunks q, q + 4, q + 8, ... of d: the
// four lanes of a row read 64 contiguous bytes of a K/V row per LDS read
// (one broadcast read serves the wave's 16 rows), and since d/2 is a
// multiple of 16 floats, the partner i + d/2 of each of a lane's RoPE
// dimensions i < d/2 is in the lane's own chunks.  Each lane forms its
// partial q.k over its d/4 dimensions; two DPP exchanges inside the quad
// give every lane of the row the full score, so the softmax state (m, l) is
// the same in the four lanes and each keeps O for its own dimensions.
__device__ __forceinline__ float quad_sum(float x) {
  // quad_perm [1,0,3,2], then [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attend_f32_kernel(AttendParams p) {
  constexpr int TK = kTKf;
  constexpr int H = D / 2;
  constexpr int NC = D / 16;  // 16-byte chunks per lane
  static_assert(H % 16 == 0, "pair partners in the lane's own chunks");
  __shared__ __align__(16) float kt[TK][D];
  __shared__ __align__(16) float vt[TK][D];
  __shared__ int tk[TK];
  const int tid = threadIdx.x;
  const int part = tid & 3;
  int64_t u;
  int item;
  if (!block_item(p, blockIdx.x, u, item)) return;
  const int slice = item / p.splits;
  const int split = item - slice * p.splits;
  const AUnit w = make_aunit(p, u);
  const int r0 = slice * 64;
  if (r0 >= w.R) return;
  const int kbeg = split * p.keys_per_split;
  int kend = kbeg + p.keys_per_split;
  if (kend > w.nkeys) kend = w.nkeys;

  const int row = r0 + (tid >> 2);
  const bool row_ok = row < w.R;
  const int qloc = row_ok ? row / p.G : 0;
  const int hl = row_ok ? row - qloc * p.G : 0;
  const int qpos = static_cast<int>(w.qlo) + qloc;
  const double qrot = static_cast<double>(rope_base(p.rope, w.qlo) + qloc);
  // chunk c of the lane covers dimensions 4 * (part + 4 c) .. + 3
  auto dim0 = [&](int c) { return 4 * (part + 4 * c); };
  float q[NC][4];
  {
    const float* src = static_cast<const float*>(p.q) +
        ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (qpos - p.q_row0)) * D;
    float4 raw[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c)
      raw[c] = row_ok ? *reinterpret_cast<const float4*>(src + dim0(c)) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int c = 0; c < NC / 2; ++c) {
      const float a[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
      const float b[4] = {raw[c + NC / 2].x, raw[c + NC / 2].y, raw[c + NC / 2].z, raw[c + NC / 2].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float cs, sn;
        rope_cs(qrot, rope_freq(p.rope, dim0(c) + e), cs, sn);
        q[c][e] = (a[e] * cs - b[e] * sn) * p.scale_log2;
        q[c + NC / 2][e] = (a[e] * sn + b[e] * cs) * p.scale_log2;
      }
    }
  }
  float o[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int e = 0; e < 4; ++e) o[c][e] = 0.f;
  float m_run = kNegBig, l_run = 0.f;
  const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap;
  const int cur0 = static_cast<int>(w.t * p.C);
  for (int kb = kbeg; kb < kend; kb += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * D / 4; idx += 256) {
      const int s = idx / (D / 4), c4 = idx - s * (D / 4);
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      const int tok = kb + s < kend ? slot_token(p, w, kb + s) : -1;
      if (tok >= 0 && tok < w.qlo + w.nq) {  // past the last query: unread (may be unwritten)
        int64_t ko, vo;
        kv_offsets<D>(p, w, kb + s, tok, slab, ko, vo);
        kk = reinterpret_cast<const float4*>(static_cast<const float*>(p.k) + ko)[c4];
        vv = reinterpret_cast<const float4*>(static_cast<const float*>(p.v) + vo)[c4];
      }
      reinterpret_cast<float4*>(&kt[s][0])[c4] = kk;
      reinterpret_cast<float4*>(&vt[s][0])[c4] = vv;
    }
    if (tid < TK) tk[tid] = (kb + tid < kend) ? slot_token(p, w, kb + tid) : -1;
    __syncthreads();
    float sc[TK];
    float mx = kNegBig;
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 kk = *reinterpret_cast<const float4*>(&kt[s][dim0(c)]);
        acc = fmaf(q[c][0], kk.x, acc);
        acc = fmaf(q[c][1], kk.y, acc);
        acc = fmaf(q[c][2], kk.z, acc);
        acc = fmaf(q[c][3], kk.w, acc);
      }
      acc = quad_sum(acc);
      const int tok = tk[s];
      const bool ok = tok >= 0 && (tok < cur0 || tok <= qpos);
      sc[s] = ok ? acc : -INFINITY;
      mx = fmaxf(mx, sc[s]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[c][e] *= alpha;
#pragma unroll
    for (int s = 0; s < TK; ++s) {
      const float e = exp2f(sc[s] - m_new);
      l_run += e;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const float4 vv = *reinterpret_cast<const float4*>(&vt[s][dim0(c)]);
        o[c][0] = fmaf(e, vv.x, o[c][0]);
        o[c][1] = fmaf(e, vv.y, o[c][1]);
        o[c][2] = fmaf(e, vv.z, o[c][2]);
        o[c][3] = fmaf(e, vv.w, o[c][3]);
      }
    }
    m_run = m_new;
  }
  if (!row_ok) return;
  const int64_t orow = (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (qpos - p.q_row0);
  if (p.splits == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = static_cast<float*>(p.out) + orow * D;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *reinterpret_cast<float4*>(out + dim0(c)) =
          make_float4(o[c][0] * inv, o[c][1] * inv, o[c][2] * inv, o[c][3] * inv);
    if (p.lse != nullptr && part == 0) p.lse[orow] = (m_run + log2f(l_run)) * kLn2;
  } else {
    const int64_t pr = (w.slot * p.splits + split) * p.Rcap + row;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      *reinterpret_cast<float4*>(p.ws_o + pr * D + dim0(c)) = make_float4(o[c][0], o[c][1], o[c][2], o[c][3]);
    if (part == 0) {
      p.ws_ml[pr * 2] = m_run;
      p.ws_ml[pr * 2 + 1] = l_run;
    }
  }
}

// Merge split-key partials: m = max m_s, l = sum l_s 2^(m_s - m),
// O = sum O_s 2^(m_s - m) / l.  One wave per row.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void combine_kernel(AttendParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t gr = static_cast<int64_t>(blockIdx.x) * 4 + wave;  // (unit, row)
  if (gr >= p.units * p.Rcap) return;
  const int64_t u = gr / p.Rcap;
  const int row = static_cast<int>(gr - u * p.Rcap);
  // The decode kernel writes every split's partial (empty ones as m = -big,
  // l = 0), so it needs no key count; the other kernels skip splits past the
  // unit's keys.
  const AUnit w = make_aunit(p, u, !p.all_splits);
  if (row >= w.R) return;
  // Splits that hold partials of this unit; they are read eight at a time,
  // every load of a group issued before any is used.
  int ns = p.splits;
  if (!p.all_splits) {
    ns = (w.nkeys + p.keys_per_split - 1) / p.keys_per_split;
    ns = ns < p.splits ? ns : p.splits;
  }
  constexpr int kG = 8;
  constexpr int kD = D / 64 > 0 ? D / 64 : 1;
  float m = kNegBig, l = 0.f;
  float acc[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kG) {
    float2 ml[kG];
    float o[kG][kD];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const bool on = s0 + j < ns;
      const int64_t pr = (w.slot * p.splits + (on ? s0 + j : 0)) * p.Rcap + row;
      ml[j] = on ? *reinterpret_cast<const float2*>(p.ws_ml + pr * 2) : make_float2(kNegBig, 0.f);
#pragma unroll
      for (int i = 0; i < kD; ++i) o[j][i] = on ? p.ws_o[pr * D + lane + 64 * i] : 0.f;
    }
    float mn = m;
#pragma unroll
    for (int j = 0; j < kG; ++j) mn = fmaxf(mn, ml[j].x);
    const float c = exp2f(m - mn);
    l *= c;
#pragma unroll
    for (int i = 0; i < kD; ++i) acc[i] *= c;
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const float sc = exp2f(ml[j].x - mn);
      l += ml[j].y * sc;
#pragma unroll
      for (int i = 0; i < kD; ++i) acc[i] += o[j][i] * sc;
    }
    m = mn;
  }
  const int qloc = row / p.G, hl = row - qloc * p.G;
  const int64_t orow =
      (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (w.qlo + qloc - p.q_row0);
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) store1<BF16>(p.out, orow * D + lane + 64 * i, acc[i] * inv);
  if (p.lse != nullptr && lane == 0) p.lse[orow] = (m + log2f(l)) * kLn2;
}

// Decode-shaped calls (at most kDecRows query rows per unit: one query's
// GQA group, or a few queries): one workgroup of four waves per (unit,
// split of kDecKeys keys).  Each wave takes 32 keys: K rows go from HBM
// straight into the A operands of 16x16x32 bf16 products (S^T = K Q^T,
// query rows on N); the softmax runs in registers; P (bf16) and the wave's
// V rows go through LDS, V read back transposed, for O = P V on the same
// products.  The four waves' (m, l, O) are merged in LDS; the item writes its
// partial to the workspace (several splits) or the normalised output.
constexpr int kDecRows = 16;
constexpr int kDecWaveKeys = 32;
constexpr int kDecKeys = 4 * kDecWaveKeys;
constexpr int kDecPP = kDecWaveKeys + 4;  // floats per P row in LDS (padded)

template <int D>
__global__ __launch_bounds__(256) void attend_decode_kernel(AttendParams p) {
  constexpr int KS = D / 32;        // k-steps of the QK product
  constexpr int H = D / 2;
  constexpr int DP = D / 64;        // V elements per lane as loaded
  constexpr int NT = D / 16;        // output column tiles
  constexpr int VP = D * 2 + 4;     // bytes per V row in LDS (padded)
  constexpr int kVBuf = 4 * kDecWaveKeys * VP;
  static_assert(kVBuf >= 4 * kDecRows * D * 4, "merge buffer aliases the V rows");
  __shared__ float2 cs[kDecRows * H];
  __shared__ __align__(16) float pw[4][kDecRows][kDecPP];
  __shared__ __align__(16) char vbuf[kVBuf];
  __shared__ float wm[4][kDecRows], wl[4][kDecRows];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t u = blockIdx.x / p.splits;
  const int split = static_cast<int>(blockIdx.x - u * p.splits);
  const AUnit w = uniform_unit(make_aunit(p, u, false));
  const int64_t kw = static_cast<int64_t>(split) * kDecKeys + wave * kDecWaveKeys;  // wave's first key
  const int64_t slab = (static_cast<int64_t>(w.b) * p.Hkv + w.kvh) * p.kv_cap;
  const int64_t qhi = w.qlo + w.nq;

  // This lane's query row as the B operand column n = lane % 16 (rows past
  // the unit's last repeat it; their outputs are never used).  Its loads go
  // out first.
  const int n = lane & 15, sub = lane >> 4;
  const int rn = n < w.R ? n : w.R - 1;
  const int qn = rn / p.G, hn = rn - qn * p.G;
  float xq[KS][8];
  {
    const int64_t base =
        ((static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hn) * p.q_stride + (w.qlo + qn - p.q_row0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load8<true>(p.q, base + ks * 32 + sub * 8, xq[ks]);
  }
  // Wave key kw + (lane % 32): its token, or -1 (past the list or the causal
  // end), and the row of its K: the token in the (sequence, KV head) slab,
  // or in pool mode row (2*slot)*g_s + offset of the granule's pool slot
  // (its V row g_s further).
  const bool pool = p.pool_slot != nullptr;
  const int64_t kbase = pool ? 0 : slab;
  const int64_t vshift = pool ? p.gs : 0;
  int tok = -1, row = 0;
  {
    const int64_t k = kw + (lane & 31);
    if (p.dense) {
      tok = k < qhi ? static_cast<int>(k) : -1;
      row = tok >= 0 ? tok : 0;
    } else {
      const int64_t gi = k >> p.lg_gs;
      const int64_t e = w.slot * p.gmax + gi;
      const int g = gi < p.gmax ? p.gran[e] : -1;
      const int off = static_cast<int>(k & (p.gs - 1));
      tok = g >= 0 ? g * p.gs + off : -1;
      if (g >= 0) row = pool ? 2 * p.pool_slot[e] * p.gs + off : tok;
    }
  }
  // K rows of the two 16-key tiles (A operands: key lane % 16, d slots
  // ks*32 + 8*(lane/16) + i) and the V elements of all 32 keys (lane owns
  // columns DP*lane ...).
  Pack8 ka[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int kr = __shfl(row, t * 16 + n);
    const int64_t e = (kbase + kr) * D + sub * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[t][ks].q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + e + ks * 32);
  }
  // Keys past the list or past the unit's last query read V as zeros: their
  // P is zero, but the row they would read (row 0, a pool slot the step did
  // not fill, or a token not yet written) may hold a non-finite value, and
  // 0 * NaN is NaN.
  uint32_t vv[kDecWaveKeys];
#pragma unroll
  for (int j = 0; j < kDecWaveKeys; ++j) {
    const int vr = __builtin_amdgcn_readlane(row, j);
    const int vt = __builtin_amdgcn_readlane(tok, j);
    const bool present = vt >= 0 && vt < qhi;
    const int64_t e = (kbase + vshift + vr) * D + lane * DP;
    if constexpr (DP == 2)
      vv[j] = present ? *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.v) + e) : 0u;
    else
      vv[j] = present ? static_cast<const uint16_t*>(p.v)[e] : 0u;
  }
  // RoPE table of the unit's queries, then the rotated, scaled query
  // operand (bf16).
  for (int i = threadIdx.x; i < w.nq * H; i += 256) {
    const int qi = i / H, pr = i - qi * H;
    float c, s;
    rope_cs(static_cast<double>(rope_base(p.rope, w.qlo) + qi), rope_freq(p.rope, pr), c, s);
    cs[i] = make_float2(c, s);
  }
  __syncthreads();
  Pack8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float2 t = cs[qn * H + ks * 32 + sub * 8 + i];
      const float a = xq[ks][i], b = xq[ks + KS / 2][i];
      qb[ks].h[i] = f32_to_bf16((a * t.x - b * t.y) * p.scale_log2);
      qb[ks + KS / 2].h[i] = f32_to_bf16((a * t.y + b * t.x) * p.scale_log2);
    }
  }
  // S^T tiles: lane holds keys 16t + 4*(lane/16) + i of row n.
  const int64_t qpos = w.qlo + qn;
  float sv[2][4];
  float mx = kNegBig;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(ka[t][ks].v, qb[ks].v, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kt = __shfl(tok, t * 16 + sub * 4 + i);
      const bool ok = kt >= 0 && kt <= qpos;
      sv[t][i] = ok ? acc[i] : -INFINITY;
      mx = fmaxf(mx, sv[t][i]);
    }
  }
  mx = xor32_max(xor16_max(mx));
  // P (f32, rows x keys) and the wave's V rows into its LDS regions.
  float ls = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float4 e4;
    e4.x = exp2f(sv[t][0] - mx);  // 0 for masked keys
    e4.y = exp2f(sv[t][1] - mx);
    e4.z = exp2f(sv[t][2] - mx);
    e4.w = exp2f(sv[t][3] - mx);
    ls += (e4.x + e4.y) + (e4.z + e4.w);
    *reinterpret_cast<float4*>(&pw[wave][n][t * 16 + sub * 4]) = e4;
  }
  ls = xor32_sum(xor16_sum(ls));
  char* vw = vbuf + wave * kDecWaveKeys * VP;
#pragma unroll
  for (int j = 0; j < kDecWaveKeys; ++j) {
    if constexpr (DP == 2) *reinterpret_cast<uint32_t*>(vw + j * VP + lane * 4) = vv[j];
    else *reinterpret_cast<uint16_t*>(vw + j * VP + lane * 2) = static_cast<uint16_t>(vv[j]);
  }
  // O = P V: A = P (row lane % 16, keys 8*(lane/16) + i), B = V (column
  // lane % 16 of the tile, the same keys), read transposed from LDS.
  Pack8 pa;
  {
    const float4 a = *reinterpret_cast<const float4*>(&pw[wave][n][sub * 8]);
    const float4 b = *reinterpret_cast<const float4*>(&pw[wave][n][sub * 8 + 4]);
    pa.h[0] = f32_to_bf16(a.x); pa.h[1] = f32_to_bf16(a.y);
    pa.h[2] = f32_to_bf16(a.z); pa.h[3] = f32_to_bf16(a.w);
    pa.h[4] = f32_to_bf16(b.x); pa.h[5] = f32_to_bf16(b.y);
    pa.h[6] = f32_to_bf16(b.z); pa.h[7] = f32_to_bf16(b.w);
  }
  f32x4 ot[NT];
#pragma unroll
  for (int c = 0; c < NT; ++c) {
    Pack8 vb;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      vb.h[i] = *reinterpret_cast<const uint16_t*>(vw + (sub * 8 + i) * VP + (c * 16 + n) * 2);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    ot[c] = mfma16x16x32(pa.v, vb.v, z);
  }
  // Merge the four waves (the merge buffer reuses the V rows' space).
  __syncthreads();
  float* wo = reinterpret_cast<float*>(vbuf);  // [4][kDecRows][D]
  if (sub == 0) {
    wm[wave][n] = mx;
    wl[wave][n] = ls;
  }
#pragma unroll
  for (int c = 0; c < NT; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = sub * 4 + i;
      if (r < w.R) wo[(wave * kDecRows + r) * D + c * 16 + n] = ot[c][i];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < w.R * D; i += 256) {
    const int r = i / D, d = i - r * D;
    float m = kNegBig;
#pragma unroll
    for (int x = 0; x < 4; ++x) m = fmaxf(m, wm[x][r]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float sc = exp2f(wm[x][r] - m);
      l += wl[x][r] * sc;
      acc += wo[(x * kDecRows + r) * D + d] * sc;
    }
    if (p.splits > 1) {
      const int64_t pr = (w.slot * p.splits + split) * p.Rcap + r;
      p.ws_o[pr * D + d] = acc;
      if (d == 0) {
        p.ws_ml[pr * 2] = m;
        p.ws_ml[pr * 2 + 1] = l;
      }
    } else {
      const int qloc = r / p.G, hl = r - qloc * p.G;
      const int64_t orow =
          (static_cast<int64_t>(w.b) * p.Hq + w.kvh * p.G + hl) * p.q_stride + (w.qlo + qloc - p.q_row0);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      store1<true>(p.out, orow * D + d, acc * inv);
      if (p.lse != nullptr && d == 0) p.lse[orow] = (m + log2f(l)) * kLn2;
    }
  }
}

struct Plan {
  int nw, slices, splits, kps, rcap;
  bool decode;
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
  pl.decode = false;
  if (g.bf16 && allow_split && rows <= kDecRows) {
    // decode kernel: kDecKeys keys per item
    const int64_t keys = max_keys(g, dense);
    pl.decode = true;
    pl.nw = 4;
    pl.slices = 1;
    pl.kps = kDecKeys;
    pl.splits = static_cast<int>((keys + kDecKeys - 1) / kDecKeys);
    if (pl.splits < 1) pl.splits = 1;
    return pl;
  }
  if (g.bf16) {
    const int64_t wblocks = (rows + 31) / 32;  // waves needed
    // Always 8 waves: the LDS stages hold one workgroup per CU, and waves
    // without rows (few-row units such as decode) still share the loads.
    pl.nw = 8;
    pl.slices = static_cast<int>((wblocks + pl.nw - 1) / pl.nw);
  } else {
    pl.nw = 4;
    pl.slices = static_cast<int>((rows + 63) / 64);
  }
  const int64_t wgs = pl.units * pl.slices;
  const int64_t keys = max_keys(g, dense);
  pl.splits = 1;
  pl.kps = static_cast<int>(keys);
  if (allow_split && wgs < 512 && keys > (g.bf16 ? 256 : 64)) {
    int64_t sp, want;
    if (g.bf16) {
      // About one work item per CU (the bf16 kernel keeps one workgroup per
      // CU, so a second item per workgroup would run after the first), each
      // at least one LDS stage of keys.
      sp = (keys + kTK - 1) / kTK;
      want = (device_cus() + wgs - 1) / wgs;
    } else {
      // f32: splits of about 64 keys, up to about 1024 workgroups
      sp = (keys + 63) / 64;
      want = (1024 + wgs - 1) / wgs;
    }
    if (sp > want) sp = want;
    if (sp > 1) {
      pl.kps = static_cast<int>(((keys + sp - 1) / sp + kTK - 1) / kTK * kTK);
      pl.splits = static_cast<int>((keys + pl.kps - 1) / pl.kps);
    }
  }
  // A bf16 item reads at most kTab granules (a multiple of kTK keys).
  const int64_t cap = static_cast<int64_t>(kTab) * g.gs;
  if (g.bf16 && allow_split && pl.kps > cap) {
    pl.kps = static_cast<int>(cap);
    pl.splits = static_cast<int>((keys + cap - 1) / cap);
  }
  return pl;
}

// Workgroups that fit on the device at once for kernel k (a multiple of 8,
// so that blockIdx.x and every bx it takes sit on the same XCD), at most n.
// Cached per (device, kernel, block size) under a lock.
template <typename Kernel>
unsigned resident_grid(Kernel k, int threads, int64_t n) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int>, int> slots;
  const int dev = current_device();
  const auto key = std::make_tuple(dev, reinterpret_cast<const void*>(k), threads);
  int v = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = slots.find(key);
    if (it != slots.end()) v = it->second;
  }
  if (v == 0) {
    int cus = 0, occ = 0;
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(k), threads, 0);
    v = (cus > 0 ? cus : 8) * (occ > 0 ? occ : 1);
    v -= v % 8;
    if (v < 8) v = 8;
    std::lock_guard<std::mutex> lock(mu);
    slots[key] = v;
  }
  return static_cast<unsigned>(n < v ? n : v);
}

// bf16 calls always run 8 waves per workgroup (make_plan).
template <int D, int RB, bool POOL>
void launch_mfma(int64_t nblocks, hipStream_t stream, const AttendParams& p) {
  auto k = attend_mfma_kernel<D, 8, RB, POOL>;
  hipLaunchKernelGGL(k, dim3(resident_grid(k, 512, nblocks)), dim3(512), 0, stream, p);
}

template <int D, int RB>
void launch_mfma_pool(int64_t nblocks, hipStream_t stream, const AttendParams& p) {
  if (p.pool_slot != nullptr)
    launch_mfma<D, RB, true>(nblocks, stream, p);
  else
    launch_mfma<D, RB, false>(nblocks, stream, p);
}

template <int D>
hipError_t launch_attend_d(const Geometry& g, AttendParams& p, const Plan& pl, hipStream_t stream) {
  if (pl.decode) {
    p.nblocks = pl.units * pl.splits;
    hipLaunchKernelGGL((attend_decode_kernel<D>), dim3(static_cast<unsigned>(p.nblocks)), dim3(256), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.splits == 1) return e;
    const unsigned cgrid = static_cast<unsigned>((pl.units * pl.rcap + 3) / 4);
    hipLaunchKernelGGL((combine_kernel<true, D>), dim3(cgrid), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t groups = (pl.units + 7) / 8;
  p.nblocks = groups * 8 * p.per_unit;
  const unsigned grid = static_cast<unsigned>(p.nblocks);
  if (g.bf16) {
    launch_mfma_pool<D, 1>(p.nblocks, stream, p);
  } else {
    hipLaunchKernelGGL((attend_f32_kernel<D>), dim3(grid), dim3(256), 0, stream, p);
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

bool attend_supported(const Geometry& g) {
  if (!((g.d == 64 || g.d == 128) && (g.gs & (g.gs - 1)) == 0 && g.C <= 64)) return false;
  // bf16 K/V slabs are addressed through buffer resources with 32-bit offsets
  return !g.bf16 || g.kv_cap * g.d * 2 < (int64_t{1} << 31);
}

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
  p.units = pl.units;
  p.B = g.B;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.G = g.G;
  p.d = g.d;
  p.C = g.C;
  p.gs = g.gs;
  p.lg_gs = 0;
  while ((1 << p.lg_gs) < g.gs) ++p.lg_gs;
  p.gmax = g.gmax;
  p.Rcap = pl.rcap;
  p.slices = pl.slices;
  p.splits = pl.splits;
  p.keys_per_split = pl.kps;
  p.per_unit = pl.slices * pl.splits;
  p.dense = dense ? 1 : 0;
  p.all_splits = pl.decode ? 1 : 0;
  p.scale_log2 = g.scale * kLog2e;
  p.rope = g.rope;
  return g.d == 128 ? launch_attend_d<128>(g, p, pl, stream) : launch_attend_d<64>(g, p, pl, stream);
}

hipError_t attend_noalloc_scratch(void** ptr) {
  // Resolved once per device, with that device current; the array's own
  // name is a host-side stand-in, not its device address.
  static std::mutex mu;
  static std::map<int, void*> addr;
  const int dev = current_device();
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  addr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

}  // namespace hga
