// Exact top-k selection inside one workgroup, shared by the routing kernels:
// the indices of the k largest 32-bit order keys, equal keys going to the
// lowest index (the tie rule of the selection equation of the xllm-io
// review page, section 3, as fixed for this path), returned ascending.
// Rank selection (one candidate per thread), register bitonic sorts for
// small inputs, and an exact block radix select otherwise; all three give
// the same result.
#pragma once

#include "hga_device.h"

namespace hga {
namespace {

constexpr int kRankMax = 512;  // rank_select: at most one candidate per thread

struct SelScratch {
  int hist[256];
  int wsum[16];
  int bcast[4];
  uint64_t cand[128];
  __attribute__((aligned(16))) uint64_t rk[kRankMax];
};

// 64-bit selection key: the score's order key above the inverted index, so
// that a larger key means a larger score or, at equal scores, a lower index.
__device__ __forceinline__ uint64_t sel_key(uint32_t k, int i) {
  return (static_cast<uint64_t>(k) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const unsigned lo = __shfl_xor(static_cast<unsigned>(v), m);
  const unsigned hi = __shfl_xor(static_cast<unsigned>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t shfl_xor_key(uint32_t v, int m) { return __shfl_xor(v, m); }
__device__ __forceinline__ uint64_t shfl_xor_key(uint64_t v, int m) { return shfl_xor64(v, m); }

// Bitonic sort of the wave's 64*M keys (element s*64 + lane in v[s]) into
// descending order, entirely in registers.
template <int M, typename T>
__device__ __forceinline__ void wave_sort_desc(T (&v)[M]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int size = 2; size <= 64 * M; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int s = 0; s < M; ++s) {
        const bool up = ((s * 64 + lane) & size) == 0;  // this pair ends larger-first
        if (stride >= 64) {
          const int ps = s ^ (stride >> 6);
          if (ps > s) {
            const T a = v[s], b = v[ps];
            const bool sw = up ? (a < b) : (a > b);
            v[s] = sw ? b : a;
            v[ps] = sw ? a : b;
          }
        } else {
          const T o = shfl_xor_key(v[s], stride);
          const bool lower = (lane & stride) == 0;
          const T mx = v[s] > o ? v[s] : o, mn = v[s] > o ? o : v[s];
          v[s] = (lower == up) ? mx : mn;
        }
      }
    }
  }
}

// One wave: given its sorted keys (top k in lanes 0..k-1 of slot 0, k <= 64),
// writes their indices to out[] in ascending order.
__device__ __forceinline__ void wave_emit_ascending(uint64_t top, int k, int* out) {
  const int lane = threadIdx.x & 63;
  const uint32_t idx = ~static_cast<uint32_t>(top);
  uint64_t v[1] = {lane < k ? static_cast<uint64_t>(~idx) : 0ull};  // larger = lower index
  wave_sort_desc<1>(v);
  if (lane < k) out[lane] = static_cast<int>(~static_cast<uint32_t>(v[0]));
}

// Top-k for k < n <= blockDim.x: every thread ranks one key against all n
// (broadcast LDS reads, eight keys per step; the list is padded with zero
// keys, which rank below every real key); the k of rank < k are compacted
// in index order with wave ballots.  Same result as block_select.
// Block-wide.
__device__ __forceinline__ int rank_select(const uint32_t* keys, int n, int k, int* out, SelScratch& s) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int n8 = (n + 7) & ~7;
  uint64_t mine = 0;
  if (tid < n) mine = sel_key(keys[tid], tid);
  if (tid < n8) s.rk[tid] = mine;
  __syncthreads();
  int rank = 0;
  if (tid < n) {
    const ulonglong2* r2 = reinterpret_cast<const ulonglong2*>(s.rk);
    for (int j = 0; j < n8 / 2; j += 4) {
      const ulonglong2 a = r2[j], b = r2[j + 1], c = r2[j + 2], d = r2[j + 3];
      rank += (a.x > mine) + (a.y > mine) + (b.x > mine) + (b.y > mine) + (c.x > mine) +
              (c.y > mine) + (d.x > mine) + (d.y > mine);
    }
  }
  const bool take = tid < n && rank < k;
  const uint64_t m = __ballot(take);
  if (lane == 0) s.wsum[wave] = __popcll(m);
  __syncthreads();
  int pos = __popcll(m & ((1ull << lane) - 1ull));
  for (int w = 0; w < nw; ++w) pos += w < wave ? s.wsum[w] : 0;
  if (take) out[pos] = tid;
  __syncthreads();
  return k;
}

// Top-k (0 < k < n <= 64*S) by one wave, no barrier: the k-th largest key
// by a most-significant-bit-first search over wave ballots (key i held by
// lane i % 64 of slot i / 64; per bit, the alive keys with the bit set are
// counted from the ballots), the keys above it all taken, then the
// lowest-index keys equal to it; indices written to out[] ascending.  Same
// result as block_select.  key(i) gives the order key of candidate i.
template <int S, typename KeyAt>
__device__ __forceinline__ void wave_select(KeyAt key, int n, int k, int* out) {
  const int lane = threadIdx.x & 63;
  uint32_t v[S];
  uint64_t alive[S], sel[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int i = s * 64 + lane;
    v[s] = i < n ? key(i) : 0u;
    alive[s] = __ballot(i < n);
    sel[s] = 0ull;
  }
  int need = k, na = n;  // na: alive keys
  for (int b = 31; b >= 0 && need < na; --b) {
    uint64_t on[S];
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      on[s] = alive[s] & __ballot((v[s] >> b) & 1u);
      cnt += __popcll(on[s]);
    }
    if (cnt >= need) {
#pragma unroll
      for (int s = 0; s < S; ++s) alive[s] = on[s];
      na = cnt;
    } else {
      need -= cnt;
      na -= cnt;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        sel[s] |= on[s];
        alive[s] &= ~on[s];
      }
    }
  }
  // need == na: every alive key is taken; need < na only when the alive
  // keys are all equal (every bit decided), and the lowest indices go first
#pragma unroll
  for (int s = 0; s < S; ++s) {
    while (need > 0 && alive[s] != 0ull) {
      const uint64_t low = alive[s] & (~alive[s] + 1ull);
      sel[s] |= low;
      alive[s] ^= low;
      --need;
    }
  }
  int base = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if ((sel[s] >> lane) & 1ull) out[base + __popcll(sel[s] & ((1ull << lane) - 1ull))] = s * 64 + lane;
    base += __popcll(sel[s]);
  }
}

// Top-k selection for small inputs without the radix passes: n <= 128 with
// k <= 64 (one wave sorts everything), or n <= 128 * waves with k <= 16 (each
// wave sorts 128 keys and keeps its top k, one wave sorts the survivors).
// Same result as block_select.  Block-wide; every thread must call it.
__device__ __forceinline__ bool small_select_ok(int n, int k) {
  return (n <= 128 && k <= 64) || (k <= 16 && n <= 128 * static_cast<int>(blockDim.x >> 6));
}

__device__ __forceinline__ int small_select(const uint32_t* keys, int n, int k, int* out, SelScratch& sc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (n <= 128) {
    if (wave == 0) {
      uint64_t v[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int i = s * 64 + lane;
        v[s] = i < n ? sel_key(keys[i], i) : 0ull;
      }
      wave_sort_desc<2>(v);
      wave_emit_ascending(v[0], k, out);
    }
    __syncthreads();
    return k;
  }
  {
    uint64_t v[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int i = wave * 128 + s * 64 + lane;
      v[s] = i < n ? sel_key(keys[i], i) : 0ull;
    }
    wave_sort_desc<2>(v);
    if (lane < 16) sc.cand[wave * 16 + lane] = lane < k ? v[0] : 0ull;
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t v[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int i = s * 64 + lane;
      v[s] = i < nw * 16 ? sc.cand[i] : 0ull;
    }
    wave_sort_desc<2>(v);
    wave_emit_ascending(v[0], k, out);
  }
  __syncthreads();
  return k;
}

__device__ __forceinline__ int block_excl_scan(int v, SelScratch& s, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) s.wsum[wave] = inc;
  __syncthreads();
  int pre = 0;
  total = 0;
  for (int w = 0; w < nw; ++w) {
    const int x = s.wsum[w];
    if (w < wave) pre += x;
    total += x;
  }
  __syncthreads();
  return pre + inc - v;
}

// The k-th largest of keys[0..n) (0 < k < n) by an exact radix select over
// the 32-bit keys (four 8-bit digits, most significant first); need is set
// to how many keys equal to it rank among the k largest.  Block-wide; every
// thread must call it.
__device__ __forceinline__ uint32_t radix_kth(const uint32_t* keys, int n, int k, SelScratch& s, int& need) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t prefix = 0, pmask = 0;
  need = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += nt) s.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += nt) {
      const uint32_t kk = keys[i];
      if ((kk & pmask) == prefix) atomicAdd(&s.hist[(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      int c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s.hist[255 - 4 * tid - j];
        tot += c[j];
      }
      int inc = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(inc, off);
        if (tid >= off) inc += y;
      }
      const int excl = inc - tot;
      if (excl < need && need <= inc) {
        int above = excl;
        for (int j = 0; j < 4; ++j) {
          if (above + c[j] >= need) {
            s.bcast[0] = 255 - 4 * tid - j;
            s.bcast[1] = above;
            break;
          }
          above += c[j];
        }
      }
    }
    __syncthreads();
    const int digit = s.bcast[0];
    need -= s.bcast[1];
    prefix |= static_cast<uint32_t>(digit) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  return prefix;
}

// The k-th largest of keys[0..n) (0 < k < n).  For n <= 64 * waves and
// k <= 16: every wave sorts its 64 keys in registers and keeps its k
// largest, and one wave sorts the 16 * waves survivors (the k largest of
// the whole set are among them); otherwise radix_kth.  Block-wide; every
// thread must call it.
__device__ __forceinline__ uint32_t block_kth(const uint32_t* keys, int n, int k, SelScratch& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (n > 64 * nw || k > 16 || nw > 8) {
    int need;
    return radix_kth(keys, n, k, s, need);
  }
  uint32_t* cand = reinterpret_cast<uint32_t*>(s.cand);  // 128 entries
  {
    const int i = wave * 64 + lane;
    uint32_t v[1] = {i < n ? keys[i] : 0u};  // 0 ranks below every real key
    wave_sort_desc<1>(v);
    if (lane < 16) cand[wave * 16 + lane] = lane < k ? v[0] : 0u;
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t v[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = j * 64 + lane;
      v[j] = i < nw * 16 ? cand[i] : 0u;
    }
    wave_sort_desc<2>(v);
    if (lane == k - 1) s.bcast[2] = static_cast<int>(v[0]);
  }
  __syncthreads();
  return static_cast<uint32_t>(s.bcast[2]);
}

// Indices i < n with keys[i] >= thr into out[], ascending; returns their
// count.  Block-wide; every thread must call it.
__device__ __forceinline__ int block_compact_ge(const uint32_t* keys, int n, uint32_t thr, int* out,
                                                SelScratch& s) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (n <= nt) {  // one key per thread: wave ballots
    const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
    const bool take = tid < n && keys[tid] >= thr;
    const uint64_t m = __ballot(take);
    if (lane == 0) s.wsum[wave] = __popcll(m);
    __syncthreads();
    int pos = __popcll(m & ((1ull << lane) - 1ull)), total = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = s.wsum[w];
      pos += w < wave ? c : 0;
      total += c;
    }
    if (take) out[pos] = tid;
    __syncthreads();
    return total;
  }
  const int per = (n + nt - 1) / nt;
  const int lo = tid * per;
  const int hi = lo + per < n ? lo + per : n;
  int c = 0;
  for (int i = lo; i < hi; ++i) c += keys[i] >= thr;
  int total;
  int pos = block_excl_scan(c, s, total);
  for (int i = lo; i < hi; ++i)
    if (keys[i] >= thr) out[pos++] = i;
  __syncthreads();
  return total;
}

// Indices of the k largest keys[0..n) (ties to the lower index), ascending,
// into out[].  Exact radix select over the 32-bit keys, then a stable
// compaction in index order.  Block-wide; every thread must call it.
__device__ __forceinline__ int block_select(const uint32_t* keys, int n, int k, int* out, SelScratch& s) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (k <= 0 || n <= 0) return 0;
  if (n <= k) {
    for (int i = tid; i < n; i += nt) out[i] = i;
    __syncthreads();
    return n;
  }
  if (n <= static_cast<int>(blockDim.x) && n <= kRankMax) return rank_select(keys, n, k, out, s);
  if (small_select_ok(n, k)) return small_select(keys, n, k, out, s);
  int need;
  const uint32_t prefix = radix_kth(keys, n, k, s, need);
  const uint32_t thr = prefix;
  const int per = (n + nt - 1) / nt;
  const int lo = tid * per;
  const int hi = lo + per < n ? lo + per : n;
  int n_eq = 0;
  for (int i = lo; i < hi; ++i) n_eq += keys[i] == thr;
  int total;
  int eq_before = block_excl_scan(n_eq, s, total);
  int n_sel = 0;
  {
    int e = eq_before;
    for (int i = lo; i < hi; ++i) {
      const uint32_t kk = keys[i];
      if (kk > thr) {
        ++n_sel;
      } else if (kk == thr) {
        if (e < need) ++n_sel;
        ++e;
      }
    }
  }
  int pos = block_excl_scan(n_sel, s, total);
  {
    int e = eq_before;
    for (int i = lo; i < hi; ++i) {
      const uint32_t kk = keys[i];
      bool take = kk > thr;
      if (kk == thr) {
        take = e < need;
        ++e;
      }
      if (take) out[pos++] = i;
    }
  }
  __syncthreads();
  return k;
}

}  // namespace
}  // namespace hga
