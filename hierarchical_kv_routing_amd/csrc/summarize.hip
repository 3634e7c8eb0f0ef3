// Mixed-RoPE chunk and group key summaries plus the rotated key cache.
//
// Source: xllm-io paper-review page of "Hierarchical Global Attention",
// section 3, Mixed-RoPE routing summaries (summary equation) and the
// framework paragraph (chunks of C tokens split into groups of g_s tokens;
// closed chunks carry a chunk summary and group summaries).
//
// One workgroup per (chunk, kv head, sequence), 4 waves.  Lane p owns RoPE
// pair p = (k[p], k[p + d/2]); wave w walks groups w, w+4, ... of the chunk
// token by token (each token row is read once, coalesced across lanes), so
// the group sums live in registers.  The chunk sum is the sum of the group
// sums taken over the 4 waves in a fixed order, so results are bitwise
// reproducible.  Work is HBM-streaming: d*elem bytes read per token plus the
// k_rot write.
#include "hga_device.h"

namespace hga {
namespace {

constexpr int kSumWaves = 4;

// sin and cos of a (double): reduction to r in [-pi, pi] (two-part 2*pi,
// as rope_cs), Taylor series at x = r/16 (|x| < 0.2; terms through x^11
// and x^12, below 1e-18), then four angle doublings; for the per-token step
// of the rotation, where a relative error of 1e-15 is far below the f32
// rounding that follows.
__device__ __forceinline__ void sincos_step(double a, double& sn, double& cs) {
  const double kTwoPiHi = 6.283185307179586;
  const double kTwoPiLo = 2.4492935982947064e-16;
  const double kInvTwoPi = 0.15915494309189535;
  const double k = rint(a * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, a);
  r = fma(-k, kTwoPiLo, r);
  const double x = r * 0.0625;
  const double x2 = x * x;
  double sv = fma(x2, -1.0 / 39916800.0, 1.0 / 362880.0);
  sv = fma(x2, sv, -1.0 / 5040.0);
  sv = fma(x2, sv, 1.0 / 120.0);
  sv = fma(x2, sv, -1.0 / 6.0);
  sv = fma(x2 * x, sv, x);
  double cv = fma(x2, 1.0 / 479001600.0, -1.0 / 3628800.0);
  cv = fma(x2, cv, 1.0 / 40320.0);
  cv = fma(x2, cv, -1.0 / 720.0);
  cv = fma(x2, cv, 1.0 / 24.0);
  cv = fma(x2, cv, -0.5);
  cv = fma(x2, cv, 1.0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double s2 = 2.0 * sv * cv;
    cv = fma(cv, cv, -sv * sv);
    sv = s2;
  }
  sn = sv;
  cs = cv;
}

struct SumParams {
  const void* k_raw;
  void* k_rot;
  float* chunk_sum;
  float* group_sum;
  int64_t kv_cap, tok_begin, tok_end, chunk_first;
  // k_raw / k_rot hold tokens [k_first, k_first + k_rows) of every
  // (sequence, KV head), k_rows rows apart (the whole cache: 0, kv_cap)
  int64_t k_first, k_rows;
  int Hkv, d, C, gs, r, n_hf;
  RopeFreqs rope;
};

template <bool BF16, int D>
__global__ __launch_bounds__(kSumWaves * 64) void summarize_kernel(SumParams p) {
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  constexpr int h = D / 2;
  const int64_t m = p.chunk_first + blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t slab = (static_cast<int64_t>(b) * p.Hkv + kvh) * p.k_rows - p.k_first;
  const int64_t c0 = m * p.C;
  const int64_t c1 = c0 + p.C;
  const int64_t tend = c1 < p.tok_end ? c1 : p.tok_end;
  const bool active = lane < h;
  const double freq = active ? rope_freq(p.rope, lane) : 0.0;
  const bool high = lane < p.n_hf;
  double cs1, sn1;  // cos/sin of one position step of the pair
  sincos_step(freq, sn1, cs1);

  float cx = 0.f, cy = 0.f;  // chunk partial sums of this wave (rotated or raw per pair kind)
  for (int g = wave; g < p.r; g += kSumWaves) {
    const int64_t g0 = c0 + static_cast<int64_t>(g) * p.gs;
    const int64_t g1 = g0 + p.gs;
    const int64_t jend = g1 < tend ? g1 : tend;
    const int64_t gw = rope_base(p.rope, g0);  // rotation position of token g0
    float sx = 0.f, sy = 0.f;
    if (active) {
      // cos/sin at the group's first position as rope_cs gives them; each
      // later token's by one more rotation by theta, carried in double so
      // that the g_s - 1 steps add no f32 roundings (every token's pair is
      // within about one f32 ulp of the exact cos/sin, like rope_cs's)
      float c0, s0;
      rope_cs(static_cast<double>(gw), freq, c0, s0);
      double c = c0, s = s0;
      constexpr int kBatch = 8;  // token rows in flight per lane
      for (int64_t j0 = g0; j0 < jend; j0 += kBatch) {
        float xs[kBatch], ys[kBatch];
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
          const int64_t e = (slab + (j0 + t < jend ? j0 + t : j0)) * D + lane;
          xs[t] = load1<BF16>(p.k_raw, e);
          ys[t] = load1<BF16>(p.k_raw, e + h);
        }
#pragma unroll
        for (int t = 0; t < kBatch; ++t) {
          const int64_t j = j0 + t;
          if (j < jend) {
            const float x = xs[t], y = ys[t];
            const float cf = static_cast<float>(c), sf = static_cast<float>(s);
            const float rx = x * cf - y * sf;
            const float ry = x * sf + y * cf;
            if (p.k_rot != nullptr && j >= p.tok_begin) {
              const int64_t e = (slab + j) * D + lane;
              store1<BF16>(p.k_rot, e, rx);
              store1<BF16>(p.k_rot, e + h, ry);
            }
            // high-frequency pairs average rotated keys, low-frequency pairs raw keys
            sx += high ? rx : x;
            sy += high ? ry : y;
            const double cn = c * cs1 - s * sn1;
            s = s * cs1 + c * sn1;
            c = cn;
          }
        }
      }
      const bool done = g1 <= p.tok_end && g1 > p.tok_begin;
      if (done && p.group_sum != nullptr) {
        const float inv_n = static_cast<float>(p.gs);
        float ox = sx / inv_n, oy = sy / inv_n;
        if (!high) {
          float c, s;
          rope_cs(static_cast<double>(gw) + 0.5 * (p.gs - 1), freq, c, s);
          const float mx = ox, my = oy;
          ox = mx * c - my * s;
          oy = mx * s + my * c;
        }
        const int64_t row = (static_cast<int64_t>(b) * p.Hkv + kvh) * (p.kv_cap / p.gs) + g0 / p.gs;
        p.group_sum[row * D + lane] = ox;
        p.group_sum[row * D + lane + h] = oy;
      }
    }
    cx += sx;
    cy += sy;
  }

  const bool chunk_done = c1 <= p.tok_end && c1 > p.tok_begin;  // uniform over the block
  if (!chunk_done) return;
  __shared__ float part[kSumWaves][64][2];
  part[wave][lane][0] = cx;
  part[wave][lane][1] = cy;
  __syncthreads();
  if (wave == 0 && active) {
    float sx = 0.f, sy = 0.f;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) {
      sx += part[w][lane][0];
      sy += part[w][lane][1];
    }
    const float n = static_cast<float>(p.C);
    float ox = sx / n, oy = sy / n;
    if (!high) {
      float c, s;
      rope_cs(static_cast<double>(rope_base(p.rope, c0)) + 0.5 * (p.C - 1), freq, c, s);
      const float mx = ox, my = oy;
      ox = mx * c - my * s;
      oy = mx * s + my * c;
    }
    const int64_t row = (static_cast<int64_t>(b) * p.Hkv + kvh) * (p.kv_cap / p.C) + m;
    p.chunk_sum[row * D + lane] = ox;
    p.chunk_sum[row * D + lane + h] = oy;
  }
}

}  // namespace

hipError_t launch_summarize(const Geometry& g, const void* k_raw, int64_t tok_begin,
                            int64_t tok_end, void* k_rot, float* chunk_sum,
                            float* group_sum, hipStream_t stream, int64_t k_first,
                            int64_t k_rows) {
  SumParams p;
  p.k_first = k_first;
  p.k_rows = k_rows > 0 ? k_rows : g.kv_cap;
  p.k_raw = k_raw;
  p.k_rot = k_rot;
  p.chunk_sum = chunk_sum;
  p.group_sum = group_sum;
  p.kv_cap = g.kv_cap;
  p.tok_begin = tok_begin;
  p.tok_end = tok_end;
  p.chunk_first = tok_begin / g.C;
  p.Hkv = g.Hkv;
  p.d = g.d;
  p.C = g.C;
  p.gs = g.gs;
  p.r = g.r;
  p.n_hf = g.n_hf;
  p.rope = g.rope;
  const int64_t chunk_last = (tok_end - 1) / g.C;
  dim3 grid(static_cast<unsigned>(chunk_last - p.chunk_first + 1), g.Hkv, g.B);
  dim3 block(kSumWaves * 64);
  // head_dim is 64 or 128 (checked with the configuration)
  if (g.bf16) {
    if (g.d == 128) hipLaunchKernelGGL((summarize_kernel<true, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((summarize_kernel<true, 64>), grid, block, 0, stream, p);
  } else {
    if (g.d == 128) hipLaunchKernelGGL((summarize_kernel<false, 128>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((summarize_kernel<false, 64>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace hga
