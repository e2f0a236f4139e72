// Attention-aware drift test and tracking-set update, plus the FP8 codec check kernel.
//
// What it computes: Elastic-Cache (DAIR academy paper card), core idea -- cosine similarity
// of the previous step's most-attended tokens; when it drops below gamma the later layers are
// recomputed; the most-attended token drifts least, so the minimum over heads is a
// conservative trigger.  Flash-dLLM news summary, selective cache tracking -- a fixed budget
// of the 32 most-attended tokens.
//
// drift_track: one workgroup per (b, h).  The K||V rows of the tracked slots are compared in
// fp64 (16-byte loads, wave butterflies, then the four waves in order).  Then, when this
// step's mass is given, a radix select over the order-preserving bits of the mass (staged in
// LDS) finds the k-th largest value in four 8-bit passes; values above it are taken, and of
// the values equal to it the lowest positions, using two block scans so the set comes out in
// ascending position order; the tracking buffer is refilled from the current cache.
// drift_decide: one wave per sequence, any head below gamma.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) v += __shfl_xor(v, msk, kWave);
  return v;
}

// Block-wide exclusive scan of one count per thread (256 threads); returns this thread's
// exclusive prefix and writes the block total to *total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t base = inc - v;
  for (int q = 0; q < wave; ++q) base += wsum[q];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  return base;
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Elements of type E in one 16-byte chunk, read as fp64.
template <typename E>
__device__ __forceinline__ void load_chunk_f64(const E* p, double* out) {
  if constexpr (sizeof(E) == 2) {
    const uint4 w = *(const uint4*)p;
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = (double)__uint_as_float(x[e] << 16);
      out[2 * e + 1] = (double)__uint_as_float(x[e] & 0xffff0000u);
    }
  } else {
    const float4 w = *(const float4*)p;
    out[0] = w.x; out[1] = w.y; out[2] = w.z; out[3] = w.w;
  }
}

// One workgroup per (b, h): the drift of the previous tracked set, then (do_update) the new
// top-k set and the tracking-buffer refill.  All reads of the old set happen before the
// barrier that precedes the first write.
template <typename E>
__global__ __launch_bounds__(256) void drift_track(DriftArgs a, int do_update) {
  extern __shared__ uint32_t keys[];             // [S] order keys of this head's mass
  constexpr int EPC = 16 / (int)sizeof(E);       // elements per 16-byte chunk
  const int h = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int D = a.D, k = a.k, S = a.S;
  int32_t* T = a.track_idx + ((size_t)b * a.Hq + h) * k;
  E* buf = (E*)a.track_buf + ((size_t)b * a.Hq + h) * k * 2 * D;
  const E* kc = (const E*)a.kc;
  const E* vc = (const E*)a.vc;
  const size_t head_base = ((size_t)b * a.Hkv + g) * S;
  const int cpr = D / EPC;                       // chunks per K (or V) row

  __shared__ double red[3][4];
  __shared__ int sflag[4];
  __shared__ int32_t sT[64];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_rem, wsum[4];

  // ---- sigma over the previous tracked set (fp64) ----
  double uw = 0.0, uu = 0.0, ww = 0.0;
  int neq = 0;
  for (int c = t; c < k * 2 * cpr; c += 256) {
    const int slot = c / (2 * cpr), part = (c / cpr) & 1, d0 = (c % cpr) * EPC;
    const int j = T[slot];
    if (j < 0 || j >= S) continue;
    double u[EPC], w[EPC];
    load_chunk_f64<E>(buf + (size_t)c * EPC, u);
    load_chunk_f64<E>((part ? vc : kc) + (head_base + j) * D + d0, w);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      uw += u[e] * w[e];
      uu += u[e] * u[e];
      ww += w[e] * w[e];
      neq |= (u[e] != w[e]);
    }
  }
  const int valid_slot = (t < k) ? (T[t] >= 0 && T[t] < S) : 0;
  uw = wave_sum_f64(uw);
  uu = wave_sum_f64(uu);
  ww = wave_sum_f64(ww);
  const int wflags = (__any(neq) ? 1 : 0) | (__any(valid_slot) ? 2 : 0);
  if (lane == 0) {
    red[0][wave] = uw;
    red[1][wave] = uu;
    red[2][wave] = ww;
    sflag[wave] = wflags;
  }
  __syncthreads();
  if (t == 0) {
    double UW = 0.0, UU = 0.0, WW = 0.0;
    int F = 0;
    for (int q = 0; q < 4; ++q) {
      UW += red[0][q];
      UU += red[1][q];
      WW += red[2][q];
      F |= sflag[q];
    }
    double sigma;
    if (!(F & 2)) sigma = 1.0;
    else {
      const double den = sqrt(UU) * sqrt(WW);
      sigma = (den == 0.0) ? ((F & 1) ? 0.0 : 1.0) : UW / den;
    }
    // Report in fp32 on the side of gamma the fp64 value lies on.
    float f = (float)sigma;
    if (sigma < (double)a.gamma && !(f < a.gamma)) f = nextafterf(a.gamma, -INFINITY);
    a.sigma[(size_t)b * a.Hq + h] = f;
  }
  if (!do_update) return;
  __syncthreads();

  // ---- top-k of this step's mass: k-th largest value by 8-bit radix passes ----
  const float* mass = a.mass + ((size_t)b * a.Hq + h) * S;
  for (int j = t; j < S; j += 256) keys[j] = order_key(mass[j]);
  const uint32_t want = (uint32_t)min(k, S);
  uint32_t prefix = 0, pmask = 0, rem = want;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[t] = 0;
    __syncthreads();
    for (int j = t; j < S; j += 256) {
      const uint32_t u = keys[j];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // Lane L owns digits 255-4L .. 252-4L (descending); inclusive scan over lanes.
      uint32_t cnt[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt[e] = hist[255 - 4 * lane - e];
        own += cnt[e];
      }
      uint32_t inc = own;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
      }
      const uint32_t exc = inc - own;
      if (exc < rem && rem <= inc) {
        uint32_t above = exc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (above + cnt[e] >= rem) {
            s_digit = 255u - 4u * lane - e;
            s_rem = rem - above;
            break;
          }
          above += cnt[e];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 0xffu << shift;
    rem = s_rem;
  }
  // prefix is the k-th largest value; `rem` of the values equal to it are taken, lowest
  // positions first.  Selection in ascending position order over contiguous ranges.
  const int per = (S + 255) / 256;
  const int j0 = min(S, t * per), j1 = min(S, j0 + per);
  uint32_t ties = 0;
  for (int j = j0; j < j1; ++j) ties += (keys[j] == prefix);
  uint32_t tot;
  uint32_t tie_base = block_exclusive_scan(ties, wsum, &tot);
  uint32_t sel = 0;
  {
    uint32_t tb = tie_base;
    for (int j = j0; j < j1; ++j) {
      const uint32_t u = keys[j];
      if (u > prefix) ++sel;
      else if (u == prefix) sel += (tb++ < rem);
    }
  }
  uint32_t pos = block_exclusive_scan(sel, wsum, &tot);
  {
    uint32_t tb = tie_base;
    for (int j = j0; j < j1; ++j) {
      const uint32_t u = keys[j];
      const bool take = (u > prefix) || (u == prefix && tb++ < rem);
      if (take) {
        if (pos < (uint32_t)k) sT[pos] = j;
        ++pos;
      }
    }
  }
  __syncthreads();
  for (int sl = (int)want + t; sl < k; sl += 256) sT[sl] = -1;
  __syncthreads();
  for (int sl = t; sl < k; sl += 256) T[sl] = sT[sl];

  // ---- refill the tracking buffer with the K||V rows at the new positions ----
  for (int c = t; c < k * 2 * cpr; c += 256) {
    const int slot = c / (2 * cpr), part = (c / cpr) & 1, d0 = (c % cpr) * EPC;
    const int j = sT[slot];
    uint4 val = {0u, 0u, 0u, 0u};
    if (j >= 0) val = *(const uint4*)((part ? vc : kc) + (head_base + j) * D + d0);
    *(uint4*)(buf + (size_t)c * EPC) = val;
  }
}

// refresh[b] = any head of sequence b with sigma < gamma.  One wave per sequence.
__global__ __launch_bounds__(64) void drift_decide(DriftArgs a) {
  const int b = blockIdx.x;
  int any = 0;
  for (int h = threadIdx.x; h < a.Hq; h += 64) any |= (a.sigma[(size_t)b * a.Hq + h] < a.gamma);
  any = __any(any);
  if (threadIdx.x == 0) a.refresh[b] = (uint8_t)(any ? 1 : 0);
}

__global__ void fp8_roundtrip(const float* x, int64_t n, float scale, uint8_t* codes, float* dec) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t c = e4m3_encode(x[i] / scale);
  codes[i] = (uint8_t)c;
  if (dec) {
    uint32_t lo, hi;
    e4m3x4_to_bf16x4(c, lo, hi);
    dec[i] = bf16_to_f32((bf16_t)(lo & 0xffffu)) * scale;
  }
}

}  // namespace

hipError_t launch_drift(const DriftArgs& a, hipStream_t s) {
  dim3 grid(a.Hq, a.B);
  const int upd = a.mass != nullptr;
  const size_t lds = upd ? (size_t)a.S * sizeof(uint32_t) : 0;
  if (a.kind == kCacheF32) drift_track<float><<<grid, 256, lds, s>>>(a, upd);
  else drift_track<bf16_t><<<grid, 256, lds, s>>>(a, upd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  drift_decide<<<a.B, 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fp8_roundtrip(const float* x, int64_t n, float scale, uint8_t* codes,
                                float* decoded, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  fp8_roundtrip<<<(unsigned)blocks, 256, 0, s>>>(x, n, scale, codes, decoded);
  return hipGetLastError();
}

}  // namespace dllm
