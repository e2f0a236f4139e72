// Attention-aware drift test and tracking-set update, plus the FP8 codec check kernel.
//
// What it computes: Elastic-Cache (DAIR academy paper card), core idea -- cosine similarity
// of the previous step's most-attended tokens; when it drops below gamma the later layers are
// recomputed; the most-attended token drifts least, so the minimum over heads is a
// conservative trigger.  Flash-dLLM news summary, selective cache tracking -- a fixed budget
// of the 32 most-attended tokens.
//
// drift_sigma: one workgroup per (b, h); the K||V rows of the tracked slots are compared in
// fp64 (wave butterflies, then the four waves in order).  track_update: one workgroup per
// (b, h); radix select over 64-bit keys (order-preserving mass bits, then the inverted
// position so lower positions win ties) finds the k-th largest key in eight 8-bit passes,
// a block scan writes the selected positions in ascending order, and the tracking buffer
// is refilled from the current cache.
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

template <typename E>
__device__ __forceinline__ double load_f64(const E* p, size_t i) {
  if constexpr (sizeof(E) == 2) return (double)bf16_to_f32(((const bf16_t*)p)[i]);
  else return (double)((const float*)p)[i];
}

template <typename E>
__global__ __launch_bounds__(256) void drift_sigma(DriftArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int D = a.D, k = a.k;
  const int32_t* T = a.track_idx + ((size_t)b * a.Hq + h) * k;
  const E* buf = (const E*)a.track_buf + ((size_t)b * a.Hq + h) * k * 2 * D;
  const E* kc = (const E*)a.kc;
  const E* vc = (const E*)a.vc;
  const size_t head_base = ((size_t)b * a.Hkv + g) * a.S;
  double uw = 0.0, uu = 0.0, ww = 0.0;
  int neq = 0;
  const int total = k * 2 * D;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int slot = e / (2 * D), part = (e / D) & 1, d = e % D;
    const int j = T[slot];
    if (j < 0 || j >= a.S) continue;
    const double u = load_f64(buf, (size_t)e);
    const double w = load_f64(part ? vc : kc, (head_base + j) * D + d);
    uw += u * w;
    uu += u * u;
    ww += w * w;
    neq |= (u != w);
  }
  __shared__ double red[3][4];
  __shared__ int sneq[4];
  uw = wave_sum_f64(uw);
  uu = wave_sum_f64(uu);
  ww = wave_sum_f64(ww);
  const int wn = __any(neq) ? 1 : 0;
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = uw;
    red[1][wave] = uu;
    red[2][wave] = ww;
    sneq[wave] = wn;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double UW = 0.0, UU = 0.0, WW = 0.0;
  int NEQ = 0;
  for (int q = 0; q < 4; ++q) {
    UW += red[0][q];
    UU += red[1][q];
    WW += red[2][q];
    NEQ |= sneq[q];
  }
  int valid = 0;
  for (int s = 0; s < k; ++s) valid += (T[s] >= 0 && T[s] < a.S);
  double sigma;
  if (!valid) sigma = 1.0;
  else {
    const double den = sqrt(UU) * sqrt(WW);
    sigma = (den == 0.0) ? (NEQ ? 0.0 : 1.0) : UW / den;
  }
  // Report in fp32 on the side of gamma the fp64 value lies on.
  float f = (float)sigma;
  if (sigma < (double)a.gamma && !(f < a.gamma)) f = nextafterf(a.gamma, -INFINITY);
  a.sigma[(size_t)b * a.Hq + h] = f;
}

__device__ __forceinline__ uint64_t rank_key(float mass, int j) {
  uint32_t u = __float_as_uint(mass);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
}

template <typename E>
__global__ __launch_bounds__(256) void track_update(DriftArgs a, int do_update) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (h == 0 && t == 0) {
    int any = 0;
    for (int hh = 0; hh < a.Hq; ++hh) any |= (a.sigma[(size_t)b * a.Hq + hh] < a.gamma);
    a.refresh[b] = (uint8_t)any;
  }
  if (!do_update) return;

  const int S = a.S, k = a.k, D = a.D;
  const float* mass = a.mass + ((size_t)b * a.Hq + h) * S;
  const int want = min(k, S);

  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_rem;
  __shared__ uint32_t wsum[4];
  __shared__ int32_t sT[64];

  uint64_t prefix = 0, pmask = 0;
  uint32_t rem = (uint32_t)want;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    hist[t] = 0;
    __syncthreads();
    for (int j = t; j < S; j += 256) {
      const uint64_t key = rank_key(mass[j], j);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // Lane L owns digits 255-4L .. 252-4L (descending); inclusive scan over lanes.
      uint32_t c[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * lane - e];
        own += c[e];
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
          if (above + c[e] >= rem) {
            s_digit = 255u - 4u * lane - e;
            s_rem = rem - above;
            break;
          }
          above += c[e];
        }
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s_digit << shift;
    pmask |= (uint64_t)0xffu << shift;
    rem = s_rem;
    __syncthreads();
  }
  const uint64_t kth = prefix;

  // Selected positions in ascending order: contiguous ranges per thread + block scan.
  const int per = (S + 255) / 256;
  const int j0 = t * per, j1 = min(S, j0 + per);
  uint32_t cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += rank_key(mass[j], j) >= kth;
  uint32_t inc = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t base = inc - cnt;
  for (int q = 0; q < wave; ++q) base += wsum[q];
  for (int j = j0; j < j1; ++j)
    if (rank_key(mass[j], j) >= kth) {
      if (base < (uint32_t)k) sT[base] = j;
      ++base;
    }
  __syncthreads();
  for (int s = want + t; s < k; s += 256) sT[s] = -1;
  __syncthreads();

  int32_t* T = a.track_idx + ((size_t)b * a.Hq + h) * k;
  for (int s = t; s < k; s += 256) T[s] = sT[s];

  // Refill the tracking buffer with the K||V rows at the new positions.
  const int G = a.Hq / a.Hkv, g = h / G;
  const size_t head_base = ((size_t)b * a.Hkv + g) * S;
  E* buf = (E*)a.track_buf + ((size_t)b * a.Hq + h) * k * 2 * D;
  const E* kc = (const E*)a.kc;
  const E* vc = (const E*)a.vc;
  for (int e = t; e < k * 2 * D; e += 256) {
    const int slot = e / (2 * D), part = (e / D) & 1, d = e % D;
    const int j = sT[slot];
    E val = E(0);
    if (j >= 0) val = (part ? vc : kc)[(head_base + j) * D + d];
    buf[e] = val;
  }
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
  if (a.kind == kCacheF32) {
    drift_sigma<float><<<grid, 256, 0, s>>>(a);
    track_update<float><<<grid, 256, 0, s>>>(a, a.mass != nullptr);
  } else {
    drift_sigma<bf16_t><<<grid, 256, 0, s>>>(a);
    track_update<bf16_t><<<grid, 256, 0, s>>>(a, a.mass != nullptr);
  }
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
