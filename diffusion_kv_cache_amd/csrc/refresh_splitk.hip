// Refresh for small M (a block step of one or a few sequences): the weight stream dominates,
// so the projection is split over the four fixed K-partitions across workgroups.
//
//   refresh_partial: workgroup (192 output columns, partition p, 32 rows).  The 32 x H/4 slice
//     of the gathered hidden rows is staged once in LDS with coalesced 16-byte loads; each of
//     the twelve waves streams 16 W rows of that partition from global memory with a deep
//     register prefetch and chains 16x16x32 MFMAs over the partition in ascending k.  The
//     partition's fp32 tile goes to the workspace as whole rows (staged in LDS).
//   refresh_reduce: adds the four partitions in order (((0 + P0) + P1) + P2) + P3 -- exactly
//     the arithmetic of the tiled kernel -- rotates the Q and K pairs (i, i + D/2), and writes
//     Q, K and V rows (bf16, or per-row FP8 with its fp32 scale).
//
// What it computes: Flash-dLLM news summary (skillfed.io), memory paragraph -- projection,
// RoPE and cache write of the refreshed rows; LaCache (gist.science), Technical Summary,
// Methodology 1 (RoPECache: post-projection, post-RoPE states) and 2 (1 x 128 FP8 groups).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

constexpr int kPrefetch = 8;   // k-steps of W in flight per wave
constexpr int kPartWaves = 12;                 // waves per workgroup, 16 columns each
constexpr int kPartCols = 16 * kPartWaves;     // output columns per workgroup
constexpr int kPartLd = kPartCols + 4;         // floats per staged partial row (no bank conflicts)

// A 4096-hidden, 12288-column step is 4 x 64 workgroups: one per CU, three waves per SIMD,
// each wave streaming 32 KB of W.  (Eight partitions of 128-column workgroups, three per CU,
// took 27.0 against 25.1 us for the pair of kernels on that step: the partials they write and
// read back are twice as large.)  Up to 64 rows, two workgroups share a CU.
__global__ __launch_bounds__(64 * kPartWaves) __attribute__((amdgpu_waves_per_eu(6)))
void refresh_partial(RefreshArgs a, float* part) {
  extern __shared__ u32x4 As[];                  // [32 rows][cpr chunks], swizzled
  // Rows present (a variable-length batch may hold fewer than its capacity): they set the
  // workspace's row stride here and in refresh_reduce alike.
  a.M = live_rows(a.cu, a.B, a.M);
  if ((int)blockIdx.z * 32 >= a.M) return;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, l16 = lane & 15, lg = lane >> 4;
  const int N = (a.Hq + 2 * a.Hkv) * a.D;
  const int p = blockIdx.x;                      // partitions fastest: the four workgroups
  const int m0 = blockIdx.z * 32;                // of a column tile are dispatched together
  const int Lp = a.H / kKSplit, kb = p * Lp;
  const int cpr = Lp / 8;                        // 16-byte chunks per staged row
  const int mask = (cpr % 8 == 0) ? 7 : 3;

  // Prologue: the first W steps go out before anything else (they depend on nothing); then
  // the 32 row positions, then the gathered A slice global -> LDS by DMA (each lane fetches
  // the source chunk that lands, swizzled, at its LDS slot).  Rows past M gather the last
  // valid row: their accumulators are never stored.
  const int col = blockIdx.y * kPartCols + wave * 16 + l16;  // columns past N compute, not stored
  const bf16_t* wr = (const bf16_t*)a.w + (size_t)min(col, N - 1) * a.H + kb + lg * 8;
  const int steps = Lp / 32;
  u32x4 wv[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) wv[u] = *(const u32x4*)(wr + min(u, steps - 1) * 32);
  __shared__ int s_row[32];                      // hidden row offset (b * S + pos) per A row
  if (t < 32) {
    const int m = min(m0 + t, a.M - 1);
    s_row[t] = seq_of_row(a.cu, a.B, a.n, m) * a.S + a.idx[m];
  }
  lds_barrier();
  const bf16_t* hid = (const bf16_t*)a.hidden;
  const int nblk = 32 * cpr / 64;                // 1 KB DMA blocks of the A slice
  for (int blk = wave; blk < nblk; blk += kPartWaves) {
    const int P = blk * 64 + lane;               // chunk slot in As
    const int r = P / cpr, j = P % cpr;
    const bf16_t* src = hid + (size_t)s_row[r] * a.H + kb + (j ^ (r & mask)) * 8;
    dma_16B(src, As + blk * 64);
  }
  DLLM_WAIT_VMCNT(0);
  __syncthreads();

  // A ring of kPrefetch W steps in registers: slot u holds step s0 + u; right after it is
  // consumed it is refilled with step s0 + u + kPrefetch, so kPrefetch - 1 loads stay in
  // flight while each step's MFMAs run.  The last round issues no loads (no branch around a
  // load anywhere, which keeps the compiler's count of loads in flight exact).
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  auto step = [&](int st, const u32x4& wq) {
    const int c = st * 4 + lg;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = rt * 16 + l16;
      acc[rt] = mfma_bf16(as_bf16x8(As[r * cpr + (c ^ (r & mask))]), as_bf16x8(wq), acc[rt]);
    }
  };
  int s0 = 0;
  for (; s0 + kPrefetch < steps; s0 += kPrefetch) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      step(s0 + u, wv[u]);
      wv[u] = *(const u32x4*)(wr + min(s0 + u + kPrefetch, steps - 1) * 32);
    }
  }
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u)
    if (s0 + u < steps) step(s0 + u, wv[u]);

  // The 32 x 192 partial tile goes out as whole rows: staged in LDS (over the A slice, which
  // every wave is done reading), then 16-byte stores of 768-byte row segments.
  __syncthreads();
  float* T = (float*)As;                         // [32][kPartLd]
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) T[(rt * 16 + lg * 4 + v) * kPartLd + wave * 16 + l16] = acc[rt][v];
  __syncthreads();
  constexpr int V4 = kPartCols / 4;              // 16-byte vectors per staged row
#pragma unroll
  for (int u = 0; u < 32 * V4 / (64 * kPartWaves); ++u) {
    const int id = u * 64 * kPartWaves + t, r = id / V4, c4 = (id % V4) * 4;
    const int m = m0 + r, cc = blockIdx.y * kPartCols + c4;
    if (m < a.M && cc < N)
      *(float4*)(part + ((size_t)p * a.M + m) * N + cc) = *(const float4*)(T + r * kPartLd + c4);
  }
}

// One 16-lane group per (row, head): lane L of the group owns the rotary pairs
// (i, i + D/2) for i in [L * PPL, L * PPL + PPL), read as PPL-float vectors from each
// partition.  A wave takes four consecutive (row, head) items.
template <int D, int KIND>
__global__ __launch_bounds__(64) void refresh_reduce(RefreshArgs a, const float* part) {
  constexpr int HALF = D / 2;
  a.M = live_rows(a.cu, a.B, a.M);
  constexpr int PPL = HALF / 16;                 // pairs per lane: 4 (D = 128) or 2 (D = 64)
  typedef __attribute__((ext_vector_type(PPL))) float fvec;
  const int lane = threadIdx.x, L = lane & 15;
  const int heads = a.Hq + 2 * a.Hkv, N = heads * D;
  const int item = blockIdx.x * 4 + (lane >> 4);
  const bool ok = item < a.M * heads;
  const int it = ok ? item : 0;
  const int m = it / heads, j = it % heads;
  // All the partials and the row position are requested first: one round trip, and the
  // rotation frequencies below (fp64) are formed while it is in flight.
  const int pos = a.idx[m];
  fvec px[kKSplit], py[kKSplit];
#pragma unroll
  for (int p = 0; p < kKSplit; ++p) {
    const float* row = part + ((size_t)p * a.M + m) * N + j * D + L * PPL;
    px[p] = *(const fvec*)row;
    py[p] = *(const fvec*)(row + HALF);
  }
  __builtin_amdgcn_sched_barrier(0);             // keep every load ahead of the arithmetic
  // every lane forms the rotation frequency of pair (lane mod D/2); the group's lanes
  // fetch theirs by shuffle
  float hi_own, lo_own;
  rope_turns(lane % HALF, D, a.rope_base, hi_own, lo_own);
  fvec x = {}, y = {};
#pragma unroll
  for (int p = 0; p < kKSplit; ++p) {
    x = x + px[p];
    y = y + py[p];
  }
  const bool rot = j < a.Hq + a.Hkv;
#pragma unroll
  for (int e = 0; e < PPL; ++e) {
    const float hi = __shfl(hi_own, L * PPL + e, kWave), lo = __shfl(lo_own, L * PPL + e, kWave);
    if (rot) {
      float sn, cs, xe = x[e], ye = y[e];
      rope_sincos(pos, hi, lo, sn, cs);
      rope_rotate(xe, ye, sn, cs);
      x[e] = xe;
      y[e] = ye;
    }
  }
  const int b = seq_of_row(a.cu, a.B, a.n, m);
  const int i0 = L * PPL;
  if (j < a.Hq) {
    if (ok) {
      bf16_t* q = (bf16_t*)a.q_out + ((size_t)m * a.Hq + j) * D;
#pragma unroll
      for (int e = 0; e < PPL; ++e) {
        q[i0 + e] = f32_to_bf16(x[e]);
        q[i0 + e + HALF] = f32_to_bf16(y[e]);
      }
    }
    return;
  }
  const bool is_k = j < a.Hq + a.Hkv;
  const int g = is_k ? j - a.Hq : j - a.Hq - a.Hkv;
  const size_t row = ((size_t)b * a.Hkv + g) * a.S + pos;
  if constexpr (KIND == kCacheFP8) {
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < PPL; ++e) am = fmaxf(am, fmaxf(fabsf(x[e]), fabsf(y[e])));
#pragma unroll
    for (int msk = 1; msk < 16; msk <<= 1) am = fmaxf(am, __shfl_xor(am, msk, kWave));
    const float scale = (am == 0.f) ? 1.f : am / 448.f;
    if (ok) {
      uint8_t* dst = (uint8_t*)(is_k ? a.kc : a.vc) + row * D;
#pragma unroll
      for (int e = 0; e < PPL; ++e) {
        dst[i0 + e] = (uint8_t)e4m3_encode(x[e] / scale);
        dst[i0 + e + HALF] = (uint8_t)e4m3_encode(y[e] / scale);
      }
      if (L == 0) (is_k ? a.ks : a.vs)[row] = scale;
    }
  } else {
    if (ok) {
      bf16_t* dst = (bf16_t*)(is_k ? a.kc : a.vc) + row * D;
#pragma unroll
      for (int e = 0; e < PPL; ++e) {
        dst[i0 + e] = f32_to_bf16(x[e]);
        dst[i0 + e + HALF] = f32_to_bf16(y[e]);
      }
    }
  }
}

template <int D>
hipError_t launch_reduce(const RefreshArgs& a, const float* part, hipStream_t s) {
  const long long items = (long long)a.M * (a.Hq + 2 * a.Hkv);
  const unsigned grid = (unsigned)((items + 3) / 4);
  if (a.kind == kCacheFP8) refresh_reduce<D, kCacheFP8><<<grid, 64, 0, s>>>(a, part);
  else refresh_reduce<D, kCacheBF16><<<grid, 64, 0, s>>>(a, part);
  return hipGetLastError();
}

}  // namespace

size_t splitk_workspace_bytes(int M, int N) { return (size_t)kKSplit * M * N * sizeof(float); }

hipError_t launch_refresh_splitk(const RefreshArgs& a, float* part, hipStream_t s) {
  const int N = (a.Hq + 2 * a.Hkv) * a.D;
  dim3 grid(kKSplit, (N + kPartCols - 1) / kPartCols, (a.M + 31) / 32);
  const size_t lds = std::max((size_t)32 * (a.H / kKSplit) * sizeof(bf16_t),
                              (size_t)32 * kPartLd * sizeof(float));
  refresh_partial<<<grid, 64 * kPartWaves, lds, s>>>(a, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.D == 128 ? launch_reduce<128>(a, part, s) : launch_reduce<64>(a, part, s);
}

}  // namespace dllm
