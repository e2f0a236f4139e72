// Split-KV merge and the column attention-mass pass of the block attention, the fp32 path,
// and the launcher (the MFMA forward pass is in attention_fwd.hip).
//
// What it computes: softmax(q k^T * scale) v with no mask (Flash-Cache article, section 3.1;
// LaCache Technical Summary, Problem Statement: bidirectional attention over the full
// context); the online-softmax state (m, l, O~) and its merge over disjoint key ranges
// (LaCache Methodology 1, FACache); the column mass sum_i p_ij that ranks the most-attended
// tokens (Flash-dLLM summary, selective cache tracking).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKeys = 32;          // keys per tile

// Combine split partial states in split order: one wave per packed query row.
template <typename OutT, int D>
__global__ __launch_bounds__(64) void attn_merge(AttnArgs a, int splits) {
  const int G = a.Hq / a.Hkv;
  const int rows = a.n * G;
  const size_t nrows_all = (size_t)a.B * a.Hkv * rows;
  const size_t pr0 = blockIdx.x;  // bg * rows + r
  const int bg = (int)(pr0 / rows), r = (int)(pr0 % rows);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const float* ml = a.part + (size_t)splits * nrows_all * D;
  float mm = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) mm = fmaxf(mm, ml[((size_t)sp * nrows_all + pr0) * 2]);
  float L = 0.f;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const size_t pr = (size_t)sp * nrows_all + pr0;
    const float ms = ml[pr * 2], ls = ml[pr * 2 + 1];
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - mm);
    L += ls * wgt;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += a.part[pr * D + threadIdx.x + 64 * e] * wgt;
  }
  const int i = r / G, h = g * G + r % G;
  OutT* out = (OutT*)a.out + (((size_t)b * a.n + i) * a.Hq + h) * D;
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float val = o[e] * inv;
    if constexpr (sizeof(OutT) == 2) out[threadIdx.x + 64 * e] = f32_to_bf16(val);
    else out[threadIdx.x + 64 * e] = val;
  }
  if (threadIdx.x == 0) a.lse[((size_t)b * a.Hq + h) * a.n + i] = (mm + log2f(L)) * kLn2;
}

// Largest packed-row count (n * G) whose log-sum-exp the fused merge + mass kernel stages in
// LDS (32 KB); larger problems merge in attn_merge first.
constexpr int kFusedMergeRows = 8192;

// Merged state of packed row pr0 from the split partials, in split order (the same arithmetic
// as attn_merge): running max mm and normaliser L.
__device__ __forceinline__ void merged_ml(const float* ml, size_t nrows_all, size_t pr0, int splits,
                                          float& mm, float& L) {
  mm = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) mm = fmaxf(mm, ml[((size_t)sp * nrows_all + pr0) * 2]);
  L = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const size_t pr = (size_t)sp * nrows_all + pr0;
    const float ms = ml[pr * 2], ls = ml[pr * 2 + 1];
    L += ls * ((ms == -INFINITY) ? 0.f : exp2f(ms - mm));
  }
}

// Column attention mass, second pass after the log-sum-exp is known:
//   mass[b, h, j] = sum_i exp(<q_i, k_j> * scale - lse_i).
// One workgroup per (b, KV head g) and 128 keys, so each K row is read once for all G query
// heads of its group: each wave keeps 32 keys' K rows as MFMA A operands (S^T = K Q^T), then
// for each query head streams its n queries in tiles of 16 (the next tile's loads in flight
// during the current one's MFMAs and exponentials).  Lane (l16, lg) sums query column l16 over
// the tiles in order; the 16 lanes of a key are added at the end in a fixed butterfly order.
//
// MERGE (the attention was split over keys): the kernel first forms every packed row's
// log-sum-exp from the split partials (staged in LDS), the workgroups of key chunk 0 write
// it, and the rows' outputs are merged here too (rows dealt round-robin over the key chunks),
// so no separate merge launch is needed.
template <int KIND, int D, bool MERGE>
__global__ __launch_bounds__(256) void attn_mass_mfma(AttnArgs a, int splits) {
  extern __shared__ float lse2_s[];              // MERGE: [n * G] log2-domain LSE
  constexpr int DS = D / 32;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  // All key chunks of one (b, KV head) run on one XCD: the group's queries are fetched into
  // that L2 once.
  const int nkc = (a.S + 127) / 128;
  int bg, kchunk;
  xcd_group_unit(blockIdx.x, a.B * a.Hkv, nkc, bg, kchunk);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = a.n * G;
  const int key0 = kchunk * 128 + wave * 32;
  const size_t head_base = ((size_t)b * a.Hkv + g) * a.S;
  constexpr int ELT = (KIND == kCacheFP8) ? 1 : 2;
  const char* kc = (const char*)a.kc;

  bf16x8 kf[2][DS];
  float ksc[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = key0 + kt * 16 + l16;
    const bool ok = key < a.S;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const size_t off = ((head_base + (ok ? key : 0)) * D + ds * 32 + lg * 8) * ELT;
      u32x4 x;
      if constexpr (KIND == kCacheFP8) {
        const uint2 w8 = *(const uint2*)(kc + off);
        x = e4m3x8_to_bf16x8(w8.x, w8.y);
      } else {
        x = *(const u32x4*)(kc + off);
      }
      kf[kt][ds] = as_bf16x8(ok ? x : u32x4{0u, 0u, 0u, 0u});
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int kr = key0 + kt * 16 + lg * 4 + v;
      if constexpr (KIND == kCacheFP8) ksc[kt][v] = (kr < a.S) ? a.ks[head_base + kr] : 0.f;
      else ksc[kt][v] = 1.f;
    }
  }

  const size_t nrows_all = (size_t)a.B * a.Hkv * rows;
  const float* ml = a.part + (size_t)splits * nrows_all * D;
  if constexpr (MERGE) {
    for (int r = t; r < rows; r += 256) {
      float mm, L;
      merged_ml(ml, nrows_all, (size_t)bg * rows + r, splits, mm, L);
      const float l2 = mm + log2f(L);
      lse2_s[r] = l2;
      if (kchunk == 0) {
        const int i = r / G, h = g * G + r % G;
        a.lse[((size_t)b * a.Hq + h) * a.n + i] = l2 * kLn2;
      }
    }
    __syncthreads();
  }

  const float c = a.scale * kLog2e;
  const bf16_t* q = (const bf16_t*)a.q;
  const int ntq = (a.n + 15) / 16;
  const int iters = G * ntq;
  // Q^T fragments of tile `it` = (query head g*G + it / ntq, queries 16 (it % ntq) ...).
  // Rows past n read row 0 (finite data) and are masked out of the sums.
  // Without MERGE the row's log-sum-exp comes from global memory and is fetched with Q.
  auto load_q = [&](int it, u32x4 (&qf)[DS], float& l) {
    const int hh = it / ntq, i = (it % ntq) * 16 + l16;
    const int ic = i < a.n ? i : 0;
    const bf16_t* src = q + (((size_t)b * a.n + ic) * a.Hq + g * G + hh) * D + lg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = *(const u32x4*)(src + ds * 32);
    if constexpr (!MERGE) l = a.lse[((size_t)b * a.Hq + g * G + hh) * a.n + ic];
  };
  u32x4 qcur[DS], qnext[DS];
  float lcur = 0.f, lnext = 0.f;
  if (iters > 0) load_q(0, qcur, lcur);
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int it = 0; it < iters; ++it) {
    if (it + 1 < iters) load_q(it + 1, qnext, lnext);
    const int hh = it / ntq, i = (it % ntq) * 16 + l16;
    const bool ok = i < a.n;
    float lse2;
    if constexpr (MERGE) lse2 = ok ? lse2_s[i * G + hh] : 0.f;
    else lse2 = ok ? lcur * kLog2e : 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) sv = mfma_bf16(kf[kt][ds], as_bf16x8(qcur[ds]), sv);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[kt][v] += ok ? exp2f(sv[v] * ksc[kt][v] * c - lse2) : 0.f;
    }
    if ((it + 1) % ntq == 0) {                   // last tile of this head: reduce and store
      const int h = g * G + hh;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = acc[kt][v];
          x += __shfl_xor(x, 1, kWave);
          x += __shfl_xor(x, 2, kWave);
          x += __shfl_xor(x, 4, kWave);
          x += __shfl_xor(x, 8, kWave);
          const int key = key0 + kt * 16 + lg * 4 + v;
          if (l16 == 0 && key < a.S) a.mass[((size_t)b * a.Hq + h) * a.S + key] = x;
          acc[kt][v] = 0.f;
        }
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qcur[ds] = qnext[ds];
    lcur = lnext;
  }

  if constexpr (MERGE) {
    // outputs of the rows r = kchunk + nkc * (4 it + wave), one wave per row
    constexpr int PER = D / 64;
    for (int r = kchunk + nkc * wave; r < rows; r += 4 * nkc) {
      const size_t pr0 = (size_t)bg * rows + r;
      float mm, L;
      merged_ml(ml, nrows_all, pr0, splits, mm, L);
      float o[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = 0.f;
      for (int sp = 0; sp < splits; ++sp) {
        const size_t pr = (size_t)sp * nrows_all + pr0;
        const float ms = ml[pr * 2];
        const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - mm);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += a.part[pr * D + lane + 64 * e] * wgt;
      }
      const int i = r / G, h = g * G + r % G;
      bf16_t* out = (bf16_t*)a.out + (((size_t)b * a.n + i) * a.Hq + h) * D;
      const float inv = 1.f / L;
#pragma unroll
      for (int e = 0; e < PER; ++e) out[lane + 64 * e] = f32_to_bf16(o[e] * inv);
    }
  }
}

// ---------------------------------------------------------------- fp32 (small shapes) ---
// One wave per (b, h, i): scores into LDS, exact softmax, output; fp32 FMA in key order.
__global__ __launch_bounds__(64) void attn_f32(AttnArgs a) {
  extern __shared__ float z[];
  const int lane = threadIdx.x;
  const int i = blockIdx.x % a.n, bh = blockIdx.x / a.n;
  const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
  const int D = a.D;
  const float* q = (const float*)a.q + (((size_t)b * a.n + i) * a.Hq + h) * D;
  const float* K = (const float*)a.kc + ((size_t)b * a.Hkv + g) * a.S * D;
  const float* V = (const float*)a.vc + ((size_t)b * a.Hkv + g) * a.S * D;
  float mx = -INFINITY;
  for (int j = lane; j < a.S; j += 64) {
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = fmaf(q[d], K[(size_t)j * D + d], s);
    s *= a.scale;
    z[j] = s;
    mx = fmaxf(mx, s);
  }
  for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk, kWave));
  float l = 0.f;
  for (int j = lane; j < a.S; j += 64) {
    const float p = expf(z[j] - mx);
    z[j] = p;
    l += p;
  }
  for (int msk = 1; msk < 64; msk <<= 1) l += __shfl_xor(l, msk, kWave);
  __syncthreads();
  float* o = (float*)a.out + (((size_t)b * a.n + i) * a.Hq + h) * D;
  for (int d = lane; d < D; d += 64) {
    float acc = 0.f;
    for (int j = 0; j < a.S; ++j) acc = fmaf(z[j], V[(size_t)j * D + d], acc);
    o[d] = acc / l;
  }
  if (lane == 0) a.lse[((size_t)b * a.Hq + h) * a.n + i] = mx + logf(l);
}

__global__ __launch_bounds__(64) void attn_mass_f32(AttnArgs a) {
  const int j = blockIdx.x * 64 + threadIdx.x;
  const int bh = blockIdx.y, b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
  if (j >= a.S) return;
  const int D = a.D;
  const float* K = (const float*)a.kc + (((size_t)b * a.Hkv + g) * a.S + j) * D;
  float acc = 0.f;
  for (int i = 0; i < a.n; ++i) {
    const float* q = (const float*)a.q + (((size_t)b * a.n + i) * a.Hq + h) * D;
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = fmaf(q[d], K[d], s);
    acc += expf(s * a.scale - a.lse[((size_t)b * a.Hq + h) * a.n + i]);
  }
  a.mass[((size_t)b * a.Hq + h) * a.S + j] = acc;
}

template <int KIND, int D>
hipError_t launch_mfma(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int rows = a.n * G;
  const int qtiles = (rows + p.qt - 1) / p.qt;
  hipError_t e = launch_attn_fwd<KIND, D>(a, p, qtiles, s);
  if (e != hipSuccess) return e;
  const bool fuse = a.mass && p.splits > 1 && rows <= kFusedMergeRows;
  if (p.splits > 1 && !fuse) {
    attn_merge<bf16_t, D><<<a.B * a.Hkv * rows, 64, 0, s>>>(a, p.splits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mass) {
    const int grid2 = ((a.S + 127) / 128) * a.B * a.Hkv;
    if (fuse)
      attn_mass_mfma<KIND, D, true><<<grid2, 256, (size_t)rows * sizeof(float), s>>>(a, p.splits);
    else
      attn_mass_mfma<KIND, D, false><<<grid2, 256, 0, s>>>(a, p.splits);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

AttnPlan plan_attention(int B, int n, int Hq, int Hkv, int S, int D, int act, int kind) {
  AttnPlan p{32, 1, 0, 0};
  if (act == DLLM_F32) {
    p.kps = S;
    return p;
  }
  const int rows = n * (Hq / Hkv);
  p.qt = rows >= 512 ? 128 : rows > 32 ? 64 : 32;
  const int qtiles = (rows + p.qt - 1) / p.qt;
  const long wgs = (long)B * Hkv * qtiles;
  // Enough workgroups to cover the 256 compute units about twice, keeping at least one key
  // tile per wave.
  const int kw = 4 / (p.qt / 32);
  const int tiles = (S + kKeys - 1) / kKeys;
  int splits = 1;
  while (wgs * splits < 512 && tiles / (splits * 2) >= kw) splits *= 2;
  p.splits = splits;
  p.kps = ((tiles + splits - 1) / splits) * kKeys;
  p.splits = (S + p.kps - 1) / p.kps;
  if (p.splits > 1) {
    const size_t nrows_all = (size_t)B * Hkv * rows;
    p.part_bytes = (size_t)p.splits * nrows_all * (D + 2) * sizeof(float);
  }
  return p;
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  if (a.act == DLLM_F32) {
    attn_f32<<<a.B * a.Hq * a.n, 64, (size_t)a.S * sizeof(float), s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.mass) return e;
    dim3 grid((a.S + 63) / 64, a.B * a.Hq);
    attn_mass_f32<<<grid, 64, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.kind == kCacheFP8) return a.D == 128 ? launch_mfma<kCacheFP8, 128>(a, p, s) : launch_mfma<kCacheFP8, 64>(a, p, s);
  return a.D == 128 ? launch_mfma<kCacheBF16, 128>(a, p, s) : launch_mfma<kCacheBF16, 64>(a, p, s);
}

}  // namespace dllm
