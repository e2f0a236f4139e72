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

// Merged state of packed row pr0 from the split partials, in split order (the same arithmetic
// as attn_merge): running max mm and normaliser L.  Up to eight splits are loaded together
// (clamped, unconditional loads) before any arithmetic, so the row costs one round trip.
constexpr int kMergeBatch = 8;

__device__ __forceinline__ void merged_ml(const float* ml, size_t nrows_all, size_t pr0, int splits,
                                          float& mm, float& L) {
  if (splits <= kMergeBatch) {
    float ms[kMergeBatch], ls[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const float2 v = *(const float2*)(ml + ((size_t)min(e, splits - 1) * nrows_all + pr0) * 2);
      ms[e] = v.x;
      ls[e] = v.y;
    }
    mm = -INFINITY;
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e)
      if (e < splits) mm = fmaxf(mm, ms[e]);
    L = 0.f;
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e)
      if (e < splits) L += ls[e] * ((ms[e] == -INFINITY) ? 0.f : exp2f(ms[e] - mm));
    return;
  }
  mm = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) mm = fmaxf(mm, ml[((size_t)sp * nrows_all + pr0) * 2]);
  L = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const size_t pr = (size_t)sp * nrows_all + pr0;
    const float ms = ml[pr * 2], ls = ml[pr * 2 + 1];
    L += ls * ((ms == -INFINITY) ? 0.f : exp2f(ms - mm));
  }
}

// Merged state and unnormalised output (lane's columns lane + 64 e) of packed row pr0, in
// split order; up to eight splits' loads are issued together before the arithmetic.
template <int D>
__device__ __forceinline__ void merge_row(const float* part, const float* ml, size_t nrows_all, size_t pr0,
                                          int splits, int lane, float (&o)[D / 64], float& mm, float& L) {
  constexpr int PER = D / 64;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  mm = -INFINITY;
  L = 0.f;
  if (splits <= kMergeBatch) {
    float ms[kMergeBatch], ls[kMergeBatch], po[kMergeBatch][PER];
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
      const size_t pr = (size_t)min(q, splits - 1) * nrows_all + pr0;
      const float2 v = *(const float2*)(ml + pr * 2);
      ms[q] = v.x;
      ls[q] = v.y;
#pragma unroll
      for (int e = 0; e < PER; ++e) po[q][e] = part[pr * D + lane + 64 * e];
    }
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q)
      if (q < splits) mm = fmaxf(mm, ms[q]);
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
      if (q >= splits) continue;
      const float wgt = (ms[q] == -INFINITY) ? 0.f : exp2f(ms[q] - mm);
      L += ls[q] * wgt;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] += po[q][e] * wgt;
    }
    return;
  }
  for (int sp = 0; sp < splits; ++sp) mm = fmaxf(mm, ml[((size_t)sp * nrows_all + pr0) * 2]);
  for (int sp = 0; sp < splits; ++sp) {
    const size_t pr = (size_t)sp * nrows_all + pr0;
    const float ms = ml[pr * 2], ls = ml[pr * 2 + 1];
    const float wgt = (ms == -INFINITY) ? 0.f : exp2f(ms - mm);
    L += ls * wgt;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += part[pr * D + lane + 64 * e] * wgt;
  }
}

// Combine split partial states in split order: one wave per packed query row.
template <typename OutT, int D>
__global__ __launch_bounds__(64) void attn_merge(AttnArgs a, int splits) {
  const int G = a.Hq / a.Hkv;
  const size_t nrows_all = (size_t)a.T * a.Hq;
  const size_t pr0 = blockIdx.x;  // q0 * Hq + g * rows + r (q0: the sequence's first row)
  if (pr0 >= (size_t)live_rows(a.cu, a.B, a.T) * a.Hq) return;   // past the rows present
  const int b = seq_of_row(a.cu, a.B, a.n, (int)(pr0 / a.Hq));
  const int nb = seq_rows(a.cu, a.n, b), q0 = seq_row0(a.cu, a.n, b);
  const int rows = nb * G;
  const int local = (int)(pr0 - (size_t)q0 * a.Hq);
  const int g = local / rows, r = local % rows;
  const float* ml = a.part + (size_t)splits * nrows_all * D;
  constexpr int PER = D / 64;
  float mm, L, o[PER];
  merge_row<D>(a.part, ml, nrows_all, pr0, splits, threadIdx.x, o, mm, L);
  const int i = r / G, h = g * G + r % G;
  OutT* out = (OutT*)a.out + (((size_t)q0 + i) * a.Hq + h) * D;
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float val = o[e] * inv;
    if constexpr (sizeof(OutT) == 2) out[threadIdx.x + 64 * e] = f32_to_bf16(val);
    else out[threadIdx.x + 64 * e] = val;
  }
  if (threadIdx.x == 0) a.lse[(size_t)q0 * a.Hq + (size_t)h * nb + i] = (mm + log2f(L)) * kLn2;
}

// Column attention mass, second pass after the log-sum-exp is known:
//   mass[b, h, j] = sum_i exp(<q_i, k_j> * scale - lse_i).
// One workgroup per (b, KV head g) and 128 keys, so each K row is read once for all G query
// heads of its group: each wave keeps 32 keys' K rows as MFMA A operands (S^T = K Q^T).  The
// group's queries stream through an LDS ring in tiles of 32 rows of one head (DMA, three
// stages, shared by the four waves), and every row's log-sum-exp sits in LDS.  Lane (l16, lg)
// sums query column l16 over the tiles in order; the 16 lanes of a key are added at the end
// of each head in a fixed DPP order (row16_sum).
//
// MERGE (the attention was split over keys): the rows' outputs are merged here (rows dealt
// round-robin over the key chunks), first thing after the prologue's loads are issued, so no
// separate merge launch is needed; then every packed row's log-sum-exp is formed from the
// split partials and the workgroups of key chunk 0 write it.
constexpr int kMassNst = 3;                      // ring stages
// Largest packed-row count (n * G) whose log-sum-exp the mass pass stages in LDS (32 KB);
// beyond it the rows' log-sum-exp is read from memory (and split attention merges first).
constexpr int kMassLdsRows = 8192;

template <int D>
__device__ __forceinline__ int swz_q(int r) {   // chunk swizzle of a staged query row
  return D == 128 ? ((r & 3) | (((r >> 2) & 3) << 2)) : ((r & 3) | (((r >> 2) & 1) << 2));
}

// QR: query rows per ring tile (64, or 32 when the block has at most 32 rows).
template <int KIND, int D, bool MERGE, bool LDS_LSE, int QR>
__global__ __launch_bounds__(256) void attn_mass_mfma(AttnArgs a, int splits) {
  static_assert(LDS_LSE || !MERGE, "the fused merge stages the log-sum-exp in LDS");
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  constexpr int DS = D / 32;
  constexpr int RB = D * 2;                      // bytes per query row
  constexpr int QTILE = QR * RB;         // bytes per ring tile
  constexpr int RPI = 1024 / RB;                 // rows per DMA block
  constexpr int NBLK = QTILE / 1024;             // DMA blocks per tile
  constexpr int BPW = (NBLK + 3) / 4;            // per wave (the last wave may have fewer)
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  char* ring = dyn;                              // [kMassNst][QTILE]
  float* lse2_s = (float*)(dyn + kMassNst * QTILE);  // [n * G] log2-domain LSE
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  // All key chunks of one (b, KV head) run on one XCD: the group's queries are fetched into
  // that L2 once.
  const int nkc = (a.S + 127) / 128;
  int bg, kchunk;
  xcd_group_unit(blockIdx.x, a.B * a.Hkv, nkc, bg, kchunk);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nb = seq_rows(a.cu, a.n, b), q0 = seq_row0(a.cu, a.n, b);
  const int klen = seq_keys(a.lens, a.S, b);
  const int rows = nb * G;
  const int key0 = kchunk * 128 + wave * 32;
  if (nb == 0) {                                 // a sequence without queries: no mass
    for (int e = t; e < G * 128; e += 256) {
      const int key = kchunk * 128 + (e & 127);
      if (key < a.S) a.mass[((size_t)b * a.Hq + g * G + (e >> 7)) * a.S + key] = 0.f;
    }
    return;
  }
  const size_t head_base = ((size_t)b * a.Hkv + g) * a.S;
  constexpr int ELT = (KIND == kCacheFP8) ? 1 : 2;
  const char* kc = (const char*)a.kc;

  // Query tiles: it = hh * ntq + (i0 / 32), rows i0 .. i0 + 31 of head g * G + hh (rows past
  // n read row n - 1 and are masked out of the sums).
  const int ntq = (nb + QR - 1) / QR;
  const int iters = G * ntq;
  const bf16_t* q = (const bf16_t*)a.q;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform: scalar DMA bases
  const uint32_t ring_lds = lds_addr(dyn);
  auto issue = [&](int it, int slot) {
    const int hh = it / ntq, i0 = (it % ntq) * QR;
    const bf16_t* qb = q + ((size_t)q0 * a.Hq + g * G + hh) * D;   // row 0 of this head
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int blk = wave_u * BPW + u;
      if (blk < NBLK) {
        const int r = blk * RPI + lane / CPR, sc = lane % CPR;
        const int i = min(i0 + r, nb - 1);
        const uint32_t voff = (uint32_t)(((size_t)i * a.Hq * D + (sc ^ swz_q<D>(r)) * 8) * sizeof(bf16_t));
        dma_16B_sbase(voff, qb, ring_lds + (uint32_t)(slot * QTILE + blk * 1024));
      }
    }
  };
#pragma unroll
  for (int st = 0; st < kMassNst - 1; ++st)
    if (st < iters) issue(st, st);

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

  const size_t nrows_all = (size_t)a.T * a.Hq;
  const size_t pr_base = (size_t)q0 * a.Hq + (size_t)g * rows;   // packed row of (b, g, r = 0)
  const float* ml = a.part + (size_t)splits * nrows_all * D;
  // The rows' outputs are merged first: their loads then travel with the prologue's.
  if constexpr (MERGE) {
    // outputs of the rows r = kchunk + nkc * (4 it + wave), one wave per row
    constexpr int PER = D / 64;
    for (int r = kchunk + nkc * wave; r < rows; r += 4 * nkc) {
      const size_t pr0 = pr_base + r;
      float mm, L, o[PER];
      merge_row<D>(a.part, ml, nrows_all, pr0, splits, lane, o, mm, L);
      const int i = r / G, h = g * G + r % G;
      bf16_t* out = (bf16_t*)a.out + (((size_t)q0 + i) * a.Hq + h) * D;
      const float inv = 1.f / L;
#pragma unroll
      for (int e = 0; e < PER; ++e) out[lane + 64 * e] = f32_to_bf16(o[e] * inv);
    }
  }

  // log-sum-exp of every packed row r = i * G + hh, log2 domain
  for (int r = t; LDS_LSE && r < rows; r += 256) {
    const int i = r / G, h = g * G + r % G;
    if constexpr (MERGE) {
      float mm, L;
      merged_ml(ml, nrows_all, pr_base + r, splits, mm, L);
      const float l2 = mm + log2f(L);
      lse2_s[r] = l2;
      if (kchunk == 0) a.lse[(size_t)q0 * a.Hq + (size_t)h * nb + i] = l2 * kLn2;
    } else {
      lse2_s[r] = a.lse[(size_t)q0 * a.Hq + (size_t)h * nb + i] * kLog2e;
    }
  }
  __syncthreads();

  const float c = a.scale * kLog2e;
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  constexpr int PEND = BPW;                      // this wave's DMA ops per tile (at most)
  for (int it = 0; it < iters; ++it) {
    if (it + kMassNst - 2 < iters) DLLM_WAIT_VMCNT(PEND * (kMassNst - 2));
    else DLLM_WAIT_VMCNT(0);
    lds_barrier();
    if (it + kMassNst - 1 < iters) issue(it + kMassNst - 1, (it + kMassNst - 1) % kMassNst);
    const char* Q = ring + (it % kMassNst) * QTILE;
    const int hh = it / ntq, i0 = (it % ntq) * QR;
#pragma unroll
    for (int ct = 0; ct < QR / 16; ++ct) {
      const int r = ct * 16 + l16;
      const int i = i0 + r;
      const int ic = min(i, nb - 1);
      // rows past n (they read row n - 1) take lse = +inf, so their terms are exp2(-inf) = 0
      const float lse2 = (i < nb) ? (LDS_LSE ? lse2_s[ic * G + hh]
                                             : a.lse[(size_t)q0 * a.Hq + (size_t)(g * G + hh) * nb + ic] * kLog2e)
                                  : INFINITY;
      bf16x8 qf[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int ch = ds * 4 + lg;
        qf[ds] = as_bf16x8(*(const u32x4*)(Q + r * RB + ((ch ^ swz_q<D>(r)) << 4)));
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 sv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) sv = mfma_bf16(kf[kt][ds], qf[ds], sv);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          acc[kt][v] += __builtin_amdgcn_exp2f(fmaf(sv[v] * ksc[kt][v], c, -lse2));
        }
      }
    }
    if ((it + 1) % ntq == 0) {                   // last tile of this head: reduce and store
      const int h = g * G + hh;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float x = row16_sum(acc[kt][v]);
          const int key = key0 + kt * 16 + lg * 4 + v;
          // keys past the sequence's length (a variable-length batch) get no mass
          if (l16 == 0 && key < a.S) a.mass[((size_t)b * a.Hq + h) * a.S + key] = key < klen ? x : 0.f;
          acc[kt][v] = 0.f;
        }
    }
  }

}

// ---------------------------------------------------------------- fp32 (small shapes) ---
// One workgroup per (b, h, i): q staged in LDS, one thread per key for the scores (fp32 FMA
// in d order), block max / sum, then the output with 256 / D key groups per column, their
// partial sums added in group order.
template <int D>
__global__ __launch_bounds__(256) void attn_f32(AttnArgs a) {
  extern __shared__ float z[];                   // [S] scores, then [D] q, then reductions
  constexpr int NG = 256 / D;                    // key groups of the output pass
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int i = blockIdx.x % a.n, bh = blockIdx.x / a.n;
  const int b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
  float* qs = z + a.S;
  float* red = qs + D;                           // [4] wave results, then [NG][D] partials
  const float* q = (const float*)a.q + (((size_t)b * a.n + i) * a.Hq + h) * D;
  const float* K = (const float*)a.kc + ((size_t)b * a.Hkv + g) * a.S * D;
  const float* V = (const float*)a.vc + ((size_t)b * a.Hkv + g) * a.S * D;
  if (t < D) qs[t] = q[t];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = t; j < a.S; j += 256) {
    const float4* kr = (const float4*)(K + (size_t)j * D);
    float s = 0.f;
#pragma unroll 8
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 k4 = kr[d4];
      s = fmaf(qs[4 * d4], k4.x, s);
      s = fmaf(qs[4 * d4 + 1], k4.y, s);
      s = fmaf(qs[4 * d4 + 2], k4.z, s);
      s = fmaf(qs[4 * d4 + 3], k4.w, s);
    }
    s *= a.scale;
    z[j] = s;
    mx = fmaxf(mx, s);
  }
  for (int msk = 1; msk < 64; msk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, msk, kWave));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.f;
  for (int j = t; j < a.S; j += 256) {
    const float p = expf(z[j] - mx);
    z[j] = p;
    l += p;
  }
  for (int msk = 1; msk < 64; msk <<= 1) l += __shfl_xor(l, msk, kWave);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  l = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  const int d = t % D, grp = t / D;
  float acc = 0.f;
  for (int j = grp; j < a.S; j += NG) acc = fmaf(z[j], V[(size_t)j * D + d], acc);
  red[4 + grp * D + d] = acc;
  __syncthreads();
  if (t < D) {
    float o = 0.f;
    for (int q2 = 0; q2 < NG; ++q2) o += red[4 + q2 * D + t];
    ((float*)a.out)[(((size_t)b * a.n + i) * a.Hq + h) * D + t] = o / l;
  }
  if (t == 0) a.lse[((size_t)b * a.Hq + h) * a.n + i] = mx + logf(l);
}

// One thread per key (64 keys per workgroup) with its K row in registers; the head's queries
// and their log-sum-exp are staged in LDS 64 at a time and summed in query order.
template <int D>
__global__ __launch_bounds__(64) void attn_mass_f32(AttnArgs a) {
  __shared__ float qs[64][D + 1];
  __shared__ float ls[64];
  const int t = threadIdx.x;
  const int j = blockIdx.x * 64 + t;
  const int bh = blockIdx.y, b = bh / a.Hq, h = bh % a.Hq, g = h / (a.Hq / a.Hkv);
  const float* K = (const float*)a.kc + (((size_t)b * a.Hkv + g) * a.S + (j < a.S ? j : 0)) * D;
  float kr[D];
#pragma unroll
  for (int d4 = 0; d4 < D / 4; ++d4) {
    const float4 k4 = ((const float4*)K)[d4];
    kr[4 * d4] = k4.x; kr[4 * d4 + 1] = k4.y; kr[4 * d4 + 2] = k4.z; kr[4 * d4 + 3] = k4.w;
  }
  float acc = 0.f;
  for (int i0 = 0; i0 < a.n; i0 += 64) {
    const int cnt = min(64, a.n - i0);
    __syncthreads();
    for (int r = 0; r < cnt; ++r)
      for (int d = t; d < D; d += 64) qs[r][d] = ((const float*)a.q)[(((size_t)b * a.n + i0 + r) * a.Hq + h) * D + d];
    if (t < cnt) ls[t] = a.lse[((size_t)b * a.Hq + h) * a.n + i0 + t];
    __syncthreads();
    for (int r = 0; r < cnt; ++r) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qs[r][d], kr[d], s);
      acc += expf(s * a.scale - ls[r]);
    }
  }
  if (j < a.S) a.mass[((size_t)b * a.Hq + h) * a.S + j] = acc;
}

template <int KIND, int D>
hipError_t launch_mfma(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int rows = a.n * G;
  const int qtiles = (rows + p.qt - 1) / p.qt;
  hipError_t e = launch_attn_fwd<KIND, D>(a, p, qtiles, s);
  if (e != hipSuccess) return e;
  const bool lds_lse = rows <= kMassLdsRows;
  const bool fuse = a.mass && p.splits > 1 && lds_lse;
  if (p.splits > 1 && !fuse) {
    attn_merge<bf16_t, D><<<(unsigned)((size_t)a.T * a.Hq), 64, 0, s>>>(a, p.splits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mass) {
    const int grid2 = ((a.S + 127) / 128) * a.B * a.Hkv;
    const bool wide = a.n > 32;
    const size_t lds = (size_t)kMassNst * (wide ? 64 : 32) * D * 2 + (lds_lse ? (size_t)rows * sizeof(float) : 0);
#define DLLM_MASS(M_, L_)                                                                  \
    (wide ? (attn_mass_mfma<KIND, D, M_, L_, 64><<<grid2, 256, lds, s>>>(a, p.splits), 0) \
          : (attn_mass_mfma<KIND, D, M_, L_, 32><<<grid2, 256, lds, s>>>(a, p.splits), 0))
    if (fuse)
      DLLM_MASS(true, true);
    else if (lds_lse)
      DLLM_MASS(false, true);
    else
      DLLM_MASS(false, false);
#undef DLLM_MASS
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

AttnPlan plan_attention(int B, int n, int Hq, int Hkv, int S, int D, int act, int kind, long long T) {
  AttnPlan p{32, 1, 0, 0};
  if (act == DLLM_F32) {
    p.kps = S;
    return p;
  }
  const int rows = n * (Hq / Hkv);
  p.qt = rows >= 512 ? 128 : rows > 32 ? 64 : 32;
  const int qtiles = (rows + p.qt - 1) / p.qt;
  const long wgs = (long)B * Hkv * qtiles;
  // Enough workgroups to cover the 256 compute units about twice (once for FP8 caches with
  // four key groups, whose rings fill a CU's LDS), keeping at least one key tile per wave.
  const int kw = 4 / (p.qt / 32);
  const int tiles = (S + kKeys - 1) / kKeys;
  const long target = (kind == kCacheFP8 && kw == 4) ? 256 : 512;
  int splits = 1;
  while (wgs * splits < target && tiles / (splits * 2) >= kw) splits *= 2;
  p.splits = splits;
  p.kps = ((tiles + splits - 1) / splits) * kKeys;
  p.splits = (S + p.kps - 1) / p.kps;
  if (p.splits > 1) {
    const size_t nrows_all = (size_t)T * Hq;
    p.part_bytes = (size_t)p.splits * nrows_all * (D + 2) * sizeof(float);
  }
  return p;
}

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  if (a.act == DLLM_F32) {
    const size_t lds = ((size_t)a.S + a.D + 4 + 256) * sizeof(float);
    if (a.D == 128) attn_f32<128><<<a.B * a.Hq * a.n, 256, lds, s>>>(a);
    else attn_f32<64><<<a.B * a.Hq * a.n, 256, lds, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.mass) return e;
    dim3 grid((a.S + 63) / 64, a.B * a.Hq);
    if (a.D == 128) attn_mass_f32<128><<<grid, 64, 0, s>>>(a);
    else attn_mass_f32<64><<<grid, 64, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.kind == kCacheFP8) return a.D == 128 ? launch_mfma<kCacheFP8, 128>(a, p, s) : launch_mfma<kCacheFP8, 64>(a, p, s);
  if (attn_fused_fits(a, p)) return launch_attn_fused(a, s);
  return a.D == 128 ? launch_mfma<kCacheBF16, 128>(a, p, s) : launch_mfma<kCacheBF16, 64>(a, p, s);
}

}  // namespace dllm
