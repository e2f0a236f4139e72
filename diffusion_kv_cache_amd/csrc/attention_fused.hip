// Bidirectional block attention and the column attention mass in one launch, for steps whose
// query rows of one KV head fit a single 32-row tile (one query head per KV head, n <= 32).
//
// What it computes: O = softmax(q k^T * scale) v over every cache row, no mask (Flash-Cache
// article, section 3.1; LaCache Technical Summary, Problem Statement), its log-sum-exp, and
// the column mass a[b, h, j] = sum_i exp(<q_i, k_j> * scale - lse_i) that ranks the most
// attended tokens (Flash-dLLM news summary, selective cache tracking).
//
// One workgroup per (b, KV head) holds all of the head's query rows, so nothing has to be
// merged across workgroups: its four waves take every fourth 32-key tile and
//   pass 1 streams K and keeps each query row's running max and normaliser,
//   the waves combine their row states in wave order (exact log-sum-exp of every row),
//   pass 2 streams V (and K again, unless every wave has at most six tiles: then pass 1
//     kept its raw scores in registers), forms the exact probabilities
//     p = exp2(s * scale * log2 e - lse_2), adds them down each key column (the column mass,
//     finished inside the wave: all query rows are here) and accumulates O^T += V^T P^T,
//   the four partial outputs are added in wave order through LDS.
// K and V tiles are loaded row-contiguous into registers (whole 128-byte lines per load, several
// tiles in flight per wave), then written to one LDS stage per wave, from which the MFMA
// operand reads (K) and the transposing reads (V) are served.  With few workgroups (one per
// head of a single sequence) the bytes in flight per CU decide the speed, and registers hold
// far more of them than an LDS ring fed by DMA.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKeys = 32;          // keys per tile
constexpr int kWaves = 4;          // key groups (waves) per workgroup
constexpr float kLazy = 8.0f;      // log2 headroom before the running max is moved
constexpr int kDepth1 = 4;         // K tiles in flight per wave, pass 1
constexpr int kDepth2 = 2;         // K and V tiles in flight per wave, pass 2
constexpr int kFusedMaxSeq = 16384; // the column masses of a head are staged in LDS

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A K or V tile in registers, row-contiguous: chunk u * 64 + lane of the 32 x D tile (whole
// 128-byte lines per load instruction).
template <int D>
struct Tile {
  u32x4 r[D / 16];
};

template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& x, const char* base, int key0, int S, int lane) {
  constexpr int RB = 2 * D, CPR = D / 8;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const int id = u * 64 + lane, row = id / CPR, ch = id % CPR;
    const int key = min(key0 + row, S - 1);     // past the end: masked
    x.r[u] = *(const u32x4*)(base + (size_t)key * RB + ch * 16);
  }
}

// K tile chunk swizzle: the 16 rows one MFMA operand read touches hit 16 (D = 128) or 8
// (D = 64) distinct chunk slots.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? ((r & 3) | (((r >> 3) & 3) << 2)) : ((r & 3) | (((r >> 3) & 1) << 2));
}

// Registers -> this wave's LDS stage, chunk slots swizzled per row by SWZ.
template <int D, bool IS_K>
__device__ __forceinline__ void stage_tile(const Tile<D>& x, char* st, int lane) {
  constexpr int RB = 2 * D, CPR = D / 8;
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const int id = u * 64 + lane, row = id / CPR, ch = id % CPR;
    const int sw = IS_K ? swz_k<D>(row) : attn_swz_v(row);
    *(u32x4*)(st + row * RB + ((ch ^ sw) << 4)) = x.r[u];
  }
}

template <int D>
__device__ __forceinline__ void scores(const char* kst, const u32x4 (&qf)[2][D / 32], f32x4 (&s)[2][2],
                                       int l16, int lg) {
  constexpr int RB = 2 * D;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[ct][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int R = attn_perm_key(kt, l16), ch = ds * 4 + lg;
      const bf16x8 kf = as_bf16x8(*(const u32x4*)(kst + R * RB + ((ch ^ swz_k<D>(R)) << 4)));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) s[ct][kt] = mfma_bf16(kf, as_bf16x8(qf[ct][ds]), s[ct][kt]);
    }
}

// Pass 1 on one tile: lazily rescaled running max m (log2 domain) and normaliser l per query
// column; lane group lg holds keys 8 lg .. 8 lg + 7 of the tile.  FULL: no key past the end.
template <bool FULL>
__device__ __forceinline__ void stats_from(const f32x4 (&s)[2][2], float (&m)[2], float (&l)[2], int key0,
                                           int S, float c, int lg) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = s[ct][e >> 2][e & 3];
    if constexpr (!FULL) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (key0 + lg * 8 + e >= S) sv[e] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    const float mt = max_across_rows(mx) * c;
    if (__any(mt > m[ct] + kLazy)) {
      const float mn = fmaxf(m[ct], mt);
      l[ct] *= (m[ct] == -INFINITY) ? 0.f : exp2f(m[ct] - mn);
      m[ct] = mn;
    }
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ps += __builtin_amdgcn_exp2f(fmaf(sv[e], c, -m[ct]));
    l[ct] += ps;
  }
}

template <int D, bool FULL>
__device__ __forceinline__ void tile_stats(const Tile<D>& k, char* kst, const u32x4 (&qf)[2][D / 32],
                                           float (&m)[2], float (&l)[2], int key0, int S, float c,
                                           int lane, int l16, int lg) {
  stage_tile<D, true>(k, kst, lane);
  f32x4 s[2][2];
  scores<D>(kst, qf, s, l16, lg);
  stats_from<FULL>(s, m, l, key0, S, c, lg);
}

// Pass 2 on one tile, given its scores: exact probabilities, the tile's 32 column masses,
// and O^T += V^T P^T.
template <int D, bool FULL>
__device__ __forceinline__ void out_from(const f32x4 (&s)[2][2], const Tile<D>& v, char* vst,
                                         const float (&L2)[2], const bool (&rowok)[2],
                                         f32x4 (&oacc)[2][D / 16], float* mass_s, int key0, int S,
                                         float c, int lane, int l16, int lg) {
  constexpr int RB = 2 * D, DT = D / 16;
  stage_tile<D, false>(v, vst, lane);
  bf16x8 pb[2];
  float col[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) col[e] = 0.f;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sv = s[ct][e >> 2][e & 3];
      if (!FULL && key0 + lg * 8 + e >= S) sv = -INFINITY;
      p[e] = __builtin_amdgcn_exp2f(fmaf(sv, c, -L2[ct]));   // argument <= 0 (or -inf)
      col[e] += rowok[ct] ? p[e] : 0.f;
    }
    u32x4 pw;
    pw.x = pack_bf16x2(p[0], p[1]);
    pw.y = pack_bf16x2(p[2], p[3]);
    pw.z = pack_bf16x2(p[4], p[5]);
    pw.w = pack_bf16x2(p[6], p[7]);
    pb[ct] = as_bf16x8(pw);
  }
  // column masses (staged in LDS: a global store here would sit in the vector-memory count
  // that the next tile's loads are waited on): lane l16 < 8 of lane group lg holds key
  // 8 lg + l16
  float mine = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = row16_sum(col[e]);
    mine = (l16 == e) ? x : mine;
  }
  const int key = key0 + lg * 8 + l16;
  if (l16 < 8 && key < S) mass_s[key] = mine;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    s16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int R = 8 * lg + 4 * hh + (l16 >> 2);
      const int d0 = 16 * dt + 4 * (l16 & 3);
      const int ch = d0 >> 3;
      const char* addr = vst + R * RB + ((ch ^ attn_swz_v(R)) << 4) + ((d0 & 4) ? 8 : 0);
      h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)addr);
    }
    const u32x4 vw = {(uint32_t)(uint16_t)h[0][0] | ((uint32_t)(uint16_t)h[0][1] << 16),
                      (uint32_t)(uint16_t)h[0][2] | ((uint32_t)(uint16_t)h[0][3] << 16),
                      (uint32_t)(uint16_t)h[1][0] | ((uint32_t)(uint16_t)h[1][1] << 16),
                      (uint32_t)(uint16_t)h[1][2] | ((uint32_t)(uint16_t)h[1][3] << 16)};
    const bf16x8 vf = as_bf16x8(vw);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) oacc[ct][dt] = mfma_bf16(vf, pb[ct], oacc[ct][dt]);
  }
}

// Pass 2 on one tile, K staged again and its scores recomputed.
template <int D, bool FULL>
__device__ __forceinline__ void tile_out(const Tile<D>& k, const Tile<D>& v, char* kst, char* vst,
                                         const u32x4 (&qf)[2][D / 32], const float (&L2)[2],
                                         const bool (&rowok)[2], f32x4 (&oacc)[2][D / 16],
                                         float* mass_s, int key0, int S, float c, int lane, int l16,
                                         int lg) {
  stage_tile<D, true>(k, kst, lane);
  f32x4 s[2][2];
  scores<D>(kst, qf, s, l16, lg);
  out_from<D, FULL>(s, v, vst, L2, rowok, oacc, mass_s, key0, S, c, lane, l16, lg);
}

// TPW > 0: every wave has at most TPW tiles, and pass 1 keeps their scores in registers, so
// pass 2 reads only V (no second K pass, no recomputed scores).  TPW = 0: K is streamed twice.
template <int D, int TPW>
__global__ __launch_bounds__(256) void attn_fused(AttnArgs a) {
  constexpr int DS = D / 32, DT = D / 16, RB = 2 * D;
  constexpr int TB = kKeys * RB;                 // one K or V tile in LDS
  constexpr int MB = 2 * DT * 4 * 64;            // floats of one wave's output partial
  constexpr int LDS_BYTES = kWaves * MB * 4 > kWaves * 2 * TB ? kWaves * MB * 4 : kWaves * 2 * TB;
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  __shared__ float st_m[kWaves][32], st_l[kWaves][32];
  extern __shared__ float mass_s[];              // [S] this head's column masses

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int bg = blockIdx.x, b = bg / a.Hkv, g = bg % a.Hkv;   // one query head: h = g
  const int S = a.S, n = a.n;
  const float c = a.scale * kLog2e;
  const size_t head_base = ((size_t)b * a.Hkv + g) * S;
  const char* kh = (const char*)a.kc + head_base * RB;
  const char* vh = (const char*)a.vc + head_base * RB;

  // Q^T operands of the 32 query columns (rows past n read row 0 and are never stored)
  u32x4 qf[2][DS];
  bool rowok[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = ct * 16 + l16;
    rowok[ct] = r < n;
    const bf16_t* src = (const bf16_t*)a.q + (((size_t)b * n + (rowok[ct] ? r : 0)) * a.Hq + g) * D + lg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ct][ds] = *(const u32x4*)(src + ds * 32);
  }

  // this wave's tiles: wave, wave + 4, ...  (every wave runs `iters` rounds; rounds past its
  // last tile compute nothing)
  const int ntiles = (S + kKeys - 1) / kKeys;
  const int iters = (ntiles + kWaves - 1) / kWaves;
  auto key0_of = [&](int it) { return min(it * kWaves + wave, ntiles - 1) * kKeys; };
  auto live = [&](int it) { return it * kWaves + wave < ntiles; };

  // ---- pass 1: row max and normaliser over this wave's keys ----
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  char* kst = lds + wave * 2 * TB;               // this wave's K and V stages
  char* vst = kst + TB;
  auto stats = [&](const Tile<D>& k, int key0) {  // only the last tile can hold keys past S
    if (key0 + kKeys <= S) tile_stats<D, true>(k, kst, qf, m, l, key0, S, c, lane, l16, lg);
    else tile_stats<D, false>(k, kst, qf, m, l, key0, S, c, lane, l16, lg);
  };
  constexpr int KT = TPW > 0 ? TPW : 1;
  f32x4 sk[KT][2][2];                            // TPW > 0: the scores of this wave's tiles
  if constexpr (TPW > 0) {
    constexpr int DK = 2;                        // K tiles in flight
    Tile<D> kr[DK];
#pragma unroll
    for (int u = 0; u < DK; ++u) load_tile<D>(kr[u], kh, key0_of(min(u, iters - 1)), S, lane);
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      if (it < iters) {
        if (live(it)) {
          const int key0 = key0_of(it);
          stage_tile<D, true>(kr[it % DK], kst, lane);
          scores<D>(kst, qf, sk[it], l16, lg);
          if (key0 + kKeys <= S) stats_from<true>(sk[it], m, l, key0, S, c, lg);
          else stats_from<false>(sk[it], m, l, key0, S, c, lg);
        }
        load_tile<D>(kr[it % DK], kh, key0_of(min(it + DK, iters - 1)), S, lane);
      }
    }
  } else {
    Tile<D> kr[kDepth1];
#pragma unroll
    for (int u = 0; u < kDepth1; ++u) load_tile<D>(kr[u], kh, key0_of(min(u, iters - 1)), S, lane);
    int it0 = 0;
    for (; it0 + kDepth1 < iters; it0 += kDepth1) {
#pragma unroll
      for (int u = 0; u < kDepth1; ++u) {
        if (live(it0 + u)) stats(kr[u], key0_of(it0 + u));
        load_tile<D>(kr[u], kh, key0_of(it0 + u + kDepth1), S, lane);
      }
    }
#pragma unroll
    for (int u = 0; u < kDepth1; ++u)
      if (it0 + u < iters && live(it0 + u)) stats(kr[u], key0_of(it0 + u));
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) l[ct] = sum_across_rows(l[ct]);

  // ---- the waves' row states combined in wave order: log2-domain log-sum-exp per row ----
  if (lg == 0) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      st_m[wave][ct * 16 + l16] = m[ct];
      st_l[wave][ct * 16 + l16] = l[ct];
    }
  }
  __syncthreads();
  float L2[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = ct * 16 + l16;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, st_m[w][r]);
    float ls = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = st_m[w][r];
      ls += st_l[w][r] * ((mw == -INFINITY) ? 0.f : exp2f(mw - mm));
    }
    L2[ct] = mm + log2f(ls);
  }

  // ---- pass 2: probabilities, column masses, output partials ----
  f32x4 oacc[2][DT];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto out_tile = [&](const Tile<D>& k, const Tile<D>& v, int key0) {
    if (key0 + kKeys <= S) tile_out<D, true>(k, v, kst, vst, qf, L2, rowok, oacc, mass_s, key0, S, c, lane, l16, lg);
    else tile_out<D, false>(k, v, kst, vst, qf, L2, rowok, oacc, mass_s, key0, S, c, lane, l16, lg);
  };
  if constexpr (TPW > 0) {
    constexpr int DV = 2;                        // V tiles in flight
    Tile<D> vr[DV];
#pragma unroll
    for (int u = 0; u < DV; ++u) load_tile<D>(vr[u], vh, key0_of(min(u, iters - 1)), S, lane);
#pragma unroll
    for (int it = 0; it < TPW; ++it) {
      if (it < iters) {
        if (live(it)) {
          const int key0 = key0_of(it);
          if (key0 + kKeys <= S)
            out_from<D, true>(sk[it], vr[it % DV], vst, L2, rowok, oacc, mass_s, key0, S, c, lane, l16, lg);
          else
            out_from<D, false>(sk[it], vr[it % DV], vst, L2, rowok, oacc, mass_s, key0, S, c, lane, l16, lg);
        }
        load_tile<D>(vr[it % DV], vh, key0_of(min(it + DV, iters - 1)), S, lane);
      }
    }
  } else {
    Tile<D> kr[kDepth2], vr[kDepth2];
#pragma unroll
    for (int u = 0; u < kDepth2; ++u) {
      load_tile<D>(kr[u], kh, key0_of(min(u, iters - 1)), S, lane);
      load_tile<D>(vr[u], vh, key0_of(min(u, iters - 1)), S, lane);
    }
    int it0 = 0;
    for (; it0 + kDepth2 < iters; it0 += kDepth2) {
#pragma unroll
      for (int u = 0; u < kDepth2; ++u) {
        if (live(it0 + u)) out_tile(kr[u], vr[u], key0_of(it0 + u));
        load_tile<D>(kr[u], kh, key0_of(it0 + u + kDepth2), S, lane);
        load_tile<D>(vr[u], vh, key0_of(it0 + u + kDepth2), S, lane);
      }
    }
#pragma unroll
    for (int u = 0; u < kDepth2; ++u)
      if (it0 + u < iters && live(it0 + u)) out_tile(kr[u], vr[u], key0_of(it0 + u));
  }

  // ---- the four output partials added in wave order; each wave finishes 1/4 of d ----
  __syncthreads();                               // every wave is done with its stages
  float* mass_h = a.mass + ((size_t)b * a.Hq + g) * S;
  for (int j = t; j < S; j += 256) mass_h[j] = mass_s[j];
  float* mb = (float*)lds;
  {
    float* dst = mb + wave * MB;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) dst[((ct * DT + dt) * 4 + v) * 64 + lane] = oacc[ct][dt][v];
  }
  __syncthreads();
  constexpr int DTW = DT / kWaves;               // 16-column output tiles per wave
  const int dt0 = wave * DTW;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = ct * 16 + l16;
    f32x4 o[DTW];
#pragma unroll
    for (int u = 0; u < DTW; ++u) {
      o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[u][v] += mb[w * MB + ((ct * DT + dt0 + u) * 4 + v) * 64 + lane];
    }
    if (!rowok[ct]) continue;
    bf16_t* out = (bf16_t*)a.out + (((size_t)b * n + r) * a.Hq + g) * D;
#pragma unroll
    for (int u = 0; u < DTW; ++u) {
      const int d = (dt0 + u) * 16 + lg * 4;
      uint2 w2;
      w2.x = pack_bf16x2(o[u][0], o[u][1]);
      w2.y = pack_bf16x2(o[u][2], o[u][3]);
      *(uint2*)(out + d) = w2;
    }
    if (wave == 0 && lg == 0) a.lse[((size_t)b * a.Hq + g) * n + r] = L2[ct] * kLn2;
  }
}

}  // namespace

bool attn_fused_fits(const AttnArgs& a, const AttnPlan& p) {
  return a.cu == nullptr && a.lens == nullptr &&
         a.act == DLLM_BF16 && a.kind == kCacheBF16 && a.mass != nullptr && a.Hq == a.Hkv &&
         a.n <= 32 && (a.D == 128 || a.D == 64) && a.S >= 1 && a.S <= kFusedMaxSeq && p.splits == 1;
}

hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.Hkv);
  const size_t lds = (size_t)a.S * sizeof(float);
  const int iters = ((a.S + kKeys - 1) / kKeys + kWaves - 1) / kWaves;   // tiles per wave
  if (a.D == 128) {
    if (iters <= 6) attn_fused<128, 6><<<grid, 256, lds, s>>>(a);
    else attn_fused<128, 0><<<grid, 256, lds, s>>>(a);
  } else {
    if (iters <= 6) attn_fused<64, 6><<<grid, 256, lds, s>>>(a);
    else attn_fused<64, 0><<<grid, 256, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace dllm
