// Attention of every row of a block step with cached softmax statistics (FACache).
//
// What it computes: LaCache (gist.science explainer), Technical Summary, Methodology 1,
// FACache -- for query rows outside the current generation block, the online-softmax state
// (running maximum m, normaliser l, unnormalised output O~) over the keys of the invariant
// region is kept; in later steps of the block a (query tile, KV tile) pair that lies wholly in
// the invariant region is skipped and the kept state seeds the accumulators, so only the
// block's KV tiles are processed for those rows; Inference Workflow -- the first step of a
// block computes everything and fills the caches.  The result is softmax(q k^T * scale) v
// over all S keys for every row (Flash-Cache article, section 3.1), exactly in arithmetic.
//
// One workgroup per (b, KV head g, 32 packed query rows r = i * G + (h - g * G)); its four
// waves are key groups that take every fourth 32-key tile of a phase (two-stage LDS ring per
// wave, DMA staging), with the tile compute and the key-group merge of the forward pass
// (attention_tile.hpp):
//   phase U  the keys outside the block [g0, g0 + n) (tiles cut by the block boundary are
//            masked), then the key groups are merged; in a build step the merged state of the
//            tile's invariant rows is stored.  In a reuse step a tile whose rows are all
//            invariant skips this phase and loads the stored state instead;
//   seed     the merged (or loaded) state goes into key group 0's accumulators;
//   phase G  the block's keys, then the final merge and the output.
// The block rows' queries come from q_blk and are written into q_cache (the cached queries of
// every row); the other rows' queries are read from q_cache.
#include "attention_tile.hpp"

namespace dllm {
namespace {

template <int D>
using FacCfg = Cfg<kCacheBF16, 1, D>;

// One phase of the key loop for key group kw: tiles t0 + kw, t0 + kw + 4, ... below t1,
// through this group's two-stage ring.  inside: the keys that count are those in [gb, ge)
// (else those outside); a tile with no key that counts is skipped, a tile with some keys that
// do not count (or past S) is masked.
template <int D>
__device__ __forceinline__ void fac_phase(char* ring, uint32_t ring_lds, int kw, int lane, int l16, int lg,
                                          const char* kh, const char* vh,
                                          const uint32_t (&koff)[FacCfg<D>::DMA_W],
                                          const uint32_t (&voff)[FacCfg<D>::DMA_W], int t0, int t1,
                                          int S, int gb, int ge, bool inside,
                                          const u32x4 (&qf)[2][D / 32], f32x4 (&oacc)[2][D / 16],
                                          float (&m)[2], float (&lsum)[2], float c) {
  using C = FacCfg<D>;
  const int first = t0 + kw;
  const int cnt = first < t1 ? (t1 - first + 3) / 4 : 0;
  char* ring_kw = ring + kw * 2 * C::STAGE;
  const uint32_t st_lds = ring_lds + (uint32_t)(kw * 2 * C::STAGE);
  if (cnt > 0) dma_tile<kCacheBF16, 1, D>(st_lds, kh, vh, first * kKeys, 0, S, 0, lane, koff, voff);
  for (int j = 0; j < cnt; ++j) {
    DLLM_WAIT_VMCNT(0);
    lds_wave_fence();                            // the wave owns its ring: no barrier
    if (j + 1 < cnt)
      dma_tile<kCacheBF16, 1, D>(st_lds + (uint32_t)(((j + 1) & 1) * C::STAGE), kh, vh,
                                 (first + 4 * (j + 1)) * kKeys, 0, S, 0, lane, koff, voff);
    const int key0 = (first + 4 * j) * kKeys, kend = min(key0 + kKeys, S);
    const bool touches = key0 < ge && kend > gb, within = key0 >= gb && kend <= ge;
    if (inside ? !touches : within) continue;
    const char* st = ring_kw + (j & 1) * C::STAGE;
    if (key0 + kKeys > S || (inside ? !within : touches))
      tile_compute<kCacheBF16, 1, D, true>(st, qf, oacc, m, lsum, key0, S, c, l16, lg, gb, ge, inside);
    else
      tile_compute<kCacheBF16, 1, D, false>(st, qf, oacc, m, lsum, key0, S, c, l16, lg);
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_facache(FacArgs a, int qtiles) {
  using C = FacCfg<D>;
  constexpr int KW = 4, DT = C::DT, DS = C::DS, DTW = DT / KW;
  constexpr int MERGE = KW * 2 * (DT * 4 * 64 + 2 * 64) * 4;
  constexpr int SEED = 2 * DT * 4 * 64 * 4;
  constexpr int RING = KW * 2 * C::STAGE;
  constexpr int LDS = RING > MERGE + SEED ? RING : MERGE + SEED;
  __shared__ __attribute__((aligned(16))) char ring[LDS];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int kw = __builtin_amdgcn_readfirstlane(wave);
  int bg, qt;
  xcd_group_unit(blockIdx.x, a.B * a.Hkv, qtiles, bg, qt);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv, S = a.S;
  const int rows = S * G, row0 = qt * 32;
  const int gb = min(max(a.block_start[b], 0), S - a.n), ge = gb + a.n;
  const bool pure_inv = (min(row0 + 31, rows - 1) / G < gb) || (row0 / G >= ge);
  const bool seeded_from_cache = !a.build && pure_inv;
  const float c = a.scale * kLog2e;

  // Query fragments of the tile's rows.  No address here depends on a divergent branch (a
  // select between the two query buffers under control flow was compiled into one that read
  // the block buffer for every row): row indices are clamped to valid rows (rows past the end
  // read the last row and are never stored), every lane loads from both buffers at in-range
  // addresses, and the value its row needs is selected.
  u32x4 qf[2][DS];
  int ri[2], rh[2];
  bool rok[2], rblk[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = row0 + ct * 16 + l16;
    const int rc = min(r, rows - 1);
    rok[ct] = r < rows;
    ri[ct] = rc / G;
    rh[ct] = g * G + rc % G;
    rblk[ct] = rok[ct] && ri[ct] >= gb && ri[ct] < ge;
    const int ib = min(max(ri[ct] - gb, 0), a.n - 1);
    const bf16_t* sb = (const bf16_t*)a.q_blk + (((size_t)b * a.n + ib) * a.Hq + rh[ct]) * D + lg * 8;
    const bf16_t* sc = (const bf16_t*)a.q_cache + (((size_t)b * S + ri[ct]) * a.Hq + rh[ct]) * D + lg * 8;
    u32x4 xb[DS], xc[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      xb[ds] = *(const u32x4*)(sb + ds * 32);
      xc[ds] = *(const u32x4*)(sc + ds * 32);
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ct][ds] = rblk[ct] ? xb[ds] : xc[ds];
  }
  if (kw == 0) {                                 // the block rows' queries into the query cache
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
      if (rblk[ct]) {
        bf16_t* dst = (bf16_t*)a.q_cache + (((size_t)b * S + ri[ct]) * a.Hq + rh[ct]) * D;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) *(u32x4*)(dst + ds * 32 + lg * 8) = qf[ct][ds];
      }
  }

  constexpr int RPI = 1024 / C::RB;
  uint32_t koff[C::DMA_W], voff[C::DMA_W];
#pragma unroll
  for (int u = 0; u < C::DMA_W; ++u) {
    const int r = u * RPI + lane / C::CPR, sc = lane % C::CPR;
    koff[u] = (uint32_t)(r * C::RB + ((sc ^ swz_k<D>(r)) << 4));
    voff[u] = (uint32_t)(r * C::RB + ((sc ^ attn_swz_v(r)) << 4));
  }
  const size_t head_base = ((size_t)b * a.Hkv + g) * S;
  const char* kh = (const char*)a.kc + head_base * C::RB;
  const char* vh = (const char*)a.vc + head_base * C::RB;
  const uint32_t ring_lds = lds_addr(ring);
  float* mb = (float*)ring;
  float* seedb = (float*)(ring + MERGE);
  const size_t st_row0 = ((size_t)b * a.Hq) * S;          // state row of (b, h = 0, i = 0)
  float* st_o = a.state;                                  // [B, Hq, S, D]
  float* st_ml = a.state + (size_t)a.B * a.Hq * S * D;    // [B, Hq, S, 2]

  f32x4 oacc[2][DT];
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 ofin[2][DTW];
  int dt0 = 0;

  if (!seeded_from_cache) {
    // phase U: the invariant keys, all four key groups, then their merge
    fac_phase<D>(ring, ring_lds, kw, lane, l16, lg, kh, vh, koff, voff, 0, (S + kKeys - 1) / kKeys, S,
                 gb, ge, false, qf, oacc, m, lsum, c);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) lsum[ct] = sum_across_rows(lsum[ct]);
    group_merge<1, D>(mb, oacc, m, lsum, kw, 0, lane, ofin, dt0);
    if (a.build) {                               // keep the invariant rows' state
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        if (!rok[ct] || rblk[ct]) continue;
        const size_t sr = st_row0 + (size_t)rh[ct] * S + ri[ct];
#pragma unroll
        for (int u = 0; u < DTW; ++u)
          *(float4*)(st_o + sr * D + (dt0 + u) * 16 + lg * 4) =
              make_float4(ofin[ct][u][0], ofin[ct][u][1], ofin[ct][u][2], ofin[ct][u][3]);
        if (kw == 0 && lg == 0) *(float2*)(st_ml + sr * 2) = make_float2(m[ct], lsum[ct]);
      }
    }
    // seed: every wave's column slice through LDS into key group 0
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int u = 0; u < DTW; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) seedb[((ct * DT + dt0 + u) * 4 + v) * 64 + lane] = ofin[ct][u][v];
    __syncthreads();
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          oacc[ct][dt][v] = (kw == 0) ? seedb[((ct * DT + dt) * 4 + v) * 64 + lane] : 0.f;
      lsum[ct] = (kw == 0 && lg == 0) ? lsum[ct] : 0.f;
      if (kw != 0) m[ct] = -INFINITY;
    }
    __syncthreads();                             // seed read before the ring is reused
  } else if (kw == 0) {
    // the kept state of the tile's rows (all invariant) seeds key group 0; the loads are
    // unconditional (clamped rows are valid rows) and rows past the end start empty
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const size_t sr = st_row0 + (size_t)rh[ct] * S + ri[ct];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float4 x = *(const float4*)(st_o + sr * D + dt * 16 + lg * 4);
        oacc[ct][dt] = rok[ct] ? f32x4{x.x, x.y, x.z, x.w} : f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const float2 ml = *(const float2*)(st_ml + sr * 2);
      m[ct] = rok[ct] ? ml.x : -INFINITY;
      lsum[ct] = (rok[ct] && lg == 0) ? ml.y : 0.f;
    }
  }

  // phase G: the block's keys
  fac_phase<D>(ring, ring_lds, kw, lane, l16, lg, kh, vh, koff, voff, gb / kKeys, (ge - 1) / kKeys + 1, S,
               gb, ge, true, qf, oacc, m, lsum, c);
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) lsum[ct] = sum_across_rows(lsum[ct]);
  group_merge<1, D>(mb, oacc, m, lsum, kw, 0, lane, ofin, dt0);

#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    if (!rok[ct]) continue;
    const float inv = 1.f / lsum[ct];
    bf16_t* o = (bf16_t*)a.out + (((size_t)b * S + ri[ct]) * a.Hq + rh[ct]) * D;
#pragma unroll
    for (int u = 0; u < DTW; ++u) {
      uint2 w2;
      w2.x = pack_bf16x2(ofin[ct][u][0] * inv, ofin[ct][u][1] * inv);
      w2.y = pack_bf16x2(ofin[ct][u][2] * inv, ofin[ct][u][3] * inv);
      *(uint2*)(o + (dt0 + u) * 16 + lg * 4) = w2;
    }
    if (a.lse && lg == 0 && kw == 0)
      a.lse[((size_t)b * a.Hq + rh[ct]) * S + ri[ct]] = (m[ct] + log2f(lsum[ct])) * kLn2;
  }
}

}  // namespace

hipError_t launch_facache(const FacArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  const int qtiles = (a.S * G + 31) / 32;
  const long long grid = (long long)a.B * a.Hkv * qtiles;
  if (a.D == 128) attn_facache<128><<<(unsigned)grid, 256, 0, s>>>(a, qtiles);
  else attn_facache<64><<<(unsigned)grid, 256, 0, s>>>(a, qtiles);
  return hipGetLastError();
}

}  // namespace dllm
