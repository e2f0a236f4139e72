// Tile machinery of the MFMA block attention, shared by the forward pass (attention_fwd.hip)
// and the cached-statistics attention (attention_facache.hip): tile layout and staging in
// LDS, the per-tile score / online-softmax / output update of one wave, and the merge of a
// workgroup's key groups.  See attention_fwd.hip for the layout and the softmax scheme.
#pragma once

#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKeys = 32;          // keys per tile
constexpr float kLazy = 8.0f;      // log2 headroom before the running max is moved

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Per-row chunk swizzle of K tiles (chunk index XOR f(row)): the 16 rows one MFMA operand
// read touches hit 16 (D = 128) or 8 (D = 64) distinct chunk slots.  V tiles use
// attn_swz_v, and the key order of the score MFMAs is attn_perm_key (common.hpp).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? ((r & 3) | (((r >> 3) & 3) << 2)) : ((r & 3) | (((r >> 3) & 1) << 2));
}

template <int KIND, int QW, int D>
struct Cfg {
  static constexpr int KW = 4 / QW;              // key groups
  static constexpr int RB = D * 2;               // bytes per LDS row
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int TILE = kKeys * RB;        // bytes of one K (or V) tile
  static constexpr int SC = (KIND == kCacheFP8) ? 2 * kKeys * 4 : 0;
  static constexpr int STAGE = 2 * TILE + SC;    // K, V, scales
  static constexpr int DS = D / 32, DT = D / 16;
  static constexpr int GT = 64 * QW;             // threads per group
  static constexpr int DMA_T = TILE / 1024;      // 1 KB DMA blocks per tensor tile
  static constexpr int DMA_W = DMA_T / QW;       // ... per wave
  // ring depth: one key group (QW = 4) keeps three tiles in flight; four groups fit two
  // stages each in LDS
  static constexpr int NST = (KIND == kCacheFP8) ? 2 : (QW == 4 ? 4 : QW == 2 ? 3 : 2);
};

// bf16: this wave's share of the DMA blocks of one tile (K and V) into the stage at LDS
// address st (wave-uniform).  koff / voff: this lane's byte offsets within a tile (row r of
// block blk, swizzled chunk), fixed for the whole loop; a full tile's base address is
// wave-uniform (scalar registers), so a transfer costs no vector arithmetic.  The partial last
// tile clamps rows past the end to the split's first row (their scores are masked).
template <int KIND, int QW, int D>
__device__ __forceinline__ void dma_tile(uint32_t st, const char* kh, const char* vh, int key0, int kbeg,
                                         int kend, int qw, int lane, const uint32_t* koff,
                                         const uint32_t* voff) {
  using C = Cfg<KIND, QW, D>;
  constexpr int RPI = 1024 / C::RB;              // rows per DMA block
  if (key0 + kKeys <= kend) {
    const char* kt = kh + (size_t)key0 * C::RB;
    const char* vt = vh + (size_t)key0 * C::RB;
#pragma unroll
    for (int u = 0; u < C::DMA_W; ++u) {
      const uint32_t blk = (uint32_t)(qw + QW * u) * 1024u;
      dma_16B_sbase(koff[u], kt, st + blk);
      dma_16B_sbase(voff[u], vt, st + C::TILE + blk);
    }
  } else {
#pragma unroll
    for (int u = 0; u < C::DMA_W; ++u) {
      const int blk = qw + QW * u;
      const int r = blk * RPI + lane / C::CPR;
      const int key = key0 + r;
      const uint32_t rowb = (uint32_t)((key < kend ? key : kbeg) - r) * C::RB;
      dma_16B_sbase(rowb + koff[u], kh, st + blk * 1024);
      dma_16B_sbase(rowb + voff[u], vh, st + C::TILE + blk * 1024);
    }
  }
}

// FP8: registers for this thread's units of one tile (16 codes each) and its scale.
template <int KIND, int QW, int D>
struct Fp8Stage {
  static constexpr int UNITS = kKeys * D / 16;   // 16-byte units per tensor tile
  static constexpr int UPT = (UNITS + 64 * QW - 1) / (64 * QW);
  u32x4 k[UPT], v[UPT];
  float sc;
};

template <int KIND, int QW, int D>
__device__ __forceinline__ void fp8_load(Fp8Stage<KIND, QW, D>& f, const AttnArgs& a, const char* kc,
                                         const char* vc, size_t head_base, int key0, int kbeg,
                                         int kend, int gt) {
  constexpr int UPR = D / 16;                    // units per row
#pragma unroll
  for (int u = 0; u < Fp8Stage<KIND, QW, D>::UPT; ++u) {
    const int unit = gt + u * 64 * QW;
    if (unit >= Fp8Stage<KIND, QW, D>::UNITS) break;
    const int r = unit / UPR, c = unit % UPR;
    const int key = key0 + r;
    const size_t off = (head_base + (key < kend ? key : kbeg)) * D + c * 16;
    f.k[u] = *(const u32x4*)(kc + off);
    f.v[u] = *(const u32x4*)(vc + off);
  }
  if (gt < 2 * kKeys) {
    const int r = gt % kKeys, key = key0 + r;
    const float* sp = gt < kKeys ? a.ks : a.vs;
    f.sc = key < kend ? sp[head_base + key] : 0.f;
  }
}

template <int KIND, int QW, int D>
__device__ __forceinline__ void fp8_store(const Fp8Stage<KIND, QW, D>& f, char* st, int gt) {
  using C = Cfg<KIND, QW, D>;
  constexpr int UPR = D / 16;
#pragma unroll
  for (int u = 0; u < Fp8Stage<KIND, QW, D>::UPT; ++u) {
    const int unit = gt + u * 64 * QW;
    if (unit >= Fp8Stage<KIND, QW, D>::UNITS) break;
    const int r = unit / UPR, c0 = 2 * (unit % UPR);
    const u32x4 k0 = e4m3x8_to_bf16x8(f.k[u].x, f.k[u].y), k1 = e4m3x8_to_bf16x8(f.k[u].z, f.k[u].w);
    const u32x4 v0 = e4m3x8_to_bf16x8(f.v[u].x, f.v[u].y), v1 = e4m3x8_to_bf16x8(f.v[u].z, f.v[u].w);
    *(u32x4*)(st + r * C::RB + ((c0 ^ swz_k<D>(r)) << 4)) = k0;
    *(u32x4*)(st + r * C::RB + (((c0 + 1) ^ swz_k<D>(r)) << 4)) = k1;
    *(u32x4*)(st + C::TILE + r * C::RB + ((c0 ^ attn_swz_v(r)) << 4)) = v0;
    *(u32x4*)(st + C::TILE + r * C::RB + (((c0 + 1) ^ attn_swz_v(r)) << 4)) = v1;
  }
  if (gt < 2 * kKeys) ((float*)(st + 2 * C::TILE))[gt] = f.sc;
}

// One 32-key tile for one wave: scores, lazy online softmax, O^T update.  MASKED: the tile
// may hold keys that do not count: keys at or past kend, and keys whose membership of
// [mlo, mhi) is not `inside` (only a split's last tile, or a tile cut by a block boundary, so
// the key loops carry no masking work on the other tiles).  The tile must hold at least one
// key that counts.
template <int KIND, int QW, int D, bool MASKED>
__device__ __forceinline__ void tile_compute(const char* st, const u32x4 (&qf)[2][D / 32],
                                             f32x4 (&oacc)[2][D / 16], float (&m)[2],
                                             float (&lsum)[2], int key0, int kend, float c,
                                             int l16, int lg, int mlo = 0,
                                             int mhi = 0x7fffffff, bool inside = true) {
  using C = Cfg<KIND, QW, D>;
  const char* K = st;
  const char* V = st + C::TILE;
  const float* SC = (const float*)(st + 2 * C::TILE);
  f32x4 sacc[2][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sacc[ct][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ds = 0; ds < C::DS; ++ds) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int R = attn_perm_key(kt, l16), ch = ds * 4 + lg;
      const bf16x8 kf = as_bf16x8(*(const u32x4*)(K + R * C::RB + ((ch ^ swz_k<D>(R)) << 4)));
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) sacc[ct][kt] = mfma_bf16(kf, as_bf16x8(qf[ct][ds]), sacc[ct][kt]);
    }
  }
  float ksc[8], vsc[8];
  if constexpr (KIND == kCacheFP8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ksc[e] = SC[lg * 8 + e];
      vsc[e] = SC[kKeys + lg * 8 + e];
    }
  }
  bf16x8 pb[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sv[e] = sacc[ct][e >> 2][e & 3];
      if constexpr (KIND == kCacheFP8) sv[e] *= ksc[e];
    }
    if constexpr (MASKED) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = key0 + lg * 8 + e;
        if (j >= kend || ((j >= mlo && j < mhi) != inside)) sv[e] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mx = max_across_rows(mx);
    const float mt = mx * c;                     // this tile's column max, log2 domain
    // Lazy rescale: move the running max only when a score would exceed it by 2^kLazy.
    if (__any(mt > m[ct] + kLazy)) {
      const float mn = fmaxf(m[ct], mt);
      const float alpha = (mn == -INFINITY || m[ct] == -INFINITY) ? 0.f : exp2f(m[ct] - mn);
      lsum[ct] *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) oacc[ct][dt] = oacc[ct][dt] * alpha;
      m[ct] = mn;
    }
    // Every tile holds a valid key, so m[ct] is finite here; masked keys give exp2(-inf) = 0.
    // The exponent is at most kLazy, so the raw hardware exp2 needs no range handling.
    const float mneg = -m[ct];
    float p[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], c, mneg));
      ps += p[e];
    }
    lsum[ct] += ps;
    if constexpr (KIND == kCacheFP8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] *= vsc[e];
    }
    u32x4 pw;
    pw.x = pack_bf16x2(p[0], p[1]);
    pw.y = pack_bf16x2(p[2], p[3]);
    pw.z = pack_bf16x2(p[4], p[5]);
    pw.w = pack_bf16x2(p[6], p[7]);
    pb[ct] = as_bf16x8(pw);
  }
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    s16x4 h[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int R = 8 * lg + 4 * hh + (l16 >> 2);
      const int d0 = 16 * dt + 4 * (l16 & 3);
      const int ch = d0 >> 3;
      const char* addr = V + R * C::RB + ((ch ^ attn_swz_v(R)) << 4) + ((d0 & 4) ? 8 : 0);
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

// Merge of the KW key groups of a workgroup (disjoint key sets) through LDS `mb` (at least
// KW * QW * 2 * (D / 16 * 4 * 64 + 2 * 64) floats, free when called): every wave writes its
// state (unnormalised output, running max and normaliser), then each wave combines a 1/KW
// slice of the output columns for all groups, in group order.  On return ofin[ct][u] holds
// output columns (dt0 + u) * 16 + 4 lg + v of the wave's rows and m / lsum the merged max and
// normaliser (log2 domain).  lsum must already be summed across the four row groups.
template <int QW, int D>
__device__ __forceinline__ void group_merge(float* mb, const f32x4 (&oacc)[2][D / 16], float (&m)[2],
                                            float (&lsum)[2], int kw, int qw, int lane,
                                            f32x4 (&ofin)[2][D / 16 / (4 / QW)], int& dt0) {
  constexpr int KW = 4 / QW, DT = D / 16, DTW = DT / KW;
  constexpr int BLK = 2 * (DT * 4 * 64 + 2 * 64);
  if constexpr (KW > 1) {
    __syncthreads();                             // every wave is done with the buffer
    {
      float* dst = mb + (kw * QW + qw) * BLK;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float* dc = dst + ct * (DT * 4 * 64 + 2 * 64);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 4; ++v) dc[(dt * 4 + v) * 64 + lane] = oacc[ct][dt][v];
        dc[DT * 4 * 64 + lane] = m[ct];
        dc[DT * 4 * 64 + 64 + lane] = lsum[ct];
      }
    }
    __syncthreads();
    dt0 = kw * DTW;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float mm = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < KW; ++w2)
        mm = fmaxf(mm, mb[(w2 * QW + qw) * BLK + ct * (DT * 4 * 64 + 2 * 64) + DT * 4 * 64 + lane]);
      float L = 0.f;
#pragma unroll
      for (int u = 0; u < DTW; ++u) ofin[ct][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w2 = 0; w2 < KW; ++w2) {
        const float* src = mb + (w2 * QW + qw) * BLK + ct * (DT * 4 * 64 + 2 * 64);
        const float mw = src[DT * 4 * 64 + lane];
        const float aw = (mw == -INFINITY) ? 0.f : exp2f(mw - mm);
        L += src[DT * 4 * 64 + 64 + lane] * aw;
#pragma unroll
        for (int u = 0; u < DTW; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) ofin[ct][u][v] += src[((dt0 + u) * 4 + v) * 64 + lane] * aw;
      }
      m[ct] = mm;
      lsum[ct] = L;
    }
  } else {
    dt0 = 0;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int u = 0; u < DTW; ++u) ofin[ct][u] = oacc[ct][u];
  }
}

}  // namespace
}  // namespace dllm
