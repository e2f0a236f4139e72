// Bidirectional block attention, forward pass (MFMA, split over keys).
//
// What it computes: softmax(q k^T * scale) v with no mask over every cache row (Flash-Cache
// article, section 3.1; LaCache Technical Summary, Problem Statement: bidirectional attention
// over the full context), plus the online-softmax state (m, l, O~) of each key split, merged
// in a fixed order (the FACache identity, LaCache Methodology 1).
//
// A workgroup owns (b, KV head g, a tile of packed query rows r = i * G + (h - g * G), one
// key split).  Its four waves form KW groups of QW waves; each wave holds 32 query rows, each
// group streams its own share of the split's 32-key tiles through an LDS ring of its own.
//
// Layout of a tile in LDS: K and V rows as in the cache (row-major, bf16), 16-byte chunks
// XOR-swizzled per row.  bf16 caches are copied global -> LDS by the DMA path of the vector
// memory unit (no registers); FP8 caches go through registers, are converted to bf16 (exact)
// and stored in the same layout.
//
// Scores are computed transposed, S^T = K Q^T (A = K rows, read with their key order
// permuted so that each lane's eight score slots are eight consecutive keys; B = Q^T held in
// registers).  O^T += V^T P^T takes P^T straight from the score registers; V^T comes from two
// transposing LDS reads (ds_read_b64_tr_b16), which hand each lane four consecutive keys of
// one column.  Softmax rescaling is lazy: the running maximum used for the exponentials only
// moves when a score exceeds it by more than 2^8 (in base 2), so most tiles skip the rescale
// of the accumulators.  FP8: the K row scale multiplies the score column and the V row scale
// is folded into P.
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
// may hold keys past the split's end (only a split's last tile, which the key loop leaves for
// after the loop, so the loop carries no masking work).
template <int KIND, int QW, int D, bool MASKED>
__device__ __forceinline__ void tile_compute(const char* st, const u32x4 (&qf)[2][D / 32],
                                             f32x4 (&oacc)[2][D / 16], float (&m)[2],
                                             float (&lsum)[2], int key0, int kend, float c,
                                             int l16, int lg) {
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
      for (int e = 0; e < 8; ++e)
        if (key0 + lg * 8 + e >= kend) sv[e] = -INFINITY;
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

template <int KIND, int QW, int D>
__global__ __launch_bounds__(256) void attn_fwd(AttnArgs a, int qtiles, int splits, int kps) {
  using C = Cfg<KIND, QW, D>;
  constexpr int KW = C::KW, QT = 32 * QW;
  // NST-stage ring per key group (bf16: NST - 1 tiles in flight; FP8 uses two stages).
  constexpr int NST = C::NST;
  // (also the key-group merge buffer: KW x QW waves x two column tiles of D x 16 + 2 values)
  constexpr int MERGE_BYTES = (KW > 1) ? KW * QW * 2 * (C::DT * 4 * 64 + 2 * 64) * 4 : 0;
  constexpr int RING_BYTES = KW * NST * C::STAGE > MERGE_BYTES ? KW * NST * C::STAGE : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) char ring[RING_BYTES];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  // wave-uniform indices (scalar registers: the DMA stage addresses derive from them)
  const int qw = __builtin_amdgcn_readfirstlane(wave % QW), kw = __builtin_amdgcn_readfirstlane(wave / QW);
  const int gt = qw * 64 + lane;

  // All query tiles and key splits of one (b, KV head) run on one XCD: its K/V rows are
  // fetched into that L2 once.
  int bg, unit;
  xcd_group_unit(blockIdx.x, a.B * a.Hkv, qtiles * splits, bg, unit);
  const int split = unit % splits;
  const int qt = unit / splits;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = a.n * G;
  const float c = a.scale * kLog2e;

  const bf16_t* q = (const bf16_t*)a.q;
  u32x4 qf[2][C::DS];
  const int row0 = qt * QT + qw * 32;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = row0 + ct * 16 + l16;
    const bool ok = r < rows;
    const int i = ok ? r / G : 0, hh = ok ? r % G : 0;
    const bf16_t* src = q + (((size_t)b * a.n + i) * a.Hq + g * G + hh) * D + lg * 8;
    // Rows past the end read row 0 (finite data): their score columns are never stored, and
    // not selecting here keeps these loads in flight together with the first tile's.
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) qf[ct][ds] = *(const u32x4*)(src + ds * 32);
  }

  const int kbeg = split * kps;
  const int kend = min(a.S, kbeg + kps);
  const int ntiles = (kend - kbeg + kKeys - 1) / kKeys;
  const int iters = (ntiles + KW - 1) / KW;
  const size_t head_base = ((size_t)b * a.Hkv + g) * a.S;
  const char* kc = (const char*)a.kc;
  const char* vc = (const char*)a.vc;
  char* ring_kw = ring + kw * NST * C::STAGE;
  char* st0 = ring_kw;
  char* st1 = ring_kw + C::STAGE;

  f32x4 oacc[2][C::DT];
  float m[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) oacc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (KIND == kCacheFP8) {
    Fp8Stage<KIND, QW, D> f;
    fp8_load<KIND, QW, D>(f, a, kc, vc, head_base, kbeg + kw * kKeys, kbeg, kend, gt);
    fp8_store<KIND, QW, D>(f, st0, gt);
    for (int it = 0; it < iters; ++it) {
      const int tile = it * KW + kw;
      // One wave per key group stages and reads its own tiles (LDS operations of a wave take
      // effect in issue order), so only groups of several waves need the barrier.
      if constexpr (QW > 1) __syncthreads();
      if (it + 1 < iters) fp8_load<KIND, QW, D>(f, a, kc, vc, head_base, kbeg + (tile + KW) * kKeys, kbeg, kend, gt);
      if (tile < ntiles && kbeg + (tile + 1) * kKeys <= kend)
        tile_compute<KIND, QW, D, false>((it & 1) ? st1 : st0, qf, oacc, m, lsum, kbeg + tile * kKeys,
                                         kend, c, l16, lg);
      if (it + 1 < iters) fp8_store<KIND, QW, D>(f, (it & 1) ? st0 : st1, gt);
    }
    // The split's partial last tile (if this group owns it) is still in its stage.
    const int last = ntiles - 1;
    if (last >= 0 && last % KW == kw && kbeg + (last + 1) * kKeys > kend)
      tile_compute<KIND, QW, D, true>(((last / KW) & 1) ? st1 : st0, qf, oacc, m, lsum,
                                      kbeg + last * kKeys, kend, c, l16, lg);
  } else {
    constexpr int PEND = 2 * C::DMA_W;           // DMA ops of one tile per wave
    constexpr int RPI = 1024 / C::RB;
    uint32_t koff[C::DMA_W], voff[C::DMA_W];
#pragma unroll
    for (int u = 0; u < C::DMA_W; ++u) {
      const int r = (qw + QW * u) * RPI + lane / C::CPR, sc = lane % C::CPR;
      koff[u] = (uint32_t)(r * C::RB + ((sc ^ swz_k<D>(r)) << 4));
      voff[u] = (uint32_t)(r * C::RB + ((sc ^ attn_swz_v(r)) << 4));
    }
    const char* kh = kc + head_base * C::RB;
    const char* vh = vc + head_base * C::RB;
    const uint32_t ring_st = lds_addr(ring) + (uint32_t)(kw * NST * C::STAGE);   // this group's ring
    // prologue: the first NST - 1 tiles of this key group
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
      if (st < iters)
        dma_tile<KIND, QW, D>(ring_st + st * C::STAGE, kh, vh, kbeg + (st * KW + kw) * kKeys, kbeg,
                              kend, qw, lane, koff, voff);
    // The query operands (ordinary loads, issued first) are complete here as far as the
    // compiler can tell: otherwise it keeps waiting for them inside the loop, on a counter
    // that also counts the tile transfers in flight, and drains the ring on every tile.
    DLLM_WAIT_VMCNT(0);
    // Unrolled by the ring depth, so the LDS addresses of every slot are constant offsets
    // from one per-lane base (no address arithmetic per tile).
    for (int it0 = 0; it0 < iters; it0 += NST) {
#pragma unroll
      for (int u = 0; u < NST; ++u) {
        const int it = it0 + u;                  // it % NST == u
        if (it >= iters) break;
        // this wave's transfers for tile `it` are done once at most those of the later tiles
        // already issued are outstanding
        if (it + NST - 2 < iters) DLLM_WAIT_VMCNT(PEND * (NST - 2));
        else DLLM_WAIT_VMCNT(0);
        // tile `it` visible; slot of it - 1 free (a one-wave group owns its ring: no barrier)
        if constexpr (QW == 1) lds_wave_fence();
        else lds_barrier();
        if (it + NST - 1 < iters)
          dma_tile<KIND, QW, D>(ring_st + ((u + NST - 1) % NST) * C::STAGE, kh, vh,
                                kbeg + ((it + NST - 1) * KW + kw) * kKeys, kbeg, kend, qw, lane, koff,
                                voff);
        const int tile = it * KW + kw;
        if (tile < ntiles && kbeg + (tile + 1) * kKeys <= kend)
          tile_compute<KIND, QW, D, false>(ring_kw + u * C::STAGE, qf, oacc, m, lsum, kbeg + tile * kKeys,
                                           kend, c, l16, lg);
      }
    }
    // The split's partial last tile, if this group owns it: its stage was filled at the
    // group's last iteration and no transfer was issued after that.
    const int last = ntiles - 1;
    if (last >= 0 && last % KW == kw && kbeg + (last + 1) * kKeys > kend)
      tile_compute<KIND, QW, D, true>(ring_kw + ((last / KW) % NST) * C::STAGE, qf, oacc, m, lsum,
                                      kbeg + last * kKeys, kend, c, l16, lg);
    lds_barrier();                               // ring reads done before the merge reuses it
  }

  // Normaliser: each lane group held its own keys' share.
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) lsum[ct] = sum_across_rows(lsum[ct]);

  // Merge the KW key groups (disjoint key ranges) through the idle ring: every wave writes its
  // state, then each wave combines a 1/KW slice of the output columns d for all groups, in
  // group order, and writes that slice.
  constexpr int DTW = C::DT / KW;                // output 16-column tiles per wave
  int dt0 = 0;
  f32x4 ofin[2][DTW];
  if constexpr (KW > 1) {
    constexpr int BLK = 2 * (C::DT * 4 * 64 + 2 * 64);
    static_assert(KW * QW * BLK * 4 <= RING_BYTES, "merge buffer does not fit");
    float* mb = (float*)ring;
    __syncthreads();                             // every wave is done with the ring
    {
      float* dst = mb + (kw * QW + qw) * BLK;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float* dc = dst + ct * (C::DT * 4 * 64 + 2 * 64);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int v = 0; v < 4; ++v) dc[(dt * 4 + v) * 64 + lane] = oacc[ct][dt][v];
        dc[C::DT * 4 * 64 + lane] = m[ct];
        dc[C::DT * 4 * 64 + 64 + lane] = lsum[ct];
      }
    }
    __syncthreads();
    dt0 = kw * DTW;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float mm = -INFINITY;
#pragma unroll
      for (int w2 = 0; w2 < KW; ++w2)
        mm = fmaxf(mm, mb[(w2 * QW + qw) * BLK + ct * (C::DT * 4 * 64 + 2 * 64) + C::DT * 4 * 64 + lane]);
      float L = 0.f;
#pragma unroll
      for (int u = 0; u < DTW; ++u) ofin[ct][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w2 = 0; w2 < KW; ++w2) {
        const float* src = mb + (w2 * QW + qw) * BLK + ct * (C::DT * 4 * 64 + 2 * 64);
        const float mw = src[C::DT * 4 * 64 + lane];
        const float aw = (mw == -INFINITY) ? 0.f : exp2f(mw - mm);
        L += src[C::DT * 4 * 64 + 64 + lane] * aw;
#pragma unroll
        for (int u = 0; u < DTW; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) ofin[ct][u][v] += src[((dt0 + u) * 4 + v) * 64 + lane] * aw;
      }
      m[ct] = mm;
      lsum[ct] = L;
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int u = 0; u < DTW; ++u) ofin[ct][u] = oacc[ct][u];
  }

  // This wave's slice of the final output when unsplit, else of this split's partial state.
  const size_t nrows_all = (size_t)a.B * a.Hkv * rows;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = row0 + ct * 16 + l16;
    if (r >= rows) continue;
    const int i = r / G, h = g * G + r % G;
    if (splits == 1) {
      const float inv = 1.f / lsum[ct];
      bf16_t* o = (bf16_t*)a.out + (((size_t)b * a.n + i) * a.Hq + h) * D;
#pragma unroll
      for (int u = 0; u < DTW; ++u) {
        const int d = (dt0 + u) * 16 + lg * 4;
        uint2 w2;
        w2.x = pack_bf16x2(ofin[ct][u][0] * inv, ofin[ct][u][1] * inv);
        w2.y = pack_bf16x2(ofin[ct][u][2] * inv, ofin[ct][u][3] * inv);
        *(uint2*)(o + d) = w2;
      }
      if (lg == 0 && kw == 0) a.lse[((size_t)b * a.Hq + h) * a.n + i] = (m[ct] + log2f(lsum[ct])) * kLn2;
    } else {
      const size_t pr = (size_t)split * nrows_all + (size_t)bg * rows + r;
      float* po = a.part + pr * D;
#pragma unroll
      for (int u = 0; u < DTW; ++u) {
        const int d = (dt0 + u) * 16 + lg * 4;
        *(float4*)(po + d) = make_float4(ofin[ct][u][0], ofin[ct][u][1], ofin[ct][u][2], ofin[ct][u][3]);
      }
      if (lg == 0 && kw == 0) {
        float* ml = a.part + (size_t)splits * nrows_all * D + pr * 2;
        ml[0] = m[ct];
        ml[1] = lsum[ct];
      }
    }
  }
}

}  // namespace

template <int KIND, int D>
hipError_t launch_attn_fwd(const AttnArgs& a, const AttnPlan& p, int qtiles, hipStream_t s) {
  const int grid = a.B * a.Hkv * qtiles * p.splits;
  if (p.qt == 128) attn_fwd<KIND, 4, D><<<grid, 256, 0, s>>>(a, qtiles, p.splits, p.kps);
  else if (p.qt == 64) attn_fwd<KIND, 2, D><<<grid, 256, 0, s>>>(a, qtiles, p.splits, p.kps);
  else attn_fwd<KIND, 1, D><<<grid, 256, 0, s>>>(a, qtiles, p.splits, p.kps);
  return hipGetLastError();
}

template hipError_t launch_attn_fwd<kCacheBF16, 128>(const AttnArgs&, const AttnPlan&, int, hipStream_t);
template hipError_t launch_attn_fwd<kCacheBF16, 64>(const AttnArgs&, const AttnPlan&, int, hipStream_t);
template hipError_t launch_attn_fwd<kCacheFP8, 128>(const AttnArgs&, const AttnPlan&, int, hipStream_t);
template hipError_t launch_attn_fwd<kCacheFP8, 64>(const AttnArgs&, const AttnPlan&, int, hipStream_t);

}  // namespace dllm
