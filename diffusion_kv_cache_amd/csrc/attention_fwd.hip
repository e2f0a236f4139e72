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

#include "attention_tile.hpp"

namespace dllm {
namespace {

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
  const int nb = seq_rows(a.cu, a.n, b), q0 = seq_row0(a.cu, a.n, b);
  const int rows = nb * G;
  // query tiles past this sequence's rows (a variable-length batch): nothing to do
  if (qt * QT >= rows) return;
  const float c = a.scale * kLog2e;

  const bf16_t* q = (const bf16_t*)a.q;
  u32x4 qf[2][C::DS];
  const int row0 = qt * QT + qw * 32;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = row0 + ct * 16 + l16;
    const bool ok = r < rows;
    const int i = ok ? r / G : 0, hh = ok ? r % G : 0;
    const bf16_t* src = q + (((size_t)q0 + i) * a.Hq + g * G + hh) * D + lg * 8;
    // Rows past the end read row 0 (finite data): their score columns are never stored, and
    // not selecting here keeps these loads in flight together with the first tile's.
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) qf[ct][ds] = *(const u32x4*)(src + ds * 32);
  }

  const int kbeg = split * kps;
  const int kend = min(seq_keys(a.lens, a.S, b), kbeg + kps);
  const int ntiles = max(0, (kend - kbeg + kKeys - 1) / kKeys);   // 0: no key of this split counts
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

  // Merge the KW key groups (disjoint key ranges) through the idle ring.
  constexpr int DTW = C::DT / KW;                // output 16-column tiles per wave
  static_assert(KW == 1 || KW * QW * 2 * (C::DT * 4 * 64 + 2 * 64) * 4 <= RING_BYTES,
                "merge buffer does not fit");
  int dt0 = 0;
  f32x4 ofin[2][DTW];
  group_merge<QW, D>((float*)ring, oacc, m, lsum, kw, qw, lane, ofin, dt0);

  // This wave's slice of the final output when unsplit, else of this split's partial state.
  const size_t nrows_all = (size_t)a.T * a.Hq;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = row0 + ct * 16 + l16;
    if (r >= rows) continue;
    const int i = r / G, h = g * G + r % G;
    if (splits == 1) {
      const float inv = 1.f / lsum[ct];
      bf16_t* o = (bf16_t*)a.out + (((size_t)q0 + i) * a.Hq + h) * D;
#pragma unroll
      for (int u = 0; u < DTW; ++u) {
        const int d = (dt0 + u) * 16 + lg * 4;
        uint2 w2;
        w2.x = pack_bf16x2(ofin[ct][u][0] * inv, ofin[ct][u][1] * inv);
        w2.y = pack_bf16x2(ofin[ct][u][2] * inv, ofin[ct][u][3] * inv);
        *(uint2*)(o + d) = w2;
      }
      if (lg == 0 && kw == 0) a.lse[(size_t)q0 * a.Hq + (size_t)h * nb + i] = (m[ct] + log2f(lsum[ct])) * kLn2;
    } else {
      const size_t pr = (size_t)split * nrows_all + (size_t)q0 * a.Hq + (size_t)g * rows + r;
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
