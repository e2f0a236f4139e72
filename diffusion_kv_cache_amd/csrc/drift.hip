// Attention-aware drift test and tracking-set update, plus the FP8 codec check kernel.
//
// What it computes: Elastic-Cache (DAIR academy paper card), core idea -- cosine similarity
// of the previous step's most-attended tokens; when it drops below gamma the later layers are
// recomputed; the most-attended token drifts least, so the minimum over heads is a
// conservative trigger.  Flash-dLLM news summary, selective cache tracking -- a fixed budget
// of the 32 most-attended tokens.
//
// drift_track: one workgroup per (b, h).  The K||V rows of the tracked slots are compared in
// fp64 (16-byte loads, one partial per chunk, DPP sums over rows of 16 lanes, row swaps over
// the four rows, then the four wave sums in order).  Then, when this step's mass is given, a
// radix select over the order-preserving bits of the mass (held in registers) finds the k-th
// largest value in 8-bit passes over the bits below those all keys share (it stops as soon as
// every key of the boundary digit is taken); values above it are taken, and of the values
// equal to it the lowest positions, placed by a prefix count over threads so the set comes out
// in ascending position order; the tracking buffer is refilled from the current cache.  Scans
// within a wave are DPP moves.
// The decision (any head of a sequence below gamma) is taken by the last head of the sequence
// to finish, through an arrival word in a caller workspace, or else by drift_decide, one wave
// per sequence.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

// One DPP move of both halves of a double (all lanes have a source for the patterns used).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over each row of 16 lanes, left in every lane of the row: partners at lane distance
// 1 and 2 (quad permutes), then the mirrored half-row and the mirrored row.  Every step adds
// two operands that are swapped between the partners, so all 16 lanes hold the same bits.
__device__ __forceinline__ double row_sum_f64(double v) {
  v += dpp_f64<0xb1>(v);                         // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4e>(v);                         // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);                        // row_half_mirror
  v += dpp_f64<0x140>(v);                        // row_mirror
  return v;
}

// Sum over the four rows of 16 lanes of a wave (each row holding one value in all its
// lanes), left in every lane: the gfx950 row swaps pair lane l with l ^ 32, then with l ^ 16;
// both partners add the same two operands, so every lane ends with the same bits.
__device__ __forceinline__ double rows_sum_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  v = __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[0] << 32) | (uint32_t)lo[0]) +
      __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi[1] << 32) | (uint32_t)lo[1]);
  const uint64_t w = __builtin_bit_cast(uint64_t, v);
  const auto lo2 = __builtin_amdgcn_permlane16_swap((uint32_t)w, (uint32_t)w, false, false);
  const auto hi2 = __builtin_amdgcn_permlane16_swap((uint32_t)(w >> 32), (uint32_t)(w >> 32), false, false);
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi2[0] << 32) | (uint32_t)lo2[0]) +
         __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi2[1] << 32) | (uint32_t)lo2[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts of 1, 2, 4 and 8
// lanes inside each row of 16, then the running totals of rows 0 and 2 (lanes 15, 47) into
// rows 1 and 3, then that of rows 0-1 (lane 31) into rows 2 and 3.  Lanes without a source
// add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Largest and smallest value over the 64 lanes of a wave, in every lane: DPP moves inside
// each row of 16 (quad permutes, half-row and row mirrors), then the gfx950 row swaps
// (v_permlane32_swap pairs lane l with l ^ 32, v_permlane16_swap with l ^ 16; with both
// operands = v, the two results are v of the lane and of its partner).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  const auto x = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max((uint32_t)x[0], (uint32_t)x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max((uint32_t)y[0], (uint32_t)y[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  const auto x = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = min((uint32_t)x[0], (uint32_t)x[1]);
  const auto y = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return min((uint32_t)y[0], (uint32_t)y[1]);
}

// Order-preserving map of fp32 bits to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Elements of type E in one 16-byte chunk (held in registers), as fp64.
template <typename E>
__device__ __forceinline__ void chunk_f64(const u32x4& w, double* out) {
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = (double)__uint_as_float(w[e] << 16);
      out[2 * e + 1] = (double)__uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = (double)__uint_as_float(w[e]);
  }
}

// Sixteen E4M3 codes (one 16-byte chunk) as fp64 values code * scale (exact: a 4-bit
// significand times a 24-bit one).
__device__ __forceinline__ void chunk_f64_e4m3(const u32x4& w, double scale, double* out) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t lo, hi;
    e4m3x4_to_bf16x4(w[e], lo, hi);
    out[4 * e] = (double)__uint_as_float(lo << 16) * scale;
    out[4 * e + 1] = (double)__uint_as_float(lo & 0xffff0000u) * scale;
    out[4 * e + 2] = (double)__uint_as_float(hi << 16) * scale;
    out[4 * e + 3] = (double)__uint_as_float(hi & 0xffff0000u) * scale;
  }
}

// One workgroup per (b, h): the drift of the previous tracked set, then (do_update) the new
// top-k set and the tracking-buffer refill.  The old set and the buffer are read before any
// write.  Global loads that do not depend on each other are issued together (old positions,
// buffer rows, this step's mass), the cache rows of the cosine stay in flight while the
// top-k runs, and the rows of the new set are requested as soon as it is known, so they
// arrive while the cosine is formed.
// CH: 16-byte chunks of the tracked K||V rows per thread (k * 2 * D / elements per chunk /
// 256, rounded up to a power of two).  Chunk indices past the end are clamped to the last
// chunk, so every load is issued unconditionally, back to back.
// KP: mass values per thread (4, 16 or 64; S <= 256 KP): thread t holds the order keys of
// positions [t KP, t KP + KP) in registers, so position order is (thread, slot) order.
// E: float, bf16_t or uint8_t (FP8: E4M3 codes with one fp32 scale per row, the tracking
// buffer holding the codes and then the scales of its rows).
template <typename E, int CH, int KP>
__global__ __launch_bounds__(256) void drift_track(DriftArgs a, int do_update) {
  constexpr bool F8 = sizeof(E) == 1;
  constexpr int EPC = 16 / (int)sizeof(E);       // elements per 16-byte chunk
  constexpr int kMaxChunks = CH;
  const int h = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int D = a.D, k = a.k, S = a.S;
  int32_t* T = a.track_idx + ((size_t)b * a.Hq + h) * k;
  E* buf = (E*)a.track_buf + ((size_t)b * a.Hq + h) * k * 2 * D;
  const size_t head_base = ((size_t)b * a.Hkv + g) * S * D;  // this KV head's rows
  const E* kh = (const E*)a.kc + head_base;
  const E* vh = (const E*)a.vc + head_base;
  const int cpr = D / EPC;                       // chunks per K (or V) row (power of 2)
  const int cs = __builtin_ctz(cpr);
  const int nch = k * 2 * cpr;                   // chunks of the tracked rows
  // FP8: row scales of this KV head in the cache, and of this head's buffer rows (slot,
  // part) at index 2 slot + part = chunk >> cs, after the codes of the whole buffer
  const float* ksh = F8 ? a.ks + head_base / D : nullptr;
  const float* vsh = F8 ? a.vs + head_base / D : nullptr;
  float* bsc = F8 ? (float*)((uint8_t*)a.track_buf + (size_t)a.B * a.Hq * k * 2 * D) +
                        ((size_t)b * a.Hq + h) * k * 2
                  : nullptr;

  __shared__ double red[3][4];                   // wave sums: [quantity][wave]
  __shared__ int sflag[4];
  __shared__ int32_t sT[64];                     // old tracked positions
  __shared__ int32_t sTn[64 + 256];              // new ones, then a discard slot per thread
  __shared__ __align__(16) uint32_t hist[4][256 + 64];  // per radix pass: 256 digit counts,
                                                        // then one discard slot per lane
  __shared__ __align__(16) uint32_t wext[2][4];  // per wave: largest and smallest key
  __shared__ __align__(16) uint32_t wsum[4];     // per wave: (keys above << 16) + keys equal

  // ---- loads issued together: old positions, buffer rows, this step's mass ----
  const int told = (t < k) ? T[t] : -1;
  u32x4 ub[kMaxChunks];
  float sb[kMaxChunks];                          // FP8: the buffer row's scale
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = min(t + 256 * i, nch - 1);
    ub[i] = *(const u32x4*)(buf + (size_t)c * EPC);
    if constexpr (F8) sb[i] = bsc[c >> cs];
  }
  const int p0 = t * KP;                         // this thread's first position
  const int nv = do_update ? max(0, min(KP, S - p0)) : 0;  // its positions below S
  const float* mass = a.mass + ((size_t)b * a.Hq + h) * S;
  const bool vec_mass = (S % 4 == 0) && (((uintptr_t)a.mass & 15) == 0);
  float mv[KP];
  if (vec_mass) {
#pragma unroll
    for (int u = 0; u < KP / 4; ++u) {
      float4 m4 = {0.f, 0.f, 0.f, 0.f};
      if (4 * u < nv) m4 = *(const float4*)(mass + p0 + 4 * u);
      mv[4 * u] = m4.x;
      mv[4 * u + 1] = m4.y;
      mv[4 * u + 2] = m4.z;
      mv[4 * u + 3] = m4.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < KP; ++i) mv[i] = (i < nv) ? mass[p0 + i] : 0.f;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) hist[p][t] = 0;   // (discard slots are never read)
  if (t < k) sT[t] = told;
  uint32_t key[KP];
  uint32_t kmax = 0u, kmin = 0xffffffffu;        // range of the keys (none: empty range)
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    key[i] = order_key(mv[i]);
    if (i < nv) {
      kmax = max(kmax, key[i]);
      kmin = min(kmin, key[i]);
    }
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  if (lane == 0) {
    wext[0][wave] = kmax;
    wext[1][wave] = kmin;
  }
  __syncthreads();

  // ---- cache rows of the old set: in flight during the top-k ----
  // (okc: the chunk exists and its slot holds a position; the others read row 0 and count
  // as zeros in the cosine)
  u32x4 uc[kMaxChunks];
  bool okc[kMaxChunks];
  float sc[kMaxChunks];                          // FP8: the cache row's scale
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = min(t + 256 * i, nch - 1);
    const int slot = c >> (cs + 1), part = (c >> cs) & 1, d0 = (c & (cpr - 1)) * EPC;
    const int j = sT[slot];
    okc[i] = t + 256 * i < nch && j >= 0 && j < S;
    const int jr = okc[i] ? j : 0;
    uc[i] = *(const u32x4*)((part ? vh : kh) + (jr * D + d0));
    if constexpr (F8) sc[i] = (part ? vsh : ksh)[jr];
  }

  if (do_update) {
    // ---- top-k of this step's mass: the k-th largest key by radix passes ----
    // Every key lies between the largest and the smallest, so the bits above the highest bit
    // where those two differ are common to all keys and need no pass; the passes take 8-bit
    // digits from that bit down (the last one narrower).  Every wave scans the pass's
    // histogram itself, so a pass costs one barrier.
    const uint4 x4 = *(const uint4*)wext[0], n4 = *(const uint4*)wext[1];
    kmax = max(max(x4.x, x4.y), max(x4.z, x4.w));
    kmin = min(min(n4.x, n4.y), min(n4.z, n4.w));
    const uint32_t want = (uint32_t)min(k, S);
    const uint32_t diff = kmax ^ kmin;
    int top = diff ? 31 - __builtin_clz(diff) : -1;  // highest bit not common to all keys
    // the common bits (all 32 when every key is equal: then the lowest positions are taken)
    uint32_t pmask = top < 0 ? 0xffffffffu : top >= 31 ? 0u : ~((2u << top) - 1u);
    uint32_t prefix = kmax & pmask, rem = want;
    for (int pass = 0; top >= 0; ++pass) {
      const int w = min(8, top + 1), shift = top + 1 - w;
      const uint32_t dmask = (1u << w) - 1u;
      uint32_t* hp = hist[pass];
      // keys outside the candidate set count into this lane's discard slot (no branch)
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const bool cand = i < nv && (key[i] & pmask) == prefix;
        atomicAdd(&hp[cand ? (key[i] >> shift) & dmask : 256u + lane], 1u);
      }
      lds_barrier();
      // lane L owns digits 255-4L .. 252-4L (descending, one 16-byte read); inclusive scan
      // over lanes
      const uint4 h4 = *(const uint4*)&hp[252 - 4 * lane];
      const uint32_t cnt[4] = {h4.w, h4.z, h4.y, h4.x};
      const uint32_t own = (h4.x + h4.y) + (h4.z + h4.w);
      const uint32_t inc = wave_inclusive_scan(own);
      const uint32_t exc = inc - own;
      // the digit holding the rem-th largest candidate, how many of it are taken, and how
      // many keys it holds
      uint32_t digit = 0, left = 0, size = 0, above = exc;
      bool found = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!found && above + cnt[e] >= rem) {
          digit = 255u - 4u * lane - e;
          left = rem - above;
          size = cnt[e];
          found = true;
        }
        above += cnt[e];
      }
      const int src = __ffsll((unsigned long long)__ballot(exc < rem && rem <= inc)) - 1;
      digit = __builtin_amdgcn_readlane(digit, src);
      left = __builtin_amdgcn_readlane(left, src);
      size = __builtin_amdgcn_readlane(size, src);
      prefix |= digit << shift;
      pmask |= dmask << shift;
      rem = left;
      top = shift - 1;
      if (left == size) break;                   // the whole digit is taken: the set is known
    }

    // prefix holds the leading bits of the k-th largest key (all 32 unless the passes stopped
    // early because every key of the last digit is taken); `rem` of the keys whose leading
    // bits equal it are taken, lowest positions first.  An exclusive scan over threads of
    // (keys above << 16) + keys equal gives each thread the counts before its positions; a
    // key above goes to slot #above before + min(#equal before, rem), an equal key to
    // #above before + #equal before if that count is below rem.
    uint32_t own = 0;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const uint32_t m = key[i] & pmask;
      if (i < nv) own += m > prefix ? 0x10000u : (m == prefix ? 1u : 0u);
    }
    const uint32_t inc = wave_inclusive_scan(own);
    if (lane == 63) wsum[wave] = inc;
    lds_barrier();
    const uint4 ws = *(const uint4*)wsum;        // one LDS read, summed by selects
    const uint32_t before = inc - own + (wave > 0 ? ws.x : 0u) + (wave > 1 ? ws.y : 0u) +
                            (wave > 2 ? ws.z : 0u);
    // (no branches: a key not taken is written to this thread's discard slot)
    uint32_t ga = before >> 16, ge = before & 0xffffu;
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const uint32_t m = key[i] & pmask;
      const bool ab = i < nv && m > prefix, eq = i < nv && m == prefix;
      const uint32_t slot = ab ? ga + min(ge, rem) : ga + ge;
      const bool take = (ab || (eq && ge < rem)) && slot < (uint32_t)k;
      sTn[take ? slot : 64u + t] = p0 + i;
      ga += ab ? 1u : 0u;
      ge += eq ? 1u : 0u;
    }
    for (int sl = (int)want + t; sl < k; sl += 256) sTn[sl] = -1;
    lds_barrier();
  }

  // ---- rows of the new set: in flight during the cosine (row 0 without an update, so the
  // loads need no branch) ----
  u32x4 un[kMaxChunks];
  bool emp[kMaxChunks];                          // empty slot of the new set (S < k): zero row
  float sn[kMaxChunks];                          // FP8: the new row's scale
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = min(t + 256 * i, nch - 1);
    const int slot = c >> (cs + 1), part = (c >> cs) & 1, d0 = (c & (cpr - 1)) * EPC;
    const int j = do_update ? sTn[slot] : 0;
    emp[i] = j < 0;
    const int jr = j >= 0 ? j : 0;
    un[i] = *(const u32x4*)((part ? vh : kh) + (jr * D + d0));
    if constexpr (F8) sn[i] = (part ? vsh : ksh)[jr];
  }

  // ---- sigma over the previous tracked set (fp64) ----
  // One partial sum per chunk and quantity (independent chains), added in chunk order (a
  // chunk without a tracked row adds zeros); then the 16 lanes of a row, the four rows of a
  // wave and the four waves, each in a fixed order.  When |u| |w| = 0 the rows are equal
  // exactly when both are all zero (a sum of squares is zero only for zero elements).
  double uw = 0.0, uu = 0.0, ww = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    double u[EPC], w[EPC];
    if constexpr (F8) {
      chunk_f64_e4m3(ub[i], (double)sb[i], u);
      chunk_f64_e4m3(uc[i], (double)sc[i], w);
    } else {
      chunk_f64<E>(ub[i], u);
      chunk_f64<E>(uc[i], w);
    }
    double puw = 0.0, puu = 0.0, pww = 0.0;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      puw += u[e] * w[e];
      puu += u[e] * u[e];
      pww += w[e] * w[e];
    }
    uw += okc[i] ? puw : 0.0;
    uu += okc[i] ? puu : 0.0;
    ww += okc[i] ? pww : 0.0;
  }
  const int valid_slot = (t < k) ? (told >= 0 && told < S) : 0;
  uw = rows_sum_f64(row_sum_f64(uw));
  uu = rows_sum_f64(row_sum_f64(uu));
  ww = rows_sum_f64(row_sum_f64(ww));
  const int any_valid = __any(valid_slot) ? 1 : 0;
  if (lane == 0) {
    red[0][wave] = uw;
    red[1][wave] = uu;
    red[2][wave] = ww;
    sflag[wave] = any_valid;
  }
  lds_barrier();

  if (do_update) {
    // ---- new set out, and the tracking buffer refilled with its K||V rows (issued before
    // the sigma below, which only thread 0 forms) ----
    for (int sl = t; sl < k; sl += 256) T[sl] = sTn[sl];
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int c = t + 256 * i;
      if (c < nch) *(u32x4*)(buf + (size_t)c * EPC) = emp[i] ? u32x4{0u, 0u, 0u, 0u} : un[i];
      if constexpr (F8)                          // the row's first chunk carries its scale
        if (c < nch && (c & (cpr - 1)) == 0) bsc[c >> cs] = emp[i] ? 0.f : sn[i];
    }
  }
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
    if (!F) sigma = 1.0;
    else {
      const double den = sqrt(UU) * sqrt(WW);
      sigma = (den == 0.0) ? ((UU == 0.0 && WW == 0.0) ? 1.0 : 0.0) : UW / den;
    }
    // Report in fp32 on the side of gamma the fp64 value lies on.
    float f = (float)sigma;
    if (sigma < (double)a.gamma && !(f < a.gamma)) f = nextafterf(a.gamma, -INFINITY);
    a.sigma[(size_t)b * a.Hq + h] = f;
    if (a.arrive) {
      // The decision in the same launch: every head of sequence b adds 1 + (below gamma) << 32
      // to the sequence's arrival word (device-scope atomic; the data travels in the word, so
      // no other memory needs to be visible); the head that brings the count to Hq is the
      // last, writes refresh[b] from the summed flags and resets the word for the next call.
      unsigned long long* wd = a.arrive + (size_t)b * kDriftArriveStride;
      const unsigned long long inc = 1ull | ((unsigned long long)(f < a.gamma ? 1 : 0) << 32);
      const unsigned long long old = atomicAdd(wd, inc);
      if ((uint32_t)old == (uint32_t)(a.Hq - 1)) {
        a.refresh[b] = ((old >> 32) + (inc >> 32)) ? 1 : 0;
        atomicExch(wd, 0ull);
      }
    }
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

// Keys per thread by row length (the update takes S <= 16384).
template <typename E, int CH>
void launch_drift_track(const DriftArgs& a, int upd, hipStream_t s) {
  dim3 grid(a.Hq, a.B);
  if (a.S <= 1024) drift_track<E, CH, 4><<<grid, 256, 0, s>>>(a, upd);
  else if (a.S <= 4096) drift_track<E, CH, 16><<<grid, 256, 0, s>>>(a, upd);
  else drift_track<E, CH, 64><<<grid, 256, 0, s>>>(a, upd);
}

}  // namespace

hipError_t launch_drift(const DriftArgs& a, hipStream_t s) {
  const int upd = a.mass != nullptr;
  const int esz = a.kind == kCacheF32 ? 4 : a.kind == kCacheFP8 ? 1 : 2;
  const int per = (a.k * 2 * a.D * esz / 16 + 255) / 256;  // chunks per thread, <= 16
  const int ch = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
  if (a.kind == kCacheF32) {
    switch (ch) {
      case 1: launch_drift_track<float, 1>(a, upd, s); break;
      case 2: launch_drift_track<float, 2>(a, upd, s); break;
      case 4: launch_drift_track<float, 4>(a, upd, s); break;
      case 8: launch_drift_track<float, 8>(a, upd, s); break;
      default: launch_drift_track<float, 16>(a, upd, s); break;
    }
  } else if (a.kind == kCacheFP8) {
    switch (ch) {
      case 1: launch_drift_track<uint8_t, 1>(a, upd, s); break;
      case 2: launch_drift_track<uint8_t, 2>(a, upd, s); break;
      default: launch_drift_track<uint8_t, 4>(a, upd, s); break;
    }
  } else {
    switch (ch) {
      case 1: launch_drift_track<bf16_t, 1>(a, upd, s); break;
      case 2: launch_drift_track<bf16_t, 2>(a, upd, s); break;
      case 4: launch_drift_track<bf16_t, 4>(a, upd, s); break;
      default: launch_drift_track<bf16_t, 8>(a, upd, s); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.arrive) return e;
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
