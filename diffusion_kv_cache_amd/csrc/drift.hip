// Attention-aware drift test and tracking-set update, plus the FP8 codec check kernel.
//
// What it computes: Elastic-Cache (DAIR academy paper card), core idea -- cosine similarity
// of the previous step's most-attended tokens; when it drops below gamma the later layers are
// recomputed; the most-attended token drifts least, so the minimum over heads is a
// conservative trigger.  Flash-dLLM news summary, selective cache tracking -- a fixed budget
// of the 32 most-attended tokens.
//
// drift_track: one workgroup per (b, h).  The K||V rows of the tracked slots are compared in
// fp64 (16-byte loads, DPP sums over rows of 16 lanes, then the 16 row sums in order).  Then,
// when this step's mass is given, a radix select over the order-preserving bits of the mass
// (staged in LDS) finds the k-th largest value in up to four 8-bit passes (it stops as soon as
// every key of the boundary digit is taken); values above it are taken, and of the values
// equal to it the lowest positions, placed by ballot counts so the set comes out in ascending
// position order; the tracking buffer is refilled from the current cache.  Scans within a
// wave are DPP moves.
// drift_decide: one wave per sequence, any head below gamma.
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

// Mass values per thread loaded ahead of everything else (four 16-byte loads): S <= 4096
// needs one round, longer rows take further rounds after it.
constexpr int kMassAhead = 4;

// One workgroup per (b, h): the drift of the previous tracked set, then (do_update) the new
// top-k set and the tracking-buffer refill.  The old set and the buffer are read before any
// write.  Global loads that do not depend on each other are issued together (old positions,
// buffer rows, this step's mass), the cache rows of the cosine stay in flight while the
// top-k runs on LDS, and the rows of the new set are requested as soon as it is known, so
// they arrive while the cosine is formed.
// CH: 16-byte chunks of the tracked K||V rows per thread (k * 2 * D / elements per chunk /
// 256, rounded up to a power of two).  Chunk indices past the end are clamped to the last
// chunk, so every load is issued unconditionally, back to back.
template <typename E, int CH>
__global__ __launch_bounds__(256) void drift_track(DriftArgs a, int do_update) {
  extern __shared__ uint32_t keys[];             // [S] order keys of this head's mass
  constexpr int EPC = 16 / (int)sizeof(E);       // elements per 16-byte chunk
  constexpr int kMaxChunks = CH;
  const int h = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int D = a.D, k = a.k, S = a.S;
  int32_t* T = a.track_idx + ((size_t)b * a.Hq + h) * k;
  E* buf = (E*)a.track_buf + ((size_t)b * a.Hq + h) * k * 2 * D;
  const E* kc = (const E*)a.kc;
  const E* vc = (const E*)a.vc;
  const size_t head_base = ((size_t)b * a.Hkv + g) * S;
  const int cpr = D / EPC;                       // chunks per K (or V) row (power of 2)
  const int cs = __builtin_ctz(cpr);
  const int nch = k * 2 * cpr;                   // chunks of the tracked rows

  __shared__ double red[3][16];                  // row sums: [quantity][wave * 4 + row]
  __shared__ int sflag[4];
  __shared__ int32_t sT[64], sTn[64];            // old and new tracked positions
  __shared__ uint32_t hist[4][256];              // one digit histogram per radix pass
  __shared__ uint32_t wcnt[2][4];                // per wave: keys above, keys equal

  // ---- loads issued together: old positions, buffer rows, the first round of mass ----
  const int told = (t < k) ? T[t] : -1;
  u32x4 ub[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = min(t + 256 * i, nch - 1);
    ub[i] = *(const u32x4*)(buf + (size_t)c * EPC);
  }
  const float* mass = a.mass + ((size_t)b * a.Hq + h) * S;
  const bool vec_mass = do_update && (S % 4 == 0) && (((uintptr_t)a.mass & 15) == 0);
  float4 mr[kMassAhead];
  if (vec_mass) {
#pragma unroll
    for (int u = 0; u < kMassAhead; ++u) {
      const int q = t + 256 * u;
      if (q < S / 4) mr[u] = ((const float4*)mass)[q];
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) hist[p][t] = 0;
  if (t < k) sT[t] = told;
  if (vec_mass) {
#pragma unroll
    for (int u = 0; u < kMassAhead; ++u) {
      const int q = t + 256 * u;
      if (q < S / 4) {
        keys[4 * q] = order_key(mr[u].x);
        keys[4 * q + 1] = order_key(mr[u].y);
        keys[4 * q + 2] = order_key(mr[u].z);
        keys[4 * q + 3] = order_key(mr[u].w);
      }
    }
  }
  __syncthreads();

  // ---- cache rows of the old set: in flight during the top-k ----
  u32x4 uc[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = min(t + 256 * i, nch - 1);
    const int slot = c >> (cs + 1), part = (c >> cs) & 1, d0 = (c & (cpr - 1)) * EPC;
    const int j = sT[slot];
    const int jc = (j >= 0 && j < S) ? j : 0;    // empty slots read row 0, unused below
    uc[i] = *(const u32x4*)((part ? vc : kc) + (head_base + jc) * D + d0);
  }

  if (do_update) {
    // the rest of the mass (rows longer than the first round, or not a multiple of 4)
    if (vec_mass) {
      for (int q = t + 256 * kMassAhead; q < S / 4; q += 256) {
        const float4 m4 = ((const float4*)mass)[q];
        keys[4 * q] = order_key(m4.x);
        keys[4 * q + 1] = order_key(m4.y);
        keys[4 * q + 2] = order_key(m4.z);
        keys[4 * q + 3] = order_key(m4.w);
      }
    } else {
      for (int j = t; j < S; j += 256) keys[j] = order_key(mass[j]);
    }
    lds_barrier();

    // ---- top-k of this step's mass: the k-th largest key by four 8-bit radix passes ----
    // Every wave scans the pass's histogram itself, so a pass costs one barrier.
    const uint32_t want = (uint32_t)min(k, S);
    uint32_t prefix = 0, pmask = 0, rem = want;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      uint32_t* hp = hist[pass];
#pragma unroll 4
      for (int j = t; j < S; j += 256) {
        const uint32_t u = keys[j];
        if ((u & pmask) == prefix) atomicAdd(&hp[(u >> shift) & 255u], 1u);
      }
      lds_barrier();
      // lane L owns digits 255-4L .. 252-4L (descending); inclusive scan over lanes
      uint32_t cnt[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt[e] = hp[255 - 4 * lane - e];
        own += cnt[e];
      }
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
      pmask |= 0xffu << shift;
      rem = left;
      if (left == size) break;                   // the whole digit is taken: the set is known
    }

    // prefix holds the leading bytes of the k-th largest key (all four unless the passes
    // stopped early because every key of the last digit is taken); `rem` of the keys whose
    // leading bytes equal it are taken, lowest positions first.  Wave w walks the positions
    // [w Q, w Q + Q) 64 at a time: ballots count the keys above and equal, the four waves'
    // counts are exchanged once, and a second walk places every taken key at its slot in
    // ascending position order (keys above: #above before it + min(#equal before it, rem);
    // equal keys: #above before + #equal before, if that is below rem).  Q is a multiple of
    // 256 so each round reads four keys per lane before any ballot.
    const int Q = (S + 1023) / 1024 * 256;       // positions per wave, 256 per round
    const int jb = wave * Q;
    uint32_t ngt = 0, neq = 0;
    for (int c = 0; c < Q; c += 256) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = keys[min(jb + c + 64 * e + lane, S - 1)] & pmask;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = jb + c + 64 * e + lane < S;
        ngt += (uint32_t)__builtin_popcountll(__ballot(in && u[e] > prefix));
        neq += (uint32_t)__builtin_popcountll(__ballot(in && u[e] == prefix));
      }
    }
    if (lane == 0) {
      wcnt[0][wave] = ngt;
      wcnt[1][wave] = neq;
    }
    lds_barrier();
    uint32_t gb = 0, eb = 0;
    for (int q = 0; q < wave; ++q) {
      gb += wcnt[0][q];
      eb += wcnt[1][q];
    }
    for (int c = 0; c < Q; c += 256) {
      uint32_t u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) u[e] = keys[min(jb + c + 64 * e + lane, S - 1)] & pmask;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = jb + c + 64 * e + lane;
        const bool in = j < S, above = in && u[e] > prefix, equal = in && u[e] == prefix;
        const unsigned long long ba = __ballot(above), be = __ballot(equal);
        const uint32_t ga = gb + __builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(ba >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ba, 0u));
        const uint32_t ge = eb + __builtin_amdgcn_mbcnt_hi(
                                     (uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
        if (above) {
          const uint32_t slot = ga + min(ge, rem);
          if (slot < (uint32_t)k) sTn[slot] = j;
        } else if (equal && ge < rem && ga + ge < (uint32_t)k) {
          sTn[ga + ge] = j;
        }
        gb += (uint32_t)__builtin_popcountll(ba);
        eb += (uint32_t)__builtin_popcountll(be);
      }
    }
    for (int sl = (int)want + t; sl < k; sl += 256) sTn[sl] = -1;
    lds_barrier();
  }

  // ---- rows of the new set: in flight during the cosine (row 0 without an update, so the
  // loads need no branch) ----
  u32x4 un[kMaxChunks];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = min(t + 256 * i, nch - 1);
    const int slot = c >> (cs + 1), part = (c >> cs) & 1, d0 = (c & (cpr - 1)) * EPC;
    const int j = do_update ? sTn[slot] : 0;
    un[i] = *(const u32x4*)((part ? vc : kc) + (head_base + (j >= 0 ? j : 0)) * D + d0);
  }

  // ---- sigma over the previous tracked set (fp64) ----
  double uw = 0.0, uu = 0.0, ww = 0.0;
  int neq = 0;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = t + 256 * i;
    if (c >= nch) continue;
    const int j = sT[c >> (cs + 1)];
    if (j < 0 || j >= S) continue;
    double u[EPC], w[EPC];
    chunk_f64<E>(ub[i], u);
    chunk_f64<E>(uc[i], w);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      uw += u[e] * w[e];
      uu += u[e] * u[e];
      ww += w[e] * w[e];
      neq |= (u[e] != w[e]);
    }
  }
  const int valid_slot = (t < k) ? (told >= 0 && told < S) : 0;
  uw = row_sum_f64(uw);
  uu = row_sum_f64(uu);
  ww = row_sum_f64(ww);
  const int wflags = (__any(neq) ? 1 : 0) | (__any(valid_slot) ? 2 : 0);
  if ((lane & 15) == 0) {
    red[0][wave * 4 + (lane >> 4)] = uw;
    red[1][wave * 4 + (lane >> 4)] = uu;
    red[2][wave * 4 + (lane >> 4)] = ww;
  }
  if (lane == 0) sflag[wave] = wflags;
  lds_barrier();
  float sig = 1.f;                               // thread 0: this head's sigma
  if (t == 0) {
    double UW = 0.0, UU = 0.0, WW = 0.0;
    int F = 0;
    for (int q = 0; q < 16; ++q) {
      UW += red[0][q];
      UU += red[1][q];
      WW += red[2][q];
    }
    for (int q = 0; q < 4; ++q) F |= sflag[q];
    double sigma;
    if (!(F & 2)) sigma = 1.0;
    else {
      const double den = sqrt(UU) * sqrt(WW);
      sigma = (den == 0.0) ? ((F & 1) ? 0.0 : 1.0) : UW / den;
    }
    // Report in fp32 on the side of gamma the fp64 value lies on.
    float f = (float)sigma;
    if (sigma < (double)a.gamma && !(f < a.gamma)) f = nextafterf(a.gamma, -INFINITY);
    sig = f;
  }
  if (!do_update) {
    if (t == 0) a.sigma[(size_t)b * a.Hq + h] = sig;
    return;
  }

  // ---- new set out, and the tracking buffer refilled with its K||V rows ----
  if (t == 0) a.sigma[(size_t)b * a.Hq + h] = sig;
  for (int sl = t; sl < k; sl += 256) T[sl] = sTn[sl];
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = t + 256 * i;
    if (c < nch) {
      const bool empty = sTn[c >> (cs + 1)] < 0;   // empty slot (S < k): zero row
      *(u32x4*)(buf + (size_t)c * EPC) = empty ? u32x4{0u, 0u, 0u, 0u} : un[i];
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

}  // namespace

hipError_t launch_drift(const DriftArgs& a, hipStream_t s) {
  dim3 grid(a.Hq, a.B);
  const int upd = a.mass != nullptr;
  const size_t lds = upd ? (size_t)a.S * sizeof(uint32_t) : 0;
  const int esz = a.kind == kCacheF32 ? 4 : 2;
  const int per = (a.k * 2 * a.D * esz / 16 + 255) / 256;  // chunks per thread, <= 16
  const int ch = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 16;
  if (a.kind == kCacheF32) {
    switch (ch) {
      case 1: drift_track<float, 1><<<grid, 256, lds, s>>>(a, upd); break;
      case 2: drift_track<float, 2><<<grid, 256, lds, s>>>(a, upd); break;
      case 4: drift_track<float, 4><<<grid, 256, lds, s>>>(a, upd); break;
      case 8: drift_track<float, 8><<<grid, 256, lds, s>>>(a, upd); break;
      default: drift_track<float, 16><<<grid, 256, lds, s>>>(a, upd); break;
    }
  } else {
    switch (ch) {
      case 1: drift_track<bf16_t, 1><<<grid, 256, lds, s>>>(a, upd); break;
      case 2: drift_track<bf16_t, 2><<<grid, 256, lds, s>>>(a, upd); break;
      case 4: drift_track<bf16_t, 4><<<grid, 256, lds, s>>>(a, upd); break;
      default: drift_track<bf16_t, 8><<<grid, 256, lds, s>>>(a, upd); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
