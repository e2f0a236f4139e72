// Bidirectional block attention over the whole cache, its split-KV merge, and the column
// attention-mass pass.
//
// What it computes: softmax(q k^T * scale) v with no mask (Flash-Cache article, section 3.1;
// LaCache Technical Summary, Problem Statement: bidirectional attention over the full
// context); the online-softmax state (m, l, O~) and its merge over disjoint key ranges
// (LaCache Methodology 1, FACache); the column mass sum_i p_ij that ranks the most-attended
// tokens (Flash-dLLM summary, selective cache tracking).
//
// MFMA formulation (bf16 / fp8 caches).  A workgroup owns (b, KV head g, a tile of packed
// query rows r = i * G + (h - g * G), one key split).  Scores are computed transposed,
// S^T = K Q^T (A = K rows from LDS, B = Q^T held in registers), so each lane owns one query
// and eight keys; the key rows of the two 16-row MFMA tiles are permuted so those eight keys
// are consecutive.  Then O^T += V^T P^T takes P^T straight from the score registers and V^T
// from a transposed LDS copy (one 16-byte read per MFMA).  The running max needs two lane
// exchanges per tile; the normaliser is reduced once at the end.  FP8: K and V are converted
// to bf16 exactly (every E4M3 value is a bf16 value); the K row scale multiplies the score
// column and the V row scale is folded into P.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kKeys = 32;          // keys per tile
constexpr int kVtStride = 40;      // bf16 per transposed-V row (32 keys + 8 pad)

__device__ __forceinline__ int perm_row(int r) {  // key r of a 32-key tile -> LDS row
  return ((r >> 2) & 1) * 16 + ((r >> 3) << 2) + (r & 3);
}

template <int KIND, int QW, int D>
__global__ __launch_bounds__(256) void attn_mfma(AttnArgs a, int qtiles, int splits, int kps) {
  constexpr int KW = 4 / QW;
  constexpr int QT = 32 * QW;
  constexpr int DC = D / 8;          // bf16 chunks per key row
  constexpr int DT = D / 16;         // output d tiles
  constexpr int DS = D / 32;         // score d steps
  constexpr int K_BYTES = kKeys * D * 2;
  constexpr int VT_BYTES = D * kVtStride * 2;
  constexpr int REGION = K_BYTES + VT_BYTES + 2 * kKeys * 4;
  constexpr int UNITS = kKeys * DC;                 // 8-element units per tile per tensor
  constexpr int UPT = UNITS / (64 * QW);            // units per thread
  constexpr int MERGE = (KW - 1) * QW * (2 * DT * 4 * 64 + 4 * 64) * 4;
  constexpr int SMEM = (KW * REGION > MERGE) ? KW * REGION : MERGE;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int qw = wave % QW, kw = wave / QW;
  const int gt = qw * 64 + lane;                    // thread index within the kw group

  int id = blockIdx.x;
  const int split = id % splits;
  id /= splits;
  const int qt = id % qtiles;
  const int bg = id / qtiles;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int rows = a.n * G;
  const float c = a.scale * kLog2e;

  // Q^T fragments for the wave's 32 packed rows (two 16-column tiles).
  const bf16_t* q = (const bf16_t*)a.q;
  u32x4 qf[2][DS];
  const int row0 = qt * QT + qw * 32;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = row0 + ct * 16 + l16;
    const bool ok = r < rows;
    const int i = ok ? r / G : 0, hh = ok ? r % G : 0;
    const bf16_t* src = q + (((size_t)b * a.n + i) * a.Hq + g * G + hh) * D + lg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 x = *(const u32x4*)(src + ds * 32);
      qf[ct][ds] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int kbeg = split * kps;
  const int kend = min(a.S, kbeg + kps);
  const int ntiles = (kend - kbeg + kKeys - 1) / kKeys;
  const int iters = (ntiles + KW - 1) / KW;

  const size_t head_base = ((size_t)b * a.Hkv + g) * a.S;
  const char* kc = (const char*)a.kc;
  const char* vc = (const char*)a.vc;
  constexpr int ELT = (KIND == kCacheFP8) ? 1 : 2;

  // Register-staged loads of one tile (this thread's units of K and V, plus scales).
  u32x4 kreg[UPT], vreg[UPT];
  float sreg = 0.f;
  auto load_tile = [&](int tile) {
    const int key0 = kbeg + tile * kKeys;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = gt + u * 64 * QW;
      const int r = unit / DC, ch = unit % DC;
      const int key = key0 + r;
      const bool ok = tile < ntiles && key < kend;
      const size_t off = ((head_base + (ok ? key : kbeg)) * D + ch * 8) * ELT;
      if constexpr (KIND == kCacheFP8) {
        const uint2 kx = *(const uint2*)(kc + off);
        const uint2 vx = *(const uint2*)(vc + off);
        const u32x4 k8 = e4m3x8_to_bf16x8(kx.x, kx.y);
        const u32x4 v8 = e4m3x8_to_bf16x8(vx.x, vx.y);
        kreg[u] = ok ? k8 : u32x4{0u, 0u, 0u, 0u};
        vreg[u] = ok ? v8 : u32x4{0u, 0u, 0u, 0u};
      } else {
        const u32x4 kx = *(const u32x4*)(kc + off);
        const u32x4 vx = *(const u32x4*)(vc + off);
        kreg[u] = ok ? kx : u32x4{0u, 0u, 0u, 0u};
        vreg[u] = ok ? vx : u32x4{0u, 0u, 0u, 0u};
      }
    }
    if constexpr (KIND == kCacheFP8) {
      if (gt < 2 * kKeys) {
        const int r = gt % kKeys, key = key0 + r;
        const bool ok = tile < ntiles && key < kend;
        const float* sp = gt < kKeys ? a.ks : a.vs;
        sreg = ok ? sp[head_base + key] : 0.f;
      }
    }
  };
  auto store_tile = [&]() {
    char* R = smem + kw * REGION;
    char* KT = R;
    bf16_t* VT = (bf16_t*)(R + K_BYTES);
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = gt + u * 64 * QW;
      const int r = unit / DC, ch = unit % DC;
      const int pr = perm_row(r);
      *(u32x4*)(KT + (pr * DC + (ch ^ (pr & 7))) * 16) = kreg[u];
      const uint32_t vw[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        VT[(ch * 8 + 2 * e) * kVtStride + r] = (bf16_t)(vw[e] & 0xffffu);
        VT[(ch * 8 + 2 * e + 1) * kVtStride + r] = (bf16_t)(vw[e] >> 16);
      }
    }
    if constexpr (KIND == kCacheFP8) {
      if (gt < 2 * kKeys) ((float*)(R + K_BYTES + VT_BYTES))[gt] = sreg;
    }
  };

  f32x4 oacc[2][DT];
  float m[2], lsum[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    m[ct] = -INFINITY;
    lsum[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  load_tile(kw);
  for (int it = 0; it < iters; ++it) {
    const int tile = it * KW + kw;
    store_tile();
    __syncthreads();
    if (it + 1 < iters) load_tile(tile + KW);
    if (tile < ntiles) {
      const char* R = smem + kw * REGION;
      const bf16_t* VT = (const bf16_t*)(R + K_BYTES);
      const float* SC = (const float*)(R + K_BYTES + VT_BYTES);
      const int key0 = kbeg + tile * kKeys;
      bf16x8 kf[2][DS];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const int row = kt * 16 + l16, ch = ds * 4 + lg;
          kf[kt][ds] = as_bf16x8(*(const u32x4*)(R + (row * DC + (ch ^ (row & 7))) * 16));
        }
      bf16x8 vf[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        vf[dt] = as_bf16x8(*(const u32x4*)(VT + (dt * 16 + l16) * kVtStride + lg * 8));
      float ksc[8], vsc[8];
      bool kval[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kval[e] = key0 + lg * 8 + e < kend;
        if constexpr (KIND == kCacheFP8) {
          ksc[e] = SC[lg * 8 + e];
          vsc[e] = SC[kKeys + lg * 8 + e];
        }
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) sacc[kt] = mfma_bf16(kf[kt][ds], as_bf16x8(qf[ct][ds]), sacc[kt]);
        float y[8];
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float sv = sacc[e >> 2][e & 3];
          if constexpr (KIND == kCacheFP8) sv *= ksc[e];
          y[e] = kval[e] ? sv * c : -INFINITY;
          mt = fmaxf(mt, y[e]);
        }
        mt = wave_max_xor(mt, 16);
        mt = wave_max_xor(mt, 32);
        const float mnew = fmaxf(m[ct], mt);
        const bool none = (mnew == -INFINITY);
        const float alpha = none ? 1.f : exp2f(m[ct] - mnew);
        float p[8], ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = none ? 0.f : exp2f(y[e] - mnew);
          ps += p[e];
        }
        lsum[ct] = lsum[ct] * alpha + ps;
        m[ct] = mnew;
        if constexpr (KIND == kCacheFP8) {
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] *= vsc[e];
        }
        u32x4 pw;
        pw.x = pack_bf16x2(p[0], p[1]);
        pw.y = pack_bf16x2(p[2], p[3]);
        pw.z = pack_bf16x2(p[4], p[5]);
        pw.w = pack_bf16x2(p[6], p[7]);
        const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          oacc[ct][dt] = oacc[ct][dt] * alpha;
          oacc[ct][dt] = mfma_bf16(vf[dt], pb, oacc[ct][dt]);
        }
      }
    }
    __syncthreads();
  }

  // Normaliser: each lane group held its own keys' share.
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    lsum[ct] += __shfl_xor(lsum[ct], 16, kWave);
    lsum[ct] += __shfl_xor(lsum[ct], 32, kWave);
  }

  // Merge the KW key groups in order (their ranges are disjoint).
  if constexpr (KW > 1) {
    float* mb = (float*)smem;
    constexpr int BLK = 2 * DT * 4 * 64 + 4 * 64;
    if (kw > 0) {
      float* dst = mb + ((kw - 1) * QW + qw) * BLK;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 4; ++v) dst[((ct * DT + dt) * 4 + v) * 64 + lane] = oacc[ct][dt][v];
        dst[2 * DT * 4 * 64 + (ct * 2) * 64 + lane] = m[ct];
        dst[2 * DT * 4 * 64 + (ct * 2 + 1) * 64 + lane] = lsum[ct];
      }
    }
    __syncthreads();
    if (kw > 0) return;
    for (int w2 = 1; w2 < KW; ++w2) {
      const float* src = mb + ((w2 - 1) * QW + qw) * BLK;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const float m2 = src[2 * DT * 4 * 64 + (ct * 2) * 64 + lane];
        const float l2 = src[2 * DT * 4 * 64 + (ct * 2 + 1) * 64 + lane];
        const float mm = fmaxf(m[ct], m2);
        const float a0 = (m[ct] == -INFINITY) ? 0.f : exp2f(m[ct] - mm);
        const float a1 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mm);
        lsum[ct] = lsum[ct] * a0 + l2 * a1;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            oacc[ct][dt][v] = oacc[ct][dt][v] * a0 + src[((ct * DT + dt) * 4 + v) * 64 + lane] * a1;
        m[ct] = mm;
      }
    }
  }

  // Write: final output when unsplit, else the partial state of this split.
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
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + lg * 4;
        uint2 w2;
        w2.x = pack_bf16x2(oacc[ct][dt][0] * inv, oacc[ct][dt][1] * inv);
        w2.y = pack_bf16x2(oacc[ct][dt][2] * inv, oacc[ct][dt][3] * inv);
        *(uint2*)(o + d) = w2;
      }
      if (lg == 0) a.lse[((size_t)b * a.Hq + h) * a.n + i] = (m[ct] + log2f(lsum[ct])) * kLn2;
    } else {
      const size_t pr = (size_t)split * nrows_all + (size_t)bg * rows + r;
      float* po = a.part + pr * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + lg * 4;
        *(float4*)(po + d) = make_float4(oacc[ct][dt][0], oacc[ct][dt][1], oacc[ct][dt][2], oacc[ct][dt][3]);
      }
      if (lg == 0) {
        float* ml = a.part + (size_t)splits * nrows_all * D + pr * 2;
        ml[0] = m[ct];
        ml[1] = lsum[ct];
      }
    }
  }
}

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

// Column attention mass, second pass after the log-sum-exp is known:
//   mass[b, h, j] = sum_i exp(<q_i, k_j> * scale - lse_i).
// One workgroup per (b, h) and 128 keys; each wave keeps 32 keys' K rows as MFMA operands,
// streams the n queries of head h, and each lane sums its own query's share; the 16 lanes of
// a key are added at the end in a fixed butterfly order.
template <int KIND, int D>
__global__ __launch_bounds__(256) void attn_mass_mfma(AttnArgs a) {
  constexpr int DS = D / 32;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.y, b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int key0 = blockIdx.x * 128 + wave * 32;
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

  const float c = a.scale * kLog2e;
  float acc[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const bf16_t* q = (const bf16_t*)a.q;
  for (int i0 = 0; i0 < a.n; i0 += 16) {
    const int i = i0 + l16;
    const bool ok = i < a.n;
    const bf16_t* src = q + (((size_t)b * a.n + (ok ? i : 0)) * a.Hq + h) * D + lg * 8;
    bf16x8 qf[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const u32x4 x = *(const u32x4*)(src + ds * 32);
      qf[ds] = as_bf16x8(ok ? x : u32x4{0u, 0u, 0u, 0u});
    }
    const float lse2 = ok ? a.lse[((size_t)b * a.Hq + h) * a.n + i] * kLog2e : 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) s = mfma_bf16(kf[kt][ds], qf[ds], s);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[kt][v] += ok ? exp2f(s[v] * ksc[kt][v] * c - lse2) : 0.f;
    }
  }
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
  const int grid = a.B * a.Hkv * qtiles * p.splits;
  if (p.qt == 128) attn_mfma<KIND, 4, D><<<grid, 256, 0, s>>>(a, qtiles, p.splits, p.kps);
  else if (p.qt == 64) attn_mfma<KIND, 2, D><<<grid, 256, 0, s>>>(a, qtiles, p.splits, p.kps);
  else attn_mfma<KIND, 1, D><<<grid, 256, 0, s>>>(a, qtiles, p.splits, p.kps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    attn_merge<bf16_t, D><<<a.B * a.Hkv * rows, 64, 0, s>>>(a, p.splits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mass) {
    dim3 grid2((a.S + 127) / 128, a.B * a.Hq);
    attn_mass_mfma<KIND, D><<<grid2, 256, 0, s>>>(a);
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
