// Fused refresh kernel for large M: gather the refreshed hidden rows, QKV projection on MFMA,
// rotary embedding in registers, scatter of K/V rows into the flat cache (optionally as
// per-row FP8), compact Q out -- one launch, no intermediate in HBM.  Small M (a block step)
// takes the split-K path of refresh_splitk.hip instead.
//
// What it computes: Flash-dLLM news summary (skillfed.io), memory paragraph -- projection,
// RoPE and cache write in one kernel with on-chip intermediates; LaCache (gist.science),
// Technical Summary, Methodology 1 -- only rows outside the invariant region are recomputed,
// RoPECache holds post-projection, post-RoPE states; Methodology 2 -- 1 x 128 FP8 groups.
//
// Reduction order (identical here and in the split-K path, for any M and tiling): each output
// element is (((0 + P0) + P1) + P2) + P3, where Pp is the chain of 16x16 MFMAs over the p-th
// quarter of H in ascending k, each MFMA taking k0..k0+31 (bf16) or k0..k0+3 (fp32) with lane
// group l/16 holding the slots k0 + 8(l/16) .. +7 (bf16) or k0 + l/16 (fp32).  A row's
// result is therefore independent of n and of the other rows: a step stores exactly what a
// refresh of all S rows would.
//
// Rotary pairing (i, i + D/2): every wave owns column tiles in pairs (c, c + D/2), so both
// members of a pair sit in the same lane and register of the MFMA accumulator and the
// rotation needs no data exchange.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

// Destination of output row m (= b * n + i, position pos) of head slot j; element type chosen
// by caller.
__device__ __forceinline__ size_t out_row_offset(const RefreshArgs& a, int m, int j, int pos, int& which) {
  const int b = seq_of_row(a.cu, a.B, a.n, m);
  if (j < a.Hq) {
    which = 0;
    return ((size_t)m * a.Hq + j) * (size_t)a.D;
  }
  const int g = (j < a.Hq + a.Hkv) ? j - a.Hq : j - a.Hq - a.Hkv;
  which = (j < a.Hq + a.Hkv) ? 1 : 2;
  return (((size_t)b * a.Hkv + g) * a.S + pos) * (size_t)a.D;
}

// Rotation frequencies (in turns, hi + lo) of the column pairs this lane rotates in the
// epilogue; formed before the main loop, so their fp64 arithmetic overlaps the first
// transfers instead of delaying the epilogue.
template <int D>
__device__ __forceinline__ void epilogue_turns(const RefreshArgs& a, float (&hi)[D / 64], float (&lo)[D / 64]) {
  const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
#pragma unroll
  for (int sb = 0; sb < D / 64; ++sb) rope_turns(wn * (D / 4) + sb * 16 + (lane & 15), D, a.rope_base, hi[sb], lo[sb]);
}

// Epilogue of a finished (TM rows) x (one head) tile held as per-wave accumulators tot:
// rotary embedding of Q and K heads in registers, the fp32 tile staged in LDS (smem, at least
// TM * (D + 4) floats, free when called), then whole rows out: bf16 / fp32 rows, or per-row
// FP8 codes with their scale.
// WM waves along the rows (2 * WM waves, 128 * WM threads); wave w owns rows
// (w / 2) * TM / WM + [0, TM / WM).
template <typename T, int KIND, int TM, int D, int WM>
__device__ __forceinline__ void tile_epilogue(const RefreshArgs& a,
                                              f32x4 (&tot)[TM / (16 * WM)][D / 32], char* smem,
                                              int j, int m0, const int (&colv)[D / 32],
                                              const float (&hi)[D / 64], const float (&lo)[D / 64]) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int RT = TM / (16 * WM), CT = D / 32, CH = CT / 2;
  constexpr int NT = 128 * WM;
  constexpr int EPI_STRIDE = D + 4;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  // Positions of the rows this lane rotates, and of the rows this thread stores: all loaded
  // together (clamped, unconditional), one round trip instead of one per row.
  constexpr int TPR = D / 8;                     // threads per stored row
  constexpr int SPT = TM / (NT / TPR);           // stored rows per thread
  int rpos[RT][4], spos[SPT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int v = 0; v < 4; ++v) rpos[rt][v] = a.idx[min(m0 + wm * (TM / WM) + rt * 16 + lg * 4 + v, a.M - 1)];
#pragma unroll
  for (int k = 0; k < SPT; ++k) spos[k] = a.idx[min(m0 + t / TPR + k * (NT / TPR), a.M - 1)];

  // Rotary embedding of Q and K heads, in registers.
  if (j < a.Hq + a.Hkv) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int pos = rpos[rt][v];
#pragma unroll
        for (int sb = 0; sb < CH; ++sb) {
          float s, c;
          rope_sincos(pos, hi[sb], lo[sb], s, c);
          float x = tot[rt][sb][v], y = tot[rt][CH + sb][v];
          rope_rotate(x, y, s, c);
          tot[rt][sb][v] = x;
          tot[rt][CH + sb][v] = y;
        }
      }
  }

  // Stage the fp32 tile in LDS (the loop's last barrier already retired the stage buffers).
  float* tile = (float*)smem;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        tile[(wm * (TM / WM) + rt * 16 + lg * 4 + v) * EPI_STRIDE + colv[ct]] = tot[rt][ct][v];
  __syncthreads();

  // Whole rows out: D/8 threads per row, eight values each.
  const int cpos = (t % TPR) * 8;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int r = t / TPR + k * (NT / TPR);
    const int m = m0 + r;
    if (m >= a.M) continue;  // uniform over the TPR threads of a row
    float x[8];
    const float4 x0 = *(const float4*)(tile + r * EPI_STRIDE + cpos);
    const float4 x1 = *(const float4*)(tile + r * EPI_STRIDE + cpos + 4);
    x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
    x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
    int which;
    const size_t off = out_row_offset(a, m, j, spos[k], which);
    if (which == 0 || KIND != kCacheFP8) {
      void* base = which == 0 ? a.q_out : which == 1 ? a.kc : a.vc;
      if constexpr (BF) {
        u32x4 o;
        o.x = pack_bf16x2(x[0], x[1]);
        o.y = pack_bf16x2(x[2], x[3]);
        o.z = pack_bf16x2(x[4], x[5]);
        o.w = pack_bf16x2(x[6], x[7]);
        *(u32x4*)((bf16_t*)base + off + cpos) = o;
      } else {
        float* dst = (float*)base + off + cpos;
        *(float4*)dst = x0;
        *(float4*)(dst + 4) = x1;
      }
    } else {
      // Per-row FP8: amax over the row (TPR consecutive lanes), scale = amax / 448.
      float am = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
#pragma unroll
      for (int msk = 1; msk < TPR; msk <<= 1) am = fmaxf(am, __shfl_xor(am, msk, kWave));
      const float scale = (am == 0.f) ? 1.f : am / 448.f;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo |= e4m3_encode(x[e] / scale) << (8 * e);
        hi |= e4m3_encode(x[4 + e] / scale) << (8 * e);
      }
      uint8_t* dst = (uint8_t*)(which == 1 ? a.kc : a.vc) + off + cpos;
      *(uint2*)dst = make_uint2(lo, hi);
      if ((t % TPR) == 0) (which == 1 ? a.ks : a.vs)[off / D] = scale;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Tiled kernel: one workgroup per (TM rows) x (one head = D columns), four waves as 2 (rows)
// x 2 (rotary-pair column groups).  A (gathered hidden rows) and W tiles go through LDS,
// double buffered, with chunk = c ^ (row % 8) swizzling.  The finished tile is rotated in
// registers, staged as fp32 in LDS and written as whole cache rows (16-byte stores, or per-row
// FP8 with its scale).
// ------------------------------------------------------------------------------------------
template <typename T, int KIND, int TM, int D, int BKC>
__global__ __launch_bounds__(256) void refresh_tiled(RefreshArgs a) {
  a.M = live_rows(a.cu, a.B, a.M);
  if ((int)blockIdx.y * TM >= a.M) return;       // row tiles past the packed rows present
  constexpr bool BF = sizeof(T) == 2;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int BK = BKC * EPC;              // elements of K per stage
  constexpr int RT = TM / 32;                // 16-row tiles per wave
  constexpr int CT = D / 32;                 // 16-column tiles per wave
  constexpr int CH = CT / 2;
  constexpr int A_PER_T = TM * BKC / 256;
  constexpr int W_PER_T = D * BKC / 256;
  static_assert(A_PER_T >= 1 && W_PER_T >= 1, "tile too small for 256 threads");
  constexpr int STAGE = (TM + D) * BKC * 16;
  constexpr int EPI_STRIDE = D + 4;
  constexpr int EPI = TM * EPI_STRIDE * 4;
  constexpr int SMEM = (2 * STAGE > EPI) ? 2 * STAGE : EPI;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int j = blockIdx.x;
  const int m0 = blockIdx.y * TM;

  const T* hid = (const T*)a.hidden;
  const T* w = (const T*)a.w;
  const int cchunk = t % BKC;

  // Global sources of this thread's chunks (fixed rows; k advances).
  const T* asrc[A_PER_T];
  bool aval[A_PER_T];
  int prow[A_PER_T];
#pragma unroll
  for (int u = 0; u < A_PER_T; ++u) prow[u] = a.idx[min(m0 + t / BKC + u * (256 / BKC), a.M - 1)];
#pragma unroll
  for (int u = 0; u < A_PER_T; ++u) {
    const int r = t / BKC + u * (256 / BKC);
    const int m = min(m0 + r, a.M - 1);
    aval[u] = m0 + r < a.M;
    asrc[u] = hid + ((size_t)seq_of_row(a.cu, a.B, a.n, m) * a.S + prow[u]) * a.H + cchunk * EPC;
  }
  const T* wsrc[W_PER_T];
#pragma unroll
  for (int u = 0; u < W_PER_T; ++u) {
    const int c = t / BKC + u * (256 / BKC);
    wsrc[u] = w + (size_t)(j * D + c) * a.H + cchunk * EPC;
  }

  // Stage loads and stores are written out as macros, not lambdas: a lambda capturing these
  // per-thread arrays by reference left them in scratch memory.
  u32x4 areg[A_PER_T], wreg[W_PER_T];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#define DLLM_LOAD_STAGE(k0)                                                   \
  do {                                                                        \
    _Pragma("unroll") for (int u = 0; u < A_PER_T; ++u) {                     \
      const u32x4 x_ = *(const u32x4*)(asrc[u] + (k0));                       \
      areg[u] = aval[u] ? x_ : zero;                                          \
    }                                                                         \
    _Pragma("unroll") for (int u = 0; u < W_PER_T; ++u)                       \
      wreg[u] = *(const u32x4*)(wsrc[u] + (k0));                              \
  } while (0)
#define DLLM_STORE_STAGE(buf)                                                 \
  do {                                                                        \
    char* A_ = smem + (buf) * STAGE;                                          \
    char* W_ = A_ + TM * BKC * 16;                                            \
    _Pragma("unroll") for (int u = 0; u < A_PER_T; ++u) {                     \
      const int r_ = t / BKC + u * (256 / BKC);                               \
      *(u32x4*)(A_ + (r_ * BKC + (cchunk ^ (r_ & (BKC - 1)))) * 16) = areg[u]; \
    }                                                                         \
    _Pragma("unroll") for (int u = 0; u < W_PER_T; ++u) {                     \
      const int c_ = t / BKC + u * (256 / BKC);                               \
      *(u32x4*)(W_ + (c_ * BKC + (cchunk ^ (c_ & (BKC - 1)))) * 16) = wreg[u]; \
    }                                                                         \
  } while (0)

  int colv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    colv[ct] = (ct / CH) * (D / 2) + wn * (D / 4) + (ct % CH) * 16 + l16;

  f32x4 acc[RT][CT], tot[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      tot[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int stages = a.H / BK;
  const int per_part = stages / kKSplit;
  DLLM_LOAD_STAGE(0);
  float hi[D / 64], lo[D / 64];
  epilogue_turns<D>(a, hi, lo);
  DLLM_STORE_STAGE(0);
  __syncthreads();
  for (int s = 0; s < stages; ++s) {
    if (s + 1 < stages) DLLM_LOAD_STAGE((s + 1) * BK);
    const char* A = smem + (s & 1) * STAGE;
    const char* W = A + TM * BKC * 16;
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < BKC / 4; ++ks) {
        const int c = ks * 4 + lg;
        bf16x8 af[RT], bfr[CT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int r = wm * (TM / 2) + rt * 16 + l16;
          af[rt] = as_bf16x8(*(const u32x4*)(A + (r * BKC + (c ^ (r & (BKC - 1)))) * 16));
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int col = colv[ct];
          bfr[ct] = as_bf16x8(*(const u32x4*)(W + (col * BKC + (c ^ (col & (BKC - 1)))) * 16));
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = mfma_bf16(af[rt], bfr[ct], acc[rt][ct]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BKC; ++ks) {  // four fp32 k per chunk = one MFMA step
        float af[RT], bfr[CT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int r = wm * (TM / 2) + rt * 16 + l16;
          af[rt] = *(const float*)(A + (r * BKC + (ks ^ (r & (BKC - 1)))) * 16 + lg * 4);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int col = colv[ct];
          bfr[ct] = *(const float*)(W + (col * BKC + (ks ^ (col & (BKC - 1)))) * 16 + lg * 4);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = mfma_f32(af[rt], bfr[ct], acc[rt][ct]);
      }
    }
    if ((s + 1) % per_part == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          tot[rt][ct] = tot[rt][ct] + acc[rt][ct];
          acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (s + 1 < stages) DLLM_STORE_STAGE((s + 1) & 1);
    __syncthreads();
  }

  tile_epilogue<T, KIND, TM, D, 2>(a, tot, smem, j, m0, colv, hi, lo);
}

// ------------------------------------------------------------------------------------------
// Pipelined bf16 kernel (large M): the same tile, partitioning and epilogue as refresh_tiled,
// with the A (gathered rows) and W tiles moved global -> LDS by DMA through an NST-stage
// ring, so NST - 1 stages are in flight while one is multiplied.  Each lane fetches the
// source chunk that lands, swizzled (chunk c of row r at slot c ^ (r % BKC)), at its LDS
// slot.  A barrier per stage; each wave waits only for its own transfers of the stage it is
// about to read.  SB: the hidden states and W both span less than 4 GB, so each transfer
// takes a wave-uniform base (advanced per stage in scalar registers) and a fixed 32-bit
// per-lane offset, and costs no vector address arithmetic.  The stage loop is unrolled by the
// ring depth, so every LDS slot address is a constant offset.
// ------------------------------------------------------------------------------------------
template <int KIND, int TM, int D, int BKC, int NST, int WM, bool SB>
__global__ __launch_bounds__(128 * WM) void refresh_gemm(RefreshArgs a) {
  a.M = live_rows(a.cu, a.B, a.M);
  if ((int)blockIdx.y * TM >= a.M) return;       // row tiles past the packed rows present
  constexpr int NW = 2 * WM;                 // waves: WM along the rows x 2 column groups
  constexpr int EPC = 8;                     // bf16 per 16-byte chunk
  constexpr int BK = BKC * EPC;              // k per stage
  constexpr int RT = TM / (16 * WM), CT = D / 32, CH = CT / 2;
  constexpr int RPI = 64 / BKC;              // rows (or columns) per DMA instruction
  constexpr int IA = TM / RPI, IW = D / RPI; // DMA instructions per stage for A and W
  constexpr int NI = (IA + IW) / NW;         // per wave
  static_assert((IA + IW) % NW == 0, "DMA instructions must split evenly over the waves");
  constexpr int A_BYTES = TM * BKC * 16;
  constexpr int STAGE = (TM + D) * BKC * 16;
  constexpr int EPI = TM * (D + 4) * 4;
  constexpr int SMEM = (NST * STAGE > EPI) ? NST * STAGE : EPI;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int j = blockIdx.x;
  const int m0 = blockIdx.y * TM;

  // Source of this lane's chunk for each of the wave's NI DMA instructions (k = 0).  The row
  // positions are loaded for every instruction (clamped, unconditional) before any address is
  // formed, so they cost one round trip.
  const bf16_t* src[NI];
  uint32_t voff[NI];                             // SB: byte offset from hidden (A) or w (W)
  int mrow[NI], prow[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int r = min((wave * NI + i) * RPI + lane / BKC, TM - 1);
    mrow[i] = min(m0 + r, a.M - 1);              // rows past M: never stored
    prow[i] = a.idx[mrow[i]];
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int gi = wave * NI + i;
    const int cp = lane % BKC;
    size_t e;                                    // element offset of the chunk
    if (gi < IA) {
      const int r = gi * RPI + lane / BKC;
      const size_t hrow = (size_t)seq_of_row(a.cu, a.B, a.n, mrow[i]) * a.S + prow[i];
      e = hrow * a.H + (cp ^ (r & (BKC - 1))) * EPC;
      src[i] = (const bf16_t*)a.hidden + e;
    } else {
      const int c = (gi - IA) * RPI + lane / BKC;
      e = (size_t)(j * D + c) * a.H + (cp ^ (c & (BKC - 1))) * EPC;
      src[i] = (const bf16_t*)a.w + e;
    }
    voff[i] = (uint32_t)(e * sizeof(bf16_t));
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds_w = lds_addr(smem) + (uint32_t)(wave_u * NI * 1024);   // this wave's blocks
  auto issue = [&](int stage, int slot) {
    if constexpr (SB) {
      const char* hb = (const char*)a.hidden + (size_t)stage * BK * sizeof(bf16_t);
      const char* wb = (const char*)a.w + (size_t)stage * BK * sizeof(bf16_t);
#pragma unroll
      for (int i = 0; i < NI; ++i)
        dma_16B_sbase(voff[i], (wave_u * NI + i < IA) ? hb : wb, lds_w + (uint32_t)(slot * STAGE + i * 1024));
    } else {
      char* base = smem + slot * STAGE;
#pragma unroll
      for (int i = 0; i < NI; ++i) dma_16B(src[i] + stage * BK, base + (wave * NI + i) * 1024);
    }
  };

  int colv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
    colv[ct] = (ct / CH) * (D / 2) + wn * (D / 4) + (ct % CH) * 16 + l16;

  f32x4 acc[RT][CT], tot[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      tot[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int stages = a.H / BK;
  const int per_part = stages / kKSplit;
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < stages) issue(st, st);
  float hi[D / 64], lo[D / 64];
  epilogue_turns<D>(a, hi, lo);
  for (int s0 = 0; s0 < stages; s0 += NST) {
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int s = s0 + u;                        // s % NST == u
    if (s >= stages) break;
    // this wave's transfers for stage s are done once at most those of the later stages
    // already issued (min(NST - 2, stages - 1 - s) of them) are outstanding
    if (s + NST - 2 < stages) DLLM_WAIT_VMCNT(NI * (NST - 2));
    else DLLM_WAIT_VMCNT(0);
    lds_barrier();
    if (s + NST - 1 < stages) issue(s + NST - 1, (u + NST - 1) % NST);
    const char* A = smem + u * STAGE;
    const char* W = A + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BKC / 4; ++ks) {
      const int c = ks * 4 + lg;
      bf16x8 af[RT], bfr[CT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = wm * (TM / WM) + rt * 16 + l16;
        af[rt] = as_bf16x8(*(const u32x4*)(A + (r * BKC + (c ^ (r & (BKC - 1)))) * 16));
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = colv[ct];
        bfr[ct] = as_bf16x8(*(const u32x4*)(W + (col * BKC + (c ^ (col & (BKC - 1)))) * 16));
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = mfma_bf16(af[rt], bfr[ct], acc[rt][ct]);
    }
    if ((s + 1) % per_part == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          tot[rt][ct] = tot[rt][ct] + acc[rt][ct];
          acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
  }
  lds_barrier();  // every wave is done reading the ring before the epilogue reuses it
  tile_epilogue<bf16_t, KIND, TM, D, WM>(a, tot, smem, j, m0, colv, hi, lo);
}

template <int KIND, int TM, int D, int BKC, int NST, int WM>
hipError_t launch_gemm(const RefreshArgs& a, hipStream_t s) {
  const int heads = a.Hq + 2 * a.Hkv;
  dim3 grid(heads, (a.M + TM - 1) / TM);
  // 32-bit per-lane offsets reach every chunk when both operands span less than 4 GB
  // (the DLLM_OPT_WIDE_OFFSETS option takes the 64-bit form regardless, so it can be tested).
  const uint64_t hid_bytes = (uint64_t)a.B * a.S * a.H * sizeof(bf16_t);
  const uint64_t w_bytes = (uint64_t)heads * D * a.H * sizeof(bf16_t);
  const bool wide = (options() & DLLM_OPT_WIDE_OFFSETS) != 0;
  if (hid_bytes < (1ull << 32) && w_bytes < (1ull << 32) && !wide)
    refresh_gemm<KIND, TM, D, BKC, NST, WM, true><<<grid, 128 * WM, 0, s>>>(a);
  else
    refresh_gemm<KIND, TM, D, BKC, NST, WM, false><<<grid, 128 * WM, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int KIND, int D, int BKC>
hipError_t launch_tiled(const RefreshArgs& a, hipStream_t s) {
  dim3 grid(a.Hq + 2 * a.Hkv, (a.M + 63) / 64);
  refresh_tiled<T, KIND, 64, D, BKC><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const RefreshArgs& a, hipStream_t s) {
  // H is a multiple of 256 (checked at the boundary), so each of the four partitions holds
  // whole 64-wide k stages (32-wide for fp32).
  if ((a.H / kKSplit) % 64) return hipErrorInvalidValue;
  if (a.act == DLLM_F32) return launch_tiled<float, kCacheF32, D, 8>(a, s);
  // 128 rows x one head per workgroup, eight waves of 32 rows x half the head's column pairs.
  // Small M streams W at the HBM rate and wants a third stage in flight; large M wants the
  // occupancy of two stages.
  // At most 256 rows (two row tiles, fewer workgroups than compute units, one per CU) run
  // sixteen waves of 16 rows for D = 128: the extra waves hide the stage latency (49.2 against
  // 50.2 us on a 256-row, 4096-hidden step); with more rows two 8-wave workgroups share a CU.
  const bool deep = a.M <= 512;
  const bool wide = D == 128 && a.M <= 256;
  constexpr int WW = D == 128 ? 8 : 4;
  if (a.kind == kCacheFP8) {
    if (wide) return launch_gemm<kCacheFP8, 128, D, 8, 3, WW>(a, s);
    return deep ? launch_gemm<kCacheFP8, 128, D, 8, 3, 4>(a, s) : launch_gemm<kCacheFP8, 128, D, 8, 2, 4>(a, s);
  }
  if (wide) return launch_gemm<kCacheBF16, 128, D, 8, 3, WW>(a, s);
  return deep ? launch_gemm<kCacheBF16, 128, D, 8, 3, 4>(a, s) : launch_gemm<kCacheBF16, 128, D, 8, 2, 4>(a, s);
}

}  // namespace

bool refresh_uses_splitk(int act, int M, int H) {
  return act == DLLM_BF16 && M <= kSplitKMaxRows && H <= kSplitKMaxHidden;
}

size_t refresh_workspace_bytes(int act, int M, int N, int H) {
  return refresh_uses_splitk(act, M, H) ? splitk_workspace_bytes(M, N) : 0;
}

hipError_t launch_refresh(const RefreshArgs& a, hipStream_t s) {
  if (refresh_uses_splitk(a.act, a.M, a.H)) return launch_refresh_splitk(a, a.ws, s);
  if (a.D == 128) return launch_d<128>(a, s);
  return launch_d<64>(a, s);
}

}  // namespace dllm
