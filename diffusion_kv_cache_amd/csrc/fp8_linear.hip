// Per-group FP8 linear layer on the gfx950 FP8 matrix cores (LaCache Technical Summary,
// Methodology 2: 1 x 128 groups for activations, 128 x 128 blocks for weights):
//   fp8_quant_groups  activations [M, K] bf16 -> e4m3 codes and one fp32 scale per row and
//                     128-column group (scale = amax / 448, code = e4m3(x / scale))
//   fp8_quant_blocks  weights [N, K] bf16 -> codes and one scale per 128 x 128 block
//   fp8_gemm          y[m, n] = sum_kb sx[m, kb] sw[n / 128, kb] sum_{k in kb} qx[m, k] qw[n, k]
//                     One 16x16x128 MFMA covers exactly one 128-group of k, so each group's
//                     product leaves the matrix core unscaled and is scaled and added in fp32
//                     (tot = part * (sx sw) + tot), groups in ascending order.  The MFMA forms
//                     the transposed tile (weight rows as its A operand): a lane then holds one
//                     activation row and four consecutive output columns, so it needs one row
//                     scale per 16-row tile and stores its columns with one vector store.
//   fp8_splitk_reduce the fixed split-K form: partial sums of contiguous group ranges added in
//                     split order.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kGroup = 128;
constexpr int kUnitScale = 0x7f7f7f7f;           // E8M0 127 = 2^0 in every byte

// D(16x16 fp32) = A(16x128 e4m3) B(128x16 e4m3).  Lane l supplies 32 codes of A row l%16 and
// of B column l%16 for k slot group l/16; both operands use the same slot -> k assignment, so
// the sum runs over every k once whatever that assignment is.
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, kUnitScale, 0,
                                                          kUnitScale);
}

// Eight e4m3 codes of x / scale (fp32 quotient), packed low byte first.
__device__ __forceinline__ uint2 encode8(const u32x4& v, float scale) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w = v[e >> 1];
    const float x0 = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    lo |= e4m3_encode(x0 / scale) << (8 * e);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w = v[2 + (e >> 1)];
    const float x1 = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    hi |= e4m3_encode(x1 / scale) << (8 * e);
  }
  return make_uint2(lo, hi);
}

__device__ __forceinline__ float amax8(const u32x4& v) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t w = v[e >> 1];
    m = fmaxf(m, fabsf(__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16))));
  }
  return m;
}

// One 128-value group per 16 lanes (eight values each); 16 groups per workgroup.  Groups of
// padding rows (m in [M, Mp)) get scale 0 and no codes.  Scales are stored group-major:
// sT[kb * Mp + m].
__global__ __launch_bounds__(256) void fp8_quant_groups(const bf16_t* x, int M, int K, int Mp,
                                                        uint8_t* q, float* sT) {
  const int G = K / kGroup;
  const long long gid = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (gid >= (long long)Mp * G) return;          // uniform over the 16 lanes of a group
  const int m = (int)(gid / G), kb = (int)(gid % G);
  if (m >= M) {
    if (l == 0) sT[(size_t)kb * Mp + m] = 0.f;
    return;
  }
  const size_t off = (size_t)m * K + (size_t)kb * kGroup + l * 8;
  const u32x4 v = *(const u32x4*)(x + off);
  float am = amax8(v);
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) am = fmaxf(am, __shfl_xor(am, s, kWave));
  const float scale = am == 0.f ? 1.f : am / 448.f;
  *(uint2*)(q + off) = encode8(v, scale);
  if (l == 0) sT[(size_t)kb * Mp + m] = scale;
}

// One workgroup per 128 x 128 block: each thread eight chunks of eight values.
__global__ __launch_bounds__(256) void fp8_quant_blocks(const bf16_t* w, int N, int K, uint8_t* q,
                                                        float* s) {
  __shared__ float red[4];
  const int KB = K / kGroup;
  const int nb = blockIdx.x / KB, kb = blockIdx.x % KB;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  u32x4 v[8];
  float am = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = u * 256 + t;                   // chunk id in the block: row c / 16, col chunk c % 16
    const size_t off = (size_t)(nb * kGroup + c / 16) * K + (size_t)kb * kGroup + (c % 16) * 8;
    v[u] = *(const u32x4*)(w + off);
    am = fmaxf(am, amax8(v[u]));
  }
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) am = fmaxf(am, __shfl_xor(am, sh, kWave));
  if (lane == 0) red[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = am == 0.f ? 1.f : am / 448.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = u * 256 + t;
    const size_t off = (size_t)(nb * kGroup + c / 16) * K + (size_t)kb * kGroup + (c % 16) * 8;
    *(uint2*)(q + off) = encode8(v[u], scale);
  }
  if (t == 0) s[(size_t)nb * KB + kb] = scale;
}

// ------------------------------------------------------------------------------------------
// GEMM: workgroup tile TM x TN, WM x WN waves of (TM / WM) x (TN / WN).  Each stage is one
// 128-group of k: the A rows (codes), the B rows (codes) and the stage's row scales move
// global -> LDS by DMA through an NST-stage ring; chunk j of a 128-byte row r sits at slot
// j ^ (r % 8).
// ------------------------------------------------------------------------------------------
template <int TM, int TN, int WM, int WN, int NST>
__global__ __launch_bounds__(64 * WM * WN) void fp8_gemm(Fp8GemmArgs a) {
  constexpr int NW = WM * WN;
  constexpr int RT = TM / WM / 16, CT = TN / WN / 16;
  constexpr int A_BYTES = TM * kGroup, B_BYTES = TN * kGroup, S_BYTES = 1024;
  constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  constexpr int IA = A_BYTES / 1024, IB = B_BYTES / 1024;
  static_assert((IA + IB) % NW == 0, "DMA blocks must split evenly over the waves");
  static_assert(TM <= 256 && TN <= kGroup && kGroup % TN == 0, "tile shape");
  constexpr int NI = (IA + IB) / NW;             // A / B blocks per wave and stage
  constexpr int PEND = NI + 1;                   // + the scale block (every wave issues it)
  __shared__ __attribute__((aligned(16))) char smem[NST * STAGE];
  __shared__ float s_sw[kFp8MaxGroups];          // this column block's weight scales

  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;
  // All row tiles (and k ranges) of one column tile run on one XCD, back to back: the weight
  // tile is fetched into that L2 once and the concurrent column tiles share the row tiles.
  const int nN = (a.N + TN - 1) / TN, nM = (a.M + TM - 1) / TM;
  int nt, unit;
  xcd_group_unit(blockIdx.x, nN, nM * a.splits, nt, unit);
  const int mt = unit % nM, split = unit / nM;
  const int n0 = nt * TN, m0 = mt * TM;
  const int KB = a.K / kGroup;
  const int kb0 = split * a.kb_per_split;
  const int kb1 = min(KB, kb0 + a.kb_per_split);
  const int stages = kb1 - kb0;

  // Per-lane byte offsets of this wave's DMA blocks (k = 0), fixed over the stages.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int gi = wave_u * NI + i;
    const bool isa = gi < IA;
    const int r = (isa ? gi : gi - IA) * 8 + lane / 8, c = lane % 8;
    const int row = isa ? min(m0 + r, a.M - 1) : min(n0 + r, a.N - 1);
    voff[i] = (uint32_t)((size_t)row * a.K + ((c ^ (r & 7)) << 4));
  }
  // scale block: lane l fetches rows m0 + 4 l .. + 3 of the stage's group (clamped inside Mp)
  const uint32_t soff = (uint32_t)(min(m0 + 4 * lane, a.Mp - 4) * 4);
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int kb, int slot) {
    const uint32_t st = lds0 + (uint32_t)(slot * STAGE);
    const char* ab = (const char*)a.xq + (size_t)kb * kGroup;
    const char* bb = (const char*)a.wq + (size_t)kb * kGroup;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int gi = wave_u * NI + i;
      dma_16B_sbase(voff[i], gi < IA ? ab : bb,
                    st + (uint32_t)(gi < IA ? gi * 1024 : A_BYTES + (gi - IA) * 1024));
    }
    dma_16B_sbase(soff, (const char*)(a.sxT + (size_t)kb * a.Mp), st + A_BYTES + B_BYTES);
  };

  f32x4 tot[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) tot[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The weight scales of the block's groups go to LDS first (ordinary loads, complete before
  // the ring starts), so the loop reads them without waiting on the memory counter that the
  // ring's transfers also count.
  const float* swp = a.sw + (size_t)(n0 / kGroup) * KB + kb0;
  for (int i = t; i < stages; i += 64 * NW) s_sw[i] = swp[i];
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < stages) issue(kb0 + s, s);
  for (int s0 = 0; s0 < stages; s0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int s = s0 + u;
      if (s >= stages) break;
      if (s + NST - 2 < stages) DLLM_WAIT_VMCNT(PEND * (NST - 2));
      else DLLM_WAIT_VMCNT(0);
      lds_barrier();
      if (s + NST - 1 < stages) issue(kb0 + s + NST - 1, (u + NST - 1) % NST);
      const char* A = smem + u * STAGE;
      const char* Bt = A + A_BYTES;
      const float* Sx = (const float*)(Bt + B_BYTES);
      const float swv = s_sw[s];
      i32x8 af[RT], bfr[CT];
      float sr[RT];                              // scale of this lane's row in each row tile
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = wm * (TM / WM) + rt * 16 + l16;
        const u32x4 lo = *(const u32x4*)(A + r * kGroup + (((2 * lg) ^ (r & 7)) << 4));
        const u32x4 hi = *(const u32x4*)(A + r * kGroup + (((2 * lg + 1) ^ (r & 7)) << 4));
        af[rt] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sr[rt] = Sx[r] * swv;
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int r = wn * (TN / WN) + ct * 16 + l16;
        const u32x4 lo = *(const u32x4*)(Bt + r * kGroup + (((2 * lg) ^ (r & 7)) << 4));
        const u32x4 hi = *(const u32x4*)(Bt + r * kGroup + (((2 * lg + 1) ^ (r & 7)) << 4));
        bfr[ct] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      // Every product of the group first (independent MFMAs back to back, each into its own
      // registers), then the scaled adds: no add waits on the MFMA issued just before it.
      // p[rt][ct][v]: activation row rt * 16 + l16, weight row (output column) ct * 16 + 4 lg + v.
      f32x4 p[RT][CT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) p[rt][ct] = mfma_fp8(bfr[ct], af[rt]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v) tot[rt][ct][v] = fmaf(p[rt][ct][v], sr[rt], tot[rt][ct][v]);
    }
  }

  // Out: bf16 y (one split) or the fp32 partial of this split, four consecutive columns per
  // store (N is a multiple of 128, y 8-byte and the partials 16-byte aligned).
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int m = m0 + wm * (TM / WM) + rt * 16 + l16;
    if (m >= a.M) continue;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int n = n0 + wn * (TN / WN) + ct * 16 + lg * 4;
      if (n >= a.N) continue;
      if (a.part) {
        *(f32x4*)(a.part + ((size_t)split * a.M + m) * a.N + n) = tot[rt][ct];
      } else {
        uint2 o;
        o.x = pack_bf16x2(tot[rt][ct][0], tot[rt][ct][1]);
        o.y = pack_bf16x2(tot[rt][ct][2], tot[rt][ct][3]);
        *(uint2*)((bf16_t*)a.y + (size_t)m * a.N + n) = o;
      }
    }
  }
}

// y = bf16(((P0 + P1) + ...) + P_{splits-1}), four columns per thread.
__global__ __launch_bounds__(256) void fp8_splitk_reduce(const float* part, int splits, long long MN,
                                                         bf16_t* y) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4 s = *(const f32x4*)(part + i);
  for (int p = 1; p < splits; ++p) s = s + *(const f32x4*)(part + (size_t)p * MN + i);
  uint2 o;
  o.x = pack_bf16x2(s.x, s.y);
  o.y = pack_bf16x2(s.z, s.w);
  *(uint2*)(y + i) = o;
}

template <int TM, int TN, int WM, int WN, int NST>
hipError_t launch_cfg(const Fp8GemmArgs& a, int splits, hipStream_t s) {
  const long long grid = (long long)((a.N + TN - 1) / TN) * ((a.M + TM - 1) / TM) * splits;
  fp8_gemm<TM, TN, WM, WN, NST><<<(unsigned)grid, 64 * WM * WN, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

Fp8Plan plan_fp8_linear(int M, int N, int K) {
  Fp8Plan p{};
  p.tile = M <= 64 ? 0 : M <= 256 ? 1 : 2;
  const int TM = p.tile == 0 ? 64 : p.tile == 1 ? 128 : 256, TN = p.tile == 0 ? 64 : 128;
  p.Mp = (M + 255) / 256 * 256;
  const int KB = K / kGroup;
  const long long tiles = (long long)((N + TN - 1) / TN) * ((M + TM - 1) / TM);
  // enough workgroups to keep every CU streaming: split k into contiguous group ranges
  int splits = (int)std::min<long long>(KB, std::max<long long>(1, (512 + tiles - 1) / tiles));
  p.kb_per_split = (KB + splits - 1) / splits;
  p.splits = (KB + p.kb_per_split - 1) / p.kb_per_split;
  p.part_bytes = p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
  p.codes_bytes = (size_t)M * K;
  p.scales_bytes = (size_t)KB * p.Mp * sizeof(float);
  return p;
}

hipError_t launch_fp8_quant_groups(const void* x, int M, int K, int Mp, uint8_t* q, float* sT,
                                   bool zero_pad, hipStream_t s) {
  // Without zero_pad the scales of rows M .. Mp - 1 are left as they are: the GEMM reads them
  // only for rows it never stores.
  const long long groups = (long long)(zero_pad ? Mp : M) * (K / kGroup);
  fp8_quant_groups<<<(unsigned)((groups + 15) / 16), 256, 0, s>>>((const bf16_t*)x, M, K, Mp, q, sT);
  return hipGetLastError();
}

hipError_t launch_fp8_quant_blocks(const void* w, int N, int K, uint8_t* q, float* sc,
                                   hipStream_t s) {
  fp8_quant_blocks<<<(unsigned)((N / kGroup) * (K / kGroup)), 256, 0, s>>>((const bf16_t*)w, N, K, q, sc);
  return hipGetLastError();
}

hipError_t launch_fp8_gemm(const Fp8GemmArgs& a, const Fp8Plan& p, hipStream_t s) {
  hipError_t e = p.tile == 0 ? launch_cfg<64, 64, 2, 2, 6>(a, p.splits, s)
                 : p.tile == 1 ? launch_cfg<128, 128, 2, 2, 4>(a, p.splits, s)
                               : launch_cfg<256, 128, 4, 2, 3>(a, p.splits, s);
  if (e != hipSuccess || p.splits == 1) return e;
  const long long MN = (long long)a.M * a.N;
  fp8_splitk_reduce<<<(unsigned)((MN / 4 + 255) / 256), 256, 0, s>>>(a.part, p.splits, MN, (bf16_t*)a.y);
  return hipGetLastError();
}

}  // namespace dllm
