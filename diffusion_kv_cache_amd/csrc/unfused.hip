// The unfused form of the refresh, for comparison with the fused kernels (Flash-dLLM news
// summary, memory paragraph: the projection, the rotary embedding and the cache write as
// separate kernels, each a round trip through HBM).  With the gather and the projection done
// by any GEMM into y [M, ld] (columns Q heads | K heads | V heads):
//   rope_rows        rotates the Q and K head columns of y in place at each row's position;
//   scatter_kv_rows  copies each row's K and V head columns into the flat cache at
//                    (b, g, position), 16-byte chunks, every other cache row untouched.
// Also the attainable matrix-core rate and read-stream rate microbenchmarks of the roofline
// report (mfma_probe, read_probe).
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

// One thread per rotary pair (row m, head j, pair i): (x_i, x_{i + D/2}) of y[m, j*D ...].
__global__ __launch_bounds__(256) void rope_rows(bf16_t* y, int M, int ld, int heads, int D,
                                                 const int32_t* pos, double base) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const int half = D / 2;
  const long long total = (long long)M * heads * half;
  if (t >= total) return;
  const int i = (int)(t % half);
  const long long rh = t / half;
  const int j = (int)(rh % heads), m = (int)(rh / heads);
  bf16_t* row = y + (size_t)m * ld + (size_t)j * D;
  float x = bf16_to_f32(row[i]), z = bf16_to_f32(row[i + half]);
  float hi, lo, s, c;
  rope_turns(i, D, base, hi, lo);
  rope_sincos(pos[m], hi, lo, s, c);
  rope_rotate(x, z, s, c);
  row[i] = f32_to_bf16(x);
  row[i + half] = f32_to_bf16(z);
}

// One thread per 16-byte chunk of a K or V row: chunk c of (row m, KV head g, part).
__global__ __launch_bounds__(256) void scatter_kv_rows(const bf16_t* y, int ld, int k_col, int v_col,
                                                       bf16_t* kc, bf16_t* vc, int n, int Hkv,
                                                       int S, int D, const int32_t* idx, int M) {
  const int cpr = D / 8;                         // chunks per row
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)M * Hkv * 2 * cpr;
  if (t >= total) return;
  const int c = (int)(t % cpr);
  long long r = t / cpr;
  const int part = (int)(r % 2);
  r /= 2;
  const int g = (int)(r % Hkv), m = (int)(r / Hkv);
  const int b = m / n, p = idx[m];
  const u32x4 v = *(const u32x4*)(y + (size_t)m * ld + (part ? v_col : k_col) + (size_t)g * D + c * 8);
  bf16_t* dst = (part ? vc : kc) + (((size_t)b * Hkv + g) * S + p) * D + c * 8;
  *(u32x4*)dst = v;
}

}  // namespace

hipError_t launch_rope_rows(void* y, int M, int ld, int heads, int D, const int32_t* pos,
                            double base, hipStream_t s) {
  const long long total = (long long)M * heads * (D / 2);
  if (total == 0) return hipSuccess;
  rope_rows<<<(unsigned)((total + 255) / 256), 256, 0, s>>>((bf16_t*)y, M, ld, heads, D, pos, base);
  return hipGetLastError();
}

hipError_t launch_scatter_kv_rows(const void* y, int ld, int k_col, int v_col, void* kc, void* vc,
                                  int B, int n, int Hkv, int S, int D, const int32_t* idx,
                                  hipStream_t s) {
  const int M = B * n;
  const long long total = (long long)M * Hkv * 2 * (D / 8);
  if (total == 0) return hipSuccess;
  scatter_kv_rows<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
      (const bf16_t*)y, ld, k_col, v_col, (bf16_t*)kc, (bf16_t*)vc, n, Hkv, S, D, idx, M);
  return hipGetLastError();
}

}  // namespace dllm

// ------------------------------------------------------------------------------------------
// Attainable matrix-core rate: every wave chains `iters` rounds of independent MFMAs on
// register operands (no memory traffic in the loop): eight 16 x 16 chains (bf16 K = 32, FP8
// K = 128) or four 32 x 32 chains (bf16 K = 16, FP8 K = 64); one value per wave is stored so
// the work is kept.
// ------------------------------------------------------------------------------------------
namespace dllm {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_probe;

typedef __attribute__((ext_vector_type(16))) float f32x16_probe;

// BIG: 32 x 32 output tiles (bf16 K = 16, FP8 K = 64) instead of 16 x 16 (K = 32, 128).
template <int KIND, bool BIG>
__global__ __launch_bounds__(256) void mfma_probe(int iters, float* out) {
  const int t = threadIdx.x;
  const uint32_t s = 0x3c003c00u ^ (uint32_t)(t & 7);
  float sum = 0.f;
  if constexpr (KIND == kCacheFP8) {
    const i32x8_probe a = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                           0x38383838, 0x38383838, 0x38383838, 0x38383838};
    if constexpr (BIG) {
      f32x16_probe acc[4] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, acc[c], 0, 0, 0, 0x7f7f7f7f,
                                                                  0, 0x7f7f7f7f);
#pragma unroll
      for (int c = 0; c < 4; ++c) sum += acc[c][0];
    } else {
      f32x4 acc[8] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < 8; ++c)
          acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, acc[c], 0, 0, 0, 0x7f7f7f7f,
                                                                   0, 0x7f7f7f7f);
#pragma unroll
      for (int c = 0; c < 8; ++c) sum += acc[c][0];
    }
  } else {
    const u32x4 av = {s, s, s, s};
    const bf16x8 a = as_bf16x8(av);
    if constexpr (BIG) {
      f32x16_probe acc[4] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) sum += acc[c][0];
    } else {
      f32x4 acc[8] = {};
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = mfma_bf16(a, a, acc[c]);
#pragma unroll
      for (int c = 0; c < 8; ++c) sum += acc[c][0];
    }
  }
  if ((t & 63) == 0) out[blockIdx.x * 4 + (t >> 6)] = sum;
}

// Read-only stream: workgroups stride over the buffer in 16 KB steps (each thread four 16-byte
// loads 4 KB apart, all issued before they are combined), XOR-folding every 32-bit word;
// each workgroup writes the fold of the words it read.
__global__ __launch_bounds__(256) void read_probe(const u32x4* __restrict__ p, size_t n, uint32_t* out) {
  const int t = threadIdx.x;
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * 1024;
  for (size_t i = (size_t)blockIdx.x * 1024 + t; i < n; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (i + u * 256 < n) ? p[i + u * 256] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m, kWave);
  __shared__ uint32_t w[4];
  if ((t & 63) == 0) w[t >> 6] = x;
  __syncthreads();
  if (t == 0) out[blockIdx.x] = (w[0] ^ w[1]) ^ (w[2] ^ w[3]);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, int workgroups, uint32_t* out, hipStream_t s) {
  read_probe<<<workgroups, 256, 0, s>>>((const u32x4*)buf, bytes / 16, out);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int kind, int big, int workgroups, int iters, float* out, hipStream_t s) {
  if (kind == kCacheFP8) {
    if (big) mfma_probe<kCacheFP8, true><<<workgroups, 256, 0, s>>>(iters, out);
    else mfma_probe<kCacheFP8, false><<<workgroups, 256, 0, s>>>(iters, out);
  } else {
    if (big) mfma_probe<kCacheBF16, true><<<workgroups, 256, 0, s>>>(iters, out);
    else mfma_probe<kCacheBF16, false><<<workgroups, 256, 0, s>>>(iters, out);
  }
  return hipGetLastError();
}

}  // namespace dllm
