// Device-side helpers shared by the gfx950 kernels of the cached denoising step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dllm_cache.h"

namespace dllm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
// 16 bytes as a native vector: arrays of these stay in registers (arrays of HIP's uint4,
// a union-based struct, were left in scratch memory by the compiler).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef uint16_t bf16_t;  // raw bf16 bits in memory

constexpr int kWave = 64;
// Fixed number of K-partitions of the projection: every output element is
// (((0 + P0) + P1) + P2) + P3, each Pp an MFMA chain over its partition in ascending k.
constexpr int kKSplit = 4;

enum CacheKind : int { kCacheF32 = DLLM_F32, kCacheBF16 = DLLM_BF16, kCacheFP8 = DLLM_FP8_E4M3 };

// ------------------------------------------------------------------------ conversions ---

// fp32 -> bf16 bits, round to nearest even (NaN stays a NaN): the hardware conversion
// (v_cvt_pk_bf16_f32), branch-free.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two fp32 values -> packed bf16 pair (lo in bits 0..15), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> OCP E4M3 ("fn") code: round to nearest even, saturate to +-448, NaN -> 0x7f|sign.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;            // |x| >= 448 (incl. inf)
  if (a >= 0x3c800000u) {                               // |x| >= 2^-6: normal range
    uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;  // keep 3 mantissa bits, RNE
    uint32_t code = r - (120u << 3);                    // rebias exponent 127 -> 7
    return sign | (code > 0x7eu ? 0x7eu : code);
  }
  float m = rintf(__uint_as_float(a) * 512.0f);         // subnormal: m * 2^-9, m in 0..8
  return sign | (uint32_t)m;
}

// Four E4M3 codes (one 32-bit word, byte 0 first) -> four bf16 values (exact: every E4M3
// value is a bf16 value), via the hardware packed conversion with unit scale.
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  lo = __builtin_bit_cast(uint32_t, a);
  hi = __builtin_bit_cast(uint32_t, b);
}

// Eight E4M3 codes (two words) -> eight bf16 values packed in 16 bytes.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  uint32_t a, b, c, d;
  e4m3x4_to_bf16x4(w0, a, b);
  e4m3x4_to_bf16x4(w1, c, d);
  return u32x4{a, b, c, d};
}

// --------------------------------------------------------------------------- MFMA -------

// D(16x16, fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l supplies A row l%16 and B column
// l%16, eight K values each (slot group l/16); it receives D rows 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Same shape with K = 4 in fp32: lane l supplies A[l%16][l/16] and B[l/16][l%16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------------ LDS staging -------

// Workgroup barrier for data exchanged through LDS only: this wave's LDS operations are
// complete (lgkmcnt 0), but vector-memory loads still in flight stay in flight (the release
// fence of __syncthreads would wait for them too).  Callers wait for LDS-DMA transfers
// explicitly.  The empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same wait without the barrier, for LDS that only the issuing wave reads and writes: its
// LDS reads have completed (so a transfer may overwrite what they read).
__device__ __forceinline__ void lds_wave_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0 << 8) | (7 << 4) | 15 | (3 << 14));
  asm volatile("" ::: "memory");
}

// s_waitcnt with only the vector-memory count set (N outstanding allowed, 0..63).
#define DLLM_WAIT_VMCNT(N) \
  __builtin_amdgcn_s_waitcnt(((N) & 15) | (7 << 4) | (15 << 8) | (((N) >> 4) << 14))

// One LDS-DMA instruction: lane l copies 16 bytes from its global address g to
// lds_block + 16 l (lds_block is the same for the whole wave).  Issued from inline asm so
// that the compiler's wait insertion, which cannot tell apart LDS regions written this way,
// does not drain every transfer in flight before each LDS read; callers wait on the
// vector-memory counter themselves (DLLM_WAIT_VMCNT) before a barrier.  M0 is written here
// and nowhere else in the kernels that use it.
__device__ __forceinline__ void dma_16B(const void* g, const void* lds_block) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_block);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(base)
               : "memory");
}

// LDS byte address of a __shared__ object (a constant for a named array; no null check).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One LDS-DMA instruction with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset: lane l copies 16 bytes from sbase + voff to lds + 16 l.  sbase and lds
// must be wave-uniform (scalar registers); waiting is the caller's, as for dma_16B.
__device__ __forceinline__ void dma_16B_sbase(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}

// ------------------------------------------------------------ attention tile layout ----

// Score tiles are computed transposed, S^T = K Q^T, over 32-key tiles made of two 16-row
// MFMA subtiles kt.  Key of the tile that MFMA row rho of subtile kt reads: the eight score
// slots of lane group lg (rows 4 lg .. 4 lg + 3 of both subtiles) are then the consecutive
// keys 8 lg .. 8 lg + 7.
__device__ __forceinline__ int attn_perm_key(int kt, int rho) {
  return ((rho >> 2) << 3) + (kt << 2) + (rho & 3);
}

// Chunk swizzle (16-byte chunk index XOR f(row)) of a V tile in LDS: the four rows of one
// transposing read (ds_read_b64_tr_b16) hit distinct 32-byte slot pairs.
__device__ __forceinline__ int attn_swz_v(int r) { return (r & 3) << 1; }

// ------------------------------------------------------------------ XCD placement -----

// Workgroups are dealt round-robin to the 8 XCDs (each with its own L2): workgroup id goes to
// XCD id % 8.  For a grid of `groups` x `per` units in which the `per` units of a group share
// their inputs (one KV head's cache rows, one head's queries), this maps the id to (group,
// unit) so that every unit of a group runs on the same XCD, consecutively, and the shared
// data is fetched into one L2 once.  Needs groups % 8 == 0 (else the plain row-major order).
__device__ __forceinline__ void xcd_group_unit(int id, int groups, int per, int& group, int& unit) {
  if ((groups & 7) == 0) {
    const int local = id >> 3;
    group = (id & 7) + 8 * (local / per);
    unit = local % per;
  } else {
    group = id / per;
    unit = id % per;
  }
}

// ------------------------------------------------------------------- batch layout -----

// Rows of a batch (refreshed rows, queries) are packed: the rows of sequence b are rows
// [row0, row0 + count) of the packed arrays.  With a row-offset array cu ([B + 1], variable-
// length batches: Elastic-Cache card, deployment notes) row0 = cu[b] and count = cu[b + 1] -
// cu[b]; without one every sequence has n rows and row0 = b * n.  The keys of sequence b are
// its first len cache rows: lens[b], or all S.
__device__ __forceinline__ int seq_row0(const int32_t* cu, int n, int b) { return cu ? cu[b] : b * n; }
__device__ __forceinline__ int seq_rows(const int32_t* cu, int n, int b) {
  return cu ? cu[b + 1] - cu[b] : n;
}
__device__ __forceinline__ int seq_keys(const int32_t* lens, int S, int b) { return lens ? lens[b] : S; }
// Packed rows actually present: cu[B] (a device-side schedule may fill fewer rows than the
// packed arrays hold), never more than the capacity cap; cap without offsets.
__device__ __forceinline__ int live_rows(const int32_t* cu, int B, int cap) {
  return cu ? min(cu[B], cap) : cap;
}
// The sequence that packed row m belongs to (the last b with cu[b] <= m, so sequences without
// rows are passed over).
__device__ __forceinline__ int seq_of_row(const int32_t* cu, int B, int n, int m) {
  if (!cu) return m / n;
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= m) lo = mid;
    else hi = mid;
  }
  return lo;
}

// ------------------------------------------------------------------------ reductions ----

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// Max and sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48), with the
// gfx950 row swaps instead of LDS permutes: v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second, v_permlane16_swap the odd rows of the
// first with the even rows of the second; with both operands = x, the two results hold x of
// lane l and of its partner, in some order, so max / sum of the pair is the same on both.
__device__ __forceinline__ float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the 16 lanes of a row (lanes 16 r .. 16 r + 15), left in every lane of the row:
// DPP partners at distance 1 and 2 (quad permutes), then the mirrored half-row and the
// mirrored row.  Each step adds two operands that are swapped between the partners, so all
// 16 lanes end with the same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xb1, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4e, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xf, 0xf, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xf, 0xf, false));
  return x;
}

// ------------------------------------------------------------------------ rotary --------

// Turns of rotary pair i: t_i = base^(-2i/D) / (2 pi), split into two floats (hi + lo).
__device__ __forceinline__ void rope_turns(int i, int D, double base, float& hi, float& lo) {
  double t = pow(base, -2.0 * (double)i / (double)D) * 0.15915494309189533577;  // 1/(2 pi)
  hi = (float)t;
  lo = (float)(t - (double)hi);
}

// sin and cos of the angle 2 pi * pos * (hi + lo).  The product pos * hi is split exactly
// (fma), its integer turns are dropped exactly, and the hardware sin/cos (argument in turns)
// see a fraction in [-0.5, 0.5].
// Every multiply-add is written as an explicit fmaf so that all kernels using these helpers
// round identically, whatever the compiler contracts elsewhere.  Contraction is off here: the
// split needs a - rint(a) of the ROUNDED product a; fused into fma(pos, hi, -rint(a)) it would
// count the product's rounding residual twice (an angle error of up to half an ulp of
// pos * hi turns, 2e-4 rad at position 4000).
__device__ __forceinline__ void rope_sincos(int pos, float hi, float lo, float& s, float& c) {
#pragma clang fp contract(off)
  const float p = (float)pos;
  const float a = p * hi;
  const float e = fmaf(p, hi, -a);
  const float f = (a - rintf(a)) + fmaf(p, lo, e);
  s = __builtin_amdgcn_sinf(f);
  c = __builtin_amdgcn_cosf(f);
}

// Rotate the pair (x, y) = (x_i, x_{i+D/2}) by the angle with sine s and cosine c.
__device__ __forceinline__ void rope_rotate(float& x, float& y, float s, float c) {
  const float ys = y * s, xs = x * s;
  const float x2 = fmaf(x, c, -ys);
  const float y2 = fmaf(y, c, xs);
  x = x2;
  y = y2;
}

}  // namespace dllm
