// Row selection and the per-layer row schedule, on the device so that no layer waits for the
// host:
//   * feature_sim + select_rows: the rows a sequence refreshes at this step -- its window rows
//     plus the k response rows whose input features moved most since their cache rows were
//     computed (lowest cosine; dLLM-Cache record, abstract: partial response updates guided by
//     feature similarity; Elastic-Cache card, core idea: the live window);
//   * sched_union + sched_pack: the rows one layer refreshes -- every row of a sequence whose
//     drift test fired at an earlier layer (Elastic-Cache card, core idea: recompute from layer
//     l + 1 to L), else its step rows together with its tracked positions, packed as a
//     variable-length batch (row offsets cu) for the refresh and attention calls;
//   * copy_rows: the refreshed rows' cached features become the current ones.
#include "common.hpp"
#include "kernels.hpp"

namespace dllm {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

// The EPC values of one 16-byte chunk as fp32 (bf16: the low half of each word first).
__device__ __forceinline__ float chunk_value(const u32x4& v, int e, bool bf) {
  const uint32_t w = v[bf ? e >> 1 : e];
  if (!bf) return __uint_as_float(w);
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Cosine of row j of sequence b (j >= lo) of the current and cached features, one wave per
// row, fp64.  Products of bf16 or fp32 values are exact in fp64, so only the additions round:
// lane partial sums in ascending chunk order, then a fixed butterfly over the wave.
template <typename T>
__global__ __launch_bounds__(256) void feature_sim(const T* cur, const T* cached, int B, int S, int H,
                                                   int lo, double* sim) {
  constexpr int EPC = 16 / (int)sizeof(T);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int R = S - lo;
  const long long row = (long long)blockIdx.x * 4 + wave;
  if (row >= (long long)B * R) return;          // wave-uniform; the kernel has no barrier
  const int b = (int)(row / R), j = lo + (int)(row % R);
  const size_t base = ((size_t)b * S + j) * H;
  const u32x4* xc = (const u32x4*)(cur + base);
  const u32x4* yc = (const u32x4*)(cached + base);
  double dot = 0.0, xx = 0.0, yy = 0.0;
  const int chunks = H / EPC;
#pragma unroll 4
  for (int c = lane; c < chunks; c += kWave) {
    const u32x4 xv = xc[c], yv = yc[c];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const double x = (double)chunk_value(xv, e, EPC == 8), y = (double)chunk_value(yv, e, EPC == 8);
      dot += x * y;
      xx += x * x;
      yy += y * y;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    dot += __shfl_xor(dot, m, kWave);
    xx += __shfl_xor(xx, m, kWave);
    yy += __shfl_xor(yy, m, kWave);
  }
  if (lane == 0) {
    const bool zx = xx == 0.0, zy = yy == 0.0;
    double s = (zx && zy) ? 1.0 : (zx || zy) ? 0.0 : dot / (sqrt(xx) * sqrt(yy));
    if (s == 0.0) s = 0.0;                       // -0 stored as +0: the two sort alike
    sim[(size_t)b * S + j] = s;
  }
}

// Order-preserving map of fp64 onto uint64 (ascending values -> ascending keys).
__device__ __forceinline__ uint64_t ordered_key(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

// Exclusive prefix sum over the block (1024 threads) of one int per thread, in thread order;
// total gets the sum.  wsum: kSelWaves ints of LDS.
__device__ __forceinline__ int block_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int s = wsum[w];
    before += (w < wave) ? s : 0;
    all += s;
  }
  __syncthreads();                               // wsum is free again
  total = all;
  return before + x - v;
}

// One workgroup per sequence: the k candidates (rows [lo, S) outside the window) of lowest
// similarity, ties to the lower row, found by an 8-pass radix select on the ordered fp64 keys;
// then the window rows and the chosen rows written in ascending row order.  Thread t owns the
// PER consecutive rows [t * PER, t * PER + PER).
template <int PER>
__global__ __launch_bounds__(kSelThreads) void select_rows(const double* sim, int S, int lo,
                                                           const int32_t* window_start, int window,
                                                           int k, int32_t* idx_out) {
  __shared__ int hist[256];
  __shared__ int wsum[kSelWaves];
  __shared__ int pick[2];
  const int b = blockIdx.x, t = threadIdx.x;
  const int ws = window > 0 ? window_start[b] : 0;
  uint64_t key[PER];
  bool cand[PER], win[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = t * PER + i;
    win[i] = j < S && j >= ws && j < ws + window;
    cand[i] = j < S && j >= lo && !win[i];
    key[i] = cand[i] ? ordered_key(sim[(size_t)b * S + j]) : ~0ull;
  }
  // k-th smallest key: digits from the top, each pass counting the candidates that share the
  // digits fixed so far.
  uint64_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int pass = 0; pass < 8 && k > 0; ++pass) {
    const int shift = 56 - 8 * pass;
    if (t < 256) hist[t] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (cand[i] && (key[i] & pmask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255], 1);
    __syncthreads();
    if (t < kWave) {
      // lane l holds bins 4l .. 4l + 3; inclusive scan over lanes finds the digit
      int c[4], own = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[u] = hist[4 * t + u];
        own += c[u];
      }
      int incl = own;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(incl, d, kWave);
        if (t >= d) incl += y;
      }
      int run = incl - own;                      // candidates in bins below 4t
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (run < remaining && remaining <= run + c[u]) {
          pick[0] = 4 * t + u;
          pick[1] = remaining - run;
        }
        run += c[u];
      }
    }
    __syncthreads();
    prefix |= (uint64_t)pick[0] << shift;
    pmask |= 0xffull << shift;
    remaining = pick[1];
    __syncthreads();                             // pick is rewritten by the next pass
  }
  // Chosen: every candidate below the k-th key, and the first `remaining` (by row) equal to it.
  int eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) eq += (k > 0 && cand[i] && key[i] == prefix) ? 1 : 0;
  int eq_total;
  int eq_rank = block_scan(eq, wsum, eq_total);
  bool mark[PER];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    bool chosen = false;
    if (k > 0 && cand[i]) {
      if (key[i] < prefix) chosen = true;
      else if (key[i] == prefix) chosen = (eq_rank++ < remaining);
    }
    mark[i] = chosen || win[i];
    cnt += mark[i] ? 1 : 0;
  }
  int total;
  int pos = block_scan(cnt, wsum, total);
  const int nout = window + k;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (mark[i]) {
      if (pos < nout) idx_out[(size_t)b * nout + pos] = t * PER + i;
      ++pos;
    }
}

// Per sequence: the flag (full_in | decision) and, unless it is set, the sorted union of the
// step rows and the tracked positions (values outside [0, S) are skipped) into temp[b, :]
// with its size in counts[b]; a flagged sequence counts S rows (written by sched_pack).
template <int PER>
__global__ __launch_bounds__(kSelThreads) void sched_union(int S, const int32_t* idx, int n,
                                                           const int32_t* tracked, int m,
                                                           const uint8_t* full_in,
                                                           const uint8_t* decision,
                                                           uint8_t* full_out, int32_t* temp,
                                                           int32_t* counts) {
  extern __shared__ unsigned char map[];         // [S]
  __shared__ int wsum[kSelWaves];
  const int b = blockIdx.x, t = threadIdx.x;
  const bool full = (full_in && full_in[b]) || (decision && decision[b]);
  if (t == 0 && full_out) full_out[b] = full ? 1 : 0;
  if (full) {
    if (t == 0) counts[b] = S;
    return;                                      // uniform over the workgroup
  }
  for (int j = t; j < S; j += kSelThreads) map[j] = 0;
  __syncthreads();
  for (int i = t; i < n; i += kSelThreads) {
    const int j = idx[(size_t)b * n + i];
    if (j >= 0 && j < S) map[j] = 1;
  }
  for (int i = t; tracked && i < m; i += kSelThreads) {
    const int j = tracked[(size_t)b * m + i];
    if (j >= 0 && j < S) map[j] = 1;
  }
  __syncthreads();
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = t * PER + i;
    cnt += (j < S && map[j]) ? 1 : 0;
  }
  int total;
  int pos = block_scan(cnt, wsum, total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = t * PER + i;
    if (j < S && map[j]) temp[(size_t)b * S + pos++] = j;
  }
  if (t == 0) counts[b] = total;
}

// Packs sequence b's rows at its offset (the counts of the sequences before it) and writes
// the offsets cu.
__global__ __launch_bounds__(256) void sched_pack(int B, int S, const int32_t* temp,
                                                  const int32_t* counts, int32_t* rows,
                                                  int32_t* cu) {
  __shared__ int part[4];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int s = 0;
  for (int i = t; i < b; i += 256) s += counts[i];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, kWave);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  const int base = part[0] + part[1] + part[2] + part[3];
  const int cnt = counts[b];
  if (t == 0) {
    cu[b + 1] = base + cnt;
    if (b == 0) cu[0] = 0;
  }
  for (int i = t; i < cnt; i += 256) rows[base + i] = (cnt == S) ? i : temp[(size_t)b * S + i];
}

// dst[b, rows[r]] = src[b, rows[r]] for the packed rows r < cu[B] (row_bytes per row, a
// multiple of 16), one wave per row.
__global__ __launch_bounds__(256) void copy_rows(const char* src, char* dst, int row_bytes, int B,
                                                 int S, const int32_t* rows, const int32_t* cu,
                                                 int cap) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= live_rows(cu, B, cap)) return;        // wave-uniform; no barrier
  const int b = seq_of_row(cu, B, 0, r);
  const size_t off = ((size_t)b * S + rows[r]) * row_bytes;
  const u32x4* s4 = (const u32x4*)(src + off);
  u32x4* d4 = (u32x4*)(dst + off);
  for (int c = lane; c < row_bytes / 16; c += kWave) d4[c] = s4[c];
}

template <int PER>
hipError_t launch_select_per(const SelectArgs& a, hipStream_t s) {
  select_rows<PER><<<a.B, kSelThreads, 0, s>>>(a.sim, a.S, a.lo, a.window_start, a.window, a.k,
                                               a.idx_out);
  return hipGetLastError();
}

template <int PER>
hipError_t launch_union_per(const SchedArgs& a, hipStream_t s) {
  sched_union<PER><<<a.B, kSelThreads, a.S, s>>>(a.S, a.idx, a.n, a.tracked, a.m, a.full_in,
                                                  a.decision, a.full_out, a.temp, a.counts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_similarity_select(const SelectArgs& a, hipStream_t s) {
  const long long rows = (long long)a.B * (a.S - a.lo);
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (grid) {
    if (a.act == DLLM_BF16)
      feature_sim<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)a.cur, (const bf16_t*)a.cached, a.B,
                                               a.S, a.H, a.lo, a.sim);
    else
      feature_sim<float><<<grid, 256, 0, s>>>((const float*)a.cur, (const float*)a.cached, a.B, a.S,
                                              a.H, a.lo, a.sim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int per = (a.S + kSelThreads - 1) / kSelThreads;
  if (per <= 1) return launch_select_per<1>(a, s);
  if (per <= 2) return launch_select_per<2>(a, s);
  if (per <= 4) return launch_select_per<4>(a, s);
  return launch_select_per<8>(a, s);
}

hipError_t launch_schedule_rows(const SchedArgs& a, hipStream_t s) {
  const int per = (a.S + kSelThreads - 1) / kSelThreads;
  hipError_t e;
  if (per <= 1) e = launch_union_per<1>(a, s);
  else if (per <= 2) e = launch_union_per<2>(a, s);
  else if (per <= 4) e = launch_union_per<4>(a, s);
  else if (per <= 8) e = launch_union_per<8>(a, s);
  else if (per <= 16) e = launch_union_per<16>(a, s);
  else e = launch_union_per<32>(a, s);
  if (e != hipSuccess) return e;
  sched_pack<<<a.B, 256, 0, s>>>(a.B, a.S, a.temp, a.counts, a.rows, a.cu);
  return hipGetLastError();
}

hipError_t launch_copy_rows(const void* src, void* dst, int row_bytes, int B, int S,
                            const int32_t* rows, const int32_t* cu, int cap, hipStream_t s) {
  const unsigned grid = (unsigned)((cap + 3) / 4);
  if (!grid) return hipSuccess;
  copy_rows<<<grid, 256, 0, s>>>((const char*)src, (char*)dst, row_bytes, B, S, rows, cu, cap);
  return hipGetLastError();
}

}  // namespace dllm
