// C ABI of the library: argument validation, launch planning, the process-wide options and
// the thread-local error.  The operations themselves are documented in include/dllm_cache.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "dllm_cache.h"
#include "kernels.hpp"

namespace dllm {

// Process-wide switches (DLLM_OPT_*): read from the environment once, on first use, then
// only through dllm_set_options.
namespace {
std::atomic<int> g_options{-1};

int env_options() {
  int f = 0;
  const char* d = getenv("DLLM_DEBUG");
  if (d && d[0] == '1') f |= DLLM_OPT_DEBUG;
  const char* w = getenv("DLLM_GEMM_WIDE_OFFSETS");
  if (w && w[0] == '1') f |= DLLM_OPT_WIDE_OFFSETS;
  return f;
}
}  // namespace

void set_options(int f) { g_options.store(f, std::memory_order_relaxed); }

int options() {
  int f = g_options.load(std::memory_order_relaxed);
  if (f < 0) {
    int expect = -1;
    g_options.compare_exchange_strong(expect, env_options(), std::memory_order_relaxed);
    f = g_options.load(std::memory_order_relaxed);
  }
  return f;
}

}  // namespace dllm

namespace {

thread_local char g_err[512] = "";

dllm_status fail(dllm_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool debug_mode() { return (dllm::options() & DLLM_OPT_DEBUG) != 0; }

// ---- library-owned device memory (one copy per GPU, zero at load, kept to process end) ----

// First invalid position found by the debug-mode index check: the flat index b * n + i, or
// 0x7f7f7f7f when every list is valid.
__device__ __align__(256) int32_t debug_index_report[64];

// Per-device addresses of the library's __device__ arrays.  In host code an array's name is
// only a host-side stand-in; its device address comes from hipGetSymbolAddress, taken once
// per device with that device current.
// Scratch of the allocation-free attention call (dllm_block_attention_noalloc): the split
// partial states and, when the caller passes no lse, the log-sum-exp.  Every call on one GPU
// shares it; nothing in it has to start at zero (each launch writes what it later reads).
__device__ __align__(256) unsigned char scratch[DLLM_NOALLOC_SCRATCH_BYTES];

struct DeviceSymbols {
  int32_t* debug_report = nullptr;
  void* scratch = nullptr;       // device address of `scratch` on this GPU
  bool ready = false;
};
constexpr int kMaxDevices = 64;
DeviceSymbols g_symbols[kMaxDevices];
std::mutex g_symbols_mutex;

dllm_status device_symbols(DeviceSymbols** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DLLM_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DLLM_EUNSUPPORTED, "device id %d", dev);
  std::lock_guard<std::mutex> lock(g_symbols_mutex);
  DeviceSymbols& d = g_symbols[dev];
  if (!d.ready) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_index_report));
    if (e != hipSuccess) return fail(DLLM_ELAUNCH, "hipGetSymbolAddress: %s", hipGetErrorString(e));
    d.debug_report = (int32_t*)p;
    p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(DLLM_ELAUNCH, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    d.scratch = p;
    d.ready = true;
  }
  *out = &d;
  return DLLM_OK;
}

// Debug-mode device pass over the refresh index lists: one workgroup per sequence; every
// position that is out of [0, S) or not above its predecessor is reported, the lowest packed
// index winning.  With row offsets cu (a variable-length batch) sequence b's list is
// idx[cu[b] .. cu[b + 1]); offsets that do not rise from 0, stay within the capacity T and
// give each sequence at most max_rows rows are reported as -1 - b.
__global__ __launch_bounds__(256) void check_index_lists(const int32_t* idx, const int32_t* cu, int n,
                                                         int T, int S, int32_t* report) {
  const int b = blockIdx.x;
  int r0 = b * n, cnt = n;
  if (cu) {
    r0 = cu[b];
    cnt = cu[b + 1] - r0;
    const bool bad_cu = (b == 0 && r0 != 0) || r0 < 0 || cnt < 0 || cnt > n || cu[b + 1] > T;
    if (bad_cu) {
      if (threadIdx.x == 0) atomicMin(&report[0], -1 - b);
      return;
    }
  }
  const int32_t* row = idx + r0;
  for (int i = threadIdx.x; i < cnt; i += 256) {
    const int32_t x = row[i];
    const bool bad = x < 0 || x >= S || (i > 0 && x <= row[i - 1]);
    if (bad) atomicMin(&report[0], r0 + i);
  }
}

// Debug-mode pass over the offsets of a variable-length attention call: sequence b is
// reported as -1 - b when its row offsets leave [0, T] (T: the capacity), decrease, give it
// more than n rows or do not start at 0, or when its key count is outside [1, S].
__global__ __launch_bounds__(256) void check_varlen_offsets(const int32_t* cu, const int32_t* lens,
                                                            int B, int n, int T, int S,
                                                            int32_t* report) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int r0 = cu[b], r1 = cu[b + 1], len = lens ? lens[b] : S;
  const bool bad = r0 < 0 || r1 < r0 || r1 - r0 > n || r1 > T || (b == 0 && r0 != 0) ||
                   len < 1 || len > S;
  if (bad) atomicMin(report, -1 - b);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t elem_bytes(int dtype) { return dtype == DLLM_F32 ? 4 : dtype == DLLM_BF16 ? 2 : 1; }

dllm_status check_desc(const dllm_cache_desc* d) {
  if (!d) return fail(DLLM_EINVAL, "null cache descriptor");
  if (d->batch <= 0 || d->num_kv_heads <= 0 || d->max_seq <= 0 || d->head_dim <= 0)
    return fail(DLLM_EINVAL, "cache dims must be positive (B=%d Hkv=%d S=%d D=%d)", d->batch,
                d->num_kv_heads, d->max_seq, d->head_dim);
  if (d->kv_dtype != DLLM_F32 && d->kv_dtype != DLLM_BF16 && d->kv_dtype != DLLM_FP8_E4M3)
    return fail(DLLM_EINVAL, "unknown kv_dtype %d", d->kv_dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DLLM_EUNSUPPORTED, "head_dim %d: only 64 and 128", d->head_dim);
  if (d->kv_dtype == DLLM_FP8_E4M3 && d->group_size != d->head_dim)
    return fail(DLLM_EUNSUPPORTED, "FP8 cache needs group_size == head_dim (got %d, %d)",
                d->group_size, d->head_dim);
  const double elems = (double)d->batch * d->num_kv_heads * d->max_seq * d->head_dim;
  if (elems > 4.0e12) return fail(DLLM_EINVAL, "cache too large");
  return DLLM_OK;
}

dllm_status check_cache(const dllm_cache* c) {
  if (!c) return fail(DLLM_EINVAL, "null cache");
  dllm_status st = check_desc(&c->desc);
  if (st) return st;
  if (!c->k || !c->v) return fail(DLLM_EINVAL, "cache k/v pointers are null");
  if (!aligned16(c->k) || !aligned16(c->v)) return fail(DLLM_EINVAL, "cache k/v not 16-byte aligned");
  if (c->desc.kv_dtype == DLLM_FP8_E4M3 && (!c->k_scale || !c->v_scale))
    return fail(DLLM_EINVAL, "FP8 cache needs k_scale and v_scale");
  return DLLM_OK;
}

dllm_status finish(hipError_t e, hipStream_t s, const char* what) {
  if (e != hipSuccess) return fail(DLLM_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  if (debug_mode()) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(DLLM_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
  }
  g_err[0] = '\0';
  return DLLM_OK;
}

// Debug mode: a device pass over the index lists (and the row offsets cu, if given); the
// report comes back to the host and the stream is synchronised.
dllm_status debug_check_lists(const int32_t* refresh_idx, const int32_t* cu, int n, int T,
                              const dllm_cache_desc& d, hipStream_t s) {
  DeviceSymbols* sym = nullptr;
  dllm_status st = device_symbols(&sym);
  if (st) return st;
  hipError_t e = hipMemsetAsync(sym->debug_report, 0x7f, sizeof(int32_t), s);
  if (e == hipSuccess) {
    check_index_lists<<<d.batch, 256, 0, s>>>(refresh_idx, cu, n, T, d.max_seq, sym->debug_report);
    e = hipGetLastError();
  }
  int32_t flat = 0, val = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&flat, sym->debug_report, sizeof flat, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && flat >= 0 && flat != 0x7f7f7f7f)
    e = hipMemcpy(&val, refresh_idx + flat, sizeof val, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(DLLM_ELAUNCH, "debug index check: %s", hipGetErrorString(e));
  if (flat < 0) return fail(DLLM_EINVAL, "row offsets broken at sequence %d", -1 - flat);
  if (flat != 0x7f7f7f7f) {
    if (val < 0 || val >= d.max_seq)
      return fail(DLLM_EINVAL, "refresh_idx[%d] = %d outside [0, %d)", flat, val, d.max_seq);
    return fail(DLLM_EINVAL, "refresh_idx not strictly increasing at packed row %d (value %d)", flat, val);
  }
  return DLLM_OK;
}

// Body of both refresh calls.  cu: row offsets [B + 1] of a variable-length batch (n is then
// the largest rows per sequence and total all rows), or null (n rows per sequence).
dllm_status refresh_call(const dllm_cache* c, const void* hidden, int32_t hidden_size,
                         int32_t act_dtype, const int32_t* refresh_idx, const int32_t* cu,
                         int32_t n, long long total, const void* w_qkv, int32_t num_q_heads,
                         float rope_base, void* q_out, void* workspace, size_t ws_bytes,
                         void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (n < 0 || n > d.max_seq) return fail(DLLM_EINVAL, "n=%d outside [0, S=%d]", n, d.max_seq);
  if (total < 0 || total > (long long)d.batch * n)
    return fail(DLLM_EINVAL, "total rows %lld outside [0, B * max rows = %lld]", total,
                (long long)d.batch * n);
  if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
    return fail(DLLM_EINVAL, "num_q_heads %d is not a positive multiple of Hkv %d", num_q_heads,
                d.num_kv_heads);
  if (hidden_size <= 0 || hidden_size % 256)
    return fail(DLLM_EUNSUPPORTED, "hidden_size %d: must be a positive multiple of 256", hidden_size);
  if (act_dtype == DLLM_F32) {
    if (d.kv_dtype != DLLM_F32) return fail(DLLM_EUNSUPPORTED, "fp32 activations need an fp32 cache");
  } else if (act_dtype == DLLM_BF16) {
    if (d.kv_dtype == DLLM_F32) return fail(DLLM_EUNSUPPORTED, "bf16 activations need a bf16 or FP8 cache");
  } else {
    return fail(DLLM_EINVAL, "act_dtype %d: DLLM_F32 or DLLM_BF16", act_dtype);
  }
  if (!(rope_base > 0.f)) return fail(DLLM_EINVAL, "rope_base must be positive");
  if (total == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!hidden || !refresh_idx || !w_qkv || !q_out) return fail(DLLM_EINVAL, "null input/output pointer");
  if (!aligned16(hidden) || !aligned16(w_qkv) || !aligned16(q_out))
    return fail(DLLM_EINVAL, "hidden, w_qkv and q_out must be 16-byte aligned");
  const long long M = total;
  if (M > (1LL << 30)) return fail(DLLM_EINVAL, "too many rows");
  const int N = (num_q_heads + 2 * d.num_kv_heads) * d.head_dim;
  const size_t need = dllm::refresh_workspace_bytes(act_dtype, (int)M, N, hidden_size);
  if (ws_bytes < need) return fail(DLLM_ESIZE, "refresh workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (need && (!workspace || !aligned16(workspace)))
    return fail(DLLM_EINVAL, "refresh workspace must be a 16-byte aligned device pointer");
  hipStream_t s = (hipStream_t)stream;

  if (debug_mode()) {
    st = debug_check_lists(refresh_idx, cu, n, (int)M, d, s);
    if (st) return st;
  }

  dllm::RefreshArgs a;
  a.hidden = hidden;
  a.w = w_qkv;
  a.idx = refresh_idx;
  a.q_out = q_out;
  a.kc = c->k;
  a.vc = c->v;
  a.ks = c->k_scale;
  a.vs = c->v_scale;
  a.B = d.batch;
  a.S = d.max_seq;
  a.H = hidden_size;
  a.n = n;
  a.M = (int)M;
  a.Hq = num_q_heads;
  a.Hkv = d.num_kv_heads;
  a.D = d.head_dim;
  a.act = act_dtype;
  a.kind = d.kv_dtype;
  a.rope_base = (double)rope_base;
  a.ws = (float*)workspace;
  a.cu = cu;
  return finish(dllm::launch_refresh(a, s), s, "refresh");
}

}  // namespace

extern "C" {

const char* dllm_last_error(void) { return g_err; }

int32_t dllm_set_options(int32_t flags) {
  const int prev = dllm::options();
  dllm::set_options(flags & (DLLM_OPT_DEBUG | DLLM_OPT_WIDE_OFFSETS));
  return prev;
}

size_t dllm_cache_bytes(const dllm_cache_desc* d) {
  if (check_desc(d) != DLLM_OK) return 0;
  const size_t rows = (size_t)d->batch * d->num_kv_heads * d->max_seq;
  const size_t kv = round_up(rows * d->head_dim * elem_bytes(d->kv_dtype), 256);
  size_t total = 2 * kv;
  if (d->kv_dtype == DLLM_FP8_E4M3) total += 2 * round_up(rows * sizeof(float), 256);
  return total;
}

dllm_status dllm_cache_alloc(const dllm_cache_desc* d, void* base, size_t nbytes, dllm_cache* out) {
  dllm_status st = check_desc(d);
  if (st) return st;
  if (!base || !out) return fail(DLLM_EINVAL, "null base or out");
  if (((uintptr_t)base & 255u) != 0) return fail(DLLM_EINVAL, "cache base not 256-byte aligned");
  const size_t need = dllm_cache_bytes(d);
  if (nbytes < need) return fail(DLLM_ESIZE, "cache needs %zu bytes, got %zu", need, nbytes);
  const size_t rows = (size_t)d->batch * d->num_kv_heads * d->max_seq;
  const size_t kv = round_up(rows * d->head_dim * elem_bytes(d->kv_dtype), 256);
  char* p = (char*)base;
  out->desc = *d;
  out->k = p;
  out->v = p + kv;
  out->k_scale = nullptr;
  out->v_scale = nullptr;
  if (d->kv_dtype == DLLM_FP8_E4M3) {
    const size_t sc = round_up(rows * sizeof(float), 256);
    out->k_scale = (float*)(p + 2 * kv);
    out->v_scale = (float*)(p + 2 * kv + sc);
  }
  g_err[0] = '\0';
  return DLLM_OK;
}

dllm_status dllm_refresh_qkv_rope_scatter(const dllm_cache* c, const void* hidden,
                                          int32_t hidden_size, int32_t act_dtype,
                                          const int32_t* refresh_idx, int32_t n,
                                          const void* w_qkv, int32_t num_q_heads,
                                          float rope_base, void* q_out, void* workspace,
                                          size_t ws_bytes, void* stream) {
  const long long total = c ? (long long)c->desc.batch * (n > 0 ? n : 0) : 0;
  return refresh_call(c, hidden, hidden_size, act_dtype, refresh_idx, nullptr, n, total, w_qkv,
                      num_q_heads, rope_base, q_out, workspace, ws_bytes, stream);
}

dllm_status dllm_refresh_qkv_rope_scatter_varlen(const dllm_cache* c, const void* hidden,
                                                 int32_t hidden_size, int32_t act_dtype,
                                                 const int32_t* refresh_idx, const int32_t* cu_rows,
                                                 int32_t total_rows, int32_t max_rows,
                                                 const void* w_qkv, int32_t num_q_heads,
                                                 float rope_base, void* q_out, void* workspace,
                                                 size_t ws_bytes, void* stream) {
  if (total_rows > 0 && !cu_rows) return fail(DLLM_EINVAL, "null cu_rows");
  return refresh_call(c, hidden, hidden_size, act_dtype, refresh_idx, cu_rows, max_rows, total_rows,
                      w_qkv, num_q_heads, rope_base, q_out, workspace, ws_bytes, stream);
}

size_t dllm_refresh_workspace_bytes(const dllm_cache_desc* d, int32_t hidden_size,
                                    int32_t act_dtype, int32_t n, int32_t num_q_heads) {
  if (check_desc(d) != DLLM_OK || n < 0 || num_q_heads <= 0 || num_q_heads % d->num_kv_heads ||
      hidden_size <= 0)
    return 0;
  const long long M = (long long)d->batch * n;
  if (M > (1LL << 30)) return 0;
  const int N = (num_q_heads + 2 * d->num_kv_heads) * d->head_dim;
  return dllm::refresh_workspace_bytes(act_dtype, (int)M, N, hidden_size);
}

}  // extern "C"

namespace {

// Workspace of an attention call over `total` query rows, at most n per sequence.
size_t attention_ws_bytes(const dllm_cache_desc* d, int32_t num_q_heads, int32_t n, long long total) {
  if (check_desc(d) != DLLM_OK || num_q_heads <= 0 || num_q_heads % d->num_kv_heads || n < 0 ||
      total < 0)
    return 0;
  const int act = d->kv_dtype == DLLM_F32 ? DLLM_F32 : DLLM_BF16;
  dllm::AttnPlan p = dllm::plan_attention(d->batch, n, num_q_heads, d->num_kv_heads,
                                          d->max_seq, d->head_dim, act, d->kv_dtype, total);
  const size_t lse = (size_t)total * num_q_heads * sizeof(float);
  return round_up(p.part_bytes, 256) + round_up(lse, 256) + 256;
}

}  // namespace

extern "C" {

size_t dllm_attention_workspace_bytes(const dllm_cache_desc* d, int32_t num_q_heads, int32_t n) {
  if (!d || n < 0) return 0;
  return attention_ws_bytes(d, num_q_heads, n, (long long)d->batch * n);
}

size_t dllm_attention_varlen_workspace_bytes(const dllm_cache_desc* d, int32_t num_q_heads,
                                             int32_t total_rows, int32_t max_rows) {
  return attention_ws_bytes(d, num_q_heads, max_rows, total_rows);
}

}  // extern "C"

namespace {

// Body of both attention calls.  noalloc: the workspace is the library's scratch on the
// current GPU (looked up here), and a shape that needs more than it holds is rejected.
// Variable-length batches: cu (row offsets [B + 1]) and lens (keys per sequence [B]) given, n
// the largest rows per sequence and total all rows; otherwise n rows per sequence.
dllm_status attention_call(const dllm_cache* c, const void* q, int32_t act_dtype,
                           int32_t num_q_heads, int32_t n, float softmax_scale, void* out,
                           float* lse, float* attn_mass, void* workspace, size_t ws_bytes,
                           bool noalloc, void* stream, const int32_t* cu = nullptr,
                           const int32_t* lens = nullptr, long long total = -1) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (n < 0 || n > d.max_seq) return fail(DLLM_EINVAL, "n=%d outside [0, S=%d]", n, d.max_seq);
  const bool varlen = total >= 0;
  if (!varlen) total = (long long)d.batch * n;
  if (total > (long long)d.batch * n)
    return fail(DLLM_EINVAL, "total rows %lld above B * max rows = %lld", total, (long long)d.batch * n);
  if (varlen && total > 0 && !cu) return fail(DLLM_EINVAL, "null cu_rows");
  if (varlen && act_dtype == DLLM_F32)
    return fail(DLLM_EUNSUPPORTED, "variable-length batches need bf16 queries");
  if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
    return fail(DLLM_EINVAL, "num_q_heads %d is not a positive multiple of Hkv %d", num_q_heads,
                d.num_kv_heads);
  if (act_dtype == DLLM_F32) {
    if (d.kv_dtype != DLLM_F32) return fail(DLLM_EUNSUPPORTED, "fp32 queries need an fp32 cache");
    if (d.max_seq > 8192) return fail(DLLM_EUNSUPPORTED, "fp32 attention supports S <= 8192");
  } else if (act_dtype == DLLM_BF16) {
    if (d.kv_dtype == DLLM_F32) return fail(DLLM_EUNSUPPORTED, "bf16 queries need a bf16 or FP8 cache");
  } else {
    return fail(DLLM_EINVAL, "act_dtype %d: DLLM_F32 or DLLM_BF16", act_dtype);
  }
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(DLLM_EINVAL, "softmax_scale must be positive and finite");
  if (n == 0 || total == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!q || !out) return fail(DLLM_EINVAL, "null q or out");
  if (!aligned16(q) || !aligned16(out)) return fail(DLLM_EINVAL, "q and out must be 16-byte aligned");
  const size_t need = attention_ws_bytes(&d, num_q_heads, n, total);
  if (noalloc) {
    if (need > (size_t)DLLM_NOALLOC_SCRATCH_BYTES)
      return fail(DLLM_ESIZE, "attention needs %zu bytes of scratch; the allocation-free call "
                  "has %zu", need, (size_t)DLLM_NOALLOC_SCRATCH_BYTES);
    DeviceSymbols* sym = nullptr;
    st = device_symbols(&sym);
    if (st) return st;
    workspace = sym->scratch;
    ws_bytes = DLLM_NOALLOC_SCRATCH_BYTES;
  }
  if (ws_bytes < need) return fail(DLLM_ESIZE, "attention workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (!workspace) return fail(DLLM_EINVAL, "null workspace");
  hipStream_t s = (hipStream_t)stream;
  if (varlen && debug_mode()) {
    DeviceSymbols* sym = nullptr;
    st = device_symbols(&sym);
    if (st) return st;
    hipError_t e = hipMemsetAsync(sym->debug_report, 0x7f, sizeof(int32_t), s);
    if (e == hipSuccess) {
      check_varlen_offsets<<<(d.batch + 255) / 256, 256, 0, s>>>(cu, lens, d.batch, n, (int)total,
                                                                  d.max_seq, sym->debug_report);
      e = hipGetLastError();
    }
    int32_t flat = 0;
    if (e == hipSuccess) e = hipMemcpyAsync(&flat, sym->debug_report, sizeof flat, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(DLLM_ELAUNCH, "debug offset check: %s", hipGetErrorString(e));
    if (flat < 0)
      return fail(DLLM_EINVAL, "row offsets or key count broken at sequence %d", -1 - flat);
  }
  dllm::AttnPlan p = dllm::plan_attention(d.batch, n, num_q_heads, d.num_kv_heads, d.max_seq,
                                          d.head_dim, act_dtype, d.kv_dtype, total);
  char* ws = (char*)round_up((uintptr_t)workspace, 256);
  dllm::AttnArgs a;
  a.q = q;
  a.out = out;
  a.part = (float*)ws;
  a.lse = lse ? lse : (float*)(ws + round_up(p.part_bytes, 256));
  a.mass = attn_mass;
  a.kc = c->k;
  a.vc = c->v;
  a.ks = c->k_scale;
  a.vs = c->v_scale;
  a.B = d.batch;
  a.n = n;
  a.Hq = num_q_heads;
  a.Hkv = d.num_kv_heads;
  a.S = d.max_seq;
  a.D = d.head_dim;
  a.act = act_dtype;
  a.kind = d.kv_dtype;
  a.scale = softmax_scale;
  a.cu = cu;
  a.lens = lens;
  a.T = (int)total;
  return finish(dllm::launch_attention(a, p, s), s, "attention");
}

}  // namespace

extern "C" {

dllm_status dllm_block_attention(const dllm_cache* c, const void* q, int32_t act_dtype,
                                 int32_t num_q_heads, int32_t n, float softmax_scale, void* out,
                                 float* lse, float* attn_mass, void* workspace, size_t ws_bytes,
                                 void* stream) {
  return attention_call(c, q, act_dtype, num_q_heads, n, softmax_scale, out, lse, attn_mass,
                        workspace, ws_bytes, false, stream);
}

dllm_status dllm_block_attention_varlen(const dllm_cache* c, const void* q, int32_t act_dtype,
                                        int32_t num_q_heads, const int32_t* cu_rows,
                                        const int32_t* seq_lens, int32_t total_rows,
                                        int32_t max_rows, float softmax_scale, void* out,
                                        float* lse, float* attn_mass, void* workspace,
                                        size_t ws_bytes, void* stream) {
  if (total_rows < 0) return fail(DLLM_EINVAL, "total_rows < 0");
  return attention_call(c, q, act_dtype, num_q_heads, max_rows, softmax_scale, out, lse,
                        attn_mass, workspace, ws_bytes, false, stream, cu_rows, seq_lens,
                        total_rows);
}

dllm_status dllm_block_attention_noalloc(const dllm_cache* c, const void* q, int32_t act_dtype,
                                         int32_t num_q_heads, int32_t n, float softmax_scale,
                                         void* out, float* lse, float* attn_mass, void* stream) {
  return attention_call(c, q, act_dtype, num_q_heads, n, softmax_scale, out, lse, attn_mass,
                        nullptr, 0, true, stream);
}

size_t dllm_facache_state_bytes(const dllm_cache_desc* d, int32_t num_q_heads) {
  if (check_desc(d) != DLLM_OK || num_q_heads <= 0 || num_q_heads % d->num_kv_heads) return 0;
  return (size_t)d->batch * num_q_heads * d->max_seq * (d->head_dim + 2) * sizeof(float);
}

dllm_status dllm_facache_attention(const dllm_cache* c, void* q_cache, const void* q_block,
                                   const int32_t* block_start, int32_t n, int32_t num_q_heads,
                                   float softmax_scale, float* fa_state, int32_t build, void* out,
                                   float* lse, void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (d.kv_dtype != DLLM_BF16) return fail(DLLM_EUNSUPPORTED, "FACache attention needs a bf16 cache");
  if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
    return fail(DLLM_EINVAL, "num_q_heads %d is not a positive multiple of Hkv %d", num_q_heads,
                d.num_kv_heads);
  if (n < 1 || n > d.max_seq) return fail(DLLM_EINVAL, "n=%d outside [1, S=%d]", n, d.max_seq);
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(DLLM_EINVAL, "softmax_scale must be positive and finite");
  if (build != 0 && build != 1) return fail(DLLM_EINVAL, "build must be 0 or 1");
  if (!q_cache || !q_block || !block_start || !fa_state || !out)
    return fail(DLLM_EINVAL, "null q_cache, q_block, block_start, fa_state or out");
  if (!aligned16(q_cache) || !aligned16(q_block) || !aligned16(fa_state) || !aligned16(out))
    return fail(DLLM_EINVAL, "q_cache, q_block, fa_state and out must be 16-byte aligned");
  const int G = num_q_heads / d.num_kv_heads;
  const long long grid = (long long)d.batch * d.num_kv_heads * (((long long)d.max_seq * G + 31) / 32);
  if (grid > 0x7fffffffLL) return fail(DLLM_EINVAL, "too many query tiles");
  dllm::FacArgs a;
  a.q_cache = q_cache;
  a.q_blk = q_block;
  a.block_start = block_start;
  a.state = fa_state;
  a.out = out;
  a.lse = lse;
  a.kc = c->k;
  a.vc = c->v;
  a.B = d.batch;
  a.S = d.max_seq;
  a.n = n;
  a.Hq = num_q_heads;
  a.Hkv = d.num_kv_heads;
  a.D = d.head_dim;
  a.build = build;
  a.scale = softmax_scale;
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_facache(a, s), s, "facache attention");
}

size_t dllm_track_buffer_bytes(const dllm_cache_desc* d, int32_t num_q_heads, int32_t k) {
  if (!d || d->batch <= 0 || d->head_dim <= 0 || num_q_heads <= 0 || k <= 0) return 0;
  const size_t rows = (size_t)d->batch * num_q_heads * k * 2;
  switch (d->kv_dtype) {
    case DLLM_F32: return rows * d->head_dim * 4;
    case DLLM_BF16: return rows * d->head_dim * 2;
    case DLLM_FP8_E4M3: return rows * (d->head_dim + sizeof(float));
    default: return 0;
  }
}

size_t dllm_drift_workspace_bytes(int32_t batch) {
  if (batch <= 0) return 0;
  return (size_t)batch * dllm::kDriftArriveStride * sizeof(unsigned long long);
}

dllm_status dllm_drift_check(const dllm_cache* c, int32_t num_q_heads, int32_t k, float gamma,
                             int32_t* track_idx, void* track_buf, const float* attn_mass,
                             float* sigma_out, uint8_t* refresh_out, void* workspace,
                             size_t ws_bytes, void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
    return fail(DLLM_EINVAL, "num_q_heads %d is not a positive multiple of Hkv %d", num_q_heads,
                d.num_kv_heads);
  if (k < 1 || k > 64) return fail(DLLM_EINVAL, "k=%d outside [1, 64]", k);
  if (!(gamma == gamma)) return fail(DLLM_EINVAL, "gamma is NaN");
  if (!track_idx || !track_buf || !sigma_out || !refresh_out)
    return fail(DLLM_EINVAL, "null tracking / output pointer");
  if (!aligned16(track_buf)) return fail(DLLM_EINVAL, "track_buf must be 16-byte aligned");
  if (attn_mass && d.max_seq > 16384)
    return fail(DLLM_EUNSUPPORTED, "tracking update supports S <= 16384 (S=%d)", d.max_seq);
  if ((int64_t)d.max_seq * d.head_dim >= ((int64_t)1 << 31))
    return fail(DLLM_EUNSUPPORTED, "drift check needs S * head_dim < 2^31");
  if (workspace) {
    const size_t need = dllm_drift_workspace_bytes(d.batch);
    if (ws_bytes < need) return fail(DLLM_ESIZE, "drift workspace needs %zu bytes, got %zu", need, ws_bytes);
    if ((uintptr_t)workspace % 8) return fail(DLLM_EINVAL, "drift workspace must be 8-byte aligned");
  }
  dllm::DriftArgs a;
  a.kc = c->k;
  a.vc = c->v;
  a.ks = c->k_scale;
  a.vs = c->v_scale;
  a.track_idx = track_idx;
  a.track_buf = track_buf;
  a.mass = attn_mass;
  a.sigma = sigma_out;
  a.refresh = refresh_out;
  a.arrive = (unsigned long long*)workspace;
  a.B = d.batch;
  a.Hq = num_q_heads;
  a.Hkv = d.num_kv_heads;
  a.S = d.max_seq;
  a.D = d.head_dim;
  a.k = k;
  a.kind = d.kv_dtype;
  a.gamma = gamma;
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_drift(a, s), s, "drift");
}

size_t dllm_similarity_select_workspace_bytes(int32_t batch, int32_t max_seq) {
  if (batch <= 0 || max_seq <= 0) return 0;
  return (size_t)batch * max_seq * sizeof(double);
}

dllm_status dllm_similarity_select(int32_t batch, int32_t max_seq, int32_t hidden_size,
                                   int32_t act_dtype, const void* hidden_cur,
                                   const void* hidden_cached, int32_t lo,
                                   const int32_t* window_start, int32_t window, int32_t k,
                                   int32_t* idx_out, double* sim_out, void* workspace,
                                   size_t ws_bytes, void* stream) {
  if (batch <= 0 || max_seq <= 0) return fail(DLLM_EINVAL, "batch and max_seq must be positive");
  if (max_seq > dllm::kSelectMaxSeq)
    return fail(DLLM_EUNSUPPORTED, "similarity selection supports S <= %d", dllm::kSelectMaxSeq);
  if (act_dtype != DLLM_BF16 && act_dtype != DLLM_F32)
    return fail(DLLM_EINVAL, "act_dtype %d: DLLM_BF16 or DLLM_F32", act_dtype);
  const int epc = act_dtype == DLLM_BF16 ? 8 : 4;
  if (hidden_size <= 0 || hidden_size % epc)
    return fail(DLLM_EINVAL, "hidden_size %d must be a positive multiple of %d", hidden_size, epc);
  if (lo < 0 || lo >= max_seq) return fail(DLLM_EINVAL, "lo=%d outside [0, S=%d)", lo, max_seq);
  if (window < 0 || k < 0 || (long long)window + k > (long long)max_seq - lo)
    return fail(DLLM_EINVAL, "window=%d, k=%d: need window + k <= S - lo = %d", window, k, max_seq - lo);
  if (window > 0 && !window_start) return fail(DLLM_EINVAL, "null window_start with window > 0");
  if (window + k == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!hidden_cur || !hidden_cached || !idx_out) return fail(DLLM_EINVAL, "null input or output");
  if (!aligned16(hidden_cur) || !aligned16(hidden_cached))
    return fail(DLLM_EINVAL, "hidden arrays must be 16-byte aligned");
  double* sim = sim_out;
  if (!sim) {
    const size_t need = dllm_similarity_select_workspace_bytes(batch, max_seq);
    if (ws_bytes < need) return fail(DLLM_ESIZE, "selection workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (!workspace || ((uintptr_t)workspace & 7u)) return fail(DLLM_EINVAL, "workspace must be an 8-byte aligned device pointer");
    sim = (double*)workspace;
  } else if ((uintptr_t)sim_out & 7u) {
    return fail(DLLM_EINVAL, "sim_out must be 8-byte aligned");
  }
  dllm::SelectArgs a;
  a.cur = hidden_cur;
  a.cached = hidden_cached;
  a.sim = sim;
  a.window_start = window_start;
  a.idx_out = idx_out;
  a.B = batch;
  a.S = max_seq;
  a.H = hidden_size;
  a.act = act_dtype;
  a.lo = lo;
  a.window = window;
  a.k = k;
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_similarity_select(a, s), s, "similarity select");
}

size_t dllm_schedule_rows_workspace_bytes(int32_t batch, int32_t max_seq) {
  if (batch <= 0 || max_seq <= 0) return 0;
  return round_up((size_t)batch * max_seq * sizeof(int32_t), 256) + (size_t)batch * sizeof(int32_t);
}

dllm_status dllm_schedule_rows(int32_t batch, int32_t max_seq, const int32_t* idx, int32_t n,
                               const int32_t* tracked, int32_t m, const uint8_t* full_in,
                               const uint8_t* decision, uint8_t* full_out, int32_t* rows_out,
                               int32_t capacity, int32_t* cu_out, void* workspace,
                               size_t ws_bytes, void* stream) {
  if (batch <= 0 || max_seq <= 0) return fail(DLLM_EINVAL, "batch and max_seq must be positive");
  if (max_seq > dllm::kScheduleMaxSeq)
    return fail(DLLM_EUNSUPPORTED, "the row schedule supports S <= %d", dllm::kScheduleMaxSeq);
  if (n < 0 || m < 0) return fail(DLLM_EINVAL, "n and m must be >= 0");
  if (n > 0 && !idx) return fail(DLLM_EINVAL, "null idx with n > 0");
  if (m > 0 && !tracked) return fail(DLLM_EINVAL, "null tracked with m > 0");
  if ((long long)capacity < (long long)batch * max_seq)
    return fail(DLLM_ESIZE, "capacity %d below B * S = %lld", capacity, (long long)batch * max_seq);
  if (!rows_out || !cu_out) return fail(DLLM_EINVAL, "null rows_out or cu_out");
  const size_t need = dllm_schedule_rows_workspace_bytes(batch, max_seq);
  if (ws_bytes < need) return fail(DLLM_ESIZE, "schedule workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (!workspace || ((uintptr_t)workspace & 255u))
    return fail(DLLM_EINVAL, "workspace must be a 256-byte aligned device pointer");
  dllm::SchedArgs a;
  a.idx = idx;
  a.tracked = m > 0 ? tracked : nullptr;
  a.full_in = full_in;
  a.decision = decision;
  a.full_out = full_out;
  a.rows = rows_out;
  a.cu = cu_out;
  a.temp = (int32_t*)workspace;
  a.counts = (int32_t*)((char*)workspace + round_up((size_t)batch * max_seq * sizeof(int32_t), 256));
  a.B = batch;
  a.S = max_seq;
  a.n = n;
  a.m = m;
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_schedule_rows(a, s), s, "schedule rows");
}

dllm_status dllm_copy_rows_varlen(int32_t batch, int32_t max_seq, int32_t row_bytes,
                                  const void* src, void* dst, const int32_t* rows,
                                  const int32_t* cu_rows, int32_t capacity, void* stream) {
  if (batch <= 0 || max_seq <= 0) return fail(DLLM_EINVAL, "batch and max_seq must be positive");
  if (row_bytes <= 0 || row_bytes % 16) return fail(DLLM_EINVAL, "row_bytes %d: a positive multiple of 16", row_bytes);
  if (capacity < 0) return fail(DLLM_EINVAL, "capacity < 0");
  if (capacity == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!src || !dst || !rows || !cu_rows) return fail(DLLM_EINVAL, "null pointer argument");
  if (!aligned16(src) || !aligned16(dst)) return fail(DLLM_EINVAL, "src and dst must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_copy_rows(src, dst, row_bytes, batch, max_seq, rows, cu_rows, capacity, s),
                s, "copy rows");
}

namespace {
// Workspace of one schedule layer: the similarities, the row schedule's scratch, the refresh's
// partials (capacity B * S rows) and the attention's split states.
struct StepWs {
  size_t sim, sched, refresh, attn, total;
};
StepWs step_ws(const dllm_cache_desc* d, int32_t H, int32_t Hq) {
  StepWs w{};
  const long long cap = (long long)d->batch * d->max_seq;
  const int N = (Hq + 2 * d->num_kv_heads) * d->head_dim;
  w.sim = round_up(dllm_similarity_select_workspace_bytes(d->batch, d->max_seq), 256);
  w.sched = round_up(dllm_schedule_rows_workspace_bytes(d->batch, d->max_seq), 256);
  w.refresh = round_up(dllm::refresh_workspace_bytes(DLLM_BF16, (int)cap, N, H), 256);
  w.attn = round_up(attention_ws_bytes(d, Hq, d->max_seq, cap), 256);
  w.total = w.sim + w.sched + w.refresh + w.attn + 256;
  return w;
}
}  // namespace

size_t dllm_layer_step_workspace_bytes(const dllm_cache_desc* d, int32_t hidden_size,
                                       int32_t num_q_heads) {
  if (check_desc(d) != DLLM_OK || hidden_size <= 0 || num_q_heads <= 0 ||
      num_q_heads % d->num_kv_heads || (long long)d->batch * d->max_seq > 0x7fffffffLL)
    return 0;
  return step_ws(d, hidden_size, num_q_heads).total;
}

dllm_status dllm_elastic_layer_step(const dllm_cache* c, const dllm_layer_step* a,
                                    void* workspace, size_t ws_bytes, void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  if (!a) return fail(DLLM_EINVAL, "null step arguments");
  const dllm_cache_desc& d = c->desc;
  if (d.kv_dtype != DLLM_BF16) return fail(DLLM_EUNSUPPORTED, "the layer step needs a bf16 cache");
  if ((long long)d.batch * d.max_seq > 0x7fffffffLL) return fail(DLLM_EINVAL, "B * S too large");
  const size_t need = dllm_layer_step_workspace_bytes(&d, a->hidden_size, a->num_q_heads);
  if (!need) return fail(DLLM_EINVAL, "invalid hidden_size or num_q_heads");
  if (ws_bytes < need) return fail(DLLM_ESIZE, "layer step workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (!workspace) return fail(DLLM_EINVAL, "null workspace");
  if (!a->full || !a->decision) return fail(DLLM_EINVAL, "null full or decision");
  const StepWs w = step_ws(&d, a->hidden_size, a->num_q_heads);
  char* base = (char*)round_up((uintptr_t)workspace, 256);
  char* ws_sim = base;
  char* ws_sched = ws_sim + w.sim;
  char* ws_ref = ws_sched + w.sched;
  char* ws_att = ws_ref + w.refresh;
  const int B = d.batch, S = d.max_seq, Hq = a->num_q_heads;
  const int cap = B * S;
  st = dllm_similarity_select(B, S, a->hidden_size, DLLM_BF16, a->hidden_cur, a->hidden_feat,
                              a->lo, a->window_start, a->window, a->k_select, a->step_rows,
                              nullptr, ws_sim, w.sim, stream);
  if (st) return st;
  st = dllm_schedule_rows(B, S, a->step_rows, a->window + a->k_select, a->track_idx,
                          Hq * a->k_track, a->full, a->decision, a->full, a->rows, cap,
                          a->cu_rows, ws_sched, w.sched, stream);
  if (st) return st;
  st = refresh_call(c, a->hidden_cur, a->hidden_size, DLLM_BF16, a->rows, a->cu_rows, S, cap,
                    a->w_qkv, Hq, a->rope_base, a->q, ws_ref, w.refresh, stream);
  if (st) return st;
  st = attention_call(c, a->q, DLLM_BF16, Hq, S, a->softmax_scale, a->out, a->lse, a->attn_mass,
                      ws_att, w.attn, false, stream, a->cu_rows, nullptr, cap);
  if (st) return st;
  st = dllm_drift_check(c, Hq, a->k_track, a->gamma, a->track_idx, a->track_buf, a->attn_mass,
                        a->sigma, a->decision, nullptr, 0, stream);
  if (st) return st;
  return dllm_copy_rows_varlen(B, S, a->hidden_size * 2, a->hidden_cur, a->hidden_feat, a->rows,
                               a->cu_rows, cap, stream);
}

dllm_status dllm_fp8_quantize_weight(const void* w, int32_t N, int32_t K, uint8_t* codes,
                                     float* scales, void* stream) {
  if (N <= 0 || K <= 0 || N % 128 || K % 128)
    return fail(DLLM_EINVAL, "N=%d, K=%d: positive multiples of 128", N, K);
  if (!w || !codes || !scales) return fail(DLLM_EINVAL, "null pointer argument");
  if (!aligned16(w) || !aligned16(codes) || !aligned16(scales))
    return fail(DLLM_EINVAL, "w, codes and scales must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_fp8_quant_blocks(w, N, K, codes, scales, s), s, "fp8 weight quantisation");
}

dllm_status dllm_fp8_quantize_activations(const void* x, int32_t M, int32_t K, uint8_t* codes,
                                          float* scales_t, int32_t pitch, void* stream) {
  if (M < 0 || K <= 0 || K % 128) return fail(DLLM_EINVAL, "M=%d, K=%d: M >= 0, K a positive multiple of 128", M, K);
  if (pitch < M) return fail(DLLM_EINVAL, "pitch %d below M %d", pitch, M);
  if (pitch == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if ((M > 0 && (!x || !codes)) || !scales_t) return fail(DLLM_EINVAL, "null pointer argument");
  if ((M > 0 && (!aligned16(x) || !aligned16(codes))) || ((uintptr_t)scales_t & 3u))
    return fail(DLLM_EINVAL, "x and codes must be 16-byte aligned, scales_t 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_fp8_quant_groups(x, M, K, pitch, codes, scales_t, true, s), s,
                "fp8 activation quantisation");
}

namespace {
struct Fp8Ws {
  size_t codes, scales, part, total;
};
Fp8Ws fp8_ws(const dllm::Fp8Plan& p) {
  Fp8Ws w{};
  w.codes = round_up(p.codes_bytes, 256);
  w.scales = round_up(p.scales_bytes, 256);
  w.part = round_up(p.part_bytes, 256);
  w.total = w.codes + w.scales + w.part + 256;
  return w;
}
bool fp8_shape_ok(int32_t M, int32_t N, int32_t K) {
  return M >= 0 && N > 0 && K > 0 && N % 128 == 0 && K % 128 == 0 && K / 128 <= dllm::kFp8MaxGroups &&
         (long long)M * K < (1LL << 32) && (long long)N * K < (1LL << 32);
}
}  // namespace

size_t dllm_fp8_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (!fp8_shape_ok(M, N, K) || M == 0) return 0;
  return fp8_ws(dllm::plan_fp8_linear(M, N, K)).total;
}

dllm_status dllm_fp8_linear(const void* x, int32_t M, int32_t K, const uint8_t* w_codes,
                            const float* w_scales, int32_t N, void* y, void* workspace,
                            size_t ws_bytes, void* stream) {
  if (!fp8_shape_ok(M, N, K))
    return fail(DLLM_EINVAL, "M=%d, N=%d, K=%d: N, K positive multiples of 128, K <= 65536, M * K and N * K below 2^32", M, N, K);
  if (M == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!x || !w_codes || !w_scales || !y) return fail(DLLM_EINVAL, "null pointer argument");
  if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || ((uintptr_t)y & 7u))
    return fail(DLLM_EINVAL, "x, w_codes, w_scales must be 16-byte aligned, y 8-byte aligned");
  const dllm::Fp8Plan p = dllm::plan_fp8_linear(M, N, K);
  const Fp8Ws w = fp8_ws(p);
  if (ws_bytes < w.total) return fail(DLLM_ESIZE, "fp8 linear workspace needs %zu bytes, got %zu", w.total, ws_bytes);
  if (!workspace) return fail(DLLM_EINVAL, "null workspace");
  char* base = (char*)round_up((uintptr_t)workspace, 256);
  dllm::Fp8GemmArgs a;
  a.xq = (const uint8_t*)base;
  a.sxT = (const float*)(base + w.codes);
  a.wq = w_codes;
  a.sw = w_scales;
  a.y = y;
  a.part = p.splits > 1 ? (float*)(base + w.codes + w.scales) : nullptr;
  a.M = M;
  a.N = N;
  a.K = K;
  a.Mp = p.Mp;
  a.kb_per_split = p.kb_per_split;
  a.splits = p.splits;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dllm::launch_fp8_quant_groups(x, M, K, p.Mp, (uint8_t*)base, (float*)(base + w.codes), false, s);
  if (e == hipSuccess) e = dllm::launch_fp8_gemm(a, p, s);
  return finish(e, s, "fp8 linear");
}

dllm_status dllm_rope_rows(void* y, int32_t M, int32_t ld, int32_t heads, int32_t head_dim,
                           const int32_t* pos, float rope_base, void* stream) {
  if (M < 0 || heads <= 0 || (head_dim != 64 && head_dim != 128))
    return fail(DLLM_EINVAL, "M=%d, heads=%d, head_dim=%d: M >= 0, heads >= 1, head_dim 64 or 128", M, heads, head_dim);
  if ((long long)ld < (long long)heads * head_dim) return fail(DLLM_EINVAL, "ld %d below heads * head_dim", ld);
  if (!(rope_base > 0.f)) return fail(DLLM_EINVAL, "rope_base must be positive");
  if (M == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!y || !pos) return fail(DLLM_EINVAL, "null y or pos");
  if ((uintptr_t)y & 1u) return fail(DLLM_EINVAL, "y must be 2-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_rope_rows(y, M, ld, heads, head_dim, pos, (double)rope_base, s), s,
                "rope rows");
}

dllm_status dllm_scatter_kv_rows(const dllm_cache* c, const void* y, int32_t ld, int32_t k_col,
                                 int32_t v_col, const int32_t* refresh_idx, int32_t n,
                                 void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (d.kv_dtype != DLLM_BF16) return fail(DLLM_EUNSUPPORTED, "the row scatter takes a bf16 cache");
  if (n < 0 || n > d.max_seq) return fail(DLLM_EINVAL, "n=%d outside [0, S=%d]", n, d.max_seq);
  const long long span = (long long)d.num_kv_heads * d.head_dim;
  if (ld % 8 || k_col % 8 || v_col % 8 || k_col < 0 || v_col < 0 || k_col + span > ld || v_col + span > ld)
    return fail(DLLM_EINVAL, "ld %d, k_col %d, v_col %d: multiples of 8 with Hkv * D columns inside ld", ld, k_col, v_col);
  if (n == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!y || !refresh_idx) return fail(DLLM_EINVAL, "null y or refresh_idx");
  if (!aligned16(y)) return fail(DLLM_EINVAL, "y must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (debug_mode()) {
    st = debug_check_lists(refresh_idx, nullptr, n, d.batch * n, d, s);
    if (st) return st;
  }
  return finish(dllm::launch_scatter_kv_rows(y, ld, k_col, v_col, c->k, c->v, d.batch, n,
                                             d.num_kv_heads, d.max_seq, d.head_dim, refresh_idx, s),
                s, "row scatter");
}

dllm_status dllm_mfma_rate_probe(int32_t kind, int32_t tile, int32_t workgroups, int32_t iters,
                                 float* out, void* stream) {
  if (kind != DLLM_BF16 && kind != DLLM_FP8_E4M3) return fail(DLLM_EINVAL, "kind: DLLM_BF16 or DLLM_FP8_E4M3");
  if (tile != 16 && tile != 32) return fail(DLLM_EINVAL, "tile: 16 or 32");
  if (workgroups <= 0 || iters <= 0) return fail(DLLM_EINVAL, "workgroups and iters must be positive");
  if (!out) return fail(DLLM_EINVAL, "null out");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_mfma_probe(kind, tile == 32, workgroups, iters, out, s), s, "mfma probe");
}

dllm_status dllm_read_rate_probe(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* out,
                                 void* stream) {
  if (bytes < 0 || bytes % 16) return fail(DLLM_EINVAL, "bytes must be a non-negative multiple of 16");
  if (bytes > 0 && !buf) return fail(DLLM_EINVAL, "null buf");
  if ((uintptr_t)buf % 16) return fail(DLLM_EINVAL, "buf must be 16-byte aligned");
  if (workgroups <= 0) return fail(DLLM_EINVAL, "workgroups must be positive");
  if (!out) return fail(DLLM_EINVAL, "null out");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_read_probe(buf, (size_t)bytes, workgroups, out, s), s, "read probe");
}

dllm_status dllm_fp8_e4m3_roundtrip(const float* x, int64_t n, float scale, uint8_t* codes,
                                    float* decoded, void* stream) {
  if (n < 0) return fail(DLLM_EINVAL, "n < 0");
  if (n > 0 && (!x || !codes)) return fail(DLLM_EINVAL, "null x or codes");
  if (!(scale > 0.f) || !(scale < 1e38f)) return fail(DLLM_EINVAL, "scale must be positive and finite");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_fp8_roundtrip(x, n, scale, codes, decoded, s), s, "fp8 roundtrip");
}

}  // extern "C"
