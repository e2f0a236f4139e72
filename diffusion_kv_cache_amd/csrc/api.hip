// C ABI of the library: argument validation, launch planning and the thread-local error.
// The operations themselves are documented in include/dllm_cache.h.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "dllm_cache.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

dllm_status fail(dllm_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool debug_mode() {
  const char* e = getenv("DLLM_DEBUG");
  return e && e[0] == '1';
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

}  // namespace

extern "C" {

const char* dllm_last_error(void) { return g_err; }

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
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (n < 0 || n > d.max_seq) return fail(DLLM_EINVAL, "n=%d outside [0, S=%d]", n, d.max_seq);
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
  if (n == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!hidden || !refresh_idx || !w_qkv || !q_out) return fail(DLLM_EINVAL, "null input/output pointer");
  if (!aligned16(hidden) || !aligned16(w_qkv) || !aligned16(q_out))
    return fail(DLLM_EINVAL, "hidden, w_qkv and q_out must be 16-byte aligned");
  const long long M = (long long)d.batch * n;
  if (M > (1LL << 30)) return fail(DLLM_EINVAL, "too many rows");
  const int N = (num_q_heads + 2 * d.num_kv_heads) * d.head_dim;
  const size_t need = dllm::refresh_workspace_bytes(act_dtype, (int)M, N, hidden_size);
  if (ws_bytes < need) return fail(DLLM_ESIZE, "refresh workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (need && (!workspace || !aligned16(workspace)))
    return fail(DLLM_EINVAL, "refresh workspace must be a 16-byte aligned device pointer");
  hipStream_t s = (hipStream_t)stream;

  if (debug_mode()) {
    std::vector<int32_t> h((size_t)M);
    hipError_t e = hipMemcpyAsync(h.data(), refresh_idx, (size_t)M * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(DLLM_ELAUNCH, "debug index copy: %s", hipGetErrorString(e));
    for (int b = 0; b < d.batch; ++b)
      for (int i = 0; i < n; ++i) {
        const int32_t x = h[(size_t)b * n + i];
        if (x < 0 || x >= d.max_seq)
          return fail(DLLM_EINVAL, "refresh_idx[%d][%d] = %d outside [0, %d)", b, i, x, d.max_seq);
        if (i > 0 && x <= h[(size_t)b * n + i - 1])
          return fail(DLLM_EINVAL, "refresh_idx[%d] not strictly increasing at %d", b, i);
      }
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
  return finish(dllm::launch_refresh(a, s), s, "refresh");
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

size_t dllm_attention_workspace_bytes(const dllm_cache_desc* d, int32_t num_q_heads, int32_t n) {
  if (check_desc(d) != DLLM_OK || num_q_heads <= 0 || num_q_heads % d->num_kv_heads || n < 0)
    return 0;
  const int act = d->kv_dtype == DLLM_F32 ? DLLM_F32 : DLLM_BF16;
  dllm::AttnPlan p = dllm::plan_attention(d->batch, n, num_q_heads, d->num_kv_heads,
                                          d->max_seq, d->head_dim, act, d->kv_dtype);
  const size_t lse = (size_t)d->batch * num_q_heads * n * sizeof(float);
  return round_up(p.part_bytes, 256) + round_up(lse, 256) + 256;
}

dllm_status dllm_block_attention(const dllm_cache* c, const void* q, int32_t act_dtype,
                                 int32_t num_q_heads, int32_t n, float softmax_scale, void* out,
                                 float* lse, float* attn_mass, void* workspace, size_t ws_bytes,
                                 void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (n < 0 || n > d.max_seq) return fail(DLLM_EINVAL, "n=%d outside [0, S=%d]", n, d.max_seq);
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
  if (n == 0) {
    g_err[0] = '\0';
    return DLLM_OK;
  }
  if (!q || !out) return fail(DLLM_EINVAL, "null q or out");
  if (!aligned16(q) || !aligned16(out)) return fail(DLLM_EINVAL, "q and out must be 16-byte aligned");
  const size_t need = dllm_attention_workspace_bytes(&d, num_q_heads, n);
  if (ws_bytes < need) return fail(DLLM_ESIZE, "attention workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (!workspace) return fail(DLLM_EINVAL, "null workspace");
  dllm::AttnPlan p = dllm::plan_attention(d.batch, n, num_q_heads, d.num_kv_heads, d.max_seq,
                                          d.head_dim, act_dtype, d.kv_dtype);
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
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_attention(a, p, s), s, "attention");
}

dllm_status dllm_drift_check(const dllm_cache* c, int32_t num_q_heads, int32_t k, float gamma,
                             int32_t* track_idx, void* track_buf, const float* attn_mass,
                             float* sigma_out, uint8_t* refresh_out, void* stream) {
  dllm_status st = check_cache(c);
  if (st) return st;
  const dllm_cache_desc& d = c->desc;
  if (d.kv_dtype == DLLM_FP8_E4M3) return fail(DLLM_EUNSUPPORTED, "drift check on FP8 caches");
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
  dllm::DriftArgs a;
  a.kc = c->k;
  a.vc = c->v;
  a.track_idx = track_idx;
  a.track_buf = track_buf;
  a.mass = attn_mass;
  a.sigma = sigma_out;
  a.refresh = refresh_out;
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

dllm_status dllm_fp8_e4m3_roundtrip(const float* x, int64_t n, float scale, uint8_t* codes,
                                    float* decoded, void* stream) {
  if (n < 0) return fail(DLLM_EINVAL, "n < 0");
  if (n > 0 && (!x || !codes)) return fail(DLLM_EINVAL, "null x or codes");
  if (!(scale > 0.f) || !(scale < 1e38f)) return fail(DLLM_EINVAL, "scale must be positive and finite");
  hipStream_t s = (hipStream_t)stream;
  return finish(dllm::launch_fp8_roundtrip(x, n, scale, codes, decoded, s), s, "fp8 roundtrip");
}

}  // extern "C"
