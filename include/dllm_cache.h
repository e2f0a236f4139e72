/*
 * dllm_cache.h -- C ABI of the per-layer cached denoising step for diffusion LLMs on
 * AMD Instinct MI355X (gfx950).
 *
 * One step of one layer:
 *   1. gather the hidden rows of the positions being refreshed,
 *   2. project them to Q, K, V and rotate Q and K (RoPE),
 *   3. scatter-write K and V into a flat, preallocated cache, leaving every other row as it
 *      is,
 *   4. run bidirectional (unmasked) softmax attention of the refreshed rows' queries over
 *      the whole cache,
 *   5. optionally test the drift of the previous step's most-attended tokens and refresh the
 *      tracking set.
 *
 * Sources for what each call computes:
 *   - Flash-dLLM news summary (skillfed.io), paragraph on the memory problem: projection,
 *     rotary embedding and cache write are fused into one kernel that keeps intermediates on
 *     chip, instead of four kernels that each round-trip through HBM; paragraph on batch size:
 *     a flat preallocated cache layout with no dynamic allocation.
 *   - LaCache (gist.science explainer), Technical Summary, Problem Statement: tokens of a
 *     block are updated together while bidirectional attention sees the full context;
 *     Methodology 1 (Lossless State Memoization): only positions outside the invariant
 *     region U are recomputed, and the cached post-projection, post-RoPE states of U are
 *     reused, with mathematically equal outputs; Methodology 2: per-group FP8 with 1 x 128
 *     groups.
 *   - Flash-Cache article (intl.cloud.baidu.com), section 3.1: attention is
 *     softmax(q k^T / sqrt(d)) v.
 *   - Elastic-Cache (DAIR academy paper card), core idea and knobs: cosine similarity of the
 *     previous step's most-attended tokens, refresh when it drops below gamma (default 0.9).
 *   - Flash-dLLM news summary, paragraph on selective cache tracking: a fixed budget of the
 *     32 most-attended tokens.
 *
 * Conventions for every call:
 *   - Memory.  The caller owns all device memory.  The library never allocates or frees
 *     device memory and keeps no state between calls, apart from a thread-local error
 *     message.  All pointers named "device" must be device (HBM) pointers, 16-byte aligned.
 *   - Streams.  `stream` is a hipStream_t (NULL = the null stream).  Every call enqueues its
 *     kernels on it and returns without synchronising (except in debug mode, below).
 *   - Layouts.  Contiguous, row-major, in the order given.  Indices are int32.
 *   - Errors.  A call returns DLLM_OK or an error code and enqueues nothing on error;
 *     dllm_last_error() then describes the failure.  No C++ exception crosses the ABI.
 *   - Debug mode.  With the environment variable DLLM_DEBUG=1 the refresh call copies the
 *     index list to the host, checks that every list is sorted, unique and in [0, S), and
 *     returns DLLM_EINVAL otherwise; every call synchronises its stream and reports launch
 *     failures.  Without debug mode an index list that breaks the contract is undefined
 *     behaviour.
 *   - DLLM_GEMM_WIDE_OFFSETS=1 makes the refresh of more than 64 rows address its operands
 *     with 64-bit per-lane pointers, the form it otherwise takes only when the hidden states
 *     or the weights span 4 GB or more (same results; for testing that form).
 */
#ifndef DLLM_CACHE_H
#define DLLM_CACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef DLLM_API
#define DLLM_API __attribute__((visibility("default")))
#endif

typedef int32_t dllm_status;

#define DLLM_OK 0
#define DLLM_EINVAL 1        /* bad argument: null pointer, bad dimension, misalignment */
#define DLLM_ESIZE 2         /* a caller buffer is too small */
#define DLLM_EUNSUPPORTED 3  /* valid but not implemented (dtype / head_dim combination) */
#define DLLM_ELAUNCH 4       /* a kernel launch failed */

/* Element types. */
#define DLLM_F32 0
#define DLLM_BF16 1
#define DLLM_FP8_E4M3 2      /* OCP E4M3 ("fn"): bias 7, max 448, no infinities */

/* Shape of one layer's cache. */
typedef struct dllm_cache_desc {
    int32_t batch;        /* B: sequences */
    int32_t num_kv_heads; /* Hkv */
    int32_t max_seq;      /* S: rows per sequence (prompt + response canvas) */
    int32_t head_dim;     /* D: 64 or 128 */
    int32_t kv_dtype;     /* DLLM_F32, DLLM_BF16 or DLLM_FP8_E4M3 */
    int32_t group_size;   /* FP8: values per scale; must equal head_dim.  Otherwise 0. */
} dllm_cache_desc;

/* A cache carved out of caller memory by dllm_cache_alloc. */
typedef struct dllm_cache {
    dllm_cache_desc desc;
    void *k;              /* device, [B, Hkv, S, D] of kv_dtype: K rows after RoPE */
    void *v;              /* device, [B, Hkv, S, D] of kv_dtype: V rows as projected */
    float *k_scale;       /* device, [B, Hkv, S] fp32, FP8 only (else NULL) */
    float *v_scale;       /* device, [B, Hkv, S] fp32, FP8 only (else NULL) */
} dllm_cache;

/* Bytes of one flat cache region for `d`: K, V and (FP8) the two scale arrays, each part
 * starting on a 256-byte boundary.  Returns 0 if `d` is invalid. */
DLLM_API size_t dllm_cache_bytes(const dllm_cache_desc *d);

/* Carve the flat preallocated cache (Flash-dLLM summary, batch paragraph) out of `base`
 * (device memory of at least dllm_cache_bytes(d) bytes, 256-byte aligned) and describe it
 * in `*out`.  Does not touch the memory: a first refresh over all rows (the prefill of a
 * block, LaCache workflow) fills it.
 * Errors: DLLM_EINVAL (null pointer, bad shape, misaligned base), DLLM_ESIZE (nbytes too
 * small), DLLM_EUNSUPPORTED (head_dim not 64/128, FP8 with group_size != head_dim). */
DLLM_API dllm_status dllm_cache_alloc(const dllm_cache_desc *d, void *base, size_t nbytes,
                             dllm_cache *out);

/* Refresh: gather, QKV projection, RoPE, cache scatter (the fused kernel of the
 * Flash-dLLM summary; the positions outside LaCache's invariant region).
 *   hidden       device, [B, S, H] of act_dtype: current hidden states (already normalised)
 *   hidden_size  H; a multiple of 256 (bf16) or 32 (fp32)
 *   act_dtype    DLLM_BF16 (cache BF16 or FP8) or DLLM_F32 (cache F32)
 *   refresh_idx  device, [B, n] int32: per sequence, the rows to recompute, sorted,
 *                unique, in [0, S)
 *   n            rows per sequence (0 <= n <= S); n = 0 enqueues nothing
 *   w_qkv        device, [(Hq + 2 Hkv) * D, H] of act_dtype: rows are Q heads, then K heads,
 *                then V heads, each D rows; no bias
 *   num_q_heads  Hq, a multiple of Hkv; query head h uses KV head h / (Hq / Hkv)
 *   rope_base    theta_i = rope_base^(-2i/D) for i < D/2; the pair (i, i + D/2) of each Q
 *                and K head of row s is rotated by s * theta_i (rotate-half convention)
 *   q_out        device, [B, n, Hq, D] of act_dtype: rotated queries of the refreshed rows
 *   workspace    device scratch of ws_bytes >= dllm_refresh_workspace_bytes(...) (may be NULL
 *                when that is 0): small steps split the projection over K across workgroups
 *                and keep the eight partial sums here; contents need no initialisation
 * Writes exactly the K/V rows (b, :, refresh_idx[b, i], :) (and their scales) and q_out;
 * every other cache row is left untouched.  Each output element is the fp32 sum of eight
 * fixed, equal K-partitions of H, each accumulated in ascending order and added in
 * partition order, so a row's result does not depend on n or on which other rows are
 * refreshed: a step reproduces, bit for bit, what a full refresh of all rows would store.
 * FP8 cache: per cache row, amax -> scale = amax / 448 (1 if amax = 0) -> codes = e4m3
 * (round to nearest even, saturating) of x / scale.
 * q_out must not alias hidden or the cache.
 * Errors: DLLM_EINVAL, DLLM_ESIZE (workspace too small), DLLM_EUNSUPPORTED, DLLM_ELAUNCH. */
DLLM_API dllm_status dllm_refresh_qkv_rope_scatter(const dllm_cache *c, const void *hidden,
                                          int32_t hidden_size, int32_t act_dtype,
                                          const int32_t *refresh_idx, int32_t n,
                                          const void *w_qkv, int32_t num_q_heads,
                                          float rope_base, void *q_out, void *workspace,
                                          size_t ws_bytes, void *stream);

/* Workspace bytes the refresh call needs for n rows per sequence (0 when the step runs as a
 * single fused kernel; 8 * B * n * (Hq + 2 Hkv) * D * 4 for the split-K path of small
 * bf16 steps, B * n <= 64).  Returns 0 also for invalid arguments. */
DLLM_API size_t dllm_refresh_workspace_bytes(const dllm_cache_desc *d, int32_t hidden_size,
                                             int32_t act_dtype, int32_t n,
                                             int32_t num_q_heads);

/* Workspace bytes dllm_block_attention needs for this shape: the split-KV partial states
 * (running max, normaliser and unnormalised output per query row and split) and, for the
 * mass pass, the log-sum-exp.  Returns 0 if the arguments are invalid. */
DLLM_API size_t dllm_attention_workspace_bytes(const dllm_cache_desc *d, int32_t num_q_heads,
                                      int32_t n);

/* Bidirectional block attention over the whole cache (no mask; Flash-Cache 3.1, LaCache
 * Problem Statement): for every sequence b, query row i < n and query head h,
 *   out[b, i, h] = sum_j softmax_j(<q[b, i, h], K[b, g, j]> * softmax_scale) V[b, g, j],
 *   g = h / (Hq / Hkv), j over all S cache rows.
 *   q            device, [B, n, Hq, D] of act_dtype (the refresh call's q_out)
 *   act_dtype    dtype of q and out: DLLM_BF16, or DLLM_F32 with an F32 cache
 *   softmax_scale  normally 1 / sqrt(D)
 *   out          device, [B, n, Hq, D] of act_dtype
 *   lse          device, [B, Hq, n] fp32 natural-log log-sum-exp, or NULL
 *   attn_mass    device, [B, Hq, S] fp32 or NULL: mass[b, h, j] = sum_i p[b, h, i, j], the
 *                column attention mass that ranks the most-attended tokens (a second pass
 *                after the log-sum-exp is known)
 *   workspace    device scratch of ws_bytes >= dllm_attention_workspace_bytes(...)
 * FP8 cache: K and V are dequantised with their row scales inside the kernel.
 * Results are deterministic: every reduction runs in a fixed order.
 * Errors: DLLM_EINVAL, DLLM_ESIZE (workspace too small), DLLM_EUNSUPPORTED (fp32 with
 * S > 8192), DLLM_ELAUNCH. */
DLLM_API dllm_status dllm_block_attention(const dllm_cache *c, const void *q, int32_t act_dtype,
                                 int32_t num_q_heads, int32_t n, float softmax_scale,
                                 void *out, float *lse, float *attn_mass, void *workspace,
                                 size_t ws_bytes, void *stream);

/* Attention-aware drift test and tracking update (Elastic-Cache core idea; Flash-dLLM
 * tracking budget).  Call after this step's refresh and attention.
 *   k            tracked tokens per (b, h), 1..64 (32 by default)
 *   gamma        threshold (0.9 by default)
 *   track_idx    device, [B, Hq, k] int32, in/out: on entry the previous step's tracked
 *                positions (-1 = empty slot); on exit (if attn_mass != NULL) the k
 *                positions with the largest mass (ties: lower position first), sorted
 *                ascending, -1 padded when S < k
 *   track_buf    device, [B, Hq, k, 2, D] of the cache dtype, in/out: the K and V rows of
 *                the tracked positions as saved when they were chosen; refilled from the
 *                current cache on exit (if attn_mass != NULL)
 *   attn_mass    device, [B, Hq, S] fp32 from dllm_block_attention, or NULL (no update)
 *   sigma_out    device, [B, Hq] fp32: sigma = <u, w> / (|u| |w|), u = the saved K||V rows
 *                of the previous tracked set, w = the same rows in the cache now (computed
 *                in fp64; no valid slot -> 1; |u||w| = 0 -> 1 if u == w else 0).  The fp64
 *                value is rounded to fp32 toward the side of gamma it lies on, so that
 *                sigma_out < gamma reproduces the fp64 decision exactly.
 *   refresh_out  device, [B] uint8: 1 iff min over heads of sigma < gamma, i.e. the later
 *                layers of sequence b should be recomputed.
 * Errors: DLLM_EUNSUPPORTED for FP8 caches. */
DLLM_API dllm_status dllm_drift_check(const dllm_cache *c, int32_t num_q_heads, int32_t k, float gamma,
                             int32_t *track_idx, void *track_buf, const float *attn_mass,
                             float *sigma_out, uint8_t *refresh_out, void *stream);

/* FP8 codec of the cache, exposed so the conversion can be checked element by element:
 * codes[i] = e4m3(x[i] / scale) (nearest even, saturating to +-448, NaN -> NaN) and
 * decoded[i] = decode(codes[i]) * scale.  x, codes, decoded: device arrays of n elements;
 * decoded may be NULL. */
DLLM_API dllm_status dllm_fp8_e4m3_roundtrip(const float *x, int64_t n, float scale, uint8_t *codes,
                                    float *decoded, void *stream);

/* Message describing the last error on this thread ("" if none). */
DLLM_API const char *dllm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLLM_CACHE_H */
