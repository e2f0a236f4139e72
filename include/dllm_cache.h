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
 *   - Debug mode (option DLLM_OPT_DEBUG, below).  Before launching, the refresh call runs a
 *     device pass over the index list that checks every list is sorted, unique and in
 *     [0, S), copies its finding to the host and returns DLLM_EINVAL if a list breaks the
 *     contract; every call then synchronises its stream and reports launch failures.
 *     Without debug mode an index list that breaks the contract is undefined behaviour.
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
 *   hidden_size  H; a positive multiple of 256 (both activation dtypes)
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
 *                and keep the four partial sums here; contents need no initialisation
 * Writes exactly the K/V rows (b, :, refresh_idx[b, i], :) (and their scales) and q_out;
 * every other cache row is left untouched.  Each output element is the fp32 sum of four
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

/* Variable-length batches (Elastic-Cache paper card, deployment notes: a batch implementation
 * that concatenates variable-length sequences to keep the GPU busy).  The refreshed rows of
 * all sequences are packed without padding: sequence b's rows are packed rows
 * [cu_rows[b], cu_rows[b + 1]) of refresh_idx and q_out, with cu_rows[0] = 0 and
 * cu_rows[B] <= total_rows; a sequence may have no rows.  The kernels read cu_rows[B] on the
 * device, so the offsets may come from an earlier kernel on the same stream (a device-side
 * schedule, dllm_schedule_rows) and total_rows is only the capacity the launch is sized for;
 * packed rows past cu_rows[B] are not touched.  Everything else is as in
 * dllm_refresh_qkv_rope_scatter (same arithmetic and reduction order, so a row stores the same
 * bits as in a full refresh):
 *   refresh_idx  device, [total_rows] int32: per sequence sorted, unique, in [0, S)
 *   cu_rows      device, [B + 1] int32 row offsets
 *   total_rows   capacity of the packed arrays, >= cu_rows[B] (0 enqueues nothing)
 *   max_rows     the largest rows per sequence, <= S
 *   q_out        device, [total_rows, Hq, D] of act_dtype
 *   workspace    dllm_refresh_workspace_bytes(d, H, act, total_rows / B rounded up, Hq) is
 *                enough; exactly: what the fixed call needs for B * n = total_rows rows
 * Errors: those of dllm_refresh_qkv_rope_scatter; debug mode also checks cu_rows. */
DLLM_API dllm_status dllm_refresh_qkv_rope_scatter_varlen(const dllm_cache *c, const void *hidden,
                                                          int32_t hidden_size, int32_t act_dtype,
                                                          const int32_t *refresh_idx,
                                                          const int32_t *cu_rows,
                                                          int32_t total_rows, int32_t max_rows,
                                                          const void *w_qkv, int32_t num_q_heads,
                                                          float rope_base, void *q_out,
                                                          void *workspace, size_t ws_bytes,
                                                          void *stream);

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

/* Block attention of a variable-length batch (Elastic-Cache paper card, deployment notes):
 * the query rows of all sequences are packed without padding, sequence b's rows being packed
 * rows [cu_rows[b], cu_rows[b + 1]) of q and out, and sequence b attends over its own first
 * seq_lens[b] cache rows only:
 *   out[r, h] = sum_{j < seq_lens[b]} softmax_j(<q[r, h], K[b, g, j]> * softmax_scale) V[b, g, j]
 * for every packed row r of sequence b.
 *   q, out       device, [total_rows, Hq, D] bf16 (rows past cu_rows[B] are not touched)
 *   cu_rows      device, [B + 1] int32 row offsets (cu_rows[0] = 0, cu_rows[B] <= total_rows,
 *                read on the device as in dllm_refresh_qkv_rope_scatter_varlen)
 *   total_rows   capacity of the packed arrays
 *   seq_lens     device, [B] int32, each in [1, S], or NULL: every sequence attends over all S
 *   max_rows     the largest rows per sequence (<= S)
 *   lse          device, [total_rows * Hq] fp32 or NULL: sequence b's block at
 *                cu_rows[b] * Hq, laid out [Hq][rows of b]
 *   attn_mass    device, [B, Hq, S] fp32 or NULL; keys at or past seq_lens[b] get 0
 *   workspace    ws_bytes >= dllm_attention_varlen_workspace_bytes(...)
 * Caches: bf16 or FP8.  Errors: those of dllm_block_attention; DLLM_EUNSUPPORTED for fp32;
 * debug mode (DLLM_OPT_DEBUG) checks cu_rows, max_rows and seq_lens on the device first and
 * returns DLLM_EINVAL naming the first broken sequence.  Outside debug mode offsets that break
 * these rules are undefined behaviour. */
DLLM_API size_t dllm_attention_varlen_workspace_bytes(const dllm_cache_desc *d,
                                                      int32_t num_q_heads, int32_t total_rows,
                                                      int32_t max_rows);
DLLM_API dllm_status dllm_block_attention_varlen(const dllm_cache *c, const void *q,
                                                 int32_t act_dtype, int32_t num_q_heads,
                                                 const int32_t *cu_rows, const int32_t *seq_lens,
                                                 int32_t total_rows, int32_t max_rows,
                                                 float softmax_scale, void *out, float *lse,
                                                 float *attn_mass, void *workspace,
                                                 size_t ws_bytes, void *stream);

/* Block attention that allocates nothing and takes no workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Arguments and results are those of dllm_block_attention without
 * `workspace` / `ws_bytes`.  The split partial states (and the log-sum-exp when lse is NULL)
 * go to a library-owned device array of DLLM_NOALLOC_SCRATCH_BYTES bytes, one per GPU the
 * library runs on, held until the process ends.  Every call on one GPU shares that array,
 * so calls that overlap on one GPU (different streams or threads) race: issue them one
 * after another.  The call itself allocates and frees nothing.
 * Errors: those of dllm_block_attention, and DLLM_ESIZE when the shape needs more scratch
 * than DLLM_NOALLOC_SCRATCH_BYTES (dllm_attention_workspace_bytes gives the need). */
#define DLLM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
DLLM_API dllm_status dllm_block_attention_noalloc(const dllm_cache *c, const void *q,
                                                  int32_t act_dtype, int32_t num_q_heads,
                                                  int32_t n, float softmax_scale, void *out,
                                                  float *lse, float *attn_mass, void *stream);

/* Bytes of the FACache state of dllm_facache_attention for cache `d` and Hq query heads:
 * B * Hq * S * (D + 2) * 4.  Returns 0 for invalid arguments. */
DLLM_API size_t dllm_facache_state_bytes(const dllm_cache_desc *d, int32_t num_q_heads);

/* Attention of every row of a block step, with cached softmax statistics of the rows outside
 * the block (FACache; LaCache explainer, Technical Summary, Methodology 1 and Inference
 * Workflow).  For every sequence b the block is the rows [g0, g0 + n), g0 = block_start[b];
 * every other row is invariant within the block's denoising steps.  The call computes, for
 * every row i < S and query head h,
 *   out[b, i, h] = sum_j softmax_j(<q[b, i, h], K[b, g, j]> * softmax_scale) V[b, g, j]
 * over all S rows j (no mask), where q of a block row is q_block[b, i - g0, h] and q of any
 * other row is q_cache[b, i, h].
 *   q_cache      device, [B, S, Hq, D] bf16, in/out: the queries of every row (after RoPE);
 *                the block rows are overwritten with q_block
 *   q_block      device, [B, n, Hq, D] bf16: this step's queries of the block rows (the
 *                refresh call's q_out for refresh_idx = the block)
 *   block_start  device, [B] int32: g0 per sequence; clamped to [0, S - n]
 *   fa_state     device, dllm_facache_state_bytes(...) bytes, 16-byte aligned, in/out: for
 *                every invariant row (b, h, i), the online-softmax state over the invariant
 *                keys: O~ [B, Hq, S, D] fp32 (the unnormalised output), then (m2, l)
 *                [B, Hq, S, 2] fp32, where m2 is a running maximum of the logits in log2
 *                units (the logits times log2(e)) and l the normaliser relative to 2^m2;
 *                O~ / l is the attention output over the invariant keys and
 *                (m2 + log2 l) ln 2 their log-sum-exp.  Rows of the block are not written.
 *   build        1 at the first step of a block: everything is computed and fa_state
 *                written; 0 at later steps of the same block (same g0, same invariant rows
 *                and keys): a tile of 32 invariant (row, head) pairs skips every invariant
 *                key and starts from fa_state; tiles holding block rows are computed in full.
 *   out          device, [B, S, Hq, D] bf16
 *   lse          device, [B, Hq, S] fp32 natural log-sum-exp, or NULL
 * Only bf16 caches (the first layer, where the state is kept, runs in 16-bit precision).
 * Results are deterministic.  A reuse step whose invariant rows or keys changed since the
 * build step returns stale results for those rows (the caller's contract).
 * Errors: DLLM_EINVAL, DLLM_EUNSUPPORTED (cache not bf16), DLLM_ELAUNCH. */
DLLM_API dllm_status dllm_facache_attention(const dllm_cache *c, void *q_cache,
                                            const void *q_block, const int32_t *block_start,
                                            int32_t n, int32_t num_q_heads, float softmax_scale,
                                            float *fa_state, int32_t build, void *out,
                                            float *lse, void *stream);

/* Attention-aware drift test and tracking update (Elastic-Cache core idea; Flash-dLLM
 * tracking budget).  Call after this step's refresh and attention.
 *   k            tracked tokens per (b, h), 1..64 (32 by default)
 *   gamma        threshold (0.9 by default)
 *   track_idx    device, [B, Hq, k] int32, in/out: on entry the previous step's tracked
 *                positions (-1 = empty slot); on exit (if attn_mass != NULL) the k
 *                positions with the largest mass (ties: lower position first), sorted
 *                ascending, -1 padded when S < k
 *   track_buf    device, dllm_track_buffer_bytes(desc, Hq, k) bytes, 16-byte aligned,
 *                in/out: the K and V rows of the tracked positions as saved when they were
 *                chosen; refilled from the current cache on exit (if attn_mass != NULL).
 *                bf16 / fp32 caches: [B, Hq, k, 2, D] of the cache dtype.  FP8 caches: the
 *                codes [B, Hq, k, 2, D] uint8, then the rows' scales [B, Hq, k, 2] fp32; a
 *                row's values are code * scale (LaCache Methodology 2), compared in fp64.
 *   attn_mass    device, [B, Hq, S] fp32 from dllm_block_attention, or NULL (no update)
 *   sigma_out    device, [B, Hq] fp32: sigma = <u, w> / (|u| |w|), u = the saved K||V rows
 *                of the previous tracked set, w = the same rows in the cache now (computed
 *                in fp64; no valid slot -> 1; |u||w| = 0 -> 1 if u == w else 0).  The fp64
 *                value is rounded to fp32 toward the side of gamma it lies on, so that
 *                sigma_out < gamma reproduces the fp64 decision exactly.
 *   refresh_out  device, [B] uint8: 1 iff min over heads of sigma < gamma, i.e. the later
 *                layers of sequence b should be recomputed.
 *   workspace    device, >= dllm_drift_workspace_bytes(B) bytes, 8-byte aligned, or NULL.
 *                With a workspace the decision is taken in the same launch (one arrival
 *                word per sequence, 128 bytes apart); the words must be zero when the
 *                workspace is first used (fill it with zeros once after allocating it) and
 *                every call leaves them zero.  Calls that share a workspace must not overlap
 *                in time (same stream, or ordered by events).  NULL: a second kernel takes
 *                the decision (no state).
 * Errors: DLLM_EINVAL; DLLM_ESIZE (workspace too small); DLLM_EUNSUPPORTED for an update
 * with S above 16384 and for S * head_dim of 2^31 or more. */
DLLM_API size_t dllm_track_buffer_bytes(const dllm_cache_desc *d, int32_t num_q_heads, int32_t k);
DLLM_API size_t dllm_drift_workspace_bytes(int32_t batch);
DLLM_API dllm_status dllm_drift_check(const dllm_cache *c, int32_t num_q_heads, int32_t k, float gamma,
                             int32_t *track_idx, void *track_buf, const float *attn_mass,
                             float *sigma_out, uint8_t *refresh_out, void *workspace,
                             size_t ws_bytes, void *stream);

/* ---- The layer schedule: which rows each layer refreshes, decided on the device ---- */

/* Rows each sequence refreshes at this step, chosen by feature similarity (dLLM-Cache record,
 * abstract: partial response updates guided by feature similarity) on top of a window of live
 * rows (Elastic-Cache card, core idea):
 *   sim[b, j]    = <x, y> / (|x| |y|) for x = hidden_cur[b, j], y = hidden_cached[b, j], in fp64
 *                  (both rows zero -> 1, exactly one zero -> 0), for the response rows j >= lo
 *   idx_out[b]   = the window rows [window_start[b], window_start[b] + window) together with
 *                  the k rows of [lo, S) outside the window of lowest sim (ties: lower row
 *                  first), ascending
 *   batch, max_seq  B and S; S <= 8192
 *   hidden_size  H, a multiple of 8 (bf16) or 4 (fp32)
 *   act_dtype    DLLM_BF16 or DLLM_F32: dtype of hidden_cur and hidden_cached
 *   hidden_cur, hidden_cached  device, [B, S, H]: this step's input features and the features
 *                the rows' cache entries were last computed from
 *   lo           first response row, 0 <= lo < S
 *   window_start device, [B] int32, each in [0, S - window]; may be NULL when window = 0
 *   window, k    >= 0 with window + k <= S - lo
 *   idx_out      device, [B, window + k] int32
 *   sim_out      device, [B, S] fp64, or NULL (the workspace then holds it); rows below lo are
 *                not written
 *   workspace    ws_bytes >= dllm_similarity_select_workspace_bytes(B, S) when sim_out is
 *                NULL, else unused
 * Deterministic.  Errors: DLLM_EINVAL, DLLM_EUNSUPPORTED (S above 8192), DLLM_ESIZE,
 * DLLM_ELAUNCH. */
DLLM_API size_t dllm_similarity_select_workspace_bytes(int32_t batch, int32_t max_seq);
DLLM_API dllm_status dllm_similarity_select(int32_t batch, int32_t max_seq, int32_t hidden_size,
                                            int32_t act_dtype, const void *hidden_cur,
                                            const void *hidden_cached, int32_t lo,
                                            const int32_t *window_start, int32_t window, int32_t k,
                                            int32_t *idx_out, double *sim_out, void *workspace,
                                            size_t ws_bytes, void *stream);

/* Rows one layer refreshes under the Elastic-Cache schedule (card, core idea: when the drift
 * test fires at layer l, layers l + 1 .. L are recomputed; the tracked tokens are recomputed
 * with the step rows so the test compares fresh rows):
 *   full_out[b] = full_in[b] | decision[b] (either may be NULL: 0)
 *   sequence b's rows: all S rows if full_out[b], else the union of idx[b, 0..n) and the
 *   entries of tracked[b, 0..m) in [0, S) (-1 marks an empty slot), ascending; packed in
 *   sequence order into rows_out with offsets cu_out [B + 1], ready for
 *   dllm_refresh_qkv_rope_scatter_varlen and dllm_block_attention_varlen on the same stream
 *   (capacity B * S, max_rows S).  Everything stays on the device.
 *   idx          device, [B, n] int32 (entries outside [0, S) are skipped), n >= 0
 *   tracked      device, [B, m] int32 or NULL (dllm_drift_check's track_idx, m = Hq * k)
 *   full_in, decision, full_out  device, [B] uint8 (full_out may alias full_in; the drift
 *                check's refresh_out is a decision)
 *   rows_out     device, [capacity] int32, capacity >= B * S
 *   cu_out       device, [B + 1] int32
 *   workspace    ws_bytes >= dllm_schedule_rows_workspace_bytes(B, S); S <= 32768
 * Errors: DLLM_EINVAL, DLLM_EUNSUPPORTED (S above 32768), DLLM_ESIZE, DLLM_ELAUNCH. */
DLLM_API size_t dllm_schedule_rows_workspace_bytes(int32_t batch, int32_t max_seq);
DLLM_API dllm_status dllm_schedule_rows(int32_t batch, int32_t max_seq, const int32_t *idx,
                                        int32_t n, const int32_t *tracked, int32_t m,
                                        const uint8_t *full_in, const uint8_t *decision,
                                        uint8_t *full_out, int32_t *rows_out, int32_t capacity,
                                        int32_t *cu_out, void *workspace, size_t ws_bytes,
                                        void *stream);

/* dst[b, rows[r]] = src[b, rows[r]] for the packed rows r < cu_rows[B] of a variable-length
 * batch (read on the device): after a layer's refresh, the refreshed rows' cached features
 * become the current ones.  src, dst: device [B, S, row_bytes / elem] arrays, row_bytes a
 * positive multiple of 16; rows, cu_rows as in dllm_refresh_qkv_rope_scatter_varlen, capacity
 * >= cu_rows[B]. */
DLLM_API dllm_status dllm_copy_rows_varlen(int32_t batch, int32_t max_seq, int32_t row_bytes,
                                           const void *src, void *dst, const int32_t *rows,
                                           const int32_t *cu_rows, int32_t capacity,
                                           void *stream);

/* One layer of one denoising step under the Elastic-Cache schedule with the dLLM-Cache
 * partial refresh, enqueued on `stream` with no host synchronisation (the decisions stay on
 * the device).  In order:
 *   1. step_rows = dllm_similarity_select(hidden_cur, hidden_feat, lo, window_start, window,
 *      k_select)
 *   2. full |= decision; rows / cu_rows = dllm_schedule_rows(step_rows, track_idx, full):
 *      every row of a sequence flagged at an earlier layer, else its step rows with its
 *      tracked rows
 *   3. dllm_refresh_qkv_rope_scatter_varlen of those rows from hidden_cur into the cache; q
 *   4. dllm_block_attention_varlen of q over each sequence's whole cache, with mass
 *   5. dllm_drift_check (sigma, decision = this layer's drift test; tracking update)
 *   6. dllm_copy_rows_varlen: the refreshed rows' features in hidden_feat become hidden_cur's
 * Call it for layers 1 .. L in order with the same `full` and `decision` arrays, both zeroed
 * before the first layer of a step.  Packed arrays have capacity B * S rows (rows past
 * cu_rows[B] are not written).  bf16 activations and a bf16 cache; S <= 8192.
 * Errors: as the six calls; a failing stage leaves the earlier ones enqueued. */
typedef struct dllm_layer_step {
  const void *hidden_cur;       /* [B, S, H] bf16: this step's input states of the layer */
  void *hidden_feat;            /* [B, S, H] bf16, in/out: features the cache rows came from */
  const void *w_qkv;            /* [(Hq + 2 Hkv) * D, H] bf16 */
  const int32_t *window_start;  /* [B], each in [0, S - window] (NULL if window = 0) */
  int32_t *track_idx;           /* [B, Hq, k_track], in/out (dllm_drift_check) */
  void *track_buf;              /* [B, Hq, k_track, 2, D] bf16, in/out */
  uint8_t *full;                /* [B], in/out: sequences that refresh every row */
  uint8_t *decision;            /* [B], in: the previous layer's drift decision; out: this one's */
  int32_t *step_rows;           /* [B, window + k_select] out */
  int32_t *rows;                /* [B * S] out: packed refreshed rows */
  int32_t *cu_rows;             /* [B + 1] out */
  void *q;                      /* [B * S, Hq, D] bf16 out */
  void *out;                    /* [B * S, Hq, D] bf16 out */
  float *lse;                   /* [B * S * Hq] out, or NULL */
  float *attn_mass;             /* [B, Hq, S] out */
  float *sigma;                 /* [B, Hq] out */
  int32_t hidden_size, num_q_heads, lo, window, k_select, k_track;
  float rope_base, softmax_scale, gamma;
} dllm_layer_step;
DLLM_API size_t dllm_layer_step_workspace_bytes(const dllm_cache_desc *d, int32_t hidden_size,
                                                int32_t num_q_heads);
DLLM_API dllm_status dllm_elastic_layer_step(const dllm_cache *c, const dllm_layer_step *a,
                                             void *workspace, size_t ws_bytes, void *stream);

/* ---- Per-group FP8 linear layer (LaCache Technical Summary, Methodology 2: FP8 for the
 * FFN linear layers, one scale per 1 x 128 activation group and per 128 x 128 weight block) */

/* Weights [N, K] bf16 (device) -> codes [N, K] uint8 (e4m3) and scales [N / 128, K / 128]
 * fp32: per 128 x 128 block, scale = amax / 448 in fp32 (an all-zero block: 1) and code =
 * e4m3(w / scale), the quotient formed in fp32 (nearest even, saturating).  N and K multiples
 * of 128; all pointers 16-byte aligned.  Done once per weight matrix. */
DLLM_API dllm_status dllm_fp8_quantize_weight(const void *w, int32_t N, int32_t K,
                                              uint8_t *codes, float *scales, void *stream);

/* Activations [M, K] bf16 -> codes [M, K] uint8 and scales_t [K / 128, pitch] fp32 (group-
 * major: the scale of row m, group kb at scales_t[kb * pitch + m]; rows M .. pitch - 1 get 0),
 * one scale per row and 128-column group, same rule as the weights.  pitch >= M; K a multiple
 * of 128. */
DLLM_API dllm_status dllm_fp8_quantize_activations(const void *x, int32_t M, int32_t K,
                                                   uint8_t *codes, float *scales_t,
                                                   int32_t pitch, void *stream);

/* y [M, N] bf16 = dequant(x) dequant(w)^T: the activations x [M, K] bf16 are quantised in
 * 1 x 128 groups (as dllm_fp8_quantize_activations, into the workspace), then multiplied
 * with the FP8 weights on the FP8 matrix cores: for each 128-group kb the exact e4m3 product
 * is summed in fp32 and scaled by x_scale[m, kb] * w_scale[n / 128, kb], groups added in
 * ascending order in fp32 (for small M the groups are split into contiguous ranges whose fp32
 * sums are added in range order), and the result rounded to bf16.
 *   x            device, [M, K] bf16; M >= 0 (0 enqueues nothing), K a multiple of 128
 *   w_codes, w_scales  from dllm_fp8_quantize_weight, N a multiple of 128
 *   y            device, [M, N] bf16
 *   workspace    ws_bytes >= dllm_fp8_linear_workspace_bytes(M, N, K)
 * K <= 65536; M * K and N * K below 2^32.  Deterministic.
 * Errors: DLLM_EINVAL, DLLM_ESIZE, DLLM_ELAUNCH. */
DLLM_API size_t dllm_fp8_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);
DLLM_API dllm_status dllm_fp8_linear(const void *x, int32_t M, int32_t K, const uint8_t *w_codes,
                                     const float *w_scales, int32_t N, void *y, void *workspace,
                                     size_t ws_bytes, void *stream);

/* ---- The unfused refresh, for comparison with the fused call (Flash-dLLM news summary,
 * memory paragraph: projection, rotary embedding and cache write as separate kernels, each a
 * round trip through HBM).  With y = gathered hidden rows x W_qkv^T computed by any GEMM
 * ([B * n, ld] bf16, row m = b * n + i; columns Q heads | K heads | V heads):
 *   dllm_rope_rows        rotates, in place, the pairs (i, i + D/2) of the first `heads` head
 *                         columns of every row m at position pos[m] (the same rotation as the
 *                         fused call: theta_i = rope_base^(-2i/D), rotate-half); bf16
 *   dllm_scatter_kv_rows  copies, for every row m = b * n + i and KV head g, the D values at
 *                         columns k_col + g * D and v_col + g * D into the cache rows
 *                         (b, g, refresh_idx[b, i]) of K and V; every other cache row is left
 *                         as it is.  bf16 cache; ld, k_col, v_col multiples of 8; y 16-byte
 *                         aligned; debug mode checks refresh_idx as the refresh call does.
 * Errors: DLLM_EINVAL, DLLM_EUNSUPPORTED, DLLM_ELAUNCH. */
DLLM_API dllm_status dllm_rope_rows(void *y, int32_t M, int32_t ld, int32_t heads,
                                    int32_t head_dim, const int32_t *pos, float rope_base,
                                    void *stream);
DLLM_API dllm_status dllm_scatter_kv_rows(const dllm_cache *c, const void *y, int32_t ld,
                                          int32_t k_col, int32_t v_col,
                                          const int32_t *refresh_idx, int32_t n, void *stream);

/* Attainable matrix-core rate, a microbenchmark for the roofline report: `workgroups`
 * workgroups of four waves, each wave chaining `iters` rounds of independent MFMAs on
 * register operands, no memory traffic in the loop.  tile 16: eight 16x16 chains
 * (DLLM_BF16: 16x16x32; DLLM_FP8_E4M3: 16x16x128 e4m3), 2 * 16 * 16 * K * 8 flops per wave and
 * round; tile 32: four 32x32 chains (32x32x16 bf16, 32x32x64 e4m3), 2 * 32 * 32 * K * 4.
 * out: device, [workgroups * 4] fp32 (one value per wave, meaningless, written so the work is
 * kept).  Errors: DLLM_EINVAL, DLLM_ELAUNCH. */
DLLM_API dllm_status dllm_mfma_rate_probe(int32_t kind, int32_t tile, int32_t workgroups,
                                          int32_t iters, float *out, void *stream);

/* Attainable read-only stream rate, the bandwidth counterpart of the probe above: reads the
 * `bytes` bytes at buf once (device memory, 16-byte aligned, bytes a non-negative multiple of
 * 16) with `workgroups` workgroups of 256 threads and writes no more than
 * out[0 .. workgroups): device, the XOR of the 32-bit words each workgroup read (so the XOR
 * of all of out is the XOR of every word of the buffer, and the read can be checked).
 * Errors: DLLM_EINVAL, DLLM_ELAUNCH. */
DLLM_API dllm_status dllm_read_rate_probe(const void *buf, int64_t bytes, int32_t workgroups,
                                          uint32_t *out, void *stream);

/* FP8 codec of the cache, exposed so the conversion can be checked element by element:
 * codes[i] = e4m3(x[i] / scale) (nearest even, saturating to +-448, NaN -> NaN) and
 * decoded[i] = decode(codes[i]) * scale.  x, codes, decoded: device arrays of n elements;
 * decoded may be NULL. */
DLLM_API dllm_status dllm_fp8_e4m3_roundtrip(const float *x, int64_t n, float scale, uint8_t *codes,
                                    float *decoded, void *stream);

/* Process-wide switches, for debugging and testing.  Their initial value is read once from
 * the environment (DLLM_DEBUG=1 sets DLLM_OPT_DEBUG, DLLM_GEMM_WIDE_OFFSETS=1 sets
 * DLLM_OPT_WIDE_OFFSETS); afterwards only dllm_set_options changes them.
 *   DLLM_OPT_DEBUG         index lists checked on the device before the refresh, and every
 *                          call synchronises its stream and reports launch failures
 *   DLLM_OPT_WIDE_OFFSETS  the refresh of more than 64 rows addresses its operands with 64-bit
 *                          per-lane pointers, the form it otherwise takes only when the hidden
 *                          states or the weights span 4 GB or more (same results)
 * dllm_set_options(flags) replaces the switches (unknown bits are ignored) and returns the
 * previous value.  Calls already enqueued are not affected. */
#define DLLM_OPT_DEBUG 1
#define DLLM_OPT_WIDE_OFFSETS 2
DLLM_API int32_t dllm_set_options(int32_t flags);

/* Message describing the last error on this thread ("" if none). */
DLLM_API const char *dllm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLLM_CACHE_H */
