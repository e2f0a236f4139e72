// Host-side launchers of the gfx950 kernels (internal to the library; the C ABI is in
// include/dllm_cache.h).  Each returns a hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dllm_cache.h"

namespace dllm {

// Process-wide DLLM_OPT_* switches (dllm_set_options; initially from the environment).
int options();
void set_options(int flags);

struct RefreshArgs {
  const void* hidden;    // [B, S, H]
  const void* w;         // [N, H]
  const int32_t* idx;    // [B, n]
  void* q_out;           // [B, n, Hq, D]
  void* kc;              // [B, Hkv, S, D]
  void* vc;
  float* ks;             // [B, Hkv, S] (fp8)
  float* vs;
  int B, S, H, n, M, Hq, Hkv, D;
  int act;               // DLLM_F32 / DLLM_BF16
  int kind;              // cache dtype
  double rope_base;
  float* ws;             // split-K partials [4][M][N] (small-M path only)
  const int32_t* cu;     // [B + 1] row offsets of a variable-length batch, or null (n rows each);
                         // with cu, M is the capacity and cu[B] (read on the device) the rows
};

// Rows (B * n) up to which a bf16 refresh takes the split-K path.
constexpr int kSplitKMaxRows = 64;
// Largest hidden size of the split-K path (its LDS slice is 32 x H/4 bf16, 128 KB at most).
constexpr int kSplitKMaxHidden = 8192;
bool refresh_uses_splitk(int act, int M, int H);
size_t refresh_workspace_bytes(int act, int M, int N, int H);
size_t splitk_workspace_bytes(int M, int N);

// Picks the path and tile shape for (M, N, dtypes) and launches the refresh.
hipError_t launch_refresh(const RefreshArgs& a, hipStream_t s);
hipError_t launch_refresh_splitk(const RefreshArgs& a, float* part, hipStream_t s);

struct AttnArgs {
  const void* q;         // [B, n, Hq, D] act dtype
  void* out;             // [B, n, Hq, D] act dtype
  float* lse;            // [B, Hq, n] (never null: workspace is used when the caller's is)
  float* mass;           // [B, Hq, S] or null
  const void* kc;        // [B, Hkv, S, D]
  const void* vc;
  const float* ks;       // [B, Hkv, S] (fp8)
  const float* vs;
  float* part;           // split partials (workspace)
  int B, n, Hq, Hkv, S, D;
  int act, kind;
  float scale;           // softmax scale
  // Variable-length batches: query rows of sequence b are [cu[b], cu[b + 1]) of q and out
  // (n is then the largest count), its keys the first lens[b] cache rows; null: n rows and S
  // keys each.  T: all query rows (B * n without cu), or with cu the capacity of the packed
  // arrays (the rows present, cu[B], are read on the device).
  const int32_t* cu;
  const int32_t* lens;
  int T;
};

// Shape of the attention launch for a problem: splits over S and the workspace they need.
struct AttnPlan {
  int qt;        // packed query rows per workgroup (32, 64 or 128)
  int splits;    // workgroups along S per (b, g, query tile)
  int kps;       // keys per split (multiple of 32)
  size_t part_bytes;  // workspace for split partials
};
// n: query rows per sequence (the largest, for a variable-length batch); T: all query rows.
AttnPlan plan_attention(int B, int n, int Hq, int Hkv, int S, int D, int act, int kind, long long T);

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s);
// Attention and column mass in one launch (one workgroup per (b, KV head)): taken when the
// mass is requested for a bf16 cache, one query head per KV head, n <= 32, and the batch's
// heads alone fill the GPU (the plan does not split keys).
bool attn_fused_fits(const AttnArgs& a, const AttnPlan& p);
hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t s);
// Forward pass of the MFMA attention (bf16 queries; bf16 or FP8 cache), one launch.
template <int KIND, int D>
hipError_t launch_attn_fwd(const AttnArgs& a, const AttnPlan& p, int qtiles, hipStream_t s);

// Attention of every row with cached softmax statistics of the invariant rows (FACache).
struct FacArgs {
  void* q_cache;             // [B, S, Hq, D] bf16, in/out: cached queries of every row
  const void* q_blk;         // [B, n, Hq, D] bf16: this step's queries of the block rows
  const int32_t* block_start;  // [B]: first row of each sequence's block
  float* state;              // O~ [B, Hq, S, D] fp32, then (m2, l) [B, Hq, S, 2] fp32
  void* out;                 // [B, S, Hq, D] bf16
  float* lse;                // [B, Hq, S] or null
  const void* kc;            // [B, Hkv, S, D] bf16
  const void* vc;
  int B, S, n, Hq, Hkv, D;
  int build;                 // 1: first step of the block (state written), 0: state reused
  float scale;
};
hipError_t launch_facache(const FacArgs& a, hipStream_t s);

struct DriftArgs {
  const void* kc;
  const void* vc;
  int32_t* track_idx;    // [B, Hq, k]
  void* track_buf;       // [B, Hq, k, 2, D]
  const float* mass;     // [B, Hq, S] or null
  const float* ks;       // FP8: [B, Hkv, S] row scales of K and V (else null)
  const float* vs;
  float* sigma;          // [B, Hq]
  uint8_t* refresh;      // [B]
  // arrival words, one per sequence at a 128-byte stride (zero on entry, left zero), or null:
  // the decision is then taken by a second kernel
  unsigned long long* arrive;
  int B, Hq, Hkv, S, D, k, kind;
  float gamma;
};

constexpr int kDriftArriveStride = 16;  // 64-bit words between two sequences' arrival words

hipError_t launch_drift(const DriftArgs& a, hipStream_t s);

hipError_t launch_fp8_roundtrip(const float* x, int64_t n, float scale, uint8_t* codes,
                                float* decoded, hipStream_t s);

// Feature-similarity row choice (window + k least similar response rows per sequence).
struct SelectArgs {
  const void* cur;             // [B, S, H] act dtype
  const void* cached;          // [B, S, H]
  double* sim;                 // [B, S]: rows >= lo written
  const int32_t* window_start; // [B] (window > 0)
  int32_t* idx_out;            // [B, window + k]
  int B, S, H, act, lo, window, k;
};
hipError_t launch_similarity_select(const SelectArgs& a, hipStream_t s);
// Largest S of the selection (one workgroup of 1024 threads holds a sequence, 8 rows each).
constexpr int kSelectMaxSeq = 8192;

// Per-layer rows of the Elastic-Cache schedule, packed with offsets.
struct SchedArgs {
  const int32_t* idx;          // [B, n] step rows
  const int32_t* tracked;      // [B, m] or null (-1: empty)
  const uint8_t* full_in;      // [B] or null
  const uint8_t* decision;     // [B] or null
  uint8_t* full_out;           // [B] or null
  int32_t* rows;               // packed rows (capacity >= B * S)
  int32_t* cu;                 // [B + 1]
  int32_t* temp;               // [B, S] workspace
  int32_t* counts;             // [B] workspace
  int B, S, n, m;
};
hipError_t launch_schedule_rows(const SchedArgs& a, hipStream_t s);
// Largest S of the row schedule (one byte of LDS per row, 32 rows per thread).
constexpr int kScheduleMaxSeq = 32768;

hipError_t launch_copy_rows(const void* src, void* dst, int row_bytes, int B, int S,
                            const int32_t* rows, const int32_t* cu, int cap, hipStream_t s);

// Per-group FP8 linear layer: y [M, N] bf16 = dequant(x) dequant(w)^T.
struct Fp8GemmArgs {
  const uint8_t* xq;     // [M, K] activation codes
  const float* sxT;      // [K / 128, Mp] activation scales, group-major (rows >= M: 0)
  const uint8_t* wq;     // [N, K] weight codes
  const float* sw;       // [N / 128, K / 128] weight block scales
  void* y;               // [M, N] bf16
  float* part;           // [splits, M, N] fp32 split-K partials, or null (one split)
  int M, N, K, Mp;
  int kb_per_split;      // 128-groups of k per split
  int splits;
};
struct Fp8Plan {
  int tile;              // 0: 64 x 64 tiles, deep ring (M <= 64); 1: 128 x 128; 2: 256 x 128
  int Mp;                // M rounded up to 256 (the scale array's row pitch)
  int splits, kb_per_split;
  size_t part_bytes, codes_bytes, scales_bytes;
};
Fp8Plan plan_fp8_linear(int M, int N, int K);
// Largest K / 128 of the FP8 linear layer (its weight scales of one column block sit in LDS).
constexpr int kFp8MaxGroups = 512;
hipError_t launch_fp8_quant_groups(const void* x, int M, int K, int Mp, uint8_t* q, float* sT,
                                   bool zero_pad, hipStream_t s);
hipError_t launch_fp8_quant_blocks(const void* w, int N, int K, uint8_t* q, float* sc,
                                   hipStream_t s);
hipError_t launch_fp8_gemm(const Fp8GemmArgs& a, const Fp8Plan& p, hipStream_t s);

// The unfused refresh, for comparison: rotary embedding of rows in place, K/V row scatter.
hipError_t launch_rope_rows(void* y, int M, int ld, int heads, int D, const int32_t* pos,
                            double base, hipStream_t s);
hipError_t launch_scatter_kv_rows(const void* y, int ld, int k_col, int v_col, void* kc, void* vc,
                                  int B, int n, int Hkv, int S, int D, const int32_t* idx,
                                  hipStream_t s);

// Attainable matrix-core rate (a loop of independent MFMAs on register operands).
hipError_t launch_mfma_probe(int kind, int big, int workgroups, int iters, float* out, hipStream_t s);
// Attainable read-only stream rate (bytes a multiple of 16, buf 16-byte aligned).
hipError_t launch_read_probe(const void* buf, size_t bytes, int workgroups, uint32_t* out, hipStream_t s);

}  // namespace dllm
