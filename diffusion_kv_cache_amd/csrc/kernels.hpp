// Host-side launchers of the gfx950 kernels (internal to the library; the C ABI is in
// include/dllm_cache.h).  Each returns a hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dllm_cache.h"

namespace dllm {

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
  float* ws;             // split-K partials [8][M][N] (small-M path only)
};

// Rows (B * n) up to which a bf16 refresh takes the split-K path.
constexpr int kSplitKMaxRows = 64;
// Largest hidden size of the split-K path (its LDS slice is 32 x H/8 bf16).
constexpr int kSplitKMaxHidden = 16384;
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
};

// Shape of the attention launch for a problem: splits over S and the workspace they need.
struct AttnPlan {
  int qt;        // packed query rows per workgroup (32, 64 or 128)
  int splits;    // workgroups along S per (b, g, query tile)
  int kps;       // keys per split (multiple of 32)
  size_t part_bytes;  // workspace for split partials
};
AttnPlan plan_attention(int B, int n, int Hq, int Hkv, int S, int D, int act, int kind);

hipError_t launch_attention(const AttnArgs& a, const AttnPlan& p, hipStream_t s);
// Attention and column mass in one launch (one workgroup per (b, KV head)): taken when the
// mass is requested for a bf16 cache, one query head per KV head, n <= 32, and the batch's
// heads alone fill the GPU (the plan does not split keys).
bool attn_fused_fits(const AttnArgs& a, const AttnPlan& p);
hipError_t launch_attn_fused(const AttnArgs& a, hipStream_t s);
// Forward pass of the MFMA attention (bf16 queries; bf16 or FP8 cache), one launch.
template <int KIND, int D>
hipError_t launch_attn_fwd(const AttnArgs& a, const AttnPlan& p, int qtiles, hipStream_t s);

struct DriftArgs {
  const void* kc;
  const void* vc;
  int32_t* track_idx;    // [B, Hq, k]
  void* track_buf;       // [B, Hq, k, 2, D]
  const float* mass;     // [B, Hq, S] or null
  float* sigma;          // [B, Hq]
  uint8_t* refresh;      // [B]
  int B, Hq, Hkv, S, D, k, kind;
  float gamma;
};

hipError_t launch_drift(const DriftArgs& a, hipStream_t s);

hipError_t launch_fp8_roundtrip(const float* x, int64_t n, float scale, uint8_t* codes,
                                float* decoded, hipStream_t s);

}  // namespace dllm
