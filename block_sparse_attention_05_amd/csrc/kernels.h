// Internal launcher interface between the C ABI (abi.cpp) and the gfx950
// kernels (pool.hip, route.hip, attn.hip).  Not installed, not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kBlock = 64;     // tokens per routing block
constexpr int kHeadDim = 128;  // head dimension
constexpr int kMaxRouteBlocks = 1024;  // widest per-row sort in the route kernel

// Mean of every complete 64-token video block of Q and K:
// qbar/kbar fp32 [B, H, nvb, 128].
hipError_t launch_pool(const void *q, const void *k, double *qbar, float *kbar,
                       int B, int T, int H, int nvb, hipStream_t stream);

// Route scores, Top-K and list emission for every (b, h, query block < nvb).
hipError_t launch_route(const double *qbar, const float *kbar, int B, int H, int nvb,
                        int nb, int budget, int radius, int max_sel, int32_t *block_idx,
                        int32_t *block_cnt, float *scores, hipStream_t stream);

struct AttnArgs {
  const void *q, *k, *v;      // bf16 [B, T, H, 128]
  void *out;                  // bf16 [B, T, H, 128]
  float *lse;                 // nullable fp32 [B, H, T]
  const float *key_bias;      // nullable fp32 [B, T], natural log
  const int32_t *block_idx;   // sparse only
  const int32_t *block_cnt;   // sparse only
  int B, T, H, nb, nvb, max_sel;
  float scale_log2;           // softmax_scale * log2(e)
};

// Sparse rows [0, 64*nvb) over their block lists.
hipError_t launch_attn_sparse(const AttnArgs &a, hipStream_t stream);
// Dense rows [64*nvb, T) over all keys.  With a workspace of at least
// dense_workspace_bytes() the key range of each query block is split over
// dense_splits() workgroups whose partial results are merged by a second
// kernel; otherwise one workgroup walks all keys.
hipError_t launch_attn_dense(const AttnArgs &a, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);
int dense_splits(int B, int H, int nb, int nvb);
size_t dense_workspace_bytes(int B, int H, int nb, int nvb);

}  // namespace sa
