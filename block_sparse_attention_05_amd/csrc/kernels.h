// Internal launcher interface between the C ABI (abi.cpp) and the gfx950
// kernels (pool.hip, route.hip, attn.hip).  Not installed, not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// Sets the thread's sa_last_error() text (printf format) and returns st.
sa_status set_error(sa_status st, const char *fmt, ...);
// Every host check of sparse_attn_route except the workspace (sets the
// error text on failure).
sa_status check_route_args(const void *q, const void *k, int32_t B, int32_t T, int32_t H, int32_t D,
                           int32_t sink_start, int32_t sink_tokens, int32_t video_tail_mode,
                           float topk_ratio, int32_t local_radius, const int32_t *block_idx,
                           int32_t max_sel, const int32_t *block_cnt, const float *route_scores);

constexpr int kBlock = 64;     // tokens per routing block
constexpr int kHeadDim = 128;  // head dimension
constexpr int kMaxRouteBlocks = 1024;  // widest per-row sort in the route kernel
// Longest list (max_sel) the paired-block attention kernel serves; longer
// lists take the one-block kernel.
constexpr int kMaxPairList = 512;
// Largest lists the paired kernel takes with the approximate branch: two
// fully disjoint lists plus one virtual pair per 64 video blocks fit its
// schedule of 2 * kMaxPairList entries.
constexpr int kMaxPairSparkList = kMaxPairList - kMaxRouteBlocks / 128;

// Means of the routed blocks: Q blocks [0, nvq) over rows below q_end (a
// split last block only over its real rows), K blocks [0, nvb), in the route
// kernel's operand order (query tiles ceil(nvq/16), key tiles ceil(nvb/16)).
hipError_t launch_pool(const void *q, const void *k, double *qbar, float *kbar,
                       int B, int T, int H, int nvq, int nvb, int q_end, hipStream_t stream);

// Route scores, Top-K and list emission for every (b, h, query block < nvq)
// against the key blocks [0, nvb).
hipError_t launch_route(const double *qbar, const float *kbar, int B, int H, int nvq, int nvb,
                        int nb, int budget, int radius, int max_sel, int32_t *block_idx,
                        int32_t *block_cnt, float *scores, hipStream_t stream);

struct AttnArgs {
  const void *q, *k, *v;      // bf16 [B, T, H, 128]
  void *out;                  // bf16 [B, T, H, 128]
  float *lse;                 // nullable fp32 [B, H, T]
  const float *key_bias;      // nullable fp32 [B, T], natural log
  const int32_t *block_idx;   // sparse only: [B, H, nvq, max_sel]
  const int32_t *block_cnt;   // sparse only: [B, H, nvq]
  int B, T, H, nb, nvb, max_sel;
  int nvq;                    // routed query blocks
  int rows_end;               // rows [0, rows_end) are sparse, [rows_end, T) dense
  float scale_log2;           // softmax_scale * log2(e)
  // approximate branch (nullable): one summary per (b, h, K/V block)
  const void *sum_k, *sum_v;  // bf16 [B, 1, H, nb, 128]
  const float *sum_lm;        // fp32 [B, 1, H, nb], natural log
  // fused route (nullable): pooled means in the route workspace layout,
  // Top-K budget and forced radius, optional copies of the lists
  const double *qbar;
  const float *kbar;
  int budget, radius;
  int32_t *list_out, *cnt_out;
};

// Sparse rows [0, rows_end) of query blocks [0, nvq) over their block lists.
hipError_t launch_attn_sparse(const AttnArgs &a, hipStream_t stream);
// The same plus one virtual key (sum_k, sum_v, additive logit sum_lm) per
// video block that a row's list skips.  Needs nvb <= kMaxRouteBlocks.
hipError_t launch_attn_sparse_spark(const AttnArgs &a, hipStream_t stream);
// Sparse rows with the route fused in: every workgroup scores its query
// block against the pooled key means and selects its own list (the route
// kernel's rule), then attends.  Needs nvb, max_sel <= kMaxRouteBlocks.
hipError_t launch_attn_sparse_fused(const AttnArgs &a, hipStream_t stream);
// Dense rows [rows_end, T) over all keys.  With a workspace of at least
// dense_workspace_bytes() the key range of each query block is split over
// dense_splits() workgroups whose partial results are merged by a second
// kernel; otherwise one workgroup walks all keys.
hipError_t launch_attn_dense(const AttnArgs &a, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);
int dense_splits(int B, int H, int nb, int nvb);
size_t dense_workspace_bytes(int B, int H, int nb, int nvb);

// Paired query blocks (attn_pair.hip): one workgroup serves query blocks
// 2p and 2p+1 of a (b, h) and loads a key tile once when both lists hold
// it.  Sparse rows (needs max_sel <= kMaxPairList), and the dense rows with
// nsplit key ranges (partials to part_o / part_ml when nsplit > 1).
hipError_t launch_attn_pair_sparse(const AttnArgs &a, hipStream_t stream);
// The same with the route inside (needs max_sel <= kMaxPairList, nvb <=
// kMaxRouteBlocks): every workgroup scores both query blocks against the
// pooled key means and selects their lists (the route kernel's rule).
hipError_t launch_attn_pair_fused(const AttnArgs &a, hipStream_t stream);
// The approximate branch on paired query blocks (needs max_sel <=
// kMaxPairSparkList, nvb <= kMaxRouteBlocks): the virtual tiles of A and B
// run as private pairs after the exact tiles.
hipError_t launch_attn_pair_spark(const AttnArgs &a, hipStream_t stream);
hipError_t launch_attn_pair_dense(const AttnArgs &a, float *part_o, float *part_ml, int nsplit,
                                  hipStream_t stream);
int dense_pair_splits(int B, int H, int nb, int nvb);

// Spark summaries (spark.hip).
// Global anchor: mean of the video rows [0, sink_start) of Q per (b, h),
// bf16 [B, 1, H, 128]; the workspace holds fp64 partial sums.
size_t anchor_workspace_bytes(int B, int H, int sink_start);
hipError_t launch_anchor(const void *q, void *workspace, void *anchor, int B, int T, int H,
                         int sink_start, hipStream_t stream);
// Virtual summaries of every 64-token K/V block for P anchors.
hipError_t launch_reweight(const void *anchors, const void *k, const void *v, void *ak, void *av,
                           float *lm, int B, int P, int T, int H, float scale, int pre_round,
                           hipStream_t stream);

}  // namespace sa
