// C ABI of libsparse_attn.so: host-side validation and launch plumbing.
// Every check runs before anything is enqueued; see include/sparse_attn.h.
#include "sparse_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

sa_status fail(sa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sa_status ok() {
  g_err[0] = '\0';
  return SA_OK;
}

}  // namespace

sa_status sa::set_error(sa_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Routed query blocks (NVQ) and the end of the sparse rows for a valid
// (T, sink_start, mode); NVQ = -1 when pad mode lacks the context slots that
// complete the split block.
struct Split {
  int32_t nvb, nvq, rows_end;
};

Split split_rows(int32_t T, int32_t sink_start, int32_t mode) {
  const int32_t nvb = sink_start / sa::kBlock;
  if (mode == SA_VIDEO_TAIL_DENSE || sink_start % sa::kBlock == 0)
    return {nvb, nvb, nvb * sa::kBlock};
  if ((int64_t)T < (int64_t)(nvb + 1) * sa::kBlock) return {nvb, -1, -1};
  return {nvb, nvb + 1, sink_start};
}

// Shape checks shared by the three entry points.
sa_status check_shape(int32_t B, int32_t T, int32_t H, int32_t D, int32_t sink_start,
                      int32_t sink_tokens, int32_t mode) {
  if (D != sa::kHeadDim) return fail(SA_ERR_INVALID_ARG, "D must be 128 (got %d)", D);
  if (B <= 0 || T <= 0 || H <= 0)
    return fail(SA_ERR_INVALID_ARG, "B, T, H must be positive (got %d, %d, %d)", B, T, H);
  if (sink_start < 0 || sink_start > T)
    return fail(SA_ERR_INVALID_ARG, "sink_start must lie in [0, T] (got %d, T=%d)", sink_start,
                T);
  if ((int64_t)sink_start + sink_tokens != T)
    return fail(SA_ERR_INVALID_ARG, "sink_start + sink_tokens must equal T (%d + %d != %d)",
                sink_start, sink_tokens, T);
  if (mode != SA_VIDEO_TAIL_DENSE && mode != SA_VIDEO_TAIL_PAD)
    return fail(SA_ERR_INVALID_ARG, "video_tail_mode must be 0 (dense) or 1 (pad), got %d", mode);
  if (split_rows(T, sink_start, mode).nvq < 0)
    return fail(SA_ERR_INVALID_ARG,
                "pad mode needs T >= 64*(NVB+1) = %d so the context suffix completes the split "
                "video block (T=%d)",
                (sink_start / sa::kBlock + 1) * sa::kBlock, T);
  // every launch indexes workgroups with int and elements with int64
  const int64_t nb = (T + sa::kBlock - 1) / sa::kBlock;
  if ((int64_t)B * H * nb > INT32_MAX / 2)
    return fail(SA_ERR_UNSUPPORTED, "B*H*ceil(T/64) too large");
  // K/V tiles are addressed with 32-bit byte offsets inside one batch
  if ((int64_t)(T + sa::kBlock) * H * sa::kHeadDim * 2 > INT32_MAX)
    return fail(SA_ERR_UNSUPPORTED, "T*H*256 bytes per batch must stay below 2 GiB");
  return SA_OK;
}

sa_status check_bf16(const void *p, const char *name) {
  if (p == nullptr) return fail(SA_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned(p, 16)) return fail(SA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return SA_OK;
}

sa_status check_bias(const float *key_bias, int64_t numel, int32_t B, int32_t T) {
  if (key_bias == nullptr) return SA_OK;
  if (!aligned(key_bias, 4)) return fail(SA_ERR_INVALID_ARG, "key_bias must be 4-byte aligned");
  if (numel != (int64_t)B * T)
    return fail(SA_ERR_INVALID_ARG, "key_bias must hold exactly B*T = %lld floats (got %lld)",
                (long long)B * T, (long long)numel);
  return SA_OK;
}

sa_status check_scale(float softmax_scale, float *scale_log2) {
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(SA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  const double s = softmax_scale == 0.f ? 1.0 / std::sqrt((double)sa::kHeadDim) : softmax_scale;
  *scale_log2 = (float)(s * 1.4426950408889634);
  return SA_OK;
}

}  // namespace

extern "C" {

int32_t sa_num_blocks(int32_t T) { return T <= 0 ? 0 : (T + sa::kBlock - 1) / sa::kBlock; }

int32_t sa_num_sparse_blocks(int32_t T, int32_t sink_start) {
  if (sink_start < 0 || sink_start > T) return -1;
  return sink_start / sa::kBlock;
}

int32_t sa_topk_budget(int32_t nvb, float ratio) {
  if (!(ratio > 0.f && ratio <= 1.f)) return -1;
  if (nvb <= 0) return 0;
  const double k = std::ceil((double)ratio * (double)nvb - 1e-6);
  return k < 1.0 ? 1 : (int32_t)k;
}

int32_t sa_num_query_blocks(int32_t T, int32_t sink_start, int32_t video_tail_mode) {
  if (sink_start < 0 || sink_start > T) return -1;
  if (video_tail_mode != SA_VIDEO_TAIL_DENSE && video_tail_mode != SA_VIDEO_TAIL_PAD) return -1;
  return split_rows(T, sink_start, video_tail_mode).nvq;
}

int32_t sa_max_selected(int32_t T, int32_t sink_start, int32_t video_tail_mode, float ratio,
                        int32_t radius) {
  const int32_t nvq = sa_num_query_blocks(T, sink_start, video_tail_mode);
  const int32_t nvb = sa_num_sparse_blocks(T, sink_start);
  if (nvq < 0 || radius < 0) return -1;
  const int32_t budget = sa_topk_budget(nvb, ratio);
  if (budget < 0) return -1;
  if (nvq == 0) return 0;
  const int64_t local = (int64_t)budget + 2 * (int64_t)radius + 1;
  const int32_t routed = local < nvb ? (int32_t)local : nvb;
  return routed + (sa_num_blocks(T) - nvb);
}

size_t sa_route_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t sink_start,
                                int32_t video_tail_mode) {
  const int32_t nvq = sa_num_query_blocks(T, sink_start, video_tail_mode);
  const int32_t nvb = sa_num_sparse_blocks(T, sink_start);
  if (B <= 0 || H <= 0 || nvq <= 0) return 0;
  // query means in fp64 over NVQ, then key means in fp32 over NVB, each
  // rounded up to a multiple of 16 blocks
  const size_t nvq16 = ((size_t)nvq + 15) / 16 * 16;
  const size_t nvb16 = ((size_t)nvb + 15) / 16 * 16;
  return (size_t)B * (size_t)H * sa::kHeadDim * (nvq16 * sizeof(double) + nvb16 * sizeof(float));
}

size_t sa_dense_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t sink_start) {
  const int32_t nvb = sa_num_sparse_blocks(T, sink_start);
  if (B <= 0 || H <= 0 || T <= 0 || nvb < 0) return 0;
  return sa::dense_workspace_bytes(B, H, sa_num_blocks(T), nvb);
}

const char *sa_last_error(void) { return g_err; }

sa_status sa_device_info(int32_t device, int32_t *cu_count, int32_t *clock_khz) {
  if (cu_count == nullptr || clock_khz == nullptr)
    return fail(SA_ERR_INVALID_ARG, "cu_count and clock_khz must not be NULL");
  int cu = 0, clk = 0;
  hipError_t e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&clk, hipDeviceAttributeClockRate, device);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  *cu_count = cu;
  *clock_khz = clk;
  return ok();
}

}  // extern "C"

sa_status sa::check_route_args(const void *q, const void *k, int32_t B, int32_t T, int32_t H,
                               int32_t D, int32_t sink_start, int32_t sink_tokens,
                               int32_t video_tail_mode, float topk_ratio, int32_t local_radius,
                               const int32_t *block_idx, int32_t max_sel,
                               const int32_t *block_cnt, const float *route_scores) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, video_tail_mode);
  if (st != SA_OK) return st;
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  if (!(topk_ratio > 0.f && topk_ratio <= 1.f))
    return fail(SA_ERR_INVALID_ARG, "topk_ratio must lie in (0, 1]");
  if (local_radius < 0) return fail(SA_ERR_INVALID_ARG, "local_radius must be >= 0");
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  if ((int64_t)B * H > 65535)
    return fail(SA_ERR_UNSUPPORTED, "routing supports B*H up to 65535 (got %lld)",
                (long long)B * H);
  if (sp.nvb > sa::kMaxRouteBlocks)
    return fail(SA_ERR_UNSUPPORTED, "at most %d video blocks can be routed (got %d)",
                sa::kMaxRouteBlocks, sp.nvb);
  const int32_t need_sel =
      sa_max_selected(T, sink_start, video_tail_mode, topk_ratio, local_radius);
  if (max_sel < need_sel)
    return fail(SA_ERR_INVALID_ARG, "max_sel must be >= %d (got %d)", need_sel, max_sel);
  if (sp.nvq == 0) return SA_OK;
  if (block_idx == nullptr || block_cnt == nullptr)
    return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must not be NULL");
  if (!aligned(block_idx, 4) || !aligned(block_cnt, 4) ||
      (route_scores != nullptr && !aligned(route_scores, 4)))
    return fail(SA_ERR_INVALID_ARG, "block_idx, block_cnt, route_scores must be 4-byte aligned");
  return SA_OK;
}

extern "C" {

sa_status sparse_attn_route(const void *q, const void *k, int32_t B, int32_t T, int32_t H,
                            int32_t D, int32_t sink_start, int32_t sink_tokens,
                            int32_t video_tail_mode, float topk_ratio, int32_t local_radius,
                            int32_t *block_idx, int32_t max_sel, int32_t *block_cnt,
                            float *route_scores, void *workspace, size_t workspace_bytes,
                            void *stream) {
  sa_status st = sa::check_route_args(q, k, B, T, H, D, sink_start, sink_tokens, video_tail_mode,
                                      topk_ratio, local_radius, block_idx, max_sel, block_cnt,
                                      route_scores);
  if (st != SA_OK) return st;
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  const int32_t nvb = sp.nvb;
  const int32_t nb = sa_num_blocks(T);
  if (sp.nvq == 0) return ok();
  const size_t need_ws = sa_route_workspace_bytes(B, T, H, sink_start, video_tail_mode);
  if (workspace_bytes < need_ws)
    return fail(SA_ERR_WORKSPACE, "workspace must hold %zu bytes (got %zu)", need_ws,
                workspace_bytes);
  if (workspace == nullptr || !aligned(workspace, 16))
    return fail(SA_ERR_WORKSPACE, "workspace must be a 16-byte aligned device pointer");

  const int32_t budget = sa_topk_budget(nvb, topk_ratio);
  // a radius beyond NVB forces the same blocks as NVB (and keeps i + radius
  // inside int in the kernel)
  const int32_t radius = local_radius < nvb ? local_radius : nvb;
  double *qbar = static_cast<double *>(workspace);
  float *kbar = reinterpret_cast<float *>(qbar + (size_t)B * H * (((size_t)sp.nvq + 15) / 16 * 16) * sa::kHeadDim);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = sa::launch_pool(q, k, qbar, kbar, B, T, H, sp.nvq, nvb, sp.rows_end, s);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
  e = sa::launch_route(qbar, kbar, B, H, sp.nvq, nvb, nb, budget, radius, max_sel, block_idx,
                       block_cnt, route_scores, s);
  if (e != hipSuccess) return fail(SA_ERR_HIP, "route launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status sparse_attn_fwd(const void *q, const void *k, const void *v, int32_t B, int32_t T,
                          int32_t H, int32_t D, int32_t sink_start, int32_t sink_tokens,
                          int32_t video_tail_mode, const float *key_bias, int64_t key_bias_numel,
                          const int32_t *block_idx, const int32_t *block_cnt, int32_t max_sel,
                          float softmax_scale, void *out, float *lse, void *stream) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, video_tail_mode);
  if (st != SA_OK) return st;
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  if ((st = check_bf16(v, "v")) != SA_OK) return st;
  if ((st = check_bf16(out, "out")) != SA_OK) return st;
  if ((st = check_bias(key_bias, key_bias_numel, B, T)) != SA_OK) return st;
  float scale_log2 = 0.f;
  if ((st = check_scale(softmax_scale, &scale_log2)) != SA_OK) return st;
  if (lse != nullptr && !aligned(lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  if (sp.nvq == 0) return ok();
  if (block_idx == nullptr || block_cnt == nullptr)
    return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must not be NULL");
  if (!aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must be 4-byte aligned");
  if (max_sel <= 0) return fail(SA_ERR_INVALID_ARG, "max_sel must be positive");

  sa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.key_bias = key_bias;
  a.block_idx = block_idx;
  a.block_cnt = block_cnt;
  a.B = B;
  a.T = T;
  a.H = H;
  a.nb = sa_num_blocks(T);
  a.nvb = sp.nvb;
  a.nvq = sp.nvq;
  a.rows_end = sp.rows_end;
  a.max_sel = max_sel;
  a.scale_log2 = scale_log2;
  hipError_t e = sa::launch_attn_sparse(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "sparse attention launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status dense_sink_fwd(const void *q, const void *k, const void *v, int32_t B, int32_t T,
                         int32_t H, int32_t D, int32_t sink_start, int32_t sink_tokens,
                         int32_t video_tail_mode, const float *key_bias, int64_t key_bias_numel,
                         float softmax_scale, void *out, float *lse, void *workspace,
                         size_t workspace_bytes, void *stream) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, video_tail_mode);
  if (st != SA_OK) return st;
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  if ((st = check_bf16(v, "v")) != SA_OK) return st;
  if ((st = check_bf16(out, "out")) != SA_OK) return st;
  if ((st = check_bias(key_bias, key_bias_numel, B, T)) != SA_OK) return st;
  float scale_log2 = 0.f;
  if ((st = check_scale(softmax_scale, &scale_log2)) != SA_OK) return st;
  if (lse != nullptr && !aligned(lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  if (sp.rows_end == T) return ok();
  if (workspace_bytes > 0 && (workspace == nullptr || !aligned(workspace, 16)))
    return fail(SA_ERR_WORKSPACE, "workspace must be a 16-byte aligned device pointer");

  sa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.key_bias = key_bias;
  a.B = B;
  a.T = T;
  a.H = H;
  a.nb = sa_num_blocks(T);
  a.nvb = sp.nvb;
  a.nvq = sp.nvq;
  a.rows_end = sp.rows_end;
  a.max_sel = 0;
  a.scale_log2 = scale_log2;
  hipError_t e = sa::launch_attn_dense(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "dense attention launch: %s", hipGetErrorString(e));
  return ok();
}

// ---- Spark summaries and the approximate branch ---------------------------

size_t sa_anchor_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t sink_start) {
  if (B <= 0 || H <= 0 || sink_start <= 0 || sink_start > T) return 0;
  return sa::anchor_workspace_bytes(B, H, sink_start);
}

sa_status spark_global_anchor(const void *q, int32_t B, int32_t T, int32_t H, int32_t D,
                              int32_t sink_start, int32_t sink_tokens, void *anchor,
                              void *workspace, size_t workspace_bytes, void *stream) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, SA_VIDEO_TAIL_DENSE);
  if (st != SA_OK) return st;
  if (sink_start == 0) return fail(SA_ERR_INVALID_ARG, "the anchor needs sink_start >= 1 video rows");
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(anchor, "anchor")) != SA_OK) return st;
  const size_t need = sa_anchor_workspace_bytes(B, T, H, sink_start);
  if (workspace_bytes < need)
    return fail(SA_ERR_WORKSPACE, "workspace must hold %zu bytes (got %zu)", need, workspace_bytes);
  if (workspace == nullptr || !aligned(workspace, 16))
    return fail(SA_ERR_WORKSPACE, "workspace must be a 16-byte aligned device pointer");
  hipError_t e = sa::launch_anchor(q, workspace, anchor, B, T, H, sink_start,
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "anchor launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status spark_reweight(const void *anchors, const void *k, const void *v, int32_t B, int32_t P,
                         int32_t T, int32_t H, int32_t D, float softmax_scale, int32_t logmass_key,
                         void *ak, void *av, float *lm, void *stream) {
  sa_status st = check_shape(B, T, H, D, T, 0, SA_VIDEO_TAIL_DENSE);
  if (st != SA_OK) return st;
  if (P <= 0) return fail(SA_ERR_INVALID_ARG, "P (anchors) must be positive (got %d)", P);
  if ((int64_t)B * P * H * ((T + sa::kBlock - 1) / sa::kBlock) > INT32_MAX / 2)
    return fail(SA_ERR_UNSUPPORTED, "B*P*H*ceil(T/64) too large");
  if ((int64_t)B * P > 65535) return fail(SA_ERR_UNSUPPORTED, "B*P must stay below 65536 (launch grid)");
  if (logmass_key != 0 && logmass_key != 1)
    return fail(SA_ERR_INVALID_ARG, "logmass_key must be 0 (stored bf16 key) or 1 (pre-round key)");
  if ((st = check_bf16(anchors, "anchors")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  if ((st = check_bf16(v, "v")) != SA_OK) return st;
  if ((st = check_bf16(ak, "ak")) != SA_OK) return st;
  if ((st = check_bf16(av, "av")) != SA_OK) return st;
  if (lm == nullptr || !aligned(lm, 4))
    return fail(SA_ERR_INVALID_ARG, "lm must be a non-NULL 4-byte aligned pointer");
  float scale_log2 = 0.f;
  if ((st = check_scale(softmax_scale, &scale_log2)) != SA_OK) return st;
  const float scale =
      softmax_scale == 0.f ? (float)(1.0 / std::sqrt((double)sa::kHeadDim)) : softmax_scale;
  hipError_t e = sa::launch_reweight(anchors, k, v, ak, av, lm, B, P, T, H, scale, logmass_key,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "reweight launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status sparse_attn_fwd_spark(const void *q, const void *k, const void *v, int32_t B, int32_t T,
                                int32_t H, int32_t D, int32_t sink_start, int32_t sink_tokens,
                                int32_t video_tail_mode, const float *key_bias,
                                int64_t key_bias_numel, const int32_t *block_idx,
                                const int32_t *block_cnt, int32_t max_sel, const void *ak,
                                const void *av, const float *lm, float softmax_scale, void *out,
                                float *lse, void *stream) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, video_tail_mode);
  if (st != SA_OK) return st;
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  if ((st = check_bf16(v, "v")) != SA_OK) return st;
  if ((st = check_bf16(out, "out")) != SA_OK) return st;
  if ((st = check_bias(key_bias, key_bias_numel, B, T)) != SA_OK) return st;
  float scale_log2 = 0.f;
  if ((st = check_scale(softmax_scale, &scale_log2)) != SA_OK) return st;
  if (lse != nullptr && !aligned(lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  if (sp.nvq == 0) return ok();
  if (sp.nvb > sa::kMaxRouteBlocks)
    return fail(SA_ERR_UNSUPPORTED, "the approximate branch supports at most %d video blocks (got %d)",
                sa::kMaxRouteBlocks, sp.nvb);
  if (block_idx == nullptr || block_cnt == nullptr)
    return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must not be NULL");
  if (!aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must be 4-byte aligned");
  if (max_sel <= 0) return fail(SA_ERR_INVALID_ARG, "max_sel must be positive");
  if ((st = check_bf16(ak, "ak")) != SA_OK) return st;
  if ((st = check_bf16(av, "av")) != SA_OK) return st;
  if (lm == nullptr || !aligned(lm, 4))
    return fail(SA_ERR_INVALID_ARG, "lm must be a non-NULL 4-byte aligned pointer");

  sa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.key_bias = key_bias;
  a.block_idx = block_idx;
  a.block_cnt = block_cnt;
  a.B = B;
  a.T = T;
  a.H = H;
  a.nb = sa_num_blocks(T);
  a.nvb = sp.nvb;
  a.nvq = sp.nvq;
  a.rows_end = sp.rows_end;
  a.max_sel = max_sel;
  a.scale_log2 = scale_log2;
  a.sum_k = ak;
  a.sum_v = av;
  a.sum_lm = lm;
  hipError_t e = sa::launch_attn_sparse_spark(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(SA_ERR_HIP, "sparse attention (approximate branch) launch: %s", hipGetErrorString(e));
  return ok();
}

// ---- fused route ------------------------------------------------------------

sa_status sparse_attn_pool(const void *q, const void *k, int32_t B, int32_t T, int32_t H, int32_t D,
                           int32_t sink_start, int32_t sink_tokens, int32_t video_tail_mode,
                           void *workspace, size_t workspace_bytes, void *stream) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, video_tail_mode);
  if (st != SA_OK) return st;
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  if (sp.nvb > sa::kMaxRouteBlocks)
    return fail(SA_ERR_UNSUPPORTED, "at most %d video blocks can be routed (got %d)",
                sa::kMaxRouteBlocks, sp.nvb);
  if (sp.nvq == 0) return ok();
  const size_t need_ws = sa_route_workspace_bytes(B, T, H, sink_start, video_tail_mode);
  if (workspace_bytes < need_ws)
    return fail(SA_ERR_WORKSPACE, "workspace must hold %zu bytes (got %zu)", need_ws,
                workspace_bytes);
  if (workspace == nullptr || !aligned(workspace, 16))
    return fail(SA_ERR_WORKSPACE, "workspace must be a 16-byte aligned device pointer");
  double *qbar = static_cast<double *>(workspace);
  float *kbar = reinterpret_cast<float *>(qbar + (size_t)B * H * (((size_t)sp.nvq + 15) / 16 * 16) * sa::kHeadDim);
  hipError_t e = sa::launch_pool(q, k, qbar, kbar, B, T, H, sp.nvq, sp.nvb, sp.rows_end,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SA_ERR_HIP, "pool launch: %s", hipGetErrorString(e));
  return ok();
}

sa_status sparse_attn_fwd_fused(const void *q, const void *k, const void *v, int32_t B, int32_t T,
                                int32_t H, int32_t D, int32_t sink_start, int32_t sink_tokens,
                                int32_t video_tail_mode, float topk_ratio, int32_t local_radius,
                                const float *key_bias, int64_t key_bias_numel,
                                const void *workspace, size_t workspace_bytes, float softmax_scale,
                                void *out, float *lse, int32_t *block_idx, int32_t max_sel,
                                int32_t *block_cnt, void *stream) {
  sa_status st = check_shape(B, T, H, D, sink_start, sink_tokens, video_tail_mode);
  if (st != SA_OK) return st;
  if ((st = check_bf16(q, "q")) != SA_OK) return st;
  if ((st = check_bf16(k, "k")) != SA_OK) return st;
  if ((st = check_bf16(v, "v")) != SA_OK) return st;
  if ((st = check_bf16(out, "out")) != SA_OK) return st;
  if ((st = check_bias(key_bias, key_bias_numel, B, T)) != SA_OK) return st;
  float scale_log2 = 0.f;
  if ((st = check_scale(softmax_scale, &scale_log2)) != SA_OK) return st;
  if (lse != nullptr && !aligned(lse, 4)) return fail(SA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (!(topk_ratio > 0.f && topk_ratio <= 1.f))
    return fail(SA_ERR_INVALID_ARG, "topk_ratio must lie in (0, 1]");
  if (local_radius < 0) return fail(SA_ERR_INVALID_ARG, "local_radius must be >= 0");
  const Split sp = split_rows(T, sink_start, video_tail_mode);
  if (sp.nvb > sa::kMaxRouteBlocks)
    return fail(SA_ERR_UNSUPPORTED, "at most %d video blocks can be routed (got %d)",
                sa::kMaxRouteBlocks, sp.nvb);
  const int32_t need_sel = sa_max_selected(T, sink_start, video_tail_mode, topk_ratio, local_radius);
  if ((block_idx == nullptr) != (block_cnt == nullptr))
    return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must both be given or both be NULL");
  if (block_idx != nullptr) {
    if (max_sel < need_sel)
      return fail(SA_ERR_INVALID_ARG, "max_sel must be >= %d (got %d)", need_sel, max_sel);
    if (!aligned(block_idx, 4) || !aligned(block_cnt, 4))
      return fail(SA_ERR_INVALID_ARG, "block_idx and block_cnt must be 4-byte aligned");
  } else {
    max_sel = need_sel;
  }
  if (max_sel > sa::kMaxRouteBlocks)
    return fail(SA_ERR_UNSUPPORTED, "the fused route holds lists of at most %d blocks (need %d)",
                sa::kMaxRouteBlocks, max_sel);
  if (sp.nvq == 0) return ok();
  const size_t need_ws = sa_route_workspace_bytes(B, T, H, sink_start, video_tail_mode);
  if (workspace_bytes < need_ws)
    return fail(SA_ERR_WORKSPACE, "workspace must hold %zu bytes (got %zu)", need_ws,
                workspace_bytes);
  if (workspace == nullptr || !aligned(workspace, 16))
    return fail(SA_ERR_WORKSPACE, "workspace must be a 16-byte aligned device pointer");

  const double *qbar = static_cast<const double *>(workspace);
  const float *kbar = reinterpret_cast<const float *>(qbar + (size_t)B * H * (((size_t)sp.nvq + 15) / 16 * 16) * sa::kHeadDim);
  sa::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.key_bias = key_bias;
  a.B = B;
  a.T = T;
  a.H = H;
  a.nb = sa_num_blocks(T);
  a.nvb = sp.nvb;
  a.nvq = sp.nvq;
  a.rows_end = sp.rows_end;
  a.max_sel = max_sel;
  a.scale_log2 = scale_log2;
  a.qbar = qbar;
  a.kbar = kbar;
  a.budget = sa_topk_budget(sp.nvb, topk_ratio);
  a.radius = local_radius < sp.nvb ? local_radius : sp.nvb;
  a.list_out = block_idx;
  a.cnt_out = block_cnt;
  hipError_t e = sa::launch_attn_sparse_fused(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(SA_ERR_HIP, "sparse attention (fused route) launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
