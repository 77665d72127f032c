/*
 * sparse_attn.h - C ABI of the MI355X (gfx950) routed block-sparse attention
 * library (libsparse_attn.so).
 *
 * Operation (forward only).  Q, K, V are contiguous BF16 [B, T, H, 128]
 * tensors (page "Sol-Attn and Spark for MiniMax-H3", section Install).  The
 * first `sink_start` tokens are the target video grid; the remaining
 * `sink_tokens = T - sink_start` conditioning tokens are packed after it and
 * act as exact K/V sinks (same page, "H3 pipeline integration" and "Direct
 * Sol-Attn", where sol_attn takes sink_start=video_tokens and
 * sink_tokens=T-video_tokens).  Tokens are grouped into 64-token blocks
 * (same page, "Spark primitives").  With
 *     NB  = ceil(T / 64)        all blocks (the last may be partial),
 *     NVB = sink_start / 64     complete video blocks,
 * key blocks [0, NVB) are routed, and every block holding a token >= 64*NVB
 * is a sink block.  Where the video boundary splits block NVB
 * (sink_start % 64 != 0), `video_tail_mode` says which path its real video
 * rows take (same page, "H3 pipeline integration", the video tail mode
 * paragraph, and "Spark inference integration", last paragraph):
 *   SA_VIDEO_TAIL_DENSE (0, the pages' default): query blocks [0, NVB) are
 *     routed and rows [0, 64*NVB) take the sparse path; rows [64*NVB, T)
 *     (the split block and the context rows) take the dense path over all
 *     keys.
 *   SA_VIDEO_TAIL_PAD (1): the split block is routed too, so NVQ = NVB + 1
 *     query blocks; its non-video query slots count as holding the mean Q of
 *     its real rows, so its routing centroid is that mean.  Rows
 *     [0, sink_start) take the sparse path and only the context rows
 *     [sink_start, T) the dense one.  The context suffix must complete the
 *     split block: T >= 64*(NVB+1), else SA_ERR_INVALID_ARG.
 * With sink_start % 64 == 0 the two modes are the same (NVQ = NVB).  K/V are
 * the complete, unmodified sequence for both paths in both modes.
 *
 * A full call is sparse_attn_route + sparse_attn_fwd + dense_sink_fwd on one
 * stream.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The
 *    library allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls only enqueue work; nothing synchronises the host.
 *  - Every argument is validated on the host before anything is enqueued.
 *    A violation returns SA_ERR_INVALID_ARG (or SA_ERR_UNSUPPORTED /
 *    SA_ERR_WORKSPACE) and enqueues nothing; sa_last_error() then names the
 *    argument.  A launch failure returns SA_ERR_HIP.  Nothing aborts, retries
 *    or falls back to another implementation (page "Sol-Attn and Spark for
 *    MiniMax-H3", "Spark inference integration": kernel failures propagate to
 *    the caller with no error-triggered fallback).
 *  - Pointers to BF16 tensors must be 16-byte aligned; int32/fp32 pointers
 *    4-byte aligned.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_VIDEO_TAIL_DENSE = 0,
  SA_VIDEO_TAIL_PAD = 1
} sa_video_tail_mode;

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = 1,
  SA_ERR_UNSUPPORTED = 2,
  SA_ERR_WORKSPACE = 3,
  SA_ERR_HIP = 4
} sa_status;

/* ---- shape helpers: host-only, pure, no device access ------------------ */

/* NB = ceil(T / 64); 0 if T <= 0. */
int32_t sa_num_blocks(int32_t T);

/* NVB = sink_start / 64 (complete video blocks); -1 if sink_start is not in
 * [0, T]. */
int32_t sa_num_sparse_blocks(int32_t T, int32_t sink_start);

/* NVQ, the routed query blocks: NVB, or NVB + 1 in pad mode when the video
 * boundary splits block NVB.  -1 if sink_start is not in [0, T], the mode is
 * unknown, or pad mode lacks the context slots that complete the split block
 * (T < 64*(NVB+1)). */
int32_t sa_num_query_blocks(int32_t T, int32_t sink_start, int32_t video_tail_mode);

/* Fixed-ratio Top-K budget before clamping: max(1, ceil(ratio * nvb - 1e-6))
 * with the product in double (page "Sol-Attn and Spark for MiniMax-H3",
 * "Spark inference integration": native mean Top-K routing with ratio 0.1).
 * Returns 0 when nvb <= 0 and -1 when ratio is not in (0, 1]. */
int32_t sa_topk_budget(int32_t nvb, float ratio);

/* Longest exact list any query block can get:
 * min(NVB, budget + 2*radius + 1) + (NB - NVB); 0 when NVQ == 0; -1 on
 * invalid arguments. */
int32_t sa_max_selected(int32_t T, int32_t sink_start, int32_t video_tail_mode, float ratio,
                        int32_t radius);

/* Workspace bytes sparse_attn_route needs for the pooled means of Q and K:
 * B * H * 128 * (NVQ16 * 8 + NVB16 * 4) bytes, NVQ16 / NVB16 = NVQ / NVB
 * rounded up to a multiple of 16 (Q means kept as fp64 copies, K means as
 * fp32); 0 when NVQ <= 0. */
size_t sa_route_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t sink_start,
                                int32_t video_tail_mode);

/* Workspace bytes with which dense_sink_fwd splits the key range of each
 * dense query block over several workgroups (0 when it would not split).
 * The same in both video tail modes (the dense path walks blocks
 * [NVB, NB) in both). */
size_t sa_dense_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t sink_start);

/* Message of the last failed call made by this thread ("" if none). */
const char *sa_last_error(void);

/* Compute-unit count and peak shader clock (kHz) of HIP device `device`, for
 * quoting a device-derived MFMA peak beside the published one.  Returns
 * SA_OK, or SA_ERR_HIP (with sa_last_error() set) if the runtime query
 * fails; both pointers must be non-NULL host pointers (SA_ERR_INVALID_ARG
 * otherwise). */
sa_status sa_device_info(int32_t device, int32_t *cu_count, int32_t *clock_khz);

/* ---- routing ------------------------------------------------------------- */

/*
 * sparse_attn_route - pool, score and select the exact block list of every
 * video query block.
 *
 * Defined by: page "Sol-Attn and Spark for MiniMax-H3", "Spark inference
 * integration" (native mean Top-K routing, ratio 0.1, the packed route is
 * exported once so attention does not recompute route QK; the boundary
 * selection is an exact FP32 selection) and "H3 pipeline integration" (fixed
 * Top-K routing: radius 0 forces the self block, radius 1 the self block and
 * its two neighbours, added outside the Top-K budget); page "Add key bias to
 * chunked Sol-Attn producers", Tests and source audit (sink blocks are put
 * straight into the exact list and excluded from the routed candidates).
 *
 * Computes, for every batch b, head h and query block i < NVQ:
 *   qbar_i         = mean of the Q rows of block i below 64*NVB (dense mode)
 *                    or sink_start (pad mode): 64 rows, or the real video
 *                    rows of the split block; kbar_j = mean of the 64 K rows
 *                    of block j < NVB.  The fp64 sum is exact; the mean is
 *                    the fp64 quotient by the row count rounded to fp32
 *                    (correctly rounded for 64 rows);
 *   s_ij           = qbar_i . kbar_j for j < NVB, fp32 of a float64 dot
 *                    product (unscaled);
 *   F(i)           = { j : |j - i| <= local_radius } within [0, NVB) (for
 *                    the split block i = NVB: the video blocks within the
 *                    radius below it);
 *   R(i)           = the first min(budget, NVB - |F(i)|) blocks of
 *                    [0, NVB) \ F(i) ordered by (s_ij descending, j
 *                    ascending), -0.0 equal to +0.0;
 *   list(i)        = ascending R(i) u F(i) u [NVB, NB).
 *
 * q, k          bf16 [B, T, H, 128], contiguous.
 * D             must be 128.
 * sink_start    video tokens, 0 <= sink_start <= T; sink_tokens must equal
 *               T - sink_start.
 * video_tail_mode  SA_VIDEO_TAIL_DENSE or SA_VIDEO_TAIL_PAD (see the top of
 *               this file); the same value must be passed to
 *               sparse_attn_fwd and dense_sink_fwd.
 * topk_ratio    in (0, 1].  local_radius >= 0.
 * block_idx     int32 [B, H, NVQ, max_sel] out: ascending lists, padded -1.
 * max_sel       >= sa_max_selected(T, sink_start, video_tail_mode,
 *               topk_ratio, local_radius).
 * block_cnt     int32 [B, H, NVQ] out: list lengths.
 * route_scores  nullable; fp32 [B, H, NVQ, NVB] out: s_ij.
 * workspace     device scratch of workspace_bytes >=
 *               sa_route_workspace_bytes(B, T, H, sink_start,
 *               video_tail_mode), 16-byte aligned.  The pooled means are
 *               left there: first the Q means over NVQ16 blocks (fp64 copies
 *               of the fp32 means), then the K means over NVB16 blocks
 *               (fp32), NVQ16 / NVB16 = NVQ / NVB rounded up to a multiple of
 *               16, each in the operand order of the route kernel's fp64 MFMA:
 *               mean (b, h, block i, channel d) sits at piece
 *               [b][h][i / 16][s][16 * (d / 32) + i % 16], element d % 32 - w*s,
 *               where a piece holds w = 2 (Q) or 4 (K) consecutive steps and
 *               s = (d % 32) / w.  May be NULL when that size is 0.
 * Errors: SA_ERR_UNSUPPORTED when NVB > 1024 (per-row selection width) or
 * B*H > 65535 (launch grid).
 * With NVQ == 0 nothing is enqueued and SA_OK is returned.  With NVB == 0
 * and NVQ == 1 (pad mode, no complete video block) the one list is every
 * block [0, NB).
 */
sa_status sparse_attn_route(const void *q, const void *k,
                            int32_t B, int32_t T, int32_t H, int32_t D,
                            int32_t sink_start, int32_t sink_tokens,
                            int32_t video_tail_mode,
                            float topk_ratio, int32_t local_radius,
                            int32_t *block_idx, int32_t max_sel, int32_t *block_cnt,
                            float *route_scores,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/* ---- routing without allocation ---------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 */

/* Size of the library's static device scratch (per GPU, held until the
 * process ends): 32 MiB, enough for the pooled means of B*H*NVQ16 = 21845
 * query blocks with as many key blocks (H3: 12.4 MB; 24 heads of 512 blocks:
 * 18.9 MB). */
#define SA_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * sparse_attn_route_noalloc - sparse_attn_route with the pooled means kept
 * in the library's static device array of SA_STATIC_SCRATCH_BYTES instead of
 * a caller workspace.  Same arguments (minus workspace), same computation,
 * same outputs and errors as sparse_attn_route; the caller still owns q, k,
 * block_idx, block_cnt and route_scores.
 *
 * Allocates nothing: no hipMalloc / hipFree and no allocating library call.
 * The first call on a GPU looks up that GPU's copy of the array (the device
 * of `stream`, or the current device for the null stream).
 * Errors: SA_ERR_WORKSPACE when sa_route_workspace_bytes(B, T, H,
 * sink_start, video_tail_mode) exceeds SA_STATIC_SCRATCH_BYTES (checked
 * before any device access); SA_ERR_HIP if the lookup fails.
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (concurrent streams or host
 * threads) race and must be serialised by the caller.
 */
sa_status sparse_attn_route_noalloc(const void *q, const void *k,
                                    int32_t B, int32_t T, int32_t H, int32_t D,
                                    int32_t sink_start, int32_t sink_tokens,
                                    int32_t video_tail_mode,
                                    float topk_ratio, int32_t local_radius,
                                    int32_t *block_idx, int32_t max_sel, int32_t *block_cnt,
                                    float *route_scores,
                                    void *stream);

/* ---- attention ----------------------------------------------------------- */

/*
 * sparse_attn_fwd - exact attention of the sparse query rows (rows
 * [0, 64*NVB) in dense mode, [0, sink_start) in pad mode) over the keys of
 * their block lists.
 *
 * Defined by: page "Sol-Attn and Spark for MiniMax-H3", "Spark inference
 * integration" (K/V tiles streamed through one FP32 online-softmax/output
 * accumulator) and page "Add key bias to chunked Sol-Attn producers",
 * Summary and Contract (natural-log key_bias, float32 [B, T], converted once
 * to log2 units and consumed only by the exact branch; biased key blocks must
 * be sink-routed).
 *
 * For row t of query block i < NVQ and key j in a block of list(i), j < T:
 *   l_tj = softmax_scale * (q_t . k_j) + beta_j,
 *   beta_j = key_bias[b, j] if j >= 64*NVB (a sink key) else 0,
 *   out_t = sum_j softmax_j(l_t) v_j  (bf16, round to nearest even),
 *   lse_t = log sum_j exp(l_tj)       (natural log, fp32).
 * Evaluated as an online softmax in base 2 with fp32 accumulation on bf16
 * MFMA; P is rounded to bf16 for the PV product.
 *
 * key_bias      nullable fp32 [B, T], key_bias_numel must equal B*T.  The
 *               pages require biased keys to lie in sink blocks; this
 *               library reads the bias on sink keys only and ignores any
 *               value below 64*NVB (checking it would need a device
 *               reduction and a host wait).  The Python binding checks the
 *               precondition before calling and raises on a non-zero value
 *               there.
 * block_idx, block_cnt, max_sel  as produced by sparse_attn_route with the
 *               same B, T, H, sink_start, video_tail_mode ([B, H, NVQ, ...]).
 *               Entries outside [0, NB) are skipped and counts are clamped
 *               to max_sel.  Lists from elsewhere must have the same form:
 *               ascending and without repeats, so that the sink blocks
 *               [NVB, NB) come last and the partial block (if any) is the
 *               last entry.  Other lists give unspecified values in the
 *               sparse rows; every access still stays inside the tensors.
 * softmax_scale 0 selects 1/sqrt(128).
 * out           bf16 [B, T, H, 128]; only the sparse rows are written.
 * lse           nullable fp32 [B, H, T]; only the sparse rows are written.
 * With NVQ == 0 nothing is enqueued.
 */
sa_status sparse_attn_fwd(const void *q, const void *k, const void *v,
                          int32_t B, int32_t T, int32_t H, int32_t D,
                          int32_t sink_start, int32_t sink_tokens,
                          int32_t video_tail_mode,
                          const float *key_bias, int64_t key_bias_numel,
                          const int32_t *block_idx, const int32_t *block_cnt, int32_t max_sel,
                          float softmax_scale,
                          void *out, float *lse,
                          void *stream);

/*
 * dense_sink_fwd - dense attention of the dense query rows (rows [64*NVB, T)
 * in dense mode: context rows and a video block split by the boundary;
 * rows [sink_start, T) in pad mode: context rows only) over all T keys,
 * same formula, same bias rule and the same kernel as sparse_attn_fwd (page
 * "Sol-Attn and Spark for MiniMax-H3", "H3 pipeline integration": context
 * query rows are computed with dense attention over the complete K/V).
 *
 * out / lse     only the dense rows are written.  With none (64*NVB == T)
 *               nothing is enqueued.
 * workspace     optional device scratch.  With workspace_bytes >=
 *               sa_dense_workspace_bytes(B, T, H, sink_start) > 0 the keys of
 *               each dense query block are split over several workgroups
 *               and their partial softmax states merged by a second kernel
 *               (same result up to fp32 summation order); with less (or 0,
 *               workspace NULL) one workgroup walks all keys of a block.
 */
sa_status dense_sink_fwd(const void *q, const void *k, const void *v,
                         int32_t B, int32_t T, int32_t H, int32_t D,
                         int32_t sink_start, int32_t sink_tokens,
                         int32_t video_tail_mode,
                         const float *key_bias, int64_t key_bias_numel,
                         float softmax_scale,
                         void *out, float *lse,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/* ---- fused route ------------------------------------------------------------
 *
 * Defined by: page "Sol-Attn and Spark for MiniMax-H3", Spark inference
 * integration (Top-K selected inside each CTA, removing the external cutoff
 * tensor and pass; the selection is an exact FP32 boundary selection).
 */

/*
 * sparse_attn_pool - the pooling step of sparse_attn_route alone: the Q
 * means of query blocks [0, NVQ) and the K means of blocks [0, NVB), left in
 * the workspace in the layout sparse_attn_route documents.  Same arguments,
 * errors and workspace size as sparse_attn_route.  With NVQ == 0 nothing is
 * enqueued.
 */
sa_status sparse_attn_pool(const void *q, const void *k,
                           int32_t B, int32_t T, int32_t H, int32_t D,
                           int32_t sink_start, int32_t sink_tokens,
                           int32_t video_tail_mode,
                           void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * sparse_attn_fwd_fused - sparse_attn_fwd with the route inside the
 * attention kernel: every workgroup computes s_ij for its query block i from
 * the pooled means that sparse_attn_pool left in `workspace` (fp32 of the
 * fp64 dot product of the fp32 means, summed in a different order than the
 * route kernel, so a score can differ from it by one ulp at most) and
 * selects list(i) with the rule of sparse_attn_route, then attends.  Same
 * output as sparse_attn_route + sparse_attn_fwd up to such one-ulp score
 * differences, which can only change a selection at a near-tie.
 *
 * topk_ratio, local_radius   as for sparse_attn_route.
 * workspace     the workspace sparse_attn_pool filled (read only).
 * block_idx, block_cnt  nullable (both or neither): when given, the lists
 *               are written there too, [B, H, NVQ, max_sel] and [B, H, NVQ],
 *               in sparse_attn_route's format; max_sel >= sa_max_selected().
 *               When NULL, max_sel is ignored.
 * Other arguments as for sparse_attn_fwd.
 * Errors: SA_ERR_UNSUPPORTED when NVB > 1024 or a list can exceed 1024
 * blocks (the workgroup keeps the list in LDS).
 */
sa_status sparse_attn_fwd_fused(const void *q, const void *k, const void *v,
                                int32_t B, int32_t T, int32_t H, int32_t D,
                                int32_t sink_start, int32_t sink_tokens,
                                int32_t video_tail_mode,
                                float topk_ratio, int32_t local_radius,
                                const float *key_bias, int64_t key_bias_numel,
                                const void *workspace, size_t workspace_bytes,
                                float softmax_scale,
                                void *out, float *lse,
                                int32_t *block_idx, int32_t max_sel, int32_t *block_cnt,
                                void *stream);

/* ---- Spark virtual summaries and the approximate branch --------------------
 *
 * Defined by: page "Sol-Attn and Spark for MiniMax-H3", Spark primitives (the
 * spark_reweight paragraph: per anchor and physical 64-token K/V block,
 * softmax-weighted keys and values and lm = logsumexp(a.k/sqrt(128)) -
 * a.ak/sqrt(128), partial final blocks without padding) and Spark inference
 * integration (one global representative per head, the mean of all
 * target-video queries, stored in BF16; summaries merged with exact attention
 * in one FP32 online-softmax accumulator; log-mass against the stored BF16
 * summary key by default).  Optional: the Top-K path above does not use
 * them.
 */

/* Workspace bytes spark_global_anchor needs: B * H * ceil(sink_start / 256)
 * * 128 * 8 (fp64 partial sums); 0 if sink_start is not in [1, T]. */
size_t sa_anchor_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t sink_start);

/*
 * spark_global_anchor - anchor[b, 0, h, :] = bf16(fp32(mean of Q rows
 * [0, sink_start) of batch b, head h)); the fp64 sums are exact.
 *
 * q           bf16 [B, T, H, 128].  sink_start >= 1 (SA_ERR_INVALID_ARG
 *             otherwise), sink_tokens = T - sink_start.
 * anchor      bf16 [B, 1, H, 128] out, 16-byte aligned.
 * workspace   device scratch of >= sa_anchor_workspace_bytes(...) bytes,
 *             16-byte aligned.
 */
sa_status spark_global_anchor(const void *q, int32_t B, int32_t T, int32_t H, int32_t D,
                              int32_t sink_start, int32_t sink_tokens, void *anchor,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * spark_reweight - virtual summaries of every 64-token K/V block for P
 * anchors.  For anchor p and block j (keys [64j, min(64j+64, T))):
 *   z_t = scale * a_p . k_t,  w_t = softmax_t(z),
 *   ak  = sum_t w_t k_t,  av = sum_t w_t v_t   (bf16, round to nearest even),
 *   lm  = logsumexp_t(z) - scale * a_p . key  (fp32, natural log), where key
 *         is ak as stored (logmass_key 0, the pages' default) or the fp32
 *         weighted key before rounding (logmass_key 1).
 * fp32 arithmetic throughout.
 *
 * anchors     bf16 [B, P, H, 128], contiguous, 16-byte aligned.  P >= 1.
 * k, v        bf16 [B, T, H, 128].
 * softmax_scale  0 selects 1/sqrt(128); must equal the scale later given to
 *             sparse_attn_fwd_spark.
 * ak, av      bf16 [B, P, H, NB, 128] out (NB = ceil(T / 64)), 16-byte aligned.
 * lm          fp32 [B, P, H, NB] out.
 * Errors: SA_ERR_UNSUPPORTED when B*P > 65535 (launch grid).
 */
sa_status spark_reweight(const void *anchors, const void *k, const void *v,
                         int32_t B, int32_t P, int32_t T, int32_t H, int32_t D,
                         float softmax_scale, int32_t logmass_key,
                         void *ak, void *av, float *lm, void *stream);

/*
 * sparse_attn_fwd_spark - sparse_attn_fwd plus the approximate branch: every
 * video block j < NVB that list(i) leaves out joins the softmax of the rows
 * of query block i as one virtual key with key ak[b, 0, h, j], value
 * av[b, 0, h, j] and logit scale * q_t . ak + lm[b, 0, h, j].  Sink blocks
 * are always exact and never summarised (page "Add key bias to chunked
 * Sol-Attn producers", Tests and source audit: sink blocks are excluded from
 * the pooled tail).  Arguments as for sparse_attn_fwd, plus:
 *
 * ak, av      bf16 [B, 1, H, NB, 128] (one anchor), as spark_reweight writes.
 * lm          fp32 [B, 1, H, NB].
 * Errors: SA_ERR_UNSUPPORTED when NVB > 1024.
 */
sa_status sparse_attn_fwd_spark(const void *q, const void *k, const void *v,
                                int32_t B, int32_t T, int32_t H, int32_t D,
                                int32_t sink_start, int32_t sink_tokens,
                                int32_t video_tail_mode,
                                const float *key_bias, int64_t key_bias_numel,
                                const int32_t *block_idx, const int32_t *block_cnt,
                                int32_t max_sel,
                                const void *ak, const void *av, const float *lm,
                                float softmax_scale,
                                void *out, float *lse,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
