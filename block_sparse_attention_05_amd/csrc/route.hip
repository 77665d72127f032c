// Route: pooled block scores, fixed-ratio Top-K and exact-list emission.
//
// Page "Sol-Attn and Spark for MiniMax-H3", Spark inference integration:
// the route QK of pooled means is computed once, outside attention, with an
// exact FP32 boundary selection.  H3 pipeline integration: forced self /
// neighbour blocks are added outside the Top-K budget.  Page "Add key bias to
// chunked Sol-Attn producers", Tests and source audit: sink blocks go straight
// into the exact list and are never routed candidates.
//
// One workgroup (8 wavefronts) serves 16 query blocks of one (b, h).  Query
// blocks are the nvq routed ones: the nvb complete video blocks and, in the
// pad video tail mode, block nvb, split by the video boundary (first page,
// H3 pipeline integration); it is routed like the others, its forced
// neighbours being the video blocks within the radius below it.
//  1. scores s_ij for its 16 rows against every key block j < nvb on fp64
//     MFMA (v_mfma_f64_16x16x4f64), one 16-key tile per accumulator.
//     fp32 x fp32 products are exact in fp64, so the fp64 dot product
//     rounded once to fp32 is the fp32 score of the exact value (up to fp64
//     rounding of the sum, whose order differs from a plain loop).  Scores go
//     to LDS.
//  2. per row (two per wavefront), the k best candidates under (score desc,
//     index asc) by a most-significant-bit-first radix select on
//     order-preserving 32-bit score keys: one ballot count per bit halves the
//     bucket that holds the k-th key, starting below the bits shared by all
//     candidates and stopping as soon as the bucket is taken whole; ties left
//     at the last bit go to the lowest block indices.
//  3. a ballot/popcount scan emits selected and forced blocks in ascending
//     order, then the sink blocks [nvb, nb), then -1 padding.
#include "device_util.h"
#include "kernels.h"
#include "select.h"

namespace sa {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteRows = 16;  // query blocks per workgroup (one MFMA tile)

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Score tiles: query rows 16*rb .. +15 against key tiles t = wave, wave +
// kRouteWaves, ...  MFMA lane l holds A[l%16][l/16] = q[16rb + l%16][d] and
// B[l/16][l%16] = k[16t + l%16][d] with d = 32*(l/16) + step (the 128-term
// contraction is summed in that order); D register r of lane l is the score
// of row 4r + l/16 and key 16t + l%16.  The means arrive in exactly this
// operand order (see the pooling kernel), so every load is contiguous across
// the wavefront.  Rows and keys past nvb hold unused values that only reach
// unused rows and columns of D.
__device__ __forceinline__ void route_scores_tile(const double2 *__restrict__ qt,
                                                  const float4 *__restrict__ kt, int nt,
                                                  float *sc, int ld, int lane, int wave) {
  const int g = lane >> 4, c = lane & 15;
  for (int t = wave; t < nt; t += kRouteWaves) {
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // 16 contraction steps at a time
      double a[16];
      float bk[16];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const double2 v = qt[(8 * half + x) * 64 + lane];
        a[2 * x] = v.x;
        a[2 * x + 1] = v.y;
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float4 v = kt[((int64_t)t * 8 + 4 * half + x) * 64 + lane];
        bk[4 * x] = v.x;
        bk[4 * x + 1] = v.y;
        bk[4 * x + 2] = v.z;
        bk[4 * x + 3] = v.w;
      }
#pragma unroll
      for (int st = 0; st < 16; st += 2) {  // two independent chains
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[st], (double)bk[st], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(a[st + 1], (double)bk[st + 1], acc1, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[(4 * r + g) * ld + 16 * t + c] = (float)(acc0[r] + acc1[r]);
  }
}

template <int E>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const double *__restrict__ qbar, const float *__restrict__ kbar, int H, int nvq, int nvb,
    int nb, int budget, int radius, int max_sel, int32_t *__restrict__ block_idx,
    int32_t *__restrict__ block_cnt, float *__restrict__ scores_out) {
  constexpr int ld = 64 * E;  // LDS score row stride (floats)
  extern __shared__ __align__(16) float sc[];  // [kRouteRows][ld]

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * kRouteRows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int ntq = (nvq + 15) >> 4;  // query and key tiles
  const int ntk = (nvb + 15) >> 4;
  route_scores_tile(reinterpret_cast<const double2 *>(qbar) + ((int64_t)bh * ntq + blockIdx.x) * 16 * 64,
                    reinterpret_cast<const float4 *>(kbar) + (int64_t)bh * ntk * 8 * 64, ntk, sc, ld,
                    lane, wave);
  __syncthreads();

  for (int rr = wave; rr < kRouteRows; rr += kRouteWaves) {
    const int i = i0 + rr;
    if (i >= nvq) break;  // wave-uniform
    const int cnt = select_and_emit<E>(sc + rr * ld, i, nvb, nb, budget, radius, max_sel,
                                       block_idx + ((int64_t)bh * nvq + i) * max_sel,
                                       scores_out != nullptr ? scores_out + ((int64_t)bh * nvq + i) * nvb : nullptr,
                                       lane);
    if (lane == 0) block_cnt[(int64_t)bh * nvq + i] = cnt;
  }
}

template <int E>
hipError_t launch_route_e(const double *qbar, const float *kbar, int B, int H, int nvq, int nvb,
                          int nb, int budget, int radius, int max_sel, int32_t *block_idx,
                          int32_t *block_cnt, float *scores, hipStream_t stream) {
  dim3 grid((nvq + kRouteRows - 1) / kRouteRows, B * H);
  const size_t lds = (size_t)kRouteRows * 64 * E * sizeof(float);
  hipLaunchKernelGGL((route_kernel<E>), grid, dim3(kRouteThreads), lds, stream, qbar, kbar, H,
                     nvq, nvb, nb, budget, radius, max_sel, block_idx, block_cnt, scores);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const double *qbar, const float *kbar, int B, int H, int nvq, int nvb,
                        int nb, int budget, int radius, int max_sel, int32_t *block_idx,
                        int32_t *block_cnt, float *scores, hipStream_t stream) {
  if (nvq <= 0) return hipSuccess;
#define SA_ROUTE_E(E)                                                                       \
  launch_route_e<E>(qbar, kbar, B, H, nvq, nvb, nb, budget, radius, max_sel, block_idx, \
                    block_cnt, scores, stream)
  if (nvb <= 64) return SA_ROUTE_E(1);
  if (nvb <= 128) return SA_ROUTE_E(2);
  if (nvb <= 192) return SA_ROUTE_E(3);
  if (nvb <= 256) return SA_ROUTE_E(4);
  if (nvb <= 512) return SA_ROUTE_E(8);
  if (nvb <= kMaxRouteBlocks) return SA_ROUTE_E(16);
#undef SA_ROUTE_E
  return hipErrorInvalidValue;
}

}  // namespace sa
