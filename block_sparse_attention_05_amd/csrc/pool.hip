// Block pooling: one fp32 mean vector per complete 64-token video block of Q
// and of K (the routing centroids of "native mean" Top-K routing, page
// "Sol-Attn and Spark for MiniMax-H3", Spark inference integration; pooled
// K sums come from the unweighted activations, page "Add key bias to chunked
// Sol-Attn producers", Summary).
//
// HBM-bound: every bf16 element of Q and K in video blocks is read once.
// One thread owns one 16-byte chunk (8 channels) of one (batch, head) row and
// walks the 64 tokens of its block; a wavefront reads 1 KiB of contiguous
// row per token, so every load is fully coalesced.  Sums are kept in fp64:
// adding 64 bf16 values is exact there, so the mean (a division by 64) is the
// correctly rounded fp32 value whatever the summation order.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kPoolThreads = 256;

__global__ __launch_bounds__(kPoolThreads) void pool_means_kernel(
    const uint4 *__restrict__ q, const uint4 *__restrict__ k, float *__restrict__ qbar,
    float *__restrict__ kbar, int T, int H, int nvb) {
  const int chunks = H * (kHeadDim / 8);  // 16-byte chunks per token row
  const int c = blockIdx.x * kPoolThreads + threadIdx.x;
  const int i = blockIdx.y;               // video block
  const int b = blockIdx.z >> 1;
  const bool is_k = (blockIdx.z & 1) != 0;
  if (c >= chunks) return;

  const uint4 *src = (is_k ? k : q) + ((int64_t)b * T + (int64_t)i * kBlock) * chunks + c;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;

#pragma unroll 16
  for (int t = 0; t < kBlock; ++t) {
    const uint4 w = src[(int64_t)t * chunks];
    acc[0] += (double)bf16_lo(w.x);
    acc[1] += (double)bf16_hi(w.x);
    acc[2] += (double)bf16_lo(w.y);
    acc[3] += (double)bf16_hi(w.y);
    acc[4] += (double)bf16_lo(w.z);
    acc[5] += (double)bf16_hi(w.z);
    acc[6] += (double)bf16_lo(w.w);
    acc[7] += (double)bf16_hi(w.w);
  }

  const int h = c / (kHeadDim / 8);
  const int d0 = (c % (kHeadDim / 8)) * 8;
  float *dst = (is_k ? kbar : qbar) + (((int64_t)b * H + h) * nvb + i) * kHeadDim + d0;
  const double inv = 1.0 / kBlock;  // exact power of two
  float4 lo, hi;
  lo.x = (float)(acc[0] * inv);
  lo.y = (float)(acc[1] * inv);
  lo.z = (float)(acc[2] * inv);
  lo.w = (float)(acc[3] * inv);
  hi.x = (float)(acc[4] * inv);
  hi.y = (float)(acc[5] * inv);
  hi.z = (float)(acc[6] * inv);
  hi.w = (float)(acc[7] * inv);
  reinterpret_cast<float4 *>(dst)[0] = lo;
  reinterpret_cast<float4 *>(dst)[1] = hi;
}

}  // namespace

hipError_t launch_pool(const void *q, const void *k, float *qbar, float *kbar, int B, int T,
                       int H, int nvb, hipStream_t stream) {
  if (nvb <= 0) return hipSuccess;
  const int chunks = H * (kHeadDim / 8);
  dim3 grid((chunks + kPoolThreads - 1) / kPoolThreads, nvb, 2 * B);
  hipLaunchKernelGGL(pool_means_kernel, grid, dim3(kPoolThreads), 0, stream,
                     static_cast<const uint4 *>(q), static_cast<const uint4 *>(k), qbar, kbar, T,
                     H, nvb);
  return hipGetLastError();
}

}  // namespace sa
