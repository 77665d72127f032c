// Block pooling: one fp32 mean vector per complete 64-token video block of Q
// and of K (the routing centroids of "native mean" Top-K routing, page
// "Sol-Attn and Spark for MiniMax-H3", Spark inference integration; pooled
// K sums come from the unweighted activations, page "Add key bias to chunked
// Sol-Attn producers", Summary).
//
// HBM-bound: every bf16 element of Q and K in video blocks is read once.
// A workgroup owns 16 consecutive blocks (one tile of the route kernel) of
// one (batch, head, Q|K); thread (blk, c8) walks the 64 tokens of block blk,
// reading 16 bytes (8 channels) per token, so each group of 16 threads reads
// one contiguous 256-byte head row.  Sums are kept in fp64: adding 64 bf16
// values is exact there, so the mean (a division by 64) is the correctly
// rounded fp32 value whatever the summation order.  The workgroup writes its
// tile of means whole, in the route kernel's operand order.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kPoolThreads = 256;

__global__ __launch_bounds__(kPoolThreads) void pool_means_kernel(
    const uint4 *__restrict__ q, const uint4 *__restrict__ k, double *__restrict__ qbar,
    float *__restrict__ kbar, int T, int H, int nvb) {
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const bool is_k = (blockIdx.z & 1) != 0;
  const int blk = threadIdx.x >> 4;       // block within the tile
  const int c8 = threadIdx.x & 15;        // 16-byte chunk of the head row
  const int i = 16 * tile + blk;          // video block
  if (i >= nvb) return;

  const int chunks = H * (kHeadDim / 8);  // 16-byte chunks per token row
  const uint4 *src = (is_k ? k : q) + ((int64_t)b * T + (int64_t)i * kBlock) * chunks + h * (kHeadDim / 8) + c8;
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

  const int d0 = 8 * c8;
  const double inv = 1.0 / kBlock;  // exact power of two
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] * inv);
  // Means are stored in the operand order of the route kernel's fp64 MFMA
  // (16 blocks per tile; contraction step st = d % 32 for lane 16*(d/32) +
  // block % 16): 16-byte pieces that a wavefront then reads contiguously.
  const int nt = (nvb + 15) >> 4;
  const int64_t tile_id = ((int64_t)b * H + h) * nt + tile;
  const int lane = 16 * (d0 >> 5) + blk;
  const int st0 = d0 & 31;
  if (is_k) {  // fp32, 4 steps per piece: [tile][st / 4][lane][st % 4]
#pragma unroll
    for (int x = 0; x < 2; ++x)
      reinterpret_cast<float4 *>(kbar)[(tile_id * 8 + (st0 >> 2) + x) * 64 + lane] =
          make_float4(m[4 * x], m[4 * x + 1], m[4 * x + 2], m[4 * x + 3]);
  } else {  // fp64 copies, 2 steps per piece: [tile][st / 2][lane][st % 2]
#pragma unroll
    for (int x = 0; x < 4; ++x)
      reinterpret_cast<double2 *>(qbar)[(tile_id * 16 + (st0 >> 1) + x) * 64 + lane] =
          make_double2((double)m[2 * x], (double)m[2 * x + 1]);
  }
}

}  // namespace

hipError_t launch_pool(const void *q, const void *k, double *qbar, float *kbar, int B, int T,
                       int H, int nvb, hipStream_t stream) {
  if (nvb <= 0) return hipSuccess;
  dim3 grid((nvb + 15) / 16, H, 2 * B);
  hipLaunchKernelGGL(pool_means_kernel, grid, dim3(kPoolThreads), 0, stream,
                     static_cast<const uint4 *>(q), static_cast<const uint4 *>(k), qbar, kbar, T,
                     H, nvb);
  return hipGetLastError();
}

}  // namespace sa
