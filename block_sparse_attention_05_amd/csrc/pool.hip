// Block pooling: one fp32 mean vector per routed video block of Q and K (the
// routing centroids of "native mean" Top-K routing, page "Sol-Attn and Spark
// for MiniMax-H3", Spark inference integration; pooled K sums come from the
// unweighted activations, page "Add key bias to chunked Sol-Attn producers",
// Summary).  Key blocks are the complete video blocks.  Query blocks are the
// same, plus, in the pad video tail mode, the block split by the video
// boundary, whose centroid is the mean of its real video rows only: pad mode
// fills its other query slots with exactly that mean (first page, H3
// pipeline integration).
//
// HBM-bound: every bf16 element of Q and K in routed blocks is read once.
// A workgroup owns 16 consecutive blocks (one tile of the route kernel) of
// one (batch, head, Q|K); thread (blk, c8) walks the rows of block blk,
// reading 16 bytes (8 channels) per token, so each group of 16 threads reads
// one contiguous 256-byte head row.  Sums are kept in fp64: adding up to 64
// bf16 values is exact there.  The mean is the fp64 quotient by the row
// count rounded to fp32; for 64 rows the division is exact, so that is the
// correctly rounded mean whatever the summation order.  The workgroup writes
// its tile of means whole, in the route kernel's operand order.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kPoolThreads = 256;

__global__ __launch_bounds__(kPoolThreads) void pool_means_kernel(
    const uint4 *__restrict__ q, const uint4 *__restrict__ k, double *__restrict__ qbar,
    float *__restrict__ kbar, int T, int H, int nvq, int nvb, int q_end) {
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z >> 1;
  const bool is_k = (blockIdx.z & 1) != 0;
  const int blk = threadIdx.x >> 4;       // block within the tile
  const int c8 = threadIdx.x & 15;        // 16-byte chunk of the head row
  const int i = 16 * tile + blk;          // routed block
  const int nblk = is_k ? nvb : nvq;
  if (i >= nblk) return;
  // rows of the block: 64, or the real video rows of a split query block
  const int rows = is_k || q_end - i * kBlock >= kBlock ? kBlock : q_end - i * kBlock;

  const int chunks = H * (kHeadDim / 8);  // 16-byte chunks per token row
  const uint4 *src = (is_k ? k : q) + ((int64_t)b * T + (int64_t)i * kBlock) * chunks + h * (kHeadDim / 8) + c8;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;

  auto add = [&](const uint4 w) {
    acc[0] += (double)bf16_lo(w.x);
    acc[1] += (double)bf16_hi(w.x);
    acc[2] += (double)bf16_lo(w.y);
    acc[3] += (double)bf16_hi(w.y);
    acc[4] += (double)bf16_lo(w.z);
    acc[5] += (double)bf16_hi(w.z);
    acc[6] += (double)bf16_lo(w.w);
    acc[7] += (double)bf16_hi(w.w);
  };
  if (rows == kBlock) {  // two batches of 32 loads in flight
    uint4 w[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) w[t] = src[(int64_t)t * chunks];
#pragma unroll
    for (int t = 0; t < 32; ++t) add(w[t]);
#pragma unroll
    for (int t = 0; t < 32; ++t) w[t] = src[(int64_t)(t + 32) * chunks];
#pragma unroll
    for (int t = 0; t < 32; ++t) add(w[t]);
  } else {
    for (int t = 0; t < rows; ++t) add(src[(int64_t)t * chunks]);
  }

  const int d0 = 8 * c8;
  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] / (double)rows);
  // Means are stored in the operand order of the route kernel's fp64 MFMA
  // (16 blocks per tile; contraction step st = d % 32 for lane 16*(d/32) +
  // block % 16): 16-byte pieces that a wavefront then reads contiguously.
  const int nt = (nblk + 15) >> 4;
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
                       int H, int nvq, int nvb, int q_end, hipStream_t stream) {
  const int n = nvq > nvb ? nvq : nvb;
  if (n <= 0) return hipSuccess;
  dim3 grid((n + 15) / 16, H, 2 * B);
  hipLaunchKernelGGL(pool_means_kernel, grid, dim3(kPoolThreads), 0, stream,
                     static_cast<const uint4 *>(q), static_cast<const uint4 *>(k), qbar, kbar, T,
                     H, nvq, nvb, q_end);
  return hipGetLastError();
}

}  // namespace sa
