// Spark virtual summaries: the global query anchor and, per anchor and
// physical 64-token K/V block, the softmax-weighted key and value and the
// log-mass correction (page "Sol-Attn and Spark for MiniMax-H3", Spark
// primitives, the spark_reweight paragraph; Spark inference integration: one
// global representative per head, the mean of all target-video queries,
// stored in BF16; log-mass taken against the stored BF16 summary key by
// default).
//
// Both kernels are HBM-bound streams: the anchor reads the video rows of Q
// once, the summaries read K and V once per anchor.  Neither is a
// contraction worth MFMA: the anchor-key scores are 128-term dot products of
// one anchor against 64 keys.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kAnchorThreads = 256;
constexpr int kAnchorRows = 256;     // query rows per partial sum
constexpr int kReweightThreads = 256;
constexpr int kWavesPerWg = kReweightThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Partial fp64 sums of 256 consecutive video rows of Q per (b, h): thread
// (row group rg, 16-byte chunk c8) adds rows rg, rg + 16, ... of the tile;
// the 16 row groups are then added in a fixed order.  Sums of bf16 values
// are exact in fp64, so the order does not change them.
__global__ __launch_bounds__(kAnchorThreads) void anchor_partial_kernel(
    const uint4 *__restrict__ q, double *__restrict__ part, int T, int H, int sink_start) {
  __shared__ double red[16][kHeadDim];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int rg = threadIdx.x >> 4, c8 = threadIdx.x & 15;
  const int chunks = H * (kHeadDim / 8);
  const int r0 = tile * kAnchorRows;
  const int r1 = r0 + kAnchorRows < sink_start ? r0 + kAnchorRows : sink_start;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  for (int r = r0 + rg; r < r1; r += 16) {
    const uint4 w = q[((int64_t)b * T + r) * chunks + h * (kHeadDim / 8) + c8];
    acc[0] += (double)bf16_lo(w.x);
    acc[1] += (double)bf16_hi(w.x);
    acc[2] += (double)bf16_lo(w.y);
    acc[3] += (double)bf16_hi(w.y);
    acc[4] += (double)bf16_lo(w.z);
    acc[5] += (double)bf16_hi(w.z);
    acc[6] += (double)bf16_lo(w.w);
    acc[7] += (double)bf16_hi(w.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rg][8 * c8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < kHeadDim) {
    const int d = threadIdx.x;
    double s = 0.0;
    for (int g = 0; g < 16; ++g) s += red[g][d];
    const int ntiles = gridDim.x;
    part[(((int64_t)b * H + h) * ntiles + tile) * kHeadDim + d] = s;
  }
}

// anchor[b, 0, h, d] = bf16(fp32(sum / sink_start)).  Thread (part, d) of
// 256 adds every fourth partial sum of channel d (four independent loads in
// flight per thread), then the four parts are added in a fixed order; all of
// these fp64 sums are exact.
constexpr int kFinishThreads = 4 * kHeadDim;
__global__ __launch_bounds__(kFinishThreads) void anchor_finish_kernel(const double *__restrict__ part,
                                                                       uint16_t *__restrict__ anchor,
                                                                       int H, int ntiles, int sink_start) {
  __shared__ double red[4][kHeadDim];
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x & (kHeadDim - 1), q4 = threadIdx.x >> 7;
  const double *pp = part + ((int64_t)b * H + h) * ntiles * kHeadDim + d;
  double s = 0.0;
#pragma unroll 4
  for (int t = q4; t < ntiles; t += 4) s += pp[(int64_t)t * kHeadDim];
  red[q4][d] = s;
  __syncthreads();
  if (q4 == 0) {
    const double tot = (red[0][d] + red[1][d]) + (red[2][d] + red[3][d]);
    const float m = (float)(tot / (double)sink_start);
    anchor[((int64_t)b * H + h) * kHeadDim + d] = bf16_bits(m);
  }
}

// One wavefront per (b, anchor p, h, K/V block j).  Lane (r0, c) =
// (lane / 16, lane % 16) holds channels 8c .. 8c+7 of keys / values
// 4i + r0, i = 0..15, of the block (each group of 16 lanes reads whole
// 256-byte head rows).  Per anchor:
//   z_t  = scale * a.k_t: 8-channel partial dots, summed over the 16 lanes
//          of a row by an xor butterfly (every lane ends with the same bits);
//   w_t  = exp(z_t - max), s = sum w_t (keys past T count as absent);
//   ak   = sum w_t k_t / s, av = sum w_t v_t / s, stored as bf16;
//   lm   = max + ln s - scale * a.ak, with ak as stored (bf16) or, with
//          pre_round, the fp32 weighted key.
// Several anchors re-read K and V (one anchor per head is the usual case).
__global__ __launch_bounds__(kReweightThreads) void reweight_kernel(
    const uint16_t *__restrict__ anchors, const uint4 *__restrict__ k, const uint4 *__restrict__ v,
    uint16_t *__restrict__ ak, uint16_t *__restrict__ av, float *__restrict__ lm, int P, int T, int H,
    int nb, float scale, int pre_round) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * kWavesPerWg + wave;
  const int h = blockIdx.y, b = blockIdx.z / P, p = blockIdx.z % P;
  if (j >= nb) return;  // wave-uniform
  const int c = lane & 15, r0 = lane >> 4;
  const int chunks = H * (kHeadDim / 8);
  const int nkeys = T - kBlock * j < kBlock ? T - kBlock * j : kBlock;

  uint4 kr[16], vr[16];
  const int64_t row0 = (int64_t)b * T + (int64_t)kBlock * j;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = 4 * i + r0;
    kr[i] = make_uint4(0, 0, 0, 0);
    vr[i] = make_uint4(0, 0, 0, 0);
    if (t < nkeys) {
      const int64_t off = (row0 + t) * chunks + h * (kHeadDim / 8) + c;
      kr[i] = k[off];
      vr[i] = v[off];
    }
  }
  auto unpack = [](const uint4 w, float (&f)[8]) {
    f[0] = bf16_lo(w.x);
    f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y);
    f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z);
    f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w);
    f[7] = bf16_hi(w.w);
  };

  {
    const int64_t bph = ((int64_t)b * P + p) * H + h;
    const uint4 aw = reinterpret_cast<const uint4 *>(anchors + bph * kHeadDim)[c];
    float af[8];
    unpack(aw, af);

    // bf16 pair dot products straight from the loaded words (the products
    // are exact in fp32), so K is unpacked only once, for the weighted sum.
    float z[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = 0.f;
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw.x), __builtin_bit_cast(bf16x2, kr[i].x), s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw.y), __builtin_bit_cast(bf16x2, kr[i].y), s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw.z), __builtin_bit_cast(bf16x2, kr[i].z), s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aw.w), __builtin_bit_cast(bf16x2, kr[i].w), s, false);
      z[i] = s;
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] += shfl_xor_f32(z[i], m);
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      z[i] = (4 * i + r0 < nkeys) ? z[i] * scale : -INFINITY;
      mx = fmaxf(mx, z[i]);
    }
    mx = fmaxf(mx, shfl_xor_f32(mx, 16));
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));

    float w[16], sw = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      w[i] = __builtin_amdgcn_exp2f((z[i] - mx) * kLog2e);
      sw += w[i];
    }
    sw += shfl_xor_f32(sw, 16);
    sw += shfl_xor_f32(sw, 32);

    float ka[8], va[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ka[e] = va[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float fk[8], fv[8];
      unpack(kr[i], fk);
      unpack(vr[i], fv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ka[e] = __builtin_fmaf(w[i], fk[e], ka[e]);
        va[e] = __builtin_fmaf(w[i], fv[e], va[e]);
      }
    }
    const float inv = 1.f / sw;
    uint16_t kb[8], vb[8];
    float shift_key[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ka[e] += shfl_xor_f32(ka[e], 16);
      ka[e] += shfl_xor_f32(ka[e], 32);
      va[e] += shfl_xor_f32(va[e], 16);
      va[e] += shfl_xor_f32(va[e], 32);
      ka[e] *= inv;
      va[e] *= inv;
      kb[e] = bf16_bits(ka[e]);
      vb[e] = bf16_bits(va[e]);
      shift_key[e] = pre_round ? ka[e] : __uint_as_float((uint32_t)kb[e] << 16);
    }
    if (r0 == 0) {
      const int64_t o = (bph * nb + j) * kHeadDim + 8 * c;
      uint4 pk, pv;
      pk.x = kb[0] | ((uint32_t)kb[1] << 16);
      pk.y = kb[2] | ((uint32_t)kb[3] << 16);
      pk.z = kb[4] | ((uint32_t)kb[5] << 16);
      pk.w = kb[6] | ((uint32_t)kb[7] << 16);
      pv.x = vb[0] | ((uint32_t)vb[1] << 16);
      pv.y = vb[2] | ((uint32_t)vb[3] << 16);
      pv.z = vb[4] | ((uint32_t)vb[5] << 16);
      pv.w = vb[6] | ((uint32_t)vb[7] << 16);
      *reinterpret_cast<uint4 *>(ak + o) = pk;
      *reinterpret_cast<uint4 *>(av + o) = pv;
    }
    float dp = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dp = __builtin_fmaf(af[e], shift_key[e], dp);
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) dp += shfl_xor_f32(dp, m);
    if (lane == 0) lm[bph * nb + j] = mx + __logf(sw) - scale * dp;
  }
}

}  // namespace

size_t anchor_workspace_bytes(int B, int H, int sink_start) {
  if (sink_start <= 0) return 0;
  const size_t tiles = ((size_t)sink_start + kAnchorRows - 1) / kAnchorRows;
  return (size_t)B * H * tiles * kHeadDim * sizeof(double);
}

hipError_t launch_anchor(const void *q, void *workspace, void *anchor, int B, int T, int H,
                         int sink_start, hipStream_t stream) {
  const int tiles = (sink_start + kAnchorRows - 1) / kAnchorRows;
  double *part = static_cast<double *>(workspace);
  hipLaunchKernelGGL(anchor_partial_kernel, dim3(tiles, H, B), dim3(kAnchorThreads), 0, stream,
                     static_cast<const uint4 *>(q), part, T, H, sink_start);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(anchor_finish_kernel, dim3(H, B), dim3(kFinishThreads), 0, stream, part,
                     static_cast<uint16_t *>(anchor), H, tiles, sink_start);
  return hipGetLastError();
}

hipError_t launch_reweight(const void *anchors, const void *k, const void *v, void *ak, void *av,
                           float *lm, int B, int P, int T, int H, float scale, int pre_round,
                           hipStream_t stream) {
  const int nb = (T + kBlock - 1) / kBlock;
  dim3 grid((nb + kWavesPerWg - 1) / kWavesPerWg, H, B * P);
  hipLaunchKernelGGL(reweight_kernel, grid, dim3(kReweightThreads), 0, stream,
                     static_cast<const uint16_t *>(anchors), static_cast<const uint4 *>(k),
                     static_cast<const uint4 *>(v), static_cast<uint16_t *>(ak),
                     static_cast<uint16_t *>(av), lm, P, T, H, nb, scale, pre_round);
  return hipGetLastError();
}

}  // namespace sa
