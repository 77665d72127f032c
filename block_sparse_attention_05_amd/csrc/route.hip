// Route: pooled block scores, fixed-ratio Top-K and exact-list emission.
//
// Page "Sol-Attn and Spark for MiniMax-H3", Spark inference integration:
// the route QK of pooled means is computed once, outside attention, with an
// exact FP32 boundary selection.  H3 pipeline integration: forced self /
// neighbour blocks are added outside the Top-K budget.  Page "Add key bias to
// chunked Sol-Attn producers", Tests and source audit: sink blocks go straight
// into the exact list and are never routed candidates.
//
// One workgroup (4 wavefronts) serves kRows query blocks of one (b, h):
//  1. scores s_ij for its rows against every key block j < nvb.  fp32 x fp32
//     products are exact in fp64, so the fp64 dot product rounded once to fp32
//     is the fp32 score of the exact value (up to fp64 rounding of the sum).
//  2. per row, one wavefront sorts 64-bit keys (descending-score bits, block
//     index) with a bitonic network held in registers (E keys per lane,
//     64*E >= nvb); forced blocks get the largest key so they never compete.
//  3. the first k keys flag their blocks; forced blocks are flagged too; a
//     ballot/popcount scan emits the flagged blocks in ascending order, then
//     the sink blocks [nvb, nb), then -1 padding.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRows = 8;  // query blocks per workgroup

// fp32 bits -> unsigned key that sorts ascending as the float sorts
// descending.  -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t desc_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  const uint32_t asc = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ~asc;
}

// Ascending bitonic sort of the 64*E keys of one wavefront; element x lives
// in lane x % 64, slot x / 64.
template <int E>
__device__ __forceinline__ void wave_bitonic_sort(uint64_t (&key)[E], int lane) {
  constexpr int kLogP = (E == 1) ? 6 : (E == 2) ? 7 : (E == 4) ? 8 : (E == 8) ? 9 : 10;
#pragma unroll
  for (int ls = 1; ls <= kLogP; ++ls) {
    const int size = 1 << ls;
#pragma unroll
    for (int lt = ls - 1; lt >= 0; --lt) {
      const int stride = 1 << lt;
      if (stride >= 64) {
        const int es = stride >> 6;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int e2 = e ^ es;
          if (e2 > e) {
            const int x = e * 64 + lane;
            const bool asc = (x & size) == 0;
            const uint64_t a = key[e], c = key[e2];
            const bool swap = asc ? (a > c) : (a < c);
            key[e] = swap ? c : a;
            key[e2] = swap ? a : c;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int x = e * 64 + lane;
          const uint64_t other = shfl_xor_u64(key[e], stride);
          const bool asc = (x & size) == 0;
          const bool lower = (lane & stride) == 0;
          const bool keep_min = (asc == lower);
          const uint64_t mn = key[e] < other ? key[e] : other;
          const uint64_t mx = key[e] < other ? other : key[e];
          key[e] = keep_min ? mn : mx;
        }
      }
    }
  }
}

template <int E>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float *__restrict__ qbar, const float *__restrict__ kbar, int H, int nvb, int nb,
    int budget, int radius, int max_sel, int32_t *__restrict__ block_idx,
    int32_t *__restrict__ block_cnt, float *__restrict__ scores_out) {
  constexpr int P = 64 * E;  // padded row width
  extern __shared__ __align__(16) unsigned char smem[];
  double *qs = reinterpret_cast<double *>(smem);                 // [kRows][128]
  float *sc = reinterpret_cast<float *>(qs + kRows * kHeadDim);  // [kRows][P]
  uint8_t *flags = reinterpret_cast<uint8_t *>(sc + kRows * P);  // [4 waves][P]

  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * kRows;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float *qb = qbar + (int64_t)bh * nvb * kHeadDim;
  const float *kb = kbar + (int64_t)bh * nvb * kHeadDim;

  for (int x = tid; x < kRows * kHeadDim; x += kRouteThreads) {
    const int r = x / kHeadDim;
    qs[x] = (i0 + r < nvb) ? (double)qb[(int64_t)(i0 + r) * kHeadDim + (x % kHeadDim)] : 0.0;
  }
  __syncthreads();

  // 1. scores
  for (int j = tid; j < nvb; j += kRouteThreads) {
    double acc[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = 0.0;
    const float4 *kr = reinterpret_cast<const float4 *>(kb + (int64_t)j * kHeadDim);
#pragma unroll 4
    for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
      const float4 kv = kr[d4];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const double *qr = qs + r * kHeadDim + 4 * d4;
        acc[r] = fma(qr[0], (double)kv.x, acc[r]);
        acc[r] = fma(qr[1], (double)kv.y, acc[r]);
        acc[r] = fma(qr[2], (double)kv.z, acc[r]);
        acc[r] = fma(qr[3], (double)kv.w, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const float s = (float)acc[r];
      sc[r * P + j] = s;
      if (scores_out != nullptr && i0 + r < nvb)
        scores_out[((int64_t)bh * nvb + i0 + r) * nvb + j] = s;
    }
  }
  __syncthreads();

  // 2-3. one wavefront per row
  uint8_t *fl = flags + wave * P;
  for (int rr = wave; rr < kRows; rr += 4) {
    const int i = i0 + rr;
    if (i >= nvb) break;  // wave-uniform; no workgroup barrier below
    const int f_lo = i - radius < 0 ? 0 : i - radius;
    const int f_hi = i + radius > nvb - 1 ? nvb - 1 : i + radius;
    const int n_cand = nvb - (f_hi - f_lo + 1);
    const int kk = budget < n_cand ? budget : n_cand;

    uint64_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = e * 64 + lane;
      const bool cand = j < nvb && (j < f_lo || j > f_hi);
      key[e] = cand ? ((uint64_t)desc_key(sc[rr * P + j]) << 32) | (uint32_t)j : ~0ull;
    }
    wave_bitonic_sort<E>(key, lane);

    for (int x = lane; x < P; x += 64) fl[x] = 0;
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e * 64 + lane < kk) fl[(uint32_t)key[e]] = 1;
    }
    for (int j = f_lo + lane; j <= f_hi; j += 64) fl[j] = 1;
    wave_lds_sync();

    int32_t *out = block_idx + ((int64_t)bh * nvb + i) * max_sel;
    int base = 0;
    for (int c = 0; c < nvb; c += 64) {
      const int j = c + lane;
      const bool f = j < nvb && fl[j] != 0;
      const uint64_t mask = __ballot(f);
      const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
      if (f) out[pos] = j;
      base += __popcll(mask);
    }
    for (int j = nvb + lane; j < nb; j += 64) out[base + (j - nvb)] = j;
    const int cnt = base + (nb - nvb);
    for (int x = cnt + lane; x < max_sel; x += 64) out[x] = -1;
    if (lane == 0) block_cnt[(int64_t)bh * nvb + i] = cnt;
    wave_lds_sync();  // flags are reused by this wave's next row
  }
}

template <int E>
hipError_t launch_route_e(const float *qbar, const float *kbar, int B, int H, int nvb, int nb,
                          int budget, int radius, int max_sel, int32_t *block_idx,
                          int32_t *block_cnt, float *scores, hipStream_t stream) {
  constexpr int P = 64 * E;
  const size_t lds = kRows * kHeadDim * sizeof(double) + kRows * P * sizeof(float) + 4 * P;
  dim3 grid((nvb + kRows - 1) / kRows, B * H);
  hipLaunchKernelGGL(route_kernel<E>, grid, dim3(kRouteThreads), lds, stream, qbar, kbar, H, nvb,
                     nb, budget, radius, max_sel, block_idx, block_cnt, scores);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float *qbar, const float *kbar, int B, int H, int nvb, int nb,
                        int budget, int radius, int max_sel, int32_t *block_idx,
                        int32_t *block_cnt, float *scores, hipStream_t stream) {
  if (nvb <= 0) return hipSuccess;
  if (nvb <= 64)
    return launch_route_e<1>(qbar, kbar, B, H, nvb, nb, budget, radius, max_sel, block_idx,
                             block_cnt, scores, stream);
  if (nvb <= 128)
    return launch_route_e<2>(qbar, kbar, B, H, nvb, nb, budget, radius, max_sel, block_idx,
                             block_cnt, scores, stream);
  if (nvb <= 256)
    return launch_route_e<4>(qbar, kbar, B, H, nvb, nb, budget, radius, max_sel, block_idx,
                             block_cnt, scores, stream);
  if (nvb <= 512)
    return launch_route_e<8>(qbar, kbar, B, H, nvb, nb, budget, radius, max_sel, block_idx,
                             block_cnt, scores, stream);
  if (nvb <= kMaxRouteBlocks)
    return launch_route_e<16>(qbar, kbar, B, H, nvb, nb, budget, radius, max_sel, block_idx,
                              block_cnt, scores, stream);
  return hipErrorInvalidValue;
}

}  // namespace sa
