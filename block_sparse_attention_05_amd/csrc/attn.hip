// Block-sparse flash attention on gfx950 bf16 MFMA, shared by the sparse
// (block lists) and dense (all key blocks) paths.
//
// Page "Sol-Attn and Spark for MiniMax-H3", Spark inference integration:
// selected K/V tiles stream through a single FP32 online-softmax/output
// accumulator.  Page "Add key bias to chunked Sol-Attn producers", Summary /
// Contract: the natural-log key bias is converted to log2 units and consumed
// only by the exact branch (sink keys).
//
// Workgroup = one 64-row query block of one (b, h), two wavefronts of 32 rows.
// Per 64-key tile of the block's list:
//   K tile  [64 keys][128 d] bf16 -> LDS, 16-byte chunks XOR-swizzled by row;
//   V tile  transposed to [128 d][64 keys] in LDS, keys in "MFMA order";
//   S^T = K Q^T   on v_mfma_f32_32x32x16_bf16 (K from LDS, Q in registers);
//   online softmax in base 2 per lane (each lane owns one query row);
//   O^T += V^T P^T on the same MFMA, P rounded to bf16 from registers.
// Computing S^T instead of S leaves each lane with one query row and 16 keys
// per 32x32 tile, which is exactly the B-operand fragment P^T of the PV
// product once the keys inside each 16-key group are taken in the order
// {4g..4g+3, 8+4g..8+4g+3} (g = lane / 32); V^T is stored in that order.
//
// The next tile's global loads are issued before the current tile's math so
// HBM/L2 latency hides behind the MFMAs.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 128;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Params {
  const uint16_t *q, *k, *v;
  uint16_t *out;
  float *lse;
  const float *key_bias;
  const int32_t *block_idx, *block_cnt;
  int B, T, H, nb, nvb, max_sel;
  int qb0, nqb;
  float scale_log2;
};

// 16-bit element e (0..7) of a 16-byte chunk.
__device__ __forceinline__ uint32_t elem16(const uint4 &w, int e) {
  const uint32_t x = (e >> 1) == 0 ? w.x : (e >> 1) == 1 ? w.y : (e >> 1) == 2 ? w.z : w.w;
  return (e & 1) ? (x >> 16) : (x & 0xffffu);
}

// Byte offset of (key row, 16-byte chunk) in the K tile.
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}

// Byte offset of (d row, 16-byte chunk) in the transposed V tile.
__device__ __forceinline__ int vt_off(int d, int chunk) {
  const int sw = (d & 7) ^ ((d >> 3) & 1);
  return d * 128 + ((chunk ^ sw) << 4);
}

template <bool kDense>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(Params p) {
  __shared__ __align__(16) unsigned char smem[32768];
  unsigned char *ks = smem;          // K tile
  unsigned char *vt = smem + 16384;  // V^T tile

  const int total = p.B * p.H * p.nqb;
  const int w = xcd_remap(blockIdx.x, total);
  const int qbi = w % p.nqb;
  const int bh = w / p.nqb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int qb = p.qb0 + qbi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int T = p.T;
  const int64_t rs = (int64_t)p.H * kHeadDim;                      // token stride
  const int64_t base = (int64_t)b * T * rs + (int64_t)h * kHeadDim;

  // Q^T fragments for this lane's query row: d = 16*dc + 8*g + [0, 8)
  const int tq = qb * kBlock + wave * 32 + c32;
  bf16x8 qf[8];
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(p.q + base + (int64_t)tq * rs);
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tq < T) x = qp[2 * dc + g];
      qf[dc] = __builtin_bit_cast(bf16x8, x);
    }
  }

  int ntiles;
  const int32_t *list = nullptr;
  if (kDense) {
    ntiles = p.nb;
  } else {
    const int64_t li = (int64_t)bh * p.nvb + qb;
    ntiles = p.block_cnt[li];
    ntiles = ntiles < 0 ? 0 : (ntiles > p.max_sel ? p.max_sel : ntiles);
    list = p.block_idx + li * p.max_sel;
  }
  // First token of tile `it`; an invalid list entry maps past T (all masked).
  auto tile_key0 = [&](int it) -> int {
    if (kDense) return it * kBlock;
    const int kb = list[it];
    return (kb >= 0 && kb < p.nb) ? kb * kBlock : T;
  };

  // Register staging of one K/V tile (global -> regs -> LDS).
  uint4 kr[8], vr[8];
  const int k_row = tid >> 4;   // + 8*s
  const int k_col = tid & 15;
  const int v_quad = tid & 15;  // keys 4*v_quad .. +3
  const int v_dg = tid >> 4;    // + 8*s2 : channels 8*v_dg .. +7
  auto load_tile = [&](int key0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int key = key0 + k_row + 8 * s;
      kr[s] = make_uint4(0, 0, 0, 0);
      if (key < T)
        kr[s] = *reinterpret_cast<const uint4 *>(p.k + base + (int64_t)key * rs + k_col * 8);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = key0 + 4 * v_quad + kk;
        vr[4 * s2 + kk] = make_uint4(0, 0, 0, 0);
        if (key < T)
          vr[4 * s2 + kk] = *reinterpret_cast<const uint4 *>(p.v + base + (int64_t)key * rs +
                                                             (v_dg + 8 * s2) * 8);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      *reinterpret_cast<uint4 *>(ks + k_off(k_row + 8 * s, k_col)) = kr[s];
    // key quad -> position quad inside its 16-key group (swap the two low bits)
    const int pq = (v_quad & ~3) | ((v_quad & 1) << 1) | ((v_quad >> 1) & 1);
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * (v_dg + 8 * s2) + e;
        uint2 val;
        val.x = elem16(vr[4 * s2 + 0], e) | (elem16(vr[4 * s2 + 1], e) << 16);
        val.y = elem16(vr[4 * s2 + 2], e) | (elem16(vr[4 * s2 + 3], e) << 16);
        *reinterpret_cast<uint2 *>(vt + vt_off(d, pq >> 1) + ((pq & 1) << 3)) = val;
      }
    }
  };

  float m_run = -INFINITY;  // running max, log2 units
  float l_run = 0.f;        // this lane's partial row sum
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  const float *kbias = p.key_bias ? p.key_bias + (int64_t)b * T : nullptr;
  const int sink0 = p.nvb * kBlock;

  if (ntiles > 0) load_tile(tile_key0(0));
  for (int it = 0; it < ntiles; ++it) {
    const int key0 = tile_key0(it);
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (it + 1 < ntiles) load_tile(tile_key0(it + 1));

    // S^T = K Q^T : two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[hk][r] = 0.f;
      const int row = 32 * hk + c32;
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + k_off(row, 2 * dc + g));
        s[hk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[hk], 0, 0, 0);
      }
    }

    // scale, key bias (sink keys only), mask past T; tile max
    const bool biased = (kbias != nullptr) && (key0 >= sink0) && (key0 < T);
    float mx = -INFINITY;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 32 * hk + 8 * (r >> 2) + 4 * g + (r & 3);
        float x = s[hk][r] * p.scale_log2;
        if (biased && key < T) x += kbias[key] * kLog2e;
        if (key >= T) x = -INFINITY;
        s[hk][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, shfl_xor_f32(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    bf16x8 pf[4];
    float psum = 0.f;
#pragma unroll
    for (int hk = 0; hk < 2; ++hk) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(s[hk][r] - m_use);
        psum += pv;
        pf[2 * hk + (r >> 3)][r & 7] = (__bf16)pv;
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 32 * dt + c32;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vt + vt_off(d, 2 * kc + g));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], o[dt], 0, 0, 0);
      }
    }
  }

  // Finalize: the two lanes of a row hold disjoint key subsets.
  const float l_tot = l_run + shfl_xor_f32(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (tq < T) {
    uint16_t *op = p.out + base + (int64_t)tq * rs;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * g;
        const __bf16 y0 = (__bf16)(o[dt][4 * rq + 0] * inv);
        const __bf16 y1 = (__bf16)(o[dt][4 * rq + 1] * inv);
        const __bf16 y2 = (__bf16)(o[dt][4 * rq + 2] * inv);
        const __bf16 y3 = (__bf16)(o[dt][4 * rq + 3] * inv);
        uint2 val;
        val.x = (uint32_t)__builtin_bit_cast(uint16_t, y0) |
                ((uint32_t)__builtin_bit_cast(uint16_t, y1) << 16);
        val.y = (uint32_t)__builtin_bit_cast(uint16_t, y2) |
                ((uint32_t)__builtin_bit_cast(uint16_t, y3) << 16);
        *reinterpret_cast<uint2 *>(op + d0) = val;
      }
    }
    if (p.lse != nullptr && g == 0)
      p.lse[((int64_t)b * p.H + h) * T + tq] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

Params make_params(const AttnArgs &a, int qb0, int nqb) {
  Params p;
  p.q = static_cast<const uint16_t *>(a.q);
  p.k = static_cast<const uint16_t *>(a.k);
  p.v = static_cast<const uint16_t *>(a.v);
  p.out = static_cast<uint16_t *>(a.out);
  p.lse = a.lse;
  p.key_bias = a.key_bias;
  p.block_idx = a.block_idx;
  p.block_cnt = a.block_cnt;
  p.B = a.B;
  p.T = a.T;
  p.H = a.H;
  p.nb = a.nb;
  p.nvb = a.nvb;
  p.max_sel = a.max_sel;
  p.qb0 = qb0;
  p.nqb = nqb;
  p.scale_log2 = a.scale_log2;
  return p;
}

}  // namespace

hipError_t launch_attn_sparse(const AttnArgs &a, hipStream_t stream) {
  if (a.nvb <= 0) return hipSuccess;
  const Params p = make_params(a, 0, a.nvb);
  const int total = a.B * a.H * a.nvb;
  hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_dense(const AttnArgs &a, hipStream_t stream) {
  const int nq = a.nb - a.nvb;
  if (nq <= 0) return hipSuccess;
  const Params p = make_params(a, a.nvb, nq);
  const int total = a.B * a.H * nq;
  hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
