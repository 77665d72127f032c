// Block-sparse flash attention on gfx950 bf16 MFMA, shared by the sparse
// (block lists) and dense (all key blocks) paths.
//
// Page "Sol-Attn and Spark for MiniMax-H3", Spark inference integration:
// selected K/V tiles stream through a single FP32 online-softmax/output
// accumulator.  Page "Add key bias to chunked Sol-Attn producers", Summary /
// Contract: the natural-log key bias is converted to log2 units and consumed
// only by the exact branch (sink keys).
//
// Workgroup = one 64-row query block of one (b, h) (or, on the dense path,
// one key range of such a block: split-KV), four wavefronts: wave w owns query
// rows 32*(w&1)..+31 and keys 32*(w>>1)..+31 of every tile, with its own
// online-softmax state; the two key halves of each row are merged at the end.
// Per 64-key tile of the block's list:
//   * K and V tiles (64 keys x 256 B each) arrive with buffer loads: the
//     tile's base goes into the per-lane offset, so keys past T fall outside
//     the buffer's range and read as zero; they are staged in registers one
//     tile ahead and written row-major to LDS with 16-byte chunks
//     XOR-swizzled per row (conflict-free reads below);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, K fragments from LDS, Q^T
//     fragments resident in registers.  Each lane then owns one query row and
//     16 keys per 32x32 tile, so the softmax row reductions stay in-lane
//     apart from one exchange with lane ^ 32;
//   * online softmax in base 2 (scale * log2 e folded into one FMA), lazy
//     rescaling: the running max moves only when a row's max grows by more
//     than 8 (P <= 2^8 stays exact in range), the row sum is accumulated from
//     the bf16-rounded P with v_dot2;
//   * O^T += V^T P^T on the same MFMA: P^T fragments come straight from the
//     S^T registers; V^T fragments come from the row-major V tile through
//     ds_read_b64_tr_b16, which hands each lane one column of a 4-row block.
//     Keys inside each 16-key group are contracted in the order
//     {4g..4g+3, 8+4g..8+4g+3} (g = lane / 32) on both operands.
#include "device_util.h"
#include "kernels.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;       // log2 units
constexpr int kBufferFlags = 0x00020000;    // raw buffer, 32-bit data format

struct Params {
  const uint16_t *q, *k, *v;
  uint16_t *out;
  float *lse;
  const float *key_bias;
  const int32_t *block_idx, *block_cnt;
  float *part_o;      // split-KV partial outputs (dense path), nullable
  float *part_ml;     // split-KV partial (max, sum) per row
  int B, T, H, nb, nvb, max_sel;
  int qb0, nqb;
  int nsplit, tiles_per_split;
  float scale_log2;
};

// Byte offset of (key row, 16-byte chunk) in the K tile.
__device__ __forceinline__ int k_off(int row, int chunk) {
  return row * 256 + ((chunk ^ (row & 15)) << 4);
}
// Byte offset of (key row, 16-byte chunk) in the V tile.
__device__ __forceinline__ int v_off(int row, int chunk) {
  return row * 256 + ((chunk ^ ((row & 3) << 2)) << 4);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <bool kDense>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
  __shared__ __align__(16) unsigned char smem[32768 + 512];
  unsigned char *ks = smem;            // K tile
  unsigned char *vs = smem + 16384;    // V tile
  float *bs = reinterpret_cast<float *>(smem + 32768);  // key bias of the tile, log2 units

  const int total = p.B * p.H * p.nqb * p.nsplit;
  const int w = xcd_remap(blockIdx.x, total);
  const int split = w % p.nsplit;
  const int wq = w / p.nsplit;
  const int qbi = wq % p.nqb;
  const int bh = wq / p.nqb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int qb = p.qb0 + qbi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rw = wave & 1;     // query rows 32*rw .. +31 of the block
  const int kh = wave >> 1;    // keys 32*kh .. +31 of every tile
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int T = p.T;
  const int64_t rs = (int64_t)p.H * kHeadDim;   // elements per token
  const int row_bytes = p.H * kHeadDim * 2;
  const int64_t bbase = (int64_t)b * T * rs;

  // Q^T fragments for this lane's query row: d = 16*dc + 8*g + [0, 8)
  const int tq = qb * kBlock + rw * 32 + c32;
  bf16x8 qf[8];
  {
    const uint4 *qp = reinterpret_cast<const uint4 *>(p.q + bbase + (int64_t)tq * rs + h * kHeadDim);
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (tq < T) x = qp[2 * dc + g];
      qf[dc] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Tiles of this workgroup
  int t_begin = 0, t_end;
  const int32_t *list = nullptr;
  if (kDense) {
    t_begin = split * p.tiles_per_split;
    t_end = t_begin + p.tiles_per_split;
    t_end = t_end < p.nb ? t_end : p.nb;
  } else {
    const int64_t li = (int64_t)bh * p.nvb + qb;
    int n = p.block_cnt[li];
    t_end = n < 0 ? 0 : (n > p.max_sel ? p.max_sel : n);
    list = p.block_idx + li * p.max_sel;
  }
  // First token of tile `it`; an invalid list entry maps to T (reads as zero,
  // fully masked).
  auto tile_key0 = [&](int it) -> int {
    if (kDense) return it * kBlock;
    const int kb = list[it];
    return (kb >= 0 && kb < p.nb) ? kb * kBlock : T;
  };

  // Buffer resources over this batch's K and V: offsets past T*row_bytes read 0.
  const uint32_t slab = (uint32_t)T * (uint32_t)row_bytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p.k + bbase), (short)0, (int)slab, kBufferFlags);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void *)(p.v + bbase), (short)0, (int)slab, kBufferFlags);
  const float *kbias = p.key_bias ? p.key_bias + (int64_t)b * T : nullptr;
  const int sink0 = p.nvb * kBlock;

  // Register staging: thread loads rows st_row + 16*s, chunk st_chunk.
  const int st_row = tid >> 4;
  const int st_chunk = tid & 15;
  const uint32_t lane_off = (uint32_t)(st_row * row_bytes + h * 256 + st_chunk * 16);
  i32x4 kr[4], vr[4];
  float br = 0.f;
  auto load_tile = [&](int key0, bool biased) {
    const uint32_t off0 = lane_off + (uint32_t)key0 * (uint32_t)row_bytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t off = off0 + (uint32_t)(16 * s) * (uint32_t)row_bytes;
      kr[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      vr[s] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
    if (biased && tid < kBlock) {
      const int key = key0 + tid;
      br = key < T ? kbias[key] * kLog2e : 0.f;
    }
  };
  auto store_tile = [&](bool biased) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int row = st_row + 16 * s;
      *reinterpret_cast<i32x4 *>(ks + k_off(row, st_chunk)) = kr[s];
      *reinterpret_cast<i32x4 *>(vs + v_off(row, st_chunk)) = vr[s];
    }
    if (biased && tid < kBlock) bs[tid] = br;
  };
  auto tile_biased = [&](int key0) { return kbias != nullptr && key0 >= sink0 && key0 < T; };

  // ds_read_b64_tr_b16 addressing for the V^T fragments
  const int tr_i = lane & 15;
  const int tr_r = tr_i >> 2;
  const int tr_j = tr_i & 3;
  const int tr_dh = (lane >> 4) & 1;

  float m_used = -INFINITY;   // running max (log2 units) used for P
  float l_run = 0.f;          // this lane's share of the row sum
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float c = p.scale_log2;

  if (t_begin < t_end) {
    const int k0 = tile_key0(t_begin);
    load_tile(k0, tile_biased(k0));
  }
  for (int it = t_begin; it < t_end; ++it) {
    const int key0 = tile_key0(it);
    const bool biased = tile_biased(key0);
    __syncthreads();  // previous tile fully consumed
    store_tile(biased);
    __syncthreads();
    if (it + 1 < t_end) {
      const int k1 = tile_key0(it + 1);
      load_tile(k1, tile_biased(k1));
    }

    // S^T = K Q^T over this wave's 32 keys
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    {
      const int row = 32 * kh + c32;
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ks + k_off(row, 2 * dc + g));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s, 0, 0, 0);
      }
    }
    const int kbase = key0 + 32 * kh + 4 * g;   // key of s[r] = kbase + 8*(r/4) + r%4

    // Keys past T (only in the last, partial block) are masked.
    if (key0 + kBlock > T) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 8 * (r >> 2) + (r & 3) >= T) s[r] = -INFINITY;
    }
    // Logit in log2 units: s*c (+ beta2 on sink tiles).  With a bias the
    // exponent is formed as fma(s, c, beta2 - m), so beta2 = 0 reproduces the
    // unbiased fma(s, c, -m) bit for bit.
    float bv[16];
    float mt;  // tile max of this lane's logits, log2 units
    if (biased) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 b4 = *reinterpret_cast<const float4 *>(bs + 32 * kh + 8 * q4 + 4 * g);
        bv[4 * q4 + 0] = b4.x;
        bv[4 * q4 + 1] = b4.y;
        bv[4 * q4 + 2] = b4.z;
        bv[4 * q4 + 3] = b4.w;
      }
      mt = __builtin_fmaf(s[0], c, bv[0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, __builtin_fmaf(s[r], c, bv[r]));
    } else {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mt = mx * c;
    }
    mt = fmaxf(mt, shfl_xor_f32(mt, 32));

    // Lazy rescale: move the running max only when it grows by > slack.
    if (__any(mt > m_used + kRescaleSlack)) {
      const float m_new = fmaxf(m_used, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);  // 0 when m_used = -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_used = m_new;
    }
    const float m_sub = (m_used == -INFINITY) ? 0.f : m_used;

    // P = 2^(logit - m) in bf16; row sum from the rounded values.
    bf16x8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float x0, x1;
      if (biased) {
        x0 = __builtin_fmaf(s[r], c, bv[r] - m_sub);
        x1 = __builtin_fmaf(s[r + 1], c, bv[r + 1] - m_sub);
      } else {
        x0 = __builtin_fmaf(s[r], c, -m_sub);
        x1 = __builtin_fmaf(s[r + 1], c, -m_sub);
      }
      const bf16x2 pk = {(__bf16)__builtin_amdgcn_exp2f(x0), (__bf16)__builtin_amdgcn_exp2f(x1)};
      l_run = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_run, false);
      pf[r >> 3][r & 7] = pk[0];
      pf[r >> 3][(r & 7) + 1] = pk[1];
    }

    // O^T += V^T P^T over this wave's 32 keys
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int row0 = 32 * kh + 16 * kc + 4 * g + tr_r;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int chunk = 4 * dt + 2 * tr_dh + (tr_j >> 1);
        const int sub = (tr_j & 1) * 8;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vs + v_off(row0, chunk) + sub));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vs + v_off(row0 + 8, chunk) + sub));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], o[dt], 0, 0, 0);
      }
    }
  }

  // Merge the two key halves of every row: waves 2,3 hand (m, l, O^T) to
  // waves 0,1 through LDS.
  float l_tot = l_run + shfl_xor_f32(l_run, 32);
  __syncthreads();
  float4 *xo = reinterpret_cast<float4 *>(smem);              // [rw][16 quads][64 lanes]
  float2 *xml = reinterpret_cast<float2 *>(smem + 32768);     // [rw][32 rows]
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        xo[(rw * 16 + dt * 4 + rq) * 64 + lane] =
            make_float4(o[dt][4 * rq], o[dt][4 * rq + 1], o[dt][4 * rq + 2], o[dt][4 * rq + 3]);
    if (g == 0) xml[rw * 32 + c32] = make_float2(m_used, l_tot);
  }
  __syncthreads();
  if (kh == 1) return;
  {
    const float2 mlb = xml[rw * 32 + c32];
    const float m = fmaxf(m_used, mlb.x);
    const float msub = (m == -INFINITY) ? 0.f : m;
    const float aa = __builtin_amdgcn_exp2f(m_used - msub);
    const float ab = __builtin_amdgcn_exp2f(mlb.x - msub);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 ob = xo[(rw * 16 + dt * 4 + rq) * 64 + lane];
        o[dt][4 * rq + 0] = o[dt][4 * rq + 0] * aa + ob.x * ab;
        o[dt][4 * rq + 1] = o[dt][4 * rq + 1] * aa + ob.y * ab;
        o[dt][4 * rq + 2] = o[dt][4 * rq + 2] * aa + ob.z * ab;
        o[dt][4 * rq + 3] = o[dt][4 * rq + 3] * aa + ob.w * ab;
      }
    l_tot = l_tot * aa + mlb.y * ab;
    m_used = m;
  }

  if (tq >= T) return;
  if (kDense && p.nsplit > 1) {
    // partial (unnormalised O, max, sum) of this key range
    const int64_t prow = ((int64_t)wq * p.nsplit + split) * kBlock + (rw * 32 + c32);
    float *po = p.part_o + prow * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * dt + 8 * rq + 4 * g;
        *reinterpret_cast<float4 *>(po + d0) =
            make_float4(o[dt][4 * rq + 0], o[dt][4 * rq + 1], o[dt][4 * rq + 2], o[dt][4 * rq + 3]);
      }
    if (g == 0) *reinterpret_cast<float2 *>(p.part_ml + 2 * prow) = make_float2(m_used, l_tot);
    return;
  }
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t *op = p.out + bbase + (int64_t)tq * rs + h * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = 32 * dt + 8 * rq + 4 * g;
      uint2 val;
      val.x = pack_bf16x2(o[dt][4 * rq + 0] * inv, o[dt][4 * rq + 1] * inv);
      val.y = pack_bf16x2(o[dt][4 * rq + 2] * inv, o[dt][4 * rq + 3] * inv);
      *reinterpret_cast<uint2 *>(op + d0) = val;
    }
  }
  if (p.lse != nullptr && g == 0)
    p.lse[((int64_t)b * p.H + h) * T + tq] = (m_used + __log2f(l_tot)) * kLn2;
}

// Merge the split-KV partials of the dense rows: one thread per (row, 4
// channels).  m* = max_s m_s, O = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s.
constexpr int kCombineThreads = 256;
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(Params p) {
  const int wq = blockIdx.x;              // (b*H + h) * nqb + qbi
  const int qbi = wq % p.nqb;
  const int bh = wq / p.nqb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int T = p.T;
  const int64_t rs = (int64_t)p.H * kHeadDim;
  for (int x = threadIdx.x; x < kBlock * (kHeadDim / 4); x += kCombineThreads) {
    const int row = x / (kHeadDim / 4);
    const int d0 = (x % (kHeadDim / 4)) * 4;
    const int tq = (p.qb0 + qbi) * kBlock + row;
    if (tq >= T) continue;
    float m = -INFINITY;
    for (int s = 0; s < p.nsplit; ++s)
      m = fmaxf(m, p.part_ml[2 * (((int64_t)wq * p.nsplit + s) * kBlock + row)]);
    const float msub = (m == -INFINITY) ? 0.f : m;
    float l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < p.nsplit; ++s) {
      const int64_t prow = ((int64_t)wq * p.nsplit + s) * kBlock + row;
      const float2 ml = *reinterpret_cast<const float2 *>(p.part_ml + 2 * prow);
      const float wgt = __builtin_amdgcn_exp2f(ml.x - msub);
      l += wgt * ml.y;
      const float4 po = *reinterpret_cast<const float4 *>(p.part_o + prow * kHeadDim + d0);
      acc.x += wgt * po.x;
      acc.y += wgt * po.y;
      acc.z += wgt * po.z;
      acc.w += wgt * po.w;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t *op = p.out + (int64_t)b * T * rs + (int64_t)tq * rs + h * kHeadDim + d0;
    uint2 val;
    val.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    val.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2 *>(op) = val;
    if (p.lse != nullptr && d0 == 0) p.lse[((int64_t)b * p.H + h) * T + tq] = (m + __log2f(l)) * kLn2;
  }
}

Params make_params(const AttnArgs &a, int qb0, int nqb) {
  Params p{};
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
  p.nsplit = 1;
  p.tiles_per_split = a.nb;
  p.scale_log2 = a.scale_log2;
  return p;
}

}  // namespace

int dense_splits(int B, int H, int nb, int nvb) {
  const int nq = nb - nvb;
  if (nq <= 0) return 1;
  const int64_t units = (int64_t)B * H * nq;
  constexpr int64_t kTargetWorkgroups = 1024;   // ~4 per CU
  int s = (int)((kTargetWorkgroups + units - 1) / units);
  const int max_s = nb / 8 > 1 ? nb / 8 : 1;   // at least 8 tiles per split
  s = s < 1 ? 1 : (s > max_s ? max_s : s);
  // equalise tiles per split
  const int per = (nb + s - 1) / s;
  return (nb + per - 1) / per;
}

size_t dense_workspace_bytes(int B, int H, int nb, int nvb) {
  const int s = dense_splits(B, H, nb, nvb);
  if (s <= 1) return 0;
  const size_t rows = (size_t)B * H * (nb - nvb) * s * kBlock;
  return rows * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attn_sparse(const AttnArgs &a, hipStream_t stream) {
  if (a.nvb <= 0) return hipSuccess;
  const Params p = make_params(a, 0, a.nvb);
  const int total = a.B * a.H * a.nvb;
  hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_dense(const AttnArgs &a, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const int nq = a.nb - a.nvb;
  if (nq <= 0) return hipSuccess;
  Params p = make_params(a, a.nvb, nq);
  const int s = dense_splits(a.B, a.H, a.nb, a.nvb);
  if (s > 1 && workspace != nullptr && workspace_bytes >= dense_workspace_bytes(a.B, a.H, a.nb, a.nvb)) {
    p.nsplit = s;
    p.tiles_per_split = (a.nb + s - 1) / s;
    const size_t rows = (size_t)a.B * a.H * nq * s * kBlock;
    p.part_o = static_cast<float *>(workspace);
    p.part_ml = p.part_o + rows * kHeadDim;
  }
  const int total = a.B * a.H * nq * p.nsplit;
  hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(total), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.B * a.H * nq), dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
