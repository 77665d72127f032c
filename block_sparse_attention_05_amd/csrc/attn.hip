// Block-sparse flash attention on gfx950 bf16 MFMA, one query block per
// workgroup.  It serves block lists longer than the paired kernel
// (attn_pair.hip) takes (over 512 entries, or over 504 with the approximate
// branch of virtual summary keys); the plain sparse rows, the dense rows,
// the fused route and the approximate branch otherwise run on the paired
// kernel.
// This file also holds the combine kernel of the split-KV dense rows and the
// launch dispatch between the two kernels.
//
// Page "Sol-Attn and Spark for MiniMax-H3", Spark inference integration:
// selected K/V tiles stream through a single FP32 online-softmax/output
// accumulator.  Page "Add key bias to chunked Sol-Attn producers", Summary /
// Contract: the natural-log key bias is converted to log2 units and consumed
// only by the exact branch (sink keys).
//
// Workgroup = one 64-row query block of one (b, h), four wavefronts: wave w owns query
// rows 32*(w&1)..+31 and keys 32*(w>>1)..+31 of every 64-key tile, with its
// own online-softmax state; the two key halves of each row are merged at the
// end, each of the two waves of a row finishing and storing half of its
// columns.
//
// Only rows in [row_lo, row_hi) are written.  That is how a query block split
// by the video boundary is served: in the pad video tail mode (same page, H3
// pipeline integration) the sparse path writes its real video rows and the
// dense path its context rows.  The pages fill the block's non-video query
// slots with the mean Q of its real rows; here those slots keep the context
// rows' Q and their results are dropped.  The outputs are the same: a query
// row's softmax and output do not depend on the other rows of its block, and
// the block's routing centroid (the real rows' mean) is formed by the pooling
// kernel.
//
// Data movement.  K and V tiles (64 keys x 256 B) go from HBM/L2 straight to
// LDS with buffer_load ... lds (no register staging): the tile's base is in
// the per-lane offset, so keys past T fall outside the buffer range and read
// as zero.  The LDS layout (see below) makes every operand read a constant
// offset from one base and free of bank conflicts.
//
// Math per tile (per wave, 32 rows x 32 keys):
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, K fragments from LDS, Q^T
//     fragments resident in registers.  Each lane then owns one query row and
//     16 keys, so the row reductions are in-lane plus one v_permlane32_swap;
//   * online softmax in base 2 (scale * log2 e folded into one FMA) with lazy
//     rescaling: a full tile takes P against the running max as it stands
//     and moves it only when a P would exceed 2^32 (no tile max); a masked
//     tile moves it when the tile max grows by more than 8; the row sum
//     accumulates the bf16-rounded P with v_dot2;
//   * O^T += V^T P^T: P^T fragments come straight from the S^T registers, V^T
//     fragments from the row-major V tile through ds_read_b64_tr_b16 (each
//     16-lane group reads a 4-row block, lane c receives column c).  Keys in a
//     16-key group are contracted in the order {4g..4g+3, 8+4g..8+4g+3}
//     (g = lane / 32) on both operands.
//
// Schedule.  K tiles are fetched two tiles ahead and V tiles one ahead (two
// LDS slots each), so step j issues the MFMAs of S(j+1) = K(j+1) Q^T together
// with the softmax VALU work of tile j, interleaved by sched_group_barrier,
// then O += V(j) P(j).  The exponentials of tile j are
// taken after the (rare, lazily triggered) rescale that follows the tile max.
// Sink tiles (the only biased ones) always form a suffix of the tile
// sequence and the only partial tile is the last one, so every steady-state
// step is straight-line code.
#include <type_traits>

#include "attn_common.h"
#include "device_util.h"
#include "kernels.h"
#include "select.h"

namespace sa {
namespace {

using namespace attn;

constexpr int kKOff = 0;                    // K ring: 2 x 16 KiB
constexpr int kVOff = 32768;                // V ring: 2 x 16 KiB
constexpr int kBOff = 65536;                // bias ring: 2 x 256 B
constexpr int kLdsBytes = 65536 + 512;
// Approximate branch: virtual-key logit bias (kMaxRouteBlocks floats), 64
// zeros (bias of the sink tiles without key_bias), summary row of each
// virtual key (kMaxRouteBlocks ints).
constexpr int kVbOff = kLdsBytes;
constexpr int kVrowOff = kVbOff + kMaxRouteBlocks * 4 + 256;
constexpr int kVflagOff = kVrowOff + kMaxRouteBlocks * 4;   // one byte per video block
constexpr int kVbBytes = kMaxRouteBlocks * 9 + 256;
// Fused route: the query block's pooled mean (128 fp64), its scores
// against every key block, its list and the list length.
constexpr int kFqOff = kLdsBytes;
constexpr int kFsOff = kFqOff + kHeadDim * 8;
constexpr int kFlOff = kFsOff + kMaxRouteBlocks * 4;
constexpr int kFnOff = kFlOff + kMaxRouteBlocks * 4;
constexpr int kFusedBytes = kHeadDim * 8 + kMaxRouteBlocks * 8 + 16;

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
  int row_lo, row_hi;  // rows written: [row_lo, row_hi)
  int nsplit, tiles_per_split;
  float scale_log2;
  // approximate branch: summaries of (b, h) at sum_k/sum_v + bh*nb*128 and
  // sum_lm + bh*nb
  const uint16_t *sum_k, *sum_v;
  const float *sum_lm;
  // fused route: pooled means (route workspace layout), budget, radius, and
  // optional copies of the lists it selects
  const double *qbar;
  const float *kbar;
  int budget, radius;
  int32_t *list_out, *cnt_out;
};

template <bool kSpark = false, bool kFused = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_kernel(Params p) {
  // K ring (2 tiles) | V ring (2 tiles) | natural-log key bias ring (2 tiles)
  // [| virtual-key bias, approximate branch] [| fused route]
  __shared__ __align__(16) unsigned char smem[kLdsBytes + (kSpark ? kVbBytes : 0) +
                                              (kFused ? kFusedBytes : 0)];

  const int total = p.B * p.H * p.nqb;
  const int wq = xcd_remap(blockIdx.x, total);
  const int qbi = wq % p.nqb;
  const int bh = wq / p.nqb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int qb = p.qb0 + qbi;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR
  const int rw = wave & 1;     // query rows 32*rw .. +31 of the block
  const int kh = wave >> 1;    // keys 32*kh .. +31 of every tile
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int T = p.T;
  const int64_t rs = (int64_t)p.H * kHeadDim;   // elements per token
  const int row_bytes = p.H * kHeadDim * 2;
  const int64_t bbase = (int64_t)b * T * rs;

  // ---- tile sequence ------------------------------------------------------
  // Sparse: the block list is held in VGPR lanes (lane j = entry cb + j of
  // the current 64-entry chunk) and read with v_readlane, so no memory round
  // trip sits between tiles.  Lists are ascending, so sink blocks (>= nvb)
  // form a suffix.
  const float *kbias = p.key_bias ? p.key_bias + (int64_t)b * T : nullptr;
  int t_begin = 0, t_end;
  int n_plain;                  // tiles before the first biased (sink) tile
  const int32_t *list = nullptr;
  int list_cb = 0;
  int list_v = 0;   // entries list_cb .. +63
  int list_nv = 0;  // entries list_cb + 64 .. +63, loaded one tile early
  {
    const int64_t li = (int64_t)bh * p.nqb + qbi;
    int first, n;
    if (kFused) {
      // Route of this query block inside the workgroup (same rule as the
      // route kernel): scores s_j = fp32 of the fp64 dot product of the
      // fp32 means (fp32 products are exact in fp64), then one wavefront
      // selects and emits the list into LDS.
      double *qs = reinterpret_cast<double *>(smem + kFqOff);
      float *sc = reinterpret_cast<float *>(smem + kFsOff);
      int32_t *lst = reinterpret_cast<int32_t *>(smem + kFlOff);
      int32_t *lcnt = reinterpret_cast<int32_t *>(smem + kFnOff);
      const int ntq = (p.nqb + 15) >> 4, ntk = (p.nvb + 15) >> 4;
      if (tid < kHeadDim / 2) {  // channels 2*tid, 2*tid + 1
        const double2 w2 = reinterpret_cast<const double2 *>(p.qbar)
            [(((int64_t)bh * ntq + (qb >> 4)) * 16 + (tid & 15)) * 64 + 16 * (tid >> 4) + (qb & 15)];
        qs[2 * tid] = w2.x;
        qs[2 * tid + 1] = w2.y;
      }
      __syncthreads();
      const float4 *kt = reinterpret_cast<const float4 *>(p.kbar) + (int64_t)bh * ntk * 8 * 64;
      for (int jb = tid; jb < p.nvb; jb += kThreads) {
        const float4 *kj = kt + (int64_t)(jb >> 4) * 8 * 64 + (jb & 15);
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
#pragma unroll 8
        for (int u = 0; u < kHeadDim / 4; ++u) {  // channels 4u .. 4u+3
          const float4 kv = kj[(u & 7) * 64 + 16 * (u >> 3)];
          a0 = __builtin_fma(qs[4 * u + 0], (double)kv.x, a0);
          a1 = __builtin_fma(qs[4 * u + 1], (double)kv.y, a1);
          a2 = __builtin_fma(qs[4 * u + 2], (double)kv.z, a2);
          a3 = __builtin_fma(qs[4 * u + 3], (double)kv.w, a3);
        }
        sc[jb] = (float)((a0 + a1) + (a2 + a3));
      }
      __syncthreads();
      if (wave == 0) {
        // slots per lane sized to nvb (the selection loops over all of them)
        auto sel = [&](auto e_c) {
          return select_and_emit<decltype(e_c)::value>(sc, qb, p.nvb, p.nb, p.budget, p.radius,
                                                      p.max_sel, lst, nullptr, lane);
        };
        const int c = p.nvb <= 128 ? sel(Int<2>{}) : p.nvb <= 192 ? sel(Int<3>{})
                    : p.nvb <= 256 ? sel(Int<4>{}) : sel(Int<kMaxRouteBlocks / 64>{});
        if (lane == 0) *lcnt = c;
        if (p.list_out != nullptr) {
          for (int x = lane; x < p.max_sel; x += 64) p.list_out[li * p.max_sel + x] = lst[x];
          if (lane == 0) p.cnt_out[li] = c;
        }
      }
      __syncthreads();
      list = lst;
      first = lane < p.max_sel ? lst[lane] : 0;
      n = *lcnt;
    } else {
      list = p.block_idx + li * p.max_sel;
      // The first 64 entries are read together with the count (the two
      // loads do not depend on each other).
      first = lane < p.max_sel ? list[lane] : 0;
      n = p.block_cnt[li];
    }
    const int t_cnt = n < 0 ? 0 : (n > p.max_sel ? p.max_sel : n);
    list_v = lane < t_cnt ? first : 0;
    // An ascending list holds its entries outside [0, NB) as a prefix (< 0)
    // and a suffix (>= NB); the tiles are the entries between them, video
    // blocks (< NVB) first.  Count the groups over all 64-entry chunks.
    int n_neg = 0, n_valid = 0;
    n_plain = 0;
    for (int cb = 0; cb < t_cnt; cb += 64) {
      const bool in = cb + lane < t_cnt;
      const int e = cb == 0 ? list_v : (in ? list[cb + lane] : 0);
      n_neg += __popcll(__ballot(in && e < 0));
      n_valid += __popcll(__ballot(in && e >= 0 && e < p.nb));
      n_plain += __popcll(__ballot(in && e >= 0 && e < p.nvb));
    }
    t_begin = n_neg;
    t_end = n_neg + n_valid;
    if (t_begin >= 64) {   // the first tile lies past the first chunk
      list_cb = t_begin & ~63;
      list_v = list_cb + lane < t_end ? list[list_cb + lane] : 0;
    }
  }
  const int n = t_end - t_begin;  // exact tiles
  // With the approximate branch, nv virtual tiles (64 block summaries each)
  // sit between the exact video tiles and the sink tiles (without key_bias,
  // between the complete sink tiles and a partial last block), and every
  // tile from the first virtual one on is biased: virtual tiles by their
  // log-mass, sink tiles by key_bias (or zero without it).  The biased tiles
  // stay a suffix and the partial tile stays last.
  // The virtual keys are the video blocks the list skips, packed in
  // ascending order: nvb minus the list's video entries.
  // (A caller list with repeated video entries can count more of them than
  // there are video blocks; no virtual tile then.)
  const int nv = (kSpark && p.nvb > n_plain) ? (p.nvb - n_plain + kBlock - 1) / kBlock : 0;
  const int nt = nv + n;
  if (!kSpark && kbias == nullptr) n_plain = n;
  // Approximate branch without key_bias: sink tiles carry no bias, so the
  // complete ones run with the video tiles, before the virtual tiles; only a
  // partial last block (always the last list entry) follows those.
  if (kSpark && kbias == nullptr && nv > 0) n_plain = (T % kBlock != 0) ? n - 1 : n;
  const int np_end = n_plain;          // tiles [0, np_end) are unbiased
  auto is_virt = [&](int j) { return kSpark && (uint32_t)(j - np_end) < (uint32_t)nv; };

  // Q^T fragments for this lane's query row: d = 16*dc + 8*g + [0, 8).  The
  // block's 64 Q rows are copied once into V slot 1 (free until step 0) with
  // the first tiles, in the K tile layout, and each wave reads its fragments
  // from there after the prologue's barrier.
  const int tq = qb * kBlock + rw * 32 + c32;
  bf16x8 qf[8];

  // First token of tile t_begin + j; calls come with j = 0, 1, 2, ... in
  // order.  An entry outside [0, NB) between valid ones (only in a list that
  // is not ascending, whose results are unspecified) maps to T: its tile
  // reads as zero and every access stays in bounds.
  // The next 64-entry chunk is loaded one call before it is needed, so that
  // the end-of-step wait already covers it: a wait placed by the compiler at
  // the use would also drain the K/V tile loads in flight.
  // A virtual tile returns its first summary index instead.
  auto tile_key0 = [&](int j) -> int {
    if (kSpark && j >= np_end) {
      if (j < np_end + nv) return kBlock * (j - np_end);
      j -= nv;
    }
    const int it = t_begin + j;
    if (it - list_cb >= 64) {
      list_cb += 64;
      list_v = list_nv;
    }
    const int kb = __builtin_amdgcn_readlane(list_v, it - list_cb);
    if (it - list_cb == 63 && list_cb + 64 < t_end) {
      const int e = list_cb + 64 + lane;
      list_nv = e < t_end ? list[e] : 0;
    }
    return (kb >= 0 && kb < p.nb) ? kb * kBlock : T;
  };

  // ---- loads --------------------------------------------------------------
  const uint32_t slab = (uint32_t)T * (uint32_t)row_bytes;
  const i32x4s rk = buffer_rsrc(p.k + bbase, slab);
  const i32x4s rqd = buffer_rsrc(p.q + bbase, slab);
  const i32x4s rv = buffer_rsrc(p.v + bbase, slab);
  const i32x4s rb = buffer_rsrc(kbias ? (const void *)kbias : (const void *)p.k, kbias ? T * 4u : 0u);
  const int sink0 = p.nvb * kBlock;

  // LDS tile layout.  A tile slot (K or V, 64 keys x 256 B) is 16 blocks of
  // 1 KiB; block 2*kg + hf holds keys 8*kg .. +7 and bytes 128*hf .. +127 of
  // each key row, one 128-byte row per key, in 16-byte pieces (key k' = key%8,
  // chunk c = 0..7) placed with an XOR swizzle:
  //   K: piece (k', c) at 128*k' + 16*(c ^ k' ^ (kg & 1));
  //   V: piece (k', c) at 128*k' + 16*(c ^ 2*(k' & 3)).
  // One buffer_load ... lds instruction writes 1 KiB (16 B per lane, in lane
  // order), so each group of 8 lanes fetches the full 128-byte cache line
  // half of one key row (8 lines per instruction).  The swizzles make the
  // MFMA operand reads conflict-free on the 64 four-byte banks: a K fragment
  // read (ds_read_b128) serves 16 lanes per cycle, 8 keys of an even and 8
  // of an odd key group; within a group the k' swizzle spreads one chunk of
  // the 8 keys over half of the banks and the kg parity sends the two groups
  // to opposite halves.  Each 16-lane group of ds_read_b64_tr_b16 on V
  // (4 keys x 32 B) covers 32 distinct banks.  With these, the K fragment of
  // MFMA lane l (key 32kh + l%32, channels 16dc + 8(l/32) .. +7) sits at
  // (k_rd0 ^ 32*(dc%4)) + 1024*(dc/4), and the
  // ds_read_b64_tr_b16 source of lane l (key 32kh + 16kc + 8u + 4g + r,
  // channels 32dt + 16dh + 4j .. +3; g = l/32, dh = (l/16)%2, r = (l%16)/4,
  // j = l%4) at (v_rd0 ^ 64*(dt%2)) + 4096*kc + 2048*u + 1024*(dt/2).  Wave w loads
  // blocks 4w .. 4w+3 (keys 16w .. +15).
  const uint32_t k_lane = (uint32_t)((16 * wave + (lane >> 3)) * row_bytes + h * 256 +
                                     16 * ((lane & 7) ^ (lane >> 3)));
  const uint32_t v_lane = (uint32_t)((16 * wave + (lane >> 3)) * row_bytes + h * 256 +
                                     16 * ((lane & 7) ^ (2 * ((lane >> 3) & 3))));
  const uint32_t rows8 = (uint32_t)(8 * row_bytes);
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(LDS_PTR(unsigned char, smem));
  const uint32_t wave_lds = (uint32_t)__builtin_amdgcn_readfirstlane(4096 * wave);
  // Summary rows (approximate branch) are 256 B apart, one (b, h) slab of
  // nb rows.  A virtual tile gathers the rows of its 64 virtual keys (the
  // skipped blocks, listed in LDS); same LDS placement as K/V rows.
  const int64_t sbase = (int64_t)bh * p.nb * kHeadDim;
  const i32x4s rsk = buffer_rsrc(kSpark ? p.sum_k + sbase : p.k, kSpark ? (uint32_t)p.nb * 256u : 0u);
  const i32x4s rsv = buffer_rsrc(kSpark ? p.sum_v + sbase : p.v, kSpark ? (uint32_t)p.nb * 256u : 0u);
  // (The summary-row lane offsets are formed where used, so that they hold
  // no registers through the exact-tile loops.)
  const int *vrow = reinterpret_cast<const int *>(smem + kVrowOff);
  auto issue_k = [&](int key0, int slot, bool virt) {
    const uint32_t lb = lds0 + kKOff + (uint32_t)(slot * 16384) + wave_lds;
    if (kSpark && virt) {
      const int r = key0 + 16 * wave + (lane >> 3);
      const uint32_t sw = 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
      const uint32_t ba = (uint32_t)vrow[r] * 256u + sw, bb = (uint32_t)vrow[r + 8] * 256u + sw;
      lds_dma_b128<0>(rsk, ba, lb);
      lds_dma_b128<1024>(rsk, ba + 128, lb);
      lds_dma_b128<2048>(rsk, bb ^ 16u, lb);
      lds_dma_b128<3072>(rsk, (bb ^ 16u) + 128, lb);
      return;
    }
    const uint32_t base = (uint32_t)key0 * (uint32_t)row_bytes + k_lane;
    lds_dma_b128<0>(rk, base, lb);
    lds_dma_b128<1024>(rk, base + 128, lb);
    // odd key group: chunk parity flipped (the chunk term is the only part
    // of the offset below 256)
    lds_dma_b128<2048>(rk, (base ^ 16u) + rows8, lb);
    lds_dma_b128<3072>(rk, (base ^ 16u) + rows8 + 128, lb);
  };
  auto issue_v = [&](int key0, int slot, bool virt) {
    const uint32_t lb = lds0 + kVOff + (uint32_t)(slot * 16384) + wave_lds;
    if (kSpark && virt) {
      const int r = key0 + 16 * wave + (lane >> 3);
      const uint32_t sw = 16u * (uint32_t)((lane & 7) ^ (2 * ((lane >> 3) & 3)));
      const uint32_t ba = (uint32_t)vrow[r] * 256u + sw, bb = (uint32_t)vrow[r + 8] * 256u + sw;
      lds_dma_b128<0>(rsv, ba, lb);
      lds_dma_b128<1024>(rsv, ba + 128, lb);
      lds_dma_b128<2048>(rsv, bb, lb);
      lds_dma_b128<3072>(rsv, bb + 128, lb);
      return;
    }
    const uint32_t base = (uint32_t)key0 * (uint32_t)row_bytes + v_lane;
    lds_dma_b128<0>(rv, base, lb);
    lds_dma_b128<1024>(rv, base + 128, lb);
    lds_dma_b128<2048>(rv, base + rows8, lb);
    lds_dma_b128<3072>(rv, base + rows8 + 128, lb);
    if (kbias != nullptr && key0 >= sink0 && key0 < T && wave == 0)
      lds_dma_b32(rb, (uint32_t)(key0 + lane) * 4u, lds0 + kBOff + (uint32_t)(slot * 256));
  };
  // operand read bases (bytes within a slot)
  // The other operand bases differ by an XOR of the swizzled chunk bits:
  // K chunk 2*(dc%4) + g lands at k_rd0 ^ (32*(dc%4)); V for odd dt at
  // v_rd0 ^ 64.
  uint32_t k_rd0, v_rd0;
  {
    const uint32_t kp = (uint32_t)(c32 & 7);
    k_rd0 = (uint32_t)(2048 * (4 * kh + (c32 >> 3))) + 128 * kp +
            16 * ((uint32_t)g ^ kp ^ (uint32_t)((c32 >> 3) & 1));
    const uint32_t r = (uint32_t)((lane & 15) >> 2), dh = (uint32_t)((lane >> 4) & 1), j = (uint32_t)(lane & 3);
    v_rd0 = (uint32_t)(8192 * kh + 512 * g) + 128 * r + 8 * (j & 1) + 16 * ((2 * dh + (j >> 1)) ^ (2 * r));
  }

  // ---- state --------------------------------------------------------------
  float m_used = -INFINITY;   // running max (log2 units) used for P
  float l_run = 0.f;          // this lane's share of the row sum
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const float c = p.scale_log2;

  // Bias of biased tile j (approximate branch): the virtual-key bias array
  // at the tile's first summary index, or the key-bias ring slot, or zeros.
  const float *vbp = reinterpret_cast<const float *>(smem + kVbOff);
  const float *sink_b0 = kbias != nullptr ? reinterpret_cast<const float *>(smem + kBOff) : vbp + kMaxRouteBlocks;
  const int sink_step = kbias != nullptr ? 64 : 0;   // floats between the two ring slots
  auto bias_src = [&](int j, int vs, int key0) -> const float * {
    return is_virt(j) ? vbp + key0 : sink_b0 + vs * sink_step;
  };

  // One pipeline step on tile j (scores in s_cur, V in slot VS) that also
  // computes S(j+1) into s_nxt from K slot VS^1 when DO_QK.  With the
  // approximate branch a biased step reads its bias at bsel.
  auto step = [&](auto vs_c, auto biased_c, auto masked_c, auto do_qk_c, f32x16 &s_cur,
                  f32x16 &s_nxt, int key0, const float *bsel) {
    constexpr int VS = decltype(vs_c)::value;
    constexpr bool BIASED = decltype(biased_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr bool DO_QK = decltype(do_qk_c)::value;
    const unsigned char *vbuf = smem + kVOff + VS * 16384;
    const unsigned char *kbuf = smem + kKOff + (VS ^ 1) * 16384;
    const float *bs = kSpark ? bsel : reinterpret_cast<const float *>(smem + kBOff + VS * 256);

    // S(j+1) MFMAs, issued in two groups so that they overlap the max phase
    // and the exponential phase of tile j.  Their K fragments are read from
    // LDS a few MFMAs ahead of use, so that the LDS latency is not paid once
    // per MFMA.
    auto qk_part = [&](auto lo_c, auto hi_c) {
      constexpr int LO = decltype(lo_c)::value;
      constexpr int HI = decltype(hi_c)::value;
#pragma unroll
      for (int dc = LO; dc < HI; ++dc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbuf + (k_rd0 ^ (32u * (dc & 3))) + 1024 * (dc >> 2));
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s_nxt, 0, 0, 0);
      }
    };

    // -- block A: max of tile j (+ first S(j+1) MFMAs) --
    if (DO_QK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[r] = 0.f;
      qk_part(Int<0>{}, Int<3>{});
    }
    if (MASKED) {
      const int kbase = key0 + 32 * kh + 4 * g;   // key of s[r] = kbase + 8*(r/4) + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 8 * (r >> 2) + (r & 3) >= T) s_cur[r] = -INFINITY;
    }
    // Logits in log2 units: s*c (+ beta2 on sink tiles).  The bias is read
    // from LDS in both phases (instead of being held in registers) and the
    // exponent is formed as fma(s, c, beta2 - m), so that beta2 = 0 reproduces
    // the unbiased fma(s, c, -m) bit for bit.
    auto bias4 = [&](int q4) {
      const float4 b4 = *reinterpret_cast<const float4 *>(bs + 32 * kh + 8 * q4 + 4 * g);
      return make_float4(b4.x * kLog2e, b4.y * kLog2e, b4.z * kLog2e, b4.w * kLog2e);
    };
    // tile max of this lane's logits (log2 units), shared with the lane that
    // holds the other 16 keys of the row
    auto tile_max = [&]() -> float {
      float mt;
      if (BIASED) {
        mt = -INFINITY;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 bq = bias4(q4);
          mt = fmaxf(mt, __builtin_fmaf(s_cur[4 * q4 + 0], c, bq.x));
          mt = fmaxf(mt, __builtin_fmaf(s_cur[4 * q4 + 1], c, bq.y));
          mt = fmaxf(mt, __builtin_fmaf(s_cur[4 * q4 + 2], c, bq.z));
          mt = fmaxf(mt, __builtin_fmaf(s_cur[4 * q4 + 3], c, bq.w));
        }
      } else {
        float mx = s_cur[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_cur[r]);
        mt = mx * c;
      }
      return max_with_partner(mt);
    };
    auto rescale_to = [&](float m_new) {
      const float alpha = m_new > m_used ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.f;  // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_used = m_new;
    };
    // P of tile j against m_sub into pf, their sum added to acc
    bf16x8 pf[2];
    auto exps = [&](float m_sub, float &acc) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
        if (BIASED) {
          const float4 bq = bias4(q4);
          e[0] = __builtin_fmaf(s_cur[4 * q4 + 0], c, bq.x - m_sub);
          e[1] = __builtin_fmaf(s_cur[4 * q4 + 1], c, bq.y - m_sub);
          e[2] = __builtin_fmaf(s_cur[4 * q4 + 2], c, bq.z - m_sub);
          e[3] = __builtin_fmaf(s_cur[4 * q4 + 3], c, bq.w - m_sub);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) e[u] = __builtin_fmaf(s_cur[4 * q4 + u], c, -m_sub);
        }
#pragma unroll
        for (int u = 0; u < 4; u += 2) {
          const int r = 4 * q4 + u;
          const bf16x2 pk = {(__bf16)__builtin_amdgcn_exp2f(e[u]), (__bf16)__builtin_amdgcn_exp2f(e[u + 1])};
          acc = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, acc, false);
          pf[r >> 3][r & 7] = pk[0];
          pf[r >> 3][(r & 7) + 1] = pk[1];
        }
      }
    };
    float m_sub = m_used;
    if (MASKED) {
      // masked tiles: the tile max first, the running max moved when it
      // grows by more than the slack
      const float mt = tile_max();
      if (DO_QK) {
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 3, 0);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedVALU, 4, 0);
        }
      }
      if (__any(mt > m_used + kRescaleSlack)) rescale_to(fmaxf(m_used, mt));
      m_sub = (m_used == -INFINITY) ? 0.f : m_used;
    }

    // -- block B: P of tile j (+ remaining S(j+1) MFMAs) --
    // Full tiles take P against the running max as it stands (no tile max);
    // a P above 2^32 (the running max stale by more than 32, or not yet set:
    // P = +inf) shows in the tile's sum, and then, rarely, the tile max moves
    // the running max and the tile's P are taken again.
    // The exponential and PV phases run at raised wave priority: when the
    // other workgroup's wave on this SIMD is in its max phase, issuing copies
    // or waiting at its barrier, this wave's VALU and MFMA work goes first.
    __builtin_amdgcn_s_setprio(1);
    if (DO_QK) qk_part(Int<3>{}, Int<8>{});
    float l_t = 0.f;   // full tiles: this lane's share of the tile's row sum
    if (MASKED) exps(m_sub, l_run);
    else exps(m_used, l_t);
    if (DO_QK) {
      __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, 8, 0);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, 8, 0);
      }
    }
    if (!MASKED) {
      // a sum of non-negative terms is at least its largest term; NaN (an
      // infinite logit meeting an infinite max) fails the test too
      if (__any(!(l_t <= kPMax))) {
        rescale_to(fmaxf(m_used, tile_max()));
        l_t = 0.f;
        exps(m_used == -INFINITY ? 0.f : m_used, l_t);
      }
      l_run += l_t;
    }

    // -- block C: O^T += V^T P^T over this wave's 32 keys --
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const unsigned char *src = vbuf + ((dt & 1) ? (v_rd0 ^ 64u) : v_rd0) + 4096 * kc + 1024 * (dt >> 1);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, src));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, src + 2048));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kc], o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- pipeline -----------------------------------------------------------
  // K(j) lives in K slot j%2 and V(j) in V slot j%2; K is fetched two tiles
  // ahead, V one ahead.  Step j issues V(j+1) and K(j+2) into the slots that
  // step j-1 finished reading, and ends with the barrier that publishes them.
  // Virtual keys: the video blocks the list skips, ascending.  A byte flag
  // per video block marks the list's blocks (the first 64 entries are
  // already in list_v); then every wave walks all 64-block chunks, packs the
  // unflagged blocks by ballot and writes the chunks c = wave mod 4: summary
  // row and log-mass bias at the packed position, -inf bias past the last
  // one.  The zero bias of unbiased sink tiles follows the bias array.
  // Built after the first tile loads are issued unless those tiles are
  // virtual themselves.
  auto build_virtual = [&]() {
    float *vb = reinterpret_cast<float *>(smem + kVbOff);
    int *vr = reinterpret_cast<int *>(smem + kVrowOff);
    unsigned char *fl = smem + kVflagOff;
    const float *lmp = p.sum_lm + (int64_t)bh * p.nb;
    for (int x = tid; 4 * x < p.nvb; x += kThreads) reinterpret_cast<uint32_t *>(fl)[x] = 0u;
    __syncthreads();
    for (int cb = 64 * wave; cb < t_end; cb += kThreads) {
      // list_v still holds the first chunk unless the walk started past it
      const int e = (cb == 0 && list_cb == 0) ? list_v : (cb + lane < t_end ? list[cb + lane] : -1);
      if (cb + lane < t_end && e >= 0 && e < p.nvb) fl[e] = 1;
    }
    __syncthreads();
    int base = 0;
    for (int c = 0; c * kBlock < p.nvb; ++c) {
      const int x = kBlock * c + lane;
      const bool skip = x < p.nvb && fl[x] == 0;
      const uint64_t m = __ballot(skip);
      if ((c & 3) == wave && skip) {
        const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
        vr[pos] = x;
        vb[pos] = lmp[x];
      }
      base += __popcll(m);
    }
    for (int x = base + tid; x < nv * kBlock; x += kThreads) {
      vr[x] = 0;
      vb[x] = -INFINITY;
    }
    if (tid < kBlock) vb[kMaxRouteBlocks + tid] = 0.f;
  };
  const bool virt_first = is_virt(0) || is_virt(1);
  if (kSpark && virt_first) {
    build_virtual();
    __syncthreads();
  }

  f32x16 s0, s1;
  int k_cur = 0, k_nxt = 0;
  if (nt > 0) {
    k_cur = tile_key0(0);
    issue_k(k_cur, 0, is_virt(0));
    issue_v(k_cur, 0, is_virt(0));
    if (nt > 1) {
      k_nxt = tile_key0(1);
      issue_k(k_nxt, 1, is_virt(1));
    }
  }
  {   // Q rows of the block into V slot 1, K tile layout
    const uint32_t base = (uint32_t)(qb * kBlock) * (uint32_t)row_bytes + k_lane;
    const uint32_t lb = lds0 + kVOff + 16384u + wave_lds;
    lds_dma_b128<0>(rqd, base, lb);
    lds_dma_b128<1024>(rqd, base + 128, lb);
    lds_dma_b128<2048>(rqd, (base ^ 16u) + rows8, lb);
    lds_dma_b128<3072>(rqd, (base ^ 16u) + rows8 + 128, lb);
  }
  if (kSpark && !virt_first) build_virtual();  // published by the barrier below
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  {
    const int qr = rw * 32 + c32, kg = qr >> 3, kp = qr & 7;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      const int ci = 2 * dc + g, hf = ci >> 3, cc = ci & 7;
      qf[dc] = *reinterpret_cast<const bf16x8 *>(smem + kVOff + 16384 + 1024 * (2 * kg + hf) + 128 * kp +
                                                 16 * (cc ^ kp ^ (kg & 1)));
    }
  }
  if (nt > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.f;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(smem + kKOff + (k_rd0 ^ (32u * (dc & 3))) + 1024 * (dc >> 2));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s0, 0, 0, 0);
    }
  }
  // Step 0 refills K slot 0: every wave must be done reading it.
  __syncthreads();

  // Steady-state step j < n-1 (S(j+1) computed); the last step is peeled and
  // is the only one that masks keys past T.
  auto run_step = [&](auto vs_c, auto biased, f32x16 &s_cur, f32x16 &s_nxt, int j) {
    constexpr int VS = decltype(vs_c)::value;
    const int key_j = k_cur;
    issue_v(k_nxt, VS ^ 1, is_virt(j + 1));
    int k_nn = 0;
    if (j + 2 < nt) {
      k_nn = tile_key0(j + 2);
      issue_k(k_nn, VS, is_virt(j + 2));
    }
    const float *bsel = kSpark ? bias_src(j, VS, key_j) : nullptr;
    step(vs_c, biased, Bool<false>{}, Bool<true>{}, s_cur, s_nxt, key_j, bsel);
    k_cur = k_nxt;
    k_nxt = k_nn;
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
  };
  auto last_step = [&](auto vs_c, f32x16 &s_cur, f32x16 &s_nxt) {
    constexpr int VS = decltype(vs_c)::value;
    const int key_j = k_cur;
    const bool masked = !is_virt(nt - 1) && key_j + kBlock > T;
    const float *bsel = kSpark ? bias_src(nt - 1, VS, key_j) : nullptr;
    if (nt - 1 >= np_end) {
      if (masked) step(vs_c, Bool<true>{}, Bool<true>{}, Bool<false>{}, s_cur, s_nxt, key_j, bsel);
      else step(vs_c, Bool<true>{}, Bool<false>{}, Bool<false>{}, s_cur, s_nxt, key_j, bsel);
    } else {
      if (masked) step(vs_c, Bool<false>{}, Bool<true>{}, Bool<false>{}, s_cur, s_nxt, key_j, bsel);
      else step(vs_c, Bool<false>{}, Bool<false>{}, Bool<false>{}, s_cur, s_nxt, key_j, bsel);
    }
    __syncthreads();
  };
  // Steps j < np_end are unbiased and the rest biased.  Each loop body holds
  // one step variant only: a runtime choice between the two inside a loop
  // makes the compiler route the O accumulators through copies every step.
  int j = 0;
  for (; j + 2 < nt && j + 2 <= np_end; j += 2) {
    run_step(Int<0>{}, Bool<false>{}, s0, s1, j);
    run_step(Int<1>{}, Bool<false>{}, s1, s0, j + 1);
  }
  if (j + 2 < nt && j < np_end) {  // j + 1 == np_end
    run_step(Int<0>{}, Bool<false>{}, s0, s1, j);
    run_step(Int<1>{}, Bool<true>{}, s1, s0, j + 1);
    j += 2;
  }
  for (; j + 2 < nt; j += 2) {
    run_step(Int<0>{}, Bool<true>{}, s0, s1, j);
    run_step(Int<1>{}, Bool<true>{}, s1, s0, j + 1);
  }
  if (j + 1 < nt) {
    if (j >= np_end)
      run_step(Int<0>{}, Bool<true>{}, s0, s1, j);
    else
      run_step(Int<0>{}, Bool<false>{}, s0, s1, j);
    last_step(Int<1>{}, s1, s0);
  } else if (j < nt) {
    last_step(Int<0>{}, s0, s1);
  }

  // ---- merge the two key halves of every row ------------------------------
  // Each wave finishes half of the columns of its 32 rows (the kh = 0 wave
  // d in [0, 64), the kh = 1 wave d in [64, 128)): it hands the other half of
  // its O^T and its (m, l) to its partner through LDS, merges, normalises and
  // stores.  Both waves merge in the same order, key half 0 first, so the two
  // halves of a row get the same max and sum.
  float l_tot = add_with_partner(l_run);
  float4 *xo = reinterpret_cast<float4 *>(smem);              // [rw][kh][8 quads][64 lanes]
  float2 *xml = reinterpret_cast<float2 *>(smem + kVOff);     // [kh][rw][32 rows]
  auto hand_over = [&](auto ds_c) {   // the partner's column tiles ds, ds + 1
    constexpr int DS = decltype(ds_c)::value;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        xo[((rw * 2 + kh) * 8 + u * 4 + rq) * 64 + lane] =
            make_float4(o[DS + u][4 * rq], o[DS + u][4 * rq + 1], o[DS + u][4 * rq + 2], o[DS + u][4 * rq + 3]);
  };
  if (kh == 0)
    hand_over(Int<2>{});
  else
    hand_over(Int<0>{});
  if (g == 0) xml[(kh * 2 + rw) * 32 + c32] = make_float2(m_used, l_tot);
  __syncthreads();

  auto finish = [&](auto dt_c) {   // this wave's column tiles dt0, dt0 + 1
    constexpr int DT0 = decltype(dt_c)::value;
    constexpr bool MINE_FIRST = DT0 == 0;   // this wave holds key half 0
    const float2 mlb = xml[((kh ^ 1) * 2 + rw) * 32 + c32];
    const float m0 = MINE_FIRST ? m_used : mlb.x, l0 = MINE_FIRST ? l_tot : mlb.y;
    const float m1 = MINE_FIRST ? mlb.x : m_used, l1 = MINE_FIRST ? mlb.y : l_tot;
    const float m = fmaxf(m0, m1);
    const float msub = (m == -INFINITY) ? 0.f : m;
    const float a0 = __builtin_amdgcn_exp2f(m0 - msub);
    const float a1 = __builtin_amdgcn_exp2f(m1 - msub);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 ob = xo[((rw * 2 + (kh ^ 1)) * 8 + u * 4 + rq) * 64 + lane];
        const float pb[4] = {ob.x, ob.y, ob.z, ob.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = MINE_FIRST ? o[DT0 + u][4 * rq + e] : pb[e];
          const float x1 = MINE_FIRST ? pb[e] : o[DT0 + u][4 * rq + e];
          o[DT0 + u][4 * rq + e] = __builtin_fmaf(x0, a0, x1 * a1);
        }
      }
    l_tot = __builtin_fmaf(l0, a0, l1 * a1);
    m_used = m;

    // The wave's 32 half rows (128 B) go through LDS (a free part of the V
    // ring, 16-byte chunks XOR-swizzled by row) and out as whole half rows:
    // each store instruction writes eight 128-byte half rows.
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    unsigned char *stage = smem + kVOff + 8192 + (rw * 2 + kh) * 4096;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        uint2 val;
        val.x = pack_bf16x2(o[DT0 + u][4 * rq + 0] * inv, o[DT0 + u][4 * rq + 1] * inv);
        val.y = pack_bf16x2(o[DT0 + u][4 * rq + 2] * inv, o[DT0 + u][4 * rq + 3] * inv);
        *reinterpret_cast<uint2 *>(stage + c32 * 128 + 16 * ((4 * u + rq) ^ (c32 & 7)) + 8 * g) = val;
      }
    const int row0 = qb * kBlock + rw * 32;
    uint16_t *ob = p.out + bbase + h * kHeadDim + 64 * kh;
    const int ch = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      const uint4 val = *reinterpret_cast<const uint4 *>(stage + r * 128 + 16 * (ch ^ (r & 7)));
      if (row0 + r >= p.row_lo && row0 + r < p.row_hi)
        *reinterpret_cast<uint4 *>(ob + (int64_t)(row0 + r) * rs + 8 * ch) = val;
    }
    if (MINE_FIRST && p.lse != nullptr && g == 0 && tq >= p.row_lo && tq < p.row_hi)
      p.lse[((int64_t)b * p.H + h) * T + tq] = (m_used + __log2f(l_tot)) * kLn2;
  };
  if (kh == 0)
    finish(Int<0>{});
  else
    finish(Int<2>{});
}

// Merge the split-KV partials of the dense rows: one thread per (row, 4
// channels), 8 rows per workgroup.
// m* = max_s m_s, O = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s.
constexpr int kCombineThreads = 256;
constexpr int kCombineRows = kCombineThreads / (kHeadDim / 4);
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(Params p) {
  constexpr int kChunks = kBlock / kCombineRows;
  const int wq = blockIdx.x / kChunks;     // (b*H + h) * nqb + qbi
  const int qbi = wq % p.nqb;
  const int bh = wq / p.nqb;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int T = p.T;
  const int64_t rs = (int64_t)p.H * kHeadDim;
  const int row = (blockIdx.x % kChunks) * kCombineRows + threadIdx.x / (kHeadDim / 4);
  const int d0 = (threadIdx.x % (kHeadDim / 4)) * 4;
  const int tq = (p.qb0 + qbi) * kBlock + row;
  if (tq < p.row_lo || tq >= p.row_hi) return;
  const int64_t prow0 = (int64_t)wq * p.nsplit * kBlock + row;   // split s: prow0 + s * kBlock
  // Up to kCombineRegs splits are loaded at once (one memory round trip),
  // then merged in split order; more splits take a second pass per group.
  constexpr int kCombineRegs = 4;
  float m = -INFINITY;
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.nsplit <= kCombineRegs) {
    float2 ml[kCombineRegs];
    float4 po[kCombineRegs];
#pragma unroll
    for (int s = 0; s < kCombineRegs; ++s) {
      if (s < p.nsplit) {
        const int64_t prow = prow0 + (int64_t)s * kBlock;
        ml[s] = *reinterpret_cast<const float2 *>(p.part_ml + 2 * prow);
        po[s] = *reinterpret_cast<const float4 *>(p.part_o + prow * kHeadDim + d0);
      }
    }
#pragma unroll
    for (int s = 0; s < kCombineRegs; ++s)
      if (s < p.nsplit) m = fmaxf(m, ml[s].x);
    const float msub = (m == -INFINITY) ? 0.f : m;
#pragma unroll
    for (int s = 0; s < kCombineRegs; ++s) {
      if (s < p.nsplit) {
        const float wgt = __builtin_amdgcn_exp2f(ml[s].x - msub);
        l += wgt * ml[s].y;
        acc.x += wgt * po[s].x;
        acc.y += wgt * po[s].y;
        acc.z += wgt * po[s].z;
        acc.w += wgt * po[s].w;
      }
    }
  } else {
    for (int s = 0; s < p.nsplit; ++s) m = fmaxf(m, p.part_ml[2 * (prow0 + (int64_t)s * kBlock)]);
    const float msub = (m == -INFINITY) ? 0.f : m;
    for (int s = 0; s < p.nsplit; ++s) {
      const int64_t prow = prow0 + (int64_t)s * kBlock;
      const float2 ml = *reinterpret_cast<const float2 *>(p.part_ml + 2 * prow);
      const float4 po = *reinterpret_cast<const float4 *>(p.part_o + prow * kHeadDim + d0);
      const float wgt = __builtin_amdgcn_exp2f(ml.x - msub);
      l += wgt * ml.y;
      acc.x += wgt * po.x;
      acc.y += wgt * po.y;
      acc.z += wgt * po.z;
      acc.w += wgt * po.w;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t *op = p.out + (int64_t)b * T * rs + (int64_t)tq * rs + h * kHeadDim + d0;
  uint2 val;
  val.x = pack_bf16x2(acc.x * inv, acc.y * inv);
  val.y = pack_bf16x2(acc.z * inv, acc.w * inv);
  *reinterpret_cast<uint2 *>(op) = val;
  if (p.lse != nullptr && d0 == 0) p.lse[((int64_t)b * p.H + h) * T + tq] = (m + __log2f(l)) * kLn2;
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
  p.row_lo = 0;
  p.row_hi = a.T;
  p.nsplit = 1;
  p.tiles_per_split = a.nb;
  p.scale_log2 = a.scale_log2;
  p.sum_k = static_cast<const uint16_t *>(a.sum_k);
  p.sum_v = static_cast<const uint16_t *>(a.sum_v);
  p.sum_lm = a.sum_lm;
  p.qbar = a.qbar;
  p.kbar = a.kbar;
  p.budget = a.budget;
  p.radius = a.radius;
  p.list_out = a.list_out;
  p.cnt_out = a.cnt_out;
  return p;
}

}  // namespace

int dense_splits(int B, int H, int nb, int nvb) { return dense_pair_splits(B, H, nb, nvb); }

size_t dense_workspace_bytes(int B, int H, int nb, int nvb) {
  const int s = dense_splits(B, H, nb, nvb);
  if (s <= 1) return 0;
  const size_t rows = (size_t)B * H * (nb - nvb) * s * kBlock;
  return rows * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_attn_sparse(const AttnArgs &a, hipStream_t stream) {
  if (a.nvq <= 0) return hipSuccess;
  if (a.max_sel <= kMaxPairList) return launch_attn_pair_sparse(a, stream);
  Params p = make_params(a, 0, a.nvq);
  p.row_hi = a.rows_end;
  const int total = a.B * a.H * a.nvq;
  hipLaunchKernelGGL(attn_fwd_kernel<>, dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_sparse_spark(const AttnArgs &a, hipStream_t stream) {
  if (a.nvq <= 0) return hipSuccess;
  if (a.nvb > kMaxRouteBlocks || a.sum_k == nullptr || a.sum_v == nullptr || a.sum_lm == nullptr)
    return hipErrorInvalidValue;
  if (a.max_sel <= kMaxPairSparkList) return launch_attn_pair_spark(a, stream);
  Params p = make_params(a, 0, a.nvq);
  p.row_hi = a.rows_end;
  const int total = a.B * a.H * a.nvq;
  hipLaunchKernelGGL((attn_fwd_kernel<true>), dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_sparse_fused(const AttnArgs &a, hipStream_t stream) {
  if (a.nvq <= 0) return hipSuccess;
  if (a.nvb > kMaxRouteBlocks || a.max_sel > kMaxRouteBlocks || a.qbar == nullptr ||
      (a.nvb > 0 && a.kbar == nullptr))
    return hipErrorInvalidValue;
  if (a.max_sel <= kMaxPairList) return launch_attn_pair_fused(a, stream);
  Params p = make_params(a, 0, a.nvq);
  p.row_hi = a.rows_end;
  const int total = a.B * a.H * a.nvq;
  hipLaunchKernelGGL((attn_fwd_kernel<false, true>), dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_dense(const AttnArgs &a, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const int nq = a.nb - a.nvb;
  if (nq <= 0 || a.rows_end >= a.T) return hipSuccess;
  const int s = dense_splits(a.B, a.H, a.nb, a.nvb);
  if (s <= 1 || workspace == nullptr || workspace_bytes < dense_workspace_bytes(a.B, a.H, a.nb, a.nvb))
    return launch_attn_pair_dense(a, nullptr, nullptr, 1, stream);
  const size_t rows = (size_t)a.B * a.H * nq * s * kBlock;
  float *part_o = static_cast<float *>(workspace);
  float *part_ml = part_o + rows * kHeadDim;
  hipError_t e = launch_attn_pair_dense(a, part_o, part_ml, s, stream);
  if (e != hipSuccess) return e;
  Params p = make_params(a, a.nvb, nq);
  p.row_lo = a.rows_end;
  p.nsplit = s;
  p.part_o = part_o;
  p.part_ml = part_ml;
  hipLaunchKernelGGL(combine_kernel, dim3(a.B * a.H * nq * (kBlock / kCombineRows)),
                     dim3(kCombineThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
