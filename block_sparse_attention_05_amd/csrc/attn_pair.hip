// Block-sparse flash attention on gfx950 bf16 MFMA with paired query blocks:
// one workgroup serves two adjacent 64-row query blocks A = 2p and B = 2p+1
// of one (b, h) and loads each key tile once when both lists hold it.
//
// Page "Sol-Attn and Spark for MiniMax-H3", Spark inference integration:
// selected K/V tiles stream through a single FP32 online-softmax/output
// accumulator.  Page "Add key bias to chunked Sol-Attn producers", Summary /
// Contract: the natural-log key bias is converted to log2 units and consumed
// only by the exact branch (sink keys).
//
// Approximate branch (the Spark page's virtual summaries merged into the
// same accumulator, kSpark): each of the two blocks packs the video blocks
// its list skips, ascending, into virtual tiles of 64 keys whose K and V
// rows are the summaries ak, av of those blocks (gathered by block index)
// and whose logits carry the log-mass lm as a natural-log bias.  Virtual
// tiles run as private pairs (A's tile v with B's tile v) after the exact
// tiles: full pairs with the biased tiles, a partial tile or a tile without
// a partner with the general ones, masked at the block's virtual key count.
//
// Why pairs.  A 64-row query block does 2.1 MFLOP per 64-key tile against
// 32 KiB of K/V copied from L2 into LDS, 64 FLOP per byte: at the MFMA rate
// of a CU that is the whole global-to-LDS copy bandwidth of the CU.
// Adjacent query blocks of a video (two 2-row strips of the same frame)
// select mostly the same key blocks: at the H3 shape two adjacent lists
// share about 65% of their entries (all sink blocks and most routed ones),
// so serving both from one tile stream cuts the copied bytes by about a
// third, and it halves the number of workgroups and their fixed costs.
// The copies still cost a step a good share of its time: on the H3 shape a
// paired step copies 32 KiB per workgroup, about what a CU moves from L2 to
// LDS in the time of the step's MFMAs.
//
// Workgroup: four wavefronts; wave w serves rows 32*(w&1) .. +31 of block
// A (w < 2) or B (w >= 2), over all 32 keys of a half tile per step, so every
// wave owns whole rows and there is no key-half merge.  A step consumes one
// 32-key half tile for each block: the same half tile when both lists hold
// the key block ("shared" entry, 16 KiB of K and V copied), or one half tile
// of each block's own list ("paired" entry: a key block only A holds next to
// one only B holds, 32 KiB copied).  Every list entry is two steps (the two
// 32-key halves of its 64-key block).
//
// Schedule.  Waves 0 and 1 build the entry list in LDS before the first
// tile load: they compact both lists (entries outside [0, NB) are skipped)
// and split them into shared and private entries (binary search in the
// other list); wave 0 pairs the i-th private entry of A with the i-th of B,
// sorts the entries by their larger key block (so that the workgroups that
// share an XCD sweep a head's keys together) and splits them, stably, into
// three phases:
//   U  - both tiles complete and unbiased (every entry when key_bias is NULL
//        apart from the partial block);
//   Bi - both tiles complete, at least one a sink tile with key_bias (biased;
//        the bias of a non-sink tile reads as zero);
//   G  - general: the partial last block NB-1, and private entries left over
//        when the lists differ in length (one block has no tile there).
// U and Bi steps are straight-line code; G steps mask keys past T and skip
// the softmax of a block without a tile.  The dense path (dense_sink_fwd)
// takes the implicit list [t_begin, t_end) for both blocks (all shared), in
// the same three phases; with split key ranges, a block without a partner
// (odd block count) has both wave pairs serve its rows over the two halves
// of the range (paired entries) and merges their results at the end.
//
// Data movement.  K and V half tiles go from HBM/L2 straight to LDS with
// buffer_load ... lds in the one-block kernel's tile layout (a slot is the
// 64-key layout whose key halves hold A's and B's half tiles; a shared entry
// fills the first half only).  Keys past T fall outside the buffer range and
// read as zero.  Step j issues, at its start, K of step j+2 and V of step
// j+1 into the slots step j-1 finished reading (two slots each), and ends
// with the wait and the barrier that publish them.  Each
// wave copies its Q rows into the V ring in whole rows before the schedule
// is built and reads its MFMA operand fragments from there (each wave reads only
// its own rows).
//
// Math per step and wave (32 rows x 32 keys): S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16, online softmax in base 2, P rounded to bf16,
// O^T += V^T P^T with V^T from ds_read_b64_tr_b16.  A full-tile step issues
// its copies, then runs one straight block in a fixed order: each of the
// eight S(j+1) MFMAs is followed by the exponentials of two of the lane's
// logits of tile j, taken against the running max as it stands (no tile
// max), so that the wave's matrix and vector work overlap; a tile whose P
// would exceed 2^32 (rare) moves the running max and is taken again, and
// the eight PV MFMAs close the step.  Masked steps take the tile max first
// and move the running max when it grows by more than 8.  The same arithmetic as
// the one-block kernel, with the keys of a 64-key tile accumulated in two
// sequential steps instead of two waves.
#include <atomic>

#include "attn_common.h"
#include "device_util.h"
#include "kernels.h"
#include "select.h"

namespace sa {
namespace {

using namespace attn;

constexpr int kPKOff = 0;                       // K ring: 2 slots x 16 KiB (A half | B half)
constexpr int kPVOff = 32768;                   // V ring: 2 slots x 16 KiB
constexpr int kPBOff = 65536;                   // bias ring: 2 slots x 64 floats (A | B)
constexpr int kPSchOff = 65536 + 512;           // entries: kMaxPairEntries x (first key of A's tile, of B's)
constexpr int kMaxPairEntries = 2 * kMaxPairList;
constexpr int kPCntOff = kPSchOff + kMaxPairEntries * 8;   // schedule counts and flags
constexpr int kPCntInts = 12;
constexpr int kPLdsBytes = kPCntOff + 4 * kPCntInts;
// Schedule-build temporaries, inside the K ring (no tile is loaded yet):
// compacted lists, private entries of A and B, shared entries, each private
// or shared entry's merge rank (below), and the entries in merged order.
constexpr int kListBytes = 4 * kMaxPairList;
constexpr int kLAOff = 0;
constexpr int kLBOff = kLAOff + kListBytes;
constexpr int kPAOff = kLBOff + kListBytes;
constexpr int kPBlOff = kPAOff + kListBytes;
constexpr int kSHOff = kPBlOff + kListBytes;
constexpr int kPARkOff = kSHOff + kListBytes;
constexpr int kPBRkOff = kPARkOff + kListBytes;
constexpr int kSHRkOff = kPBRkOff + kListBytes;
constexpr int kMrgOff = kSHRkOff + kListBytes;          // kMaxPairEntries x int2
// Approximate branch: one byte per video block and query block (A | B),
// marking the list's blocks while the virtual keys are packed.
constexpr int kVFlagOff = kMrgOff + 8 * kMaxPairEntries;
static_assert(kVFlagOff + 2 * kMaxRouteBlocks <= kPVOff, "build temporaries must fit the K ring");
// Approximate branch: the packed virtual keys of A and B (the video blocks
// each list skips, ascending), 16-bit block indices after the counts.
constexpr int kPVrowOff = kPLdsBytes;
constexpr int kPSparkBytes = 2 * kMaxRouteBlocks * 2;
// Entry encodings of virtual tiles: virtual tile v of block A is the block
// kVBlkA + v in the merged list and the first key kVirtA + 64 v in the
// schedule (B: kVBlkB, kVirtB).  Both key bases lie past every T, so the
// "key >= T: no exact tile" tests skip them; the virtual key at packed
// position x of block A has key kVirtA + x.
constexpr int kVBlkA = 1 << 20, kVBlkB = 1 << 21;
constexpr int kVirtA = 1 << 29, kVirtB = (1 << 29) + (1 << 27);
constexpr int kVirtBit = 1 << 29;           // set in every virtual key, clear below kVirtA
constexpr int kVirtPosMask = (1 << 27) - 1; // packed position of a virtual key
static_assert(2 * kMaxPairSparkList + kMaxRouteBlocks / kBlock <= kMaxPairEntries,
              "two disjoint lists and the virtual pairs must fit the schedule");

// Fused route: the two query blocks' pooled means (fp64), their scores and
// their selected lists, inside the V ring (unused until the first tile
// loads).
constexpr int kFqOff = kPVOff;                                  // 2 x 128 fp64
constexpr int kFsOff = kFqOff + 2 * kHeadDim * 8;               // 2 x kMaxRouteBlocks fp32
constexpr int kFlOff = kFsOff + 2 * kMaxRouteBlocks * 4;        // 2 x kMaxPairList int32
static_assert(kFlOff + 2 * kMaxPairList * 4 <= kPVOff + 32768, "fused route scratch must fit the V ring");

struct PairParams {
  const uint16_t *q, *k, *v;
  uint16_t *out;
  float *lse;
  const float *key_bias;
  const int32_t *block_idx, *block_cnt;
  float *part_o;      // split-KV partial outputs (dense path), nullable
  float *part_ml;     // split-KV partial (max, sum) per row
  int B, T, H, nb, nvb, max_sel;
  int qb0, nqb, npair;
  int row_lo, row_hi;  // rows written: [row_lo, row_hi)
  int nsplit, tiles_per_split;
  // Workgroups resident on one XCD at a time (two per CU), for the order of
  // the sparse items below; 0 keeps the plain order.
  int slots;
  float scale_log2;
  // fused route: pooled means in the route workspace layout, budget, forced
  // radius, optional copies of the selected lists
  const double *qbar;
  const float *kbar;
  int budget, radius;
  int32_t *list_out, *cnt_out;
  // approximate branch: summaries of (b, h) at sum_k/sum_v + bh*nb*128 and
  // sum_lm + bh*nb
  const uint16_t *sum_k, *sum_v;
  const float *sum_lm;
};

// Lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Whether x is among the n ascending values arr[0..n) (LDS); *pos gets the
// number of values below x.
__device__ __forceinline__ bool lds_contains(const int *arr, int n, int x, int *pos) {
  const int len = n;
  int lo = 0;
  while (n > 0) {
    const int half = n >> 1;
    if (arr[lo + half] < x) {
      lo += half + 1;
      n -= half + 1;
    } else {
      n = half;
    }
  }
  *pos = lo;
  return lo < len && arr[lo] == x;
}

// Item (pair of query blocks, head-major) of workgroup blk among total.
// Every XCD owns a contiguous, head-aligned range of items (the XCD remap).
// Its `slots` resident workgroups run consecutive items side by side and
// sweep one head's keys together, which fits the head's K and V in that
// XCD's L2 once; a head with more pairs than a multiple of `slots` would
// spill its last pairs into the next head's round and sweep its keys a
// second time.  So within the range every head's first multiple of `slots`
// pairs come first, head after head, and the spilled pairs of all heads
// follow.  Ranges that do not start and end on a head keep the plain order.
__device__ __forceinline__ int pair_order(int blk, int total, int npair, int slots) {
  const int w = xcd_remap(blk, total);
  if (slots <= 0 || npair <= slots) return w;
  constexpr int kXcd = 8;
  const int x = blk % kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  const int lo = x * per + (x < rem ? x : rem), n = per + (x < rem ? 1 : 0);
  const int full = npair - npair % slots;      // pairs per head in whole rounds
  const int left = npair - full;
  if (left == 0 || lo % npair != 0 || n % npair != 0) return w;
  const int k = w - lo, nh = n / npair;
  if (k < nh * full) return lo + (k / full) * npair + k % full;
  const int k2 = k - nh * full;
  return lo + (k2 / left) * npair + full + k2 % left;
}

// Entry list of one workgroup, in three passes separated by workgroup
// barriers (the caller's): compact (waves 0 and 1, one list each), classify
// (waves 0 and 1) and emit (wave 0).  Scalars: cnt[0..2] = nU, nBi, nE;
// cnt[3..7] = valid entries of A and B, private entries of A and B, shared
// entries; cnt[8] = 1 when a list is not strictly ascending.

// Pass 1: the valid entries of one list (lst, global or LDS), in order, to
// dst.  `first` holds entry `lane` of the list (read before anything else),
// c its length.
__device__ __forceinline__ void pair_compact(const PairParams &p, const int32_t *lst, int c, int first,
                                             int *dst, int *n_out, int lane) {
  c = c < 0 ? 0 : (c > p.max_sel ? p.max_sel : c);
  int n = 0;
  for (int cb = 0; cb < c; cb += 64) {
    const int e = cb == 0 ? (lane < c ? first : -1) : (cb + lane < c ? lst[cb + lane] : -1);
    const bool ok = e >= 0 && e < p.nb;
    const uint64_t m = __ballot(ok);
    if (ok) dst[n + lanes_below(m)] = e;
    n += __popcll(m);
  }
  if (lane == 0) *n_out = n;
}

// Pass 2: entries of `own` also in `other` go to sh (when given), the rest
// to priv.  Each entry's rank in the merged order goes beside it:
//
// The schedule walks the entries in ascending order of their larger key
// block (a shared entry x counts as (x, x)), so that the workgroups that run
// together on an XCD sweep the key range of a head together and a K/V tile
// is still in L2 when the next workgroup asks for it.  Private entries are
// paired in list order (i-th of A with i-th of B), so with both lists
// ascending the merged rank is the larger of the two list positions for a
// pair and the smaller of the two for a shared entry: a private pair i
// comes after the shared entries below its larger block (its list position
// in that list minus i) and after the i pairs before it, and a shared entry
// at position j of the shared list comes after the pairs whose both blocks
// lie below it (the smaller of its two list positions minus j).  privrk gets
// the own-list position of each private entry, shrk the merged rank of each
// shared entry.  A list that is not strictly ascending (outside the
// contract) sets *unsorted, and the entries then keep the unmerged order.
__device__ __forceinline__ void pair_classify(const int *own, int n_own, const int *other, int n_other,
                                              int *priv, int *privrk, int *n_priv_out, int *sh,
                                              int *shrk, int *n_sh_out, int *unsorted, int lane) {
  int np = 0, ns = 0;
  for (int cb = 0; cb < n_own; cb += 64) {
    const int i = cb + lane;
    const bool in = i < n_own;
    const int x = in ? own[i] : -1;
    // the merge ranks need strictly ascending lists; others keep list order
    if (__any(i + 1 < n_own && own[i + 1] <= x) && lane == 0) *unsorted = 1;
    int pos = 0;
    const bool shared = in && lds_contains(other, n_other, x, &pos);
    const uint64_t mp = __ballot(in && !shared), ms = __ballot(shared);
    if (in && !shared) {
      priv[np + lanes_below(mp)] = x;
      privrk[np + lanes_below(mp)] = i;
    }
    if (shared && sh != nullptr) {
      sh[ns + lanes_below(ms)] = x;
      shrk[ns + lanes_below(ms)] = i < pos ? i : pos;
    }
    np += __popcll(mp);
    ns += __popcll(ms);
  }
  if (lane == 0) {
    *n_priv_out = np;
    if (sh != nullptr) *n_sh_out = ns;
  }
}

// Pass 3: the entries (private pairs, leftovers, shared entries) in merged
// order (pass 2), then sorted into the three phases, stable in that order.
// Leftover private entries (one list longer than the other) follow all
// others; they are general-phase entries anyway.
__device__ __forceinline__ void pair_emit(const PairParams &p, unsigned char *smem, int lane, bool spark) {
  const int *PA = reinterpret_cast<const int *>(smem + kPAOff);
  const int *PB = reinterpret_cast<const int *>(smem + kPBlOff);
  const int *SH = reinterpret_cast<const int *>(smem + kSHOff);
  const int *PArk = reinterpret_cast<const int *>(smem + kPARkOff);
  const int *PBrk = reinterpret_cast<const int *>(smem + kPBRkOff);
  const int *SHrk = reinterpret_cast<const int *>(smem + kSHRkOff);
  int2 *mrg = reinterpret_cast<int2 *>(smem + kMrgOff);
  int2 *sch = reinterpret_cast<int2 *>(smem + kPSchOff);
  int *cnt = reinterpret_cast<int *>(smem + kPCntOff);
  const int nPA = __builtin_amdgcn_readfirstlane(cnt[5]);
  const int nPB = __builtin_amdgcn_readfirstlane(cnt[6]);
  const int nS = __builtin_amdgcn_readfirstlane(cnt[7]);
  const int partial = (p.T % kBlock) != 0 ? p.nb - 1 : -1;
  const bool biased = p.key_bias != nullptr;
  const int nX = nPA > nPB ? nPA : nPB;
  const int nMin = nPA < nPB ? nPA : nPB;
  const int nC0 = nX + nS;
  // approximate branch: virtual tiles of A and B (cnt[9], cnt[10] virtual
  // keys), appended as private pairs after the exact entries
  const int nvA = spark ? __builtin_amdgcn_readfirstlane(cnt[9]) : 0;
  const int nvB = spark ? __builtin_amdgcn_readfirstlane(cnt[10]) : 0;
  const int tA = (nvA + kBlock - 1) / kBlock, tB = (nvB + kBlock - 1) / kBlock;
  const int nC = nC0 + (tA > tB ? tA : tB);
  const bool unsorted = __builtin_amdgcn_readfirstlane(cnt[8]) != 0;
  for (int cb = 0; cb < nC; cb += 64) {
    const int c = cb + lane;
    if (c >= nC0 && c < nC) {
      const int v = c - nC0;
      mrg[c] = make_int2(v < tA ? kVBlkA + v : -1, v < tB ? kVBlkB + v : -1);
    } else if (c < nC) {
      int a, b, r;
      if (c < nX) {
        a = c < nPA ? PA[c] : -1;
        b = c < nPB ? PB[c] : -1;
        r = c < nMin ? (PArk[c] > PBrk[c] ? PArk[c] : PBrk[c]) : nS + c;
      } else {
        a = b = SH[c - nX];
        r = SHrk[c - nX];
      }
      mrg[unsorted ? c : r] = make_int2(a, b);
    }
  }
  wave_lds_sync();   // the merged entries were written by other lanes of this wave
  auto entry = [&](int c, int &a, int &b) {
    const int2 v = mrg[c];
    a = v.x;
    b = v.y;
  };
  // entries are stored as the first key of each block's tile (T: no tile)
  auto first_key = [&](int x) -> int {
    if (x < 0) return p.T;
    if (x >= kVBlkB) return kVirtB + kBlock * (x - kVBlkB);
    if (x >= kVBlkA) return kVirtA + kBlock * (x - kVBlkA);
    return x * kBlock;
  };
  auto phase = [&](int a, int b) -> int {
    if (a >= kVBlkA || b >= kVBlkA) {   // virtual: biased by the log-mass
      const bool fa = a >= kVBlkA && kBlock * (a - kVBlkA + 1) <= nvA;
      const bool fb = b >= kVBlkB && kBlock * (b - kVBlkB + 1) <= nvB;
      return fa && fb ? 1 : 2;
    }
    if (a < 0 || b < 0 || a == partial || b == partial) return 2;
    if (biased && (a >= p.nvb || b >= p.nvb)) return 1;
    return 0;
  };
  if (nC <= 64) {   // one chunk: entries stay in registers between the passes
    int a = -1, b = -1;
    if (lane < nC) entry(lane, a, b);
    const int ph = lane < nC ? phase(a, b) : 3;
    const uint64_t m0 = __ballot(ph == 0), m1 = __ballot(ph == 1), m2 = __ballot(ph == 2);
    const int n0 = __popcll(m0), n1 = __popcll(m1);
    if (ph < 3) {
      const int pos = ph == 0 ? lanes_below(m0) : ph == 1 ? n0 + lanes_below(m1) : n0 + n1 + lanes_below(m2);
      sch[pos] = make_int2(first_key(a), first_key(b));
    }
    if (lane == 0) {
      cnt[0] = n0;
      cnt[1] = n1;
      cnt[2] = nC;
    }
    return;
  }
  int n0 = 0, n1 = 0;
  for (int cb = 0; cb < nC; cb += 64) {
    const int c = cb + lane;
    int a = -1, b = -1;
    if (c < nC) entry(c, a, b);
    const int ph = c < nC ? phase(a, b) : 3;
    n0 += __popcll(__ballot(ph == 0));
    n1 += __popcll(__ballot(ph == 1));
  }
  int r0 = 0, r1 = n0, r2 = n0 + n1;
  for (int cb = 0; cb < nC; cb += 64) {
    const int c = cb + lane;
    int a = -1, b = -1;
    if (c < nC) entry(c, a, b);
    const int ph = c < nC ? phase(a, b) : 3;
    const uint64_t m0 = __ballot(ph == 0), m1 = __ballot(ph == 1), m2 = __ballot(ph == 2);
    if (ph < 3) {
      const int pos = ph == 0 ? r0 + lanes_below(m0) : ph == 1 ? r1 + lanes_below(m1) : r2 + lanes_below(m2);
      sch[pos] = make_int2(first_key(a), first_key(b));
    }
    r0 += __popcll(m0);
    r1 += __popcll(m1);
    r2 += __popcll(m2);
  }
  if (lane == 0) {
    cnt[0] = n0;
    cnt[1] = n1;
    cnt[2] = nC;
  }
}

template <bool kDense, bool kFused, bool kSpark = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_pair_kernel(PairParams p) {
  __shared__ __align__(16) unsigned char smem[kPLdsBytes + (kSpark ? kPSparkBytes : 0)];

  const int total = p.B * p.H * p.npair * p.nsplit;
  const int w = kDense ? xcd_remap(blockIdx.x, total) : pair_order(blockIdx.x, total, p.npair, p.slots);
  const int split = w % p.nsplit;
  const int wp = w / p.nsplit;
  const int pi = wp % p.npair;
  const int bh = wp / p.npair;
  const int h = bh % p.H;
  const int b = bh / p.H;
  const int qbiA = 2 * pi;
  const bool hasB = qbiA + 1 < p.nqb;
  // Dense rows split over key ranges, a block without a partner (odd block
  // count): both wave pairs serve its rows, over the two halves of the
  // split's key range, and merge at the end, instead of waves 2-3 idling.
  // (Unsplit, the dense rows keep the sparse path's tile order, and with it
  // its bits at ratio 1.)
  const bool self_wg = kDense && !hasB && p.nsplit > 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR
  const int blk = wave >> 1;   // 0: block A, 1: block B
  const int rw = wave & 1;     // rows 32*rw .. +31 of the block
  const int g = lane >> 5;
  const int c32 = lane & 31;
  const int T = p.T;
  const int64_t rs = (int64_t)p.H * kHeadDim;   // elements per token
  const int row_bytes = p.H * kHeadDim * 2;
  const int64_t bbase = (int64_t)b * T * rs;
  const int qbi = self_wg ? qbiA : qbiA + blk;
  const int qb = p.qb0 + qbi;
  const bool active = blk == 0 || hasB || self_wg;   // a missing block B computes nothing it keeps
  const int tq = qb * kBlock + rw * 32 + c32;    // this lane's query row

  // The lists go first: wave 0 reads A's count and first 64 entries, wave 1
  // B's, all in flight together ahead of the Q rows.  The count is a scalar
  // load; the entries are copied into the bias ring (unused until the first
  // tiles) by a global-to-LDS copy issued before the wave's eight Q copies,
  // so that the wait for them (vmcnt(8): loads complete in order) does not
  // also wait for Q, which then arrives while the schedule is built.
  const int64_t liA = (int64_t)bh * p.nqb + qbiA;
  const bool list_wave = !kDense && !kFused && wave < 2 && (wave == 0 || hasB);
  int lcnt = 0, lfirst = -1;
  if (list_wave) {
    const int64_t li = liA + wave;
    lcnt = p.block_cnt[li];
    // entries past max_sel read as zero; only the first lcnt are used
    const i32x4s rl = buffer_rsrc(p.block_idx + li * p.max_sel, (uint32_t)p.max_sel * 4u);
    lds_dma_b32(rl, (uint32_t)lane * 4u, (uint32_t)reinterpret_cast<uintptr_t>(LDS_PTR(unsigned char, smem)) +
                                             kPBOff + 256u * (uint32_t)wave);
  }

  // Q^T fragments of this lane's row (d = 16*dc + 8*g + [0, 8)).  Without
  // the fused route the wave's 32 rows are copied into its 8 KiB of the V
  // ring (free until the first tiles load) in whole 256-byte rows, four
  // rows per instruction (lane l: row 4i + l/16, 16-byte chunk
  // (l%16) ^ (row%16), so chunk c of row r lands at slot c ^ (r%16) and the
  // fragment reads below are free of bank conflicts), and read after the
  // schedule is built.  A lane that loads its own row instead would touch
  // 32 rows per instruction, four times the cache-line requests.  The fused
  // route keeps its scratch in the V ring and reads straight from memory.
  // Rows past T and a missing block B read as zero.
  const uint32_t slab = (uint32_t)T * (uint32_t)row_bytes;
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(LDS_PTR(unsigned char, smem));
  bf16x8 qf[8];
  if (kFused) {
    const bool ok = active && tq < T;
    const uint16_t *qrow = p.q + bbase + (int64_t)(ok ? tq : 0) * rs + h * kHeadDim + 8 * g;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      bf16x8 v = {};
      if (ok) v = *reinterpret_cast<const bf16x8 *>(qrow + 16 * dc);
      qf[dc] = v;
    }
  } else {
    const i32x4s rq = buffer_rsrc(p.q + bbase, slab);
    const uint32_t r4 = (uint32_t)(lane >> 4);
    const uint32_t row0 = (uint32_t)(qb * kBlock + rw * 32);
    const uint32_t l = lds0 + kPVOff + 8192u * (uint32_t)wave;
    auto q_off = [&](uint32_t i) -> uint32_t {
      const uint32_t r = 4 * i + r4;
      const uint32_t ch = (uint32_t)(lane & 15) ^ (r & 15);
      return active ? (row0 + r) * (uint32_t)row_bytes + (uint32_t)h * 256u + 16u * ch : slab;
    };
    lds_dma_b128<0>(rq, q_off(0), l);
    lds_dma_b128<1024>(rq, q_off(1), l);
    lds_dma_b128<2048>(rq, q_off(2), l);
    lds_dma_b128<3072>(rq, q_off(3), l);
    lds_dma_b128<4096>(rq, q_off(4), l);
    lds_dma_b128<5120>(rq, q_off(5), l);
    lds_dma_b128<6144>(rq, q_off(6), l);
    lds_dma_b128<7168>(rq, q_off(7), l);
  }
  // the wave's Q fragments from its copy (each wave reads what it copied)
  auto read_q = [&]() {
    if (kFused) return;
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    const unsigned char *qs = smem + kPVOff + 8192 * wave + 256 * c32;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc)
      qf[dc] = *reinterpret_cast<const bf16x8 *>(qs + 16 * ((2 * dc + g) ^ (c32 & 15)));
  };

  // ---- schedule ------------------------------------------------------------
  const bool has_bias = p.key_bias != nullptr;
  const int nbfull = (T % kBlock) != 0 ? p.nb - 1 : p.nb;   // blocks of 64 keys
  int nU, nBi, nE;
  int d_t0 = 0, d_nub = 0, d_lenA = 0, d_lenB = 0;
  const int2 *sch = reinterpret_cast<const int2 *>(smem + kPSchOff);
  if (kDense) {
    const int t_begin = split * p.tiles_per_split;
    int t_end = t_begin + p.tiles_per_split;
    t_end = t_end < p.nb ? t_end : p.nb;
    d_t0 = t_begin;
    if (self_wg) {
      // entry e: key block t_begin + e for waves 0-1 (e < lenA) and t_begin
      // + lenA + e for waves 2-3 (e < lenB); the partial last block and a
      // missing second tile are general entries, and with the blocks in
      // ascending order they come last
      const int n = t_end > t_begin ? t_end - t_begin : 0;
      d_lenA = (n + 1) / 2;
      d_lenB = n - d_lenA;
      const bool part = nbfull < p.nb && p.nb - 1 >= t_begin && p.nb - 1 < t_end;
      // general entries: lenB-1 when the second tile is the partial block,
      // lenA-1 (= lenB) when there is no second tile; a one-block range that
      // is the partial block is only the latter
      const int ng = (part && d_lenB > 0 ? 1 : 0) + (d_lenA > d_lenB ? 1 : 0);
      const int nfull = d_lenA - ng;   // entries with two complete tiles
      int nu = nfull;
      if (has_bias) {   // biased once the second tile is a sink block
        nu = p.nvb - t_begin - d_lenA;
        nu = nu < 0 ? 0 : (nu > nfull ? nfull : nu);
      }
      nU = nu;
      nBi = nfull - nu;
      nE = d_lenA;
    } else {
      const int ub_end = t_end < nbfull ? t_end : nbfull;
      const int nub = ub_end > t_begin ? ub_end - t_begin : 0;
      int nu = nub;
      if (has_bias) {
        nu = p.nvb - t_begin;
        nu = nu < 0 ? 0 : (nu > nub ? nub : nu);
      }
      nU = nu;
      nBi = nub - nu;
      nE = nub + ((nbfull < p.nb && p.nb - 1 >= t_begin && p.nb - 1 < t_end) ? 1 : 0);
      d_nub = nub;
    }
    read_q();
    __syncthreads();
  } else {
    int *cnt = reinterpret_cast<int *>(smem + kPCntOff);
    int *LA = reinterpret_cast<int *>(smem + kLAOff);
    int *LB = reinterpret_cast<int *>(smem + kLBOff);
    const int32_t *lst = p.block_idx + (liA + wave) * p.max_sel;
    if (kFused) {
      // Route of both query blocks inside the workgroup, with the rule of
      // the route kernel: s_j = fp32 of the fp64 dot product of the fp32
      // means (fp32 products are exact in fp64), then waves 0 and 1 select
      // and emit A's and B's lists into LDS.
      double *qs = reinterpret_cast<double *>(smem + kFqOff);
      float *sc = reinterpret_cast<float *>(smem + kFsOff);
      int32_t *fl = reinterpret_cast<int32_t *>(smem + kFlOff);
      const int ntq = (p.nqb + 15) >> 4, ntk = (p.nvb + 15) >> 4;
      if (tid < kHeadDim) {   // block A (threads 0-63) or B (64-127), channels 2t, 2t+1
        const int t = tid & 63;
        const int qq = p.qb0 + qbiA + (tid >> 6);
        double2 w2 = make_double2(0.0, 0.0);
        if (tid < 64 || hasB)
          w2 = reinterpret_cast<const double2 *>(p.qbar)
              [(((int64_t)bh * ntq + (qq >> 4)) * 16 + (t & 15)) * 64 + 16 * (t >> 4) + (qq & 15)];
        qs[(tid >> 6) * kHeadDim + 2 * t] = w2.x;
        qs[(tid >> 6) * kHeadDim + 2 * t + 1] = w2.y;
      }
      __syncthreads();
      const float4 *kt = reinterpret_cast<const float4 *>(p.kbar) + (int64_t)bh * ntk * 8 * 64;
      for (int jb = tid; jb < p.nvb; jb += kThreads) {
        const float4 *kj = kt + (int64_t)(jb >> 4) * 8 * 64 + (jb & 15);
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0, b0 = 0.0, b1 = 0.0, b2 = 0.0, b3 = 0.0;
#pragma unroll 4
        for (int u = 0; u < kHeadDim / 4; ++u) {  // channels 4u .. 4u+3
          const float4 kv = kj[(u & 7) * 64 + 16 * (u >> 3)];
          a0 = __builtin_fma(qs[4 * u + 0], (double)kv.x, a0);
          a1 = __builtin_fma(qs[4 * u + 1], (double)kv.y, a1);
          a2 = __builtin_fma(qs[4 * u + 2], (double)kv.z, a2);
          a3 = __builtin_fma(qs[4 * u + 3], (double)kv.w, a3);
          b0 = __builtin_fma(qs[kHeadDim + 4 * u + 0], (double)kv.x, b0);
          b1 = __builtin_fma(qs[kHeadDim + 4 * u + 1], (double)kv.y, b1);
          b2 = __builtin_fma(qs[kHeadDim + 4 * u + 2], (double)kv.z, b2);
          b3 = __builtin_fma(qs[kHeadDim + 4 * u + 3], (double)kv.w, b3);
        }
        sc[jb] = (float)((a0 + a1) + (a2 + a3));
        sc[kMaxRouteBlocks + jb] = (float)((b0 + b1) + (b2 + b3));
      }
      __syncthreads();
      if (wave < 2 && (wave == 0 || hasB)) {
        const int qq = p.qb0 + qbiA + wave;
        int32_t *out = fl + wave * kMaxPairList;
        const float *srow = sc + wave * kMaxRouteBlocks;
        // slots per lane sized to nvb (the selection loops over all of them)
        auto sel = [&](auto e_c) {
          return select_and_emit<decltype(e_c)::value>(srow, qq, p.nvb, p.nb, p.budget, p.radius, p.max_sel,
                                                      out, nullptr, lane);
        };
        const int c = p.nvb <= 128 ? sel(Int<2>{}) : p.nvb <= 192 ? sel(Int<3>{})
                    : p.nvb <= 256 ? sel(Int<4>{}) : sel(Int<kMaxRouteBlocks / 64>{});
        if (p.list_out != nullptr) {
          const int64_t li = liA + wave;
          for (int x = lane; x < p.max_sel; x += 64) p.list_out[li * p.max_sel + x] = out[x];
          if (lane == 0) p.cnt_out[li] = c;
        }
        wave_lds_sync();
        lcnt = c;
        lfirst = lane < p.max_sel ? out[lane] : -1;
        lst = out;
      }
    }
    if (list_wave) {
      // the list copy, not the Q copies issued after it
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      lfirst = *reinterpret_cast<const int *>(smem + kPBOff + 256 * wave + 4 * lane);
    }
    if (wave == 0 || (wave == 1 && hasB))
      pair_compact(p, lst, __builtin_amdgcn_readfirstlane(lcnt), lfirst, wave ? LB : LA, cnt + 3 + wave,
                   lane);
    if (wave == 2 && lane == 0) cnt[8] = 0;
    __syncthreads();
    if (wave < 2) {
      const int nA = __builtin_amdgcn_readfirstlane(cnt[3]);
      if (!hasB) {   // a missing block B: every entry of A is shared
        if (wave == 0) pair_classify(LA, nA, LA, 0, reinterpret_cast<int *>(smem + kSHOff),
                                     reinterpret_cast<int *>(smem + kSHRkOff), cnt + 7, nullptr,
                                     nullptr, nullptr, cnt + 8, lane);
        if (wave == 0 && lane == 0) cnt[5] = cnt[6] = 0;
      } else {
        const int nB = __builtin_amdgcn_readfirstlane(cnt[4]);
        if (wave == 0)
          pair_classify(LA, nA, LB, nB, reinterpret_cast<int *>(smem + kPAOff),
                        reinterpret_cast<int *>(smem + kPARkOff), cnt + 5,
                        reinterpret_cast<int *>(smem + kSHOff), reinterpret_cast<int *>(smem + kSHRkOff),
                        cnt + 7, cnt + 8, lane);
        else
          pair_classify(LB, nB, LA, nA, reinterpret_cast<int *>(smem + kPBlOff),
                        reinterpret_cast<int *>(smem + kPBRkOff), cnt + 6, nullptr, nullptr, nullptr,
                        cnt + 8, lane);
      }
    }
    if (kSpark && wave < 2) {
      // Approximate branch: the video blocks this wave's list skips, packed
      // ascending (a missing block B has none): a byte flag per video block
      // marks the list's entries, then a ballot per 64-block chunk packs the
      // unflagged ones.
      unsigned char *fl = smem + kVFlagOff + wave * kMaxRouteBlocks;
      uint16_t *vr = reinterpret_cast<uint16_t *>(smem + kPVrowOff) + wave * kMaxRouteBlocks;
      const int *L = reinterpret_cast<const int *>(smem + (wave ? kLBOff : kLAOff));
      const int nL = (wave == 0 || hasB) ? __builtin_amdgcn_readfirstlane(cnt[3 + wave]) : 0;
      for (int x = lane; 4 * x < p.nvb; x += 64) reinterpret_cast<uint32_t *>(fl)[x] = 0u;
      wave_lds_sync();
      for (int cb = 0; cb < nL; cb += 64) {
        const int e = cb + lane < nL ? L[cb + lane] : -1;
        if (e >= 0 && e < p.nvb) fl[e] = 1;
      }
      wave_lds_sync();
      int nv = 0;
      if (wave == 0 || hasB) {
        for (int cb = 0; cb < p.nvb; cb += 64) {
          const int x = cb + lane;
          const bool skip = x < p.nvb && fl[x] == 0;
          const uint64_t m = __ballot(skip);
          if (skip) vr[nv + lanes_below(m)] = (uint16_t)x;
          nv += __popcll(m);
        }
      }
      if (lane == 0) cnt[9 + wave] = nv;
    }
    __syncthreads();
    if (wave == 0) pair_emit(p, smem, lane, kSpark);
    read_q();
    // all waves have their Q before the first tile copies refill the V ring
    __syncthreads();
    nU = __builtin_amdgcn_readfirstlane(cnt[0]);
    nBi = __builtin_amdgcn_readfirstlane(cnt[1]);
    nE = __builtin_amdgcn_readfirstlane(cnt[2]);
  }
  // Entries in lanes (lane j = entry ch_cb + j of the current 64-entry
  // chunk), read with v_readlane; entry() is called with e = 0, 1, 2, ...
  int ch_cb = 0, ch_a = -1, ch_b = -1;
  if (!kDense && lane < nE) {
    const int2 v = sch[lane];
    ch_a = v.x;
    ch_b = v.y;
  }
  auto entry = [&](int e, int &a, int &bb) {
    if (kDense) {
      if (self_wg) {
        a = (d_t0 + e) * kBlock;
        bb = e < d_lenB ? (d_t0 + d_lenA + e) * kBlock : T;
      } else {
        a = bb = (e < d_nub ? d_t0 + e : p.nb - 1) * kBlock;
      }
      return;
    }
    if (e - ch_cb >= 64) {
      ch_cb += 64;
      const int x = ch_cb + lane;
      int2 v = make_int2(-1, -1);
      if (x < nE) v = sch[x];
      ch_a = v.x;
      ch_b = v.y;
    }
    a = __builtin_amdgcn_readlane(ch_a, e - ch_cb);
    bb = __builtin_amdgcn_readlane(ch_b, e - ch_cb);
  };
  // First key of half tile `half` of the tile whose first key is k0.  A key
  // at or past T means no tile: a missing block (k0 = T) or a half that lies
  // past T; every user below tests ">= T".
  auto hkey = [&](int k0, int half) -> int { return half == 0 ? k0 : k0 + 32; };

  // ---- loads --------------------------------------------------------------
  // entries from this index on carry key_bias on their sink tiles
  const int bias_from = (has_bias || kSpark) ? nU : 0x7fffffff;
  const i32x4s rk = buffer_rsrc(p.k + bbase, slab);
  const i32x4s rv = buffer_rsrc(p.v + bbase, slab);
  const float *kbias = has_bias ? p.key_bias + (int64_t)b * T : nullptr;
  const i32x4s rb = buffer_rsrc(kbias ? (const void *)kbias : (const void *)p.k, kbias ? T * 4u : 0u);
  const int sink0 = p.nvb * kBlock;
  // approximate branch: summary rows are 256 B apart in one (b, h) slab of
  // nb rows; log-masses 4 B apart
  const int64_t sbase = (int64_t)bh * p.nb;
  const i32x4s rsk = buffer_rsrc(kSpark ? p.sum_k + sbase * kHeadDim : p.k, kSpark ? (uint32_t)p.nb * 256u : 0u);
  const i32x4s rsv = buffer_rsrc(kSpark ? p.sum_v + sbase * kHeadDim : p.v, kSpark ? (uint32_t)p.nb * 256u : 0u);
  const i32x4s rlm = buffer_rsrc(kSpark ? (const void *)(p.sum_lm + sbase) : (const void *)p.k,
                                 kSpark ? (uint32_t)p.nb * 4u : 0u);
  const int *cntp = reinterpret_cast<const int *>(smem + kPCntOff);
  const int nvA = kSpark && !kDense ? __builtin_amdgcn_readfirstlane(cntp[9]) : 0;
  const int nvB = kSpark && !kDense ? __builtin_amdgcn_readfirstlane(cntp[10]) : 0;
  const uint16_t *vrow = reinterpret_cast<const uint16_t *>(smem + kPVrowOff);
  // LDS tile layout: the one-block kernel's.  A 64-key slot is 16 blocks of
  // 1 KiB; block 2*kg + hf holds keys 8*kg .. +7 (kg = 0..7) and bytes
  // 128*hf .. +127 of each key row, in 16-byte pieces (key k' = key%8, chunk
  // c = 0..7) placed with an XOR swizzle:
  //   K: piece (k', c) at 128*k' + 16*(c ^ k' ^ (kg & 1));
  //   V: piece (k', c) at 128*k' + 16*(c ^ 2*(k' & 3)).
  // Key groups 0-3 hold A's half tile (or the shared one), 4-7 B's.  Wave w
  // fetches key group w of A's half tile and, in a paired step, key group w
  // of B's (keys 8w .. 8w+7 of each), so every wave issues the same copies
  // whatever the step holds; the second 128 bytes of each key row come from
  // the same lane offset through the instruction's immediate offset.
  const uint32_t chk = (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t row_lane = (uint32_t)(lane >> 3) * (uint32_t)row_bytes + (uint32_t)h * 256u +
                            (uint32_t)(8 * wave) * (uint32_t)row_bytes;
  const uint32_t k_lane = row_lane + 16u * (chk ^ (uint32_t)(wave & 1));
  const uint32_t v_lane = row_lane + 16u * (uint32_t)((lane & 7) ^ (2 * ((lane >> 3) & 3)));
  const uint32_t lds_w = lds0 + 2048u * (uint32_t)wave;
  // (B's tile is copied when it is its own: kB != kA)
  // Approximate branch: a virtual half tile gathers the summary rows of its
  // 32 virtual keys (packed positions key - kVirtX .. +31, past the count:
  // row 0, masked), key group w by wave w, in the exact tiles' LDS layout.
  const uint32_t sw_k = 16u * (chk ^ (uint32_t)(wave & 1));
  const uint32_t sw_v = 16u * (uint32_t)((lane & 7) ^ (2 * ((lane >> 3) & 3)));
  const int vrow_lane = 8 * wave + (lane >> 3);
  auto vrow_of = [&](int isB, int key) -> uint32_t {
    const int pos = (key & kVirtPosMask) + vrow_lane;
    const int nv = isB ? nvB : nvA;
    return (uint32_t)vrow[isB * kMaxRouteBlocks + (pos < nv ? pos : 0)];
  };
  auto issue_k = [&](int kA, int kB, int slot) {
    const uint32_t l = lds_w + kPKOff + (uint32_t)(slot * 16384);
    if (kSpark && ((kA | kB) & kVirtBit) != 0) {
      if (kA & kVirtBit) lds_dma_b128_x2<0>(rsk, 0u, vrow_of(0, kA) * 256u + sw_k, l);
      if (kB & kVirtBit) lds_dma_b128_x2<8192>(rsk, 0u, vrow_of(1, kB) * 256u + sw_k, l);
      return;
    }
    const int kb = kB == kA ? T : kB;
    if (kA < T) lds_dma_b128_x2<0>(rk, (uint32_t)kA * (uint32_t)row_bytes, k_lane, l);
    if (kb < T) lds_dma_b128_x2<8192>(rk, (uint32_t)kb * (uint32_t)row_bytes, k_lane, l);
  };
  // e_tile: the entry index of the tile; its bias is loaded when e_tile >=
  // bias_from (the biased and general phases with key_bias)
  auto issue_v = [&](int kA, int kB, int slot, int e_tile) {
    const uint32_t l = lds_w + kPVOff + (uint32_t)(slot * 16384);
    if (kSpark && ((kA | kB) & kVirtBit) != 0) {
      if (kA & kVirtBit) lds_dma_b128_x2<0>(rsv, 0u, vrow_of(0, kA) * 256u + sw_v, l);
      if (kB & kVirtBit) lds_dma_b128_x2<8192>(rsv, 0u, vrow_of(1, kB) * 256u + sw_v, l);
      // log-masses of both half tiles (lanes 0-31: A's keys, 32-63: B's);
      // past a block's count or for a missing block they read as zero (the
      // masked step sets those logits to -inf)
      if (wave == 0) {
        const int isB = lane >> 5;
        const int k0 = isB ? kB : kA;
        const int pos = (k0 & kVirtPosMask) + (lane & 31);
        const bool ok = (k0 & kVirtBit) != 0 && pos < (isB ? nvB : nvA);
        const uint32_t idx = vrow[isB * kMaxRouteBlocks + (ok ? pos : 0)];
        lds_dma_b32(rlm, ok ? idx * 4u : (uint32_t)p.nb * 4u, lds0 + kPBOff + (uint32_t)(slot * 256));
      }
      return;
    }
    const int kb = kB == kA ? T : kB;
    if (kA < T) lds_dma_b128_x2<0>(rv, (uint32_t)kA * (uint32_t)row_bytes, v_lane, l);
    if (kb < T) lds_dma_b128_x2<8192>(rv, (uint32_t)kb * (uint32_t)row_bytes, v_lane, l);
    // natural-log bias of both half tiles (lanes 0-31: A's keys, 32-63:
    // B's); keys of non-sink blocks and past T read as zero
    if (e_tile >= bias_from && wave == 0) {
      const int k0 = lane < 32 ? kA : kB;
      const int key = k0 + (lane & 31);
      const bool sink = k0 >= sink0 && key < T;
      lds_dma_b32(rb, sink ? (uint32_t)key * 4u : (uint32_t)T * 4u, lds0 + kPBOff + (uint32_t)(slot * 256));
    }
  };
  // operand read bases (bytes within a slot half); the other operand bases
  // differ by an XOR of the swizzled chunk bits: K chunk 2*(dc%4) + g lands
  // at k_rd0 ^ (32*(dc%4)); V for odd dt at v_rd0 ^ 64.
  uint32_t k_rd0, v_rd0;
  {
    const uint32_t kp = (uint32_t)(c32 & 7);
    k_rd0 = (uint32_t)(2048 * (c32 >> 3)) + 128 * kp + 16 * ((uint32_t)g ^ kp ^ (uint32_t)((c32 >> 3) & 1));
    const uint32_t r = (uint32_t)((lane & 15) >> 2), dh = (uint32_t)((lane >> 4) & 1), j = (uint32_t)(lane & 3);
    v_rd0 = (uint32_t)(512 * g) + 128 * r + 8 * (j & 1) + 16 * ((2 * dh + (j >> 1)) ^ (2 * r));
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

  // Half of a slot this wave reads in a step with tiles (kA, kB): its own
  // block's half when the entry is paired, else the first half.
  const uint32_t blk_half = blk != 0 ? 8192u : 0u;
  auto rhalf = [&](int kA, int kB) -> uint32_t { return kA != kB ? blk_half : 0u; };

  // One pipeline step on half tile j (scores in s_cur, V in slot VS, this
  // wave's first key my_key, read half rh) that also computes S(j+1) into
  // s_nxt from K slot VS^1, half rh_n, when DO_QK.
  auto step = [&](auto vs_c, auto biased_c, auto masked_c, auto do_qk_c, f32x16 &s_cur, f32x16 &s_nxt,
                  int my_key, uint32_t rh, uint32_t rh_n, auto dma_k, auto dma_v) {
    constexpr int VS = decltype(vs_c)::value;
    constexpr bool BIASED = decltype(biased_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    constexpr bool DO_QK = decltype(do_qk_c)::value;
    const unsigned char *vbuf = smem + kPVOff + VS * 16384 + rh;
    const unsigned char *kbuf = smem + kPKOff + (VS ^ 1) * 16384 + rh_n;
    const float *bs = reinterpret_cast<const float *>(smem + kPBOff + VS * 256 + (rh >> 6));

    // K fragment dc of S(j+1) (dims 16*dc .. +15) and V fragment dt of keys
    // 16*kc .. +15 (dims 32*dt .. +31, transposed on the read)
    auto k_frag = [&](int dc) -> bf16x8 {
      return *reinterpret_cast<const bf16x8 *>(kbuf + (k_rd0 ^ (32u * (dc & 3))) + 1024 * (dc >> 2));
    };
    auto v_frag = [&](int kc, int dt) -> bf16x8 {
      const unsigned char *src = vbuf + ((dt & 1) ? (v_rd0 ^ 64u) : v_rd0) + 4096 * kc + 1024 * (dt >> 1);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, src));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, src + 2048));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto qk = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[r] = 0.f;
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(dc), qf[dc], s_nxt, 0, 0, 0);
    };
    auto bias4 = [&](int q4) {
      const float4 b4 = *reinterpret_cast<const float4 *>(bs + 8 * q4 + 4 * g);
      return make_float4(b4.x * kLog2e, b4.y * kLog2e, b4.z * kLog2e, b4.w * kLog2e);
    };
    // tile max of this lane's logits (log2 units), then the rare rescale
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
    auto rescale = [&](float mt) {
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
    };
    bf16x8 pf[2];
    // P of keys 16*h .. +15 of this lane's 32 (q4 = 2h, 2h+1) into pf[h],
    // their sum added to acc
    auto exps_half = [&](float m_sub, auto h_c, float &acc) {
      constexpr int H0 = 2 * decltype(h_c)::value;
#pragma unroll
      for (int q4 = H0; q4 < H0 + 2; ++q4) {
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
          pf[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(e[u]);
          pf[r >> 3][(r & 7) + 1] = (__bf16)__builtin_amdgcn_exp2f(e[u + 1]);
        }
      }
      // row sums of the bf16-rounded P, from the packed fragment itself
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 two = {pf[H0 >> 1][2 * i], pf[H0 >> 1][2 * i + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(two, ones, acc, false);
      }
    };
    auto exps = [&](float m_sub, float &acc) {
      exps_half(m_sub, Int<0>{}, acc);
      exps_half(m_sub, Int<1>{}, acc);
    };
    // O^T += V^T P^T over the half tile's 32 keys
    auto pv = [&]() {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(kc, dt), pf[kc], o[dt], 0, 0, 0);
    };

    if (MASKED) {
      // general step: copies and S(j+1) first, then this wave's tile if it
      // has one
      dma_k();
      dma_v();
      if (DO_QK) qk();
      // a virtual tile's keys end at its block's virtual key count
      const bool virt = kSpark && my_key >= kVirtA;
      if (!virt && my_key >= T) return;     // this wave's block has no tile in this step
      const int lim = !virt ? T : my_key >= kVirtB ? kVirtB + nvB : kVirtA + nvA;
      const int kbase = my_key + 4 * g;   // key of s[r] = kbase + 8*(r/4) + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 8 * (r >> 2) + (r & 3) >= lim) s_cur[r] = -INFINITY;
      rescale(tile_max());
      exps(m_used == -INFINITY ? 0.f : m_used, l_run);
      pv();
      return;
    }

    // Full tiles.  P is taken against the running max as it stands, with no
    // tile max: the copies come first, then one straight block in a fixed
    // order (sched_barrier fences keep the scheduler from regrouping it): the
    // K fragments of S(j+1) are read at once, every S(j+1) MFMA is followed
    // by the exponentials of two of this lane's logits (so that the matrix
    // and vector units of the wave work side by side), the V fragments are
    // read half way.  A P above 2^32 (the running max stale by more than 32,
    // or not yet set: every P is then +inf) shows in the tile's sum; then,
    // rarely, the tile max moves the running max, O and the row sum are
    // rescaled and the tile's P are taken again, so that every P fed to the
    // PV MFMAs that end the step is at most 2^32: far from fp32 and bf16
    // overflow, and no loss of relative precision.
    dma_k();
    dma_v();
    __builtin_amdgcn_s_setprio(1);
    bf16x8 kf[8];
    if (DO_QK) {
#pragma unroll
      for (int dc = 0; dc < 8; ++dc) kf[dc] = k_frag(dc);
    }
    bf16x8 vf[4], vg[4];
    float4 bq = make_float4(0.f, 0.f, 0.f, 0.f);
    float l_t = 0.f;   // this lane's share of the tile's row sum
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (DO_QK) {
        if (i == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s_nxt[r] = 0.f;
        }
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[i], s_nxt, 0, 0, 0);
      }
      // logits r = 2i, 2i+1 (q4 = i/2)
      const int r = 2 * i;
      if (BIASED && (i & 1) == 0) bq = bias4(i >> 1);
      float e0, e1;
      if (BIASED) {
        e0 = __builtin_fmaf(s_cur[r], c, ((i & 1) ? bq.z : bq.x) - m_used);
        e1 = __builtin_fmaf(s_cur[r + 1], c, ((i & 1) ? bq.w : bq.y) - m_used);
      } else {
        e0 = __builtin_fmaf(s_cur[r], c, -m_used);
        e1 = __builtin_fmaf(s_cur[r + 1], c, -m_used);
      }
      pf[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(e0);
      pf[r >> 3][(r & 7) + 1] = (__bf16)__builtin_amdgcn_exp2f(e1);
      const bf16x2 two = {pf[r >> 3][r & 7], pf[r >> 3][(r & 7) + 1]};
      l_t = __builtin_amdgcn_fdot2_f32_bf16(two, ones, l_t, false);
      // V fragments of keys 0-15 and 16-31, read while the S(j+1) MFMAs
      // run (late enough that few K fragments are still held)
      if (i == 3) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vf[dt] = v_frag(0, dt);
      }
      if (i == 5) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vg[dt] = v_frag(1, dt);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // a sum of non-negative terms is at least its largest term; NaN (from
    // an infinite logit meeting an infinite max) fails the test too
    if (__any(!(l_t <= kPMax))) {
      const float mt = tile_max();
      const float m_new = fmaxf(m_used, mt);
      const float alpha = m_new > m_used ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.f;  // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m_used = m_new;
      l_t = 0.f;
      exps(m_used == -INFINITY ? 0.f : m_used, l_t);
    }
    l_run += l_t;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt], pf[0], o[dt], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vg[dt], pf[1], o[dt], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- pipeline -----------------------------------------------------------
  // Step j = 2e + half works on half `half` of entry e.  K(j) lives in K slot
  // j%2 and V(j) in V slot j%2; K is fetched two steps ahead, V one ahead.
  // Step j issues V(j+1) and K(j+2) into the slots step j-1 finished
  // reading, and ends with the barrier that publishes them.
  int ea = T, eb = T, na = T, nb2 = T;   // first keys (T: no tile)
  if (nE > 0) entry(0, ea, eb);
  if (nE > 1) entry(1, na, nb2);
  if (nE > 0) {
    issue_k(hkey(ea, 0), hkey(eb, 0), 0);
    issue_v(hkey(ea, 0), hkey(eb, 0), 0, 0);
    issue_k(hkey(ea, 1), hkey(eb, 1), 1);
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  f32x16 s0, s1;
  if (nE > 0) {
    const unsigned char *kb0 = smem + kPKOff + rhalf(hkey(ea, 0), hkey(eb, 0));
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.f;
#pragma unroll
    for (int dc = 0; dc < 8; ++dc) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb0 + (k_rd0 ^ (32u * (dc & 3))) + 1024 * (dc >> 2));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s0, 0, 0, 0);
    }
  }
  // Step 0 refills K slot 0: every wave must be done reading it.
  __syncthreads();

  // Both steps of entry e (not the last entry), with (na, nb2) = entry e+1.
  // PH: 0 unbiased, 1 biased, 2 general (masked; biased when key_bias).
  auto run_entry = [&](auto biased_c, auto masked_c, int e) {
    const int a0 = hkey(ea, 0), b0 = hkey(eb, 0), a1 = hkey(ea, 1), b1 = hkey(eb, 1);
    const int n0a = hkey(na, 0), n0b = hkey(nb2, 0), n1a = hkey(na, 1), n1b = hkey(nb2, 1);
    // half 0
    step(Int<0>{}, biased_c, masked_c, Bool<true>{}, s0, s1, blk ? b0 : a0, rhalf(a0, b0), rhalf(a1, b1),
         [&] { issue_k(n0a, n0b, 0); }, [&] { issue_v(a1, b1, 1, e); });
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    // half 1
    step(Int<1>{}, biased_c, masked_c, Bool<true>{}, s1, s0, blk ? b1 : a1, rhalf(a1, b1), rhalf(n0a, n0b),
         [&] { issue_k(n1a, n1b, 1); }, [&] { issue_v(n0a, n0b, 0, e + 1); });
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    ea = na;
    eb = nb2;
    if (e + 2 < nE) entry(e + 2, na, nb2);
  };
  // The last entry: half 0 computes S of half 1; half 1 ends the walk.
  auto last_entry = [&](auto biased_c, auto masked_c, int e) {
    const int a0 = hkey(ea, 0), b0 = hkey(eb, 0), a1 = hkey(ea, 1), b1 = hkey(eb, 1);
    step(Int<0>{}, biased_c, masked_c, Bool<true>{}, s0, s1, blk ? b0 : a0, rhalf(a0, b0), rhalf(a1, b1),
         [] {}, [&] { issue_v(a1, b1, 1, e); });
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
    step(Int<1>{}, biased_c, masked_c, Bool<false>{}, s1, s0, blk ? b1 : a1, rhalf(a1, b1), 0u, [] {}, [] {});
  };
  // Each loop body holds one step variant only: a runtime choice between
  // variants inside a loop makes the compiler route the accumulators through
  // copies every step.
  int e = 0;
  const int nUB = nU + nBi;
  for (; e < nU && e + 1 < nE; ++e) run_entry(Bool<false>{}, Bool<false>{}, e);
  for (; e < nUB && e + 1 < nE; ++e) run_entry(Bool<true>{}, Bool<false>{}, e);
  if (has_bias || kSpark) {
    for (; e + 1 < nE; ++e) run_entry(Bool<true>{}, Bool<true>{}, e);
  } else {
    for (; e + 1 < nE; ++e) run_entry(Bool<false>{}, Bool<true>{}, e);
  }
  if (e < nE) {
    if (e < nU) last_entry(Bool<false>{}, Bool<false>{}, e);
    else if (e < nUB) last_entry(Bool<true>{}, Bool<false>{}, e);
    else if (has_bias || kSpark) last_entry(Bool<true>{}, Bool<true>{}, e);
    else last_entry(Bool<false>{}, Bool<true>{}, e);
  }

  // ---- epilogue -----------------------------------------------------------
  if (!active) return;
  if (self_wg) {
    // waves 2-3 hand (max, row-sum share, O) of the second key half to waves
    // 0-1, which own the same rows in the same lane layout: O in the K ring
    // (no longer read: the last step computes no S), 16 KiB per wave as
    // [value][lane], max and sum in the schedule area, unused by the dense
    // rows
    float *xo = reinterpret_cast<float *>(smem + kPKOff) + rw * (64 * 64);
    float *xm = reinterpret_cast<float *>(smem + kPSchOff) + rw * 128;
    if (blk == 1) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(16 * dt + r) * 64 + lane] = o[dt][r];
      xm[lane] = m_used;
      xm[64 + lane] = l_run;
    }
    __syncthreads();
    if (blk == 0) {
      const float mB = xm[lane], lB = xm[64 + lane];
      const float mN = fmaxf(m_used, mB);
      const float aA = m_used == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_used - mN);
      const float aB = mB == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mB - mN);
      l_run = l_run * aA + lB * aB;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * aA + xo[(16 * dt + r) * 64 + lane] * aB;
      m_used = mN;
    }
    // the output staging below reuses the K ring
    __syncthreads();
    if (blk == 1) return;
  }
  const float l_tot = add_with_partner(l_run);
  if (kDense && p.nsplit > 1) {
    if (tq >= T) return;
    // partial (unnormalised O, max, sum) of this key range
    const int64_t prow = (((int64_t)bh * p.nqb + qbi) * p.nsplit + split) * kBlock + (rw * 32 + c32);
    float *po = p.part_o + prow * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * dt + 8 * q4 + 4 * g;
        *reinterpret_cast<float4 *>(po + d0) =
            make_float4(o[dt][4 * q4 + 0], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]);
      }
    if (g == 0) *reinterpret_cast<float2 *>(p.part_ml + 2 * prow) = make_float2(m_used, l_tot);
    return;
  }
  // The wave's 32 rows (256 B each) go through LDS (8 KiB of the K ring per
  // wave, unused since the last step reads no K; 16-byte chunks XOR-swizzled
  // by row) and out as whole rows: each store instruction writes 4 rows.
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  unsigned char *stage = smem + kPKOff + 8192 * wave;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint2 val;
      val.x = pack_bf16x2(o[dt][4 * q4 + 0] * inv, o[dt][4 * q4 + 1] * inv);
      val.y = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2 *>(stage + c32 * 256 + 16 * ((4 * dt + q4) ^ (c32 & 15)) + 8 * g) = val;
    }
  const int row0 = qb * kBlock + rw * 32;
  uint16_t *ob = p.out + bbase + h * kHeadDim;
  const int ch = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const uint4 val = *reinterpret_cast<const uint4 *>(stage + r * 256 + 16 * (ch ^ (r & 15)));
    if (row0 + r >= p.row_lo && row0 + r < p.row_hi)
      *reinterpret_cast<uint4 *>(ob + (int64_t)(row0 + r) * rs + 8 * ch) = val;
  }
  if (p.lse != nullptr && g == 0 && tq >= p.row_lo && tq < p.row_hi)
    p.lse[((int64_t)b * p.H + h) * T + tq] = (m_used + __log2f(l_tot)) * kLn2;
}

PairParams make_pair_params(const AttnArgs &a, int qb0, int nqb) {
  PairParams p{};
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
  p.npair = (nqb + 1) / 2;
  p.row_lo = 0;
  p.row_hi = a.T;
  p.nsplit = 1;
  p.tiles_per_split = a.nb;
  p.scale_log2 = a.scale_log2;
  p.qbar = a.qbar;
  p.kbar = a.kbar;
  p.budget = a.budget;
  p.radius = a.radius;
  p.list_out = a.list_out;
  p.cnt_out = a.cnt_out;
  p.slots = 0;
  return p;
}

// Resident paired-kernel workgroups per XCD on the current device (two per
// CU, eight XCDs), looked up once per device.
int pair_slots_per_xcd() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    return 0;
  v = 2 * (cus / 8);
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

int dense_pair_splits(int B, int H, int nb, int nvb) {
  const int nq = nb - nvb;
  if (nq <= 0) return 1;
  const int64_t units = (int64_t)B * H * ((nq + 1) / 2);
  // Choose the key split that minimises (rounds of resident workgroups) x
  // (key blocks per split + the fixed cost of a workgroup, about 8 blocks:
  // prologue, stores, partial results).  Two workgroups fit a CU and the
  // device has 256 CUs.  Splits keep at least 8 blocks each; among equal
  // costs the fewer splits win (less partial traffic for the combine).
  constexpr int64_t kSlots = 2 * 256;
  constexpr int64_t kFixedTiles = 8;
  const int max_s = nb / 8 > 1 ? nb / 8 : 1;
  int best = 1;
  int64_t best_cost = -1;
  for (int s = 1; s <= max_s; ++s) {
    const int per = (nb + s - 1) / s;
    const int se = (nb + per - 1) / per;          // splits after equalising
    if (se != s) continue;
    const int64_t rounds = (units * se + kSlots - 1) / kSlots;
    const int64_t cost = rounds * (per + kFixedTiles);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = se;
    }
  }
  return best;
}

hipError_t launch_attn_pair_sparse(const AttnArgs &a, hipStream_t stream) {
  if (a.nvq <= 0) return hipSuccess;
  if (a.max_sel > kMaxPairList) return hipErrorInvalidValue;
  PairParams p = make_pair_params(a, 0, a.nvq);
  p.row_hi = a.rows_end;
  p.slots = pair_slots_per_xcd();
  const int total = a.B * a.H * p.npair;
  hipLaunchKernelGGL((attn_pair_kernel<false, false>), dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_pair_spark(const AttnArgs &a, hipStream_t stream) {
  if (a.nvq <= 0) return hipSuccess;
  if (a.max_sel > kMaxPairSparkList || a.nvb > kMaxRouteBlocks || a.sum_k == nullptr || a.sum_v == nullptr ||
      a.sum_lm == nullptr)
    return hipErrorInvalidValue;
  PairParams p = make_pair_params(a, 0, a.nvq);
  p.row_hi = a.rows_end;
  p.slots = pair_slots_per_xcd();
  p.sum_k = static_cast<const uint16_t *>(a.sum_k);
  p.sum_v = static_cast<const uint16_t *>(a.sum_v);
  p.sum_lm = a.sum_lm;
  const int total = a.B * a.H * p.npair;
  hipLaunchKernelGGL((attn_pair_kernel<false, false, true>), dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_pair_fused(const AttnArgs &a, hipStream_t stream) {
  if (a.nvq <= 0) return hipSuccess;
  if (a.max_sel > kMaxPairList || a.nvb > kMaxRouteBlocks || a.qbar == nullptr ||
      (a.nvb > 0 && a.kbar == nullptr))
    return hipErrorInvalidValue;
  PairParams p = make_pair_params(a, 0, a.nvq);
  p.row_hi = a.rows_end;
  p.slots = pair_slots_per_xcd();
  const int total = a.B * a.H * p.npair;
  hipLaunchKernelGGL((attn_pair_kernel<false, true>), dim3(total), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_pair_dense(const AttnArgs &a, float *part_o, float *part_ml, int nsplit,
                                  hipStream_t stream) {
  const int nq = a.nb - a.nvb;
  PairParams p = make_pair_params(a, a.nvb, nq);
  p.row_lo = a.rows_end;
  if (nsplit > 1) {
    p.nsplit = nsplit;
    p.tiles_per_split = (a.nb + nsplit - 1) / nsplit;
    p.part_o = part_o;
    p.part_ml = part_ml;
  }
  const int total = a.B * a.H * p.npair * p.nsplit;
  hipLaunchKernelGGL((attn_pair_kernel<true, false>), dim3(total), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sa
