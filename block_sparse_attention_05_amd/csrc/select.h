// Top-K selection of one query block's exact list, shared by the route
// kernel and the fused attention kernel (page "Sol-Attn and Spark for
// MiniMax-H3": Spark inference integration, fixed-ratio Top-K with an exact
// boundary selection; H3 pipeline integration, forced self / neighbour
// blocks outside the budget; page "Add key bias to chunked Sol-Attn
// producers", Tests and source audit: sink blocks are never candidates).
//
// One wavefront handles one row.  Lane l holds candidate blocks 64e + l
// (e < E) as order-preserving 32-bit keys; the k best under (score desc,
// index asc) are found by repeated wave-wide argmax (small budgets) or by a
// most-significant-bit-first radix select on ballot counts (large budgets);
// a ballot/popcount scan then emits selected and forced blocks ascending,
// the sink blocks [nvb, nb), and -1 padding up to max_sel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kTournamentMax = 32;  // largest budget selected by repeated argmax

// fp32 -> unsigned key with the same order (larger score, larger key); -0.0
// is mapped like +0.0.  Every finite score maps above 0.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// Mask of the bits above `bit` (bit in [-1, 32]: all bits for -1, none for
// 31 and up).
__device__ __forceinline__ uint32_t high_bits(int bit) {
  return bit >= 31 ? 0u : (bit < 0 ? 0xffffffffu : ~((2u << bit) - 1u));
}

// Wave-wide max / min of unsigned values (DPP scan inside rows of 16 lanes,
// then row broadcasts; lane 63 ends with the result).
template <bool kMax>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return kMax ? (a > b ? a : b) : (a < b ? a : b); };
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x118, 0xf, 0xf, false));  // row_shr:8
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Small budgets: kk rounds of a wave-wide argmax over the keys not yet
// taken (ties on the score key go to the lower block index j = 64e + lane).
// Returns the taken slots as a bit mask per lane.
template <int E>
__device__ __forceinline__ uint32_t tournament_select(const uint32_t (&u)[E], int kk, int lane) {
  uint32_t taken = 0;
  for (int round = 0; round < kk; ++round) {
    uint32_t cur = 0;
    int ebest = 0;
#pragma unroll
    for (int e = E - 1; e >= 0; --e) {  // lowest e wins a tie inside the lane
      const uint32_t x = ((taken >> e) & 1u) ? 0u : u[e];
      if (x >= cur) { cur = x; ebest = e; }
    }
    const uint32_t m = wave_reduce_u32<true>(cur);
    const uint64_t eq = __ballot(cur == m);
    int win_lane, win_e;
    if (popc(eq) == 1) {
      win_lane = __builtin_ctzll(eq);
      win_e = __builtin_amdgcn_readlane(ebest, win_lane);
    } else {
      const uint32_t jm = wave_reduce_u32<false>(cur == m ? (uint32_t)(64 * ebest + lane) : 0xffffffffu);
      win_lane = (int)(jm & 63u);
      win_e = (int)(jm >> 6);
    }
    if (lane == win_lane) taken |= 1u << win_e;
  }
  return taken;
}

// Selects and emits the list of query block i from its scores srow[j],
// j < nvb (any memory the wave can read).  Writes the list to out[0,
// max_sel) and, when scores_row is not null, the scores to scores_row[j].
// Returns the list length.  nvb <= 64 * E.
template <int E>
__device__ __forceinline__ int select_and_emit(const float *srow, int i, int nvb, int nb, int budget,
                                               int radius, int max_sel, int32_t *out,
                                               float *scores_row, int lane) {
  const int f_lo = i - radius < 0 ? 0 : i - radius;
  const int f_hi = i + radius > nvb - 1 ? nvb - 1 : i + radius;
  const int n_cand = nvb - (f_hi - f_lo + 1);
  const int kk = budget < n_cand ? budget : n_cand;

  // order keys; 0 (below every finite score) for non-candidates
  uint32_t u[E];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + lane;
    const float s = j < nvb ? srow[j] : 0.f;
    if (scores_row != nullptr && j < nvb) scores_row[j] = s;
    const bool v = j < nvb && (j < f_lo || j > f_hi);
    u[e] = v ? order_key(s) : 0u;
    mn = v && u[e] < mn ? u[e] : mn;
    mx = u[e] > mx ? u[e] : mx;
  }

  // 2. radix select: `pre` holds the decided high bits of the kk-th key,
  // `rem` how many keys are still to be taken from the bucket of keys that
  // match `pre` on those bits; keys above the bucket are taken.
  const int n_off = 64 * E - n_cand;  // non-candidates (key 0)
  int rem = kk;
  int stop = 32;  // 32: nothing to take; else the bit the search stopped at
  uint32_t pre = 0u;
  uint32_t taken = 0;  // tournament result (bit e: slot e)
  const bool tour = kk > 0 && kk <= kTournamentMax && kk < n_cand;
  if (tour) {
    taken = tournament_select<E>(u, kk, lane);
  } else if (kk > 0) {
    mn = wave_reduce_u32<false>(mn);
    mx = wave_reduce_u32<true>(mx);
    const int fb = mn >= mx ? -1 : 31 - __builtin_clz(mn ^ mx);
    pre = fb < 0 ? mx : (mx & high_bits(fb));
    for (int bit = fb;; --bit) {
      const uint32_t hm = high_bits(bit);
      int bucket = 0, c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool in_b = ((u[e] ^ pre) & hm) == 0u;
        bucket += popc(__ballot(in_b));
        c += popc(__ballot(in_b && bit >= 0 && ((u[e] >> (bit & 31)) & 1u)));
      }
      if ((pre & hm) == 0u) bucket -= n_off;
      if (bucket == rem || bit < 0) {
        stop = bit;
        break;
      }
      if (c >= rem) pre |= 1u << bit;
      else rem -= c;
    }
  }

  // 3. emission: keys above the bucket, the bucket whole when the search
  // stopped on it, or (stop = -1) its first rem keys by block index
  const uint32_t hm = high_bits(stop);
  const uint32_t ph = pre & hm;
  int base = 0, ties = rem;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + lane;
    const uint32_t uh = u[e] & hm;
    bool take = tour ? ((taken >> e) & 1u) != 0u && u[e] != 0u
                     : stop != 32 && u[e] != 0u && (uh > ph || (stop >= 0 && uh == ph));
    if (stop == -1) {
      const bool eq = u[e] != 0u && u[e] == pre;
      const uint64_t m = __ballot(eq);
      if (eq && popc(m & ((1ull << lane) - 1ull)) < ties) take = true;
      ties -= popc(m) < ties ? popc(m) : ties;
    }
    const bool f = j < nvb && (take || (j >= f_lo && j <= f_hi));
    const uint64_t m = __ballot(f);
    if (f) out[base + popc(m & ((1ull << lane) - 1ull))] = j;
    base += popc(m);
  }
  for (int j = nvb + lane; j < nb; j += 64) out[base + (j - nvb)] = j;
  const int cnt = base + (nb - nvb);
  for (int x = cnt + lane; x < max_sel; x += 64) out[x] = -1;
  return cnt;
}

}  // namespace sa
