// nsa_topk.h -- one wave's top-k over a row of block importances (internal).
// [P1] s4: the forced blocks come first, then the visible blocks with the
// largest group importance, ties to the lower block id.
#pragma once

#include "nsa_mfma.h"

namespace nsa {

// vals[i] holds the importance of block lane + 64 * i (-1 where the block is
// not visible, i.e. >= nvis).  Forced blocks are taken out of the running
// here.  Afterwards lane k < the returned count holds the k-th chosen block
// in cj and its score in cs (+inf for forced blocks), forced ones first, the
// rest by falling importance.  Each round finds the largest remaining value
// and the lowest block id holding it with two cross-lane reductions.  Every
// lane keeps its best and second-best candidates in the order (importance
// falling, block id rising); the winning lane moves its second-best up, and
// only a lane that wins while its second-best is unknown rescans its
// candidates (for the best one after the block it gave last).
template <int NBL>
__device__ __forceinline__ int topk_wave(float (&vals)[NBL], int64_t nvis, int64_t cur, uint32_t flags, int n,
                                         int& cj, float& cs) {
  const int lane = threadIdx.x & 63;
  const bool first = flags & NSA_F_FORCE_FIRST;
  const bool current = (flags & NSA_F_FORCE_CURRENT) && !(first && cur == 0);
  const int f0 = first ? 0 : (current ? (int)cur : -1);
  const int f1 = (first && current) ? (int)cur : -1;
  const int nf = (f0 >= 0) + (f1 >= 0);
  int ncand = (int)nvis;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int fb = f == 0 ? f0 : f1;
    if (fb >= 0 && fb < nvis) {
      --ncand;
      // selects, not indexed stores: vals stays in registers
#pragma unroll
      for (int i = 0; i < NBL; ++i) vals[i] = (lane == (fb & 63) && i == (fb >> 6)) ? -1.f : vals[i];
    }
  }
  const int r_take = (n - nf) < ncand ? (n - nf) : ncand;
  cj = -1;
  cs = -INFINITY;
  if (lane == 0 && f0 >= 0) { cj = f0; cs = INFINITY; }
  if (lane == 1 && f1 >= 0) { cj = f1; cs = INFINITY; }
  // this lane's best and second-best candidates (strict comparisons over a
  // rising index: of equal values the lower index ranks first)
  float bv = -1.f, bv2 = -1.f;
  int bi = 0, bi2 = 0;
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const float v = vals[i];
    const bool top = v > bv, second = !top && v > bv2;
    bv2 = top ? bv : (second ? v : bv2);
    bi2 = top ? bi : (second ? i : bi2);
    bv = top ? v : bv;
    bi = top ? i : bi;
  }
  bool known2 = true;  // bv2 / bi2 hold the lane's second-best
  for (int round = 0; round < r_take; ++round) {
    const float M = wave_allmax(bv);
    const int J = wave_allmin_u(bv == M ? lane + 64 * bi : 0x7fffffff);
    if (lane == nf + round) { cj = J; cs = M; }
    const bool win = lane == (J & 63);
    const bool rescan = __builtin_amdgcn_readlane((int)(win && !known2), J & 63);
    if (rescan) {
      // the winner's best candidate after (M, its index): the lane's
      // candidates in order below it
      if (win) {
        const float lv = bv;
        const int li = bi;
        bv = -1.f;
        bi = 0;
#pragma unroll
        for (int i = 0; i < NBL; ++i) {
          const float v = vals[i];
          const bool after = v < lv || (v == lv && i > li);
          if (after && v > bv) { bv = v; bi = i; }
        }
      }
    } else if (win) {
      bv = bv2;
      bi = bi2;
      known2 = false;
    }
  }
  return nf + r_take;
}

// Maximum of unsigned values over all 64 lanes, returned in every lane.
__device__ __forceinline__ unsigned wave_allmax_u32(unsigned x) {
  x = max(x, (unsigned)dpp_i<kDppXor1>((int)x));
  x = max(x, (unsigned)dpp_i<kDppXor2>((int)x));
  x = max(x, (unsigned)dpp_i<kDppHalfMirror>((int)x));
  x = max(x, (unsigned)dpp_i<kDppMirror>((int)x));
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max((unsigned)r[0], (unsigned)r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((unsigned)r[0], (unsigned)r[1]);
}

// The same selection as topk_wave for at most 1024 blocks (NBL <= 16), one
// cross-lane reduction per round: each candidate is one 32-bit key, its
// importance's exponent and top 14 mantissa bits (plus one, so every
// candidate's key is above the 0 of the non-candidates) over 10 bits of
// 1023 - block id, so a larger key means a larger importance and, among
// importances that agree to 2^-14 relative, the lower block id.  Keys are
// distinct; each lane keeps its best and second-best and rescans (below
// the key it gave last) only when it wins with its second-best unknown.
// Returns the count; lane k < count holds the k-th chosen block in cj
// (forced ones first, in lanes 0 .. nforced - 1).
template <int NBL>
__device__ __forceinline__ int topk_wave_keys(const float (&vals)[NBL], int64_t nvis, int64_t cur, uint32_t flags,
                                              int n, int& cj, int& nforced) {
  static_assert(NBL <= 16, "10 bits of block id");
  const int lane = threadIdx.x & 63;
  const bool first = flags & NSA_F_FORCE_FIRST;
  const bool current = (flags & NSA_F_FORCE_CURRENT) && !(first && cur == 0);
  const int f0 = first ? 0 : (current ? (int)cur : -1);
  const int f1 = (first && current) ? (int)cur : -1;
  const int nf = (f0 >= 0) + (f1 >= 0);
  int ncand = (int)nvis;
  if (f0 >= 0 && f0 < nvis) --ncand;
  if (f1 >= 0 && f1 < nvis) --ncand;
  unsigned kv[NBL];
  unsigned b1 = 0u, b2 = 0u;  // this lane's best and second-best key
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int j = lane + 64 * i;
    const float v = vals[i];
    const bool cand = j < nvis && j != f0 && j != f1 && v >= 0.f;
    const unsigned k = cand ? ((((unsigned)__float_as_uint(v) >> 9) + 1u) << 10) | (unsigned)(1023 - j) : 0u;
    kv[i] = k;
    b2 = k > b1 ? b1 : max(b2, k);
    b1 = max(b1, k);
  }
  const int r_take = (n - nf) < ncand ? (n - nf) : ncand;
  cj = -1;
  if (lane == 0 && f0 >= 0) cj = f0;
  if (lane == 1 && f1 >= 0) cj = f1;
  // Every step stays in the vector unit (the reduction leaves the maximum in
  // every lane): no scalar round trip per round.  Only the winning lane can
  // take the rescan branch, which the wave skips when it does not.
  bool known2 = true;
  for (int round = 0; round < r_take; ++round) {
    const unsigned M = wave_allmax_u32(b1);
    const int J = 1023 - (int)(M & 1023u);
    if (lane == nf + round && M != 0u) cj = J;  // M == 0: no candidate left (non-finite importances)
    const bool win = lane == (J & 63) && M != 0u;
    if (win && !known2) {
      // the winner's best and second-best keys below M
      unsigned c1 = 0u, c2 = 0u;
#pragma unroll
      for (int i = 0; i < NBL; ++i) {
        const unsigned k = kv[i] < M ? kv[i] : 0u;
        c2 = k > c1 ? c1 : max(c2, k);
        c1 = max(c1, k);
      }
      b1 = c1;
      b2 = c2;
      known2 = true;
    } else if (win) {
      b1 = b2;
      known2 = false;
    }
  }
  const int taken = __popcll(__ballot(lane >= nf && lane < nf + r_take && cj >= 0));
  nforced = nf;
  return nf + taken;
}

// Writes the chosen blocks of topk_wave ascending to orow[0 .. n) (padding
// -1) and their scores to srow (padding -inf) when srow is given.
__device__ __forceinline__ void topk_write(int cnt, int cj, float cs, int n, int32_t* orow, float* srow) {
  const int lane = threadIdx.x & 63;
  int rank = 0;  // lane reads into a scalar register: no LDS round trip per chosen block
  for (int k2 = 0; k2 < cnt; ++k2) rank += (__builtin_amdgcn_readlane(cj, k2) < cj) ? 1 : 0;
  if (lane < cnt) {
    orow[rank] = cj;
    if (srow) srow[rank] = cs;
  } else if (lane < n) {
    orow[lane] = -1;
    if (srow) srow[lane] = -INFINITY;
  }
}

}  // namespace nsa
