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
