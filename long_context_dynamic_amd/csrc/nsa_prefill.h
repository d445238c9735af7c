// nsa_prefill.h -- arguments and launchers of the matrix-core NSA kernels
// (internal).
#pragma once

#include "nsa_internal.h"

namespace nsa {

struct PfArgs {
  const uint16_t* q;      // [B, T, H, DQ]
  const uint16_t* k;      // [B, L, G, DQ]
  const uint16_t* kG;     // [B, G, Lp / 16, DQ / 32, 8, 2, 32] keys, per group, paired rows
  const uint16_t* vT;     // [B, G, Lp / 32, DV, 32]  values, tiled and key-contiguous
  const uint16_t* kc;     // [B, nb, G, DQ]   block summaries
  const uint16_t* vcT;    // [B, G, nbp / 32, DV, 32]  value summaries, tiled likewise
  const uint16_t* gates;  // [B, T, H, 3] or NULL
  float* acc;             // [B, T, H, DV]    gated compressed + window partial sum
  int32_t* idx;           // [B, T, G, n]
  float* score;           // [B, T, G, n] or NULL
  void* out;              // [B, T, H, DV]
  float* lse;             // [B, T, H] or NULL
  float* sv_lse;          // training forward: [3][B, T, H] per-branch natural log-sum-exp, or NULL
  uint16_t* sv_o;         // training forward: [3][B, T, H, DV] per-branch outputs (bf16), or NULL
  int64_t B, T, L, G, H, nb, nbp, Lp, n, w;
  int64_t bs, per, nbs;  // summary block, summaries per 64-token selection block, selection blocks
  uint32_t flags;
  float scale;
};

// True when the matrix-core kernels take this shape: bf16, 16 heads per
// group, 64-token selection blocks over 16-, 32- or 64-token summaries,
// d_qk in {64,128,192}, d_v in {64,128}, nb <= 2048 summaries, top_k <= 32.
bool prefill_fast_ok(const Prob& P);

hipError_t launch_group_major(const void* src, void* dst, int64_t B, int64_t L, int64_t G, int D, hipStream_t s);
hipError_t launch_transpose(const void* src, void* dst, int64_t B, int64_t N, int64_t Np, int64_t G, int D,
                            hipStream_t s);
// fwd: compressed + window + selection + gated partial (acc); else selection only.
hipError_t launch_cmpwin(const Prob& P, const PfArgs& a, bool fwd, hipStream_t s);
// fwd: out = acc + gate * selected branch; else out = selected branch (+ lse).
hipError_t launch_sel(const Prob& P, const PfArgs& a, bool fwd, bool out_f32, hipStream_t s);

}  // namespace nsa
