// nsa_prefill.h -- arguments and launchers of the matrix-core NSA kernels
// (internal).
#pragma once

#include "nsa_internal.h"
#include "nsa_paths.h"

namespace nsa {

struct PfArgs {
  const uint16_t* q;      // [B, T, H, DQ]
  uint16_t* qF;           // [B, T, G, DQ / 32, 64, 8] queries in fragment order (nsa_frag.h); the
                          // compressed/window kernel writes it, the selected branch reads it
  const uint16_t* k;      // [B, L, G, DQ]
  const uint16_t* kF;     // [B, G, Lp / 32, DQ / 32, 2, 64, 8] keys in fragment order (nsa_frag.h)
  const uint16_t* vT;     // [B, G, Lp / 32, DV, 32]  values, tiled and key-contiguous
  const uint16_t* vF;     // [B, G, Lp / 32, DV / 16, 64, 8] values in fragment order (nsa_frag.h)
  const uint16_t* kc;     // [B, nb, G, DQ]   block summaries
  const uint16_t* vcT;    // [B, G, nbp / 32, DV, 32]  value summaries, tiled likewise
  const uint16_t* gates;  // [B, T, H, 3] or NULL
  float* acc;             // [B, T, G, DV / 16, 64, 4] gated compressed + window partial sum, fragment order
  uint16_t* part_o;       // [B, T, G, 8, DV / 32, 64, 8] selected branch per XCD stripe: normalised output (bf16), in the matrix op's lane order
  float* part_l;          // [B, T, G, 16, 8]      ... and its log-sum-exp (log2 units, -inf when empty)
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
// Fragment-order images of K (from K [B, L, G, D]) and of V (from the tiled
// V^T), Lp = round_up(L, 64) keys each.
hipError_t launch_frag_k(const void* k, void* kF, int64_t B, int64_t L, int64_t G, int D, hipStream_t s);
// Fragment-order image of the queries (q [R, G * 16, D] -> [R, G, D / 32, 64, 8]).
hipError_t launch_frag_q(const void* q, void* qF, int64_t R, int64_t G, int D, hipStream_t s);
hipError_t launch_frag_v(const void* vT, void* vF, int64_t B, int64_t L, int64_t G, int D, hipStream_t s);
hipError_t launch_transpose(const void* src, void* dst, int64_t B, int64_t N, int64_t Np, int64_t G, int D,
                            hipStream_t s);
// fwd: compressed + window + selection + gated partial (acc); else selection only.
hipError_t launch_cmpwin(const Prob& P, const PfArgs& a, bool fwd, hipStream_t s);
// Two kernels: the selected branch per XCD stripe (partials), then their
// merge -- fwd: out = acc + gate * selected branch; else out = selected
// branch (+ lse).  ph (may be NULL) is marked between the two.
hipError_t launch_sel(const Prob& P, const PfArgs& a, bool fwd, bool out_f32, hipStream_t s, Phases* ph);
// Bytes of the per-stripe partials (part_o, part_l).
size_t sel_part_o_bytes(const Prob& P);
size_t sel_part_l_bytes(const Prob& P);

}  // namespace nsa
