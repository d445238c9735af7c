// nsa_decode.h -- arguments and launcher of the decoding kernels (internal).
#pragma once

#include "nsa_internal.h"
#include "nsa_paths.h"

namespace nsa {

struct DecArgs {
  const uint16_t* q;      // [B, T, H, DQ]
  const uint16_t* k;      // [B, L, G, DQ]
  const uint16_t* v;      // [B, L, G, DV]
  const uint16_t* kc;     // [B, nb, G, DQ]
  const uint16_t* vc;     // [B, nb, G, DV]
  const uint16_t* gates;  // [B, T, H, 3] or NULL
  float* zbuf;            // [R, G, 16, nbp]  scaled logits (log2 units)
  int32_t* idx;           // [R, G, n]
  float* score;           // [R, G, n] or NULL
  float* part;            // [R, G, cmp + sel + win waves, 16 * DV + 32] partial records
  void* out;              // [R, H, DV]
  float* lse;             // [R, H] selected-branch log-sum-exp, or NULL
  int64_t B, T, R, L, G, H, nb, nbp, n, w, n_cmp_waves, n_sel_waves, n_win_waves;
  int64_t bs, per, nbs;  // summary block, summaries per 64-token selection block, selection blocks
  uint32_t flags;
  float scale;
};

// True for the decoding shapes: the matrix-core shapes with q_len <= 8.
bool decode_ok(const Prob& P);
void decode_layout(const Prob& P, int64_t* n_cmp_waves, int64_t* n_sel_waves, int64_t* n_win_waves);
size_t decode_part_bytes(const Prob& P);
// mode 0: selection only (idx, score); 1: the whole forward; 2: the selected
// branch alone on the caller's idx (out, lse).
hipError_t launch_decode(const Prob& P, DecArgs a, int mode, bool out_f32, hipStream_t s, Phases* ph);

}  // namespace nsa
