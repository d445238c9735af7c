// nsa_moba.h -- arguments and launchers of the matrix-core MoBA kernels
// (internal): one head per KV group, every head its own top-k.
#pragma once

#include "nsa_internal.h"
#include "nsa_paths.h"

namespace nsa {

struct MobaArgs {
  const uint16_t* q;      // [B, T, H, D]
  const uint16_t* k;      // [B, L, H, D]
  const uint16_t* v;      // [B, L, H, D]
  const uint16_t* kc;     // [B, nb, H, D]  mean keys of the blocks
  const uint16_t* gates;  // [B, T, H, 3] or NULL (slot 1 scales the output)
  int32_t* idx;           // [B, T, H, n]
  float* score;           // [B, T, H, n] or NULL
  int32_t* counts;        // [B, H, nb]  entries listed per (b, h, block)
  int32_t* pos;           // [B, T, H, n] place of each entry in its list, -1 if unlisted
  int32_t* offsets;       // [B*H*nb + 1] list starts
  int32_t* chunk_off;     // [B*H*nb + 1] first 64-entry chunk of each list
  int32_t* lists;         // [B*T*H*n] entry ids, grouped by list
  float* part;            // [B, T, H, n] records of 2 D + 16 bytes: fp16 scaled o / l, max, sum, exponent
  void* out;              // [B, T, H, D]
  float* lse;             // [B, T, H] or NULL
  int64_t B, T, L, H, nb, nbp, Lp, bs, n;
  uint32_t flags;
  float scale;
};

// Shapes the MoBA kernels take: bf16, one head per group; selection:
// d_qk in {64, 128}, nb >= 1, 1 <= top_k <= 8; attention: d_qk = d_v,
// blocks a multiple of 64 long, top_k <= 8; the forward pass: both, and the
// selected branch alone.
bool moba_select_ok(const Prob& P);
bool moba_attend_ok(const Prob& P);
bool moba_ok(const Prob& P);

// Block scores and per-head top-k (idx, optional scores).
hipError_t launch_moba_select(const Prob& P, const MobaArgs& a, hipStream_t s);
// Entry lists, attention over the listed blocks, the own block and the
// merge; ph (optional) marks the end of each stage.
hipError_t launch_moba_attend(const Prob& P, const MobaArgs& a, bool out_f32, hipStream_t s, Phases* ph);

}  // namespace nsa
