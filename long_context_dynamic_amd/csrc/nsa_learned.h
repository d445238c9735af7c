// nsa_learned.h -- arguments and launchers of the learned block compression
// and the gate projection (internal).
#pragma once

#include "nsa_internal.h"

namespace nsa {

struct MlpArgs {
  const uint16_t* k;  // [B, L, G, dq]
  const uint16_t* v;  // [B, L, G, dv]
  const uint16_t *k_w1, *k_b1, *k_w2, *k_b2;  // [dh, bs*dq], [dh] or NULL, [dq, dh], [dq] or NULL
  const uint16_t *v_w1, *v_b1, *v_w2, *v_b2;  // the same with dv
  uint16_t* kc;       // [B, nb, G, dq]
  uint16_t* vc;       // [B, nb, G, dv]
  int64_t B, L, G, nb, bs, dh;
};

struct GateArgs {
  const uint16_t* x;     // [M, DM] hidden states
  const uint16_t* w;     // [N, DM] (N = 3H)
  const uint16_t* bias;  // [N] or NULL
  uint16_t* gates;       // [M, N]
  int64_t M, DM, N;
  int logits;            // 1: leave the sigmoid to the attention
};

// bf16; d_qk, d_v and the hidden width in {64, 128, 192, 256}; block a multiple of 4.
bool mlp_ok(const Prob& P, int64_t dh);
// bf16; d_model a multiple of 32.
bool gate_proj_ok(const Prob& P, int64_t dm);
hipError_t launch_mlp_compress(const Prob& P, const MlpArgs& a, hipStream_t s);
hipError_t launch_gate_proj(const GateArgs& a, hipStream_t s);

}  // namespace nsa
