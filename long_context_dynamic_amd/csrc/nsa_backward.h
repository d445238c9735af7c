// nsa_backward.h -- arguments, workspace plan and entry of the matrix-core
// NSA backward pass (internal).
#pragma once

#include "nsa_internal.h"
#include "nsa_paths.h"

namespace nsa {

struct BwArgs {
  const uint16_t* q;      // [B, T, H, DQ]
  const uint16_t* k;      // [B, L, G, DQ]
  const uint16_t* v;      // [B, L, G, DV]
  const uint16_t* gates;  // [B, T, H, 3] or NULL
  const int32_t* idx;     // [B, T, G, n] selection blocks of 64 tokens
  const uint16_t* dout;   // [B, T, H, DV]
  const uint16_t* kc;     // [B, nb, G, DQ] block summaries
  const uint16_t* vc;     // [B, nb, G, DV]
  const uint16_t* kG;     // fragment-order images [B, G, Lp / 32, D / 32, 2, 64, 8] of k, v (nsa_frag.h)
  const uint16_t* vG;
  const uint16_t* vT;     // tiled transpose [B, G, Lp / 32, DV, 32] of v
  const uint16_t* kcG;    // the same three images of the summaries (nbp rows)
  const uint16_t* vcG;
  const uint16_t* vcT;
  const float* sv_lse;    // training forward's statistics or NULL: [3][B*T*H] natural log-sum-exp,
  const uint16_t* sv_o;   //   [3][B*T*H][DV] normalised branch outputs (bf16)
  float* stat;            // [3 branches][3: lse (log2 units), <dout, O_b>, gate][B*T*H]
  int32_t* cnt;           // [B, G, nct, nbk] entries per (256-token chunk, block)
  int32_t* tot;           // [B*G*nbk + 1] entries per list
  int32_t* offsets;       // [B*G*nbk + 1] list starts
  int32_t* chunk_off;     // [B*G*nbk + 1] first work chunk of each list
  int32_t* lists;         // entries ((b * T + t) * G + g) * n + slot, grouped by (b, g, block), in token order
  float* srec;            // [entries][16 heads][4]: selected block's max (log2 units), sum, sum p.dP, 0
  float* part_s;          // [chunks][64][DQ + DV] selected-branch key gradients
  float* part_c;          // [B, G, nJ, nC][64][DQ + DV] compressed-branch summary gradients
  float* dkc;             // [B, G, nb][DQ + DV] summary gradients / 64
  float* dq;              // [B, T, H, DQ]
  float* dk;              // [B, L, G, DQ]
  float* dv;              // [B, L, G, DV]
  float* dgates;          // [B, T, H, 3] or NULL
  int64_t B, T, L, G, H, nb, nbp, Lp, n, w;
  int64_t nbk;            // 64-token blocks, the last one possibly partial
  int64_t nct;            // 256-token chunks of the list count
  int64_t nJ, nC;         // 64-summary tiles, token chunks of the compressed branch
  uint32_t flags;
  float scale;
};

// True when the backward kernels take this shape: bf16, 16 heads per group,
// 64-token blocks (compression = selection), d_qk in {64,128,192},
// d_v in {64,128}, top_k <= 32.
bool backward_ok(const Prob& P);
size_t backward_workspace_bytes(const Prob& P);
// Names of the kernel groups run_backward times (one event after each), in order.
int backward_phase_names(const Prob& P, const char** names, int max_names);
hipError_t run_backward(const Prob& P, const void* q, const void* k, const void* v, const void* gates,
                        const int32_t* idx, const void* dout, const void* saved, float* dq, float* dk, float* dv,
                        float* dgates, void* ws, hipStream_t s, Phases& ph);

}  // namespace nsa
