// nsa_paths.h -- workspace planning and the choice between the any-shape
// path and the matrix-core paths (internal).
#pragma once

#include "nsa_internal.h"

namespace nsa {

// Byte offsets into the caller's workspace (each 256-byte aligned); a field
// is meaningful only when the chosen path uses it.
struct Workspace {
  size_t total = 0;
  size_t kc = 0, vc = 0;  // block summaries, when the caller gives none
  size_t idx = 0;         // int32 [B, T, G, top_k]
  size_t ocmp = 0;        // fp32 [B, T, H, d_v] compressed-branch output
  size_t kG = 0;          // keys per group, fragment-order image [B, G, round_up(L, 64), d_qk]
  size_t vF = 0;          // values per group, fragment-order image [B, G, round_up(L, 64), d_v]
  size_t qF = 0;          // queries, fragment-order image [B, T, G, d_qk / 32, 64, 8]
  size_t vT = 0;          // values, tiled [B, G, round_up(L, 64) / 32, d_v, 32]
  size_t vcT = 0;         // value summaries, tiled [B, G, round_up(nb, 64) / 32, d_v, 32]
  size_t acc = 0;         // fp32 [B, T, H, d_v] gated compressed + window sum
  size_t sel_o = 0;       // bf16 [B, T, G, 8, 16, d_v] selected branch per XCD stripe
  size_t sel_l = 0;       // fp32 [B, T, G, 16, 8]      its log-sum-exps
  size_t zbuf = 0;        // decoding: fp32 [B*T, G, 16, round_up(nb, 64)] logits
  size_t part = 0;        // decoding, MoBA: partial attention records
  size_t counts = 0;      // MoBA: int32 [B, H, nb] entries per (b, h, block)
  size_t pos = 0;         // MoBA: int32 [B, T, H, top_k] place of an entry in its list
  size_t offsets = 0;     // MoBA: int32 [B*H*nb + 1] list starts
  size_t chunk_off = 0;   // MoBA: int32 [B*H*nb + 1] first 64-entry chunk per list
  size_t lists = 0;       // MoBA: int32 [B*T*H*top_k] entries grouped by list
};

// Records an event before the first and after every launch (timing hook).
struct Phases {
  void* const* ev = nullptr;
  int n = 0, i = 0;
  hipStream_t s = nullptr;
  hipError_t err = hipSuccess;
  void mark() {
    if (ev && i < n && err == hipSuccess) err = hipEventRecord((hipEvent_t)ev[i], s);
    ++i;
  }
};

// Names of the kernels run_forward launches, in order; returns the count.
int forward_phase_names(const Prob& P, bool have_cmp, const char** names, int max_names);

enum class Call { Select, SparseAttn, Forward };

Workspace plan_workspace(const Prob& P, Call call, bool have_cmp);
// The largest need over every call (what nsa_workspace_bytes reports).
size_t workspace_bytes_max(const Prob& P, bool have_cmp);

hipError_t run_select(const Prob& P, const void* q, const void* kc, int32_t* idx, float* score,
                      const Workspace& ws, void* base, hipStream_t s);
hipError_t run_sparse_attn(const Prob& P, const void* q, const void* k, const void* v, const int32_t* idx,
                           void* out, float* lse, const Workspace& ws, void* base, hipStream_t s);
// idx_out (or NULL: the workspace) receives the selection; saved (or NULL)
// the training statistics, on the matrix-core prefill path only.
hipError_t run_forward(const Prob& P, const void* q, const void* k, const void* v, const void* gates,
                       const void* kc_given, const void* vc_given, void* out, int32_t* idx_out, void* saved,
                       const Workspace& ws, void* base, hipStream_t s, Phases& ph);

}  // namespace nsa
