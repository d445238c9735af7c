// nsa_api.hip -- the C ABI declared in include/nsa.h: argument validation
// (before anything is queued), workspace planning and kernel dispatch.
#include <math.h>
#include <string.h>

#include <mutex>

#include "nsa_backward.h"
#include "nsa_decode.h"
#include "nsa_internal.h"
#include "nsa_learned.h"
#include "nsa_paths.h"
#include "nsa_prefill.h"

using nsa::Prob;

namespace {

constexpr uint32_t kAllFlags = NSA_F_FORCE_FIRST | NSA_F_FORCE_CURRENT | NSA_F_CMP | NSA_F_SLC |
                               NSA_F_WIN | NSA_F_GATE_LOGITS | NSA_F_OUT_F32;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }
bool opt_ok(const void* p) { return p == nullptr || aligned16(p); }
// an array of n elements: may be NULL when empty (no complete block: no summaries)
bool arr_ok(const void* p, int64_t n) { return n == 0 ? opt_ok(p) : ptr_ok(p); }

nsa_status describe(const nsa_params* p, Prob* P) {
  if (!p) return NSA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->q_len < 1 || p->kv_len < p->q_len || p->n_kv_groups < 1 ||
      p->heads_per_group < 1 || p->d_qk < 1 || p->d_v < 1 || p->block < 1 || p->top_k < 0 ||
      p->window < 0 || (p->flags & ~kAllFlags) || (p->dtype != NSA_BF16 && p->dtype != NSA_F32) ||
      !(p->scale >= 0.f) || isinf(p->scale))
    return NSA_ERR_INVALID_ARG;
  const int n_forced = ((p->flags & NSA_F_FORCE_FIRST) ? 1 : 0) + ((p->flags & NSA_F_FORCE_CURRENT) ? 1 : 0);
  if (p->top_k < n_forced) return NSA_ERR_INVALID_ARG;
  const int64_t nb = (int64_t)p->kv_len / p->block;
  const int64_t sb = p->sel_block > 0 ? p->sel_block : p->block;
  if (p->sel_block < 0 || sb % p->block != 0) return NSA_ERR_INVALID_ARG;
  if (p->heads_per_group > 16 || p->d_qk > 256 || p->d_v > 256 || p->block > 4096 || sb > 4096 ||
      p->top_k > 64 || (int64_t)p->top_k * sb > 16384 || p->window > 16384 || nb > 16384)
    return NSA_ERR_UNSUPPORTED;
  P->B = p->batch; P->T = p->q_len; P->L = p->kv_len;
  P->G = p->n_kv_groups; P->hpg = p->heads_per_group; P->H = P->G * P->hpg;
  P->dq = p->d_qk; P->dv = p->d_v; P->bs = p->block; P->n = p->top_k; P->w = p->window; P->nb = nb;
  P->sb = sb; P->nbs = (int64_t)p->kv_len / sb;
  P->flags = p->flags; P->dtype = p->dtype;
  P->scale = p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)p->d_qk));
  // element counts must fit the grid: one workgroup per (b, t, g) and per (b, j, g)
  // (B*T and B*nb fit int64 whatever the int32 fields hold; the products
  // with G are compared by division so that nothing overflows)
  const int64_t lim = (((int64_t)1 << 31) - 1) / P->G;
  if (P->B * P->T > lim || P->B * P->nb > lim) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

int n_branches(uint32_t f) {
  return ((f & NSA_F_CMP) ? 1 : 0) + ((f & NSA_F_SLC) ? 1 : 0) + ((f & NSA_F_WIN) ? 1 : 0);
}

nsa_status hip_status(hipError_t e) { return e == hipSuccess ? NSA_OK : NSA_ERR_HIP; }

}  // namespace

extern "C" {

const char* nsa_status_str(int s) {
  switch (s) {
    case NSA_OK: return "ok";
    case NSA_ERR_INVALID_ARG: return "invalid argument";
    case NSA_ERR_UNSUPPORTED: return "unsupported problem shape";
    case NSA_ERR_WORKSPACE: return "workspace missing or too small";
    case NSA_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

size_t nsa_workspace_bytes(const nsa_params* p) {
  Prob P;
  if (describe(p, &P) != NSA_OK) return 0;
  return nsa::workspace_bytes_max(P, p->k_cmp != nullptr && p->v_cmp != nullptr);
}

nsa_status nsa_compress(const void* k, const void* v, void* k_cmp, void* v_cmp, const nsa_params* p) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  const int64_t ns = P.B * P.nb * P.G;
  if (!ptr_ok(k) || !ptr_ok(v) || !arr_ok(k_cmp, ns) || !arr_ok(v_cmp, ns)) return NSA_ERR_INVALID_ARG;
  return hip_status(nsa::launch_pool(P, k, v, k_cmp, v_cmp, (hipStream_t)p->stream));
}

nsa_status nsa_compress_mlp(const void* k, const void* v, const nsa_mlp_weights* w, void* k_cmp, void* v_cmp,
                            const nsa_params* p) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  const int64_t ns = P.B * P.nb * P.G;
  if (!w || !ptr_ok(k) || !ptr_ok(v) || !arr_ok(k_cmp, ns) || !arr_ok(v_cmp, ns) || !ptr_ok(w->k_w1) || !ptr_ok(w->k_w2) ||
      !ptr_ok(w->v_w1) || !ptr_ok(w->v_w2) || !opt_ok(w->k_b1) || !opt_ok(w->k_b2) || !opt_ok(w->v_b1) ||
      !opt_ok(w->v_b2) || w->d_hidden < 1)
    return NSA_ERR_INVALID_ARG;
  if (!nsa::mlp_ok(P, w->d_hidden)) return NSA_ERR_UNSUPPORTED;
  nsa::MlpArgs a;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.k_w1 = (const uint16_t*)w->k_w1;
  a.k_b1 = (const uint16_t*)w->k_b1;
  a.k_w2 = (const uint16_t*)w->k_w2;
  a.k_b2 = (const uint16_t*)w->k_b2;
  a.v_w1 = (const uint16_t*)w->v_w1;
  a.v_b1 = (const uint16_t*)w->v_b1;
  a.v_w2 = (const uint16_t*)w->v_w2;
  a.v_b2 = (const uint16_t*)w->v_b2;
  a.kc = (uint16_t*)k_cmp;
  a.vc = (uint16_t*)v_cmp;
  a.B = P.B; a.L = P.L; a.G = P.G; a.nb = P.nb; a.bs = P.bs; a.dh = w->d_hidden;
  return hip_status(nsa::launch_mlp_compress(P, a, (hipStream_t)p->stream));
}

nsa_status nsa_gate_proj(const void* x, int32_t d_model, const void* w, const void* bias, void* gates,
                         const nsa_params* p) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  if (!ptr_ok(x) || !ptr_ok(w) || !opt_ok(bias) || !ptr_ok(gates) || d_model < 1) return NSA_ERR_INVALID_ARG;
  if (!nsa::gate_proj_ok(P, d_model)) return NSA_ERR_UNSUPPORTED;
  nsa::GateArgs a;
  a.x = (const uint16_t*)x;
  a.w = (const uint16_t*)w;
  a.bias = (const uint16_t*)bias;
  a.gates = (uint16_t*)gates;
  a.M = P.B * P.T;
  a.DM = d_model;
  a.N = 3 * P.H;
  a.logits = P.has(NSA_F_GATE_LOGITS) ? 1 : 0;
  return hip_status(nsa::launch_gate_proj(a, (hipStream_t)p->stream));
}

nsa_status nsa_select_topk(const void* q, const void* k_cmp, int32_t* idx, float* score, const nsa_params* p) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  if (!ptr_ok(q) || !arr_ok(k_cmp, P.B * P.nb * P.G) || !ptr_ok(idx) || !opt_ok(score)) return NSA_ERR_INVALID_ARG;
  const nsa::Workspace ws = nsa::plan_workspace(P, nsa::Call::Select, true);
  if (ws.total > 0 && (!ptr_ok(p->workspace) || p->workspace_bytes < ws.total)) return NSA_ERR_WORKSPACE;
  return hip_status(nsa::run_select(P, q, k_cmp, idx, score, ws, p->workspace, (hipStream_t)p->stream));
}

nsa_status nsa_sparse_attn(const void* q, const void* k, const void* v, const int32_t* idx, void* out,
                           float* lse, const nsa_params* p) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(idx) || !ptr_ok(out) || !opt_ok(lse))
    return NSA_ERR_INVALID_ARG;
  const nsa::Workspace ws = nsa::plan_workspace(P, nsa::Call::SparseAttn, true);
  if (ws.total > 0 && (!ptr_ok(p->workspace) || p->workspace_bytes < ws.total)) return NSA_ERR_WORKSPACE;
  return hip_status(nsa::run_sparse_attn(P, q, k, v, idx, out, lse, ws, p->workspace, (hipStream_t)p->stream));
}

}  // extern "C"

namespace {

// Everything nsa_forward and nsa_forward_noalloc check before anything is
// queued, except the workspace itself.
nsa_status forward_checks(const void* q, const void* k, const void* v, const void* gates, const nsa_params* p,
                          const void* out, Prob* P) {
  nsa_status st = describe(p, P);
  if (st != NSA_OK) return st;
  const int nbr = n_branches(P->flags);
  if (nbr == 0 || (gates == nullptr && nbr > 1)) return NSA_ERR_INVALID_ARG;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out) || !opt_ok(gates)) return NSA_ERR_INVALID_ARG;
  if ((p->k_cmp == nullptr) != (p->v_cmp == nullptr) || !opt_ok(p->k_cmp) || !opt_ok(p->v_cmp))
    return NSA_ERR_INVALID_ARG;
  if (p->n_phase_events < 0 || (p->n_phase_events > 0 && !p->phase_events)) return NSA_ERR_INVALID_ARG;
  return NSA_OK;
}

nsa_status forward_on(const void* q, const void* k, const void* v, const void* gates, const nsa_params* p,
                      void* out, const Prob& P, const nsa::Workspace& ws, void* base) {
  const bool have_cmp = p->k_cmp != nullptr;
  nsa::Phases ph;
  ph.ev = p->phase_events;
  ph.n = p->phase_events ? p->n_phase_events : 0;
  return hip_status(nsa::run_forward(P, q, k, v, gates, have_cmp ? p->k_cmp : nullptr,
                                     have_cmp ? p->v_cmp : nullptr, out, nullptr, nullptr, ws, base,
                                     (hipStream_t)p->stream, ph));
}

// ---- the allocation-free forward's scratch ---------------------------------
// One fixed array per device, the workspace of every nsa_forward_noalloc call
// on that device.  Its name is only a host-side handle: the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device (with
// that device current) on the first call there, and only that address is
// ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[NSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of scratch on each device, once looked up

// The current device's scratch address, or NULL when it cannot be had.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

nsa_status nsa_forward(const void* q, const void* k, const void* v, const void* gates, const nsa_params* p,
                       void* out) {
  Prob P;
  nsa_status st = forward_checks(q, k, v, gates, p, out, &P);
  if (st != NSA_OK) return st;
  const nsa::Workspace ws = nsa::plan_workspace(P, nsa::Call::Forward, p->k_cmp != nullptr);
  if (ws.total > 0 && (!ptr_ok(p->workspace) || p->workspace_bytes < ws.total)) return NSA_ERR_WORKSPACE;
  return forward_on(q, k, v, gates, p, out, P, ws, p->workspace);
}

nsa_status nsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gates,
                               const nsa_params* p, void* out) {
  Prob P;
  nsa_status st = forward_checks(q, k, v, gates, p, out, &P);
  if (st != NSA_OK) return st;
  const nsa::Workspace ws = nsa::plan_workspace(P, nsa::Call::Forward, p->k_cmp != nullptr);
  if (ws.total > NSA_NOALLOC_SCRATCH_BYTES) return NSA_ERR_WORKSPACE;
  void* base = device_scratch();
  if (!base) return NSA_ERR_HIP;
  return forward_on(q, k, v, gates, p, out, P, ws, base);
}

// A training forward runs the matrix-core prefill path (its kernels write the
// statistics) with mean-pooled summaries (what the backward recomputes).
static bool train_ok(const Prob& P) { return nsa::backward_ok(P) && nsa::prefill_fast_ok(P) && !nsa::decode_ok(P); }

size_t nsa_train_saved_bytes(const nsa_params* p) {
  Prob P;
  if (describe(p, &P) != NSA_OK || !train_ok(P)) return 0;
  return nsa::saved_bytes(P);
}

nsa_status nsa_forward_train(const void* q, const void* k, const void* v, const void* gates, const nsa_params* p,
                             void* out, int32_t* idx, void* saved) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  const int nbr = n_branches(P.flags);
  if (nbr == 0 || (gates == nullptr && nbr > 1)) return NSA_ERR_INVALID_ARG;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(out) || !opt_ok(gates) || !ptr_ok(idx) || !ptr_ok(saved))
    return NSA_ERR_INVALID_ARG;
  if (p->k_cmp != nullptr || p->v_cmp != nullptr || !train_ok(P)) return NSA_ERR_UNSUPPORTED;
  const nsa::Workspace ws = nsa::plan_workspace(P, nsa::Call::Forward, false);
  if (ws.total > 0 && (!ptr_ok(p->workspace) || p->workspace_bytes < ws.total)) return NSA_ERR_WORKSPACE;
  if (p->n_phase_events < 0 || (p->n_phase_events > 0 && !p->phase_events)) return NSA_ERR_INVALID_ARG;
  nsa::Phases ph;
  ph.ev = p->phase_events;
  ph.n = p->phase_events ? p->n_phase_events : 0;
  return hip_status(nsa::run_forward(P, q, k, v, gates, nullptr, nullptr, out, idx, saved, ws, p->workspace,
                                     (hipStream_t)p->stream, ph));
}

size_t nsa_backward_workspace_bytes(const nsa_params* p) {
  Prob P;
  if (describe(p, &P) != NSA_OK) return 0;
  return nsa::backward_workspace_bytes(P);
}

nsa_status nsa_backward(const void* q, const void* k, const void* v, const void* gates, const int32_t* idx,
                        const void* dout, const void* saved, float* dq, float* dk, float* dv, float* dgates,
                        const nsa_params* p) {
  Prob P;
  nsa_status st = describe(p, &P);
  if (st != NSA_OK) return st;
  const int nbr = n_branches(P.flags);
  if (nbr == 0 || (gates == nullptr && nbr > 1) || (gates == nullptr && dgates != nullptr)) return NSA_ERR_INVALID_ARG;
  if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(idx) || !ptr_ok(dout) || !ptr_ok(dq) || !ptr_ok(dk) ||
      !ptr_ok(dv) || !opt_ok(gates) || !opt_ok(dgates) || !opt_ok(saved))
    return NSA_ERR_INVALID_ARG;
  if (!nsa::backward_ok(P) || (saved && !train_ok(P))) return NSA_ERR_UNSUPPORTED;
  const size_t need = nsa::backward_workspace_bytes(P);
  if (!ptr_ok(p->workspace) || p->workspace_bytes < need) return NSA_ERR_WORKSPACE;
  if (p->n_phase_events < 0 || (p->n_phase_events > 0 && !p->phase_events)) return NSA_ERR_INVALID_ARG;
  nsa::Phases ph;
  ph.ev = p->phase_events;
  ph.n = p->phase_events ? p->n_phase_events : 0;
  ph.s = (hipStream_t)p->stream;
  return hip_status(nsa::run_backward(P, q, k, v, gates, idx, dout, saved, dq, dk, dv, dgates, p->workspace,
                                      (hipStream_t)p->stream, ph));
}

int32_t nsa_backward_phases(const nsa_params* p, const char** names, int32_t max_names) {
  Prob P;
  if (describe(p, &P) != NSA_OK || !nsa::backward_ok(P)) return 0;
  return nsa::backward_phase_names(P, names, names ? max_names : 0);
}

int32_t nsa_forward_phases(const nsa_params* p, const char** names, int32_t max_names) {
  Prob P;
  if (describe(p, &P) != NSA_OK) return 0;
  const bool have_cmp = p->k_cmp != nullptr && p->v_cmp != nullptr;
  return nsa::forward_phase_names(P, have_cmp, names, names ? max_names : 0);
}

}  // extern "C"
