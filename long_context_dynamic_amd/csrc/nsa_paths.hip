// nsa_paths.hip -- workspace planning and dispatch of the forward pass.
#include "nsa_paths.h"

namespace nsa {
namespace {

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }
size_t elem_bytes(const Prob& P) { return P.bf16() ? 2 : 4; }

template <typename T> T* at(void* base, size_t off) { return (T*)((char*)base + off); }

}  // namespace

Workspace plan_workspace(const Prob& P, Call call, bool have_cmp) {
  Workspace w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes); return o; };
  if (call != Call::Forward) return w;  // the any-shape select/attend kernels need none
  if (!have_cmp) {
    w.kc = take((size_t)(P.B * P.nb * P.G * P.dq) * elem_bytes(P));
    w.vc = take((size_t)(P.B * P.nb * P.G * P.dv) * elem_bytes(P));
  }
  w.idx = take((size_t)(P.B * P.T * P.G * P.n) * sizeof(int32_t));
  if (P.has(NSA_F_CMP)) w.ocmp = take((size_t)(P.B * P.T * P.H * P.dv) * sizeof(float));
  w.total = off;
  return w;
}

size_t workspace_bytes_max(const Prob& P, bool have_cmp) {
  size_t m = 0;
  for (Call c : {Call::Select, Call::SparseAttn, Call::Forward}) {
    const size_t t = plan_workspace(P, c, have_cmp).total;
    if (t > m) m = t;
  }
  return m;
}

hipError_t run_select(const Prob& P, const void* q, const void* kc, int32_t* idx, float* score,
                      const Workspace&, void*, hipStream_t s) {
  return launch_select_generic(P, q, kc, nullptr, idx, score, nullptr, s);
}

hipError_t run_sparse_attn(const Prob& P, const void* q, const void* k, const void* v, const int32_t* idx,
                           void* out, float* lse, const Workspace&, void*, hipStream_t s) {
  Prob S = P;
  S.flags = NSA_F_SLC | (P.flags & NSA_F_OUT_F32);
  return launch_attend_generic(S, q, k, v, nullptr, idx, nullptr, out, lse, P.has(NSA_F_OUT_F32), s);
}

hipError_t run_forward(const Prob& P, const void* q, const void* k, const void* v, const void* gates,
                       const void* kc_given, const void* vc_given, void* out, const Workspace& ws,
                       void* base, hipStream_t s) {
  const void* kc = kc_given;
  const void* vc = vc_given;
  hipError_t e;
  if (!kc) {
    kc = at<char>(base, ws.kc);
    vc = at<char>(base, ws.vc);
    if ((e = launch_pool(P, k, v, (void*)kc, (void*)vc, s)) != hipSuccess) return e;
  }
  int32_t* idx = at<int32_t>(base, ws.idx);
  float* ocmp = P.has(NSA_F_CMP) ? at<float>(base, ws.ocmp) : nullptr;
  if ((e = launch_select_generic(P, q, kc, vc, idx, nullptr, ocmp, s)) != hipSuccess) return e;
  return launch_attend_generic(P, q, k, v, gates, idx, ocmp, out, nullptr, P.has(NSA_F_OUT_F32), s);
}

}  // namespace nsa
