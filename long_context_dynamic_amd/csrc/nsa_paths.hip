// nsa_paths.hip -- workspace planning and dispatch: the matrix-core kernels
// for the shapes they take (bf16, 16 heads per group, 64-token blocks), the
// any-shape kernels otherwise.
#include "nsa_paths.h"

#include <functional>
#include "nsa_decode.h"
#include "nsa_frag.h"
#include "nsa_moba.h"
#include "nsa_prefill.h"

namespace nsa {
namespace {

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }
size_t elem_bytes(const Prob& P) { return P.bf16() ? 2 : 4; }
int64_t pad64(int64_t x) { return (x + 63) / 64 * 64; }
// a fragment-order image (nsa_frag.h): pad64(L) / 32 chunks per (b, g)
size_t frag_image_bytes(const Prob& P, int64_t D) {
  return (size_t)(P.B * P.G * (pad64(P.L) / 32) * frag_chunk((int)D)) * 2;
}

template <typename T> T* at(void* base, size_t off) { return (T*)((char*)base + off); }

DecArgs dec_args(const Prob& P) {
  DecArgs a = {};
  a.B = P.B; a.T = P.T; a.R = P.B * P.T; a.L = P.L; a.G = P.G; a.H = P.H; a.nb = P.nb;
  a.nbp = pad64(P.nb); a.n = P.n; a.w = P.w; a.flags = P.flags; a.scale = P.scale;
  a.bs = P.bs; a.per = P.sb / P.bs; a.nbs = P.nbs;
  return a;
}

PfArgs pf_args(const Prob& P) {
  PfArgs a = {};
  a.B = P.B; a.T = P.T; a.L = P.L; a.G = P.G; a.H = P.H; a.nb = P.nb;
  a.nbp = pad64(P.nb); a.Lp = pad64(P.L); a.n = P.n; a.w = P.w;
  a.bs = P.bs; a.per = P.sb / P.bs; a.nbs = P.nbs;
  a.flags = P.flags; a.scale = P.scale;
  return a;
}

MobaArgs moba_args(const Prob& P) {
  MobaArgs a = {};
  a.B = P.B; a.T = P.T; a.L = P.L; a.H = P.H; a.nb = P.nb;
  a.nbp = pad64(P.nb); a.Lp = pad64(P.L); a.bs = P.bs; a.n = P.n;
  a.flags = P.flags; a.scale = P.scale;
  return a;
}

// The MoBA attention stage: entry lists and partial records.
void take_moba(const Prob& P, Workspace& w, const std::function<size_t(size_t)>& take) {
  const size_t ne = (size_t)(P.B * P.T * P.H * P.n), nl = (size_t)(P.B * P.H * P.nb);
  w.counts = take(nl * sizeof(int32_t));
  w.pos = take(ne * sizeof(int32_t));
  w.offsets = take((nl + 1) * sizeof(int32_t));
  w.chunk_off = take((nl + 1) * sizeof(int32_t));
  w.lists = take(ne * sizeof(int32_t));
  w.part = take(ne * (size_t)(2 * P.dv + 16));  // compact partial records
}

void set_moba_ws(MobaArgs& a, const Workspace& ws, void* base) {
  a.counts = at<int32_t>(base, ws.counts);
  a.pos = at<int32_t>(base, ws.pos);
  a.offsets = at<int32_t>(base, ws.offsets);
  a.chunk_off = at<int32_t>(base, ws.chunk_off);
  a.lists = at<int32_t>(base, ws.lists);
  a.part = at<float>(base, ws.part);
}

}  // namespace

Workspace plan_workspace(const Prob& P, Call call, bool have_cmp) {
  Workspace w;
  size_t off = 0;
  std::function<size_t(size_t)> take = [&](size_t bytes) { size_t o = off; off += round_up(bytes); return o; };
  const bool fast = prefill_fast_ok(P);
  const bool dec = decode_ok(P);
  const size_t zbytes = (size_t)(P.B * P.T * P.G * 16 * pad64(P.nb)) * sizeof(float);
  if (call == Call::Select) {  // reads the caller's summaries directly
    if (dec) {
      w.zbuf = take(zbytes);
      w.part = take(decode_part_bytes(P));
    }
    w.total = off;
    return w;
  }
  if (call == Call::SparseAttn) {
    if (!dec && !fast && moba_attend_ok(P)) {
      take_moba(P, w, take);
    } else if (dec) {
      w.part = take(decode_part_bytes(P));
    } else if (fast) {
      w.kG = take(frag_image_bytes(P, P.dq));
      w.vT = take((size_t)(P.B * P.G * P.dv * pad64(P.L)) * 2);
      w.vF = take(frag_image_bytes(P, P.dv));
      w.qF = take((size_t)(P.B * P.T * P.H * P.dq) * 2);
      w.sel_o = take(sel_part_o_bytes(P));
      w.sel_l = take(sel_part_l_bytes(P));
    }
    w.total = off;
    return w;
  }
  const bool moba = !dec && !fast && moba_ok(P);
  if (!have_cmp) {
    w.kc = take((size_t)(P.B * P.nb * P.G * P.dq) * elem_bytes(P));
    if (!moba) w.vc = take((size_t)(P.B * P.nb * P.G * P.dv) * elem_bytes(P));  // MoBA scores by keys only
  }
  w.idx = take((size_t)(P.B * P.T * P.G * P.n) * sizeof(int32_t));
  if (moba) {
    take_moba(P, w, take);
  } else if (dec) {
    w.zbuf = take(zbytes);
    w.part = take(decode_part_bytes(P));
  } else if (fast) {
    w.kG = take(frag_image_bytes(P, P.dq));
    w.vT = take((size_t)(P.B * P.G * P.dv * pad64(P.L)) * 2);
    w.vF = take(frag_image_bytes(P, P.dv));
    w.qF = take((size_t)(P.B * P.T * P.H * P.dq) * 2);
    w.vcT = take((size_t)(P.B * P.G * P.dv * pad64(P.nb)) * 2);
    w.acc = take((size_t)(P.B * P.T * P.H * P.dv) * sizeof(float));
    w.sel_o = take(sel_part_o_bytes(P));
    w.sel_l = take(sel_part_l_bytes(P));
  } else if (P.has(NSA_F_CMP)) {
    w.ocmp = take((size_t)(P.B * P.T * P.H * P.dv) * sizeof(float));
  }
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

int forward_phase_names(const Prob& P, bool have_cmp, const char** names, int max_names) {
  const char* list[8];
  int n = 0;
  if (!have_cmp) list[n++] = "pool";
  if (decode_ok(P)) {
    list[n++] = "dec_step";
  } else if (moba_ok(P)) {
    list[n++] = "moba_select";
    list[n++] = "moba_lists";
    list[n++] = "moba_attn";
    list[n++] = "moba_own_block";
  } else if (prefill_fast_ok(P)) {
    list[n++] = "transpose_vc";
    list[n++] = "transpose_v";
    list[n++] = "fragment_v";
    list[n++] = "fragment_k";
    list[n++] = "cmp_select_window";
    list[n++] = "selected";
    list[n++] = "selected_merge";
  } else {
    list[n++] = "select_generic";
    list[n++] = "attend_generic";
  }
  for (int i = 0; i < n && i < max_names; ++i) names[i] = list[i];
  return n;
}

hipError_t run_select(const Prob& P, const void* q, const void* kc, int32_t* idx, float* score,
                      const Workspace& ws, void* base, hipStream_t s) {
  if (decode_ok(P)) {
    DecArgs a = dec_args(P);
    a.q = (const uint16_t*)q;
    a.kc = (const uint16_t*)kc;
    a.zbuf = at<float>(base, ws.zbuf);
    a.part = at<float>(base, ws.part);
    a.idx = idx;
    a.score = score;
    return launch_decode(P, a, 0, false, s, nullptr);
  }
  if (prefill_fast_ok(P)) {
    PfArgs a = pf_args(P);
    a.q = (const uint16_t*)q;
    a.kc = (const uint16_t*)kc;
    a.idx = idx;
    a.score = score;
    return launch_cmpwin(P, a, false, s);
  }
  if (moba_select_ok(P)) {
    MobaArgs a = moba_args(P);
    a.q = (const uint16_t*)q;
    a.kc = (const uint16_t*)kc;
    a.idx = idx;
    a.score = score;
    return launch_moba_select(P, a, s);
  }
  return launch_select_generic(P, q, kc, nullptr, idx, score, nullptr, s);
}

hipError_t run_sparse_attn(const Prob& P, const void* q, const void* k, const void* v, const int32_t* idx,
                           void* out, float* lse, const Workspace& ws, void* base, hipStream_t s) {
  Prob S = P;
  S.flags = NSA_F_SLC | (P.flags & NSA_F_OUT_F32);
  if (decode_ok(P)) {
    DecArgs a = dec_args(S);
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.idx = (int32_t*)idx;
    a.part = at<float>(base, ws.part);
    a.out = out;
    a.lse = lse;
    return launch_decode(S, a, 2, P.has(NSA_F_OUT_F32), s, nullptr);
  }
  if (prefill_fast_ok(P)) {
    PfArgs a = pf_args(S);
    uint16_t* vT = at<uint16_t>(base, ws.vT);
    uint16_t* vF = at<uint16_t>(base, ws.vF);
    uint16_t* kF = at<uint16_t>(base, ws.kG);
    hipError_t e = launch_transpose(v, vT, P.B, P.L, a.Lp, P.G, (int)P.dv, s);
    if (e != hipSuccess) return e;
    if ((e = launch_frag_v(vT, vF, P.B, P.L, P.G, (int)P.dv, s)) != hipSuccess) return e;
    if ((e = launch_frag_k(k, kF, P.B, P.L, P.G, (int)P.dq, s)) != hipSuccess) return e;
    a.qF = at<uint16_t>(base, ws.qF);
    if ((e = launch_frag_q(q, a.qF, P.B * P.T, P.G, (int)P.dq, s)) != hipSuccess) return e;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.kF = kF;
    a.vT = vT;
    a.vF = vF;
    a.idx = (int32_t*)idx;
    a.out = out;
    a.lse = lse;
    a.part_o = at<uint16_t>(base, ws.sel_o);
    a.part_l = at<float>(base, ws.sel_l);
    return launch_sel(P, a, false, P.has(NSA_F_OUT_F32), s, nullptr);
  }
  if (moba_attend_ok(P)) {
    MobaArgs a = moba_args(S);
    set_moba_ws(a, ws, base);
    a.v = (const uint16_t*)v;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.idx = (int32_t*)idx;
    a.out = out;
    a.lse = lse;
    return launch_moba_attend(P, a, P.has(NSA_F_OUT_F32), s, nullptr);
  }
  return launch_attend_generic(S, q, k, v, nullptr, idx, nullptr, out, lse, P.has(NSA_F_OUT_F32), s);
}

hipError_t run_forward(const Prob& P, const void* q, const void* k, const void* v, const void* gates,
                       const void* kc_given, const void* vc_given, void* out, int32_t* idx_out, void* saved,
                       const Workspace& ws, void* base, hipStream_t s, Phases& ph) {
  const void* kc = kc_given;
  const void* vc = vc_given;
  hipError_t e;
  ph.s = s;
  ph.mark();
  const bool moba = !decode_ok(P) && !prefill_fast_ok(P) && moba_ok(P);
  if (!kc) {
    kc = at<char>(base, ws.kc);
    vc = moba ? nullptr : at<char>(base, ws.vc);
    if ((e = launch_pool(P, k, v, (void*)kc, (void*)vc, s)) != hipSuccess) return e;
    ph.mark();
  }
  int32_t* idx = idx_out ? idx_out : at<int32_t>(base, ws.idx);
  if (saved && (decode_ok(P) || !prefill_fast_ok(P))) return hipErrorInvalidValue;
  if (decode_ok(P)) {
    DecArgs a = dec_args(P);
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.kc = (const uint16_t*)kc;
    a.vc = (const uint16_t*)vc;
    a.gates = (const uint16_t*)gates;
    a.zbuf = at<float>(base, ws.zbuf);
    a.idx = idx;
    a.part = at<float>(base, ws.part);
    a.out = out;
    if ((e = launch_decode(P, a, 1, P.has(NSA_F_OUT_F32), s, &ph)) != hipSuccess) return e;
    return ph.err;
  }
  if (prefill_fast_ok(P)) {
    PfArgs a = pf_args(P);
    uint16_t* vT = at<uint16_t>(base, ws.vT);
    uint16_t* vcT = at<uint16_t>(base, ws.vcT);
    if ((e = launch_transpose(vc, vcT, P.B, P.nb, a.nbp, P.G, (int)P.dv, s)) != hipSuccess) return e;
    ph.mark();
    if ((e = launch_transpose(v, vT, P.B, P.L, a.Lp, P.G, (int)P.dv, s)) != hipSuccess) return e;
    ph.mark();
    uint16_t* vF = at<uint16_t>(base, ws.vF);
    if ((e = launch_frag_v(vT, vF, P.B, P.L, P.G, (int)P.dv, s)) != hipSuccess) return e;
    ph.mark();
    uint16_t* kF = at<uint16_t>(base, ws.kG);
    if ((e = launch_frag_k(k, kF, P.B, P.L, P.G, (int)P.dq, s)) != hipSuccess) return e;
    ph.mark();
    a.q = (const uint16_t*)q;
    a.qF = at<uint16_t>(base, ws.qF);  // written by the compressed/window kernel
    a.k = (const uint16_t*)k;
    a.kF = kF;
    a.vT = vT;
    a.vF = vF;
    a.kc = (const uint16_t*)kc;
    a.vcT = vcT;
    a.gates = (const uint16_t*)gates;
    a.acc = at<float>(base, ws.acc);
    a.part_o = at<uint16_t>(base, ws.sel_o);
    a.part_l = at<float>(base, ws.sel_l);
    a.idx = idx;
    a.out = out;
    if (saved) {
      a.sv_lse = (float*)saved;
      a.sv_o = (uint16_t*)((char*)saved + saved_lse_bytes(P));
    }
    if ((e = launch_cmpwin(P, a, true, s)) != hipSuccess) return e;
    ph.mark();
    if ((e = launch_sel(P, a, true, P.has(NSA_F_OUT_F32), s, &ph)) != hipSuccess) return e;
    ph.mark();
    return ph.err;
  }
  if (moba) {
    MobaArgs a = moba_args(P);
    set_moba_ws(a, ws, base);
    a.v = (const uint16_t*)v;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.kc = (const uint16_t*)kc;
    a.gates = (const uint16_t*)gates;
    a.idx = idx;
    a.out = out;
    if ((e = launch_moba_select(P, a, s)) != hipSuccess) return e;
    ph.mark();
    if ((e = launch_moba_attend(P, a, P.has(NSA_F_OUT_F32), s, &ph)) != hipSuccess) return e;
    return ph.err;
  }
  float* ocmp = P.has(NSA_F_CMP) ? at<float>(base, ws.ocmp) : nullptr;
  if ((e = launch_select_generic(P, q, kc, vc, idx, nullptr, ocmp, s)) != hipSuccess) return e;
  ph.mark();
  if ((e = launch_attend_generic(P, q, k, v, gates, idx, ocmp, out, nullptr, P.has(NSA_F_OUT_F32), s)) != hipSuccess)
    return e;
  ph.mark();
  return ph.err;
}

}  // namespace nsa
