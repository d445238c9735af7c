// k_generic.hip -- any-shape path of the NSA forward: plain VALU kernels with
// fp32 arithmetic, one workgroup per (token, KV group).  It takes every
// shape the ABI accepts that no matrix-core path takes (fp32 mode, few heads
// per group, odd head dims, small blocks).  Sources: [P1] s4 (three
// branches, group-summed selection, gating), [P1] s7 and [P5] s13 (MoBA).
#include <math.h>

#include "nsa_internal.h"

namespace nsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxTopK = 64;

struct GArgs {
  int64_t B, T, L, G, hpg, H, dq, dv, bs, n, w, nb;
  int64_t sb, nbs;  // selection block, selection-block count
  float scale;
  uint32_t flags;
};

__device__ float block_max(float x, float* red) {
  x = wave_max(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
  return r;
}

__device__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += red[i];
  return r;
}

// (value, block) ordering of the selection: higher value first, then lower id.
__device__ __forceinline__ bool better(float v, int j, float bv, int bj) {
  return v > bv || (v == bv && j < bj);
}

// ---------------------------------------------------------------------------
// Compressed branch + importance + top-k for one (b, t, g).
// LDS: q row [dq] | P [nb] | I [nb] | chosen ids, scores [kMaxTopK] | red.
// The choice is over selection blocks (sb tokens, sb / bs summaries each,
// importance summed over them; P holds those sums when sb > bs).
template <typename T>
__global__ void __launch_bounds__(kThreads) k_select_generic(
    const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ vc,
    int32_t* __restrict__ idx, float* __restrict__ score, float* __restrict__ ocmp, GArgs a) {
  extern __shared__ float smem[];
  float* qs = smem;
  float* P = qs + a.dq;
  float* I = P + a.nb;
  int* chosen = (int*)(I + a.nb);
  float* chosen_score = (float*)(chosen + kMaxTopK);
  float* red = chosen_score + kMaxTopK;
  __shared__ int s_cnt;

  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x % a.G;
  const int64_t row = blockIdx.x / a.G;
  const int64_t b = row / a.T, t = row % a.T;
  const int64_t p = a.L - a.T + t;
  int64_t nvis = (p + 1) / a.bs;
  if (nvis > a.nb) nvis = a.nb;

  for (int64_t j = tid; j < nvis; j += kThreads) I[j] = 0.f;

  for (int64_t hh = 0; hh < a.hpg; ++hh) {
    const int64_t h = g * a.hpg + hh;
    __syncthreads();
    for (int64_t d = tid; d < a.dq; d += kThreads) qs[d] = ld(q, ((b * a.T + t) * a.H + h) * a.dq + d);
    __syncthreads();
    float lmax = -INFINITY;
    for (int64_t j = tid; j < nvis; j += kThreads) {
      const T* kr = kc + ((b * a.nb + j) * a.G + g) * a.dq;
      float z = 0.f;
      for (int64_t d = 0; d < a.dq; ++d) z = fmaf(qs[d], ld(kr, d), z);
      z *= a.scale;
      P[j] = z;
      lmax = fmaxf(lmax, z);
    }
    const float m = block_max(lmax, red);
    float lsum = 0.f;
    for (int64_t j = tid; j < nvis; j += kThreads) {
      const float e = expf(P[j] - m);
      P[j] = e;
      lsum += e;
    }
    const float inv = 1.0f / block_sum(lsum, red);
    for (int64_t j = tid; j < nvis; j += kThreads) {
      P[j] *= inv;
      I[j] += P[j];
    }
    __syncthreads();
    if (ocmp) {
      for (int64_t e = tid; e < a.dv; e += kThreads) {
        float acc = 0.f;
        for (int64_t j = 0; j < nvis; ++j) acc = fmaf(P[j], ld(vc, ((b * a.nb + j) * a.G + g) * a.dv + e), acc);
        ocmp[((b * a.T + t) * a.H + h) * a.dv + e] = acc;
      }
    }
  }
  __syncthreads();

  // selection blocks: importance summed over their summaries
  const int64_t per = a.sb / a.bs;
  int64_t nsel = (p + 1) / a.sb;
  if (nsel > a.nbs) nsel = a.nbs;
  const int64_t cur = p / a.sb;
  float* Isel = I;
  if (per > 1) {
    for (int64_t J = tid; J < nsel; J += kThreads) {
      float s = 0.f;
      for (int64_t i = 0; i < per; ++i) s += I[J * per + i];
      P[J] = s;
    }
    Isel = P;
    __syncthreads();
  }
  nvis = nsel;

  // forced blocks, removed from the candidates
  if (tid == 0) {
    int cnt = 0;
    if (a.flags & NSA_F_FORCE_FIRST) chosen[cnt++] = 0;
    if ((a.flags & NSA_F_FORCE_CURRENT) && !((a.flags & NSA_F_FORCE_FIRST) && cur == 0)) chosen[cnt++] = (int)cur;
    for (int f = 0; f < cnt; ++f) {
      chosen_score[f] = INFINITY;
      if (chosen[f] < nvis) Isel[chosen[f]] = -1.f;
    }
    s_cnt = cnt;
  }
  __syncthreads();
  const int nf = s_cnt;
  int ncand = (int)nvis;
  for (int f = 0; f < nf; ++f) ncand -= (chosen[f] < nvis) ? 1 : 0;
  const int r = (int)(a.n - nf) < ncand ? (int)(a.n - nf) : ncand;

  for (int round = 0; round < r; ++round) {
    float bv = -1.f;
    int bj = 0x7fffffff;
    for (int64_t j = tid; j < nvis; j += kThreads) {
      const float vj = Isel[j];
      if (vj >= 0.f && better(vj, (int)j, bv, bj)) { bv = vj; bj = (int)j; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oj = __shfl_xor(bj, o, 64);
      if (better(ov, oj, bv, bj)) { bv = ov; bj = oj; }
    }
    __syncthreads();
    if ((tid & 63) == 0) { red[tid >> 6] = bv; ((int*)red)[kWaves + (tid >> 6)] = bj; }
    __syncthreads();
    if (tid == 0) {
      float v0 = red[0];
      int j0 = ((int*)red)[kWaves];
      for (int w = 1; w < kWaves; ++w)
        if (better(red[w], ((int*)red)[kWaves + w], v0, j0)) { v0 = red[w]; j0 = ((int*)red)[kWaves + w]; }
      chosen[nf + round] = j0;
      chosen_score[nf + round] = v0;
      Isel[j0] = -1.f;
    }
    __syncthreads();
  }

  if (tid == 0) {
    const int cnt = nf + r;
    for (int i = 1; i < cnt; ++i) {  // insertion sort by block id
      const int cj = chosen[i];
      const float cs = chosen_score[i];
      int k2 = i - 1;
      while (k2 >= 0 && chosen[k2] > cj) { chosen[k2 + 1] = chosen[k2]; chosen_score[k2 + 1] = chosen_score[k2]; --k2; }
      chosen[k2 + 1] = cj;
      chosen_score[k2 + 1] = cs;
    }
    int32_t* out = idx + ((b * a.T + t) * a.G + g) * a.n;
    float* sc = score ? score + ((b * a.T + t) * a.G + g) * a.n : nullptr;
    for (int i = 0; i < a.n; ++i) {
      out[i] = i < cnt ? chosen[i] : -1;
      if (sc) sc[i] = i < cnt ? chosen_score[i] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Softmax attention of one head over a key set given by key(i), i < nkeys.
// Returns this thread's output element (thread e < dv) and the log-sum-exp.
template <typename T, typename KeyFn>
__device__ void attend_set(const T* __restrict__ k, const T* __restrict__ v, const float* qs, float* wts,
                           float* red, const GArgs& a, int64_t b, int64_t g, int64_t nkeys, KeyFn key,
                           float& o, float& lse) {
  const int tid = threadIdx.x;
  float lmax = -INFINITY;
  for (int64_t i = tid; i < nkeys; i += kThreads) {
    const int64_t s = key(i);
    float z = -INFINITY;
    if (s >= 0) {
      const T* kr = k + ((b * a.L + s) * a.G + g) * a.dq;
      float acc = 0.f;
      for (int64_t d = 0; d < a.dq; ++d) acc = fmaf(qs[d], ld(kr, d), acc);
      z = acc * a.scale;
    }
    wts[i] = z;
    lmax = fmaxf(lmax, z);
  }
  const float m = block_max(lmax, red);
  float lsum = 0.f;
  for (int64_t i = tid; i < nkeys; i += kThreads) {
    const float e = wts[i] == -INFINITY ? 0.f : expf(wts[i] - m);
    wts[i] = e;
    lsum += e;
  }
  const float l = block_sum(lsum, red);  // ends with a barrier: wts visible
  o = 0.f;
  if (tid < a.dv && l > 0.f) {
    float acc = 0.f;
    for (int64_t i = 0; i < nkeys; ++i) {
      const float wi = wts[i];
      if (wi != 0.f) acc = fmaf(wi, ld(v, ((b * a.L + key(i)) * a.G + g) * a.dv + tid), acc);
    }
    o = acc / l;
  }
  lse = l > 0.f ? m + logf(l) : -INFINITY;
  __syncthreads();  // wts reused by the next call
}

// Selected + window branches and the gated sum, one (b, t, g) per workgroup.
// LDS: q row [dq] | weights [cap] | idx row [kMaxTopK] | red.
template <typename T, typename TO>
__global__ void __launch_bounds__(kThreads) k_attend_generic(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ gates,
    const int32_t* __restrict__ idx, const float* __restrict__ ocmp, TO* __restrict__ out,
    float* __restrict__ lse_out, GArgs a, int64_t cap) {
  extern __shared__ float smem[];
  float* qs = smem;
  float* wts = qs + a.dq;
  int* sidx = (int*)(wts + cap);
  float* red = (float*)(sidx + kMaxTopK);

  const int tid = threadIdx.x;
  const int64_t g = blockIdx.x % a.G;
  const int64_t row = blockIdx.x / a.G;
  const int64_t b = row / a.T, t = row % a.T;
  const int64_t p = a.L - a.T + t;
  const bool use_cmp = a.flags & NSA_F_CMP, use_slc = a.flags & NSA_F_SLC;
  const bool use_win = (a.flags & NSA_F_WIN) && a.w > 0;
  const bool logits = a.flags & NSA_F_GATE_LOGITS;

  for (int i = tid; i < a.n; i += kThreads) sidx[i] = idx[((b * a.T + t) * a.G + g) * a.n + i];
  int64_t wlo = p - a.w + 1;
  if (wlo < 0) wlo = 0;
  const int64_t bs = a.sb;  // the chosen blocks are selection blocks

  for (int64_t hh = 0; hh < a.hpg; ++hh) {
    const int64_t h = g * a.hpg + hh;
    const int64_t qrow = (b * a.T + t) * a.H + h;
    __syncthreads();
    for (int64_t d = tid; d < a.dq; d += kThreads) qs[d] = ld(q, qrow * a.dq + d);
    __syncthreads();
    float o_slc = 0.f, o_win = 0.f, lse_slc = -INFINITY, lse_win = -INFINITY;
    if (use_slc) {
      auto key = [&](int64_t i) -> int64_t {
        const int64_t j = sidx[i / bs];
        const int64_t s = j * bs + i % bs;
        return (j >= 0 && s <= p) ? s : -1;
      };
      attend_set(k, v, qs, wts, red, a, b, g, a.n * bs, key, o_slc, lse_slc);
    }
    if (use_win) {
      auto key = [&](int64_t i) -> int64_t { return wlo + i; };
      attend_set(k, v, qs, wts, red, a, b, g, p - wlo + 1, key, o_win, lse_win);
    }
    if (tid < a.dv) {
      float g0 = 1.f, g1 = 1.f, g2 = 1.f;
      if (gates) {
        g0 = ld(gates, qrow * 3 + 0);
        g1 = ld(gates, qrow * 3 + 1);
        g2 = ld(gates, qrow * 3 + 2);
        if (logits) { g0 = sigmoid(g0); g1 = sigmoid(g1); g2 = sigmoid(g2); }
      }
      float acc = 0.f;
      if (use_cmp) acc = fmaf(g0, ocmp[qrow * a.dv + tid], acc);
      if (use_slc) acc = fmaf(g1, o_slc, acc);
      if (use_win) acc = fmaf(g2, o_win, acc);
      st(out, qrow * a.dv + tid, acc);
    }
    if (lse_out && tid == 0) lse_out[qrow] = lse_slc;
  }
}

GArgs make_args(const Prob& P) {
  GArgs a;
  a.B = P.B; a.T = P.T; a.L = P.L; a.G = P.G; a.hpg = P.hpg; a.H = P.H;
  a.dq = P.dq; a.dv = P.dv; a.bs = P.bs; a.n = P.n; a.w = P.w; a.nb = P.nb;
  a.sb = P.sb; a.nbs = P.nbs;
  a.scale = P.scale; a.flags = P.flags;
  return a;
}

}  // namespace

hipError_t launch_select_generic(const Prob& P, const void* q, const void* kc, const void* vc,
                                 int32_t* idx, float* score, float* ocmp, hipStream_t s) {
  const GArgs a = make_args(P);
  const size_t lds = sizeof(float) * (size_t)(P.dq + 2 * P.nb + 2 * kMaxTopK + 2 * kWaves);
  const unsigned grid = (unsigned)(P.B * P.T * P.G);
  if (P.bf16()) {
    auto kern = k_select_generic<uint16_t>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_select_generic<uint16_t>", kern, grid, kThreads, lds, s, (const uint16_t*)q, (const uint16_t*)kc, (const uint16_t*)vc, idx, score, ocmp, a);
  } else {
    auto kern = k_select_generic<float>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_select_generic<float>", kern, grid, kThreads, lds, s, (const float*)q, (const float*)kc, (const float*)vc, idx, score, ocmp, a);
  }
  return hipGetLastError();
}

hipError_t launch_attend_generic(const Prob& P, const void* q, const void* k, const void* v,
                                 const void* gates, const int32_t* idx, const float* ocmp,
                                 void* out, float* lse, bool out_f32, hipStream_t s) {
  const GArgs a = make_args(P);
  int64_t cap = P.n * P.sb;
  if (P.w > cap) cap = P.w;
  if (cap < 1) cap = 1;
  const size_t lds = sizeof(float) * (size_t)(P.dq + cap + kMaxTopK + 2 * kWaves);
  const unsigned grid = (unsigned)(P.B * P.T * P.G);
#define NSA_LAUNCH_ATTEND(TI, TO)                                                                    \
  do {                                                                                               \
    auto kern = k_attend_generic<TI, TO>;                                                            \
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);    \
    launch("k_attend_generic<TI, TO>", kern, grid, kThreads, lds, s, (const TI*)q, (const TI*)k, (const TI*)v, (const TI*)gates, idx, \
                                     ocmp, (TO*)out, lse, a, cap);                                   \
  } while (0)
  if (P.bf16()) {
    if (out_f32) NSA_LAUNCH_ATTEND(uint16_t, float);
    else NSA_LAUNCH_ATTEND(uint16_t, uint16_t);
  } else {
    NSA_LAUNCH_ATTEND(float, float);
  }
#undef NSA_LAUNCH_ATTEND
  return hipGetLastError();
}

}  // namespace nsa
