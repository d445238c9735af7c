// k_prefill.hip -- matrix-core path of the NSA forward for GQA groups of 16
// query heads and 64-token blocks ([P1] s4 three branches; [P1] s5 the group's
// heads stacked as the matrix M dimension instead of a block of queries).
//
//   k_transpose  V [B, N, G, D] -> tiled V^T [B, G, Np / 32, D, 32] (each
//                32-key tile one contiguous D x 32 chunk, zero padded to
//                Np = round_up(N, 64)): every P.V operand is one contiguous
//                load, a 32-key step reads whole cache lines, a 64-key block
//                is one contiguous 2 x D x 32 read.
//   k_group_major  K [B, L, G, D] -> per group, 16-row groups with rows i and
//                i + 8 interleaved every 32 dims ([B, G, Lp / 16, D / 32, 8, 2, 32],
//                zero padded to Lp = round_up(L, 64)): a 64-key block is one
//                contiguous read, and each matrix-op K load (16 rows x 32
//                dims, the rows pairing i with i + 8) reads whole cache lines.
//   k_cmpwin     one workgroup per (8-token query tile, KV group), one wave
//                per token: compressed branch (online softmax over the block
//                summaries), group importance (second pass, each head's
//                probabilities summed), top-k in registers with wave
//                reductions, window branch, gated partial sum -> fp32 acc.
//   k_sel        one wave per (token, group): the selected blocks streamed
//                straight from global memory as contiguous 32-key chunks,
//                16 heads x 32 keys per matrix op, fp32 online softmax;
//                epilogue adds the gated result to acc and stores out.
#include <math.h>

#include "nsa_frag.h"
#include "nsa_mfma.h"
#include "nsa_prefill.h"
#include "nsa_tile.h"
#include "nsa_topk.h"

namespace nsa {
namespace {

constexpr int TQ = 8;             // tokens (waves) per k_cmpwin workgroup
constexpr int MAX_NB_LANE = 32;   // pooled blocks per lane in the top-k: nb <= 2048

__device__ __forceinline__ float gate_of(const PfArgs& a, int64_t row, int branch) {
  if (!a.gates) return 1.f;
  float x = bf16_to_f32(a.gates[row * 3 + branch]);
  return (a.flags & NSA_F_GATE_LOGITS) ? sigmoid(x) : x;
}

// Training forward: branch br's natural log-sum-exp of the scaled logits
// (-inf when the branch is off or its key set empty) and its normalised
// output in bf16, for head lr of the row; o^T holds dims 16*dt + 4*lg + r.
template <int DV>
__device__ __forceinline__ void save_branch(const PfArgs& a, int br, int64_t row, bool on, float lse,
                                            const f32x4 (&o)[DV / 16], float inv_l, int lg) {
  const int64_t nrow = a.B * a.T * a.H;
  if (lg == 0) a.sv_lse[br * nrow + row] = on ? lse : -INFINITY;
  uint16_t* orow = a.sv_o + (br * nrow + row) * DV + 4 * lg;
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) {
    const f32x4 v = on ? o[dt] * inv_l : f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x2 w = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                     (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
    *(u32x2*)(orow + 16 * dt) = w;
  }
}

__device__ __forceinline__ bool better(float v, int j, float bv, int bj) {
  return v > bv || (v == bv && j < bj);
}

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_transpose(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                   int64_t N, int64_t Np, int64_t G, int D) {
  __shared__ uint16_t tile[64][256 + 8];
  const int64_t ntile = Np / 64;
  const int64_t tix = blockIdx.x % ntile;
  const int64_t g = (blockIdx.x / ntile) % G;
  const int64_t b = blockIdx.x / (ntile * G);
  const int64_t n0 = tix * 64;
  const int chunks = D / 8;
  for (int c = threadIdx.x; c < 64 * chunks; c += 256) {
    const int r = c / chunks, c8 = c % chunks;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (n0 + r < N) val = *(const u32x4*)(src + ((b * N + n0 + r) * G + g) * D + 8 * c8);
    *(u32x4*)&tile[r][8 * c8] = val;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D * 8; c += 256) {
    const int d = c / 8, k8 = c % 8;
    uint16_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = tile[8 * k8 + i][d];
    u32x4 val = {(uint32_t)w[0] | ((uint32_t)w[1] << 16), (uint32_t)w[2] | ((uint32_t)w[3] << 16),
                 (uint32_t)w[4] | ((uint32_t)w[5] << 16), (uint32_t)w[6] | ((uint32_t)w[7] << 16)};
    // keys 8*k8 .. 8*k8+7 of the 64-key tile: half k8 / 4 of it, 8*(k8 % 4) into the half
    *(u32x4*)(dst + ((b * G + g) * ntile + tix) * D * 64 + (k8 / 4) * D * 32 + d * 32 + 8 * (k8 % 4)) = val;
  }
}

// Element offset of (row, d) inside one group's paired-row K image.
__device__ __forceinline__ int64_t kp_offset(int64_t row, int64_t d, int D) {
  const int64_t rg = row >> 4, w = row & 15;
  return ((rg * (D / 32) + (d >> 5)) * 8 + (w & 7)) * 64 + (w >> 3) * 32 + (d & 31);
}

__global__ void __launch_bounds__(256) k_group_major(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     int64_t L, int64_t Lp, int64_t G, int D) {
  // one workgroup per (b, 64-row slab); rows of all groups are read once
  const int64_t nslab = Lp / 64;
  const int64_t b = blockIdx.x / nslab, s0 = (blockIdx.x % nslab) * 64;
  const int chunks = D / 8;
  for (int64_t c = threadIdx.x; c < 64 * G * chunks; c += 256) {
    const int64_t r = c / (G * chunks), g = (c / chunks) % G, c8 = c % chunks;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (s0 + r < L) val = *(const u32x4*)(src + ((b * L + s0 + r) * G + g) * D + 8 * c8);
    *(u32x4*)(dst + (b * G + g) * Lp * D + kp_offset(s0 + r, 8 * c8, D)) = val;
  }
}

// Top-k of one token's selection blocks (one wave): block J < nsel has the
// importance imp[per * J] + .. + imp[per * J + per - 1] (its summaries);
// written sorted to orow / srow.
template <int NBL>
__device__ __forceinline__ void topk_row(const float* imp, int64_t per, int64_t nsel, int64_t cur, uint32_t flags,
                                         int n, int32_t* orow, float* srow) {
  const int lane = threadIdx.x & 63;
  float vals[NBL];
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    const int64_t j = lane + 64 * i;
    float v = -1.f;
    if (j < nsel) {
      v = imp[per * j];
      for (int64_t k = 1; k < per; ++k) v += imp[per * j + k];
    }
    vals[i] = v;
  }
  int cj;
  float cs;
  const int cnt = topk_wave<NBL>(vals, nsel, cur, flags, n, cj, cs);
  topk_write(cnt, cj, cs, n, orow, srow);
}

// ---------------------------------------------------------------------------
template <int DQ, int DV, bool FWD>
__global__ void __launch_bounds__(TQ * 64) k_cmpwin(PfArgs a) {
  constexpr int KS = k_lds_stride<DQ>(), VS = kVtStride;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* kt = (uint16_t*)smem_raw;                // [64][KS]
  uint16_t* vt = kt + 64 * KS;                       // [DV][VS]
  float* imp = (float*)(vt + (FWD ? DV * VS : 0));   // [TQ][nbp]

  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t ntiles = (a.T + TQ - 1) / TQ;
  const int64_t g = blockIdx.x % a.G;
  const int64_t tile = ntiles - 1 - (blockIdx.x / a.G) % ntiles;  // longest rows first
  const int64_t b = blockIdx.x / (a.G * ntiles);
  const int64_t t = tile * TQ + wave;
  const bool active = t < a.T;
  const int64_t t_last = (tile * TQ + TQ - 1 < a.T - 1) ? tile * TQ + TQ - 1 : a.T - 1;
  const int64_t p = a.L - a.T + (active ? t : t_last);
  const int64_t p_first = a.L - a.T + tile * TQ, p_last = a.L - a.T + t_last;
  int64_t nvis = active ? (p + 1) / a.bs : 0;  // visible summaries
  if (nvis > a.nb) nvis = a.nb;
  int64_t nvis_max = (p_last + 1) / a.bs;
  if (nvis_max > a.nb) nvis_max = a.nb;
  const float c = a.scale * kLog2e;
  const float stale = kStaleLog2 / c;
  const int64_t h = g * 16 + lr;
  const int64_t row = (b * a.T + (active ? t : t_last)) * a.H + h;
  const bool use_cmp = FWD && (a.flags & NSA_F_CMP);
  const bool use_win = FWD && (a.flags & NSA_F_WIN) && a.w > 0;

  bf16x8 qf[DQ / 32];
  {
    const uint16_t* qr = a.q + row * DQ + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) qf[ks] = ld8(qr + 32 * ks);
  }

  // ---- pass 1: compressed branch, softmax statistics (+ its output) ----
  float m = -INFINITY, l = 0.f;
  f32x4 o[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  Stager<DQ, DV, TQ * 64> st;
  const int64_t ntile_cmp = (nvis_max + 63) / 64;
  if (ntile_cmp > 0) st.load(a.kc, a.nb, 0, a.vcT, a.nbp, 0, b, g, a.G, use_cmp);
  for (int64_t jt = 0; jt < ntile_cmp; ++jt) {
    __syncthreads();
    st.store(kt, vt, use_cmp, true);
    __syncthreads();
    if (jt + 1 < ntile_cmp) st.load(a.kc, a.nb, (jt + 1) * 64, a.vcT, a.nbp, (jt + 1) * 64, b, g, a.G, use_cmp);
    if (jt * 64 < nvis) {
      f32x4 s[4];
      qk_tile_T<DQ>(kt, qf, s, lr, lg);
      if (jt * 64 + 64 > nvis) mask_from(s, (int)(nvis - jt * 64), lg);
      softmax_step<DV>(s, m, l, o, c, stale, use_cmp);
      if (use_cmp) pv_tile<DV>(vt, s, o, lr, lg);
    }
  }
  const float inv_l = l > 0.f ? 1.f / l : 0.f;

  f32x4 fin[DV / 16];
  if (FWD) {
    const float g0 = use_cmp ? gate_of(a, row, 0) * inv_l : 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) fin[dt] = o[dt] * g0;
    if (a.sv_lse && active) save_branch<DV>(a, 0, row, use_cmp && l > 0.f, m * a.scale + logf(l), o, inv_l, lg);
  }

  // ---- pass 2: importance of each visible block, summed over the heads ----
  float mh[4], ih[4];  // per head 4*lg + r: m * c and 1 / l
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mh[r] = __shfl(m * c, 4 * lg + r, 64);
    ih[r] = __shfl(inv_l, 4 * lg + r, 64);
  }
  float* my_imp = imp + (int64_t)wave * a.nbp;
  if (ntile_cmp > 0) st.load(a.kc, a.nb, 0, nullptr, 0, 0, b, g, a.G, false);
  for (int64_t jt = 0; jt < ntile_cmp; ++jt) {
    __syncthreads();
    st.store(kt, vt, false, false);
    __syncthreads();
    if (jt + 1 < ntile_cmp) st.load(a.kc, a.nb, (jt + 1) * 64, nullptr, 0, 0, b, g, a.G, false);
    if (jt * 64 < nvis) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DQ / 32; ++ks) s = mfma16(qf[ks], ld8(kt + (16 * nt + lr) * KS + 8 * lg + 32 * ks), s);
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v = fmaf(fast_exp2(fmaf(s[r], c, -mh[r])), ih[r], v);
        v = xor_sum16_32(v);
        const int64_t blk = jt * 64 + 16 * nt + lr;
        if (lg == 0 && blk < nvis) my_imp[blk] = v;
      }
    }
  }
  __syncthreads();

  // the window's first tile is read while the top-k runs
  int64_t kb0 = 0, kb1 = -1;
  if (use_win) {
    int64_t lo = p_first - a.w + 1;
    if (lo < 0) lo = 0;
    kb0 = lo / 64;
    kb1 = p_last / 64;
    st.load(a.k, a.L, kb0 * 64, a.vT, a.Lp, kb0 * 64, b, g, a.G, true);
  }

  // ---- top-k of this token's row (one wave) ----
  if (active) {
    int32_t* orow = a.idx + ((b * a.T + t) * a.G + g) * a.n;
    float* srow = a.score ? a.score + ((b * a.T + t) * a.G + g) * a.n : nullptr;
    // 64-token selection blocks, complete ones are candidates
    int64_t nsel = (p + 1) / 64;
    if (nsel > a.nbs) nsel = a.nbs;
    if (a.nbs <= 1024) topk_row<16>(my_imp, a.per, nsel, p / 64, a.flags, (int)a.n, orow, srow);
    else topk_row<MAX_NB_LANE>(my_imp, a.per, nsel, p / 64, a.flags, (int)a.n, orow, srow);
  }

  if (!FWD) return;

  // ---- window branch: keys p - w < s <= p, FA-style over the tile ----
  if (use_win) {
    float m2 = -INFINITY, l2 = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t kb = kb0; kb <= kb1; ++kb) {
      __syncthreads();
      st.store(kt, vt, true, true);
      __syncthreads();
      if (kb + 1 <= kb1) st.load(a.k, a.L, (kb + 1) * 64, a.vT, a.Lp, (kb + 1) * 64, b, g, a.G, true);
      if (active && kb * 64 <= p && kb * 64 + 63 > p - a.w) {
        f32x4 s[4];
        qk_tile_T<DQ>(kt, qf, s, lr, lg);
        if (kb * 64 + 63 > p) mask_from(s, (int)(p + 1 - kb * 64), lg);
        if (kb * 64 <= p - a.w) mask_below(s, (int)(p - a.w + 1 - kb * 64), lg);
        softmax_step<DV>(s, m2, l2, o, c, stale, true);
        pv_tile<DV>(vt, s, o, lr, lg);
      }
    }
    const float g2 = gate_of(a, row, 2) * (l2 > 0.f ? 1.f / l2 : 0.f);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) fin[dt] += o[dt] * g2;
    if (a.sv_lse && active) save_branch<DV>(a, 2, row, l2 > 0.f, m2 * a.scale + logf(l2), o, 1.f / l2, lg);
  } else if (FWD && a.sv_lse && active) {
    save_branch<DV>(a, 2, row, false, 0.f, o, 0.f, lg);
  }

  if (active) {
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) *(f32x4*)(a.acc + row * DV + 16 * dt + 4 * lg) = fin[dt];
  }
}

// ---------------------------------------------------------------------------
template <typename TO> __device__ __forceinline__ void store4(TO* p, f32x4 v);
// outputs are written once and never re-read here: non-temporal stores keep
// them from evicting the K/V tiles that other tokens re-use
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) { __builtin_nontemporal_store(v, (f32x4*)p); }
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 v) {
  u32x2 w = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
             (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
  __builtin_nontemporal_store(w, (u32x2*)p);
}

// S^T for the chunk's 32 keys (raw dot products).
template <int DQ>
__device__ __forceinline__ void qk_chunk(const KFrag<DQ>& f, const bf16x8 (&qf)[DQ / 32], f32x4& s0, f32x4& s1) {
  s0 = f32x4{0.f, 0.f, 0.f, 0.f};
  s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) {
    s0 = mfma16(f.k0[ks], qf[ks], s0);
    s1 = mfma16(f.k1[ks], qf[ks], s1);
  }
}

// Online-softmax update of one wave's token (16 heads, head lr per lane)
// with a chunk whose keys start at kb; keys beyond p are masked (only the
// query's own block can have any).  m is a stale maximum in raw dot units:
// it is raised only when a score exceeds it by more than 2^kStaleLog2 in
// probability, and only then are l and o rescaled.
template <int DV>
__device__ __forceinline__ void pv_chunk(const VFrag<DV>& f, f32x4 s0, f32x4 s1, f32x4 (&o)[DV / 16], float& m,
                                         float& l, float c, float stale, int64_t kb, int64_t p, int lg) {
  if (kb + 31 > p) {
    const int rel = (int)(p - kb);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (8 * lg + r > rel) s0[r] = -INFINITY;
      if (8 * lg + 4 + r > rel) s1[r] = -INFINITY;
    }
  }
  float tmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  tmax = xor_max16_32(tmax);
  const bool raise = tmax > m + stale;
  if (__ballot(raise)) {
    const float mnew = raise ? tmax : m;
    const float alpha = fast_exp2((m - mnew) * c);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[dt] *= alpha;
    m = mnew;
  }
  const float mc = m * c;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s0[r] = fast_exp2(fmaf(s0[r], c, -mc));
    s1[r] = fast_exp2(fmaf(s1[r], c, -mc));
    rs += s0[r] + s1[r];
  }
  l += xor_sum16_32(rs);
  const bf16x8 pf = pack8(s0, s1);
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) o[dt] = mfma16(f.v[dt], pf, o[dt]);
}

template <int DQ, int DV, bool FWD, typename TO>
__global__ void __launch_bounds__(256) k_sel(PfArgs a) {
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  // 4 consecutive tokens of one group per workgroup; each XCD takes a
  // contiguous run of a group's tokens
  const int64_t nq = (a.B * a.T + 3) / 4;
  const int64_t j = xcd_run(a.G * nq);
  if (j >= a.G * nq) return;
  const int64_t g = j / nq;
  const int64_t tg = (j % nq) * 4 + wave;  // flat (b, t)
  if (tg >= a.B * a.T) return;
  const int64_t b = tg / a.T, t = tg % a.T;
  const int64_t p = a.L - a.T + t;
  const float c = a.scale * kLog2e;
  const int64_t h = g * 16 + lr;
  const int64_t row = (b * a.T + t) * a.H + h;

  bf16x8 qf[DQ / 32];
  {
    const uint16_t* qr = a.q + row * DQ + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(qr + 32 * ks)));
  }
  const bool use_slc = !FWD || (a.flags & NSA_F_SLC);
  // chunk list: lane c describes chunk c = (slot c / 2, half c % 2); n <= 32
  int64_t kbv = -1;
  {
    const int slot = lane >> 1;
    const int j = slot < a.n ? a.idx[((b * a.T + t) * a.G + g) * a.n + slot] : -1;
    const int64_t kb = (int64_t)j * 64 + 32 * (lane & 1);
    if (use_slc && j >= 0 && kb <= p) kbv = kb;
  }
  uint64_t pending = __ballot(kbv >= 0);
  const int nch = __popcll(pending);

  float m = -INFINITY, l = 0.f;
  f32x4 o[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(a.kG + (b * a.G + g) * a.Lp * DQ, (uint32_t)(a.Lp * DQ * 2));
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(a.vT + (b * a.G + g) * a.Lp * DV, (uint32_t)(a.Lp * DV * 2));
  const uint32_t kofs = 16 * lg, vofs = (lr * 32 + 8 * lg) * 2;

  // next chunk's key base, -1 once the list is exhausted (its loads then
  // fall past the end of the buffers: zeros, no memory traffic)
  auto next_kb = [&]() -> int64_t {
    if (!pending) return -1;
    const int pos = __ffsll((unsigned long long)pending) - 1;
    pending &= pending - 1;
    return __shfl(kbv, pos, 64);
  };
  // two-stage software pipeline: the next chunk's reads are in flight while
  // this one is computed (unrolled by two: fixed registers, exact waits)
  const float stale = kStaleLog2 / c;
  KFrag<DQ> k0, k1;
  VFrag<DV> v0, v1;
  auto load = [&](KFrag<DQ>& kf, VFrag<DV>& vf, int64_t kb) {
    load_k<DQ>(kf, kr, kofs, kb, lr);
    load_v<DV>(vf, vr, vofs, kb);
  };
  auto step = [&](const KFrag<DQ>& kf, const VFrag<DV>& vf, int64_t kb) {
    f32x4 s0, s1;
    qk_chunk<DQ>(kf, qf, s0, s1);
    pv_chunk<DV>(vf, s0, s1, o, m, l, c, stale, kb, p, lg);
  };
  if (nch > 0) {
    int64_t c0 = next_kb(), c1;
    load(k0, v0, c0);
    for (int ci = 0; ci < nch; ci += 2) {
      c1 = next_kb();
      load(k1, v1, c1);
      __builtin_amdgcn_sched_barrier(0);
      step(k0, v0, c0);
      __builtin_amdgcn_sched_barrier(0);
      if (ci + 1 >= nch) break;
      c0 = next_kb();
      load(k0, v0, c0);
      __builtin_amdgcn_sched_barrier(0);
      step(k1, v1, c1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  TO* orow = (TO*)a.out + row * DV + 4 * lg;
  if (FWD) {
    float g1 = 0.f;
    if (a.flags & NSA_F_SLC) g1 = gate_of(a, row, 1) * inv_l;
    if (a.sv_lse) save_branch<DV>(a, 1, row, use_slc && l > 0.f, m * a.scale + logf(l), o, inv_l, lg);
    const float* arow = a.acc + row * DV + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt)
      store4<TO>(orow + 16 * dt, __builtin_nontemporal_load((const f32x4*)(arow + 16 * dt)) + o[dt] * g1);
  } else {
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4<TO>(orow + 16 * dt, o[dt] * inv_l);
    if (a.lse && lg == 0) a.lse[row] = l > 0.f ? m * a.scale + logf(l) : -INFINITY;
  }
}

template <int DQ, int DV>
hipError_t launch_cmpwin_t(const PfArgs& a, bool fwd, hipStream_t s) {
  constexpr int KS = k_lds_stride<DQ>(), VS = kVtStride;
  const size_t lds = sizeof(uint16_t) * (64 * KS + (fwd ? DV * VS : 0)) + sizeof(float) * TQ * a.nbp;
  const unsigned grid = (unsigned)(a.B * a.G * ((a.T + TQ - 1) / TQ));
  if (fwd) {
    auto kern = k_cmpwin<DQ, DV, true>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kern<<<grid, TQ * 64, lds, s>>>(a);
  } else {
    auto kern = k_cmpwin<DQ, DV, false>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kern<<<grid, TQ * 64, lds, s>>>(a);
  }
  return hipGetLastError();
}

template <int DQ, int DV>
hipError_t launch_sel_t(const PfArgs& a, bool fwd, bool out_f32, hipStream_t s) {
  const unsigned grid = xcd_grid(a.G * ((a.B * a.T + 3) / 4));
  if (fwd) {
    if (out_f32) k_sel<DQ, DV, true, float><<<grid, 256, 0, s>>>(a);
    else k_sel<DQ, DV, true, uint16_t><<<grid, 256, 0, s>>>(a);
  } else {
    if (out_f32) k_sel<DQ, DV, false, float><<<grid, 256, 0, s>>>(a);
    else k_sel<DQ, DV, false, uint16_t><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

bool prefill_fast_ok(const Prob& P) {
  const int64_t nbp = (P.nb + 63) / 64 * 64;
  return P.bf16() && P.hpg == 16 && P.sb == 64 && (P.bs == 64 || P.bs == 32 || P.bs == 16) &&
         (P.dq == 64 || P.dq == 128 || P.dq == 192) && (P.dv == 64 || P.dv == 128) && nbp <= 64 * MAX_NB_LANE &&
         P.n <= 32;
}

hipError_t launch_group_major(const void* src, void* dst, int64_t B, int64_t L, int64_t G, int D, hipStream_t s) {
  const int64_t Lp = (L + 63) / 64 * 64;
  const unsigned grid = (unsigned)(B * (Lp / 64));
  if (grid == 0) return hipSuccess;
  k_group_major<<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, L, Lp, G, D);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int64_t B, int64_t N, int64_t Np, int64_t G, int D,
                            hipStream_t s) {
  const unsigned grid = (unsigned)(B * G * (Np / 64));
  if (grid == 0) return hipSuccess;
  k_transpose<<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, N, Np, G, D);
  return hipGetLastError();
}

hipError_t launch_cmpwin(const Prob& P, const PfArgs& a, bool fwd, hipStream_t s) {
#define CALL_CW(DQ, DV) launch_cmpwin_t<DQ, DV>(a, fwd, s)
  if (P.dq == 192 && P.dv == 128) return CALL_CW(192, 128);
  if (P.dq == 128 && P.dv == 128) return CALL_CW(128, 128);
  if (P.dq == 64 && P.dv == 64) return CALL_CW(64, 64);
  if (P.dq == 192 && P.dv == 64) return CALL_CW(192, 64);
  if (P.dq == 128 && P.dv == 64) return CALL_CW(128, 64);
  if (P.dq == 64 && P.dv == 128) return CALL_CW(64, 128);
#undef CALL_CW
  return hipErrorInvalidValue;
}

hipError_t launch_sel(const Prob& P, const PfArgs& a, bool fwd, bool out_f32, hipStream_t s) {
#define CALL_SEL(DQ, DV) launch_sel_t<DQ, DV>(a, fwd, out_f32, s)
  if (P.dq == 192 && P.dv == 128) return CALL_SEL(192, 128);
  if (P.dq == 128 && P.dv == 128) return CALL_SEL(128, 128);
  if (P.dq == 64 && P.dv == 64) return CALL_SEL(64, 64);
  if (P.dq == 192 && P.dv == 64) return CALL_SEL(192, 64);
  if (P.dq == 128 && P.dv == 64) return CALL_SEL(128, 64);
  if (P.dq == 64 && P.dv == 128) return CALL_SEL(64, 128);
#undef CALL_SEL
  return hipErrorInvalidValue;
}

}  // namespace nsa
