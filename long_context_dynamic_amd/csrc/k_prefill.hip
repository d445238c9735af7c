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
//   k_sel_part   one wave per (token, group, XCD stripe): the token's
//                selected blocks that belong to the stripe of its XCD (block
//                j mod 8) streamed straight from global memory as contiguous
//                32-key chunks, 16 heads x 32 keys per matrix op, fp32 online
//                softmax; a normalised partial output and its log-sum-exp.
//   k_sel_merge  one wave per (token, group): log-sum-exp merge of the
//                stripes' partials, plus the gated acc; stores out.
#include <math.h>

#include "nsa_frag.h"
#include "nsa_mfma.h"
#include "nsa_prefill.h"
#include "nsa_tile.h"
#include "nsa_topk.h"

namespace nsa {
namespace {

constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one CU
constexpr int MAX_NB_LANE = 32;   // pooled blocks per lane in the top-k: nb <= 2048

__device__ __forceinline__ float gate_of(const PfArgs& a, int64_t row, int branch) {
  if (!a.gates) return 1.f;
  float x = bf16_to_f32(a.gates[row * 3 + branch]);
  return (a.flags & NSA_F_GATE_LOGITS) ? sigmoid(x) : x;
}

// The gated compressed + window partial sum of (row = b T + t, group g) in
// fragment order: 16-dim block dt of the 16 heads is 1 KiB, lane (lr, lg)'s
// 4 floats (dims 16 dt + 4 lg .. + 3 of head lr, the matrix op's output
// layout) at float offset 4 lane, so its writes and the merge's reads are
// 1 KiB contiguous per instruction.
__device__ __forceinline__ float* acc_frag(const PfArgs& a, int64_t row, int64_t g, int dt, int DV) {
  return a.acc + ((row * a.G + g) * (DV / 16) + dt) * 256;
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

// Fragment-order K image (layout in nsa_frag.h): one workgroup per (b, g,
// 32-key chunk); each thread writes whole 16-byte pieces in output order,
// reading the 8 dims of one key row (keys past L give zeros).
__global__ void __launch_bounds__(256) k_frag_k(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                int64_t L, int64_t nc, int64_t G, int D) {
  const int64_t c = blockIdx.x % nc, bg = blockIdx.x / nc;
  const int64_t g = bg % G, b = bg / G;
  const int npieces = (D / 32) * 2 * 64;
  uint16_t* out = dst + (bg * nc + c) * frag_chunk(D);
  for (int P = threadIdx.x; P < npieces; P += 256) {
    const int l = P & 63, t = (P >> 6) & 1, ks = P >> 7;
    const int lr = l & 15, lg = l >> 4;
    const int64_t key = 32 * c + 8 * (lr >> 2) + 4 * t + (lr & 3);
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < L) val = *(const u32x4*)(src + ((b * L + key) * G + g) * D + 32 * ks + 8 * lg);
    *(u32x4*)(out + 8 * P) = val;
  }
}

// Fragment-order V^T image from the tiled V^T [B, G, Lp / 32, D, 32]: a
// permutation of its 16-byte pieces (one workgroup per (b, g, chunk)).
__global__ void __launch_bounds__(256) k_frag_v(const uint16_t* __restrict__ vT, uint16_t* __restrict__ dst, int64_t nc,
                                                int D) {
  const int64_t c = blockIdx.x % nc, bg = blockIdx.x / nc;
  const uint16_t* in = vT + (bg * nc + c) * 32 * D;
  uint16_t* out = dst + (bg * nc + c) * frag_chunk(D);
  const int npieces = (D / 16) * 64;
  for (int P = threadIdx.x; P < npieces; P += 256) {
    const int l = P & 63, dt = P >> 6;
    const int lr = l & 15, lg = l >> 4;
    *(u32x4*)(out + 8 * P) = *(const u32x4*)(in + (16 * dt + lr) * 32 + 8 * lg);
  }
}

// Fragment-order image of the queries: piece (ks, lane l) of row r and
// group g holds q[r, 16 g + l % 16, 32 ks + 8 (l / 16) .. + 7], the lane
// layout of the matrix op's query operand (one thread per 16-byte piece).
__global__ void __launch_bounds__(256) k_frag_q(const uint16_t* __restrict__ q, uint16_t* __restrict__ qF, int64_t n,
                                                int D) {
  const int64_t P = (int64_t)blockIdx.x * 256 + threadIdx.x;  // piece: (row, group, ks, lane)
  if (P >= n) return;
  const int l = (int)(P & 63);
  const int64_t rest = P >> 6;
  const int nks = D / 32;
  const int ks = (int)(rest % nks);
  const int64_t rg = rest / nks;  // row * G + g: the 16 heads of (row, g) are rows 16 rg .. of q
  *(u32x4*)(qF + 8 * P) = *(const u32x4*)(q + (16 * rg + (l & 15)) * D + 32 * ks + 8 * (l >> 4));
}

// Top-k of one token's selection blocks (one wave): block J < nsel has the
// importance imp[per * J] + .. + imp[per * J + per - 1] (its summaries);
// written sorted to orow / srow.
template <int NBL>
__device__ __forceinline__ void topk_row(const float* imp, int64_t per, int64_t nsel, int64_t cur, uint32_t flags,
                                         int n, int32_t* orow, float* srow) {
  const int lane = threadIdx.x & 63;
  float vals[NBL];
  if (per == 1 && nsel > 0) {
    // one summary per selection block: every lane's reads in flight together
    // (blocks past nsel read the last visible one and are then masked)
#pragma unroll
    for (int i = 0; i < NBL; ++i) vals[i] = imp[min(lane + 64 * i, (int)nsel - 1)];
#pragma unroll
    for (int i = 0; i < NBL; ++i) vals[i] = lane + 64 * i < nsel ? vals[i] : -1.f;
  } else {
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
  }
  int cj, cnt;
  float cs;
  if constexpr (NBL <= 16) {
    int nf;
    cnt = topk_wave_keys<NBL>(vals, nsel, cur, flags, n, cj, nf);
    cs = INFINITY;  // forced blocks
    if (srow && lane >= nf && lane < cnt) {
      cs = imp[per * cj];
      for (int64_t k = 1; k < per; ++k) cs += imp[per * cj + k];
    }
  } else {
    cnt = topk_wave<NBL>(vals, nsel, cur, flags, n, cj, cs);
  }
  topk_write(cnt, cj, cs, n, orow, srow);
}

// S^T of one 64-key LDS tile for the TW tokens of a wave: each K fragment
// read from LDS feeds the matrix ops of all of them.
template <int DQ, int TW>
__device__ __forceinline__ void qk_tiles(const uint16_t* kt, const bf16x8 (&qf)[TW][DQ / 32], f32x4 (&s)[TW][4],
                                         int lr, int lg) {
  if constexpr (TW == 2) qk_tile_T2<DQ>(kt, qf, s, lr, lg);
  else qk_tile_T<DQ>(kt, qf[0], s[0], lr, lg);
}
template <int DV, int TW>
__device__ __forceinline__ void pv_tiles(const uint16_t* vt, const f32x4 (&s)[TW][4], f32x4 (&o)[TW][DV / 16],
                                         int lr, int lg) {
  if constexpr (TW == 2) pv_tile2<DV>(vt, s, o, lr, lg);
  else pv_tile<DV>(vt, s[0], o[0], lr, lg);
}

// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (tile of 8 TW consecutive tokens, KV group);
// wave w takes tokens w, w + 8, .. of the tile (TW of them), so the K and V
// tiles staged in LDS feed 8 TW tokens and every fragment a wave reads from
// LDS feeds TW tokens' matrix ops.  A token past the end computes on the
// tile's last row and stores nothing.
template <int DQ, int DV, bool FWD, int TW>
__global__ void __launch_bounds__(512) k_cmpwin(PfArgs a) {
  constexpr int KS = k_lds_stride<DQ>(), VS = kVtStride;
  constexpr int TQW = 8 * TW;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* kt = (uint16_t*)smem_raw;                // [64][KS]
  uint16_t* vt = kt + 64 * KS;                       // [DV][VS]
  float* imp = (float*)(vt + (FWD ? DV * VS : 0));   // [TQW][nbp]

  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t ntiles = (a.T + TQW - 1) / TQW;
  const int64_t g = blockIdx.x % a.G;
  const int64_t tile = ntiles - 1 - (blockIdx.x / a.G) % ntiles;  // longest rows first
  const int64_t b = blockIdx.x / (a.G * ntiles);
  const int64_t t_last = (tile * TQW + TQW - 1 < a.T - 1) ? tile * TQW + TQW - 1 : a.T - 1;
  const int64_t p_first = a.L - a.T + tile * TQW, p_last = a.L - a.T + t_last;
  int64_t nvis_max = (p_last + 1) / a.bs;
  if (nvis_max > a.nb) nvis_max = a.nb;
  const float c = a.scale * kLog2e;
  const float stale = kStaleLog2 / c;
  const bool use_cmp = FWD && (a.flags & NSA_F_CMP);
  const bool use_win = FWD && (a.flags & NSA_F_WIN) && a.w > 0;

  bool active[TW];
  int64_t t[TW], p[TW], nvis[TW], row[TW];
  bf16x8 qf[TW][DQ / 32];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    t[i] = tile * TQW + wave + 8 * i;
    active[i] = t[i] < a.T;
    const int64_t tt = active[i] ? t[i] : t_last;
    p[i] = a.L - a.T + tt;
    nvis[i] = active[i] ? (p[i] + 1) / a.bs : 0;  // visible summaries
    if (nvis[i] > a.nb) nvis[i] = a.nb;
    row[i] = (b * a.T + tt) * a.H + g * 16 + lr;
    const uint16_t* qr = a.q + row[i] * DQ + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) qf[i][ks] = ld8(qr + 32 * ks);
    // the selected branch reads the queries in this lane order (1 KiB per
    // operand in lane order, coalesced) from the fragment-order image
    if (FWD && a.qF && active[i]) {
      uint16_t* qo = a.qF + ((b * a.T + t[i]) * a.G + g) * 16 * DQ + 8 * lane;
#pragma unroll
      for (int ks = 0; ks < DQ / 32; ++ks) *(bf16x8*)(qo + 512 * ks) = qf[i][ks];
    }
  }

  // ---- pass 1: compressed branch, softmax statistics (+ its output) ----
  float m[TW], l[TW];
  f32x4 o[TW][DV / 16];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  Stager<DQ, DV, 512> st;
  const int64_t ntile_cmp = (nvis_max + 63) / 64;
  if (ntile_cmp > 0) st.load(a.kc, a.nb, 0, a.vcT, a.nbp, 0, b, g, a.G, use_cmp);
  for (int64_t jt = 0; jt < ntile_cmp; ++jt) {
    __syncthreads();
    st.store(kt, vt, use_cmp, true);
    __syncthreads();
    if (jt + 1 < ntile_cmp) st.load(a.kc, a.nb, (jt + 1) * 64, a.vcT, a.nbp, (jt + 1) * 64, b, g, a.G, use_cmp);
    if (jt * 64 < nvis[TW - 1] || jt * 64 < nvis[0]) {
      f32x4 s[TW][4];
      qk_tiles<DQ, TW>(kt, qf, s, lr, lg);
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        if (jt * 64 < nvis[i]) {
          if (jt * 64 + 64 > nvis[i]) mask_from(s[i], (int)(nvis[i] - jt * 64), lg);
          softmax_step<DV>(s[i], m[i], l[i], o[i], c, stale, use_cmp);
        } else {  // no visible key here: probabilities 0
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) s[i][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      if (use_cmp) pv_tiles<DV, TW>(vt, s, o, lr, lg);
    }
  }
  float inv_l[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) inv_l[i] = l[i] > 0.f ? 1.f / l[i] : 0.f;

  // the gated compressed branch goes to acc now (the window branch adds to
  // it at the end): the registers are needed for the window's state
  if (FWD) {
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      if (!active[i]) continue;
      const float g0 = use_cmp ? gate_of(a, row[i], 0) * inv_l[i] : 0.f;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) *(f32x4*)(acc_frag(a, b * a.T + t[i], g, dt, DV) + 4 * lane) = o[i][dt] * g0;
      if (a.sv_lse)
        save_branch<DV>(a, 0, row[i], use_cmp && l[i] > 0.f, m[i] * a.scale + logf(l[i]), o[i], inv_l[i], lg);
    }
  }

  // ---- pass 2: importance of each visible block, summed over the heads ----
  float mh[TW][4], ih[TW][4];  // per head 4*lg + r: m * c and 1 / l
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      mh[i][r] = __shfl(m[i] * c, 4 * lg + r, 64);
      ih[i][r] = __shfl(inv_l[i], 4 * lg + r, 64);
    }
  if (ntile_cmp > 0) st.load(a.kc, a.nb, 0, nullptr, 0, 0, b, g, a.G, false);
  for (int64_t jt = 0; jt < ntile_cmp; ++jt) {
    __syncthreads();
    st.store(kt, vt, false, false);
    __syncthreads();
    if (jt + 1 < ntile_cmp) st.load(a.kc, a.nb, (jt + 1) * 64, nullptr, 0, 0, b, g, a.G, false);
    if (jt * 64 < nvis[TW - 1] || jt * 64 < nvis[0]) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 s[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DQ / 32; ++ks) {
          const bf16x8 kf = ld8(kt + (16 * nt + lr) * KS + 8 * lg + 32 * ks);
#pragma unroll
          for (int i = 0; i < TW; ++i) s[i] = mfma16(qf[i][ks], kf, s[i]);
        }
        const int64_t blk = jt * 64 + 16 * nt + lr;
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          float v = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) v = fmaf(fast_exp2(fmaf(s[i][r], c, -mh[i][r])), ih[i][r], v);
          v = xor_sum16_32(v);
          if (lg == 0 && blk < nvis[i]) imp[(int64_t)(wave + 8 * i) * a.nbp + blk] = v;
        }
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

  // ---- top-k of each token's row (one wave per row) ----
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    if (!active[i]) continue;
    const float* my_imp = imp + (int64_t)(wave + 8 * i) * a.nbp;
    int32_t* orow = a.idx + ((b * a.T + t[i]) * a.G + g) * a.n;
    float* srow = a.score ? a.score + ((b * a.T + t[i]) * a.G + g) * a.n : nullptr;
    // 64-token selection blocks, complete ones are candidates
    int64_t nsel = (p[i] + 1) / 64;
    if (nsel > a.nbs) nsel = a.nbs;
    if (a.nbs <= 1024) topk_row<16>(my_imp, a.per, nsel, p[i] / 64, a.flags, (int)a.n, orow, srow);
    else topk_row<MAX_NB_LANE>(my_imp, a.per, nsel, p[i] / 64, a.flags, (int)a.n, orow, srow);
  }

  if (!FWD) return;

  // ---- window branch: keys p - w < s <= p, FA-style over the tile ----
  if (use_win) {
    float m2[TW], l2[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      m2[i] = -INFINITY;
      l2[i] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t kb = kb0; kb <= kb1; ++kb) {
      __syncthreads();
      st.store(kt, vt, true, true);
      __syncthreads();
      if (kb + 1 <= kb1) st.load(a.k, a.L, (kb + 1) * 64, a.vT, a.Lp, (kb + 1) * 64, b, g, a.G, true);
      bool on[TW], any = false;
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        on[i] = active[i] && kb * 64 <= p[i] && kb * 64 + 63 > p[i] - a.w;
        any = any || on[i];
      }
      if (any) {
        f32x4 s[TW][4];
        qk_tiles<DQ, TW>(kt, qf, s, lr, lg);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          if (on[i]) {
            if (kb * 64 + 63 > p[i]) mask_from(s[i], (int)(p[i] + 1 - kb * 64), lg);
            if (kb * 64 <= p[i] - a.w) mask_below(s[i], (int)(p[i] - a.w + 1 - kb * 64), lg);
            softmax_step<DV>(s[i], m2[i], l2[i], o[i], c, stale, true);
          } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) s[i][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
        pv_tiles<DV, TW>(vt, s, o, lr, lg);
      }
    }
#pragma unroll
    for (int i = 0; i < TW; ++i) {
      if (!active[i]) continue;
      const float g2 = gate_of(a, row[i], 2) * (l2[i] > 0.f ? 1.f / l2[i] : 0.f);
      f32x4* arow = (f32x4*)(acc_frag(a, b * a.T + t[i], g, 0, DV) + 4 * lane);  // written by this lane above
      f32x4 prev[DV / 16];
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) prev[dt] = arow[64 * dt];
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) arow[64 * dt] = prev[dt] + o[i][dt] * g2;
      if (a.sv_lse)
        save_branch<DV>(a, 2, row[i], l2[i] > 0.f, m2[i] * a.scale + logf(l2[i]), o[i], 1.f / l2[i], lg);
    }
  } else if (a.sv_lse) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
      if (active[i]) save_branch<DV>(a, 2, row[i], false, 0.f, o[i], 0.f, lg);
  }
}

// ---------------------------------------------------------------------------
template <typename TO> __device__ __forceinline__ void store4(TO* p, f32x4 v);
// outputs are written once and never re-read here: non-temporal stores keep
// them from evicting the K/V tiles that other tokens re-use
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) { __builtin_nontemporal_store(v, (f32x4*)p); }
// two blocks of 4 values as one 16-byte piece of bf16
__device__ __forceinline__ void store8_nt(uint16_t* p, f32x4 a, f32x4 b) {
  const u32x4 w = {(uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16),
                   (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16),
                   (uint32_t)f32_to_bf16(b[0]) | ((uint32_t)f32_to_bf16(b[1]) << 16),
                   (uint32_t)f32_to_bf16(b[2]) | ((uint32_t)f32_to_bf16(b[3]) << 16)};
  __builtin_nontemporal_store(w, (u32x4*)p);
}
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

// The XCD (0..7) that takes selection block j of a query at position p:
// blocks are striped over the XCDs (j mod 8), so each XCD's L2 serves one
// eighth of a group's keys and values -- at most 5 MB for a 64k-token
// group, which it holds, where the whole group's 40 MB it would not.
// Block 0, chosen by every query, goes round the XCDs with the query's
// block (and never to the XCD of the query's own block, also always
// chosen), so no XCD gets more than its share.
__device__ __forceinline__ int sel_stripe(int64_t j, int64_t p) {
  return j > 0 ? (int)(j & 7) : (int)((p / 64 + 4) & 7);
}

// Selected branch, part 1: the chosen blocks of one KV group that lie in
// one XCD's stripe, streamed straight from global memory as 32-key chunks
// (16 heads x 32 keys per matrix op, fp32 online softmax), one partial
// result per (token, group, stripe): the normalised output of the 16 heads
// (bf16) and its log-sum-exp (log2 units of the scaled logits; -inf when
// the stripe holds none of the token's blocks).
//   Workgroup i runs on XCD i % 8 (the dispatcher deals workgroups to the 8
// XCDs in turn) and takes a tile of 4 * kSelTokPerWave tokens of group
// i / (8 ntiles): every XCD sweeps the groups one after another, so its L2
// holds one group's stripe at a time.  Each wave walks kSelTokPerWave
// tokens (every 4th of the tile); their index rows are staged in LDS once.
//   The stream is bound by the bytes a wave has in flight (an L2 read under
// this load takes microseconds), so a token's chunks are read two at a time
// (40 KiB) and computed on once they are in, two waves per SIMD, one
// computing while the other waits; the next token's queries are read while
// the current token is worked on.  K and V come from the fragment-order
// images (nsa_frag.h): each read instruction fetches 1 KiB in lane order.
// Partial layout: part_o [(row, group)][stripe][DV / 32][64 lanes][8]: lane
// (lr, lg)'s 16 bytes of pair q hold dims 32 q + 4 lg .. + 3 and 32 q + 16 +
// 4 lg .. + 3 of head lr (its output blocks 2 q and 2 q + 1), so each store
// and each of the merge's loads moves 1 KiB contiguous; part_l [(row,
// group)][16 heads][8 stripes].
constexpr int kSelTokPerWave = 16;
constexpr int kSelMaxTopK = 32;

template <int DQ, int DV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) k_sel_part(PfArgs a, bool use_slc) {
  __shared__ int sidx[4][kSelTokPerWave * kSelMaxTopK];
  __shared__ __align__(16) uint16_t sblk[64 * (DQ + DV)];  // the staged block: K chunks, then V chunks
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int x = (int)(blockIdx.x & 7);
  constexpr int TILE = 4 * kSelTokPerWave;
  const int64_t BT = a.B * a.T;
  const int64_t nq = (BT + TILE - 1) / TILE;
  const int64_t li = blockIdx.x >> 3;
  if (li >= a.G * nq) return;  // the whole workgroup
  const int64_t g = li / nq;
  const int64_t nc = a.Lp / 32;

  // The block every token of the tile chooses that falls in this stripe --
  // the query's own block (stripe j mod 8) or block 0 (stripe of the own
  // block + 4), taken from the tile's first token -- is read once into LDS
  // and served from there to every token that chose it (same batch row).
  const int64_t tf = (li % nq) * TILE;
  const int64_t bs0 = tf / a.T;
  const int64_t cb0 = (a.L - a.T + tf % a.T) / 64;
  int64_t stage_j = -1;
  if (use_slc) stage_j = (cb0 > 0 && x == (int)(cb0 & 7)) ? cb0 : (x == (int)((cb0 + 4) & 7) ? 0 : -1);
  if (stage_j >= 0) {
    const uint16_t* ks = a.kF + ((bs0 * a.G + g) * nc + 2 * stage_j) * frag_chunk(DQ);
    const uint16_t* vs = a.vF + ((bs0 * a.G + g) * nc + 2 * stage_j) * frag_chunk(DV);
    constexpr int NK = 64 * DQ / 8, NV = 64 * DV / 8;  // 16-byte pieces (two chunks each)
    u32x4 r[(NK + NV + 255) / 256];
#pragma unroll
    for (int i = 0; i < (NK + NV + 255) / 256; ++i) {
      const int c = (int)threadIdx.x + 256 * i;
      if (c < NK) r[i] = *(const u32x4*)(ks + (c / (NK / 2)) * frag_chunk(DQ) + 8 * (c % (NK / 2)));
      else if (c < NK + NV)
        r[i] = *(const u32x4*)(vs + ((c - NK) / (NV / 2)) * frag_chunk(DV) + 8 * ((c - NK) % (NV / 2)));
    }
#pragma unroll
    for (int i = 0; i < (NK + NV + 255) / 256; ++i) {
      const int c = (int)threadIdx.x + 256 * i;
      if (c < NK + NV) *(u32x4*)(sblk + 8 * c) = r[i];
    }
  }
  __syncthreads();

  const int64_t tg0 = tf + wave;  // token k of this wave: flat (b, t) = tg0 + 4k
  if (tg0 >= BT) return;
  const int ntok = (int)min((int64_t)kSelTokPerWave, (BT - tg0 + 3) / 4);
  const int n = (int)a.n;
  const float c = a.scale * kLog2e;
  const float stale = kStaleLog2 / c;
  auto tg_of = [&](int k) { return tg0 + 4 * (int64_t)k; };
  auto write_lse = [&](int64_t rg, float v) {
    if (lg == 0) a.part_l[(rg * 16 + lr) * 8 + x] = v;
  };

  // the index rows of the wave's tokens, staged in LDS
  int* my_idx = sidx[wave];
  for (int f = lane; f < ntok * n; f += 64) my_idx[f] = a.idx[(tg_of(f / n) * a.G + g) * n + f % n];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

  const uint32_t lofs = 16 * lane;  // fragment-order images: lane l's piece of each operand
  // queries of token k (qf) and of token k + 1 (qn, read while token k is
  // worked on; the last token's are read twice)
  bf16x8 qf[DQ / 32], qn[DQ / 32];
  auto load_q = [&](bf16x8 (&qd)[DQ / 32], int k) {  // from the fragment-order image: 1 KiB per load
    const uint16_t* qr = a.qF + (tg_of(k) * a.G + g) * 16 * DQ + 8 * lane;
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks)
      qd[ks] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4*)(qr + 512 * ks)));
  };
  load_q(qn, 0);
  int64_t b = tg0 / a.T, t = tg0 % a.T - 4;  // (b, t) of token k, stepped without divisions
  for (int k = 0; k < ntok; ++k) {
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) qf[ks] = qn[ks];
    t += 4;
    while (t >= a.T) {
      t -= a.T;
      ++b;
    }
    const int64_t p = a.L - a.T + t;
    const int64_t rg = tg_of(k) * a.G + g;
    // lane c: key base of the token's chunk c (slot c / 2, half c % 2) in this stripe, or -1
    const int slot = lane >> 1;
    const int j = slot < n ? my_idx[k * n + slot] : -1;
    const int kbl = j * 64 + 32 * (lane & 1);
    const int kbv = (use_slc && j >= 0 && kbl <= p && sel_stripe(j, p) == x) ? kbl : -1;
    // The block this stripe stages for a tile that starts at this token (its
    // own block, or block 0 in the stripe four on) has its chunks computed
    // after all others -- from LDS when this workgroup staged it -- so the
    // order of the sums, and the result, does not depend on where tiles
    // start (a batch row run alone gives bit-identical outputs).
    const int64_t cbp = p / 64;
    const int64_t spec = (cbp > 0 && x == (int)(cbp & 7)) ? cbp : (x == (int)((cbp + 4) & 7) ? 0 : -1);
    const bool from_lds = spec == stage_j && b == bs0;
    const bool last_blk = kbv >= 0 && j == spec;
    uint64_t pend = __ballot(kbv >= 0 && !last_blk);
    const uint64_t sm = __ballot(last_blk);  // lanes 2s, 2s + 1 of that block's slot s
    if (!pend && !sm) {
      write_lse(rg, -INFINITY);
      load_q(qn, k + 1 < ntok ? k + 1 : k);
      continue;
    }
    auto take = [&]() -> int {
      if (!pend) return -1;
      const int pos = __ffsll((unsigned long long)pend) - 1;
      pend &= pend - 1;
      return __builtin_amdgcn_readlane(kbv, pos);
    };
    const __amdgpu_buffer_rsrc_t kr =
        make_rsrc(a.kF + (b * a.G + g) * nc * frag_chunk(DQ), (uint32_t)(nc * frag_chunk(DQ) * 2));
    const __amdgpu_buffer_rsrc_t vr =
        make_rsrc(a.vF + (b * a.G + g) * nc * frag_chunk(DV), (uint32_t)(nc * frag_chunk(DV) * 2));
    const __amdgpu_buffer_rsrc_t kz = make_rsrc(a.kF, 0u), vz = make_rsrc(a.vF, 0u);  // zero records

    float m = -INFINITY, l = 0.f;
    f32x4 o[DV / 16];
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bool first = true;
    while (pend) {
      // a batch of two chunks: both read, then both computed (the second
      // one's reads land while the first is computed on)
      const int kb0 = take(), kb1 = take();
      KFrag<DQ> k0, k1;
      VFrag<DV> v0, v1;
      load_k_frag<DQ>(k0, kr, lofs, (uint32_t)((kb0 / 32) * frag_chunk(DQ) * 2));
      load_v_frag<DV>(v0, vr, lofs, (uint32_t)((kb0 / 32) * frag_chunk(DV) * 2));
      load_k_frag<DQ>(k1, kb1 >= 0 ? kr : kz, lofs, kb1 >= 0 ? (uint32_t)((kb1 / 32) * frag_chunk(DQ) * 2) : 0u);
      load_v_frag<DV>(v1, kb1 >= 0 ? vr : vz, lofs, kb1 >= 0 ? (uint32_t)((kb1 / 32) * frag_chunk(DV) * 2) : 0u);
      if (first) load_q(qn, k + 1 < ntok ? k + 1 : k);  // after this batch: its reads are not held up
      first = false;
      f32x4 s0, s1;
      qk_chunk<DQ>(k0, qf, s0, s1);
      pv_chunk<DV>(v0, s0, s1, o, m, l, c, stale, kb0, p, lg);
      if (kb1 >= 0) {
        qk_chunk<DQ>(k1, qf, s0, s1);
        pv_chunk<DV>(v1, s0, s1, o, m, l, c, stale, kb1, p, lg);
      }
    }
    if (first) load_q(qn, k + 1 < ntok ? k + 1 : k);
    // that block's chunks last (its first one holds a key <= p)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (!(sm & (h ? 0xAAAAAAAAAAAAAAAAull : 0x5555555555555555ull))) continue;
      KFrag<DQ> kf;
      VFrag<DV> vf;
      if (from_lds) {
        const uint16_t* kl = sblk + h * 32 * DQ + 8 * lane;
        const uint16_t* vl = sblk + 64 * DQ + h * 32 * DV + 8 * lane;
#pragma unroll
        for (int ks = 0; ks < DQ / 32; ++ks) {
          kf.k0[ks] = *(const bf16x8*)(kl + (2 * ks) * 512);
          kf.k1[ks] = *(const bf16x8*)(kl + (2 * ks + 1) * 512);
        }
#pragma unroll
        for (int dt = 0; dt < DV / 16; ++dt) vf.v[dt] = *(const bf16x8*)(vl + dt * 512);
      } else {
        load_k_frag<DQ>(kf, kr, lofs, (uint32_t)((2 * spec + h) * frag_chunk(DQ) * 2));
        load_v_frag<DV>(vf, vr, lofs, (uint32_t)((2 * spec + h) * frag_chunk(DV) * 2));
      }
      f32x4 s0, s1;
      qk_chunk<DQ>(kf, qf, s0, s1);
      pv_chunk<DV>(vf, s0, s1, o, m, l, c, stale, spec * 64 + 32 * h, p, lg);
    }

    // every chunk holds a key <= p, so l > 0
    const float inv_l = 1.f / l;
    uint16_t* orow = a.part_o + (rg * 8 + x) * 16 * DV + 8 * lane;
#pragma unroll
    for (int q = 0; q < DV / 32; ++q) store8_nt(orow + 512 * q, o[2 * q] * inv_l, o[2 * q + 1] * inv_l);
    write_lse(rg, m * c + __log2f(l));
  }
}

// Stores of 4 values that leave whole cache lines to the L2 to assemble
// (ordinary write-back stores: non-temporal ones of 32-byte pieces would go
// to memory as partial-line writes).
template <typename TO> __device__ __forceinline__ void store4_wb(TO* p, f32x4 v);
template <> __device__ __forceinline__ void store4_wb<float>(float* p, f32x4 v) { *(f32x4*)p = v; }
template <> __device__ __forceinline__ void store4_wb<uint16_t>(uint16_t* p, f32x4 v) {
  *(u32x2*)p = u32x2{(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                     (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
}

// Selected branch, part 2: the stripes' partial results of one (token,
// group) merged by log-sum-exp (their weights are 2^(lse_x - lse), lse the
// log-sum-exp of all of them: one softmax over the union of the chosen
// blocks).  FWD: out = acc + gate * the selected branch (the gated sum of all
// three branches; the training forward also keeps the branch's log-sum-exp
// and output); else out = the selected branch and lse its natural
// log-sum-exp.  Two waves per (token, group), each with half of the dims:
// lane (lr, lg) takes dims 16 dt + 4 lg .. + 3 of head lr, the layout the
// partials were written in.  The wave reads the log-sum-exps and acc, then
// all partials of the stripes that hold chosen blocks at once (two memory
// latencies per wave); a stripe without blocks has weight 0 and its partial
// is neither read nor multiplied.
template <int DV, bool FWD, typename TO>
__global__ void __launch_bounds__(256) k_sel_merge(PfArgs a) {
  constexpr int ND = DV / 32;  // 16-dim column blocks per wave
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t wv = (int64_t)blockIdx.x * 4 + wave;  // (row, group, half)
  if (wv >= 2 * a.B * a.T * a.G) return;
  const int64_t rg = wv >> 1;
  const int hv = (int)(wv & 1);
  const int64_t tg = rg / a.G, g = rg % a.G;
  const int64_t row = tg * a.H + g * 16 + lr;  // (b, t, head)

  const f32x4* lp = (const f32x4*)(a.part_l + (rg * 16 + lr) * 8);
  const f32x4 l0 = lp[0], l1 = lp[1];
  f32x4 accv[ND];
  if (FWD) {
    const float* arow = acc_frag(a, tg, g, hv * ND, DV) + 4 * lane;
#pragma unroll
    for (int i = 0; i < ND; ++i) accv[i] = __builtin_nontemporal_load((const f32x4*)(arow + 256 * i));
  }
  const float lx[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
  // the partials of the stripes that hold chosen blocks (an empty stripe's
  // log-sum-exp is -inf for all 16 heads: the wave skips its loads)
  u32x4 raw[8][ND / 2];  // pair j: this half's output blocks 2 j and 2 j + 1
  const uint16_t* pbase = a.part_o + (rg * 8 * (DV / 32) + hv * (ND / 2)) * 512 + 8 * lane;
#pragma unroll
  for (int x = 0; x < 8; ++x)
#pragma unroll
    for (int j = 0; j < ND / 2; ++j)
      raw[x][j] = lx[x] == -INFINITY
                      ? u32x4{0u, 0u, 0u, 0u}
                      : __builtin_nontemporal_load((const u32x4*)(pbase + ((int64_t)x * (DV / 32) + j) * 512));
  float M = -INFINITY;
#pragma unroll
  for (int x = 0; x < 8; ++x) M = fmaxf(M, lx[x]);
  float W = 0.f, w[8];
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    w[x] = lx[x] == -INFINITY ? 0.f : fast_exp2(lx[x] - M);
    W += w[x];
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const float wx = w[x] * inv;
    const bool on = w[x] > 0.f;
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const uint32_t u0 = raw[x][i / 2][2 * (i % 2)], u1 = raw[x][i / 2][2 * (i % 2) + 1];
      const f32x4 v = {bf16_to_f32((uint16_t)u0), bf16_to_f32((uint16_t)(u0 >> 16)),
                       bf16_to_f32((uint16_t)u1), bf16_to_f32((uint16_t)(u1 >> 16))};
#pragma unroll
      for (int e = 0; e < 4; ++e) o[i][e] += on ? v[e] * wx : 0.f;
    }
  }
  const float lse_nat = W > 0.f ? (M + __log2f(W)) * 0.69314718055994531f : -INFINITY;
  const int64_t dofs = row * DV + 16 * hv * ND + 4 * lg;
  TO* orow = (TO*)a.out + dofs;
  if (FWD) {
    const float g1 = (a.flags & NSA_F_SLC) ? gate_of(a, row, 1) : 0.f;
#pragma unroll
    for (int i = 0; i < ND; ++i) store4_wb<TO>(orow + 16 * i, accv[i] + o[i] * g1);
    if (a.sv_lse) {
      const int64_t nrow = a.B * a.T * a.H;
      if (lg == 0 && hv == 0) a.sv_lse[nrow + row] = lse_nat;
      uint16_t* srow = a.sv_o + nrow * DV + dofs;
#pragma unroll
      for (int i = 0; i < ND; ++i) store4_wb<uint16_t>(srow + 16 * i, o[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < ND; ++i) store4_wb<TO>(orow + 16 * i, o[i]);
    if (a.lse && lg == 0 && hv == 0) a.lse[row] = lse_nat;
  }
}

template <int DQ, int DV, int TW>
hipError_t launch_cmpwin_tw(const PfArgs& a, bool fwd, size_t lds, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.G * ((a.T + 8 * TW - 1) / (8 * TW)));
  if (fwd) {
    auto kern = k_cmpwin<DQ, DV, true, TW>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_cmpwin<DQ, DV, true, TW>", kern, grid, 512, lds, s, a);
  } else {
    auto kern = k_cmpwin<DQ, DV, false, TW>;
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_cmpwin<DQ, DV, false, TW>", kern, grid, 512, lds, s, a);
  }
  return hipGetLastError();
}

// Two tokens per wave where the 16 rows of block importances fit the LDS
// beside the K / V tiles, else one.
template <int DQ, int DV>
hipError_t launch_cmpwin_t(const PfArgs& a, bool fwd, hipStream_t s) {
  constexpr int KS = k_lds_stride<DQ>(), VS = kVtStride;
  const size_t tiles = sizeof(uint16_t) * (64 * KS + (fwd ? DV * VS : 0));
  const size_t lds2 = tiles + sizeof(float) * 16 * a.nbp;
  if (lds2 <= kLdsBytes) return launch_cmpwin_tw<DQ, DV, 2>(a, fwd, lds2, s);
  return launch_cmpwin_tw<DQ, DV, 1>(a, fwd, tiles + sizeof(float) * 8 * a.nbp, s);
}

template <int DQ, int DV>
hipError_t launch_sel_t(const PfArgs& a, bool fwd, bool out_f32, hipStream_t s, Phases* ph) {
  const unsigned grid = (unsigned)(8 * a.G * ((a.B * a.T + 4 * kSelTokPerWave - 1) / (4 * kSelTokPerWave)));
  launch("k_sel_part<DQ, DV>", k_sel_part<DQ, DV>, grid, 256, 0, s, a, !fwd || (a.flags & NSA_F_SLC));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ph) ph->mark();
  const unsigned mgrid = (unsigned)((2 * a.B * a.T * a.G + 3) / 4);
  if (fwd) {
    if (out_f32) launch("k_sel_merge<DV, true, float>", k_sel_merge<DV, true, float>, mgrid, 256, 0, s, a);
    else launch("k_sel_merge<DV, true, uint16_t>", k_sel_merge<DV, true, uint16_t>, mgrid, 256, 0, s, a);
  } else {
    if (out_f32) launch("k_sel_merge<DV, false, float>", k_sel_merge<DV, false, float>, mgrid, 256, 0, s, a);
    else launch("k_sel_merge<DV, false, uint16_t>", k_sel_merge<DV, false, uint16_t>, mgrid, 256, 0, s, a);
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

hipError_t launch_frag_k(const void* k, void* kF, int64_t B, int64_t L, int64_t G, int D, hipStream_t s) {
  const int64_t nc = (L + 63) / 64 * 2;
  const unsigned grid = (unsigned)(B * G * nc);
  if (grid == 0) return hipSuccess;
  launch("k_frag_k", k_frag_k, grid, 256, 0, s, (const uint16_t*)k, (uint16_t*)kF, L, nc, G, D);
  return hipGetLastError();
}

hipError_t launch_frag_q(const void* q, void* qF, int64_t R, int64_t G, int D, hipStream_t s) {
  const int64_t n = R * G * (D / 32) * 64;  // 16-byte pieces
  if (n == 0) return hipSuccess;
  launch("k_frag_q", k_frag_q, (unsigned)((n + 255) / 256), 256, 0, s, (const uint16_t*)q, (uint16_t*)qF, n, D);
  return hipGetLastError();
}

hipError_t launch_frag_v(const void* vT, void* vF, int64_t B, int64_t L, int64_t G, int D, hipStream_t s) {
  const int64_t nc = (L + 63) / 64 * 2;
  const unsigned grid = (unsigned)(B * G * nc);
  if (grid == 0) return hipSuccess;
  launch("k_frag_v", k_frag_v, grid, 256, 0, s, (const uint16_t*)vT, (uint16_t*)vF, nc, D);
  return hipGetLastError();
}

size_t sel_part_o_bytes(const Prob& P) { return (size_t)(P.B * P.T * P.G) * 8 * 16 * (size_t)P.dv * 2; }
size_t sel_part_l_bytes(const Prob& P) { return (size_t)(P.B * P.T * P.G) * 16 * 8 * 4; }

hipError_t launch_group_major(const void* src, void* dst, int64_t B, int64_t L, int64_t G, int D, hipStream_t s) {
  const int64_t Lp = (L + 63) / 64 * 64;
  const unsigned grid = (unsigned)(B * (Lp / 64));
  if (grid == 0) return hipSuccess;
  launch("k_group_major", k_group_major, grid, 256, 0, s, (const uint16_t*)src, (uint16_t*)dst, L, Lp, G, D);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int64_t B, int64_t N, int64_t Np, int64_t G, int D,
                            hipStream_t s) {
  const unsigned grid = (unsigned)(B * G * (Np / 64));
  if (grid == 0) return hipSuccess;
  launch("k_transpose", k_transpose, grid, 256, 0, s, (const uint16_t*)src, (uint16_t*)dst, N, Np, G, D);
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

hipError_t launch_sel(const Prob& P, const PfArgs& a, bool fwd, bool out_f32, hipStream_t s, Phases* ph) {
#define CALL_SEL(DQ, DV) launch_sel_t<DQ, DV>(a, fwd, out_f32, s, ph)
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
