// k_prefill.hip -- matrix-core path of the NSA forward for GQA groups of 16
// query heads and 64-token blocks ([P1] s4 three branches; [P1] s5 the group's
// heads stacked as the matrix M dimension instead of a block of queries).
//
//   k_transpose  V [B, N, G, D] -> V^T [B, G, D, Np] (key-contiguous rows,
//                zero padded to Np = round_up(N, 64)); makes every P.V operand
//                one contiguous load.
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

#include "nsa_mfma.h"
#include "nsa_prefill.h"

namespace nsa {
namespace {

constexpr int TQ = 8;             // tokens (waves) per k_cmpwin workgroup
constexpr int MAX_NB_LANE = 32;   // pooled blocks per lane in the top-k: nb <= 2048

__device__ __forceinline__ float gate_of(const PfArgs& a, int64_t row, int branch) {
  if (!a.gates) return 1.f;
  float x = bf16_to_f32(a.gates[row * 3 + branch]);
  return (a.flags & NSA_F_GATE_LOGITS) ? sigmoid(x) : x;
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
    *(u32x4*)(dst + ((b * G + g) * D + d) * Np + n0 + 8 * k8) = val;
  }
}

// ---------------------------------------------------------------------------
// Stage rows [row0, row0 + 64) of a [B, Nrows, G, DQ] tensor (rows clamped to
// Nrows - 1) into LDS with a padded row stride.
template <int DQ>
__device__ __forceinline__ void stage_rows(uint16_t* lds, const uint16_t* src, int64_t b, int64_t g, int64_t G,
                                           int64_t Nrows, int64_t row0) {
  constexpr int KS = DQ + 8, C = DQ / 8;
  for (int c = threadIdx.x; c < 64 * C; c += blockDim.x) {
    const int r = c / C, c8 = c % C;
    int64_t row = row0 + r;
    if (row > Nrows - 1) row = Nrows - 1;
    *(u32x4*)(lds + r * KS + 8 * c8) = *(const u32x4*)(src + ((b * Nrows + row) * G + g) * DQ + 8 * c8);
  }
}

// Stage columns [col0, col0 + 64) of a transposed [B, G, DV, Np] tensor.
template <int DV>
__device__ __forceinline__ void stage_cols(uint16_t* lds, const uint16_t* srcT, int64_t b, int64_t g, int64_t G,
                                           int64_t Np, int64_t col0) {
  constexpr int VS = 64 + 8;
  for (int c = threadIdx.x; c < DV * 8; c += blockDim.x) {
    const int d = c / 8, c8 = c % 8;
    *(u32x4*)(lds + d * VS + 8 * c8) = *(const u32x4*)(srcT + ((b * G + g) * DV + d) * Np + col0 + 8 * c8);
  }
}

// One 64-key online-softmax step for one token (16 heads) of one wave.
// s[mt] holds S^T for keys 16*mt + 4*lg + r (raw dot products, masked ones
// already -inf); updates (m, l) of head lr and rescales o.
template <int DV>
__device__ __forceinline__ void softmax_step(f32x4 (&s)[4], float& m, float& l, f32x4 (&o)[DV / 16], float c,
                                             bool with_o) {
  float tmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[mt][r]);
  tmax = xor_max16_32(tmax);
  const float mnew = fmaxf(m, tmax);
  const float alpha = exp2f((m - mnew) * c);
  float rs = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = exp2f((s[mt][r] - mnew) * c);
      s[mt][r] = pv;
      rs += pv;
    }
  rs = xor_sum16_32(rs);
  l = l * alpha + rs;
  m = mnew;
  if (with_o) {
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[dt] *= alpha;
  }
}

// O^T[d, h] += V^T[d, keys] P^T[keys, h] over one 64-key LDS tile.
template <int DV>
__device__ __forceinline__ void pv_tile(const uint16_t* vt, const f32x4 (&pm)[4], f32x4 (&o)[DV / 16], int lr,
                                        int lg) {
  constexpr int VS = 64 + 8;
  const bf16x8 p0 = pack8(pm[0], pm[1]);
  const bf16x8 p1 = pack8(pm[2], pm[3]);
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) {
    const uint16_t* row = vt + (16 * dt + lr) * VS;
    o[dt] = mfma16(ld4x2(row + 4 * lg, row + 16 + 4 * lg), p0, o[dt]);
    o[dt] = mfma16(ld4x2(row + 32 + 4 * lg, row + 48 + 4 * lg), p1, o[dt]);
  }
}

// S^T[key, h] for 64 keys of an LDS tile: s[mt] = K rows 16*mt.. x Q^T.
template <int DQ>
__device__ __forceinline__ void qk_tile_T(const uint16_t* kt, const bf16x8 (&qf)[DQ / 32], f32x4 (&s)[4], int lr,
                                          int lg) {
  constexpr int KS = DQ + 8;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) s[mt] = mfma16(ld8(kt + (16 * mt + lr) * KS + 8 * lg + 32 * ks), qf[ks], s[mt]);
  }
}

// ---------------------------------------------------------------------------
template <int DQ, int DV, bool FWD>
__global__ void __launch_bounds__(TQ * 64) k_cmpwin(PfArgs a) {
  constexpr int KS = DQ + 8, VS = 64 + 8;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* kt = (uint16_t*)smem_raw;                // [64][KS]
  uint16_t* vt = kt + 64 * KS;                       // [DV][VS]
  float* imp = (float*)(vt + (FWD ? DV * VS : 0));   // [TQ][nbp]

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t ntiles = (a.T + TQ - 1) / TQ;
  const int64_t g = blockIdx.x % a.G;
  const int64_t tile = ntiles - 1 - (blockIdx.x / a.G) % ntiles;  // longest rows first
  const int64_t b = blockIdx.x / (a.G * ntiles);
  const int64_t t = tile * TQ + wave;
  const bool active = t < a.T;
  const int64_t t_last = (tile * TQ + TQ - 1 < a.T - 1) ? tile * TQ + TQ - 1 : a.T - 1;
  const int64_t p = a.L - a.T + (active ? t : t_last);
  const int64_t p_first = a.L - a.T + tile * TQ, p_last = a.L - a.T + t_last;
  int64_t nvis = active ? (p + 1) / 64 : 0;
  if (nvis > a.nb) nvis = a.nb;
  int64_t nvis_max = (p_last + 1) / 64;
  if (nvis_max > a.nb) nvis_max = a.nb;
  const float c = a.scale * kLog2e;
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
  for (int64_t jt = 0; jt * 64 < nvis_max; ++jt) {
    __syncthreads();
    stage_rows<DQ>(kt, a.kc, b, g, a.G, a.nb, jt * 64);
    if (use_cmp) stage_cols<DV>(vt, a.vcT, b, g, a.G, a.nbp, jt * 64);
    __syncthreads();
    if (jt * 64 < nvis) {
      f32x4 s[4];
      qk_tile_T<DQ>(kt, qf, s, lr, lg);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (jt * 64 + 16 * mt + 4 * lg + r >= nvis) s[mt][r] = -INFINITY;
      softmax_step<DV>(s, m, l, o, c, use_cmp);
      if (use_cmp) pv_tile<DV>(vt, s, o, lr, lg);
    }
  }
  const float inv_l = l > 0.f ? 1.f / l : 0.f;

  f32x4 fin[DV / 16];
  if (FWD) {
    const float g0 = use_cmp ? gate_of(a, row, 0) * inv_l : 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) fin[dt] = o[dt] * g0;
  }

  // ---- pass 2: importance of each visible block, summed over the heads ----
  float mh[4], ih[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mh[r] = __shfl(m, 4 * lg + r, 64);
    ih[r] = __shfl(inv_l, 4 * lg + r, 64);
  }
  float* my_imp = imp + (int64_t)wave * a.nbp;
  for (int64_t jt = 0; jt * 64 < nvis_max; ++jt) {
    __syncthreads();
    stage_rows<DQ>(kt, a.kc, b, g, a.G, a.nb, jt * 64);
    __syncthreads();
    if (jt * 64 < nvis) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DQ / 32; ++ks) s = mfma16(qf[ks], ld8(kt + (16 * nt + lr) * KS + 8 * lg + 32 * ks), s);
        float v = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v += exp2f((s[r] - mh[r]) * c) * ih[r];
        v = xor_sum16_32(v);
        const int64_t blk = jt * 64 + 16 * nt + lr;
        if (lg == 0 && blk < nvis) my_imp[blk] = v;
      }
    }
  }
  __syncthreads();

  // ---- top-k of this token's row (one wave, registers + wave reductions) ----
  if (active) {
    const int64_t cur = p / 64;
    int forced[2];
    int nf = 0;
    if (a.flags & NSA_F_FORCE_FIRST) forced[nf++] = 0;
    if ((a.flags & NSA_F_FORCE_CURRENT) && !((a.flags & NSA_F_FORCE_FIRST) && cur == 0)) forced[nf++] = (int)cur;
    float vals[MAX_NB_LANE];
#pragma unroll
    for (int i = 0; i < MAX_NB_LANE; ++i) {
      const int64_t j = lane + 64 * i;
      vals[i] = j < nvis ? my_imp[j] : -1.f;
    }
    int ncand = (int)nvis;
    for (int f = 0; f < nf; ++f) {
      if (forced[f] < nvis) {
        --ncand;
#pragma unroll
        for (int i = 0; i < MAX_NB_LANE; ++i)
          if (lane + 64 * i == forced[f]) vals[i] = -1.f;
      }
    }
    const int r_take = ((int)a.n - nf) < ncand ? ((int)a.n - nf) : ncand;
    int cj = -1;
    float cs = -INFINITY;
    for (int f = 0; f < nf; ++f)
      if (lane == f) { cj = forced[f]; cs = INFINITY; }
    for (int round = 0; round < r_take; ++round) {
      float bv = -1.f;
      int bj = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < MAX_NB_LANE; ++i)
        if (vals[i] > bv) { bv = vals[i]; bj = lane + 64 * i; }  // ascending j: first max wins
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oj = __shfl_xor(bj, off, 64);
        if (better(ov, oj, bv, bj)) { bv = ov; bj = oj; }
      }
#pragma unroll
      for (int i = 0; i < MAX_NB_LANE; ++i)
        if (lane + 64 * i == bj) vals[i] = -1.f;
      if (lane == nf + round) { cj = bj; cs = bv; }
    }
    const int cnt = nf + r_take;
    int rank = 0;
    for (int k2 = 0; k2 < cnt; ++k2) rank += (__shfl(cj, k2, 64) < cj) ? 1 : 0;
    int32_t* orow = a.idx + ((b * a.T + t) * a.G + g) * a.n;
    float* srow = a.score ? a.score + ((b * a.T + t) * a.G + g) * a.n : nullptr;
    if (lane < cnt) {
      orow[rank] = cj;
      if (srow) srow[rank] = cs;
    } else if (lane < a.n) {
      orow[lane] = -1;
      if (srow) srow[lane] = -INFINITY;
    }
  }

  if (!FWD) return;

  // ---- window branch: keys p - w < s <= p, FA-style over the tile ----
  if (use_win) {
    float m2 = -INFINITY, l2 = 0.f;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    int64_t lo = p_first - a.w + 1;
    if (lo < 0) lo = 0;
    for (int64_t kb = lo / 64; kb <= p_last / 64; ++kb) {
      __syncthreads();
      stage_rows<DQ>(kt, a.k, b, g, a.G, a.L, kb * 64);
      stage_cols<DV>(vt, a.vT, b, g, a.G, a.Lp, kb * 64);
      __syncthreads();
      if (active && kb * 64 <= p && kb * 64 + 63 > p - a.w) {
        f32x4 s[4];
        qk_tile_T<DQ>(kt, qf, s, lr, lg);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t key = kb * 64 + 16 * mt + 4 * lg + r;
            if (key > p || key <= p - a.w) s[mt][r] = -INFINITY;
          }
        softmax_step<DV>(s, m2, l2, o, c, true);
        pv_tile<DV>(vt, s, o, lr, lg);
      }
    }
    const float g2 = gate_of(a, row, 2) * (l2 > 0.f ? 1.f / l2 : 0.f);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) fin[dt] += o[dt] * g2;
  }

  if (active) {
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) *(f32x4*)(a.acc + row * DV + 16 * dt + 4 * lg) = fin[dt];
  }
}

// ---------------------------------------------------------------------------
template <typename TO> __device__ __forceinline__ void store4(TO* p, f32x4 v);
template <> __device__ __forceinline__ void store4<float>(float* p, f32x4 v) { *(f32x4*)p = v; }
template <> __device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 v) {
  u32x2 w = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
             (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
  *(u32x2*)p = w;
}

template <int DQ, int DV, bool FWD, typename TO>
__global__ void __launch_bounds__(256) k_sel(PfArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t g = blockIdx.x % a.G;
  const int64_t tg = (blockIdx.x / a.G) * 4 + wave;  // flat (b, t)
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
    for (int ks = 0; ks < DQ / 32; ++ks) qf[ks] = ld8(qr + 32 * ks);
  }
  const int iv = lane < a.n ? a.idx[((b * a.T + t) * a.G + g) * a.n + lane] : -1;
  const bool use_slc = !FWD || (a.flags & NSA_F_SLC);

  float m = -INFINITY, l = 0.f;
  f32x4 o[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* kg = a.k + g * DQ + 8 * lg;
  const uint16_t* vg = a.vT + ((b * a.G + g) * DV + lr) * a.Lp + 4 * lg;

  for (int slot = 0; use_slc && slot < a.n; ++slot) {
    const int j = __shfl(iv, slot, 64);
    if (j < 0) continue;
    for (int half = 0; half < 2; ++half) {
      const int64_t kb = (int64_t)j * 64 + 32 * half;
      if (kb > p) break;
      int64_t r0 = kb + lr, r1 = kb + 16 + lr;
      if (r0 > a.L - 1) r0 = a.L - 1;
      if (r1 > a.L - 1) r1 = a.L - 1;
      const uint16_t* k0 = kg + (b * a.L + r0) * a.G * DQ;
      const uint16_t* k1 = kg + (b * a.L + r1) * a.G * DQ;
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DQ / 32; ++ks) {
        s0 = mfma16(ld8(k0 + 32 * ks), qf[ks], s0);
        s1 = mfma16(ld8(k1 + 32 * ks), qf[ks], s1);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (kb + 4 * lg + r > p) s0[r] = -INFINITY;
        if (kb + 16 + 4 * lg + r > p) s1[r] = -INFINITY;
        tmax = fmaxf(tmax, fmaxf(s0[r], s1[r]));
      }
      tmax = xor_max16_32(tmax);
      const float mnew = fmaxf(m, tmax);
      const float alpha = exp2f((m - mnew) * c);
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = exp2f((s0[r] - mnew) * c);
        s1[r] = exp2f((s1[r] - mnew) * c);
        rs += s0[r] + s1[r];
      }
      rs = xor_sum16_32(rs);
      l = l * alpha + rs;
      m = mnew;
      const bf16x8 pf = pack8(s0, s1);
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const uint16_t* vr = vg + (int64_t)16 * dt * a.Lp + kb;
        o[dt] = mfma16(ld4x2(vr, vr + 16), pf, o[dt] * alpha);
      }
    }
  }

  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  TO* orow = (TO*)a.out + row * DV + 4 * lg;
  if (FWD) {
    float g1 = 0.f;
    if (a.flags & NSA_F_SLC) g1 = gate_of(a, row, 1) * inv_l;
    const float* arow = a.acc + row * DV + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4<TO>(orow + 16 * dt, *(const f32x4*)(arow + 16 * dt) + o[dt] * g1);
  } else {
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) store4<TO>(orow + 16 * dt, o[dt] * inv_l);
    if (a.lse && lg == 0) a.lse[row] = l > 0.f ? m * a.scale + logf(l) : -INFINITY;
  }
}

template <int DQ, int DV>
hipError_t launch_cmpwin_t(const PfArgs& a, bool fwd, hipStream_t s) {
  constexpr int KS = DQ + 8, VS = 64 + 8;
  const size_t lds = sizeof(uint16_t) * (64 * KS + (fwd ? DV * VS : 0)) + sizeof(float) * TQ * a.nbp;
  const unsigned grid = (unsigned)(a.B * a.G * ((a.T + TQ - 1) / TQ));
  if (fwd) {
    auto kern = k_cmpwin<DQ, DV, true>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kern<<<grid, TQ * 64, lds, s>>>(a);
  } else {
    auto kern = k_cmpwin<DQ, DV, false>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    kern<<<grid, TQ * 64, lds, s>>>(a);
  }
  return hipGetLastError();
}

template <int DQ, int DV>
hipError_t launch_sel_t(const PfArgs& a, bool fwd, bool out_f32, hipStream_t s) {
  const unsigned grid = (unsigned)(a.G * ((a.B * a.T + 3) / 4));
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
  return P.bf16() && P.hpg == 16 && P.bs == 64 && (P.dq == 64 || P.dq == 128 || P.dq == 192) &&
         (P.dv == 64 || P.dv == 128) && nbp <= 64 * MAX_NB_LANE && P.n <= 64;
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
