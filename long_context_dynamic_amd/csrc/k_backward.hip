// k_backward.hip -- matrix-core backward pass of the NSA forward for GQA
// groups of 16 query heads and 64-token blocks ([P1] s4: the gated sum of
// the compressed, selected and window branches; [P1] s6: NSA trains end to
// end, the top-k choice passes no gradient, and the compressed branch's
// output is what carries a training signal to every block).
//
// For a branch with key set S, P = softmax(scale * q.k_s), O = sum_s P v_s,
// gate gamma and upstream gradient dout, the gradients are
//   dgamma = <dout, O>,  dS_s = gamma P_s (<dout, v_s> - dgamma),
//   dq += scale sum_s dS_s k_s,  dk_s += scale dS_s q,  dv_s += gamma P_s dout,
// and the compressed branch's key/value gradients reach each token of block
// j as dk_cmp_j / 64.  The work splits by which side owns the sums:
//
//   images     fragment-order copies of k, v and of the summaries (each
//              matrix-op operand 1 KiB in lane order, nsa_frag.h) and tiled
//              V^T copies, so that the global matrix-op operands below are
//              contiguous reads.
//   k_bwd_qcw  compressed and window branches from the query side: one
//              workgroup per 8 tokens of a group, one wave per token (16
//              heads as the matrix N), the 64-key tiles of K and V rows
//              through LDS once for all 8; per branch a statistics pass
//              (max, sum, sum p * <dout, v>) and a gradient pass that
//              recomputes P and accumulates dq (K^T operands by transposing
//              reads of the K tile).
//   k_bwd_q    the selected branch's dq, one wave per (token, group): its
//              statistics merged from the key side's records, then P
//              recomputed over the chosen blocks streamed from global
//              memory (K^T operands by transposing reads of the wave's LDS
//              copy of each 32-key chunk).
//   lists      for every (group, block), the (token, slot) entries that
//              chose it, in token order (deterministic: per 256-token chunk
//              histograms, column prefix sums, one ordered fill per chunk).
//   k_bwd_kv<KV_STAT>  the selected branch's softmax statistics from the
//              key side: per entry and head the block's max, sum and
//              sum of p * <dout, v> (a 16-byte record), so that the query
//              side never streams the selected blocks twice.
//   k_bwd_kv   one workgroup per 64 keys and a run of queries, 4 waves of 16
//              keys each: queries are taken two tokens (32 head rows) at a
//              time through LDS, and dk^T, dv^T accumulate in registers with
//              the head rows as the contraction.  Window: the keys' own
//              window of queries, written to dk, dv.  Selected: a chunk of
//              a block's token list.  Compressed: a run of tokens against 64
//              summaries.  The last two write partial sums.
//   k_bwd_reduce  one workgroup per 64-token block: window part + the
//              selected partials of the block + the block's summary gradient
//              / 64, in a fixed order.
#include <math.h>

#include "nsa_backward.h"
#include "nsa_frag.h"
#include "nsa_mfma.h"
#include "nsa_paths.h"
#include "nsa_prefill.h"
#include "nsa_tile.h"

namespace nsa {
namespace {

constexpr int kBlk = 64;         // block and selection-block size of this path
constexpr int kCountTok = 256;   // tokens per list-count chunk
constexpr int kListChunk = 256;  // listed tokens per selected-branch workgroup
constexpr int kCmpChunk = 512;   // tokens per compressed-branch workgroup

enum { BR_CMP = 0, BR_SLC = 1, BR_WIN = 2 };

// Compressed branch: token chunk c of summary tile J covers tokens
// [max(c * kCmpChunk, t0), min((c + 1) * kCmpChunk, T)), t0 the first token
// that sees summary 64 * J; an empty range writes no partial.
__host__ __device__ __forceinline__ void cmp_chunk_range(const BwArgs& a, int64_t J, int64_t c, int64_t& lo,
                                                         int64_t& hi) {
  int64_t t0 = (J * 64 + 1) * kBlk - 1 - (a.L - a.T);
  if (t0 < 0) t0 = 0;
  lo = c * kCmpChunk;
  hi = lo + kCmpChunk;
  if (lo < t0) lo = t0;
  if (hi > a.T) hi = a.T;
}

__device__ __forceinline__ uint32_t branch_flag(int br) {
  return br == BR_CMP ? NSA_F_CMP : (br == BR_SLC ? NSA_F_SLC : NSA_F_WIN);
}

__device__ __forceinline__ float gate_val(const BwArgs& a, int64_t row, int br, float* dsig) {
  if (!a.gates) {
    *dsig = 0.f;
    return 1.f;
  }
  const float x = bf16_to_f32(a.gates[row * 3 + br]);
  if (a.flags & NSA_F_GATE_LOGITS) {
    const float s = sigmoid(x);
    *dsig = s * (1.f - s);
    return s;
  }
  *dsig = 1.f;
  return x;
}

// <dout, O_b> for head lr from the training forward's saved normalised
// branch output (bf16); df holds dout dims 32*ks + 8*lg + e of that head.
template <int DV>
__device__ __forceinline__ float saved_dot(const BwArgs& a, int br, int64_t row, int64_t nrow,
                                           const bf16x8 (&df)[DV / 32], int lg) {
  const uint16_t* orow = a.sv_o + (br * nrow + row) * DV + 8 * lg;
  float s = 0.f;
#pragma unroll
  for (int ks = 0; ks < DV / 32; ++ks) {
    const u32x4 o = __builtin_bit_cast(u32x4, ld8(orow + 32 * ks));
    const u32x4 d = __builtin_bit_cast(u32x4, df[ks]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s = fmaf(__uint_as_float(o[e] << 16), __uint_as_float(d[e] << 16), s);
      s = fmaf(__uint_as_float(o[e] & 0xFFFF0000u), __uint_as_float(d[e] & 0xFFFF0000u), s);
    }
  }
  return xor_sum16_32(s);
}

// ---------------------------------------------------------------------------
// Query side.  Chunk c of a branch covers keys kb .. kb + 31 (kb a multiple
// of 32); keys outside [klo, khi] are masked.  S^T tiles s0, s1 hold keys
// kb + 8*lg + r and kb + 8*lg + 4 + r (the interleaved order of load_k).
__device__ __forceinline__ void mask_chunk(f32x4& s0, f32x4& s1, int64_t kb, int64_t klo, int64_t khi, int lg) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t k0 = kb + 8 * lg + r, k1 = k0 + 4;
    if (k0 < klo || k0 > khi) s0[r] = -INFINITY;
    if (k1 < klo || k1 > khi) s1[r] = -INFINITY;
  }
}

template <int DQ>
__device__ __forceinline__ void qk_chunk_b(const KFrag<DQ>& f, const bf16x8 (&qf)[DQ / 32], f32x4& s0, f32x4& s1) {
  s0 = f32x4{0.f, 0.f, 0.f, 0.f};
  s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) {
    s0 = mfma16(f.k0[ks], qf[ks], s0);
    s1 = mfma16(f.k1[ks], qf[ks], s1);
  }
}

// The chunks of branch br for token position p (wave-uniform loop driver).
// Selected chunks come from the lanes' list (lane c: slot c / 2, half c % 2).
struct ChunkIter {
  int br;
  int64_t next, end;      // compressed / window: next chunk start, exclusive end
  uint64_t pending;       // selected: lanes still holding a chunk
  int64_t kbv;            // selected: this lane's chunk start or -1
  int64_t klo, khi;

  __device__ __forceinline__ int64_t pop() {
    if (br == BR_SLC) {
      if (!pending) return -1;
      const int pos = __ffsll((unsigned long long)pending) - 1;
      pending &= pending - 1;
      return __shfl(kbv, pos, 64);
    }
    if (next >= end) return -1;
    const int64_t kb = next;
    next += 32;
    return kb;
  }
};

__device__ __forceinline__ ChunkIter chunks_of(const BwArgs& a, int br, int64_t b, int64_t t, int64_t g, int64_t p,
                                               int lane) {
  ChunkIter it;
  it.br = br;
  it.pending = 0;
  it.kbv = -1;
  it.next = 0;
  it.end = 0;
  if (br == BR_CMP) {
    int64_t nvis = (p + 1) / kBlk;
    if (nvis > a.nb) nvis = a.nb;
    it.end = nvis;
    it.klo = 0;
    it.khi = nvis - 1;
  } else if (br == BR_WIN) {
    int64_t lo = p - a.w + 1;
    if (lo < 0) lo = 0;
    it.next = a.w > 0 ? lo / 32 * 32 : 0;
    it.end = a.w > 0 ? p + 1 : 0;
    it.klo = lo;
    it.khi = p;
  } else {
    const int slot = lane >> 1;
    const int j = slot < a.n ? a.idx[((b * a.T + t) * a.G + g) * a.n + slot] : -1;
    const int64_t kb = (int64_t)j * kBlk + 32 * (lane & 1);
    if (j >= 0 && (int64_t)j * kBlk < a.L && kb <= p) it.kbv = kb;
    it.pending = __ballot(it.kbv >= 0);
    it.klo = 0;
    it.khi = p;
  }
  return it;
}

// The selected branch's dq (its statistics come from the key side's
// records), added to the dq that k_bwd_qcw wrote for the other two branches.
template <int DQ, int DV>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) k_bwd_q(BwArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t g = blockIdx.x % a.G;
  const int64_t tg = (blockIdx.x / a.G) * 4 + wave;  // flat (b, t)
  if (tg >= a.B * a.T) return;
  const int64_t b = tg / a.T, t = tg % a.T;
  const int64_t p = a.L - a.T + t;
  const float c2 = a.scale * kLog2e;
  const int64_t row = tg * a.H + g * 16 + lr;  // (b, t, head lr)
  const int64_t nrow = a.B * a.T * a.H;
  constexpr int KS = DQ + 16;
  __shared__ __align__(16) uint16_t ktile[4][32 * KS];  // per wave: the chunk's 32 K rows
  uint16_t* kt = ktile[wave];

  bf16x8 qf[DQ / 32], df[DV / 32];
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) qf[ks] = ld8(a.q + row * DQ + 8 * lg + 32 * ks);
#pragma unroll
  for (int ks = 0; ks < DV / 32; ++ks) df[ks] = ld8(a.dout + row * DV + 8 * lg + 32 * ks);

  const uint32_t tofs = (lr * 32 + 8 * lg) * 2;
  const int64_t bg = b * a.G + g;
  auto rs = [&](const uint16_t* base, int64_t rows, int D) {
    return make_rsrc(base + bg * rows * D, (uint32_t)(rows * D * 2));
  };

  // ---- statistics of the selected branch: log-sum-exp, <dout, O_b>, gate ----
  float lse[3], dd[3], gam[3];
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    lse[br] = INFINITY;
    dd[br] = 0.f;
    gam[br] = 0.f;
    if (br != BR_SLC) continue;  // the other two: k_bwd_qcw
    float dsig = 0.f;
    if (!(a.flags & branch_flag(br))) {
      if (lg == 0) {
        a.stat[(br * 3 + 0) * nrow + row] = INFINITY;
        a.stat[(br * 3 + 1) * nrow + row] = 0.f;
        a.stat[(br * 3 + 2) * nrow + row] = 0.f;
        if (a.dgates) a.dgates[row * 3 + br] = 0.f;
      }
      continue;
    }
    gam[br] = gate_val(a, row, br, &dsig);
    if (br == BR_SLC && a.sv_lse) {  // the training forward's statistics
      const float lse_nat = a.sv_lse[br * nrow + row];
      if (lse_nat > -INFINITY) {
        lse[br] = lse_nat * kLog2e;
        dd[br] = saved_dot<DV>(a, br, row, nrow, df, lg);
      }
      if (lg == 0) {
        a.stat[(br * 3 + 0) * nrow + row] = lse[br];
        a.stat[(br * 3 + 1) * nrow + row] = dd[br];
        a.stat[(br * 3 + 2) * nrow + row] = gam[br];
        if (a.dgates) a.dgates[row * 3 + br] = dd[br] * dsig;
      }
      continue;
    }
    if (br == BR_SLC) {  // merge the key side's per-block records of this token's entries
      float M = -INFINITY, L = 0.f, U = 0.f;
      for (int i = 0; i < a.n; ++i) {
        const int64_t e = (tg * a.G + g) * a.n + i;
        const int j = a.idx[e];
        if (!(j >= 0 && j < a.nbk && (int64_t)j * kBlk <= p)) continue;  // unlisted: no record
        const f32x4 r = *(const f32x4*)(a.srec + (e * 16 + lr) * 4);
        if (r[0] > M) {
          const float f = fast_exp2(M - r[0]);  // 0 while M is -inf
          L *= f;
          U *= f;
          M = r[0];
        }
        const float f = fast_exp2(r[0] - M);
        L += r[1] * f;
        U += r[2] * f;
      }
      if (L > 0.f) {
        lse[br] = M + __log2f(L);
        dd[br] = U / L;
      }
      if (lg == 0) {
        a.stat[(br * 3 + 0) * nrow + row] = lse[br];
        a.stat[(br * 3 + 1) * nrow + row] = dd[br];
        a.stat[(br * 3 + 2) * nrow + row] = gam[br];
        if (a.dgates) a.dgates[row * 3 + br] = dd[br] * dsig;
      }
      continue;
    }
    const bool cmp = br == BR_CMP;
    const __amdgpu_buffer_rsrc_t kr = cmp ? rs(a.kcG, a.nbp, DQ) : rs(a.kG, a.Lp, DQ);
    const __amdgpu_buffer_rsrc_t vr = cmp ? rs(a.vcT, a.nbp, DV) : rs(a.vT, a.Lp, DV);
    ChunkIter it = chunks_of(a, br, b, t, g, p, lane);
    float m = -INFINITY, l = 0.f;
    f32x4 o[DV / 16];
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t kb = it.pop(); kb >= 0; kb = it.pop()) {
      KFrag<DQ> kf;
      VFrag<DV> vf;
      load_k_frag<DQ>(kf, kr, 16 * lane, (uint32_t)(kb / 32) * 32 * DQ * 2);
      load_v<DV>(vf, vr, tofs, kb);
      f32x4 s0, s1;
      qk_chunk_b<DQ>(kf, qf, s0, s1);
      mask_chunk(s0, s1, kb, it.klo, it.khi, lg);
      float tmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
      tmax = xor_max16_32(tmax);
      if (tmax > m) {  // every chunk holds a visible key, so tmax is finite
        const float alpha = fast_exp2((m - tmax) * c2);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DV / 16; ++dt) o[dt] *= alpha;
        m = tmax;
      }
      const float mc = m * c2;
      float rsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s0[r] = fast_exp2(fmaf(s0[r], c2, -mc));
        s1[r] = fast_exp2(fmaf(s1[r], c2, -mc));
        rsum += s0[r] + s1[r];
      }
      l += xor_sum16_32(rsum);
      const bf16x8 pf = pack8(s0, s1);
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) o[dt] = mfma16(vf.v[dt], pf, o[dt]);
    }
    if (l > 0.f) {
      lse[br] = m * c2 + __log2f(l);
      // o^T: lane holds dims 16*dt + 4*lg + r of head lr
      float s = 0.f;
      const uint16_t* dr = a.dout + row * DV + 4 * lg;
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) {
        const u32x2 w = *(const u32x2*)(dr + 16 * dt);
        s += o[dt][0] * bf16_to_f32((uint16_t)(w.x & 0xFFFF)) + o[dt][1] * bf16_to_f32((uint16_t)(w.x >> 16)) +
             o[dt][2] * bf16_to_f32((uint16_t)(w.y & 0xFFFF)) + o[dt][3] * bf16_to_f32((uint16_t)(w.y >> 16));
      }
      dd[br] = xor_sum16_32(s) / l;
    }
    if (lg == 0) {
      a.stat[(br * 3 + 0) * nrow + row] = lse[br];
      a.stat[(br * 3 + 1) * nrow + row] = dd[br];
      a.stat[(br * 3 + 2) * nrow + row] = gam[br];
      if (a.dgates) a.dgates[row * 3 + br] = dd[br] * dsig;
    }
  }

  // ---- dq: recompute P, dP = dout . v, dS, dq += K^T dS ----
  f32x4 dqa[DQ / 16];
#pragma unroll
  for (int dt = 0; dt < DQ / 16; ++dt) dqa[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int br = 0; br < 3; ++br) {
    if (br != BR_SLC || !(a.flags & branch_flag(br)) || !(lse[br] < INFINITY)) continue;  // uniform per token
    const bool cmp = br == BR_CMP;
    const __amdgpu_buffer_rsrc_t kr = cmp ? rs(a.kcG, a.nbp, DQ) : rs(a.kG, a.Lp, DQ);
    const __amdgpu_buffer_rsrc_t vgr = cmp ? rs(a.vcG, a.nbp, DV) : rs(a.vG, a.Lp, DV);
    ChunkIter it = chunks_of(a, br, b, t, g, p, lane);
    const float lb = lse[br], db = dd[br], gb = gam[br];
    for (int64_t kb = it.pop(); kb >= 0; kb = it.pop()) {
      KFrag<DQ> kf;
      KFrag<DV> vf;
      load_k_frag<DQ>(kf, kr, 16 * lane, (uint32_t)(kb / 32) * 32 * DQ * 2);
      load_k_frag<DV>(vf, vgr, 16 * lane, (uint32_t)(kb / 32) * 32 * DV * 2);
      // the K fragments, back to rows (key - kb) of the wave's LDS tile, so
      // that K^T operands come out of transposing reads
      {
        const int r0 = 8 * (lr >> 2) + (lr & 3);
#pragma unroll
        for (int ks = 0; ks < DQ / 32; ++ks) {
          *(bf16x8*)(kt + r0 * KS + 32 * ks + 8 * lg) = kf.k0[ks];
          *(bf16x8*)(kt + (r0 + 4) * KS + 32 * ks + 8 * lg) = kf.k1[ks];
        }
      }
      f32x4 s0, s1;
      qk_chunk_b<DQ>(kf, qf, s0, s1);
      mask_chunk(s0, s1, kb, it.klo, it.khi, lg);
      f32x4 p0, p1;
      qk_chunk_b<DV>(vf, df, p0, p1);  // dP^T = V dout^T on the same interleaved rows
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e0 = fast_exp2(fmaf(s0[r], c2, -lb)), e1 = fast_exp2(fmaf(s1[r], c2, -lb));
        s0[r] = gb * e0 * (p0[r] - db);
        s1[r] = gb * e1 * (p1[r] - db);
      }
      const bf16x8 dsf = pack8(s0, s1);
#pragma unroll
      for (int dt = 0; dt < DQ / 16; ++dt)
        dqa[dt] = mfma16(ld_vt_pair(kt, 8 * lg, 8 * lg + 4, 16 * dt, KS, lr), dsf, dqa[dt]);
    }
  }
  // dq^T: lane holds dims 16*dt + 4*lg + r of head lr; k_bwd_qcw wrote the rest
  float* dqr = a.dq + row * DQ + 4 * lg;
#pragma unroll
  for (int dt = 0; dt < DQ / 16; ++dt) *(f32x4*)(dqr + 16 * dt) += dqa[dt] * a.scale;
}

// ---------------------------------------------------------------------------
// Compressed and window branches from the query side, for 8 consecutive
// tokens of one group per workgroup (one wave per token): the 64-key tiles of
// K rows and V rows pass through LDS once for all 8.  Per branch a
// statistics pass (max, sum and sum p * <dout, v> online) and a gradient
// pass (dS = gamma P (dP - <dout, O>), dq^T += K^T dS^T with K^T operands by
// transposing reads of the K tile).  Writes dq (the selected branch's part
// is added later), the statistics the key side reads, and dgates.
constexpr int kQTok = 8;

template <int D, int NT>
struct RowStager {  // 64 rows of a [B, N, G, D] tensor, rows clamped to N - 1
  static constexpr int C = 64 * D / 8, PT = (C + NT - 1) / NT, S = D + 16;
  u32x4 r[PT];
  __device__ __forceinline__ void load(const uint16_t* src, int64_t N, int64_t row0, int64_t b, int64_t g, int64_t G) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = threadIdx.x + NT * i;
      if (C % NT == 0 || c < C) {
        int64_t row = row0 + c / (D / 8);
        if (row > N - 1) row = N - 1;
        r[i] = *(const u32x4*)(src + ((b * N + row) * G + g) * D + 8 * (c % (D / 8)));
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst) const {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int c = threadIdx.x + NT * i;
      if (C % NT == 0 || c < C) *(u32x4*)(dst + (c / (D / 8)) * S + 8 * (c % (D / 8))) = r[i];
    }
  }
};

// SAVED: the statistics come from the training forward (a.sv_lse), and the
// first pass over the tiles is compiled out (fewer live registers).
template <int DQ, int DV, bool SAVED>
__global__ void __launch_bounds__(64 * kQTok) k_bwd_qcw(BwArgs a) {
  constexpr int KS = DQ + 16;
  __shared__ __align__(16) uint16_t kt[64 * KS];
  __shared__ __align__(16) uint16_t vr[64 * (DV + 16)];
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t ntt = (a.T + kQTok - 1) / kQTok;
  const int64_t g = blockIdx.x % a.G;
  const int64_t tile = ntt - 1 - (blockIdx.x / a.G) % ntt;  // longest rows first
  const int64_t b = blockIdx.x / (a.G * ntt);
  const int64_t t = tile * kQTok + wave;
  const bool active = t < a.T;
  const int64_t t_last = (tile * kQTok + kQTok - 1 < a.T - 1) ? tile * kQTok + kQTok - 1 : a.T - 1;
  const int64_t p = a.L - a.T + (active ? t : t_last);
  const int64_t p_first = a.L - a.T + tile * kQTok, p_last = a.L - a.T + t_last;
  const int64_t row = ((b * a.T + (active ? t : t_last)) * a.G + g) * 16 + lr;  // (b, t, head lr)
  const int64_t nrow = a.B * a.T * a.H;
  const float c2 = a.scale * kLog2e;

  bf16x8 qf[DQ / 32], df[DV / 32];
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) qf[ks] = ld8(a.q + row * DQ + 8 * lg + 32 * ks);
#pragma unroll
  for (int ks = 0; ks < DV / 32; ++ks) df[ks] = ld8(a.dout + row * DV + 8 * lg + 32 * ks);
  f32x4 dqa[DQ / 16];
#pragma unroll
  for (int dt = 0; dt < DQ / 16; ++dt) dqa[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  RowStager<DQ, 64 * kQTok> sk;
  RowStager<DV, 64 * kQTok> sv;

  // the selected branch's statistics are written by k_bwd_q; when that
  // branch is off, its defaults here
  if (!(a.flags & NSA_F_SLC) && active && lg == 0) {
    a.stat[(BR_SLC * 3 + 0) * nrow + row] = INFINITY;
    a.stat[(BR_SLC * 3 + 1) * nrow + row] = 0.f;
    a.stat[(BR_SLC * 3 + 2) * nrow + row] = 0.f;
    if (a.dgates) a.dgates[row * 3 + BR_SLC] = 0.f;
  }
  for (int br = 0; br < 3; br += 2) {  // BR_CMP, BR_WIN
    const bool on = (a.flags & branch_flag(br)) && (br == BR_CMP ? a.nb > 0 : a.w > 0);
    float dsig = 0.f;
    const float gb = on ? gate_val(a, row, br, &dsig) : 0.f;
    // tiles and this token's visible keys [klo, khi]
    const uint16_t* ksrc = br == BR_CMP ? a.kc : a.k;
    const uint16_t* vsrc = br == BR_CMP ? a.vc : a.v;
    const int64_t N = br == BR_CMP ? a.nb : a.L;
    int64_t j0 = 0, j1 = -1, klo = 0, khi = -1;  // tiles j0 .. j1
    if (on) {
      if (br == BR_CMP) {
        int64_t nvm = (p_last + 1) / kBlk;
        if (nvm > a.nb) nvm = a.nb;
        j1 = (nvm + 63) / 64 - 1;
        int64_t nv = (p + 1) / kBlk;
        if (nv > a.nb) nv = a.nb;
        khi = nv - 1;
      } else {
        int64_t lo = p_first - a.w + 1;
        if (lo < 0) lo = 0;
        j0 = lo / 64;
        j1 = p_last / 64;
        klo = p - a.w + 1 < 0 ? 0 : p - a.w + 1;
        khi = p;
      }
    }
    if (!active) khi = -1;
    // statistics (lb: log-sum-exp in log2 units, db: <dout, O_b>) from the
    // training forward, or from a first pass over the tiles
    constexpr bool saved = SAVED;
    float m = -INFINITY, l = 0.f, u = 0.f, lb = 0.f, db = 0.f;
    bool any = false;
    if (saved && on && active) {
      const float lse_nat = a.sv_lse[br * nrow + row];
      any = lse_nat > -INFINITY;
      if (any) {
        lb = lse_nat * kLog2e;
        db = saved_dot<DV>(a, br, row, nrow, df, lg);
      }
    }
    for (int pass = saved ? 1 : 0; pass < 2; ++pass) {
      if (pass == 1 && !saved) {
        any = on && l > 0.f;
        if (any) {
          lb = m * c2 + __log2f(l);
          db = u / l;
        }
      }
      // every wave stays in the tile loop (it holds barriers); a token with
      // an empty key set computes nothing in the gradient pass
      const bool live = pass == 0 || any;
      if (j1 >= j0) {
        sk.load(ksrc, N, j0 * 64, b, g, a.G);
        sv.load(vsrc, N, j0 * 64, b, g, a.G);
      }
      for (int64_t jt = j0; jt <= j1; ++jt) {
        __syncthreads();
        sk.store(kt);
        sv.store(vr);
        __syncthreads();
        if (jt + 1 <= j1) {
          sk.load(ksrc, N, (jt + 1) * 64, b, g, a.G);
          sv.load(vsrc, N, (jt + 1) * 64, b, g, a.G);
        }
        if (!live || jt * 64 > khi || jt * 64 + 63 < klo) continue;  // nothing visible to this token
        f32x4 s[4], dp[4];
        qk_tile_T<DQ>(kt, qf, s, lr, lg);
        qk_tile_T<DV>(vr, df, dp, lr, lg);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t key = jt * 64 + 16 * mt + 4 * lg + r;
            if (key < klo || key > khi) s[mt][r] = -INFINITY;
          }
        if (pass == 0) {
          float tmax = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) tmax = fmaxf(tmax, fmaxf(fmaxf(s[mt][0], s[mt][1]), fmaxf(s[mt][2], s[mt][3])));
          tmax = xor_max16_32(tmax);
          if (tmax > m) {
            const float alpha = fast_exp2((m - tmax) * c2);
            l *= alpha;
            u *= alpha;
            m = tmax;
          }
          const float mc = m * c2;
          float ls = 0.f, us = 0.f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float e = fast_exp2(fmaf(s[mt][r], c2, -mc));
              ls += e;
              us = fmaf(e, dp[mt][r], us);
            }
          l += xor_sum16_32(ls);
          u += xor_sum16_32(us);
        } else {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[mt][r] = gb * fast_exp2(fmaf(s[mt][r], c2, -lb)) * (dp[mt][r] - db);
          const bf16x8 d01 = pack8(s[0], s[1]), d23 = pack8(s[2], s[3]);
#pragma unroll
          for (int dt = 0; dt < DQ / 16; ++dt) {
            dqa[dt] = mfma16(ld_vt_pair(kt, 4 * lg, 16 + 4 * lg, 16 * dt, KS, lr), d01, dqa[dt]);
            dqa[dt] = mfma16(ld_vt_pair(kt, 32 + 4 * lg, 48 + 4 * lg, 16 * dt, KS, lr), d23, dqa[dt]);
          }
        }
      }
    }
    // statistics for the key side and dgates
    if (active && lg == 0) {
      a.stat[(br * 3 + 0) * nrow + row] = any ? lb : INFINITY;
      a.stat[(br * 3 + 1) * nrow + row] = any ? db : 0.f;
      a.stat[(br * 3 + 2) * nrow + row] = on ? gb : 0.f;
      if (a.dgates) a.dgates[row * 3 + br] = any ? db * dsig : 0.f;
    }
  }
  if (!active) return;
  float* dqr = a.dq + row * DQ + 4 * lg;
#pragma unroll
  for (int dt = 0; dt < DQ / 16; ++dt) *(f32x4*)(dqr + 16 * dt) = dqa[dt] * a.scale;
}

// ---------------------------------------------------------------------------
// Lists of the tokens that chose each (b, g, block).  A token lists block j
// when 0 <= j < nbk and the block starts at or before the token (the
// query's own block, always chosen when forced, may be the partial last one).
__global__ void __launch_bounds__(kCountTok) k_bwd_count(BwArgs a) {
  const int64_t nbs = a.nbk;
  extern __shared__ int32_t hist[];  // [nbs]
  const int64_t c = blockIdx.x % a.nct;
  const int64_t bg = blockIdx.x / a.nct;
  const int64_t g = bg % a.G, b = bg / a.G;
  for (int64_t j = threadIdx.x; j < nbs; j += blockDim.x) hist[j] = 0;
  __syncthreads();
  const int64_t t = c * kCountTok + threadIdx.x;
  if (t < a.T) {
    const int64_t p = a.L - a.T + t;
    const int32_t* ir = a.idx + ((b * a.T + t) * a.G + g) * a.n;
    for (int i = 0; i < a.n; ++i) {
      const int j = ir[i];
      if (j >= 0 && j < nbs && (int64_t)j * kBlk <= p) atomicAdd(&hist[j], 1);
    }
  }
  __syncthreads();
  int32_t* crow = a.cnt + (bg * a.nct + c) * nbs;
  for (int64_t j = threadIdx.x; j < nbs; j += blockDim.x) crow[j] = hist[j];
}

// Per (b, g, block): exclusive prefix of the chunk counts (in place) and the list length.
__global__ void __launch_bounds__(256) k_bwd_colscan(BwArgs a) {
  const int64_t nbs = a.nbk;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, g, j)
  if (i >= a.B * a.G * nbs) return;
  const int64_t j = i % nbs, bg = i / nbs;
  int32_t run = 0;
  for (int64_t c = 0; c < a.nct; ++c) {
    int32_t* x = a.cnt + (bg * a.nct + c) * nbs + j;
    const int32_t v = *x;
    *x = run;
    run += v;
  }
  a.tot[i] = run;
}

// Single workgroup: list starts and first work chunk of every list.
__global__ void __launch_bounds__(1024) k_bwd_scan(BwArgs a, int64_t nl) {
  __shared__ int32_t part_e[1024], part_c[1024];
  const int tid = threadIdx.x;
  const int64_t per = (nl + 1023) / 1024;
  const int64_t lo = tid * per, hi = lo + per < nl ? lo + per : nl;
  int32_t se = 0, sc = 0;
  for (int64_t i = lo; i < hi; ++i) {
    se += a.tot[i];
    sc += (a.tot[i] + kListChunk - 1) / kListChunk;
  }
  part_e[tid] = se;
  part_c[tid] = sc;
  __syncthreads();
  if (tid == 0) {
    int32_t ae = 0, ac = 0;
    for (int i = 0; i < 1024; ++i) {
      const int32_t xe = part_e[i], xc = part_c[i];
      part_e[i] = ae;
      part_c[i] = ac;
      ae += xe;
      ac += xc;
    }
    a.offsets[nl] = ae;
    a.chunk_off[nl] = ac;
  }
  __syncthreads();
  int32_t ae = part_e[tid], ac = part_c[tid];
  for (int64_t i = lo; i < hi; ++i) {
    a.offsets[i] = ae;
    a.chunk_off[i] = ac;
    ae += a.tot[i];
    ac += (a.tot[i] + kListChunk - 1) / kListChunk;
  }
}

// One wave per (b, g, 256-token chunk): tokens in order, one lane per slot;
// the lanes of one token hold distinct blocks, so their cursor updates touch
// distinct words and every list comes out in token order.
__global__ void __launch_bounds__(64) k_bwd_fill(BwArgs a) {
  const int64_t nbs = a.nbk;
  extern __shared__ int32_t cur[];  // [nbs]
  const int64_t c = blockIdx.x % a.nct;
  const int64_t bg = blockIdx.x / a.nct;
  const int64_t g = bg % a.G, b = bg / a.G;
  const int32_t* crow = a.cnt + (bg * a.nct + c) * nbs;
  for (int64_t j = threadIdx.x; j < nbs; j += 64) cur[j] = a.offsets[bg * nbs + j] + crow[j];
  __syncthreads();
  const int lane = threadIdx.x;
  const int64_t t1 = (c + 1) * kCountTok < a.T ? (c + 1) * kCountTok : a.T;
  for (int64_t t = c * kCountTok; t < t1; ++t) {
    const int64_t p = a.L - a.T + t;
    const int j = lane < a.n ? a.idx[((b * a.T + t) * a.G + g) * a.n + lane] : -1;
    if (j >= 0 && j < nbs && (int64_t)j * kBlk <= p)
      a.lists[atomicAdd(&cur[j], 1)] = (int32_t)(((b * a.T + t) * a.G + g) * a.n + lane);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Key side.  Wave w owns keys 16w .. 16w + 15 of the workgroup's 64; in the
// products below a lane holds key lr and head rows 4*lg + r of one token:
//   S  = Q K^T, dP = dout V^T           (A: 16 head rows of one token, from LDS)
//   dv^T += dout^T (gamma P),  dk^T += Q^T dS   (contraction over the 32 head
//          rows of two tokens: A from LDS by transposing reads)
enum { KV_WIN = 0, KV_SLC = 1, KV_CMP = 2, KV_STAT = 3 };
constexpr int kKvWaves = 8;  // waves of the window and compressed key-side workgroups

template <int DQ, int DV>
struct KvLds {
  static constexpr int QS = DQ + 16, DS = DV + 16;  // row strides (bf16): 16-byte row reads conflict-free
  uint16_t qs[2][16 * QS];
  uint16_t ds[2][16 * DS];
};

// NW waves: 16 NW keys per workgroup.  The window and compressed branches
// run 8 waves (128 keys: each staged token pair serves twice the keys), the
// listed selected-branch entries 4 (their keys are one 64-token block).
template <int DQ, int DV, int MODE, int NW>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2))) k_bwd_kv(BwArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int QS = KvLds<DQ, DV>::QS, DS = KvLds<DQ, DV>::DS;
  constexpr int QC = 16 * DQ / 8, DC = 16 * DV / 8;   // 16-byte chunks of one token's q / dout rows
  constexpr int NCH = 2 * (QC + DC);
  constexpr int CPT = (NCH + NT - 1) / NT;
  static_assert(MODE == KV_WIN || MODE == KV_CMP || NW == 4, "listed entries: 4 waves");
  __shared__ __align__(16) KvLds<DQ, DV> sm;
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int br = MODE == KV_WIN ? BR_WIN : (MODE == KV_CMP ? BR_CMP : BR_SLC);
  constexpr bool LISTED = MODE == KV_SLC || MODE == KV_STAT;
  __shared__ f32x4 red[4][2][16];  // KV_STAT: per wave, token and head: max, sum, sum p.dP

  // ---- work item: (b, g), the 64 keys, the query tokens ----
  int64_t b, g, key0;    // key0: first key (token position, or summary id)
  int64_t tfirst = 0, ntok = 0;  // window / compressed: token range
  const int32_t* elist = nullptr;  // selected: this chunk's entries
  int64_t chunk_id = 0;
  if (MODE == KV_WIN) {
    const int64_t ntile = (a.L + 16 * NW - 1) / (16 * NW);
    const int64_t K = blockIdx.x % ntile;
    const int64_t bg = blockIdx.x / ntile;
    g = bg % a.G;
    b = bg / a.G;
    key0 = K * 16 * NW;
    // tokens whose window [p - w + 1, p] meets [key0, key0 + 16 NW - 1]
    int64_t plo = key0, phi = key0 + 16 * NW - 1 + a.w - 1;
    int64_t tlo = plo - (a.L - a.T), thi = phi - (a.L - a.T);
    if (tlo < 0) tlo = 0;
    if (thi > a.T - 1) thi = a.T - 1;
    tfirst = tlo;
    ntok = thi >= tlo ? thi - tlo + 1 : 0;
  } else if (MODE == KV_CMP) {
    // NW / 4 consecutive 64-summary tiles J0, J0 + 1, ..: the token range of
    // the first, which holds every later tile's; wave w writes the partial
    // rows of tile J0 + w / 4 (tiles past the last are not written)
    constexpr int TPW = NW / 4;
    const int64_t nJw = (a.nJ + TPW - 1) / TPW;
    const int64_t c = blockIdx.x % a.nC;
    const int64_t J0 = (blockIdx.x / a.nC) % nJw * TPW;
    const int64_t bg = blockIdx.x / (a.nC * nJw);
    g = bg % a.G;
    b = bg / a.G;
    key0 = J0 * 64;
    chunk_id = (bg * a.nJ + J0 + wave / 4) * a.nC + c;
    int64_t lo, hi;
    cmp_chunk_range(a, J0, c, lo, hi);
    if (hi <= lo) return;  // the reduce skips this chunk by the same rule (for J0 and every later tile)
    tfirst = lo;
    ntok = hi - lo;
  } else {  // KV_SLC, KV_STAT
    const int64_t nl = a.B * a.G * a.nbk;
    const int32_t total = a.chunk_off[nl];
    const int32_t w = (int32_t)blockIdx.x;
    if (w >= total) return;
    int64_t lo = 0, hi = nl;  // chunk_off[lo] <= w < chunk_off[hi]
    while (hi - lo > 1) {
      const int64_t mid = (lo + hi) / 2;
      if (a.chunk_off[mid] <= w) lo = mid;
      else hi = mid;
    }
    const int64_t j = lo % a.nbk, bg = lo / a.nbk;
    g = bg % a.G;
    b = bg / a.G;
    key0 = j * kBlk;
    const int64_t first = a.offsets[lo] + (int64_t)(w - a.chunk_off[lo]) * kListChunk;
    int64_t cnt = a.offsets[lo + 1] - first;
    if (cnt > kListChunk) cnt = kListChunk;
    elist = a.lists + first;
    ntok = cnt;
    chunk_id = w;
  }

  // ---- this wave's 16 keys in registers: B operands K[key lr][dims 8*lg + 32*ks ..] ----
  const int64_t key = key0 + 16 * wave + lr;
  const int64_t nkeys = MODE == KV_CMP ? a.nb : a.L;
  const bool key_ok = key < nkeys;
  const uint16_t* krow = MODE == KV_CMP ? a.kc + ((b * a.nb + key) * a.G + g) * DQ : a.k + ((b * a.L + key) * a.G + g) * DQ;
  const uint16_t* vrow = MODE == KV_CMP ? a.vc + ((b * a.nb + key) * a.G + g) * DV : a.v + ((b * a.L + key) * a.G + g) * DV;
  bf16x8 kf[DQ / 32], vf[DV / 32];
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) kf[ks] = key_ok ? ld8(krow + 8 * lg + 32 * ks) : bf16x8{};
#pragma unroll
  for (int ks = 0; ks < DV / 32; ++ks) vf[ks] = key_ok ? ld8(vrow + 8 * lg + 32 * ks) : bf16x8{};

  f32x4 dkt[DQ / 16], dvt[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DQ / 16; ++dt) dkt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) dvt[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t nrow = a.B * a.T * a.H;
  const float c2 = a.scale * kLog2e;
  const int64_t npair = (ntok + 1) / 2;
  auto token_of = [&](int64_t i) -> int64_t {  // i-th token of the work item, or -1
    if (i >= ntok) return -1;
    return LISTED ? ((int64_t)elist[i] / (a.n * a.G)) % a.T : tfirst + i;
  };

  // register prefetch of one pair: q and dout rows (all threads), stats (per lane)
  u32x4 pre[CPT];
  f32x4 pst[2][3];
  auto fetch = [&](int64_t pi) {
    const int64_t tt[2] = {token_of(2 * pi), token_of(2 * pi + 1)};
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = threadIdx.x + NT * i;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (cc < NCH) {
        const bool isq = cc < 2 * QC;
        const int x = isq ? cc : cc - 2 * QC;
        const int per = isq ? QC : DC;
        const int tok = x / per, rem = x % per;
        const int D = isq ? DQ : DV;
        const int hh = rem / (D / 8), c8 = rem % (D / 8);
        if (tt[tok] >= 0) {
          const int64_t r = (b * a.T + tt[tok]) * a.H + g * 16 + hh;
          val = isq ? *(const u32x4*)(a.q + r * DQ + 8 * c8) : *(const u32x4*)(a.dout + r * DV + 8 * c8);
        }
      }
      pre[i] = val;
    }
    if (MODE != KV_STAT) {
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
#pragma unroll
        for (int f = 0; f < 3; ++f) {
          f32x4 s = {0.f, 0.f, 0.f, 0.f};
          if (tt[tk] >= 0) s = *(const f32x4*)(a.stat + (br * 3 + f) * nrow + (b * a.T + tt[tk]) * a.H + g * 16 + 4 * lg);
          pst[tk][f] = s;
        }
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = threadIdx.x + NT * i;
      if (cc < NCH) {
        const bool isq = cc < 2 * QC;
        const int x = isq ? cc : cc - 2 * QC;
        const int per = isq ? QC : DC;
        const int tok = x / per, rem = x % per;
        const int D = isq ? DQ : DV;
        const int hh = rem / (D / 8), c8 = rem % (D / 8);
        if (isq) *(u32x4*)(sm.qs[tok] + hh * QS + 8 * c8) = pre[i];
        else *(u32x4*)(sm.ds[tok] + hh * DS + 8 * c8) = pre[i];
      }
    }
  };

  if (npair > 0) fetch(0);
  for (int64_t pi = 0; pi < npair; ++pi) {
    const int64_t tt[2] = {token_of(2 * pi), token_of(2 * pi + 1)};
    f32x4 st[2][3];
#pragma unroll
    for (int tk = 0; tk < 2; ++tk)
#pragma unroll
      for (int f = 0; f < 3; ++f) st[tk][f] = pst[tk][f];
    __syncthreads();
    stage();
    __syncthreads();
    if (pi + 1 < npair) fetch(pi + 1);

    if (MODE == KV_STAT) {
#pragma unroll
      for (int tk = 0; tk < 2; ++tk) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DQ / 32; ++ks) s = mfma16(ld8(sm.qs[tk] + lr * QS + 8 * lg + 32 * ks), kf[ks], s);
#pragma unroll
        for (int ks = 0; ks < DV / 32; ++ks) dp = mfma16(ld8(sm.ds[tk] + lr * DS + 8 * lg + 32 * ks), vf[ks], dp);
        const bool vis = key_ok && tt[tk] >= 0 && key <= a.L - a.T + tt[tk];
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // head 4*lg + r: reduce over the wave's 16 keys (the lanes of a row)
          const float z = vis ? s[r] * c2 : -INFINITY;
          const float mx = row_max16(z);
          const float e = vis ? fast_exp2(z - mx) : 0.f;
          const float l = row_sum16(e), u = row_sum16(e * dp[r]);
          if (lr == 0) red[wave][tk][4 * lg + r] = f32x4{mx, l, u, 0.f};
        }
      }
      __syncthreads();
      if (threadIdx.x < 32) {  // combine the four waves: one (token, head) per thread
        const int tk = threadIdx.x >> 4, hh = threadIdx.x & 15;
        const int64_t i = 2 * pi + tk;
        if (i < ntok) {
          float M = -INFINITY;
#pragma unroll
          for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w][tk][hh][0]);
          float L = 0.f, U = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const f32x4 r = red[w][tk][hh];
            const float f = r[0] == -INFINITY ? 0.f : fast_exp2(r[0] - M);
            L += r[1] * f;
            U += r[2] * f;
          }
          *(f32x4*)(a.srec + ((int64_t)elist[i] * 16 + hh) * 4) = f32x4{M, L, U, 0.f};
        }
      }
      continue;
    }

    f32x4 pg[2], dsv[2];
#pragma unroll
    for (int tk = 0; tk < 2; ++tk) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DQ / 32; ++ks) s = mfma16(ld8(sm.qs[tk] + lr * QS + 8 * lg + 32 * ks), kf[ks], s);
#pragma unroll
      for (int ks = 0; ks < DV / 32; ++ks) dp = mfma16(ld8(sm.ds[tk] + lr * DS + 8 * lg + 32 * ks), vf[ks], dp);
      // visibility of key lr for this token
      bool vis = key_ok && tt[tk] >= 0;
      if (vis) {
        const int64_t pp = a.L - a.T + tt[tk];
        if (MODE == KV_WIN) vis = key <= pp && key > pp - a.w;
        else if (LISTED) vis = key <= pp;
        else vis = (key + 1) * kBlk <= pp + 1;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = vis ? fast_exp2(fmaf(s[r], c2, -st[tk][0][r])) : 0.f;
        pg[tk][r] = st[tk][2][r] * pr;
        dsv[tk][r] = pg[tk][r] * (dp[r] - st[tk][1][r]);
      }
    }
    const bf16x8 pgf = pack8(pg[0], pg[1]), dsf = pack8(dsv[0], dsv[1]);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      const u32x2 x0 = ld_tr4(sm.ds[0], 4 * lg, 16 * dt, DS, lr), x1 = ld_tr4(sm.ds[1], 4 * lg, 16 * dt, DS, lr);
      const u32x4 x = {x0.x, x0.y, x1.x, x1.y};
      dvt[dt] = mfma16(__builtin_bit_cast(bf16x8, x), pgf, dvt[dt]);
    }
#pragma unroll
    for (int dt = 0; dt < DQ / 16; ++dt) {
      const u32x2 x0 = ld_tr4(sm.qs[0], 4 * lg, 16 * dt, QS, lr), x1 = ld_tr4(sm.qs[1], 4 * lg, 16 * dt, QS, lr);
      const u32x4 x = {x0.x, x0.y, x1.x, x1.y};
      dkt[dt] = mfma16(__builtin_bit_cast(bf16x8, x), dsf, dkt[dt]);
    }
  }

  // ---- write: lane holds dims 16*dt + 4*lg + r of key lr ----
  if (MODE == KV_STAT) return;
  if (MODE == KV_WIN) {
    if (!key_ok) return;
    float* dkr = a.dk + ((b * a.L + key) * a.G + g) * DQ + 4 * lg;
    float* dvr = a.dv + ((b * a.L + key) * a.G + g) * DV + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DQ / 16; ++dt) *(f32x4*)(dkr + 16 * dt) = dkt[dt] * a.scale;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) *(f32x4*)(dvr + 16 * dt) = dvt[dt];
  } else {
    if (MODE == KV_CMP && key0 / 64 + wave / 4 >= a.nJ) return;  // past the last tile
    float* prow = (MODE == KV_SLC ? a.part_s : a.part_c) + (chunk_id * 64 + 16 * (wave % 4) + lr) * (DQ + DV) + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < DQ / 16; ++dt) *(f32x4*)(prow + 16 * dt) = dkt[dt] * a.scale;
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) *(f32x4*)(prow + DQ + 16 * dt) = dvt[dt];
  }
}

// ---------------------------------------------------------------------------
// Summary gradients: dkc[b, g, j, :] = (sum over the token chunks of j's
// tile, in chunk order) / 64, one thread per (summary, column).
template <int DQ, int DV>
__global__ void __launch_bounds__(256) k_bwd_cmpsum(BwArgs a) {
  constexpr int E = DQ + DV;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // ((b * G + g) * nb + j) * E + e
  if (i >= a.B * a.G * a.nb * E) return;
  const int64_t e = i % E, j = (i / E) % a.nb, bg = i / (E * a.nb);
  const int64_t J = j / 64, jj = j % 64;
  float cm = 0.f;
  for (int64_t c = 0; c < a.nC; ++c) {
    int64_t lo, hi;
    cmp_chunk_range(a, J, c, lo, hi);
    if (hi > lo) cm += a.part_c[(((bg * a.nJ + J) * a.nC + c) * 64 + jj) * E + e];
  }
  a.dkc[i] = cm * (1.f / kBlk);
}

// ---------------------------------------------------------------------------
// dk, dv of each 64-token tile = window part (already in dk, dv when that
// branch is on) + the selected partials of the tile's block, summed in chunk
// order + the block's summary gradient / 64.  Eight workgroups per tile, each
// on one eighth of the 64 x (DQ + DV) elements, so that the long lists (the
// forced first block is chosen by every token) are read by many waves.
constexpr int kReduceSlices = 8;

template <int DQ, int DV>
__global__ void __launch_bounds__(256) k_bwd_reduce(BwArgs a) {
  constexpr int E = DQ + DV;
  constexpr int NE = 64 * E / (256 * kReduceSlices);  // elements per thread (E is a multiple of 64)
  const int64_t ntile = (a.L + 63) / 64;
  const int slice = blockIdx.x % kReduceSlices;
  const int64_t K = (blockIdx.x / kReduceSlices) % ntile;
  const int64_t bg = blockIdx.x / (kReduceSlices * ntile);
  const int64_t g = bg % a.G, b = bg / a.G;
  const bool win = (a.flags & NSA_F_WIN) && a.w > 0;
  const bool slc = (a.flags & NSA_F_SLC) != 0;  // K < nbk always
  const bool cmp = (a.flags & NSA_F_CMP) && K < a.nb;
  const int x0 = slice * (64 * E / kReduceSlices) + threadIdx.x;  // element x0 + 256 m of the tile
  float acc[NE];
#pragma unroll
  for (int m = 0; m < NE; ++m) acc[m] = 0.f;
  if (slc) {
    const int64_t c_lo = a.chunk_off[bg * a.nbk + K], c_hi = a.chunk_off[bg * a.nbk + K + 1];
    int64_t ch = c_lo;
    for (; ch + 1 < c_hi; ch += 2) {  // two chunks' loads in flight
      const float* p0 = a.part_s + ch * 64 * E + x0;
      const float* p1 = p0 + 64 * E;
      float v0[NE], v1[NE];
#pragma unroll
      for (int m = 0; m < NE; ++m) {
        v0[m] = p0[256 * m];
        v1[m] = p1[256 * m];
      }
#pragma unroll
      for (int m = 0; m < NE; ++m) acc[m] += v0[m] + v1[m];
    }
    if (ch < c_hi) {
      const float* p0 = a.part_s + ch * 64 * E + x0;
#pragma unroll
      for (int m = 0; m < NE; ++m) acc[m] += p0[256 * m];
    }
  }
#pragma unroll
  for (int m = 0; m < NE; ++m) {
    const int x = x0 + 256 * m, i = x / E, e = x % E;
    const int64_t s = K * 64 + i;
    if (s >= a.L) continue;
    float* dst = e < DQ ? a.dk + ((b * a.L + s) * a.G + g) * DQ + e : a.dv + ((b * a.L + s) * a.G + g) * DV + (e - DQ);
    const float cm = cmp ? a.dkc[(bg * a.nb + K) * E + e] : 0.f;
    *dst = (win ? *dst : 0.f) + cm + acc[m];
  }
}

// ---------------------------------------------------------------------------
struct BwPlan {
  size_t total = 0;
  size_t kc, vc, kG, vG, vT, kcG, vcG, vcT, dkc, srec, stat, cnt, tot, offsets, chunk_off, lists, part_s, part_c;
};

BwPlan plan(const Prob& P) {
  BwPlan w;
  auto take = [&](size_t bytes) {
    const size_t off = w.total;
    w.total += (bytes + 255) / 256 * 256;
    return off;
  };
  const int64_t Lp = (P.L + 63) / 64 * 64, nbp = (P.nb + 63) / 64 * 64;
  const int64_t nbk = (P.L + kBlk - 1) / kBlk, nct = (P.T + kCountTok - 1) / kCountTok;
  const int64_t nJ = (P.nb + 63) / 64, nC = (P.T + kCmpChunk - 1) / kCmpChunk;
  const int64_t nl = P.B * P.G * nbk;
  const int64_t ne = P.B * P.T * P.G * P.n;
  const int64_t chunks = (ne + kListChunk - 1) / kListChunk + nl;
  w.kc = take(P.B * P.nb * P.G * P.dq * 2);
  w.vc = take(P.B * P.nb * P.G * P.dv * 2);
  w.kG = take(P.B * P.G * Lp * P.dq * 2);
  w.vG = take(P.B * P.G * Lp * P.dv * 2);
  w.vT = take(P.B * P.G * Lp * P.dv * 2);
  w.kcG = take(P.B * P.G * nbp * P.dq * 2);
  w.vcG = take(P.B * P.G * nbp * P.dv * 2);
  w.vcT = take(P.B * P.G * nbp * P.dv * 2);
  w.stat = take((size_t)9 * P.B * P.T * P.H * 4);
  w.srec = take((size_t)(ne > 0 ? ne : 1) * 16 * 16);
  w.cnt = take((size_t)P.B * P.G * nct * nbk * 4);
  w.tot = take((nl + 1) * 4);
  w.offsets = take((nl + 1) * 4);
  w.chunk_off = take((nl + 1) * 4);
  w.lists = take((ne > 0 ? ne : 1) * 4);
  w.part_s = take((size_t)chunks * 64 * (P.dq + P.dv) * 4);
  w.part_c = take((size_t)P.B * P.G * nJ * nC * 64 * (P.dq + P.dv) * 4);
  w.dkc = take((size_t)P.B * P.G * P.nb * (P.dq + P.dv) * 4);
  return w;
}

template <int DQ, int DV>
hipError_t launch_t(const Prob& P, BwArgs& a, hipStream_t s, Phases& ph) {
  const int64_t nl = P.B * P.G * a.nbk;
  const unsigned gq = (unsigned)(P.G * ((P.B * P.T + 3) / 4));
  const bool slc = P.has(NSA_F_SLC);
  const int64_t ne = P.B * P.T * P.G * P.n;
  const int64_t chunks_max = (ne + kListChunk - 1) / kListChunk + nl;  // surplus workgroups exit at once
  if (slc) {
    const size_t lds = (size_t)a.nbk * 4;
    launch("k_bwd_count", k_bwd_count, (unsigned)(P.B * P.G * a.nct), kCountTok, lds, s, a);
    launch("k_bwd_colscan", k_bwd_colscan, (unsigned)((nl + 255) / 256), 256, 0, s, a);
    launch("k_bwd_scan", k_bwd_scan, 1, 1024, 0, s, a, nl);
    launch("k_bwd_fill", k_bwd_fill, (unsigned)(P.B * P.G * a.nct), 64, lds, s, a);
    ph.mark();
    // with the training forward's statistics the group launches nothing
    if (!a.sv_lse) launch("k_bwd_kv<DQ, DV, KV_STAT, 4>", k_bwd_kv<DQ, DV, KV_STAT, 4>, (unsigned)chunks_max, 256, 0, s, a);
    ph.mark();
  }
  const unsigned gqcw = (unsigned)(P.B * P.G * ((P.T + kQTok - 1) / kQTok));
  if (a.sv_lse) launch("k_bwd_qcw<DQ, DV, true>", k_bwd_qcw<DQ, DV, true>, gqcw, 64 * kQTok, 0, s, a);
  else launch("k_bwd_qcw<DQ, DV, false>", k_bwd_qcw<DQ, DV, false>, gqcw, 64 * kQTok, 0, s, a);
  if (slc) launch("k_bwd_q<DQ, DV>", k_bwd_q<DQ, DV>, gq, 256, 0, s, a);
  ph.mark();
  const int64_t ntile = (P.L + 63) / 64;
  if (P.has(NSA_F_WIN) && P.w > 0) {
    launch("k_bwd_kv<DQ, DV, KV_WIN, kKvWaves>", k_bwd_kv<DQ, DV, KV_WIN, kKvWaves>, (unsigned)(P.B * P.G * ((P.L + 16 * kKvWaves - 1) / (16 * kKvWaves))), 64 * kKvWaves, 0, s, a);
    ph.mark();
  }
  if (slc) {
    launch("k_bwd_kv<DQ, DV, KV_SLC, 4>", k_bwd_kv<DQ, DV, KV_SLC, 4>, (unsigned)chunks_max, 256, 0, s, a);
    ph.mark();
  }
  if (P.has(NSA_F_CMP) && P.nb > 0) {
    launch("k_bwd_kv<DQ, DV, KV_CMP, kKvWaves>", k_bwd_kv<DQ, DV, KV_CMP, kKvWaves>, (unsigned)(P.B * P.G * ((a.nJ + kKvWaves / 4 - 1) / (kKvWaves / 4)) * a.nC), 64 * kKvWaves, 0, s, a);
    launch("k_bwd_cmpsum<DQ, DV>", k_bwd_cmpsum<DQ, DV>, (unsigned)((P.B * P.G * P.nb * (DQ + DV) + 255) / 256), 256, 0, s, a);
    ph.mark();
  }
  launch("k_bwd_reduce<DQ, DV>", k_bwd_reduce<DQ, DV>, (unsigned)(P.B * P.G * ntile * kReduceSlices), 256, 0, s, a);
  ph.mark();
  return ph.err != hipSuccess ? ph.err : hipGetLastError();
}

}  // namespace

bool backward_ok(const Prob& P) {
  return P.bf16() && P.hpg == 16 && P.bs == kBlk && P.sb == kBlk && (P.dq == 64 || P.dq == 128 || P.dq == 192) &&
         (P.dv == 64 || P.dv == 128) && P.n <= 32 && P.B * P.T * P.G * P.n < ((int64_t)1 << 31) &&
         P.B * P.T * P.H * 9 < ((int64_t)1 << 31) * 4;
}

size_t backward_workspace_bytes(const Prob& P) { return backward_ok(P) ? plan(P).total : 0; }

int backward_phase_names(const Prob& P, const char** names, int max_names) {
  const char* list[10];
  int n = 0;
  list[n++] = "bwd_images";
  if (P.has(NSA_F_SLC)) {
    list[n++] = "bwd_lists";
    list[n++] = "bwd_kv_selected_stats";
  }
  list[n++] = "bwd_q";
  if (P.has(NSA_F_WIN) && P.w > 0) list[n++] = "bwd_kv_window";
  if (P.has(NSA_F_SLC)) list[n++] = "bwd_kv_selected";
  if (P.has(NSA_F_CMP) && P.nb > 0) list[n++] = "bwd_kv_compressed";
  list[n++] = "bwd_reduce";
  for (int i = 0; i < n && i < max_names; ++i) names[i] = list[i];
  return n;
}

hipError_t run_backward(const Prob& P, const void* q, const void* k, const void* v, const void* gates,
                        const int32_t* idx, const void* dout, const void* saved, float* dq, float* dk, float* dv,
                        float* dgates, void* ws, hipStream_t s, Phases& ph) {
  const BwPlan w = plan(P);
  char* base = (char*)ws;
  BwArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.gates = (const uint16_t*)gates;
  a.idx = idx;
  a.dout = (const uint16_t*)dout;
  uint16_t* kc = (uint16_t*)(base + w.kc);
  uint16_t* vc = (uint16_t*)(base + w.vc);
  a.kc = kc;
  a.vc = vc;
  a.kG = (const uint16_t*)(base + w.kG);
  a.vG = (const uint16_t*)(base + w.vG);
  a.vT = (const uint16_t*)(base + w.vT);
  a.kcG = (const uint16_t*)(base + w.kcG);
  a.vcG = (const uint16_t*)(base + w.vcG);
  a.vcT = (const uint16_t*)(base + w.vcT);
  a.sv_lse = (const float*)saved;
  a.sv_o = saved ? (const uint16_t*)((const char*)saved + saved_lse_bytes(P)) : nullptr;
  a.stat = (float*)(base + w.stat);
  a.srec = (float*)(base + w.srec);
  a.cnt = (int32_t*)(base + w.cnt);
  a.tot = (int32_t*)(base + w.tot);
  a.offsets = (int32_t*)(base + w.offsets);
  a.chunk_off = (int32_t*)(base + w.chunk_off);
  a.lists = (int32_t*)(base + w.lists);
  a.part_s = (float*)(base + w.part_s);
  a.part_c = (float*)(base + w.part_c);
  a.dkc = (float*)(base + w.dkc);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dgates = dgates;
  a.B = P.B; a.T = P.T; a.L = P.L; a.G = P.G; a.H = P.H; a.nb = P.nb;
  a.nbp = (P.nb + 63) / 64 * 64;
  a.Lp = (P.L + 63) / 64 * 64;
  a.n = P.n; a.w = P.w;
  a.nbk = (P.L + kBlk - 1) / kBlk;
  a.nct = (P.T + kCountTok - 1) / kCountTok;
  a.nJ = (P.nb + 63) / 64;
  a.nC = (P.T + kCmpChunk - 1) / kCmpChunk;
  a.flags = P.flags;
  a.scale = P.scale;

  // summaries and the operand images
  ph.mark();
  hipError_t e = launch_pool(P, k, v, kc, vc, s);
  if (e != hipSuccess) return e;
  const int64_t B = P.B, G = P.G;
  if ((e = launch_frag_k(k, (void*)a.kG, B, P.L, G, (int)P.dq, s)) != hipSuccess) return e;
  if ((e = launch_frag_k(v, (void*)a.vG, B, P.L, G, (int)P.dv, s)) != hipSuccess) return e;
  if ((e = launch_transpose(v, (void*)a.vT, B, P.L, a.Lp, G, (int)P.dv, s)) != hipSuccess) return e;
  if (P.nb > 0) {
    if ((e = launch_frag_k(kc, (void*)a.kcG, B, P.nb, G, (int)P.dq, s)) != hipSuccess) return e;
    if ((e = launch_frag_k(vc, (void*)a.vcG, B, P.nb, G, (int)P.dv, s)) != hipSuccess) return e;
    if ((e = launch_transpose(vc, (void*)a.vcT, B, P.nb, a.nbp, G, (int)P.dv, s)) != hipSuccess) return e;
  }
  ph.mark();
#define CALL_BW(DQ, DV) return launch_t<DQ, DV>(P, a, s, ph)
  if (P.dq == 192 && P.dv == 128) CALL_BW(192, 128);
  if (P.dq == 128 && P.dv == 128) CALL_BW(128, 128);
  if (P.dq == 64 && P.dv == 64) CALL_BW(64, 64);
  if (P.dq == 192 && P.dv == 64) CALL_BW(192, 64);
  if (P.dq == 128 && P.dv == 64) CALL_BW(128, 64);
  if (P.dq == 64 && P.dv == 128) CALL_BW(64, 128);
#undef CALL_BW
  return hipErrorInvalidValue;
}

}  // namespace nsa
