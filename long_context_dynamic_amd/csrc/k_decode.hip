// k_decode.hip -- NSA forward for a few query tokens against a long cache
// (decoding, [P1] s6: memory-bound, time set by the KV bytes read, which the
// group-shared selection keeps small).  Same arithmetic as the prefill path,
// reorganised so that many waves stream the cache at once:
//
//   k_dec_fused      one workgroup per (row, group) for the whole step: the
//                    two phases below back to back, with barriers between;
//                    the logits stay in LDS, every wave computes a share of
//                    the importance (waves 1..3 with their first window tile
//                    in flight), waves 1..3 stream the window while wave 0
//                    does the top-k, and the selected and window records
//                    stay in LDS for the merge.
//   k_dec_cmpsel     one workgroup per (row, group): 4 waves share out the
//                    64-summary tiles (compressed-branch logits kept in zbuf
//                    for the importance, a partial softmax-weighted sum of
//                    the value summaries per wave); after a barrier the same
//                    workgroup works out the group importance (each wave the
//                    per-head softmax statistics and a share of the blocks)
//                    and the top-k (one wave).
//   k_dec_attnmerge  one workgroup per (row, group): 4 waves share out the
//                    chosen blocks and the window's blocks (an online softmax
//                    and a record per wave and branch); after a barrier the
//                    log-sum-exp merge of every branch's records, gates,
//                    output.
// Every streaming wave runs the same tile loop: K fragments straight from
// global memory into matrix-op registers, the V tile through LDS (read back
// transposed), the next tile's reads issued before the current softmax, and
// a partial record (max, sum, unnormalised output) at the end.
// A row is one (batch, query) pair at position p = kv_len - q_len + t.
#include <math.h>

#include <type_traits>

#include "nsa_decode.h"
#include "nsa_mfma.h"
#include "nsa_topk.h"

namespace nsa {
namespace {

constexpr int MAX_NB_LANE = 32;  // nb <= 2048
constexpr int MAX_CMP_WAVES = 4;     // compressed-branch waves per (row, group)
constexpr int kAttnWaves = 4;        // selected + window waves per (row, group)
constexpr int kMaxSlotsPerWave = 8;  // chosen blocks per such wave: top_k <= 32

__device__ __forceinline__ float dgate(const DecArgs& a, int64_t hrow, int branch) {
  if (!a.gates) return 1.f;
  float x = bf16_to_f32(a.gates[hrow * 3 + branch]);
  return (a.flags & NSA_F_GATE_LOGITS) ? sigmoid(x) : x;
}

__device__ __forceinline__ bool dbetter(float v, int j, float bv, int bj) {
  return v > bv || (v == bv && j < bj);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads also waits
// for every global access of the wave (its fence covers all memory), which
// would drain a tile prefetched across it; this one leaves such loads in
// flight.  For data handed over in LDS only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// Partial record of one wave: [16 heads][DV] unnormalised outputs, then
// [16] maxima (log2 units) and [16] sums.
template <int DV> constexpr int part_floats() { return 16 * DV + 32; }

// Where a wave writes its partial record: the unnormalised outputs of the 16
// heads (rows os floats apart) and ml = the 16 maxima, then the 16 sums.
struct RecLoc {
  float* o;
  int64_t os;
  float* ml;
};

// Partial record w of (row, group) in global memory.
template <int DV>
__device__ __forceinline__ RecLoc grec(const DecArgs& a, int64_t row, int64_t g, int64_t w) {
  const int64_t nwaves = a.n_cmp_waves + a.n_sel_waves + a.n_win_waves;
  float* r = a.part + ((row * a.G + g) * nwaves + w) * part_floats<DV>();
  return RecLoc{r, DV, r + 16 * DV};
}

// Stream 64-row tiles tile_at(0 .. nt-1) of K [B, N, G, DQ] / V [B, N, G, DV] for
// one (b, g) and the 16 heads in qf; keep rows where ok(row).  Writes scaled
// logits to zrow[h * zstride + row] when zrow is given.  Ends by writing the
// wave's partial record.  WITH_V = false: softmax statistics only, V is never
// read (its output part of the record is left as zeros).
// K fragments go from global memory straight into matrix-op registers; the V
// tile is read as whole rows into registers, passes through the wave's LDS
// region and is read back transposed.  The next tile's reads are in flight
// while the current one is computed on.
// Positions and tile starts are ints: the decoding shapes keep N below 2^31.
template <int DQ, int DV, bool WITH_V, typename TileAt, typename Ok, typename Pre>
__device__ __forceinline__ void stream_tiles(const uint16_t* K, const uint16_t* V, int64_t N, int64_t b, int64_t g,
                                             int64_t G, TileAt tile_at, int nt, Ok ok, const bf16x8 (&qf)[DQ / 32],
                                             float c, uint16_t* myv, float* zrow, int zstride, RecLoc rec,
                                             Pre pre) {
  constexpr int VS = DV + 8;
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  float m = -INFINITY, l = 0.f;
  f32x4 o[DV / 16];
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 kf[4][DQ / 32];
  u32x4 vreg[DV / 8];
  // row 0 of (b, g) and the row pitch; a row past N - 1 (the last tile of
  // a cache whose length is not a multiple of 64) reads row N - 1
  const int nlast = (int)N - 1;
  const int64_t pk = G * DQ, pv = G * DV;
  const uint16_t* K0 = K + (b * N * G + g) * DQ + 8 * lg;
  const uint16_t* V0 = V + (b * N * G + g) * DV + 8 * (lane % (DV / 8));
  auto load_k = [&](int i) {
    const int kb = tile_at(i) * 64;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int r = min(kb + 16 * mt + lr, nlast);
      const uint16_t* kr = K0 + r * pk;
#pragma unroll
      for (int ks = 0; ks < DQ / 32; ++ks) kf[mt][ks] = ld8(kr + 32 * ks);
    }
  };
  auto load_v = [&](int i) {
    const int kb = tile_at(i) * 64;
#pragma unroll
    for (int q = 0; q < DV / 8; ++q) {
      const int r = min(kb + (lane + 64 * q) / (DV / 8), nlast);  // 64 rows x DV/8 chunks
      vreg[q] = *(const u32x4*)(V0 + r * pv);
    }
  };
  auto lds_order = [] {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  };
  if (nt > 0) {
    load_k(0);
    if (WITH_V) load_v(0);
  }
  pre();  // other work of the wave while the first tile's reads are in flight
  // the next tile's reads are issued as soon as this tile's registers are
  // free; the last tile is peeled so no tile is read twice
  auto tile = [&](int i, auto prefetch) {
    constexpr bool PF = decltype(prefetch)::value;
    const int kb = tile_at(i) * 64;
    f32x4 s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < DQ / 32; ++ks) s[mt] = mfma16(kf[mt][ks], qf[ks], s[mt]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (PF) load_k(i + 1);
    if (WITH_V) {
      lds_order();  // the previous tile's V reads are done
#pragma unroll
      for (int q = 0; q < DV / 8; ++q) {
        const int cidx = lane + 64 * q;
        const int r = cidx / (DV / 8), c8 = cidx % (DV / 8);
        *(u32x4*)(myv + r * VS + 8 * c8) = vreg[q];
      }
      __builtin_amdgcn_sched_barrier(0);
      if (PF) load_v(i + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    // s[mt][r]: row kb + 16*mt + 4*lg + r, head lr
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!ok(kb + 16 * mt + 4 * lg + r)) s[mt][r] = -INFINITY;
        tmax = fmaxf(tmax, s[mt][r]);
      }
      // scaled logits, 4 consecutive rows per lane (masked rows hold -inf)
      if (zrow) *(f32x4*)(zrow + lr * zstride + kb + 16 * mt + 4 * lg) = s[mt] * c;
    }
    tmax = xor_max16_32(tmax);
    const float mnew = fmaxf(m, tmax);
    // the bare exp2: weights below 2^-126 of the running maximum's flush to 0
    const float alpha = mnew == -INFINITY ? 1.f : fast_exp2((m - mnew) * c);
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = mnew == -INFINITY ? 0.f : fast_exp2((s[mt][r] - mnew) * c);
        s[mt][r] = pr;
        rs += pr;
      }
    rs = xor_sum16_32(rs);
    l = l * alpha + rs;
    m = mnew;
    if (!WITH_V) return;
    lds_order();
    const bf16x8 p0 = pack8(s[0], s[1]);
    const bf16x8 p1 = pack8(s[2], s[3]);
#pragma unroll
    for (int dt = 0; dt < DV / 16; ++dt) {
      // slot e (< 4) of lane (lr, lg) holds V[row 4*lg + e][d = 16*dt + lr],
      // slots 4.. the rows 16 further on (the key order of p0 / p1)
      const bf16x8 va = ld_vt_pair(myv, 4 * lg, 16 + 4 * lg, 16 * dt, VS, lr);
      const bf16x8 vb = ld_vt_pair(myv, 32 + 4 * lg, 48 + 4 * lg, 16 * dt, VS, lr);
      o[dt] = mfma16(va, p0, o[dt] * alpha);
      o[dt] = mfma16(vb, p1, o[dt]);
    }
  };
  for (int i = 0; i + 1 < nt; ++i) tile(i, std::true_type{});
  if (nt > 0) tile(nt - 1, std::false_type{});
  // o^T: lane holds d = 16*dt + 4*lg + r of head lr
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) *(f32x4*)(rec.o + lr * rec.os + 16 * dt + 4 * lg) = o[dt];
  if (lg == 0) {
    rec.ml[lr] = m == -INFINITY ? -INFINITY : m * c;
    rec.ml[16 + lr] = l;
  }
}

template <int DQ>
__device__ __forceinline__ void load_q(const DecArgs& a, int64_t row, int64_t g, bf16x8 (&qf)[DQ / 32]) {
  const int lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const uint16_t* qr = a.q + (row * a.H + g * 16 + lr) * DQ + 8 * lg;
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) qf[ks] = ld8(qr + 32 * ks);
}

// ---------------------------------------------------------------------------
// The compressed branch of one (row, group) on one wave: every
// n_cmp_waves-th summary tile from its own, logits to zbuf, a partial record.
template <int DQ, int DV, bool WITH_V>
__device__ __forceinline__ void cmp_wave(const DecArgs& a, int64_t row, int64_t g, int wave, uint16_t* myv,
                                         float* zrow, int zstride, RecLoc rec) {
  const int64_t b = row / a.T, t = row % a.T;
  const int64_t p = a.L - a.T + t;
  int64_t nvis = (p + 1) / a.bs;  // visible summaries
  if (nvis > a.nb) nvis = a.nb;
  const int ncw = (int)a.n_cmp_waves;
  const int64_t ntv = (nvis + 63) / 64;  // tiles with a visible summary
  const int nt = ntv > wave ? (int)((ntv - wave + ncw - 1) / ncw) : 0;
  bf16x8 qf[DQ / 32];
  load_q<DQ>(a, row, g, qf);
  stream_tiles<DQ, DV, WITH_V>(a.kc, a.vc, a.nb, b, g, a.G, [&](int i) { return wave + i * ncw; }, nt,
                               [nv = (int)nvis](int j) { return j < nv; }, qf, a.scale * kLog2e, myv, zrow, zstride,
                               rec, [] {});
}

// The chosen blocks of one (row, group) on wave w of kAttnWaves: slots w,
// w + 4, .. of list (the row's n chosen blocks, global memory or LDS; a
// record at rec).
template <int DQ, int DV>
__device__ __forceinline__ void sel_wave(const DecArgs& a, int64_t row, int64_t g, int w, const int32_t* list,
                                         const bf16x8 (&qf)[DQ / 32], uint16_t* myv, RecLoc rec) {
  const int64_t b = row / a.T, t = row % a.T;
  const int64_t p = a.L - a.T + t;
  int sel[kMaxSlotsPerWave];
  int ns = 0;
  if (a.flags & NSA_F_SLC) {
    for (int i = 0; i < kMaxSlotsPerWave; ++i) {
      const int64_t slot = w + kAttnWaves * i;
      const int j = slot < a.n ? list[slot] : -1;
      if (j >= 0 && (int64_t)j * 64 <= p) sel[ns++] = j;
    }
  }
  stream_tiles<DQ, DV, true>(a.k, a.v, a.L, b, g, a.G, [&](int i) { return sel[i]; }, ns,
                             [pi = (int)p](int s) { return s <= pi; }, qf, a.scale * kLog2e, myv, nullptr, 0, rec,
                             [] {});
}

// The window's 64-key tiles first, first + stride, .. of one (row, group)
// (a record at rec; none of them gives an empty record).
// pre(): other work done while the first tile's reads are in flight.
template <int DQ, int DV, typename Pre>
__device__ __forceinline__ void win_wave(const DecArgs& a, int64_t row, int64_t g, int first, int stride,
                                         const bf16x8 (&qf)[DQ / 32], uint16_t* myv, RecLoc rec, Pre pre) {
  const int64_t b = row / a.T, t = row % a.T;
  const int64_t p = a.L - a.T + t;
  int64_t lo = p - a.w + 1;
  if (lo < 0) lo = 0;
  const int64_t kb0 = lo / 64, nwt = ((a.flags & NSA_F_WIN) && a.w > 0) ? p / 64 - kb0 + 1 : 0;
  const int nt = nwt > first ? (int)((nwt - first + stride - 1) / stride) : 0;
  stream_tiles<DQ, DV, true>(a.k, a.v, a.L, b, g, a.G, [&](int i) { return (int)(kb0 + first + stride * i); }, nt,
                             [pi = (int)p, li = (int)lo](int s) { return s <= pi && s >= li; }, qf, a.scale * kLog2e,
                             myv, nullptr, 0, rec, pre);
}

// The group importance of visible summaries j = tid + 256 i of one (row,
// group): each wave works out the per-head softmax statistics from the
// compressed-branch records itself, so no barrier is needed before; imp[j]
// = sum over heads of exp2(z - M) / L.
// The caller holds a barrier before imp is read.  NBL: blocks per lane of
// one wave (nbp <= 64 NBL).
template <int DV, int NBL, typename MlOf>
__device__ __forceinline__ void importance_share(const DecArgs& a, int64_t row, int64_t g, int tid, const float* z,
                                                 int zstride, MlOf ml_of, float* imp) {
  const int lane = tid & 63;
  const int64_t p = a.L - a.T + row % a.T;
  int64_t nvis64 = (p + 1) / a.bs;  // visible summaries
  if (nvis64 > a.nb) nvis64 = a.nb;
  const int nvis = (int)nvis64;
  if (nvis <= 0) return;
  // this thread's logits (z[h * zstride + j]), loaded while the statistics
  // are worked out; j past the visible ones reads the last visible column
  float zv[NBL / 4][16];
#pragma unroll
  for (int i = 0; i < NBL / 4; ++i) {
    const int j = min(tid + 256 * i, nvis - 1);
#pragma unroll
    for (int h = 0; h < 16; ++h) zv[i][h] = z[h * zstride + j];
  }
  // head lane % 16's softmax statistics over the compressed-branch records
  // (each 16-lane group works them out), handed to the whole wave as
  // scalars by v_readlane
  const int hh = lane & 15;
  float M = -INFINITY, L = 0.f;
  for (int w = 0; w < (int)a.n_cmp_waves; ++w) M = fmaxf(M, ml_of(w)[hh]);
  for (int w = 0; w < (int)a.n_cmp_waves; ++w) {
    const float mw = ml_of(w)[hh];
    if (mw != -INFINITY) L = fmaf(exp2f(mw - M), ml_of(w)[16 + hh], L);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float hm[16], hl[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    hm[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), h));
    hl[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv), h));
  }
#pragma unroll
  for (int i = 0; i < NBL / 4; ++i) {
    const int j = tid + 256 * i;
    if (j < nvis) {
      float sum = 0.f;
      // the bare exp2 (no denormal fix-up): terms below 2^-126 of a sum of
      // probabilities change nothing
#pragma unroll
      for (int h = 0; h < 16; ++h) sum += fast_exp2(zv[i][h] - hm[h]) * hl[h];
      imp[j] = sum;
    }
  }
}

// The top-k of one (row, group) from the importance in imp (one wave).
template <int NBL>
__device__ __forceinline__ void topk_part(const DecArgs& a, int64_t row, int64_t g, const float* imp,
                                          int32_t* lsel = nullptr) {
  const int lane = threadIdx.x & 63;
  const int64_t p = a.L - a.T + row % a.T;
  int32_t* orow = a.idx + (row * a.G + g) * a.n;
  float* srow = a.score ? a.score + (row * a.G + g) * a.n : nullptr;
  int cj;
  float cs;
  // 64-token selection blocks of `per` summaries each, complete ones are
  // candidates; importance summed over the summaries
  int64_t nsel = (p + 1) / 64;
  if (nsel > a.nbs) nsel = a.nbs;
  float vals[NBL];
  if (a.per == 1 && nsel > 0) {
    // one summary per selection block: every lane's reads in flight together
    // (blocks past nsel read the last visible one and are then masked)
#pragma unroll
    for (int i = 0; i < NBL; ++i) vals[i] = imp[min(lane + 64 * i, (int)nsel - 1)];
#pragma unroll
    for (int i = 0; i < NBL; ++i) vals[i] = lane + 64 * i < nsel ? vals[i] : -1.f;
  } else {
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const int64_t J = lane + 64 * i;
      float v = -1.f;
      if (J < nsel) {
        v = imp[a.per * J];
        for (int64_t k = 1; k < a.per; ++k) v += imp[a.per * J + k];
      }
      vals[i] = v;
    }
  }
  int cnt;
  if constexpr (NBL <= 16) {
    int nf;
    cnt = topk_wave_keys<NBL>(vals, nsel, p / 64, a.flags, (int)a.n, cj, nf);
    cs = INFINITY;  // forced blocks
    if (srow && lane >= nf && lane < cnt) {
      cs = imp[a.per * cj];
      for (int64_t k = 1; k < a.per; ++k) cs += imp[a.per * cj + k];
    }
  } else {
    cnt = topk_wave<NBL>(vals, nsel, p / 64, a.flags, (int)a.n, cj, cs);
  }
  topk_write(cnt, cj, cs, (int)a.n, orow, srow);
  if (lsel) {  // the same list, ascending, for the workgroup's own use
    int rank = 0;
    for (int k2 = 0; k2 < cnt; ++k2) rank += (__builtin_amdgcn_readlane(cj, k2) < cj) ? 1 : 0;
    if (lane < cnt) lsel[rank] = cj;
    else if (lane < a.n) lsel[lane] = -1;
  }
}

// Importance (every thread of the workgroup, then a barrier) and the top-k
// (wave 0).  Threads 64.. return after the barrier.
template <int DV, int NBL>
__device__ __forceinline__ void select_body(const DecArgs& a, int64_t row, int64_t g, int tid, float* imp) {
  importance_share<DV, NBL>(a, row, g, tid, a.zbuf + (row * a.G + g) * 16 * a.nbp, (int)a.nbp,
                            [&](int w) { return (const float*)grec<DV>(a, row, g, w).ml; }, imp);
  __syncthreads();
  if (tid >= 64) return;
  topk_part<NBL>(a, row, g, imp);
}

// Log-sum-exp merge of each branch's partial records, gates, output.  With
// gates == NULL every enabled branch has weight 1; lse (selected branch only,
// natural log) is written when given.  Every thread of the workgroup calls it
// (it holds a barrier); the 16 x DV/4 output slices are dealt over nthr threads.
constexpr int kMaxRecords = 32;

template <int DV, typename TO, typename RecOf>
__device__ __forceinline__ void merge_body(const DecArgs& a, int64_t row, int64_t g, int tid, int nthr,
                                           float (*coef)[kMaxRecords], float* slse, RecOf rec_of) {
  const int nc = (int)a.n_cmp_waves, ns = (int)a.n_sel_waves, nwaves = nc + ns + (int)a.n_win_waves;
  if (tid < 48) {
    const int hh = tid & 15, br = tid >> 4;  // 0 cmp, 1 sel, 2 win
    const int w0 = br == 0 ? 0 : (br == 1 ? nc : nc + ns), w1 = br == 0 ? nc : (br == 1 ? nc + ns : nwaves);
    float M = -INFINITY;
    for (int w = w0; w < w1; ++w) M = fmaxf(M, rec_of(w).ml[hh]);
    float den = 0.f;
    for (int w = w0; w < w1; ++w) {
      const RecLoc r = rec_of(w);
      const float mw = r.ml[hh];
      const float sc = (M == -INFINITY || mw == -INFINITY) ? 0.f : exp2f(mw - M);
      coef[hh][w] = sc;
      den = fmaf(sc, r.ml[16 + hh], den);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int w = w0; w < w1; ++w) coef[hh][w] *= inv;
    if (br == 1) slse[hh] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
  __syncthreads();
  const bool use_cmp = a.flags & NSA_F_CMP, use_slc = a.flags & NSA_F_SLC;
  const bool use_win = (a.flags & NSA_F_WIN) && a.w > 0;
  for (int it = tid; it < 16 * (DV / 4); it += nthr) {
    const int h = it / (DV / 4), d = 4 * (it % (DV / 4));
    const int64_t hrow = row * a.H + g * 16 + h;
    f32x4 br[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // records in groups of 8 loads in flight (the streaming phase before
    // sets the register budget)
    for (int w0 = 0; w0 < nwaves; w0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (w0 + i < nwaves) {
          const RecLoc r = rec_of(w0 + i);
          v[i] = *(const f32x4*)(r.o + h * r.os + d);
        }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int w = w0 + i;
        if (w < nwaves) br[w < nc ? 0 : (w < nc + ns ? 1 : 2)] += v[i] * coef[h][w];
      }
    }
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    if (use_cmp) out += br[0] * dgate(a, hrow, 0);
    if (use_slc) out += br[1] * dgate(a, hrow, 1);
    if (use_win) out += br[2] * dgate(a, hrow, 2);
    if (sizeof(TO) == 2) {
      u32x2 wv = {(uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16),
                  (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16)};
      *(u32x2*)((uint16_t*)a.out + hrow * DV + d) = wv;
    } else {
      *(f32x4*)((float*)a.out + hrow * DV + d) = out;
    }
  }
  if (a.lse && tid < 16) a.lse[row * a.H + g * 16 + tid] = slse[tid];
}

// The merge of the whole-step kernel in two parts.  merge_prefetch loads a
// thread's global inputs -- the compressed-branch record pieces of its output
// slices and their gates -- before the barrier that ends the streaming, so
// their latency overlaps the slowest wave's last tile; merge_finish weighs
// every record (the others in LDS or, without ZLDS, global memory) and
// writes the output.  Same arithmetic as merge_body.
template <int DV>
struct MergeIn {
  static constexpr int NI = (16 * (DV / 4) + 255) / 256;  // output slices per thread
  f32x4 c[NI][MAX_CMP_WAVES];
  float gt[NI][3];
};

template <int DV, typename RecOf>
__device__ __forceinline__ void merge_prefetch(const DecArgs& a, int64_t row, int64_t g, int tid, RecOf rec_of,
                                               MergeIn<DV>& in) {
  const int nc = (int)a.n_cmp_waves;
#pragma unroll
  for (int i = 0; i < MergeIn<DV>::NI; ++i) {
    const int it = tid + 256 * i;
    if (it >= 16 * (DV / 4)) continue;
    const int h = it / (DV / 4), d = 4 * (it % (DV / 4));
    const int64_t hrow = row * a.H + g * 16 + h;
#pragma unroll
    for (int w = 0; w < MAX_CMP_WAVES; ++w) {
      if (w < nc) {
        const RecLoc r = rec_of(w);
        in.c[i][w] = *(const f32x4*)(r.o + h * r.os + d);
      } else {
        in.c[i][w] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int br = 0; br < 3; ++br) in.gt[i][br] = dgate(a, hrow, br);
  }
}

// rec_of(w): any record; srec_of(w): a selected or window one (w >= nc).
template <int DV, typename TO, typename RecOf, typename SRecOf>
__device__ __forceinline__ void merge_finish(const DecArgs& a, int64_t row, int64_t g, int tid,
                                             float (*coef)[kMaxRecords], float* slse, RecOf rec_of, SRecOf srec_of,
                                             const MergeIn<DV>& in) {
  const int nc = (int)a.n_cmp_waves, ns = (int)a.n_sel_waves, nwaves = nc + ns + (int)a.n_win_waves;
  if (tid < 48) {
    const int hh = tid & 15, br = tid >> 4;  // 0 cmp, 1 sel, 2 win
    const int w0 = br == 0 ? 0 : (br == 1 ? nc : nc + ns), w1 = br == 0 ? nc : (br == 1 ? nc + ns : nwaves);
    float M = -INFINITY;
    for (int w = w0; w < w1; ++w) M = fmaxf(M, rec_of(w).ml[hh]);
    float den = 0.f;
    for (int w = w0; w < w1; ++w) {
      const RecLoc r = rec_of(w);
      const float mw = r.ml[hh];
      const float sc = (M == -INFINITY || mw == -INFINITY) ? 0.f : exp2f(mw - M);
      coef[hh][w] = sc;
      den = fmaf(sc, r.ml[16 + hh], den);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int w = w0; w < w1; ++w) coef[hh][w] *= inv;
    if (br == 1) slse[hh] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
  lds_barrier();
  const bool use_cmp = a.flags & NSA_F_CMP, use_slc = a.flags & NSA_F_SLC;
  const bool use_win = (a.flags & NSA_F_WIN) && a.w > 0;
#pragma unroll
  for (int i = 0; i < MergeIn<DV>::NI; ++i) {
    const int it = tid + 256 * i;
    if (it >= 16 * (DV / 4)) continue;
    const int h = it / (DV / 4), d = 4 * (it % (DV / 4));
    const int64_t hrow = row * a.H + g * 16 + h;
    f32x4 br[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int w = 0; w < MAX_CMP_WAVES; ++w)
      if (w < nc) br[0] += in.c[i][w] * coef[h][w];
    for (int w0 = nc; w0 < nwaves; w0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (w0 + j < nwaves) {
          const RecLoc r = srec_of(w0 + j);
          v[j] = *(const f32x4*)(r.o + h * r.os + d);
        }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int w = w0 + j;
        if (w < nwaves) br[w < nc + ns ? 1 : 2] += v[j] * coef[h][w];
      }
    }
    f32x4 out = {0.f, 0.f, 0.f, 0.f};
    if (use_cmp) out += br[0] * in.gt[i][0];
    if (use_slc) out += br[1] * in.gt[i][1];
    if (use_win) out += br[2] * in.gt[i][2];
    if (sizeof(TO) == 2) {
      u32x2 wv = {(uint32_t)f32_to_bf16(out[0]) | ((uint32_t)f32_to_bf16(out[1]) << 16),
                  (uint32_t)f32_to_bf16(out[2]) | ((uint32_t)f32_to_bf16(out[3]) << 16)};
      *(u32x2*)((uint16_t*)a.out + hrow * DV + d) = wv;
    } else {
      *(f32x4*)((float*)a.out + hrow * DV + d) = out;
    }
  }
  if (a.lse && tid < 16) a.lse[row * a.H + g * 16 + tid] = slse[tid];
}

// ---------------------------------------------------------------------------
// One workgroup of 4 waves per (row, group): the compressed branch (each wave
// with its own LDS V tile), then, after a barrier, the selection.  The waves'
// logits and records go through global memory and are read back by the same
// workgroup (no launch in between).
template <int DQ, int DV, bool WITH_V, int NBL>
__global__ void __launch_bounds__(256) k_dec_cmpsel(DecArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* imp = (float*)smem;                    // [64 * NBL]
  uint16_t* vt = (uint16_t*)(imp + 64 * NBL);   // [4][64 * (DV + 8)] when WITH_V
  const int wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.x % a.G, row = blockIdx.x / a.G;
  if (wave < a.n_cmp_waves)
    cmp_wave<DQ, DV, WITH_V>(a, row, g, wave, vt + (WITH_V ? wave * 64 * (DV + 8) : 0),
                             a.zbuf + (row * a.G + g) * 16 * a.nbp, (int)a.nbp, grec<DV>(a, row, g, wave));
  __syncthreads();
  select_body<DV, NBL>(a, row, g, threadIdx.x, imp);
}

// One workgroup of 4 waves per (row, group): the selected and window blocks,
// a barrier, the merge of every branch's records, gates, output.
template <int DQ, int DV, typename TO>
__global__ void __launch_bounds__(256) k_dec_attnmerge(DecArgs a) {
  __shared__ __align__(16) uint16_t vt[kAttnWaves][64 * (DV + 8)];
  __shared__ float coef[16][kMaxRecords];
  __shared__ float slse[16];
  const int wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.x % a.G, row = blockIdx.x / a.G;
  bf16x8 qf[DQ / 32];
  load_q<DQ>(a, row, g, qf);
  const int64_t nc = a.n_cmp_waves, ns = a.n_sel_waves;
  sel_wave<DQ, DV>(a, row, g, wave, a.idx + (row * a.G + g) * a.n, qf, vt[wave], grec<DV>(a, row, g, nc + wave));
  win_wave<DQ, DV>(a, row, g, wave, kAttnWaves, qf, vt[wave], grec<DV>(a, row, g, nc + ns + wave), [] {});
  __syncthreads();
  merge_body<DV, TO>(a, row, g, threadIdx.x, 256, coef, slse, [&](int w) { return grec<DV>(a, row, g, w); });
}

// The whole decoding step of one (row, group) in one workgroup: compressed
// branch, selection, chosen and window blocks, merge -- three barriers, no
// launch in between, and the (row, group)s of the batch at different phases
// across the chip.  ZLDS: the compressed-branch logits stay in LDS (rows of
// nbp + 4 floats, so the 16 heads' rows start in different banks) instead of
// going through global memory.
template <int DQ, int DV, int NBL, bool ZLDS, typename TO>
__global__ void __launch_bounds__(256) k_dec_fused(DecArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* imp = (float*)smem;                          // [64 * NBL]
  float(*coef)[kMaxRecords] = (float(*)[kMaxRecords])(imp + 64 * NBL);  // [16][kMaxRecords]
  float* slse = (float*)(coef + 16);                  // [16]
  float* mlr = slse + 16;                             // ZLDS: [kMaxRecords][32] record maxima and sums
  int32_t* lsel = (int32_t*)(mlr + kMaxRecords * 32);  // [32] the chosen blocks
  uint16_t* vt = (uint16_t*)(lsel + 32);               // [4][64 * (DV + 8)]
  // ZLDS: the logits [16][nbp + 4]; after the importance the same space
  // holds the selected and window records' outputs [8][16][DV + 4]
  float* zl = (float*)(vt + 4 * 64 * (DV + 8));
  const int wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.x % a.G, row = blockIdx.x / a.G;
  uint16_t* myv = vt + wave * 64 * (DV + 8);
  float* z = ZLDS ? zl : a.zbuf + (row * a.G + g) * 16 * a.nbp;
  const int zstride = (int)(ZLDS ? a.nbp + 4 : a.nbp);
  const int64_t nc = a.n_cmp_waves, ns = a.n_sel_waves;
  // record w: compressed-branch outputs in global memory, the rest in LDS
  auto rec_of = [&](int w) -> RecLoc {
    if (!ZLDS) return grec<DV>(a, row, g, w);
    if (w < nc) return RecLoc{grec<DV>(a, row, g, w).o, DV, mlr + 32 * w};
    return RecLoc{zl + (w - nc) * 16 * (DV + 4), DV + 4, mlr + 32 * w};
  };
  if (wave < nc) cmp_wave<DQ, DV, true>(a, row, g, wave, myv, z, zstride, rec_of(wave));
  __syncthreads();  // the compressed-branch records (global memory) and logits are complete
  bf16x8 qf[DQ / 32];
  load_q<DQ>(a, row, g, qf);
  // every wave computes its share of the importance -- waves 1..3 with
  // their first window tile's reads in flight, which the LDS-only barrier
  // leaves in flight -- then wave 0 makes the top-k while waves 1..3 stream
  // the rest of the window, which does not depend on it (wave 0's window
  // record is empty)
  auto share = [&] {
    importance_share<DV, NBL>(a, row, g, threadIdx.x, z, zstride, [&](int w) { return (const float*)rec_of(w).ml; },
                              imp);
    lds_barrier();
  };
  if (wave == 0) {
    share();
    topk_part<NBL>(a, row, g, imp, lsel);
    win_wave<DQ, DV>(a, row, g, 1 << 30, 1, qf, myv, rec_of(nc + ns), [] {});
  } else {
    win_wave<DQ, DV>(a, row, g, wave - 1, kAttnWaves - 1, qf, myv, rec_of(nc + ns + wave), share);
  }
  lds_barrier();  // the chosen blocks are in lsel
  sel_wave<DQ, DV>(a, row, g, wave, lsel, qf, myv, rec_of(nc + wave));
  MergeIn<DV> min_;
  merge_prefetch<DV>(a, row, g, threadIdx.x, rec_of, min_);
  if (ZLDS) lds_barrier();  // every record is complete (the selected and window ones in LDS)
  else __syncthreads();     // ... in global memory
  // the selected and window records: in LDS with ZLDS (a pointer the
  // compiler sees as LDS), else in global memory
  auto srec_of = [&](int w) -> RecLoc {
    if (!ZLDS) return grec<DV>(a, row, g, w);
    return RecLoc{zl + (w - nc) * 16 * (DV + 4), DV + 4, mlr + 32 * w};
  };
  merge_finish<DV, TO>(a, row, g, threadIdx.x, coef, slse, rec_of, srec_of, min_);
}

template <int DQ, int DV, typename TO>
hipError_t launch_fused(const DecArgs& a, hipStream_t s) {
  const size_t fixed = (16 * kMaxRecords + 16 + kMaxRecords * 32 + 32) * 4 + (size_t)4 * 64 * (DV + 8) * 2;
  if (a.nbp <= 1024) {  // logits, then 8 records, in LDS: at most 66 KiB more
    auto k = k_dec_fused<DQ, DV, 16, true, TO>;
    const size_t zbytes = (size_t)16 * (a.nbp + 4) * 4, rbytes = (size_t)8 * 16 * (DV + 4) * 4;
    const size_t lds = 64 * 16 * 4 + fixed + (zbytes > rbytes ? zbytes : rbytes);
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_dec_fused<DQ, DV, 16, true, TO>", k, (unsigned)(a.R * a.G), 256, lds, s, a);
  } else {
    auto k = k_dec_fused<DQ, DV, MAX_NB_LANE, false, TO>;
    const size_t lds = 64 * MAX_NB_LANE * 4 + fixed;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_dec_fused<DQ, DV, MAX_NB_LANE, false, TO>", k, (unsigned)(a.R * a.G), 256, lds, s, a);
  }
  return hipGetLastError();
}

template <int DQ, int DV, bool WITH_V>
hipError_t launch_cmpsel(const DecArgs& a, hipStream_t s) {
  const size_t vbytes = WITH_V ? (size_t)4 * 64 * (DV + 8) * 2 : 0;
  if (a.nbp <= 1024) {
    auto k = k_dec_cmpsel<DQ, DV, WITH_V, 16>;
    const size_t lds = 64 * 16 * 4 + vbytes;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_dec_cmpsel<DQ, DV, WITH_V, 16>", k, (unsigned)(a.R * a.G), 256, lds, s, a);
  } else {
    auto k = k_dec_cmpsel<DQ, DV, WITH_V, MAX_NB_LANE>;
    const size_t lds = 64 * MAX_NB_LANE * 4 + vbytes;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    launch("k_dec_cmpsel<DQ, DV, WITH_V, MAX_NB_LANE>", k, (unsigned)(a.R * a.G), 256, lds, s, a);
  }
  return hipGetLastError();
}

// mode: 0 selection only, 1 whole forward, 2 selected branch on a given idx
template <int DQ, int DV>
hipError_t run_t(const DecArgs& a, int mode, bool out_f32, hipStream_t s, Phases* ph) {
  hipError_t e;
  if (mode == 0) {
    // selection only: the value summaries are not an input (and not read)
    e = launch_cmpsel<DQ, DV, false>(a, s);
  } else if (mode == 1) {
    e = out_f32 ? launch_fused<DQ, DV, float>(a, s) : launch_fused<DQ, DV, uint16_t>(a, s);
  } else {
    if (out_f32) launch("k_dec_attnmerge<DQ, DV, float>", k_dec_attnmerge<DQ, DV, float>, (unsigned)(a.R * a.G), 256, 0, s, a);
    else launch("k_dec_attnmerge<DQ, DV, uint16_t>", k_dec_attnmerge<DQ, DV, uint16_t>, (unsigned)(a.R * a.G), 256, 0, s, a);
    e = hipGetLastError();
  }
  if (ph) ph->mark();
  return e;
}

}  // namespace

void decode_layout(const Prob& P, int64_t* n_cmp_waves, int64_t* n_sel_waves, int64_t* n_win_waves) {
  const int64_t nbp = (P.nb + 63) / 64 * 64;
  // the summary tiles dealt round-robin over at most 4 waves; the chosen
  // blocks and the window's blocks round-robin over 4 waves, one record each
  *n_cmp_waves = nbp / 64 < MAX_CMP_WAVES ? nbp / 64 : MAX_CMP_WAVES;
  if (*n_cmp_waves < 1) *n_cmp_waves = 1;
  *n_sel_waves = kAttnWaves;
  *n_win_waves = kAttnWaves;
}

bool decode_ok(const Prob& P) {
  const int64_t nbp = (P.nb + 63) / 64 * 64;
  if (!(P.bf16() && P.hpg == 16 && P.sb == 64 && (P.bs == 64 || P.bs == 32 || P.bs == 16) && P.T <= 8 &&
        (P.dq == 64 || P.dq == 128 || P.dq == 192) &&
        (P.dv == 64 || P.dv == 128) && nbp <= 64 * MAX_NB_LANE && P.n <= 32 && P.n >= 1))
    return false;
  int64_t nc, ns, nw;
  decode_layout(P, &nc, &ns, &nw);
  return nc + ns + nw <= 32;  // partial records one merge workgroup weighs
}

size_t decode_part_bytes(const Prob& P) {
  int64_t nc, ns, nw;
  decode_layout(P, &nc, &ns, &nw);
  return (size_t)(P.B * P.T * P.G * (nc + ns + nw) * (16 * P.dv + 32)) * sizeof(float);
}

hipError_t launch_decode(const Prob& P, DecArgs a, int mode, bool out_f32, hipStream_t s, Phases* ph) {
  decode_layout(P, &a.n_cmp_waves, &a.n_sel_waves, &a.n_win_waves);
#define CALL_DEC(DQ, DV) run_t<DQ, DV>(a, mode, out_f32, s, ph)
  if (P.dq == 192 && P.dv == 128) return CALL_DEC(192, 128);
  if (P.dq == 128 && P.dv == 128) return CALL_DEC(128, 128);
  if (P.dq == 64 && P.dv == 64) return CALL_DEC(64, 64);
  if (P.dq == 192 && P.dv == 64) return CALL_DEC(192, 64);
  if (P.dq == 128 && P.dv == 64) return CALL_DEC(128, 64);
  if (P.dq == 64 && P.dv == 128) return CALL_DEC(64, 128);
#undef CALL_DEC
  return hipErrorInvalidValue;
}

}  // namespace nsa
