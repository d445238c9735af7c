// k_moba.hip -- MoBA on the matrix cores ([P1] s7, [P5] s13): every head has
// its own K/V, scores its past blocks by the mean key, keeps its own top-k
// (the current block always), and attends with one softmax to the chosen
// blocks, causally inside the current one.
//
// With one head per KV group the matrix M dimension cannot come from heads,
// so the work is reorganised around the blocks ([P1] s7: the queries that
// chose a block are gathered and run against it as one dense product):
//
//   k_moba_select  one workgroup per (head, 64-token tile): block scores
//                  Q . kmean^T on the matrix cores, per-token softmax and top-k
//                  with row reductions (DPP), sorted idx (+ scores).
//   k_moba_count / k_moba_scan / k_moba_fill
//                  list, for every (head, block), the (token, slot) entries
//                  that chose it (the current block excluded).
//   k_moba_attn    one workgroup per 128 listed entries of one (head, block):
//                  the block's K and V tiles are staged through LDS once (V as
//                  rows, read back transposed by ds_read_b64_tr_b16) and
//                  shared by the 128 gathered queries; writes a (max, sum,
//                  output) partial per entry.
//   k_moba_diag    one workgroup per (head, 128-token tile): causal attention
//                  over the query's own block, then the log-sum-exp merge with
//                  the entries' partials, output.
#include <math.h>

#include "nsa_mfma.h"
#include "nsa_moba.h"
#include "nsa_tile.h"

namespace nsa {
namespace {

constexpr int kRows = 64;    // tokens per selection workgroup (4 waves x 16)
constexpr int kChunk = 128;  // listed entries per attention workgroup (4 waves x 2 x 16)
constexpr int kCountTok = 256;  // tokens per list-counting workgroup
constexpr int kXcds = 8;     // the chip's compute dies, each with its own L2
constexpr int kMaxN = 8;     // most blocks one token selects on this path
constexpr int kRecBatch = 4; // partial records whose values one merge step loads together

// Partial record of one entry (16-byte aligned): the normalised output o / l
// as D fp16 values scaled by 2^-ex so that all lie in (-1, 1) (a relative
// error of 2^-11 of the record's largest value), then the fp32 max (log2
// units), the fp32 sum l, ex, and a spare word.
template <int D> constexpr int rec_bytes() { return 2 * D + 16; }

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// Descending list insertion without branches: x goes after equal values (the
// earlier block keeps a tie); -inf changes nothing.
template <int LS>
__device__ __forceinline__ void list_insert(float (&v)[LS], int (&j)[LS], float x, int blk) {
  bool c[LS];
#pragma unroll
  for (int k = 0; k < LS; ++k) c[k] = x > v[k];
#pragma unroll
  for (int k = LS - 1; k > 0; --k) {
    v[k] = c[k - 1] ? v[k - 1] : (c[k] ? x : v[k]);
    j[k] = c[k - 1] ? j[k - 1] : (c[k] ? blk : j[k]);
  }
  v[0] = c[0] ? x : v[0];
  j[0] = c[0] ? blk : j[0];
}

// ---------------------------------------------------------------------------
// One workgroup per (head, 64 tokens), 16 tokens per wave.  Block scores
// S = Q . Kc^T come 16 blocks at a time from the matrix cores (lane: block
// 16*nt + lr, tokens 4*lg + r).  With one head per group the importance of a
// block is its softmax probability, which ranks exactly like its logit, so
// the top-k is taken on unscaled dot products while streaming: each lane
// keeps, per token, a descending list of its LS best candidates (visible, not
// forced; ties keep the earlier block), and at the end the 16 lanes of a token
// merge their lists.  Tiles wholly visible to the wave and free of forced
// blocks skip the masks.  SCORES: per-lane online softmax statistics as well, merged the same
// way, for the probabilities of the chosen blocks.  The block summaries pass
// through LDS 64 at a time, shared by the four waves, the next 64 in flight
// while these are scored.
template <int D, int LS, bool SCORES>
__global__ void __launch_bounds__(256) k_moba_select(MobaArgs a) {
  constexpr int KS = k_lds_stride<D>();
  __shared__ __align__(16) uint16_t kcs[64 * KS];
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t ntile = (a.T + kRows - 1) / kRows;
  const int64_t h = blockIdx.x % a.H;
  const int64_t tile = (blockIdx.x / a.H) % ntile;
  const int64_t b = blockIdx.x / (a.H * ntile);
  const int64_t t0 = tile * kRows + 16 * wave;  // this wave's 16 tokens
  // A = token rows (lane: token t0 + lr), B = block rows
  bf16x8 qf[D / 32];
  {
    int64_t tq = t0 + lr;
    if (tq > a.T - 1) tq = a.T - 1;
    const uint16_t* qr = a.q + ((b * a.T + tq) * a.H + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[ks] = ld8(qr + 32 * ks);
  }
  const bool first = a.flags & NSA_F_FORCE_FIRST, current = a.flags & NSA_F_FORCE_CURRENT;
  int nvis[4], cur[4];
  float lv[4][LS], lm[4], ls[4];
  int lj[4][LS];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int64_t t = t0 + 4 * lg + r;
    if (t > a.T - 1) t = a.T - 1;
    const int64_t p = a.L - a.T + t;
    const int64_t nv = (p + 1) / a.bs;
    nvis[r] = (int)(nv < a.nb ? nv : a.nb);
    cur[r] = (int)(p / a.bs);
    lm[r] = -INFINITY;
    ls[r] = 0.f;
#pragma unroll
    for (int k = 0; k < LS; ++k) { lv[r][k] = -INFINITY; lj[r][k] = 0x7fffffff; }
  }
  // blocks visible to any of this wave's tokens (the last one sees the most),
  // and to any of the workgroup's
  auto visible_to = [&](int64_t t) {
    const int64_t tl = t < a.T - 1 ? t : a.T - 1;
    const int64_t nv = (a.L - a.T + tl + 1) / a.bs;
    return nv < a.nb ? nv : a.nb;
  };
  const int64_t ntl = (visible_to(t0 + 15) + 15) / 16;
  const int64_t nvis_min = visible_to(t0);  // the wave's first token sees the fewest
  const int64_t cur_min = (a.L - a.T + (t0 < a.T - 1 ? t0 : a.T - 1)) / a.bs;
  const int64_t cur_max = (a.L - a.T + (t0 + 15 < a.T - 1 ? t0 + 15 : a.T - 1)) / a.bs;
  const int64_t nchunk = (visible_to(tile * kRows + kRows - 1) + 63) / 64;
  Stager<D, D, 256> st;
  if (nchunk > 0) st.load(a.kc, a.nb, 0, nullptr, 0, 0, b, h, a.H, false);
  for (int64_t c = 0; c < nchunk; ++c) {
    __syncthreads();
    st.store(kcs, nullptr, false, false);
    __syncthreads();
    if (c + 1 < nchunk) st.load(a.kc, a.nb, 64 * (c + 1), nullptr, 0, 0, b, h, a.H, false);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
    const int64_t nt = 4 * c + tt;
    if (nt >= ntl) break;  // wave-uniform
    const int blk = (int)(16 * nt + lr);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) sc = mfma16(qf[ks], ld8(kcs + (16 * tt + lr) * KS + 8 * lg + 32 * ks), sc);
    const bool plain = 16 * nt + 16 <= nvis_min && !(first && nt == 0) &&
                       !(current && 16 * nt <= cur_max && 16 * nt + 15 >= cur_min);  // wave-uniform
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = sc[r];
      if (SCORES && blk < nvis[r]) {
        const float z = x * a.scale;
        const float nm = fmaxf(lm[r], z);
        ls[r] = ls[r] * __expf(lm[r] - nm) + __expf(z - nm);
        lm[r] = nm;
      }
      if (!plain) {
        const bool cand = blk < nvis[r] && !(first && blk == 0) && !(current && blk == cur[r]);
        x = cand ? x : -INFINITY;
      }
      list_insert<LS>(lv[r], lj[r], x, blk);
    }
    }
  }
  int chosen[4][8];  // per token: the chosen blocks, forced ones first
  float cscore[4][8];
  int cnt[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float gm = 0.f, inv = 0.f;
    if (SCORES) {
      gm = row_max16(lm[r]);
      const float part = lm[r] == -INFINITY ? 0.f : ls[r] * __expf(lm[r] - gm);
      const float gs = row_sum16(part);
      inv = gs > 0.f ? 1.f / gs : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) { chosen[r][i] = 0x7fffffff; cscore[r][i] = -INFINITY; }
    int nf = 0;
    if (first) { chosen[r][0] = 0; cscore[r][0] = INFINITY; nf = 1; }
    if (current && !(first && cur[r] == 0)) {
      if (nf == 0) { chosen[r][0] = cur[r]; cscore[r][0] = INFINITY; }
      else { chosen[r][1] = cur[r]; cscore[r][1] = INFINITY; }
      ++nf;
    }
    cnt[r] = nf;
    // merge the 16 lanes' lists: the best head, the lowest block among equal
    // heads; the winning lane pops it (uniform within the token's DPP row)
    for (int round = 0; round < 8; ++round) {
      if (cnt[r] >= a.n) break;
      const float hv = lv[r][0];
      const float M = row_max16(hv);
      if (M == -INFINITY) break;
      const int J = row_min16(hv == M ? lj[r][0] : 0x7fffffff);
      if (hv == M && lj[r][0] == J) {
#pragma unroll
        for (int k = 0; k < LS - 1; ++k) { lv[r][k] = lv[r][k + 1]; lj[r][k] = lj[r][k + 1]; }
        lv[r][LS - 1] = -INFINITY;
        lj[r][LS - 1] = 0x7fffffff;
      }
      const float score = SCORES ? __expf(M * a.scale - gm) * inv : 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i == cnt[r]) { chosen[r][i] = J; cscore[r][i] = score; }
      ++cnt[r];
    }
  }
  if (lr != 0) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = t0 + 4 * lg + r;
    if (t >= a.T) continue;
    // ascending block order (unused slots hold INT_MAX and sort last)
#pragma unroll
    for (int i = 0; i < 7; ++i)
#pragma unroll
      for (int k2 = 0; k2 < 7 - i; ++k2)
        if (chosen[r][k2] > chosen[r][k2 + 1]) {
          const int tj = chosen[r][k2];
          chosen[r][k2] = chosen[r][k2 + 1];
          chosen[r][k2 + 1] = tj;
          const float ts = cscore[r][k2];
          cscore[r][k2] = cscore[r][k2 + 1];
          cscore[r][k2 + 1] = ts;
        }
    int32_t* orow = a.idx + ((b * a.T + t) * a.H + h) * a.n;
    float* srow = a.score ? a.score + ((b * a.T + t) * a.H + h) * a.n : nullptr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i >= a.n) break;
      orow[i] = i < cnt[r] ? chosen[r][i] : -1;
      if (srow) srow[i] = i < cnt[r] ? cscore[r][i] : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
__global__ void k_moba_zero(int32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

// One workgroup per (b, h, 256 tokens), one thread per token: a chosen block
// before the token's own goes to its (b, h, block) list (an empty slot, the
// token's own block and a block after it, which a valid selection never
// holds, stay unlisted: pos = -1).  Places are counted in an LDS histogram
// first, then reserved in the global count with one atomic per touched block.
__global__ void __launch_bounds__(256) k_moba_count(MobaArgs a) {
  extern __shared__ int32_t hist[];  // [nb]
  const int64_t nr = (a.T + kCountTok - 1) / kCountTok;
  const int64_t h = blockIdx.x % a.H;
  const int64_t b = blockIdx.x / (a.H * nr);
  const int64_t t = (blockIdx.x / a.H) % nr * kCountTok + threadIdx.x;
  for (int64_t j = threadIdx.x; j < a.nb; j += blockDim.x) hist[j] = 0;
  __syncthreads();
  const bool tv = t < a.T;
  const int64_t cur = (a.L - a.T + t) / a.bs;
  const int64_t e0 = ((b * a.T + t) * a.H + h) * a.n;
  int js[8], loc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    js[i] = (tv && i < a.n) ? a.idx[e0 + i] : -1;
    const bool listed = js[i] >= 0 && (int64_t)js[i] < cur;
    loc[i] = listed ? atomicAdd(&hist[js[i]], 1) : -1;
  }
  __syncthreads();
  int32_t* cnt = a.counts + (b * a.H + h) * a.nb;
  for (int64_t j = threadIdx.x; j < a.nb; j += blockDim.x) {
    const int32_t c = hist[j];
    if (c) hist[j] = atomicAdd(&cnt[j], c);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (tv && i < a.n) a.pos[e0 + i] = loc[i] >= 0 ? hist[js[i]] + loc[i] : -1;
}

// Single workgroup: exclusive prefix sums of the list lengths and of their
// 128-entry chunk counts.
__global__ void __launch_bounds__(1024) k_moba_scan(MobaArgs a) {
  __shared__ int32_t part_e[1024], part_c[1024];
  const int64_t n = a.B * a.H * a.nb;
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t lo = tid * per, hi = lo + per < n ? lo + per : n;
  int32_t se = 0, sc = 0;
  for (int64_t i = lo; i < hi; ++i) { se += a.counts[i]; sc += (a.counts[i] + kChunk - 1) / kChunk; }
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
    a.offsets[n] = ae;
    a.chunk_off[n] = ac;
  }
  __syncthreads();
  int32_t ae = part_e[tid], ac = part_c[tid];
  for (int64_t i = lo; i < hi; ++i) {
    a.offsets[i] = ae;
    a.chunk_off[i] = ac;
    ae += a.counts[i];
    ac += (a.counts[i] + kChunk - 1) / kChunk;
  }
}

__global__ void k_moba_fill(MobaArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.B * a.T * a.H * a.n) return;
  const int pos = a.pos[e];
  if (pos < 0) return;
  const int64_t h = (e / a.n) % a.H;
  const int64_t b = e / (a.n * a.H * a.T);
  const int j = a.idx[e];
  a.lists[a.offsets[(b * a.H + h) * a.nb + j] + pos] = (int32_t)e;
}

// ---------------------------------------------------------------------------
// One workgroup per 128 listed entries of one (b, h, block) list; the
// block's K and V^T tiles pass through LDS once for all of them.  Chunks are
// dealt to the compute dies in contiguous runs (workgroup i runs on die
// i % 8), so the chunks of one list share that die's L2.
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) k_moba_attn(MobaArgs a) {
  __shared__ __align__(16) uint16_t kt[64 * k_lds_stride<D>()];
  __shared__ __align__(16) uint16_t vt[64 * v_row_stride<D>()];  // V rows of the tile, read back transposed
  const int64_t nl = a.B * a.H * a.nb;
  const int32_t total = a.chunk_off[nl];
  const int32_t per = (total + kXcds - 1) / kXcds;
  const int32_t run = (int32_t)(blockIdx.x / kXcds);
  const int32_t w = (int32_t)(blockIdx.x % kXcds) * per + run;
  if (run >= per || w >= total) return;
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  // the (b, h, block) list this chunk belongs to: the last list whose first
  // chunk is <= w, by a 64-way search (each lane tests one point of the
  // interval, so a round costs one load latency; 2 rounds for 4096 lists)
  int64_t lo = 0, hi = nl;  // chunk_off[lo] <= w < chunk_off[hi]
  while (hi - lo > 1) {
    const int64_t step = (hi - lo + 63) / 64, pos = lo + lane * step;
    const bool le = pos < hi && a.chunk_off[pos] <= w;  // a prefix of the lanes, lane 0 always
    lo += (int64_t)(__popcll(__ballot(le)) - 1) * step;
    hi = lo + step < hi ? lo + step : hi;
  }
  const int64_t bhj = lo;
  const int64_t j = bhj % a.nb, h = (bhj / a.nb) % a.H, b = bhj / (a.nb * a.H);
  const int64_t first = a.offsets[bhj] + (int64_t)(w - a.chunk_off[bhj]) * kChunk;
  const int64_t count = a.offsets[bhj + 1] - first;  // entries left in this list
  const bool busy = 32 * wave < count;  // wave-uniform: this wave has rows
  int64_t e[2];
  bf16x8 qf[2][D / 32];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = 32 * wave + 16 * q + lr;
    e[q] = a.lists[first + (row < count ? row : 0)];
    const int64_t t = (e[q] / (a.n * a.H)) % a.T;
    const uint16_t* qr = a.q + ((b * a.T + t) * a.H + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[q][ks] = ld8(qr + 32 * ks);
  }
  const float c = a.scale * kLog2e, stale = kStaleLog2 / c;
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4 o[2][D / 16];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[q][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  Stager<D, D, 256, true> st;
  const int64_t kb0 = j * a.bs, ntl = a.bs / 64;
  st.load(a.k, a.L, kb0, a.v, a.Lp, kb0, b, h, a.H, true);
  for (int64_t i = 0; i < ntl; ++i) {
    __syncthreads();
    st.store(kt, vt, true, true);
    __syncthreads();
    if (i + 1 < ntl) st.load(a.k, a.L, kb0 + 64 * (i + 1), a.v, a.Lp, kb0 + 64 * (i + 1), b, h, a.H, true);
    if (busy) {
      f32x4 s[2][4];
      qk_tile_T2<D>(kt, qf, s, lr, lg);
      softmax_step<D>(s[0], m[0], l[0], o[0], c, stale, true);
      softmax_step<D>(s[1], m[1], l[1], o[1], c, stale, true);
      pv_tile2_rows<D>(vt, s, o, lr, lg);
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    // the record's scale: the largest |o / l| over the query's lanes (all
    // lanes take part in the reduction)
    const float inv = l[q] > 0.f ? 1.f / l[q] : 0.f;
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(o[q][dt][r]));
    amax = xor_max16_32(amax * inv);
    int ex = 0;
    (void)frexpf(amax, &ex);
    const float sc = inv * ldexpf(1.f, -ex);
    if (32 * wave + 16 * q + lr >= count) continue;
    char* rec = (char*)a.part + e[q] * rec_bytes<D>();
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const f32x4 v = o[q][dt] * sc;
      const f16x4 hv = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
      *(u32x2*)(rec + 2 * (16 * dt + 4 * lg)) = __builtin_bit_cast(u32x2, hv);
    }
    if (lg == 0) {
      float* tail = (float*)(rec + 2 * D);
      tail[0] = m[q] * c;
      tail[1] = l[q];
      tail[2] = (float)ex;
    }
  }
}

// ---------------------------------------------------------------------------
template <typename TO> __device__ __forceinline__ void mstore4(TO* p, f32x4 v);
template <> __device__ __forceinline__ void mstore4<float>(float* p, f32x4 v) { *(f32x4*)p = v; }
template <> __device__ __forceinline__ void mstore4<uint16_t>(uint16_t* p, f32x4 v) {
  u32x2 w = {(uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
             (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16)};
  *(u32x2*)p = w;
}

// One workgroup per (b, h, 64*NQ query positions): causal attention over
// the query's own block, then the log-sum-exp merge with the partials of the
// earlier chosen blocks.  Query tiles follow the absolute position grid, so
// a tile never spans two blocks (block % (64*NQ) == 0) and its keys start on
// a 64-key tile; each wave holds NQ sets of 16 queries.
template <int D, int NQ, typename TO>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) k_moba_diag(MobaArgs a) {
  __shared__ __align__(16) uint16_t kt[64 * k_lds_stride<D>()];
  __shared__ __align__(16) uint16_t vt[64 * v_row_stride<D>()];  // V rows of the tile, read back transposed
  constexpr int TP = 64 * NQ;
  const int64_t P0 = a.L - a.T;  // position of token 0
  const int64_t pt0 = P0 / TP, ntile = (a.L - 1) / TP - pt0 + 1;
  const int64_t h = blockIdx.x % a.H;
  const int64_t pt = pt0 + ntile - 1 - (blockIdx.x / a.H) % ntile;  // longest rows first
  const int64_t b = blockIdx.x / (a.H * ntile);
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t p_first = TP * pt > P0 ? TP * pt : P0;
  const int64_t p_last = TP * pt + TP - 1 < a.L - 1 ? TP * pt + TP - 1 : a.L - 1;
  const int64_t cur = TP * pt / a.bs;
  // the first K / V tile is requested before anything else
  Stager<D, D, 256, true> st;
  const int64_t kt0 = cur * a.bs / 64, kt1 = p_last / 64;
  st.load(a.k, a.L, kt0 * 64, a.v, a.Lp, kt0 * 64, b, h, a.H, true);
  int64_t p[NQ], t[NQ];
  bool valid[NQ], has_cur[NQ];
  uint32_t earlier[NQ];  // bit i: the token's slot i holds a block before its own
  bf16x8 qf[NQ][D / 32];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int64_t pl = TP * pt + 16 * (NQ * wave + q) + lr;
    valid[q] = pl >= P0 && pl < a.L;
    p[q] = valid[q] ? pl : p_last;  // out-of-range lanes shadow the last row
    t[q] = p[q] - P0;
    // the token's selection (at most kMaxN slots, all loads in flight together)
    const int32_t* irow = a.idx + ((b * a.T + t[q]) * a.H + h) * a.n;
    int32_t sel[kMaxN];
#pragma unroll
    for (int i = 0; i < kMaxN; ++i) sel[i] = i < a.n ? irow[i] : -1;
    const uint16_t* qr = a.q + ((b * a.T + t[q]) * a.H + h) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) qf[q][ks] = ld8(qr + 32 * ks);
    has_cur[q] = false;
    earlier[q] = 0;
#pragma unroll
    for (int i = 0; i < kMaxN; ++i) {
      has_cur[q] |= (sel[i] == cur);
      if (sel[i] >= 0 && sel[i] < cur) earlier[q] |= 1u << i;
    }
  }
  const float c = a.scale * kLog2e, stale = kStaleLog2 / c;
  float m[NQ], l[NQ];
  f32x4 o[NQ][D / 16];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    m[q] = -INFINITY;
    l[q] = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[q][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the wave's first row: tiles that start after it have nothing for it
  const int64_t p_wave = TP * pt + 16 * NQ * wave;
  for (int64_t kb = kt0; kb <= kt1; ++kb) {
    __syncthreads();
    st.store(kt, vt, true, true);
    __syncthreads();
    if (kb + 1 <= kt1) st.load(a.k, a.L, (kb + 1) * 64, a.v, a.Lp, (kb + 1) * 64, b, h, a.H, true);
    if (kb * 64 > p_wave + 16 * NQ - 1) continue;  // wave-uniform: every key after every row
    f32x4 s[NQ][4];
    if constexpr (NQ == 2) {
      qk_tile_T2<D>(kt, qf, s, lr, lg);
    } else {
      qk_tile_T<D>(kt, qf[0], s[0], lr, lg);
    }
    // keys after the query (only in the tiles that reach the first row), and
    // every key of a row whose selection lacks its own block
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (kb * 64 + 63 > p_first || !has_cur[q]) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!has_cur[q] || kb * 64 + s_key(mt, lg, r) > p[q]) s[q][mt][r] = -INFINITY;
      }
      softmax_step<D>(s[q], m[q], l[q], o[q], c, stale, true);
    }
    if constexpr (NQ == 2) {
      pv_tile2_rows<D>(vt, s, o, lr, lg);
    } else {
      pv_tile_rows<D>(vt, s[0], o[0], lr, lg);
    }
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (!valid[q]) continue;
    // merge with the partials of the earlier chosen blocks (log2 units); the
    // records' tails are loaded together, then their values, a few at a time
    const bool own = has_cur[q] && l[q] > 0.f;  // a row without its own block ran on -inf only
    const char* prow = (const char*)a.part + ((b * a.T + t[q]) * a.H + h) * a.n * rec_bytes<D>();
    f32x4 tail[kMaxN];
#pragma unroll
    for (int i = 0; i < kMaxN; ++i)
      tail[i] = (earlier[q] >> i) & 1 ? *(const f32x4*)(prow + i * rec_bytes<D>() + 2 * D)
                                      : f32x4{-INFINITY, 0.f, 0.f, 0.f};
    float M = own ? m[q] * c : -INFINITY;
#pragma unroll
    for (int i = 0; i < kMaxN; ++i) M = fmaxf(M, tail[i][0]);
    const float wd = own ? exp2f(m[q] * c - M) : 0.f;
    float den = own ? wd * l[q] : 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = own ? o[q][dt] * wd : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i0 = 0; i0 < kMaxN; i0 += kRecBatch) {
      if (!(earlier[q] >> i0)) break;  // no later slot holds an earlier block
      u32x2 hv[kRecBatch][D / 16];
#pragma unroll
      for (int i = i0; i < i0 + kRecBatch; ++i)
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
          hv[i - i0][dt] = (earlier[q] >> i) & 1
                               ? *(const u32x2*)(prow + i * rec_bytes<D>() + 2 * (16 * dt + 4 * lg))
                               : u32x2{0u, 0u};
#pragma unroll
      for (int i = i0; i < i0 + kRecBatch; ++i) {
        // the record's weight: its share of the softmax mass (0 for unused slots)
        const float ws = (earlier[q] >> i) & 1 ? exp2f(tail[i][0] - M) * tail[i][1] : 0.f;
        den += ws;
        const float f = ws * ldexpf(1.f, (int)tail[i][2]);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const f16x4 x = __builtin_bit_cast(f16x4, hv[i - i0][dt]);
          acc[dt] += f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]} * f;
        }
      }
    }
    float g = den > 0.f ? 1.f / den : 0.f;
    if (a.gates) {
      float x = bf16_to_f32(a.gates[((b * a.T + t[q]) * a.H + h) * 3 + 1]);
      if (a.flags & NSA_F_GATE_LOGITS) x = sigmoid(x);
      g *= x;
    }
    TO* orow = (TO*)a.out + ((b * a.T + t[q]) * a.H + h) * D + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) mstore4<TO>(orow + 16 * dt, acc[dt] * g);
    if (a.lse && lg == 0)
      a.lse[(b * a.T + t[q]) * a.H + h] = den > 0.f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D, bool SCORES>
hipError_t run_select_t(const MobaArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)(a.B * a.H * ((a.T + kRows - 1) / kRows));
  // list length per lane: the most candidates one token takes
  const int64_t nf_min = (a.flags & (NSA_F_FORCE_FIRST | NSA_F_FORCE_CURRENT)) ? 1 : 0;
  const int64_t need = a.n - nf_min;
  if (need <= 2) launch("k_moba_select<D, 2, SCORES>", k_moba_select<D, 2, SCORES>, grid, 256, 0, s, a);
  else if (need <= 4) launch("k_moba_select<D, 4, SCORES>", k_moba_select<D, 4, SCORES>, grid, 256, 0, s, a);
  else launch("k_moba_select<D, 8, SCORES>", k_moba_select<D, 8, SCORES>, grid, 256, 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t run_attend_t(const MobaArgs& a, bool out_f32, hipStream_t s, Phases* ph) {
  const int64_t ne = a.B * a.T * a.H * a.n, nl = a.B * a.H * a.nb;
  launch("k_moba_zero", k_moba_zero, (unsigned)((nl + 255) / 256), 256, 0, s, a.counts, nl);
  const unsigned gcount = (unsigned)(a.B * a.H * ((a.T + kCountTok - 1) / kCountTok));
  launch("k_moba_count", k_moba_count, gcount, kCountTok, (size_t)a.nb * sizeof(int32_t), s, a);
  launch("k_moba_scan", k_moba_scan, 1, 1024, 0, s, a);
  launch("k_moba_fill", k_moba_fill, (unsigned)((ne + 255) / 256), 256, 0, s, a);
  if (ph) ph->mark();
  // an upper bound of the chunk count, in whole runs of 8; surplus
  // workgroups exit at once
  const int64_t chunks_max = (ne + kChunk - 1) / kChunk + nl;
  const unsigned gattn = (unsigned)((chunks_max + kXcds - 1) / kXcds * kXcds);
  launch("k_moba_attn<D>", k_moba_attn<D>, gattn, 256, 0, s, a);
  if (ph) ph->mark();
  if (a.bs % 128 == 0) {
    const unsigned gdiag = (unsigned)(a.B * a.H * ((a.L - 1) / 128 - (a.L - a.T) / 128 + 1));
    if (out_f32) launch("k_moba_diag<D, 2, float>", k_moba_diag<D, 2, float>, gdiag, 256, 0, s, a);
    else launch("k_moba_diag<D, 2, uint16_t>", k_moba_diag<D, 2, uint16_t>, gdiag, 256, 0, s, a);
  } else {
    const unsigned gdiag = (unsigned)(a.B * a.H * ((a.L - 1) / 64 - (a.L - a.T) / 64 + 1));
    if (out_f32) launch("k_moba_diag<D, 1, float>", k_moba_diag<D, 1, float>, gdiag, 256, 0, s, a);
    else launch("k_moba_diag<D, 1, uint16_t>", k_moba_diag<D, 1, uint16_t>, gdiag, 256, 0, s, a);
  }
  if (ph) ph->mark();
  return hipGetLastError();
}

}  // namespace

bool moba_select_ok(const Prob& P) {
  return P.bf16() && P.hpg == 1 && P.sb == P.bs && (P.dq == 64 || P.dq == 128) && P.nb >= 1 && P.n >= 1 &&
         P.n <= 8;
}

bool moba_attend_ok(const Prob& P) {
  // nb >= 1: with no complete block there is no list to build (its kernels
  // would launch empty grids); the generic path takes that case
  return P.bf16() && P.hpg == 1 && P.sb == P.bs && P.dq == P.dv && (P.dq == 64 || P.dq == 128) && P.nb >= 1 &&
         P.bs % 64 == 0 && P.n >= 1 &&
         P.n <= kMaxN && P.B * P.T * P.H * P.n < ((int64_t)1 << 31) && P.B * P.H * P.nb < ((int64_t)1 << 30);
}

bool moba_ok(const Prob& P) {
  return moba_select_ok(P) && moba_attend_ok(P) && P.has(NSA_F_SLC) && !P.has(NSA_F_CMP) && !P.has(NSA_F_WIN);
}

hipError_t launch_moba_select(const Prob& P, const MobaArgs& a, hipStream_t s) {
  if (P.dq == 128) return a.score ? run_select_t<128, true>(a, s) : run_select_t<128, false>(a, s);
  return a.score ? run_select_t<64, true>(a, s) : run_select_t<64, false>(a, s);
}

hipError_t launch_moba_attend(const Prob& P, const MobaArgs& a, bool out_f32, hipStream_t s, Phases* ph) {
  if (P.dq == 128) return run_attend_t<128>(a, out_f32, s, ph);
  return run_attend_t<64>(a, out_f32, s, ph);
}

}  // namespace nsa
