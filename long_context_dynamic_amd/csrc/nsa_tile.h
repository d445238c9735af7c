// nsa_tile.h -- LDS tile machinery shared by the FA-style kernels (internal):
// a register-prefetching stager for 64-key K / V^T tiles, the 64-key online
// softmax step with a stale maximum, masks, and the two matrix-op products of
// one tile.  In an S^T tile, s[mt][r] is the key in LDS row 16*mt + 4*lg + r
// and lane column lr is one query row (a head of a token, or a token of a
// head).
#pragma once

#include "nsa_mfma.h"

namespace nsa {

// LDS row strides (bf16 elements), from gfx950's measured bank behaviour
// (counter SQ_LDS_BANK_CONFLICT over strides and lane maps).  16-byte reads
// with lane l on row l % 16 and 16 bytes per lane group are conflict-free
// when the row stride is 32 bytes past a multiple of 64: d + 16 elements for
// K rows of d = 64, 128, 192, and 64 + 16 for V^T rows of a 64-key tile.
// 16-byte writes of 128 contiguous bytes per 8 lanes are conflict-free at
// those strides.  (Two 8-byte reads that the compiler pairs into one
// ds_read2_b64 cost 8 conflict cycles per instruction at a 144-byte stride,
// which is why the V^T operand is one 16-byte read.)
template <int D> constexpr int k_lds_stride() { return D + 16; }
constexpr int kVtStride = 64 + 16;
// Row-major V tiles (keys x d) read back transposed (ld_vt_pair): rows of
// d + 8 elements, as the decoding kernels use.
template <int D> constexpr int v_row_stride() { return D + 8; }

// Permuted key order of a 64-key tile stored with perm = true: LDS row
// 16*mt + i holds key tile_key(mt, i) = 32*(mt/2) + 8*(i/4) + 4*(mt%2) + i%4.
// In the S^T tiles mt = 2h and 2h + 1, lane group lg then holds the
// probabilities of the 8 consecutive keys 32h + 8lg .. 32h + 8lg + 7, so each
// V^T operand of P.V (keys in natural order) is one 16-byte read.
__host__ __device__ constexpr int tile_key(int mt, int i) {
  return 32 * (mt >> 1) + 8 * (i >> 2) + 4 * (mt & 1) + (i & 3);
}
__host__ __device__ constexpr int tile_row(int key) {
  return 16 * (2 * (key >> 5) + ((key >> 2) & 1)) + 4 * ((key >> 3) & 3) + (key & 3);
}
// The key of S^T element s[mt][r] of lane group lg in a permuted tile.
__host__ __device__ constexpr int s_key(int mt, int lg, int r) { return 32 * (mt >> 1) + 8 * lg + 4 * (mt & 1) + r; }
// tile_row inverts tile_key on all 64 rows, and s_key is tile_key of the
// matrix-op output row 4 * lg + r
__host__ __device__ constexpr bool tile_perm_ok() {
  for (int row = 0; row < 64; ++row)
    if (tile_row(tile_key(row / 16, row % 16)) != row || s_key(row / 16, (row % 16) / 4, row % 4) != tile_key(row / 16, row % 16))
      return false;
  return true;
}
static_assert(tile_perm_ok(), "tile_row must invert tile_key");

// ---------------------------------------------------------------------------
// Register-prefetching tile stager: load() issues the global reads of one
// 64-key tile (K rows [row0, row0 + 64) of a [B, Nrows, G, DQ] tensor, rows
// clamped to Nrows - 1, and optionally V^T columns [col0, col0 + 64) of a
// tiled [B, G, Np / 32, DV, 32] tensor, or with VROWS the V rows [col0,
// col0 + 64) of a [B, Nrows, G, DV] tensor, clamped the same way) into
// registers; store() writes them to LDS, the K rows in permuted key order
// when perm is set, V rows in key order (row stride v_row_stride<DV>).  The
// next tile's reads are in flight while the current tile is computed on.
template <int DQ, int DV, int NT, bool VROWS = false>
struct Stager {
  static constexpr int KS = k_lds_stride<DQ>(), VS = VROWS ? v_row_stride<DV>() : kVtStride;
  static constexpr int KC = 64 * DQ / 8, VC = DV * 8;
  static constexpr int KPT = (KC + NT - 1) / NT, VPT = (VC + NT - 1) / NT;
  u32x4 kr[KPT], vr[VPT];

  // V^T chunk c (16 bytes = 8 keys): row d = c / 8, 32-key half (c % 8) / 4,
  // keys 8 * (c % 4) ..; 8 lanes cover one 128-byte LDS row, and a wave reads
  // two contiguous 512-byte runs (one per half).
  __device__ __forceinline__ void load(const uint16_t* rows, int64_t Nrows, int64_t row0, const uint16_t* colsT,
                                       int64_t Np, int64_t col0, int64_t b, int64_t g, int64_t G, bool with_v) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = threadIdx.x + i * NT;
      if (KC % NT == 0 || c < KC) {
        const int r = c / (DQ / 8), c8 = c % (DQ / 8);
        int64_t row = row0 + r;
        if (row > Nrows - 1) row = Nrows - 1;
        kr[i] = *(const u32x4*)(rows + ((b * Nrows + row) * G + g) * DQ + 8 * c8);
      }
    }
    if (with_v && VROWS) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * NT;
        if (VC % NT == 0 || c < VC) {
          const int r = c / (DV / 8), c8 = c % (DV / 8);
          int64_t row = col0 + r;
          if (row > Nrows - 1) row = Nrows - 1;
          vr[i] = *(const u32x4*)(colsT + ((b * Nrows + row) * G + g) * DV + 8 * c8);
        }
      }
    } else if (with_v) {
      const uint16_t* tile = colsT + ((b * G + g) * (Np / 64) + col0 / 64) * DV * 64;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * NT;
        const int d = c / 8, h = (c % 8) / 4, j8 = c % 4;
        if (VC % NT == 0 || c < VC) vr[i] = *(const u32x4*)(tile + (h * DV + d) * 32 + 8 * j8);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* kt, uint16_t* vt, bool with_v, bool perm) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = threadIdx.x + i * NT;
      if (KC % NT == 0 || c < KC) {
        const int r = c / (DQ / 8), d = 8 * (c % (DQ / 8));
        *(u32x4*)(kt + (perm ? tile_row(r) : r) * KS + d) = kr[i];
      }
    }
    if (with_v && VROWS) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * NT;
        if (VC % NT == 0 || c < VC) *(u32x4*)(vt + (c / (DV / 8)) * VS + 8 * (c % (DV / 8))) = vr[i];
      }
    } else if (with_v) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int c = threadIdx.x + i * NT;
        const int d = c / 8, h = (c % 8) / 4, j8 = c % 4;
        if (VC % NT == 0 || c < VC) *(u32x4*)(vt + d * VS + 32 * h + 8 * j8) = vr[i];
      }
    }
  }
};

// One 64-key online-softmax step for one token (16 heads) of one wave.
// s[mt] holds S^T for the tile's keys in either order (raw dot products,
// masked ones already -inf); updates the stale maximum m (raw units, raised only by more
// than 2^kStaleLog2 in probability), the sum l of head lr, and rescales o
// when m moves.
template <int DV>
__device__ __forceinline__ void softmax_step(f32x4 (&s)[4], float& m, float& l, f32x4 (&o)[DV / 16], float c,
                                             float stale, bool with_o) {
  float tmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) tmax = fmaxf(tmax, fmaxf(fmaxf(s[mt][0], s[mt][1]), fmaxf(s[mt][2], s[mt][3])));
  tmax = xor_max16_32(tmax);
  const bool raise = tmax > m + stale;
  if (__ballot(raise)) {
    const float mnew = raise ? tmax : m;
    const float alpha = fast_exp2((m - mnew) * c);
    l *= alpha;
    if (with_o) {
#pragma unroll
      for (int dt = 0; dt < DV / 16; ++dt) o[dt] *= alpha;
    }
    m = mnew;
  }
  const float mc = m * c;
  float rs = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pv = fast_exp2(fmaf(s[mt][r], c, -mc));
      s[mt][r] = pv;
      rs += pv;
    }
  l += xor_sum16_32(rs);
}

// Keys of a permuted tile at or beyond `limit` (relative to the tile start)
// are masked.
__device__ __forceinline__ void mask_from(f32x4 (&s)[4], int limit, int lg) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (s_key(mt, lg, r) >= limit) s[mt][r] = -INFINITY;
}
// ... and keys below `first`.
__device__ __forceinline__ void mask_below(f32x4 (&s)[4], int first, int lg) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (s_key(mt, lg, r) < first) s[mt][r] = -INFINITY;
}

// O^T[d, h] += V^T[d, keys] P^T[keys, h] over one 64-key LDS tile whose
// S^T (pm) came from a permuted K tile.
template <int DV>
__device__ __forceinline__ void pv_tile(const uint16_t* vt, const f32x4 (&pm)[4], f32x4 (&o)[DV / 16], int lr,
                                        int lg) {
  constexpr int VS = kVtStride;
  const bf16x8 p0 = pack8(pm[0], pm[1]);
  const bf16x8 p1 = pack8(pm[2], pm[3]);
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) {
    const uint16_t* row = vt + (16 * dt + lr) * VS + 8 * lg;
    o[dt] = mfma16(ld8(row), p0, o[dt]);
    o[dt] = mfma16(ld8(row + 32), p1, o[dt]);
  }
}

// S^T[key, h] for 64 keys of an LDS tile: s[mt] = K rows 16*mt.. x Q^T.
template <int DQ>
__device__ __forceinline__ void qk_tile_T(const uint16_t* kt, const bf16x8 (&qf)[DQ / 32], f32x4 (&s)[4], int lr,
                                          int lg) {
  constexpr int KS = k_lds_stride<DQ>();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) s[mt] = mfma16(ld8(kt + (16 * mt + lr) * KS + 8 * lg + 32 * ks), qf[ks], s[mt]);
  }
}

// S^T for two 16-query sets at once: each K fragment read from LDS feeds
// both (half the LDS reads per matrix op of one set per wave).
template <int DQ>
__device__ __forceinline__ void qk_tile_T2(const uint16_t* kt, const bf16x8 (&qf)[2][DQ / 32], f32x4 (&s)[2][4],
                                           int lr, int lg) {
  constexpr int KS = k_lds_stride<DQ>();
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    s[0][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    s[1][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DQ / 32; ++ks) {
      const bf16x8 kf = ld8(kt + (16 * mt + lr) * KS + 8 * lg + 32 * ks);
      s[0][mt] = mfma16(kf, qf[0][ks], s[0][mt]);
      s[1][mt] = mfma16(kf, qf[1][ks], s[1][mt]);
    }
  }
}

// O^T += V^T P^T for two query sets sharing each V^T fragment.
template <int DV>
__device__ __forceinline__ void pv_tile2(const uint16_t* vt, const f32x4 (&pm)[2][4], f32x4 (&o)[2][DV / 16], int lr,
                                         int lg) {
  constexpr int VS = kVtStride;
  const bf16x8 p00 = pack8(pm[0][0], pm[0][1]), p01 = pack8(pm[0][2], pm[0][3]);
  const bf16x8 p10 = pack8(pm[1][0], pm[1][1]), p11 = pack8(pm[1][2], pm[1][3]);
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) {
    const uint16_t* row = vt + (16 * dt + lr) * VS + 8 * lg;
    const bf16x8 v0 = ld8(row);
    const bf16x8 v1 = ld8(row + 32);
    o[0][dt] = mfma16(v0, p00, o[0][dt]);
    o[1][dt] = mfma16(v0, p10, o[1][dt]);
    o[0][dt] = mfma16(v1, p01, o[0][dt]);
    o[1][dt] = mfma16(v1, p11, o[1][dt]);
  }
}

// The same two products over a row-major V tile (keys in natural order,
// row stride v_row_stride<DV>): each V^T operand (keys 8 lg .. + 7, and 32
// on, of column 16 dt + lr) is two transposing 8-byte reads.
template <int DV>
__device__ __forceinline__ void pv_tile_rows(const uint16_t* vr, const f32x4 (&pm)[4], f32x4 (&o)[DV / 16], int lr,
                                             int lg) {
  constexpr int VS = v_row_stride<DV>();
  const bf16x8 p0 = pack8(pm[0], pm[1]);
  const bf16x8 p1 = pack8(pm[2], pm[3]);
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) {
    o[dt] = mfma16(ld_vt_pair(vr, 8 * lg, 8 * lg + 4, 16 * dt, VS, lr), p0, o[dt]);
    o[dt] = mfma16(ld_vt_pair(vr, 32 + 8 * lg, 36 + 8 * lg, 16 * dt, VS, lr), p1, o[dt]);
  }
}
template <int DV>
__device__ __forceinline__ void pv_tile2_rows(const uint16_t* vr, const f32x4 (&pm)[2][4], f32x4 (&o)[2][DV / 16],
                                              int lr, int lg) {
  constexpr int VS = v_row_stride<DV>();
  const bf16x8 p00 = pack8(pm[0][0], pm[0][1]), p01 = pack8(pm[0][2], pm[0][3]);
  const bf16x8 p10 = pack8(pm[1][0], pm[1][1]), p11 = pack8(pm[1][2], pm[1][3]);
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) {
    const bf16x8 v0 = ld_vt_pair(vr, 8 * lg, 8 * lg + 4, 16 * dt, VS, lr);
    const bf16x8 v1 = ld_vt_pair(vr, 32 + 8 * lg, 36 + 8 * lg, 16 * dt, VS, lr);
    o[0][dt] = mfma16(v0, p00, o[0][dt]);
    o[1][dt] = mfma16(v0, p10, o[1][dt]);
    o[0][dt] = mfma16(v1, p01, o[0][dt]);
    o[1][dt] = mfma16(v1, p11, o[1][dt]);
  }
}

}  // namespace nsa
