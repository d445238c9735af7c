// nsa_frag.h -- matrix-op fragments of one 32-key chunk read straight from
// global memory (internal): K rows from a paired-row image, V^T (or any
// key-contiguous transposed image) from a tiled image.  Buffer loads return
// zeros past the end of their resource.
#pragma once

#include "nsa_mfma.h"

namespace nsa {

// Fragments of one 32-key chunk of a selected block, in matrix-op layout.
// The two 16-row S^T tiles hold the keys in an interleaved order, row i of
// tile t <-> key kb + 8*(i/4) + 4*t + i%4, so that lane group lg ends up
// with the probabilities of the 8 consecutive keys kb + 8*lg .. kb + 8*lg + 7:
// each V^T operand (row d = 16*dt + lr) is then one 16-byte read.
template <int DQ> struct KFrag { bf16x8 k0[DQ / 32], k1[DQ / 32]; };
template <int DV> struct VFrag { bf16x8 v[DV / 16]; };

constexpr uint32_t kPastEnd = 0x7fff0000u;  // byte offset beyond any buffer: reads return zeros

// kr: buffer over this (b, g)'s paired-row K image (Lp rows); kofs: lane
// byte offset of its 8 dims (8*lg).  The chunk's key order puts rows
// w and w + 8 of each 16-row group in the same load, so each load reads
// whole lines.
template <int DQ>
__device__ __forceinline__ void load_k(KFrag<DQ>& f, __amdgpu_buffer_rsrc_t kr, uint32_t kofs, int64_t kb, int lr) {
  // tile-0 row of lane lr: kb + 8*(lr/4) + lr%4 = 16*(kb/16 + lr/8) + 8*((lr/4)%2) + lr%4
  const uint32_t rg = (uint32_t)kb / 16 + (lr >> 3), h = (lr >> 2) & 1, w8 = lr & 3;
  const uint32_t v0 = kb < 0 ? kPastEnd : ((rg * (DQ / 32) * 8 + w8) * 64 + h * 32) * 2 + kofs;
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) {
    f.k0[ks] = bld8(kr, v0, ks * 8 * 64 * 2);
    f.k1[ks] = bld8(kr, v0, ks * 8 * 64 * 2 + 4 * 64 * 2);  // tile 1: rows + 4 -> w8 + 4
  }
}

// vr: buffer over this (b, g)'s tiled V^T [Lp/32, DV, 32]; vofs: lane byte
// offset (row lr, keys 8*lg ..).  kb is a multiple of 32.
template <int DV>
__device__ __forceinline__ void load_v(VFrag<DV>& f, __amdgpu_buffer_rsrc_t vr, uint32_t vofs, int64_t kb) {
  const uint32_t v0 = kb < 0 ? kPastEnd : ((uint32_t)kb / 32) * DV * 32 * 2 + vofs;
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) f.v[dt] = bld8(vr, v0, 16 * dt * 32 * 2);
}

// The same chunk reads with the chunk's position as a wave-uniform value:
// the per-lane part of each address is fixed for the whole kernel (computed
// once), the chunk's part goes into the load's scalar offset, so streaming a
// chunk needs no per-lane arithmetic and no fresh registers.  A chunk past
// the end of the stream (kb < 0) reads through a resource of zero records:
// zeros, no memory traffic (the scalar offset is outside the hardware's
// range check, so it cannot carry that case).
template <int DQ> __device__ __forceinline__ uint32_t k_lane_ofs(int lr, int lg) {
  const uint32_t hi = (uint32_t)(lr >> 3), h = (lr >> 2) & 1, w8 = lr & 3;
  return ((hi * (DQ / 32) * 8 + w8) * 64 + h * 32) * 2 + 16 * (uint32_t)lg;
}
template <int DQ> __device__ __forceinline__ uint32_t k_chunk_ofs(int kb) {
  return kb < 0 ? 0u : (uint32_t)(kb / 16) * (DQ / 32) * 8 * 64 * 2;
}
template <int DV> __device__ __forceinline__ uint32_t v_chunk_ofs(int kb) {
  return kb < 0 ? 0u : (uint32_t)(kb / 32) * DV * 32 * 2;
}
// kr / vr: the stream's resource when kb >= 0, else a zero-record one.
template <int DQ>
__device__ __forceinline__ void load_k_u(KFrag<DQ>& f, __amdgpu_buffer_rsrc_t kr, uint32_t lofs, uint32_t cofs) {
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) {
    f.k0[ks] = bld8(kr, lofs, cofs + ks * 8 * 64 * 2);
    f.k1[ks] = bld8(kr, lofs, cofs + ks * 8 * 64 * 2 + 4 * 64 * 2);
  }
}
template <int DV>
__device__ __forceinline__ void load_v_u(VFrag<DV>& f, __amdgpu_buffer_rsrc_t vr, uint32_t vofs, uint32_t cofs) {
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) f.v[dt] = bld8(vr, vofs, cofs + 16 * dt * 32 * 2);
}

// ---- fragment-order images ------------------------------------------------
// K and V^T of every 32-key chunk stored so that each matrix-op operand of
// the chunk is 1 KiB holding lane l's 16 bytes at offset 16 l: a load
// instruction then reads 1 KiB contiguous in lane order and every 4 lanes
// share one 64-byte piece (with rows per lane, as the operands of the other
// images have it, each lane of a group of 4 touches another 64-byte piece
// and the vector L1 needs four times the accesses).
//   kF [B, G, Lp / 32][DQ / 32][2][64][8]: piece (ks, t, lane l) of chunk c
//     holds K[32 c + 8 (lr / 4) + 4 t + lr % 4][32 ks + 8 lg .. + 7]
//     (lr = l % 16, lg = l / 16: the interleaved key order of KFrag);
//   vF [B, G, Lp / 32][DV / 16][64][8]: piece (dt, l) of chunk c holds
//     V[32 c + 8 lg .. + 7][16 dt + lr] (keys along the piece).
// Consecutive chunks are frag_chunk(D) = 32 D elements apart.
__host__ __device__ constexpr int64_t frag_chunk(int D) { return 32 * (int64_t)D; }
template <int DQ>
__device__ __forceinline__ void load_k_frag(KFrag<DQ>& f, __amdgpu_buffer_rsrc_t kr, uint32_t lofs, uint32_t cofs) {
#pragma unroll
  for (int ks = 0; ks < DQ / 32; ++ks) {
    f.k0[ks] = bld8(kr, lofs, cofs + (2 * ks) * 1024);
    f.k1[ks] = bld8(kr, lofs, cofs + (2 * ks + 1) * 1024);
  }
}
template <int DV>
__device__ __forceinline__ void load_v_frag(VFrag<DV>& f, __amdgpu_buffer_rsrc_t vr, uint32_t lofs, uint32_t cofs) {
#pragma unroll
  for (int dt = 0; dt < DV / 16; ++dt) f.v[dt] = bld8(vr, lofs, cofs + dt * 1024);
}

}  // namespace nsa
