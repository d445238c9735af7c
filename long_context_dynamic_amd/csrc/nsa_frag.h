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

}  // namespace nsa
