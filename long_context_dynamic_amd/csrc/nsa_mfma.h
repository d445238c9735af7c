// nsa_mfma.h -- gfx950 matrix-core building blocks for the NSA kernels.
//
// v_mfma_f32_16x16x32_bf16 (one wave, D = A * B + C, A 16x32, B 32x16):
//   A: lane l holds A[l % 16][8 * (l / 16) + s], s = 0..7
//   B: lane l holds B[8 * (l / 16) + s][l % 16]
//   D: lane l holds D[4 * (l / 16) + r][l % 16], r = 0..3
// The 32-long contraction index only has to be the same bijection for A and
// B, so the kernels are free to assign any 32 keys (or dims) to the slots.
#pragma once

#include "nsa_internal.h"

namespace nsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16 contiguous bytes (8 bf16) from global or LDS memory.
// The wave's index in its workgroup, as a value the compiler knows to be
// uniform across the wave (so that what is derived from it, such as buffer
// resources, stays in scalar registers instead of per-lane loops).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)p);
}
// Two 8-byte halves (4 bf16 each) into one operand.
__device__ __forceinline__ bf16x8 ld4x2(const uint16_t* lo, const uint16_t* hi) {
  u32x2 a = *(const u32x2*)lo;
  u32x2 b = *(const u32x2*)hi;
  u32x4 r = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, r);
}

// Buffer resource over [base, base + bytes): loads through it take a 32-bit
// byte offset per lane and return zeros past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset voff + soff (soff uniform).
__device__ __forceinline__ bf16x8 bld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each 16-lane
// group, lane i points at 4 consecutive 16-bit elements R_i; lane 4a + c
// receives element c of R_a, R_(a+4), R_(a+8), R_(a+12).  With lane i on row
// row0 + i / 4, columns col0 + 4 * (i % 4) .. + 3 of a row-major tile, lane
// j of the group receives column col0 + j of rows row0 .. row0 + 3.
__device__ __forceinline__ u32x2 ld_tr4(const uint16_t* tile, int row0, int col0, int stride, int i) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const uint16_t* p = tile + (row0 + (i >> 2)) * stride + col0 + 4 * (i & 3);
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
  return __builtin_bit_cast(u32x2, r);
}
// A matrix-op operand of V^T: rows rowa .. rowa + 3 then rowb .. rowb + 3 of
// column col0 + lr.
__device__ __forceinline__ bf16x8 ld_vt_pair(const uint16_t* tile, int rowa, int rowb, int col0, int stride,
                                             int lr) {
  const u32x2 a = ld_tr4(tile, rowa, col0, stride, lr);
  const u32x2 b = ld_tr4(tile, rowb, col0, stride, lr);
  const u32x4 r = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, r);
}

// ---- cross-lane reductions without LDS traffic -------------------------
// gfx950 v_permlane16_swap / v_permlane32_swap called with the same value
// twice return, in every lane, its own and its partner's value (partner =
// lane ^ 16, resp. lane ^ 32), in some order.
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor_max16_32(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float xor_sum16_32(float x) { return xor32_sum(xor16_sum(x)); }

// DPP lane moves inside a row of 16 lanes.
template <int CTRL> __device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16

// Row reductions over the 16 lanes of a DPP row (lanes 16*lg .. 16*lg + 15).
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(dpp_i<kDppXor1>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<kDppXor2>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(x))));
  return fmaxf(x, __int_as_float(dpp_i<kDppMirror>(__float_as_int(x))));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(dpp_i<kDppXor1>(__float_as_int(x)));
  x += __int_as_float(dpp_i<kDppXor2>(__float_as_int(x)));
  x += __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(x)));
  return x + __int_as_float(dpp_i<kDppMirror>(__float_as_int(x)));
}
__device__ __forceinline__ int row_min16(int x) {
  x = min(x, dpp_i<kDppXor1>(x));
  x = min(x, dpp_i<kDppXor2>(x));
  x = min(x, dpp_i<kDppHalfMirror>(x));
  return min(x, dpp_i<kDppMirror>(x));
}

// Maximum over all 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_allmax(float x) {
  x = fmaxf(x, __int_as_float(dpp_i<kDppXor1>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<kDppXor2>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(x))));
  x = fmaxf(x, __int_as_float(dpp_i<kDppMirror>(__float_as_int(x))));
  return xor_max16_32(x);
}
// Minimum of non-negative ints over all 64 lanes, returned in every lane.
__device__ __forceinline__ int wave_allmin_u(int x) {
  x = min(x, dpp_i<kDppXor1>(x));
  x = min(x, dpp_i<kDppXor2>(x));
  x = min(x, dpp_i<kDppHalfMirror>(x));
  x = min(x, dpp_i<kDppMirror>(x));
  auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  x = min((int)r[0], (int)r[1]);
  r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return min((int)r[0], (int)r[1]);
}

// 2^x with the bare hardware instruction (no denormal range fix-up: results
// below 2^-126 flush to zero, which softmax weights can afford).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax keeps a stale running maximum: it is only raised when a new
// score exceeds it by more than 2^8 in probability, so the rescale of the
// accumulators is rare; probabilities then stay below 2^8 (no overflow).
constexpr float kStaleLog2 = 8.0f;

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace nsa
