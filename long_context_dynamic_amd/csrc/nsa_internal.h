// nsa_internal.h -- shared definitions of the gfx950 NSA library (not part
// of the public ABI).  Everything here is device/host plumbing: the problem
// descriptor the launchers take, element conversions and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "nsa.h"

namespace nsa {

// ---- launch logging: with NSA_LOG set (and not "0") in the environment,
// every kernel launch prints its name, grid, block and dynamic LDS to
// stderr (read at each launch, so it can be switched at run time) ----
inline bool log_on() {
  const char* e = getenv("NSA_LOG");
  return e && *e && !(e[0] == '0' && e[1] == 0);
}
template <typename K, typename... A>
inline void launch(const char* name, K kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, A... args) {
  if (log_on())
    fprintf(stderr, "[nsa] %s grid %u x %u block %u lds %zu\n", name, grid.x, grid.y, block.x, lds);
  kern<<<grid, block, lds, s>>>(args...);
}


// Problem sizes widened to 64 bits, plus derived quantities.
struct Prob {
  int64_t B, T, L, G, hpg, H, dq, dv, bs, n, w, nb;
  int64_t sb, nbs;  // selection block and selection-block count (sb = bs unless decoupled)
  uint32_t flags;
  int dtype;
  float scale;
  bool bf16() const { return dtype == NSA_BF16; }
  bool has(uint32_t f) const { return (flags & f) != 0; }
  int n_forced() const { return (has(NSA_F_FORCE_FIRST) ? 1 : 0) + (has(NSA_F_FORCE_CURRENT) ? 1 : 0); }
};

// Statistics a training forward keeps for the backward: per branch and
// (b, t, h) the natural log-sum-exp of the scaled logits (fp32 [3][B, T, H],
// -inf for an empty or disabled branch), then, 256-byte aligned, the
// branch's normalised output (bf16 [3][B, T, H, d_v], zeros when empty).
inline size_t saved_lse_bytes(const Prob& P) { return ((size_t)3 * P.B * P.T * P.H * 4 + 255) / 256 * 256; }
inline size_t saved_bytes(const Prob& P) { return saved_lse_bytes(P) + (size_t)3 * P.B * P.T * P.H * P.dv * 2; }

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup i to XCD
// i % 8), each XCD with its own L2.  xcd_run renumbers them so that XCD x
// takes the contiguous run [x * per, (x + 1) * per) of n logical ids:
// neighbouring work items, which read the same keys, then share one L2
// instead of fetching them into every XCD's.  Launch xcd_grid(n)
// workgroups; ids >= n have nothing to do.
__device__ __forceinline__ int64_t xcd_run(int64_t n) {
  const int64_t per = (n + 7) / 8;
  return (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
}
inline unsigned xcd_grid(int64_t n) { return (unsigned)((n + 7) / 8 * 8); }

// ---- element conversions (device) ----------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 with a single rounding to nearest even: go to fp32 rounding
// to odd (truncate, then force the last bit if anything was dropped), which
// keeps 16 spare bits and so cannot create a double-rounding error.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  float t = __double2float_rz(x);
  uint32_t u = __float_as_uint(t);
  if ((double)t != x) u |= 1u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }

template <typename T> __device__ __forceinline__ void st(T* p, int64_t i, float x);
template <> __device__ __forceinline__ void st<uint16_t>(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
template <> __device__ __forceinline__ void st<float>(float* p, int64_t i, float x) { p[i] = x; }

template <typename T> __device__ __forceinline__ void st64(T* p, int64_t i, double x);
template <> __device__ __forceinline__ void st64<uint16_t>(uint16_t* p, int64_t i, double x) { p[i] = f64_to_bf16(x); }
template <> __device__ __forceinline__ void st64<float>(float* p, int64_t i, double x) { p[i] = __double2float_rn(x); }

// ---- wave64 reductions ---------------------------------------------------

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// Sigmoid for gate logits.
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// ---- launchers (each returns hipGetLastError() of its launches) ----------

hipError_t launch_pool(const Prob& P, const void* k, const void* v, void* kc, void* vc, hipStream_t s);

// Generic any-shape path (VALU, fp32 arithmetic).
hipError_t launch_select_generic(const Prob& P, const void* q, const void* kc, const void* vc,
                                 int32_t* idx, float* score, float* ocmp, hipStream_t s);
hipError_t launch_attend_generic(const Prob& P, const void* q, const void* k, const void* v,
                                 const void* gates, const int32_t* idx, const float* ocmp,
                                 void* out, float* lse, bool out_f32, hipStream_t s);

}  // namespace nsa
