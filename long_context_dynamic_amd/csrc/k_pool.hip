// k_pool.hip -- block compression: the mean of each complete block's keys and
// values ([P1] s4 compression of each block into one summary; [P1] s7 mean
// pooling).  HBM-bound streaming: each thread owns summary elements and
// walks the block's tokens in order.
//
// Arithmetic contract: the sum is taken in fp64 in token order (one add at a
// time), divided by the block size, and rounded once to the storage type, so
// the result is reproducible bit for bit by any fp64 implementation that adds
// in the same order.
#include "nsa_internal.h"

namespace nsa {
namespace {

// One workgroup per (b, j, g) summary row: d_qk key dims then d_v value dims
// (keys only when vc is NULL),
// one output element per thread and pass; consecutive threads read
// consecutive dims of a token, so every load instruction is contiguous.
template <typename T>
__global__ void __launch_bounds__(256) k_pool(const T* __restrict__ k, const T* __restrict__ v,
                                              T* __restrict__ kc, T* __restrict__ vc,
                                              int64_t L, int64_t G, int64_t dq, int64_t dv,
                                              int64_t bs, int64_t nb) {
  const int64_t row = blockIdx.x;  // (b * nb + j) * G + g
  const int64_t g = row % G;
  const int64_t j = (row / G) % nb;
  const int64_t b = row / (G * nb);
  const int64_t ne = vc ? dq + dv : dq;  // no value summaries asked for: keys only
  for (int64_t e = threadIdx.x; e < ne; e += blockDim.x) {
    const bool is_k = e < dq;
    const int64_t d = is_k ? e : e - dq;
    const int64_t width = is_k ? dq : dv;
    const T* src = (is_k ? k : v) + ((b * L + j * bs) * G + g) * width + d;
    const int64_t stride = G * width;
    double sum = 0.0;
    for (int64_t s = 0; s < bs; ++s) sum += (double)ld(src, s * stride);
    const double mean = sum / (double)bs;
    if (is_k) st64(kc, row * dq + d, mean);
    else st64(vc, row * dv + d, mean);
  }
}

// One thread per 16-byte column chunk of a summary row (8 bf16 or 4 fp32
// dims), consecutive threads on consecutive chunks of the same tokens: every
// load instruction reads whole contiguous runs.  Same arithmetic as above,
// dim by dim (each dim its own fp64 sum in token order).
template <typename T>
__global__ void __launch_bounds__(256) k_pool_vec(const T* __restrict__ k, const T* __restrict__ v,
                                                  T* __restrict__ kc, T* __restrict__ vc, int64_t L, int64_t G,
                                                  int64_t dq, int64_t dv, int64_t bs, int64_t nb, int64_t rows) {
  constexpr int VE = 16 / sizeof(T);
  const int64_t cq = dq / VE, cpr = cq + (vc ? dv / VE : 0);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cpr) return;
  const int64_t row = idx / cpr, c = idx % cpr;  // row = (b * nb + j) * G + g
  const int64_t g = row % G;
  const int64_t j = (row / G) % nb;
  const int64_t b = row / (G * nb);
  const bool is_k = c < cq;
  const int64_t width = is_k ? dq : dv, c0 = (is_k ? c : c - cq) * VE;
  const T* src = (is_k ? k : v) + ((b * L + j * bs) * G + g) * width + c0;
  const int64_t stride = G * width;
  double sum[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) sum[e] = 0.0;
  // the tokens' loads go out kBatch at a time (long blocks would otherwise
  // wait on one load after another); the adds stay in token order
  constexpr int kBatch = 32;
  auto add = [&](uint4 w) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float x;
      if (sizeof(T) == 2) x = __uint_as_float((e & 1) ? (u[e / 2] & 0xffff0000u) : (u[e / 2] << 16));
      else x = __uint_as_float(u[e]);
      sum[e] += (double)x;
    }
  };
  int64_t t = 0;
  for (; t + kBatch <= bs; t += kBatch) {
    uint4 w[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) w[i] = *(const uint4*)(src + (t + i) * stride);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) add(w[i]);
  }
  for (; t < bs; ++t) add(*(const uint4*)(src + t * stride));
  T* dst = (is_k ? kc : vc) + row * width + c0;
#pragma unroll
  for (int e = 0; e < VE; ++e) st64(dst, e, sum[e] / (double)bs);
}

}  // namespace

hipError_t launch_pool(const Prob& P, const void* k, const void* v, void* kc, void* vc, hipStream_t s) {
  const int64_t rows = P.B * P.nb * P.G;
  if (rows == 0) return hipSuccess;
  const int ve = P.bf16() ? 8 : 4;
  if (P.dq % ve == 0 && P.dv % ve == 0) {  // whole 16-byte chunks (bases are 16-byte aligned)
    const int64_t threads = rows * (P.dq + (vc ? P.dv : 0)) / ve;
    const unsigned grid = (unsigned)((threads + 255) / 256);
    if (P.bf16())
      launch("k_pool_vec<uint16_t>", k_pool_vec<uint16_t>, grid, 256, 0, s, (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)kc,
                                                (uint16_t*)vc, P.L, P.G, P.dq, P.dv, P.bs, P.nb, rows);
    else
      launch("k_pool_vec<float>", k_pool_vec<float>, grid, 256, 0, s, (const float*)k, (const float*)v, (float*)kc, (float*)vc, P.L, P.G,
                                             P.dq, P.dv, P.bs, P.nb, rows);
    return hipGetLastError();
  }
  if (P.bf16())
    launch("k_pool<uint16_t>", k_pool<uint16_t>, dim3((unsigned)rows), dim3(256), 0, s,
        (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)kc, (uint16_t*)vc, P.L, P.G, P.dq, P.dv, P.bs, P.nb);
  else
    launch("k_pool<float>", k_pool<float>, dim3((unsigned)rows), dim3(256), 0, s,
        (const float*)k, (const float*)v, (float*)kc, (float*)vc, P.L, P.G, P.dq, P.dv, P.bs, P.nb);
  return hipGetLastError();
}

}  // namespace nsa
