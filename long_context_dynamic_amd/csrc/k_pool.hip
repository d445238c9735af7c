// k_pool.hip -- block compression: the mean of each complete block's keys and
// values ([P1] s4 compression of each block into one summary; [P1] s7 mean
// pooling).  HBM-bound streaming: each workgroup owns one (batch, block,
// group) summary row and its threads walk the block's tokens in order.
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

}  // namespace

hipError_t launch_pool(const Prob& P, const void* k, const void* v, void* kc, void* vc, hipStream_t s) {
  const int64_t rows = P.B * P.nb * P.G;
  if (rows == 0) return hipSuccess;
  if (P.bf16())
    k_pool<uint16_t><<<dim3((unsigned)rows), dim3(256), 0, s>>>(
        (const uint16_t*)k, (const uint16_t*)v, (uint16_t*)kc, (uint16_t*)vc, P.L, P.G, P.dq, P.dv, P.bs, P.nb);
  else
    k_pool<float><<<dim3((unsigned)rows), dim3(256), 0, s>>>(
        (const float*)k, (const float*)v, (float*)kc, (float*)vc, P.L, P.G, P.dq, P.dv, P.bs, P.nb);
  return hipGetLastError();
}

}  // namespace nsa
