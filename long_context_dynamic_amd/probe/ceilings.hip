// ceilings.hip -- measurement kernels for the benchmark's reference ceilings
// (not part of the attention library): the rate at which the chip serves
// random whole-block gathers, the access pattern of the selected branch
// (each wave reads whole 40 KiB blocks, K and V of 64 keys, at random).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockChunks = 2560;  // 40 KiB in 16-byte chunks

// One wave per work item: per_wave blocks table[pick[...]], each read once as
// 40 chunks of 1 KiB (20 loads in flight per lane), folded into one word.
// NT: non-temporal loads (kept out of the caches where possible).
template <bool NT>
__global__ void __launch_bounds__(256) k_gather(const u32x4* __restrict__ table, const int* __restrict__ pick,
                                                int npick, unsigned* __restrict__ out, int64_t waves, int per_wave) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= waves) return;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int i = 0; i < per_wave; ++i) {
    const int blk = pick[(w * per_wave + i) % npick];
    const u32x4* p = table + (int64_t)blk * kBlockChunks + lane;
    u32x4 r[20];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int k = 0; k < 20; ++k) r[k] = NT ? __builtin_nontemporal_load(p + 1280 * h + 64 * k) : p[1280 * h + 64 * k];
#pragma unroll
      for (int k = 0; k < 20; ++k) acc ^= r[k];
    }
  }
  out[w * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// table: nblocks x 40 KiB (device); pick: npick block ids < nblocks (device);
// out: waves x 64 words (device); nontemporal: 1 for non-temporal loads, 0
// for ordinary (cached) ones.  Queues one launch on stream; returns the
// hipError_t of the launch as int.
int nsa_probe_gather(const void* table, const int* pick, int npick, unsigned* out, int64_t waves, int per_wave,
                     int nontemporal, void* stream) {
  if (!table || !pick || !out || npick < 1 || waves < 1 || per_wave < 1) return (int)hipErrorInvalidValue;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  if (nontemporal)
    k_gather<true><<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)table, pick, npick, out, waves, per_wave);
  else
    k_gather<false><<<grid, 256, 0, (hipStream_t)stream>>>((const u32x4*)table, pick, npick, out, waves, per_wave);
  return (int)hipGetLastError();
}

}  // extern "C"
