// k_learned.hip -- the learned parts around the NSA forward ([P1] s4: each
// block is compressed into a learned representation and each branch is
// weighted by a gate learned from the token's input through a projection;
// [P1] s7: NSA's block representation comes from an MLP):
//
//   k_mlp_compress  phi(X) = W2 relu(W1 vec(X) + b1) + b2 over each block's
//                   tokens flattened in order.  One workgroup per 16 block
//                   rows of one tensor (K or V): the 4 waves split the
//                   block*d contraction of the first layer (16 rows as the
//                   matrix M, W1 rows as N), their partial sums meet in LDS,
//                   the bias and ReLU are applied, the hidden rows (bf16)
//                   stay in LDS for the second layer, whose output tiles the
//                   waves share out.
//   k_gate_proj     gates = sigmoid(x W^T + b): one workgroup per 128 tokens,
//                   a wave per 16 tokens, 192 outputs at a time in registers
//                   across the d_model contraction, the weight slices shared
//                   through LDS; the sigmoid (unless gate logits are asked
//                   for) and the bf16 rounding in the epilogue.
// Both are dense contractions on bf16 matrix cores with fp32 accumulation.
#include <math.h>

#include "nsa_learned.h"
#include "nsa_mfma.h"

namespace nsa {
namespace {

// ---------------------------------------------------------------------------
template <int D, int DH>
__global__ void __launch_bounds__(256) k_mlp_compress(MlpArgs a, int which) {
  constexpr int HS = DH + 16;  // LDS row stride of the hidden rows (16-byte reads conflict-free)
  constexpr int NTH = DH / 16, NTO = D / 16;
  __shared__ float part[3][16][DH + 4];  // waves 1..3's partial sums
  __shared__ __align__(16) uint16_t hid[16 * HS];
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const uint16_t* x = which ? a.v : a.k;
  const uint16_t* w1 = which ? a.v_w1 : a.k_w1;
  const uint16_t* b1 = which ? a.v_b1 : a.k_b1;
  const uint16_t* w2 = which ? a.v_w2 : a.k_w2;
  const uint16_t* b2 = which ? a.v_b2 : a.k_b2;
  uint16_t* out = which ? a.vc : a.kc;
  const int64_t R = a.B * a.nb * a.G;
  const int64_t r0 = (int64_t)blockIdx.x * 16;
  // this lane's input row (block summary row (b, j, g)), clamped at the end
  int64_t r = r0 + lr;
  if (r > R - 1) r = R - 1;
  const int64_t g = r % a.G, j = (r / a.G) % a.nb, b = r / (a.G * a.nb);
  const uint16_t* xrow = x + ((b * a.L + j * a.bs) * a.G + g) * D;  // token i of the block at + i * G * D

  // ---- layer 1: the wave's quarter of the block * D contraction ----
  const int64_t KIN = a.bs * D;
  const int64_t kq = KIN / 4, k0 = wave * kq;
  f32x4 acc[NTH];
#pragma unroll
  for (int n = 0; n < NTH; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t kk = k0; kk < k0 + kq; kk += 32) {
    // A: X[row lr][kk + 8 lg ..]: token (kk + 8 lg) / D of the block, dims (kk + 8 lg) % D
    const int64_t e = kk + 8 * lg;
    const bf16x8 af = ld8(xrow + (e / D) * a.G * D + e % D);
#pragma unroll
    for (int n = 0; n < NTH; ++n) acc[n] = mfma16(af, ld8(w1 + (int64_t)(16 * n + lr) * KIN + e), acc[n]);
  }
  // D layout: lane holds H[row 4 lg + q][hidden 16 n + lr]; wave 0 adds the
  // other waves' partial sums, the bias and the ReLU
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NTH; ++n)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[wave - 1][4 * lg + q][16 * n + lr] = acc[n][q];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int n = 0; n < NTH; ++n) {
      const int h = 16 * n + lr;
      const float bias = b1 ? bf16_to_f32(b1[h]) : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 4 * lg + q;
        const float sum = acc[n][q] + part[0][row][h] + part[1][row][h] + part[2][row][h] + bias;
        hid[row * HS + h] = f32_to_bf16(fmaxf(sum, 0.f));
      }
    }
  }
  __syncthreads();

  // ---- layer 2: output tiles shared out over the waves ----
  for (int n = wave; n < NTO; n += 4) {
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks)
      y = mfma16(ld8(hid + lr * HS + 8 * lg + 32 * ks), ld8(w2 + (int64_t)(16 * n + lr) * DH + 8 * lg + 32 * ks), y);
    const int c = 16 * n + lr;
    const float bias = b2 ? bf16_to_f32(b2[c]) : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = r0 + 4 * lg + q;
      if (row < R) out[row * D + c] = f32_to_bf16(y[q] + bias);  // kc row (b, j, g) = row
    }
  }
}

// ---------------------------------------------------------------------------
// N = 3H outputs in passes of 16 * kGateNT columns; the weight slice of each
// 64-wide step of the contraction passes through LDS once for the
// workgroup's 8 waves (128 tokens), the next slice's reads in flight while
// the current one is used.
constexpr int kGateNT = 12;
constexpr int kGateWS = 64 + 16;  // LDS row stride of a weight slice (16-byte reads conflict-free)

__global__ void __launch_bounds__(512) k_gate_proj(GateArgs a) {
  __shared__ __align__(16) uint16_t ws[16 * kGateNT * kGateWS];
  const int wave = wave_id(), lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 128 + 16 * wave;
  int64_t m = m0 + lr;
  if (m > a.M - 1) m = a.M - 1;
  const uint16_t* xrow = a.x + m * a.DM + 8 * lg;
  constexpr int CH = 16 * kGateNT * 64 / 8;  // 16-byte chunks of one slice
  constexpr int CPT = (CH + 511) / 512;
  for (int64_t n0 = 0; n0 < a.N; n0 += 16 * kGateNT) {
    f32x4 acc[kGateNT];
#pragma unroll
    for (int n = 0; n < kGateNT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 pre[CPT];
    auto fetch = [&](int64_t k) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + 512 * i;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (c < CH) {
          const int64_t col = n0 + c / 8, kk = k + 8 * (c % 8);  // past N or d_model: zeros
          if (col < a.N && kk < a.DM) val = *(const u32x4*)(a.w + col * a.DM + kk);
        }
        pre[i] = val;
      }
    };
    fetch(0);
    for (int64_t k = 0; k < a.DM; k += 64) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        const int c = threadIdx.x + 512 * i;
        if (c < CH) *(u32x4*)(ws + (c / 8) * kGateWS + 8 * (c % 8)) = pre[i];
      }
      __syncthreads();
      if (k + 64 < a.DM) fetch(k + 64);
      const int kn = a.DM - k >= 64 ? 2 : 1;  // d_model is a multiple of 32
      for (int ks = 0; ks < kn; ++ks) {
        const bf16x8 af = ld8(xrow + k + 32 * ks);
#pragma unroll
        for (int n = 0; n < kGateNT; ++n)
          acc[n] = mfma16(af, ld8(ws + (16 * n + lr) * kGateWS + 32 * ks + 8 * lg), acc[n]);
      }
    }
    // lane holds Z[token 4 lg + q][column 16 n + lr]
#pragma unroll
    for (int n = 0; n < kGateNT; ++n) {
      const int64_t c = n0 + 16 * n + lr;
      if (c >= a.N) continue;
      const float bias = a.bias ? bf16_to_f32(a.bias[c]) : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + 4 * lg + q;
        if (row >= a.M) continue;
        float z = acc[n][q] + bias;
        if (!a.logits) z = 1.f / (1.f + __expf(-z));
        a.gates[row * a.N + c] = f32_to_bf16(z);
      }
    }
  }
}

template <int D>
hipError_t launch_mlp_d(const MlpArgs& a, int which, int DH, hipStream_t s) {
  const unsigned grid = (unsigned)((a.B * a.nb * a.G + 15) / 16);
  switch (DH) {
    case 64: launch("k_mlp_compress<D, 64>", k_mlp_compress<D, 64>, grid, 256, 0, s, a, which); break;
    case 128: launch("k_mlp_compress<D, 128>", k_mlp_compress<D, 128>, grid, 256, 0, s, a, which); break;
    case 192: launch("k_mlp_compress<D, 192>", k_mlp_compress<D, 192>, grid, 256, 0, s, a, which); break;
    case 256: launch("k_mlp_compress<D, 256>", k_mlp_compress<D, 256>, grid, 256, 0, s, a, which); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mlp_one(const MlpArgs& a, int which, int D, int DH, hipStream_t s) {
  switch (D) {
    case 64: return launch_mlp_d<64>(a, which, DH, s);
    case 128: return launch_mlp_d<128>(a, which, DH, s);
    case 192: return launch_mlp_d<192>(a, which, DH, s);
    case 256: return launch_mlp_d<256>(a, which, DH, s);
  }
  return hipErrorInvalidValue;
}

bool dim_ok(int64_t d) { return d == 64 || d == 128 || d == 192 || d == 256; }

}  // namespace

bool mlp_ok(const Prob& P, int64_t dh) {
  return P.bf16() && dim_ok(P.dq) && dim_ok(P.dv) && dim_ok(dh) && P.bs % 4 == 0 && P.B * P.nb * P.G < (1LL << 31);
}

bool gate_proj_ok(const Prob& P, int64_t dm) {
  return P.bf16() && dm >= 32 && dm % 32 == 0 && P.B * P.T < (1LL << 31);
}

hipError_t launch_mlp_compress(const Prob& P, const MlpArgs& a, hipStream_t s) {
  if (a.B * a.nb * a.G == 0) return hipSuccess;
  hipError_t e = launch_mlp_one(a, 0, (int)P.dq, (int)a.dh, s);
  if (e != hipSuccess) return e;
  return launch_mlp_one(a, 1, (int)P.dv, (int)a.dh, s);
}

hipError_t launch_gate_proj(const GateArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.M + 127) / 128);
  if (grid == 0) return hipSuccess;
  launch("k_gate_proj", k_gate_proj, grid, 512, 0, s, a);
  return hipGetLastError();
}

}  // namespace nsa
