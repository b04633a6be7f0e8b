// Packing of fn [K, N] fp32 into bf16 hi/lo MFMA B fragments.
//
// Fragment (s * NCB + cb) * 64 + lane holds 8 bf16: B[k][col] for
// k = 32 s + 8 (lane / 16) + e (e = 0..7) and col = 16 cb + lane % 16, where
// B[k][col] = hi(fn[k][col]) for col < N, lo(fn[k][col - N]) for
// N <= col < 2N, and 0 for padding columns or k >= K, with hi = bf16(f) and
// lo = bf16(f - hi). The residual is exact in bf16, so x*hi + x*lo reproduces
// x*fn to about 2^-17 relative with fp32 MFMA accumulation (a bf16-only fn
// perturbs the comb logits by ~1e-2, which the Sinkhorn iterations amplify).
// The A operand uses the same k order, so the MFMA lane layout of the k index
// never matters.
#pragma once

#include "mhc_device.h"

namespace mhc {

constexpr int kPackSteps = 2;   // k-steps (32 fn rows each) per 256-thread block
constexpr int kPackMaxN = 24;   // n <= 4

// One block packs k-steps [blockIdx.x * kPackSteps, ... + kPackSteps): the
// rows (contiguous in fn) are read with consecutive threads on consecutive
// 16-byte vectors (4-byte words when fn is not 16-byte aligned) into the LDS
// `tile` (kPackSteps * 32 * (kPackMaxN + 1) floats), then each thread builds
// fragments; consecutive threads write consecutive fragments.
__device__ __forceinline__ void pack_fn_block(const float* __restrict__ fn, u32x4* __restrict__ fnp, int64_t K,
                                              int N, int NCB, int ksteps, bool vec4, float* tile) {
  const int s0 = blockIdx.x * kPackSteps;
  const int64_t k0 = (int64_t)s0 * 32;
  const int64_t left = K - k0;
  const int rows = (int)(left < kPackSteps * 32 ? left : kPackSteps * 32);
  const float* src = fn + k0 * N;
  const int nval = rows * N;
  if (vec4 && (nval & 3) == 0) {
    const f32x4* s4 = reinterpret_cast<const f32x4*>(src);
    for (int i = threadIdx.x; i < nval / 4; i += blockDim.x) {
      const f32x4 v = s4[i];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = 4 * i + u;
        const int r = e / N, c = e - r * N;
        tile[r * (N + 1) + c] = v[u];
      }
    }
  } else {
    for (int i = threadIdx.x; i < nval; i += blockDim.x) {
      const int r = i / N, c = i - r * N;
      tile[r * (N + 1) + c] = src[i];
    }
  }
  __syncthreads();
  for (int f = threadIdx.x; f < kPackSteps * NCB * 64; f += blockDim.x) {
    const int sl = f / (NCB * 64);
    const int cb = (f / 64) % NCB;
    const int lane = f & 63;
    if (s0 + sl >= ksteps) continue;
    const int col = cb * 16 + (lane & 15);
    const bool is_hi = col < N;
    const bool is_lo = !is_hi && col < 2 * N;
    const int c = is_hi ? col : col - N;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = sl * 32 + (lane >> 4) * 8 + e;
      const float x = ((is_hi || is_lo) && r < rows) ? tile[r * (N + 1) + c] : 0.0f;
      const float hi = (float)(__bf16)x;
      v[e] = is_hi ? hi : (x - hi);  // x - hi is exact in fp32
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    fnp[((int64_t)(s0 + sl) * NCB + cb) * 64 + lane] = out;
  }
}

}  // namespace mhc
