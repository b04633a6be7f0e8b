// Packing of fn [K, N] fp32 into bf16 MFMA B fragments.
//
// Fragment (s * NCB + cb) * 64 + lane holds 8 bf16: B[k][col] for
// k = 32 s + 8 (lane / 16) + e (e = 0..7) and col = 16 cb + lane % 16, with
// the column blocks [hi | lo | lo2 | 0]:
//   col <  N            hi(fn[k][col])            hi  = bf16(f)
//   N  <= col < 2N      lo(fn[k][col - N])        lo  = bf16(f - hi)
//   2N <= col < 2N + n  lo2(fn[k][col - 2N])      lo2 = bf16(f - hi - lo)
// and 0 beyond or for k >= K (NCB = ceil((2N + n) / 16)). Both differences
// are exact in fp32. The residual is exact in bf16, so with fp32 MFMA
// accumulation x*hi + x*lo reproduces x*fn to about 2^-17 relative (a bf16
// fn alone would move the comb logits by ~1e-2, which Sinkhorn amplifies),
// and the pre-gate columns (the first n) add x*lo2 to reach fp32 accuracy:
// y = sum_i pre_i x_i cancels to near zero for some positions, where an error
// of 2^-17 in pre shows against the output's own magnitude. The A operand
// uses the same k order, so the MFMA lane layout of the k index never matters.
#pragma once

#include "mhc_device.h"

namespace mhc {

constexpr int kPackSteps = 2;   // k-steps (32 fn rows each) per 256-thread block
constexpr int kPackMaxN = 80;   // n <= 8

// 16-column blocks of [hi | lo | lo2 of the pre columns] for n streams.
__host__ __device__ constexpr int pack_blocks(int n) { return (2 * n * (n + 2) + n + 15) / 16; }

// n from N = n (n + 2).
__host__ __device__ constexpr int n_pre(int N) {
  int n = 1;
  while (n * (n + 2) < N) ++n;
  return n;
}

// Part `part` (0 = hi, 1 = lo, 2 = lo2) of the three-term bf16 split of x,
// as a float (exactly representable in bf16); part 3 is a zero column.
__device__ __forceinline__ float split3(float x, int part) {
  const float hi = (float)(__bf16)x;
  const float r1 = x - hi;                  // exact
  const float lo = (float)(__bf16)r1;
  const float r2 = r1 - lo;                 // exact
  return part == 0 ? hi : (part == 1 ? (float)(__bf16)r1 : (part == 2 ? (float)(__bf16)r2 : 0.0f));
}

// hi, lo and lo2 words (two bf16 each) of the three-term split of the pair
// (x0, x1); the same values as split3 parts 0, 1 and 2.
__device__ __forceinline__ void split3_pair(float x0, float x1, uint32_t& h, uint32_t& l, uint32_t& l2) {
  h = pack_bf16x2(x0, x1);
  const float r0 = x0 - bf16_lo(h), r1 = x1 - bf16_hi(h);   // exact
  l = pack_bf16x2(r0, r1);
  l2 = pack_bf16x2(r0 - bf16_lo(l), r1 - bf16_hi(l));       // exact differences
}

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
  const int npre = n_pre(N);
  for (int f = threadIdx.x; f < kPackSteps * NCB * 64; f += blockDim.x) {
    const int sl = f / (NCB * 64);
    const int cb = (f / 64) % NCB;
    const int lane = f & 63;
    if (s0 + sl >= ksteps) continue;
    const int col = cb * 16 + (lane & 15);
    const int part = col < N ? 0 : (col < 2 * N ? 1 : (col < 2 * N + npre ? 2 : 3));
    const int c = col - part * N;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = sl * 32 + (lane >> 4) * 8 + e;
      const float x = (part < 3 && r < rows) ? tile[r * (N + 1) + c] : 0.0f;
      v[e] = split3(x, part);
    }
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    fnp[((int64_t)(s0 + sl) * NCB + cb) * 64 + lane] = out;
  }
}

}  // namespace mhc
