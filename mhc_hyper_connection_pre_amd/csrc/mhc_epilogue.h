// Per-token epilogue of mhc_pre on 16 lanes of a wave (n <= 4) or on a whole
// wave (n <= 8): RMS factor, hc_scale, bias, sigmoid gates and the Sinkhorn
// normalisation of the comb logits.
//
// The pre call of sglang PR #24355 analysis ("AMD ROCm DeepSeek-V4
// performance optimisation: Aiter MHC kernel integration"), section 2, returns
// post and comb; the closing list of that page says the fused kernel covers
// the Sinkhorn iterations and the normalisation. Conventions (not fixed by the
// pages): logits are [pre | post | comb row-major]; gates are the logistic
// function; comb = Sinkhorn(exp(Z)) with each repeat normalising rows then
// columns; the RMS mean runs over all n*D elements with eps inside the root.
#pragma once

#include "mhc_device.h"

namespace mhc {

// DPP controls (within each 16-lane row of the wave).
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1, 0, 3, 2]: partner lane ^ 1
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2, 3, 0, 1]: partner lane ^ 2
constexpr int kRowRor4 = 0x124;   // row rotate by 4
constexpr int kRowRor8 = 0x128;   // row rotate by 8

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Per-lane constants of the epilogue: lane e of a 16-lane group scales and
// biases gate logit e (pre for e < n, post for n <= e < 2n) and comb logit
// (e / 4, e % 4). Loading them ahead of the epilogue keeps their global loads
// (and the wait on the memory counter that would also cover every store still
// in flight) off the finalise path.
struct EpiConst {
  float sg, bg;   // gate: hc_scale[0 or 1], bias[e]
  float sc, bc;   // comb: hc_scale[2], bias[2n + n i + j]
};

template <int NS>
__device__ __forceinline__ EpiConst epi_const(const float* __restrict__ hc_scale, const float* __restrict__ bias) {
  const int e = threadIdx.x & 15;
  const int i = e >> 2, jj = e & 3;
  const int cc = (i < NS && jj < NS) ? 2 * NS + i * NS + jj : 0;
  const int cg = e < 2 * NS ? e : 0;
  return EpiConst{hc_scale[e < NS ? 0 : 1], bias[cg], hc_scale[2], bias[cc]};
}

// One 16-lane group handles one token. Lane e of the group holds the reduced
// column sums c = e (v0) and c = e + 16 (v1) of the token's logit row
// (N = n(n+2) mixing sums, then the sum of squares at c = N).
// logits16 returns, in lane e: `gate` = sigmoid logit e for e < 2n (pre then
// post), and the comb logit zc = z[2n + 4 i + j] of the 4 x 4 padded layout
// (i = e / 4, j = e % 4; `act` when i < n and j < n). sinkhorn16 then returns
// comb[e / 4][e % 4]. The normalisations multiply by the hardware reciprocal
// (about 1 ulp) instead of dividing. The group must be 16-lane aligned and all
// 16 lanes must execute the calls (they exchange values within the group).
template <int NS>
__device__ __forceinline__ void logits16(float v0, float v1, const EpiConst& k, float K, float eps, float& gate,
                                         float& zc, bool& act) {
  constexpr int N = NS * (NS + 2);
  const int lane = threadIdx.x & 63;
  const int gb = lane & ~15;
  const int e = lane & 15;
  auto col = [&](int c) {  // column sum c of this group's token
    const float a = __shfl(v0, gb + (c & 15));
    const float b = __shfl(v1, gb + (c & 15));
    return c < 16 ? a : b;
  };
  const float ssq = col(N);
  const float r = 1.0f / sqrtf(ssq / K + eps);
  const int i = e >> 2, jj = e & 3;
  act = i < NS && jj < NS;
  const int cc = act ? 2 * NS + i * NS + jj : 0;
  const float mc = col(cc);
  const int cg = e < 2 * NS ? e : 0;
  const float mg = col(cg);
  gate = sigmoidf_ieee(k.sg * (r * mg) + k.bg);
  zc = act ? k.sc * (r * mc) + k.bc : -INFINITY;
}

__device__ __forceinline__ float sinkhorn16(float zc, bool act, int repeat) {
  // 4 x 4 padded layout in a 16-lane DPP row: a row of comb is a quad (quad
  // permutations), a column is lanes j, j+4, j+8, j+12 (row rotations by 8, 4).
  float rmax = fmaxf(zc, dpp_f32<kQuadSwap1>(zc));
  rmax = fmaxf(rmax, dpp_f32<kQuadSwap2>(rmax));
  float M = act ? expf(zc - rmax) : 0.0f;
  for (int it = 0; it < repeat; ++it) {
    float rs = M + dpp_f32<kQuadSwap1>(M);
    rs = rs + dpp_f32<kQuadSwap2>(rs);
    M = act ? M * __builtin_amdgcn_rcpf(rs) : 0.0f;
    float cs = M + dpp_f32<kRowRor8>(M);
    cs = cs + dpp_f32<kRowRor4>(cs);
    M = act ? M * __builtin_amdgcn_rcpf(cs) : 0.0f;
  }
  return M;
}

template <int NS>
__device__ __forceinline__ void epilogue16(float v0, float v1, const EpiConst& k, float K, float eps, int repeat,
                                           float& gate, float& comb) {
  float zc;
  bool act;
  logits16<NS>(v0, v1, k, K, eps, gate, zc, act);
  comb = sinkhorn16(zc, act, repeat);
}

// The same epilogue for up to 8 streams on a whole wave (one token per wave).
// Lane l brings the column sums c = l (v0) and c = l + 64 (v1) of the token's
// logit row (the sum of squares at c = N). Lane e holds gate logit e for
// e < 2n and comb entry (e / 8, e % 8) of an 8 x 8 padded layout: a comb row is
// 8 consecutive lanes (xor 1, 2, 4), a column is lanes j, j + 8, ..., j + 56
// (xor 8, 16, 32). All 64 lanes must execute the calls.
template <int NS>
__device__ __forceinline__ EpiConst epi_const64(const float* __restrict__ hc_scale,
                                                const float* __restrict__ bias) {
  const int e = threadIdx.x & 63;
  const int i = e >> 3, jj = e & 7;
  const int cc = (i < NS && jj < NS) ? 2 * NS + i * NS + jj : 0;
  const int cg = e < 2 * NS ? e : 0;
  return EpiConst{hc_scale[e < NS ? 0 : 1], bias[cg], hc_scale[2], bias[cc]};
}

template <int NS>
__device__ __forceinline__ void logits64(float v0, float v1, const EpiConst& k, float K, float eps, float& gate,
                                         float& zc, bool& act) {
  constexpr int N = NS * (NS + 2);
  static_assert(N < 128, "two column sums per lane");
  const int e = threadIdx.x & 63;
  auto col = [&](int c) {  // column sum c of the token
    const float a = __shfl(v0, c & 63);
    const float b = __shfl(v1, c & 63);
    return c < 64 ? a : b;
  };
  const float ssq = col(N);
  const float r = 1.0f / sqrtf(ssq / K + eps);
  const int i = e >> 3, jj = e & 7;
  act = i < NS && jj < NS;
  const int cc = act ? 2 * NS + i * NS + jj : 0;
  const float mc = col(cc);
  const int cg = e < 2 * NS ? e : 0;
  const float mg = col(cg);
  gate = sigmoidf_ieee(k.sg * (r * mg) + k.bg);
  zc = act ? k.sc * (r * mc) + k.bc : -INFINITY;
}

__device__ __forceinline__ float sinkhorn64(float zc, bool act, int repeat) {
  float rmax = fmaxf(zc, __shfl_xor(zc, 1));
  rmax = fmaxf(rmax, __shfl_xor(rmax, 2));
  rmax = fmaxf(rmax, __shfl_xor(rmax, 4));
  float M = act ? expf(zc - rmax) : 0.0f;
  for (int it = 0; it < repeat; ++it) {
    float rs = M + __shfl_xor(M, 1);
    rs = rs + __shfl_xor(rs, 2);
    rs = rs + __shfl_xor(rs, 4);
    M = act ? M * __builtin_amdgcn_rcpf(rs) : 0.0f;
    float cs = M + __shfl_xor(M, 8);
    cs = cs + __shfl_xor(cs, 16);
    cs = cs + __shfl_xor(cs, 32);
    M = act ? M * __builtin_amdgcn_rcpf(cs) : 0.0f;
  }
  return M;
}

template <int NS>
__device__ __forceinline__ void epilogue64(float v0, float v1, const EpiConst& k, float K, float eps, int repeat,
                                           float& gate, float& comb) {
  float zc;
  bool act;
  logits64<NS>(v0, v1, k, K, eps, gate, zc, act);
  comb = sinkhorn64(zc, act, repeat);
}

}  // namespace mhc
