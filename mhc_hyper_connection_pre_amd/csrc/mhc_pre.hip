// mhc_pre on gfx950: RMS factor + split-K mixing GEMM, then gates, Sinkhorn and
// the pre-weighted stream reduce.
//
// The pre step of an mHC layer boundary: sglang PR #24355 analysis ("AMD ROCm
// DeepSeek-V4 performance optimisation: Aiter MHC kernel integration"),
// section 2 (the pre call returning post, comb, y) and section 3 (a split-K
// GEMM fused with the per-token sum of squares, tiled over the hidden axis).
//
// Three launches on the caller's stream:
//   1. pack_fn        fn fp32 [K, N] -> bf16 hi/lo pairs in MFMA B-fragment order
//   2. pre_gemm       residual x [T, K] (bf16) x [fn_hi | fn_lo] on MFMA
//                     16x16x32, plus sum of squares with v_dot2; one fp32
//                     partial row (N sums + sum of squares) per token and split
//   3. pre_epilogue   one workgroup per token: fixed-order split reduction,
//                     RMS factor, hc_scale, bias, sigmoid gates, Sinkhorn in
//                     registers of 16 lanes, then y = sum_i pre_i x_i from the
//                     token row prefetched before the epilogue runs.
// The fp32-residual path replaces 1-2 with a VALU dot-product kernel.
//
// fn is split as hi = bf16(fn), lo = bf16(fn - hi): x is exact in bf16, so
// x*hi + x*lo reproduces x*fn to about 2^-17 relative, with fp32 MFMA
// accumulation. A bf16-only fn would perturb the comb logits by ~1e-2, which
// the Sinkhorn iterations amplify.

#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

// ------------------------------------------------------------------ packing
// fnp[(s * NCB + cb) * 64 + lane] holds 8 bf16: B[k][col] for
// k = 32 s + 8 (lane / 16) + e (e = 0..7) and col = 16 cb + lane % 16, where
// B[k][col] = hi(fn[k][col]) for col < N, lo(fn[k][col - N]) for N <= col < 2N,
// and 0 for padding columns or k >= K. The same k-order is used for the A
// operand, so the MFMA lane layout of the k index never matters.
__global__ __launch_bounds__(256) void pack_fn_kernel(const float* __restrict__ fn, u32x4* __restrict__ fnp,
                                                      int64_t K, int N, int NCB, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const int64_t sc = idx >> 6;
  const int cb = (int)(sc % NCB);
  const int64_t s = sc / NCB;
  const int col = cb * 16 + (lane & 15);
  const int64_t kb = s * 32 + (lane >> 4) * 8;
  const bool is_hi = col < N;
  const bool is_lo = !is_hi && col < 2 * N;
  const int c = is_hi ? col : col - N;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = kb + e;
    float f = 0.0f;
    if ((is_hi || is_lo) && k < K) f = fn[k * N + c];
    const float hi = (float)(__bf16)f;
    v[e] = is_hi ? hi : (f - hi);   // f - hi is exact in fp32
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
  fnp[idx] = out;
}

hipError_t launch_pack_fn(const PrePlan& p, const float* fn, void* fnp, hipStream_t s) {
  const int64_t total = (int64_t)p.ksteps * p.NCB * 64;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(pack_fn_kernel, dim3(blocks), dim3(256), 0, s, fn, reinterpret_cast<u32x4*>(fnp), p.K,
                     p.N, p.NCB, total);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bf16 GEMM
// acc + lo^2 + hi^2 of a packed bf16 pair (products exact, fp32 sum).
__device__ __forceinline__ float dot2_self(uint32_t w, float acc) {
  const bf16x2 p = __builtin_bit_cast(bf16x2, w);
  return __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
}

// Workgroup = NW waves = one tile of 16*MT tokens x one split of the k-steps.
// Wave w takes k-steps s_begin + w, + NW, ... (the NW waves read NW adjacent
// 64-byte segments of every row at a time). Each wave keeps MT x NCB fp32
// accumulator tiles; the waves are summed in LDS in a fixed order.
template <int MT, int NW, int NCB>
__global__ __launch_bounds__(NW * 64) void pre_gemm_bf16_kernel(const uint16_t* __restrict__ x,
                                                                const u32x4* __restrict__ fnp,
                                                                float* __restrict__ part, int64_t T, int64_t K,
                                                                int N, int NP, int ksteps, int steps_per_split) {
  constexpr int CW = NCB * 16 + 1;  // LDS row: padded [hi | lo] columns, then the sum of squares
  __shared__ float red[NW * MT * 16 * CW];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int r16 = lane & 15;
  const int64_t tok0 = (int64_t)blockIdx.x * (16 * MT);
  const int split = blockIdx.y;
  const int s_begin = split * steps_per_split;
  const int s_end = min(ksteps, s_begin + steps_per_split);

  const uint16_t* arow[MT];
  bool rok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t row = tok0 + mt * 16 + r16;
    rok[mt] = row < T;
    arow[mt] = x + (rok[mt] ? row : 0) * K + q * 8;
  }

  f32x4 acc[MT][NCB];
  float ss[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ss[mt] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[mt][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const u32x4* bl = fnp + lane;
  auto load = [&](int s, u32x4* a, u32x4* b) {
    const int64_t k = (int64_t)s * 32;
    const bool kok = k + q * 8 < K;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = (rok[mt] && kok) ? ld16(arow[mt] + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) b[cb] = bl[((int64_t)s * NCB + cb) * 64];
  };

  int s = s_begin + w;
  u32x4 a_cur[MT], b_cur[NCB];
  if (s < s_end) load(s, a_cur, b_cur);
  for (; s < s_end; s += NW) {
    u32x4 a_nxt[MT], b_nxt[NCB];
    const bool more = s + NW < s_end;
    if (more) load(s + NW, a_nxt, b_nxt);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a_cur[mt]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[mt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b_cur[cb]),
                                                              acc[mt][cb], 0, 0, 0);
      // Sum of squares from the same A fragment: v_dot2 of each bf16 pair with
      // itself. The four dwords are named explicitly: indexing the vector with
      // the unrolled loop variable inside the bit_cast made this compiler read
      // the first dword four times.
      const u32x4 aw = a_cur[mt];
      ss[mt] = dot2_self(aw.x, ss[mt]);
      ss[mt] = dot2_self(aw.y, ss[mt]);
      ss[mt] = dot2_self(aw.z, ss[mt]);
      ss[mt] = dot2_self(aw.w, ss[mt]);
    }
    if (more) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a_cur[mt] = a_nxt[mt];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) b_cur[cb] = b_nxt[cb];
    }
  }

  // Lanes r16, r16+16, r16+32, r16+48 hold the same token row's squares.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ss[mt] += __shfl_xor(ss[mt], 16);
    ss[mt] += __shfl_xor(ss[mt], 32);
  }
  // C tile layout: lane holds rows 4*q + i (i = 0..3), column r16 of block cb.
  float* rw = red + w * (MT * 16 * CW);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rw[(mt * 16 + q * 4 + i) * CW + cb * 16 + r16] = acc[mt][cb][i];
    if (q == 0) rw[(mt * 16 + r16) * CW + NCB * 16] = ss[mt];
  }
  __syncthreads();

  // partial[split][token][c] = sum over waves of (hi + lo) for c < N, squares at c = N.
  const int outs = MT * 16 * (N + 1);
  for (int idx = threadIdx.x; idx < outs; idx += NW * 64) {
    const int row = idx / (N + 1);
    const int c = idx - row * (N + 1);
    const int64_t tok = tok0 + row;
    if (tok >= T) continue;
    float v = 0.0f;
    if (c < N) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float* r = red + ww * (MT * 16 * CW) + row * CW;
        v += r[c] + r[c + N];
      }
    } else {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) v += red[ww * (MT * 16 * CW) + row * CW + NCB * 16];
    }
    part[((int64_t)split * T + tok) * NP + c] = v;
  }
}

// ------------------------------------------------------------------ f32 GEMM
// One wave per (token, split); lanes stride over k; butterfly reduction.
constexpr int kF32MaxN = 24;

__global__ __launch_bounds__(256) void pre_gemm_f32_kernel(const float* __restrict__ x, const float* __restrict__ fn,
                                                           float* __restrict__ part, int64_t T, int64_t K, int N,
                                                           int NP, int64_t k_per_split) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wave leaves; this kernel has no barrier
  const int split = blockIdx.y;
  const int64_t kb = (int64_t)split * k_per_split;
  const int64_t ke = min(K, kb + k_per_split);
  float acc[kF32MaxN];
#pragma unroll
  for (int c = 0; c < kF32MaxN; ++c) acc[c] = 0.0f;
  float ss = 0.0f;
  const float* xt = x + t * K;
  for (int64_t k = kb + lane; k < ke; k += 64) {
    const float v = xt[k];
    ss = fmaf(v, v, ss);
    const float* f = fn + k * N;
#pragma unroll
    for (int c = 0; c < kF32MaxN; ++c)
      if (c < N) acc[c] = fmaf(v, f[c], acc[c]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ss += __shfl_xor(ss, off);
#pragma unroll
    for (int c = 0; c < kF32MaxN; ++c) acc[c] += __shfl_xor(acc[c], off);
  }
  if (lane == 0) {
    float* o = part + ((int64_t)split * T + t) * NP;
#pragma unroll
    for (int c = 0; c < kF32MaxN; ++c)
      if (c < N) o[c] = acc[c];
    o[N] = ss;
  }
}

template <int MT, int NW>
static hipError_t launch_gemm_bf16_ncb(const PrePlan& p, const uint16_t* x, const u32x4* fnp, float* part,
                                       hipStream_t s) {
  const dim3 grid((unsigned)((p.T + 16 * MT - 1) / (16 * MT)), (unsigned)p.S);
  const dim3 block(NW * 64);
  switch (p.NCB) {
    case 1:
      hipLaunchKernelGGL((pre_gemm_bf16_kernel<MT, NW, 1>), grid, block, 0, s, x, fnp, part, p.T, p.K, p.N, p.NP,
                         p.ksteps, p.steps_per_split);
      break;
    case 2:
      hipLaunchKernelGGL((pre_gemm_bf16_kernel<MT, NW, 2>), grid, block, 0, s, x, fnp, part, p.T, p.K, p.N, p.NP,
                         p.ksteps, p.steps_per_split);
      break;
    default:
      hipLaunchKernelGGL((pre_gemm_bf16_kernel<MT, NW, 3>), grid, block, 0, s, x, fnp, part, p.T, p.K, p.N, p.NP,
                         p.ksteps, p.steps_per_split);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_pre_gemm(const PrePlan& p, const void* residual, const void* fnp, const float* fn, float* part,
                           hipStream_t s) {
  if (p.dt == MHC_F32) {
    const dim3 grid((unsigned)((p.T + 3) / 4), (unsigned)p.S);
    const int64_t kps = (int64_t)p.steps_per_split * 64;
    hipLaunchKernelGGL(pre_gemm_f32_kernel, grid, dim3(256), 0, s, static_cast<const float*>(residual), fn, part,
                       p.T, p.K, p.N, p.NP, kps);
    return hipGetLastError();
  }
  const uint16_t* x = static_cast<const uint16_t*>(residual);
  const u32x4* f = static_cast<const u32x4*>(fnp);
  if (p.MT == 1) return launch_gemm_bf16_ncb<1, 16>(p, x, f, part, s);
  return launch_gemm_bf16_ncb<4, 4>(p, x, f, part, s);
}

// ------------------------------------------------------------------ epilogue + y
// One 256-thread workgroup per token. The token row (n streams x D) is
// prefetched in 16-byte vectors first; wave 0 meanwhile reduces the split
// partials and runs the gates and Sinkhorn with lane e = 4 i + j holding
// comb[i][j] (rows: xor 1, 2; columns: xor 4, 8; padded to 4 x 4 for n < 4).
constexpr int kEpiThreads = 256;

template <class S, int NS, int CPT>
__global__ __launch_bounds__(kEpiThreads) void pre_epilogue_kernel(
    const typename S::elem* __restrict__ x, const float* __restrict__ part, int nsplit, int NP,
    const float* __restrict__ hc_scale, const float* __restrict__ bias, float* __restrict__ post,
    float* __restrict__ comb, typename S::elem* __restrict__ y, int64_t T, int64_t D, int repeat, float eps) {
  constexpr int V = S::V;
  constexpr int N = NS * (NS + 2);
  __shared__ float pre_s[NS];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t nch = D / V;
  const typename S::elem* xt = x + t * NS * D;
  typename S::elem* yt = y + t * D;

  u32x4 buf[CPT][NS];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = tid + (int64_t)j * kEpiThreads;
    if (c < nch)
#pragma unroll
      for (int i = 0; i < NS; ++i) buf[j][i] = ld16(xt + i * D + c * V);
  }

  if (tid < kWave) {
    const int e = tid & 15;
    const int i = e >> 2, jj = e & 3;
    const bool act = i < NS && jj < NS;
    const float* pt = part + t * NP;
    const int64_t sstride = T * NP;
    float ssq = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) ssq += pt[sp * sstride + N];
    const float r = 1.0f / sqrtf(ssq / (float)(NS * D) + eps);

    float zc = -INFINITY;
    if (act) {
      const int c = 2 * NS + i * NS + jj;
      float m = 0.0f;
      for (int sp = 0; sp < nsplit; ++sp) m += pt[sp * sstride + c];
      zc = hc_scale[2] * (r * m) + bias[c];
    }
    if (tid < 2 * NS) {
      const int c = tid;
      float m = 0.0f;
      for (int sp = 0; sp < nsplit; ++sp) m += pt[sp * sstride + c];
      const float g = sigmoidf_ieee(hc_scale[c < NS ? 0 : 1] * (r * m) + bias[c]);
      if (c < NS) pre_s[c] = g;
      else post[t * NS + (c - NS)] = g;
    }
    float rmax = zc;
    rmax = fmaxf(rmax, __shfl_xor(rmax, 1));
    rmax = fmaxf(rmax, __shfl_xor(rmax, 2));
    float M = act ? expf(zc - rmax) : 0.0f;
    for (int it = 0; it < repeat; ++it) {
      float rs = M + __shfl_xor(M, 1);
      rs = rs + __shfl_xor(rs, 2);
      M = act ? M / rs : 0.0f;
      float cs = M + __shfl_xor(M, 4);
      cs = cs + __shfl_xor(cs, 8);
      M = act ? M / cs : 0.0f;
    }
    if (act && tid < 16) comb[t * NS * NS + i * NS + jj] = M;
  }
  __syncthreads();

  float p[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) p[i] = pre_s[i];

  auto emit = [&](int64_t c, const u32x4* xs) {
    float acc[V];
    float f[V];
    Vec<S>::unpack(xs[0], f);
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = p[0] * f[v];
#pragma unroll
    for (int i = 1; i < NS; ++i) {
      Vec<S>::unpack(xs[i], f);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = fmaf(p[i], f[v], acc[v]);
    }
    st16(yt + c * V, Vec<S>::pack(acc));
  };

#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = tid + (int64_t)j * kEpiThreads;
    if (c < nch) emit(c, buf[j]);
  }
  // Rows longer than one prefetch pass (D > 256 * CPT * V) continue here.
  for (int64_t base = (int64_t)kEpiThreads * CPT; base < nch; base += (int64_t)kEpiThreads * CPT) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = base + tid + (int64_t)j * kEpiThreads;
      if (c < nch)
#pragma unroll
        for (int i = 0; i < NS; ++i) buf[j][i] = ld16(xt + i * D + c * V);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = base + tid + (int64_t)j * kEpiThreads;
      if (c < nch) emit(c, buf[j]);
    }
  }
}

template <class S, int NS>
static hipError_t launch_epi_n(const PrePlan& p, const void* residual, const float* part, const float* hc_scale,
                               const float* bias, float* post, float* comb, void* y, int repeat, float eps,
                               hipStream_t s) {
  typedef typename S::elem E;
  const int64_t nch = p.D / S::V;
  int cpt = (int)((nch + kEpiThreads - 1) / kEpiThreads);
  cpt = cpt < 1 ? 1 : (cpt > 4 ? 4 : cpt);
  const dim3 grid((unsigned)p.T), block(kEpiThreads);
  const E* x = static_cast<const E*>(residual);
  E* yy = static_cast<E*>(y);
#define MHC_EPI(C)                                                                                                 \
  hipLaunchKernelGGL((pre_epilogue_kernel<S, NS, C>), grid, block, 0, s, x, part, p.S, p.NP, hc_scale, bias, post, \
                     comb, yy, p.T, p.D, repeat, eps)
  switch (cpt) {
    case 1: MHC_EPI(1); break;
    case 2: MHC_EPI(2); break;
    case 3: MHC_EPI(3); break;
    default: MHC_EPI(4); break;
  }
#undef MHC_EPI
  return hipGetLastError();
}

template <class S>
static hipError_t launch_epi_s(const PrePlan& p, const void* residual, const float* part, const float* hc_scale,
                               const float* bias, float* post, float* comb, void* y, int repeat, float eps,
                               hipStream_t s) {
  switch (p.n) {
    case 1: return launch_epi_n<S, 1>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, s);
    case 2: return launch_epi_n<S, 2>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, s);
    case 3: return launch_epi_n<S, 3>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, s);
    default: return launch_epi_n<S, 4>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, s);
  }
}

hipError_t launch_pre_epilogue(const PrePlan& p, const void* residual, const float* part, const float* hc_scale,
                               const float* bias, float* post, float* comb, void* y, int repeat, float eps,
                               hipStream_t s) {
  if (p.dt == MHC_F32) return launch_epi_s<F32>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, s);
  return launch_epi_s<BF16>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, s);
}

}  // namespace mhc
