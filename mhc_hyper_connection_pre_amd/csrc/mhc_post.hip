// mhc_post and the fused post + next-layer combine + RMSNorm on gfx950.
//
// mhc_post is the post call of sglang PR #24355 analysis ("AMD ROCm
// DeepSeek-V4 performance optimisation: Aiter MHC kernel integration"),
// section 2: out_j = post_j * h + sum_i comb[i][j] * residual_i, written into
// a tensor shaped like the residual. The fused variant follows sglang PR
// #39704 analysis ("DeepSeek-V4.1 performance optimisation: mHC and metadata
// overhead"), section 1 (one row per workgroup, combine into a bf16 row, then
// RMSNorm) and section 2 (the row is stored as `normalized`).
//
// Both kernels are pure HBM streams: one workgroup per token, 16-byte vector
// loads of h and the n residual streams, fp32 FMAs, one RNE rounding per
// stored value. post/comb are per-token scalars (uniform across the
// workgroup, so they live in SGPRs). All loads of a thread are issued before
// its first FMA so every wave keeps several vectors in flight.

#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

constexpr int kPostMaxThreads = 1024;   // rows of up to 1024 vectors: one vector per thread
constexpr int kPostWideThreads = 256;   // longer rows: up to four vectors per thread and round

template <class S, int NS, int CPT>
__global__ __launch_bounds__(CPT == 1 ? kPostMaxThreads : kPostWideThreads) void post_kernel(typename S::elem* __restrict__ out,
                                                            const typename S::elem* __restrict__ h,
                                                            const typename S::elem* __restrict__ x,
                                                            const float* __restrict__ post,
                                                            const float* __restrict__ comb, int64_t D) {
  constexpr int V = S::V;
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nch = D / V;
  float pj[NS], cij[NS][NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) pj[j] = post[t * NS + j];
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) cij[i][j] = comb[t * NS * NS + i * NS + j];
  const typename S::elem* ht = h + t * D;
  const typename S::elem* xt = x + t * NS * D;
  typename S::elem* ot = out + t * NS * D;

  const int nthr = blockDim.x;
  for (int64_t base = 0; base < nch; base += (int64_t)nthr * CPT) {
    u32x4 hv[CPT], xv[CPT][NS];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t c = base + tid + (int64_t)k * nthr;
      if (c < nch) {   // streaming loads: nothing of h or the residual is read twice here
        hv[k] = ld16_stream(ht + c * V);
#pragma unroll
        for (int i = 0; i < NS; ++i) xv[k][i] = ld16_stream(xt + i * D + c * V);
      }
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int64_t c = base + tid + (int64_t)k * nthr;
      if (c >= nch) continue;
      float hf[V], xf[NS][V];
      Vec<S>::unpack(hv[k], hf);
#pragma unroll
      for (int i = 0; i < NS; ++i) Vec<S>::unpack(xv[k][i], xf[i]);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
          float a = pj[j] * hf[v];
#pragma unroll
          for (int i = 0; i < NS; ++i) a = fmaf(cij[i][j], xf[i][v], a);
          o[v] = a;
        }
        st16_stream(ot + j * D + c * V, Vec<S>::pack(o));
      }
    }
  }
}

template <class S, int NS>
static hipError_t launch_post_n(const void* h, const void* residual, const float* post, const float* comb,
                                void* out, int64_t T, int64_t D, hipStream_t s) {
  typedef typename S::elem E;
  const int64_t nch = D / S::V;
  constexpr int kMaxCpt = NS > 4 ? 2 : 4;   // vectors in flight per thread: (n + 1) x CPT x 4 registers
  // one thread per 16-byte vector of the row, in whole waves, up to 1024:
  // at D = 7168 (896 threads, one vector of h and of each stream per thread)
  // this measured 48.5 us per call after a cache sweep against 52.4 us with
  // 256 threads holding four vectors each (T = 2048, n = 4), 354 against
  // 377 us at T = 16384; more waves per CU issue the same bytes sooner
  // (rows longer than 1024 vectors keep 256 threads with up to kMaxCpt
  // vectors each, within the registers that block size leaves)
  int threads = (int)((nch + 63) / 64 * 64), cpt = 1;
  if (nch > kPostMaxThreads) {
    threads = kPostWideThreads;
    cpt = (int)((nch + threads - 1) / threads);
    cpt = cpt < 2 ? 2 : (cpt > kMaxCpt ? kMaxCpt : cpt);
  }
  const dim3 grid((unsigned)T), block(threads);
  E* o = static_cast<E*>(out);
  const E* hh = static_cast<const E*>(h);
  const E* x = static_cast<const E*>(residual);
#define MHC_POST(C) hipLaunchKernelGGL((post_kernel<S, NS, C>), grid, block, 0, s, o, hh, x, post, comb, D)
  if constexpr (kMaxCpt == 2) {
    if (cpt == 1) MHC_POST(1);
    else MHC_POST(2);
  } else {
    switch (cpt) {
      case 1: MHC_POST(1); break;
      case 2: MHC_POST(2); break;
      case 3: MHC_POST(3); break;
      default: MHC_POST(4); break;
    }
  }
#undef MHC_POST
  return hipGetLastError();
}

template <class S>
static hipError_t launch_post_s(const void* h, const void* residual, const float* post, const float* comb,
                                void* out, int n, int64_t T, int64_t D, hipStream_t s) {
  switch (n) {
    case 1: return launch_post_n<S, 1>(h, residual, post, comb, out, T, D, s);
    case 2: return launch_post_n<S, 2>(h, residual, post, comb, out, T, D, s);
    case 3: return launch_post_n<S, 3>(h, residual, post, comb, out, T, D, s);
    case 8: return launch_post_n<S, 8>(h, residual, post, comb, out, T, D, s);
    default: return launch_post_n<S, 4>(h, residual, post, comb, out, T, D, s);
  }
}

hipError_t launch_post(const void* h, const void* residual, const float* post, const float* comb, void* out,
                       mhc_dtype dt, int64_t T, int n, int64_t D, hipStream_t s) {
  if (dt == MHC_F32) return launch_post_s<F32>(h, residual, post, comb, out, n, T, D, s);
  return launch_post_s<BF16>(h, residual, post, comb, out, n, T, D, s);
}

// ------------------------------------------------------------------ fused post + combine + RMSNorm
// One workgroup of up to 1024 threads per token (512 at n = 8, whose eight
// streams per vector need the registers of two waves per SIMD); each thread
// keeps at most CPT vectors of the combined row in registers (stored values,
// already rounded), so the row is read from HBM once. The sum of squares is
// reduced across the workgroup in a fixed order (wave butterfly, then LDS).
template <class S, int NS, int CPT>
__global__ __launch_bounds__(kPcnThreads<NS>) void post_combine_norm_kernel(
    typename S::elem* __restrict__ normalized, typename S::elem* __restrict__ out,
    const typename S::elem* __restrict__ h, const typename S::elem* __restrict__ x, const float* __restrict__ post,
    const float* __restrict__ comb, const float* __restrict__ combine_w, const float* __restrict__ norm_weight,
    float eps, int64_t D) {
  constexpr int V = S::V;
  __shared__ float wsum[16];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int64_t nch = D / V;
  float pj[NS], wj[NS], cij[NS][NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    pj[j] = post[t * NS + j];
    wj[j] = combine_w[t * NS + j];
  }
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int j = 0; j < NS; ++j) cij[i][j] = comb[t * NS * NS + i * NS + j];
  const typename S::elem* ht = h + t * D;
  const typename S::elem* xt = x + t * NS * D;

  u32x4 hv[CPT], xv[CPT][NS];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = tid + (int64_t)k * nthr;
    if (c < nch) {
      hv[k] = ld16(ht + c * V);
#pragma unroll
      for (int i = 0; i < NS; ++i) xv[k][i] = ld16(xt + i * D + c * V);
    }
  }

  float cv[CPT][V];
  float ssq = 0.0f;
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = tid + (int64_t)k * nthr;
    if (c >= nch) continue;
    float hf[V], xf[NS][V];
    Vec<S>::unpack(hv[k], hf);
#pragma unroll
    for (int i = 0; i < NS; ++i) Vec<S>::unpack(xv[k][i], xf[i]);
#pragma unroll
    for (int v = 0; v < V; ++v) cv[k][v] = 0.0f;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      float o[V];
#pragma unroll
      for (int v = 0; v < V; ++v) {
        float a = pj[j] * hf[v];
#pragma unroll
        for (int i = 0; i < NS; ++i) a = fmaf(cij[i][j], xf[i][v], a);
        o[v] = Vec<S>::round_trip(a);       // the stored post value
        cv[k][v] = fmaf(wj[j], o[v], cv[k][v]);
      }
      if (out != nullptr) st16_stream(out + (t * NS + j) * D + c * V, Vec<S>::pack(o));
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
      cv[k][v] = Vec<S>::round_trip(cv[k][v]);  // the combined row is held in the storage type
      ssq = fmaf(cv[k][v], cv[k][v], ssq);
    }
  }

#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ssq += __shfl_xor(ssq, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ssq;
  __syncthreads();
  float tot = 0.0f;
  const int nw = (nthr + 63) >> 6;
  for (int w = 0; w < nw; ++w) tot += wsum[w];
  const float qn = 1.0f / sqrtf(tot / (float)D + eps);

#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int64_t c = tid + (int64_t)k * nthr;
    if (c >= nch) continue;
    const float* g = norm_weight + c * V;
    float o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) o[v] = (cv[k][v] * qn) * g[v];
    st16_stream(normalized + t * D + c * V, Vec<S>::pack(o));
  }
}

template <class S, int NS>
static hipError_t launch_pcn_n(void* normalized, void* out, const void* h, const void* residual, const float* post,
                               const float* comb, const float* w, const float* g, float eps, int64_t T, int64_t D,
                               hipStream_t s) {
  typedef typename S::elem E;
  const int64_t nch = D / S::V;
  int64_t thr = ((nch + 63) / 64) * 64;
  if (thr > kPcnThreads<NS>) thr = kPcnThreads<NS>;
  const int cpt = (int)((nch + thr - 1) / thr);
  const dim3 grid((unsigned)T), block((unsigned)thr);
  E* nz = static_cast<E*>(normalized);
  E* o = static_cast<E*>(out);
  const E* hh = static_cast<const E*>(h);
  const E* x = static_cast<const E*>(residual);
#define MHC_PCN(C) \
  hipLaunchKernelGGL((post_combine_norm_kernel<S, NS, C>), grid, block, 0, s, nz, o, hh, x, post, comb, w, g, eps, D)
  switch (cpt) {
    case 1: MHC_PCN(1); break;
    case 2: MHC_PCN(2); break;
    case 3: MHC_PCN(3); break;
    default: MHC_PCN(4); break;
  }
#undef MHC_PCN
  return hipGetLastError();
}

template <class S>
static hipError_t launch_pcn_s(void* normalized, void* out, const void* h, const void* residual, const float* post,
                               const float* comb, const float* w, const float* g, float eps, int n, int64_t T,
                               int64_t D, hipStream_t s) {
  switch (n) {
    case 1: return launch_pcn_n<S, 1>(normalized, out, h, residual, post, comb, w, g, eps, T, D, s);
    case 2: return launch_pcn_n<S, 2>(normalized, out, h, residual, post, comb, w, g, eps, T, D, s);
    case 3: return launch_pcn_n<S, 3>(normalized, out, h, residual, post, comb, w, g, eps, T, D, s);
    case 8: return launch_pcn_n<S, 8>(normalized, out, h, residual, post, comb, w, g, eps, T, D, s);
    default: return launch_pcn_n<S, 4>(normalized, out, h, residual, post, comb, w, g, eps, T, D, s);
  }
}

hipError_t launch_post_combine_norm(void* normalized, void* out, const void* h, const void* residual,
                                    const float* post, const float* comb, const float* combine_w,
                                    const float* norm_weight, float eps, mhc_dtype dt, int64_t T, int n, int64_t D,
                                    hipStream_t s) {
  if (dt == MHC_F32)
    return launch_pcn_s<F32>(normalized, out, h, residual, post, comb, combine_w, norm_weight, eps, n, T, D, s);
  return launch_pcn_s<BF16>(normalized, out, h, residual, post, comb, combine_w, norm_weight, eps, n, T, D, s);
}

}  // namespace mhc
