// mhc_pre on gfx950: RMS factor + split-K mixing GEMM, then gates, Sinkhorn and
// the pre-weighted stream reduce.
//
// The pre step of an mHC layer boundary: sglang PR #24355 analysis ("AMD ROCm
// DeepSeek-V4 performance optimisation: Aiter MHC kernel integration"),
// section 2 (the pre call returning post, comb, y) and section 3 (a split-K
// GEMM fused with the per-token sum of squares, tiled over the hidden axis).
//
// Three launches on the caller's stream:
//   1. pack_fn        fn fp32 [K, N] -> bf16 hi/lo(/lo2) terms in MFMA B-fragment order
//   2. pre_gemm       residual x [T, K] (bf16) x [fn_hi | fn_lo | fn_lo2] on MFMA
//                     16x16x32, plus sum of squares with v_dot2; one fp32
//                     partial row (N sums + sum of squares) per token and split
//   3. pre_epilogue   one workgroup per token: fixed-order split reduction,
//                     RMS factor, hc_scale, bias, sigmoid gates, Sinkhorn in
//                     registers of 16 lanes, then y = sum_i pre_i x_i from the
//                     token row prefetched before the epilogue runs.
// The fp32-residual path replaces 1-2 with a VALU dot-product kernel.
//
// fn is split into bf16 terms hi = bf16(fn), lo = bf16(fn - hi) and, for the
// pre-gate columns, lo2 = bf16(fn - hi - lo) (mhc_pack.h): x is exact in bf16,
// so with fp32 MFMA accumulation the mixing sums reach about 2^-17 relative
// (2^-24 for the pre columns).

#include "mhc_device.h"
#include "mhc_epilogue.h"
#include "mhc_pack.h"
#include "mhc_internal.h"

namespace mhc {

// ------------------------------------------------------------------ packing
__global__ __launch_bounds__(256) void pack_fn_kernel(const float* __restrict__ fn, u32x4* __restrict__ fnp,
                                                      int64_t K, int N, int NCB, int ksteps, bool vec4) {
  __shared__ float tile[kPackSteps * 32 * (kPackMaxN + 1)];
  pack_fn_block(fn, fnp, K, N, NCB, ksteps, vec4, tile);
}

template <int N, int NCB>
__global__ __launch_bounds__(256) void pack_fn_kernel_n(const float* __restrict__ fn, u32x4* __restrict__ fnp,
                                                        int64_t K, int ksteps, bool vec4) {
  __shared__ float tile[kPackSteps * 32 * (kPackMaxN + 1)];
  pack_fn_block(fn, fnp, K, N, NCB, ksteps, vec4, tile);
}

hipError_t launch_pack_fn(const PrePlan& p, const float* fn, void* fnp, hipStream_t s) {
  const unsigned blocks = (unsigned)((p.ksteps + kPackSteps - 1) / kPackSteps);
  const bool vec4 = (reinterpret_cast<uintptr_t>(fn) & 15) == 0;
  // n = 4 and n = 8 with the column counts as constants (the packing's index
  // arithmetic then has no runtime divisions: 15.1 -> 13.5 us at n = 8,
  // D = 7168); other n with them as arguments
  if (p.N == 80 && p.NCB == pack_blocks(8)) {
    hipLaunchKernelGGL((pack_fn_kernel_n<80, pack_blocks(8)>), dim3(blocks), dim3(256), 0, s, fn,
                       reinterpret_cast<u32x4*>(fnp), p.K, p.ksteps, vec4);
    return hipGetLastError();
  }
  if (p.N == 24 && p.NCB == pack_blocks(4)) {
    hipLaunchKernelGGL((pack_fn_kernel_n<24, pack_blocks(4)>), dim3(blocks), dim3(256), 0, s, fn,
                       reinterpret_cast<u32x4*>(fnp), p.K, p.ksteps, vec4);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(pack_fn_kernel, dim3(blocks), dim3(256), 0, s, fn, reinterpret_cast<u32x4*>(fnp), p.K, p.N,
                     p.NCB, p.ksteps, vec4);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bf16 GEMM
// Workgroup = NW waves = one tile of 16*MT tokens x one split of the k-steps.
// Wave w takes k-steps s_begin + w, + NW, ... (the NW waves read NW adjacent
// 64-byte segments of every row at a time). Each wave keeps MT x NCB fp32
// accumulator tiles; the waves are summed in LDS in a fixed order.
// Four-wave workgroups get the register budget of two waves per SIMD, so
// that two of them share a CU: left free, the compiler gave the n = 4 kernel
// (four 16-token tiles per wave) 160 VGPRs and 128 AGPRs, one wave per SIMD,
// and a CU then had half the residual loads in flight (per pre call after a
// cache sweep, T = 16384, n = 4, D = 7168: 462 -> 449 us with 4 splits,
// 494 -> 459 us with 8; T = 2048 with 4 splits: 88 -> 83.5 us).
// PAIR (four waves): waves 0 and 1 store their tiles in LDS, then waves 2
// and 3 add theirs to the same places, so the sums take half the LDS; for
// n = 8 (eleven column blocks; with a shorter prefetch ring to fit the
// budget) that is what lets two workgroups share a CU: T = 2048, D = 7168,
// 176 -> 165 us per pre call; T = 16384: 1274 -> 1197 us.
template <int MT, int NW, int NCB, int PF = 3, bool PAIR = false>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void pre_gemm_bf16_kernel(const uint16_t* __restrict__ x,
                                                                const u32x4* __restrict__ fnp,
                                                                float* __restrict__ part, int64_t T, int64_t K,
                                                                int N, int NP, int ksteps, int steps_per_split) {
  constexpr int CW = NCB * 16 + 1;  // LDS row: padded [hi | lo | lo2] columns, then the sum of squares
  static_assert(!PAIR || NW == 4, "the paired reduction is written for four waves");
  constexpr int RW = PAIR ? 2 : NW;   // wave tiles held in LDS at once
  __shared__ float red[RW * MT * 16 * CW];
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
    // Loads are unconditional from an in-bounds address (row 0 / k 0 stand in
    // for rows past T and the K tail) and masked afterwards: no branches.
    const int64_t k = (int64_t)s * 32;
    const bool kok = k + q * 8 < K;
    const int64_t ko = kok ? k : 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 v = ld16(arow[mt] + ko);
      a[mt] = (rok[mt] && kok) ? v : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) b[cb] = bl[((int64_t)s * NCB + cb) * 64];
  };

  // Prefetch ring of PF k-steps per wave: step j of this wave is
  // s_begin + w + j * NW. Buffer p holds step j + p; after it is consumed it
  // is refilled with step j + p + PF (clamped to the wave's last step, so
  // every load is in bounds and the load count per iteration is fixed).
  const int s0 = s_begin + w;
  const int nst = s0 < s_end ? (s_end - s0 + NW - 1) / NW : 0;
  auto compute = [&](const u32x4* a, const u32x4* b) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, a[mt]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[mt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b[cb]), acc[mt][cb], 0, 0,
                                                              0);
      // Sum of squares from the same A fragment: v_dot2 of each bf16 pair with
      // itself. The four dwords are named explicitly: indexing the vector with
      // the unrolled loop variable inside the bit_cast made this compiler read
      // the first dword four times.
      const u32x4 aw = a[mt];
      ss[mt] = dot2_self(aw.x, ss[mt]);
      ss[mt] = dot2_self(aw.y, ss[mt]);
      ss[mt] = dot2_self(aw.z, ss[mt]);
      ss[mt] = dot2_self(aw.w, ss[mt]);
    }
  };
  if (nst > 0) {
    u32x4 abuf[PF][MT], bbuf[PF][NCB];
#pragma unroll
    for (int p = 0; p < PF; ++p) load(s0 + min(p, nst - 1) * NW, abuf[p], bbuf[p]);
    int j = 0;
    for (; j + PF <= nst; j += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        compute(abuf[p], bbuf[p]);
        load(s0 + min(j + p + PF, nst - 1) * NW, abuf[p], bbuf[p]);
      }
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < nst - j) compute(abuf[p], bbuf[p]);
  }

  // Lanes r16, r16+16, r16+32, r16+48 hold the same token row's squares.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ss[mt] += __shfl_xor(ss[mt], 16);
    ss[mt] += __shfl_xor(ss[mt], 32);
  }
  // C tile layout: lane holds rows 4*q + i (i = 0..3), column r16 of block cb.
  if constexpr (PAIR) {
    // place (w & 1): wave w & 1 stores, then wave (w & 1) + 2 adds (each lane
    // to the elements it stored itself), so each place holds w0 + w2 or w1 + w3
    float* rw = red + (w & 1) * (MT * 16 * CW);
    for (int ph = 0; ph < 2; ++ph) {
      if ((w >> 1) == ph) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float& d = rw[(mt * 16 + q * 4 + i) * CW + cb * 16 + r16];
              d = ph ? d + acc[mt][cb][i] : acc[mt][cb][i];
            }
          if (q == 0) {
            float& d = rw[(mt * 16 + r16) * CW + NCB * 16];
            d = ph ? d + ss[mt] : ss[mt];
          }
        }
      }
      __syncthreads();
    }
  } else {
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
  }

  // partial[split][token][c] = sum over the LDS places of (hi + lo (+ lo2
  // for the first n columns)) for c < N, squares at c = N.
  const int outs = MT * 16 * (N + 1);
  const int npre = n_pre(N);
  for (int idx = threadIdx.x; idx < outs; idx += NW * 64) {
    const int row = idx / (N + 1);
    const int c = idx - row * (N + 1);
    const int64_t tok = tok0 + row;
    if (tok >= T) continue;
    float v = 0.0f;
    if (c < N) {
#pragma unroll
      for (int ww = 0; ww < RW; ++ww) {
        const float* r = red + ww * (MT * 16 * CW) + row * CW;
        v += c < npre ? r[c] + r[c + N] + r[c + 2 * N] : r[c] + r[c + N];
      }
    } else {
#pragma unroll
      for (int ww = 0; ww < RW; ++ww) v += red[ww * (MT * 16 * CW) + row * CW + NCB * 16];
    }
    part[((int64_t)split * T + tok) * NP + c] = v;
  }
}

// ------------------------------------------------------------------ f32 GEMM
// One wave per (token, split); lanes stride over k; butterfly reduction.
// kF32MaxN: N = n (n + 2) sums per lane (24 for n <= 4, 80 for n = 8).
template <int kF32MaxN>
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

template <int MT, int NW, int NCB, int PF = 3, bool PAIR = false>
static void launch_gemm_bf16(const PrePlan& p, const uint16_t* x, const u32x4* fnp, float* part, hipStream_t s) {
  const dim3 grid((unsigned)((p.T + 16 * MT - 1) / (16 * MT)), (unsigned)p.S);
  hipLaunchKernelGGL((pre_gemm_bf16_kernel<MT, NW, NCB, PF, PAIR>), grid, dim3(NW * 64), 0, s, x, fnp, part, p.T,
                     p.K, p.N, p.NP, p.ksteps, p.steps_per_split);
}

template <int MT, int NW>
static hipError_t launch_gemm_bf16_ncb(const PrePlan& p, const uint16_t* x, const u32x4* fnp, float* part,
                                       hipStream_t s) {
  switch (p.NCB) {
    case 1: launch_gemm_bf16<MT, NW, 1>(p, x, fnp, part, s); break;
    case 2: launch_gemm_bf16<MT, NW, 2>(p, x, fnp, part, s); break;
    case 3: launch_gemm_bf16<MT, NW, 3>(p, x, fnp, part, s); break;
    default: launch_gemm_bf16<MT, NW, 4>(p, x, fnp, part, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_pre_gemm(const PrePlan& p, const void* residual, const void* fnp, const float* fn, float* part,
                           hipStream_t s) {
  if (p.dt == MHC_F32) {
    const dim3 grid((unsigned)((p.T + 3) / 4), (unsigned)p.S);
    const int64_t kps = (int64_t)p.steps_per_split * 64;
    const float* x = static_cast<const float*>(residual);
    if (p.N <= 24)
      hipLaunchKernelGGL(pre_gemm_f32_kernel<24>, grid, dim3(256), 0, s, x, fn, part, p.T, p.K, p.N, p.NP, kps);
    else
      hipLaunchKernelGGL(pre_gemm_f32_kernel<80>, grid, dim3(256), 0, s, x, fn, part, p.T, p.K, p.N, p.NP, kps);
    return hipGetLastError();
  }
  const uint16_t* x = static_cast<const uint16_t*>(residual);
  const u32x4* f = static_cast<const u32x4*>(fnp);
  if (p.n == 8) {   // 11 column blocks, four waves, MT 16-token tiles per wave, two workgroups per CU
    if (p.MT == 2)
      launch_gemm_bf16<2, 4, pack_blocks(8), 2, true>(p, x, f, part, s);
    else
      launch_gemm_bf16<1, 4, pack_blocks(8), 2, true>(p, x, f, part, s);
    return hipGetLastError();
  }
  if (p.MT == 1) return launch_gemm_bf16_ncb<1, 16>(p, x, f, part, s);
  return launch_gemm_bf16_ncb<4, 4>(p, x, f, part, s);
}

// ------------------------------------------------------------------ epilogue + y
// One 256-thread workgroup per token. The token row (n streams x D) is
// prefetched in 16-byte vectors first; wave 0 meanwhile reduces the split
// partials and runs the gates and Sinkhorn with lane e = 4 i + j holding
// comb[i][j] (rows: xor 1, 2; columns: xor 4, 8; padded to 4 x 4 for n < 4),
// or, for n = 8, lane e = 8 i + j on the whole wave.
constexpr int kEpiThreads = 256;

template <class S, int NS, int CPT>
__global__ __launch_bounds__(kEpiThreads) void pre_epilogue_kernel(
    const typename S::elem* __restrict__ x, const float* __restrict__ part, int nsplit, int NP,
    const float* __restrict__ hc_scale, const float* __restrict__ bias, float* __restrict__ post,
    float* __restrict__ comb, typename S::elem* __restrict__ y, int64_t T, int64_t D, int repeat, float eps,
    unsigned long long* __restrict__ status) {
  constexpr int V = S::V;
  constexpr int N = NS * (NS + 2);
  __shared__ float pre_s[NS];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t nch = D / V;
  const typename S::elem* xt = x + t * NS * D;
  typename S::elem* yt = y + t * D;
  // The two-pass path overwrites the region where the single-pass path keeps
  // its tagged exchange words: clear that path's shape marker (its next call
  // zeroes the region first) and its time-out record.
  if (t == 0 && tid == 0) {
    status[kStMarker] = 0;
    status[kStTimeout] = 0;
  }

  u32x4 buf[CPT][NS];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = tid + (int64_t)j * kEpiThreads;
    if (c < nch)
#pragma unroll
      for (int i = 0; i < NS; ++i) buf[j][i] = ld16(xt + i * D + c * V);
  }

  if (tid < kWave) {
    // Lane e of wave 0 sums columns e and e + CS of the split partials (the
    // sum of squares is column N) in ascending split order; the loads of each
    // group of 8 splits are in flight together. CS = 16 lanes run the epilogue
    // for n <= 4 (lanes 16..63 repeat lane & 15), the whole wave for n = 8.
    constexpr bool kWide = NS > 4;
    constexpr int CS = kWide ? 64 : 16;
    const int e = tid & (CS - 1);
    const EpiConst kc = kWide ? epi_const64<NS>(hc_scale, bias) : epi_const<NS>(hc_scale, bias);
    const float* pt = part + t * NP;
    const int64_t sstride = T * NP;
    float v0 = 0.0f, v1 = 0.0f;
    for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {
      float a0[8], a1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = sp0 + u < nsplit;
        a0[u] = (in && e <= N) ? pt[(int64_t)(sp0 + u) * sstride + e] : 0.0f;
        a1[u] = (in && e + CS <= N) ? pt[(int64_t)(sp0 + u) * sstride + e + CS] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v0 += a0[u];
        v1 += a1[u];
      }
    }
    float gate, combv;
    if constexpr (kWide) {
      epilogue64<NS>(v0, v1, kc, (float)(NS * D), eps, repeat, gate, combv);
    } else {
      epilogue16<NS>(v0, v1, kc, (float)(NS * D), eps, repeat, gate, combv);
    }
    if (tid < NS) pre_s[tid] = gate;
    else if (tid < 2 * NS) post[t * NS + (tid - NS)] = gate;
    constexpr int RW = kWide ? 8 : 4;   // lanes per row of the padded comb layout
    if (tid < RW * RW && e / RW < NS && e % RW < NS) comb[t * NS * NS + (e / RW) * NS + e % RW] = combv;
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
    st16_stream(yt + c * V, Vec<S>::pack(acc));
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
                               unsigned long long* status, hipStream_t s) {
  typedef typename S::elem E;
  const int64_t nch = p.D / S::V;
  constexpr int kMaxCpt = NS > 4 ? 2 : 4;   // prefetched vectors per thread: n x CPT x 4 registers
  int cpt = (int)((nch + kEpiThreads - 1) / kEpiThreads);
  cpt = cpt < 1 ? 1 : (cpt > kMaxCpt ? kMaxCpt : cpt);
  const dim3 grid((unsigned)p.T), block(kEpiThreads);
  const E* x = static_cast<const E*>(residual);
  E* yy = static_cast<E*>(y);
#define MHC_EPI(C)                                                                                                 \
  hipLaunchKernelGGL((pre_epilogue_kernel<S, NS, C>), grid, block, 0, s, x, part, p.S, p.NP, hc_scale, bias, post, \
                     comb, yy, p.T, p.D, repeat, eps, status)
  if constexpr (kMaxCpt == 2) {
    if (cpt == 1) MHC_EPI(1);
    else MHC_EPI(2);
  } else {
    switch (cpt) {
      case 1: MHC_EPI(1); break;
      case 2: MHC_EPI(2); break;
      case 3: MHC_EPI(3); break;
      default: MHC_EPI(4); break;
    }
  }
#undef MHC_EPI
  return hipGetLastError();
}

template <class S>
static hipError_t launch_epi_s(const PrePlan& p, const void* residual, const float* part, const float* hc_scale,
                               const float* bias, float* post, float* comb, void* y, int repeat, float eps,
                               unsigned long long* status, hipStream_t s) {
  switch (p.n) {
    case 1: return launch_epi_n<S, 1>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
    case 2: return launch_epi_n<S, 2>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
    case 3: return launch_epi_n<S, 3>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
    case 8: return launch_epi_n<S, 8>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
    default: return launch_epi_n<S, 4>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
  }
}

hipError_t launch_pre_epilogue(const PrePlan& p, const void* residual, const float* part, const float* hc_scale,
                               const float* bias, float* post, float* comb, void* y, int repeat, float eps,
                               unsigned long long* status, hipStream_t s) {
  if (p.dt == MHC_F32)
    return launch_epi_s<F32>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
  return launch_epi_s<BF16>(p, residual, part, hc_scale, bias, post, comb, y, repeat, eps, status, s);
}

}  // namespace mhc
