// Single-pass mhc_pre on gfx950: the residual is read from HBM once.
//
// The pre step (sglang PR #24355 analysis, "AMD ROCm DeepSeek-V4 performance
// optimisation: Aiter MHC kernel integration", section 2: the pre call returns
// post, comb and y; section 3: the GEMM is split over the hidden axis and fused
// with the sum of squares) needs a reduction over all n*D hidden elements of a
// token before y = sum_i pre_i x_i can be formed. A two-pass design reads the
// residual twice; here a workgroup keeps its residual slice in registers while
// the slices of its token tile exchange partial sums through memory.
//
// Work split: a work item is (tile, slice): TM = 64 tokens x all n streams x
// the hidden positions [128 s, 128 s + 128). Wave w holds tokens 16 w .. 16 w
// + 15 x n streams x 128 positions as MFMA A fragments (64 VGPRs at n = 4).
// The grid is persistent: P = G x S workgroups, all resident at once (two per
// CU), workgroup b always takes slice s = b % S and tiles b / S, + G, + 2G...
// So each workgroup packs its slice of fn into LDS once (bf16 hi/lo B
// fragments, 48 KB at n = 4) and software-pipelines its tiles: the residual
// slice of the next tile is loaded while the current tile's partial sums are
// exchanged, so HBM stays busy during the exchange latency. The split-K GEMM
// runs on v_mfma_f32_16x16x32_bf16 and the sum of squares on v_dot2.
//
// Exchange protocol: every exchanged value is a 64-bit word, tag (low 32 bits
// of this call's epoch) in the high half and fp32 bits in the low half,
// written with an agent-scope relaxed atomic store (write-through, no wait)
// and polled with agent-scope relaxed atomic loads until every tag matches.
// The epoch lives in the workspace: a call uses (last finished epoch) + 1 and
// the last workgroup to finish records it, so a graph replay gets a new one
// too, and a word left by an earlier call never matches. When the workspace's
// shape marker differs (first use, another shape or the two-pass path since),
// the workgroups first zero the tag region and meet at a grid barrier. Steps
// per tile:
//   1. partial[s][token][0..N] (N mixing sums + sum of squares)
//   2. workgroup s finalises tokens s, s + S, ... of the tile: it reduces
//      their S partial rows in a fixed order, runs the gates and Sinkhorn (16
//      lanes per token), writes post and comb and publishes pre
//   3. every wave reads pre for its 16 tokens and writes y for its slice.
// Every poll gives up after 100 ms (wall clock) and records the call as timed
// out in the workspace, so the kernel always terminates.
//
// Deadlock freedom: a work item waits only for items of its own tile. With
// P <= the resident capacity and S <= P, the lowest unfinished tile's items
// are all held by running workgroups whose earlier items (lower tiles) are
// done, so that tile completes; by induction every tile does.

#include <atomic>

#include "mhc_device.h"
#include "mhc_epilogue.h"
#include "mhc_internal.h"

namespace mhc {

namespace {

constexpr int kTM = 64;         // tokens per tile
constexpr int kDS = 128;        // hidden positions per slice
constexpr int kCPS = kDS / 32;  // 32-position k-steps per stream
constexpr int kThreads = 256;   // 4 waves x 16 tokens
constexpr int kLoads = 16;      // partial words per thread per finalise batch
constexpr int kMaxSplits = 128;
constexpr long long kPollTicks = 10000000LL;  // 100 ms of the 100 MHz wall clock

typedef unsigned long long u64;

__device__ __forceinline__ void put_tagged(u64* p, unsigned tag, float v) {
  __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_agent(const u64* p) {
  return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(u64 w, unsigned tag) { return (unsigned)(w >> 32) == tag; }
__device__ __forceinline__ float tag_val(u64 w) { return __uint_as_float((unsigned)(w & 0xffffffffull)); }
// Arrival counters (one atomic add per workgroup; the last arrival of a call
// sets them back to zero).
__device__ __forceinline__ u64 count_in(u64* p) {
  return __hip_atomic_fetch_add(p, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
}
// Wait until this wave's outstanding vector memory operations (loads and
// stores) have completed: vmcnt = 0, other counters unconstrained.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0f70); }

}  // namespace

struct FusedArgs {
  const uint16_t* x;
  const float* fn;
  const float* hc_scale;
  const float* bias;
  float* post;
  float* comb;
  uint16_t* y;
  u64* part;          // [S][T][N + 1] tagged
  u64* prebuf;        // [T][4] tagged
  u64* status;        // status words (kSt*)
  u64 marker;
  int64_t ntag;       // tagged words from part to the end of prebuf
  int64_t T, D;
  int S, G, P, repeat;
  float eps, K;
};

template <int NS>
struct FusedShape {
  static constexpr int N = NS * (NS + 2);
  static constexpr int NCB = (2 * N + 15) / 16;   // 16-column blocks of [fn_hi | fn_lo]
  static constexpr int CW = NCB * 16 + 1;         // partial-row scratch: columns + sum of squares
  static constexpr int KSW = NS * kCPS;           // k-steps of a slice
  static constexpr int NFRAG = KSW * NCB * 64;    // B fragments (16 bytes each)
  static constexpr int kRed = 4 * 16 * CW;        // per-wave partial rows
  static constexpr int kStage = kDS * (N + 1);    // fn rows of one stream while packing
  static constexpr int kGs = 8 * 32;              // finalise group sums
  static constexpr int kScratch = kRed > kStage ? (kRed > kGs ? kRed : kGs) : (kStage > kGs ? kStage : kGs);
  static constexpr size_t lds_bytes = (size_t)NFRAG * 16 + (size_t)kScratch * 4;
};

// TB = tokens finalised per batch (2 when S <= 64, else 1): thread (c =
// tid % 32, group = tid / 32) sums column c of splits sub, sub + SUBS, ...
// for token mm of the batch, sub = group % SUBS, mm = group / SUBS.
template <int NS, int TB>
__global__ __launch_bounds__(kThreads, 2) void pre_fused_kernel(FusedArgs a) {
  typedef FusedShape<NS> F;
  constexpr int N = F::N, NCB = F::NCB, CW = F::CW, KSW = F::KSW;
  constexpr int SUBS = 8 / TB;
  extern __shared__ u32x4 lds[];      // F::NFRAG B fragments, then the scratch
  float* scratch = reinterpret_cast<float*>(lds + F::NFRAG);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int S = a.S, G = a.G;
  const int sg = (int)(blockIdx.x % S);
  const int64_t T = a.T, D = a.D;
  const int tiles = (int)((T + kTM - 1) / kTM);
  const int64_t d0 = (int64_t)sg * kDS;

  u64 epoch = ld_agent(a.status + kStEpoch) + 1;
  if ((unsigned)epoch == 0u) ++epoch;   // tag 0 never matches a zeroed word
  const unsigned tag = (unsigned)epoch;
  const bool fresh = ld_agent(a.status + kStMarker) != a.marker;

  // Residual slice of tile t for this wave's 16 tokens (rows past T read row 0
  // and are never published or stored).
  auto load_tile = [&](int t, u32x4 (&A)[KSW]) {
    const int64_t row = (int64_t)t * kTM + w * 16 + r16;
    const uint16_t* xr = a.x + (row < T ? row : 0) * NS * D + d0 + q * 8;
#pragma unroll
    for (int j = 0; j < KSW; ++j) A[j] = ld16(xr + (j / kCPS) * D + (j % kCPS) * 32);
  };

  int t = (int)(blockIdx.x / S);
  u32x4 Acur[KSW], Anext[KSW];
  if (t < tiles) load_tile(t, Acur);

  // ---- fn slice -> B fragments in LDS, one stream at a time: fn rows i*D + d0
  // .. + 127 are contiguous; they are staged in LDS (coalesced reads), then
  // every thread builds fragments (hi = bf16(f), lo = bf16(f - hi)).
  // Fragment (j * NCB + cb) * 64 + l holds B[k][col] for the slice's k-step j,
  // k = 32 j + 8 (l / 16) + e, col = 16 cb + l % 16; columns N .. 2N-1 hold
  // the lo parts, the rest are zero.
  for (int i = 0; i < NS; ++i) {
    const float* src = a.fn + ((int64_t)i * D + d0) * N;
    for (int v = tid; v < kDS * N; v += kThreads) {
      const int r = v / N, c = v - r * N;
      scratch[r * (N + 1) + c] = src[v];
    }
    __syncthreads();
    for (int f = tid; f < kCPS * NCB * 64; f += kThreads) {
      const int kk = f / (NCB * 64);
      const int cb = (f / 64) % NCB;
      const int l = f & 63;
      const int col = cb * 16 + (l & 15);
      const bool is_hi = col < N, is_lo = !is_hi && col < 2 * N;
      const int c = is_hi ? col : col - N;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (is_hi || is_lo) ? scratch[(kk * 32 + (l >> 4) * 8 + e) * (N + 1) + c] : 0.0f;
        const float hi = (float)(__bf16)x;
        v[e] = is_hi ? hi : x - hi;   // x - hi is exact in fp32
      }
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
      lds[((i * kCPS + kk) * NCB + cb) * 64 + l] = o;
    }
    __syncthreads();
  }

  // ---- first use of the workspace for this shape: zero the tag region, then
  // a grid barrier (every workgroup is resident)
  if (fresh) {
    const int64_t nthr = (int64_t)a.P * kThreads;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + tid; v < a.ntag; v += nthr) st_agent(a.part + v, 0ull);
    wait_vm();
    __syncthreads();
    if (tid == 0) {
      count_in(a.status + kStArrive);
      const long long t0 = wall_clock64();
      while (ld_agent(a.status + kStArrive) < (u64)a.P) {
        if (wall_clock64() - t0 > kPollTicks) {
          st_agent(a.status + kStTimeout, epoch);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
  }

  float* rw = scratch + w * (16 * CW);
  const int nmine = sg < kTM ? (kTM - 1 - sg) / S + 1 : 0;
  for (; t < tiles; t += G) {
    const int64_t row = (int64_t)t * kTM + w * 16 + r16;
    const bool rok = row < T;

    // ---- 1. split-K GEMM + sum of squares over the slice
    f32x4 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, Acur[j]);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, lds[(j * NCB + cb) * 64 + lane]),
                                                          acc[cb], 0, 0, 0);
      const u32x4 aw = Acur[j];
      ss = dot2_self(aw.x, ss);
      ss = dot2_self(aw.y, ss);
      ss = dot2_self(aw.z, ss);
      ss = dot2_self(aw.w, ss);
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);

    // ---- 2. publish the partial rows of this wave's 16 tokens (hi + lo
    // columns combined through LDS; the scratch is free: every reader of the
    // previous tile's group sums passed the barrier that ended its finalise)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) rw[(q * 4 + i) * CW + cb * 16 + r16] = acc[cb][i];
    if (q == 0) rw[r16 * CW + NCB * 16] = ss;
    __syncthreads();
    for (int idx = lane; idx < 16 * (N + 1); idx += 64) {
      const int r = idx / (N + 1);
      const int c = idx - r * (N + 1);
      const int64_t tok = (int64_t)t * kTM + w * 16 + r;
      if (tok < T) {
        const float* rr = rw + r * CW;
        put_tagged(a.part + ((int64_t)sg * T + tok) * (N + 1) + c, tag, c < N ? rr[c] + rr[c + N] : rr[NCB * 16]);
      }
    }
    __syncthreads();   // the scratch is reused below

    // ---- 3. prefetch the next tile's slice (lands while the exchange runs)
    const int tn = t + G;
    if (tn < tiles) load_tile(tn, Anext);

    // ---- 4. finalise tokens sg, sg + S, ... of the tile, TB at a time
    {
      const int c = tid & 31, grp = tid >> 5;
      const int sub = grp % SUBS, mm = grp / SUBS;
      const int64_t rstride = T * (N + 1);
      float* gs = scratch;   // [TB][SUBS][32] group sums
      const long long t0 = wall_clock64();
      for (int m0 = 0; m0 < nmine; m0 += TB) {
        const int m = m0 + mm;
        const int64_t tok = (int64_t)t * kTM + sg + (int64_t)S * m;
        const bool ok = m < nmine && tok < T && c <= N;
        const u64* pc = a.part + (ok ? tok * (N + 1) + c : 0);
        float accm = 0.0f;
        for (;;) {
          u64 vv[kLoads];
#pragma unroll
          for (int u = 0; u < kLoads; ++u) {
            const int sp = sub + SUBS * u;
            vv[u] = (ok && sp < S) ? ld_agent(pc + sp * rstride) : ((u64)tag << 32);
          }
          bool ready = true;
          accm = 0.0f;
#pragma unroll
          for (int u = 0; u < kLoads; ++u) {
            ready = ready && tag_is(vv[u], tag);
            accm += tag_val(vv[u]);
          }
          if (__syncthreads_and(ready)) break;
          if (wall_clock64() - t0 > kPollTicks) {
            if (tid == 0) st_agent(a.status + kStTimeout, epoch);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        gs[(mm * SUBS + sub) * 32 + c] = accm;
        __syncthreads();
        if (w < TB && m0 + w < nmine) {
          const int64_t tk = (int64_t)t * kTM + sg + (int64_t)S * (m0 + w);
          float tot = 0.0f;
          const int cc = lane & 31;
#pragma unroll
          for (int g = 0; g < SUBS; ++g) tot += gs[(w * SUBS + g) * 32 + cc];
          const float v0 = __shfl(tot, lane & 15);
          const float v1 = __shfl(tot, (lane & 15) + 16);
          float gate, combv;
          epilogue16<NS>(v0, v1, a.hc_scale, a.bias, a.K, a.eps, a.repeat, gate, combv);
          if (tk < T && lane < 16) {
            const int e = lane;
            if (e < NS) put_tagged(a.prebuf + tk * 4 + e, tag, gate);
            else if (e < 2 * NS) a.post[tk * NS + (e - NS)] = gate;
            if ((e >> 2) < NS && (e & 3) < NS) a.comb[tk * NS * NS + (e >> 2) * NS + (e & 3)] = combv;
          }
        }
        __syncthreads();
      }
    }

    // ---- 5. pre of this wave's 16 tokens (polled), then y for the slice
    float pre[NS];
    {
      const u64* pp = a.prebuf + (rok ? row : 0) * 4;
      const long long t0 = wall_clock64();
      for (;;) {
        bool ready = true;
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const u64 wv = rok ? ld_agent(pp + i) : ((u64)tag << 32);
          ready = ready && tag_is(wv, tag);
          pre[i] = tag_val(wv);
        }
        if (__all(ready)) break;
        if (wall_clock64() - t0 > kPollTicks) {
          if (lane == 0) st_agent(a.status + kStTimeout, epoch);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    if (rok) {
      uint16_t* yr = a.y + row * D + d0 + q * 8;
#pragma unroll
      for (int c = 0; c < kCPS; ++c) {
        float o[8], f[8];
        Vec<BF16>::unpack(Acur[c], f);
#pragma unroll
        for (int v = 0; v < 8; ++v) o[v] = pre[0] * f[v];
#pragma unroll
        for (int i = 1; i < NS; ++i) {
          Vec<BF16>::unpack(Acur[i * kCPS + c], f);
#pragma unroll
          for (int v = 0; v < 8; ++v) o[v] = fmaf(pre[i], f[v], o[v]);
        }
        st16(yr + c * 32, Vec<BF16>::pack(o));
      }
    }
#pragma unroll
    for (int j = 0; j < KSW; ++j) Acur[j] = Anext[j];
  }

  // ---- the last workgroup to finish records the shape marker and the epoch
  // and re-arms the counters for the next call
  __syncthreads();
  if (tid == 0 && count_in(a.status + kStDone) == (u64)a.P) {
    st_agent(a.status + kStDone, 0ull);
    st_agent(a.status + kStArrive, 0ull);
    st_agent(a.status + kStMarker, a.marker);
    st_agent(a.status + kStEpoch, epoch);
  }
}

bool fused_supported(int64_t T, int n, int64_t D, mhc_dtype dt) {
  return dt == MHC_BF16 && T > 0 && n >= 1 && n <= 4 && D % kDS == 0 && D / kDS <= kMaxSplits;
}

int fused_splits(int64_t D) { return (int)(D / kDS); }

int fused_tile_tokens() { return kTM; }

template <int NS, int TB>
static int fused_resident_per_cu() {
  const size_t lds = FusedShape<NS>::lds_bytes;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(pre_fused_kernel<NS, TB>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return 0;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, pre_fused_kernel<NS, TB>, kThreads, lds) != hipSuccess)
    return 0;
  return occ;
}

template <int NS>
static int fused_resident_per_cu_n() {
  const int a = fused_resident_per_cu<NS, 1>();
  const int b = fused_resident_per_cu<NS, 2>();
  return a < b ? a : b;
}

// Cached per device and n: the first query also raises the kernels' dynamic
// LDS limit, which must happen before their first launch on the device.
int fused_resident_capacity(int n) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev][5];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || n < 1 || n > 4) return 0;
  if (dev < kMaxDev) {
    const int c = cache[dev][n].load(std::memory_order_acquire);
    if (c > 0) return c - 1;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  int occ = 0;
  switch (n) {
    case 1: occ = fused_resident_per_cu_n<1>(); break;
    case 2: occ = fused_resident_per_cu_n<2>(); break;
    case 3: occ = fused_resident_per_cu_n<3>(); break;
    default: occ = fused_resident_per_cu_n<4>(); break;
  }
  const int cap = occ * cus;
  if (dev < kMaxDev) cache[dev][n].store(cap + 1, std::memory_order_release);
  return cap;
}

template <int NS>
static void launch_fused_n(const FusedArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.P), block(kThreads);
  if (a.S <= 64)
    hipLaunchKernelGGL((pre_fused_kernel<NS, 2>), grid, block, FusedShape<NS>::lds_bytes, s, a);
  else
    hipLaunchKernelGGL((pre_fused_kernel<NS, 1>), grid, block, FusedShape<NS>::lds_bytes, s, a);
}

hipError_t launch_pre_fused(const PrePlan& p, const void* residual, const float* fn, const float* hc_scale,
                            const float* bias, float* post, float* comb, void* y, void* workspace, int repeat,
                            float eps, int capacity, hipStream_t s) {
  char* ws = static_cast<char*>(workspace);
  FusedArgs a;
  a.x = static_cast<const uint16_t*>(residual);
  a.fn = fn;
  a.hc_scale = hc_scale;
  a.bias = bias;
  a.post = post;
  a.comb = comb;
  a.y = static_cast<uint16_t*>(y);
  a.part = reinterpret_cast<u64*>(ws + p.off_fpart);
  a.prebuf = reinterpret_cast<u64*>(ws + p.off_pre);
  a.status = reinterpret_cast<u64*>(ws);
  a.marker = 0x6d68632d70726532ull ^ ((u64)p.T * 0x9E3779B97F4A7C15ull) ^ ((u64)p.D << 20) ^ ((u64)p.n << 56) ^
             (u64)p.fS;
  a.ntag = (int64_t)((p.off_tags_end - p.off_fpart) / 8);
  a.T = p.T;
  a.D = p.D;
  a.S = p.fS;
  const int tiles = (int)((p.T + kTM - 1) / kTM);
  int G = capacity / p.fS;
  if (G > tiles) G = tiles;
  if (G < 1) G = 1;
  a.G = G;
  a.P = G * p.fS;
  a.repeat = repeat;
  a.eps = eps;
  a.K = (float)p.K;
  switch (p.n) {
    case 1: launch_fused_n<1>(a, s); break;
    case 2: launch_fused_n<2>(a, s); break;
    case 3: launch_fused_n<3>(a, s); break;
    default: launch_fused_n<4>(a, s); break;
  }
  return hipGetLastError();
}

}  // namespace mhc
