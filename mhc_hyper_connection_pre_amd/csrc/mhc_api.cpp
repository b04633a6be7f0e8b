// C ABI of the mHC library: argument validation, split-K planning, launches.
// Every check runs before the first HIP call, so a rejected call launches
// nothing and touches no output.

#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>
#include <cstdio>

#include "mhc_internal.h"
#include "mhc_pack.h"

namespace mhc {
namespace {

thread_local char g_last_error[256] = "";

}  // namespace

int hip_fail(hipError_t e) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return MHC_ERR_HIP;
}

int fail_with(int status, const char* text) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s", text);
  return status;
}

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int vec_elems(mhc_dtype dt) { return dt == MHC_BF16 ? 8 : 4; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Shape checks shared by every entry point.
int check_shape(int64_t T, int n, int64_t D, mhc_dtype dt) {
  if (dt != MHC_BF16 && dt != MHC_F32) return MHC_ERR_INVALID_ARG;
  if (T < 0 || n < 1 || D < 1) return MHC_ERR_INVALID_ARG;
  if (n > 4 && n != 8) return MHC_ERR_UNSUPPORTED;
  if (D % vec_elems(dt) != 0) return MHC_ERR_MISALIGNED;
  // grid.x is the token count; keep every byte offset far from int64 overflow
  if (T > 0x7fffffffLL || D > (1LL << 26)) return MHC_ERR_UNSUPPORTED;
  return MHC_OK;
}

}  // namespace

int make_pre_plan(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt, PrePlan* p, bool boundary) {
  int st = check_shape(T, n, D, dt);
  if (st != MHC_OK) return st;
  if (n_splits < -kMaxSlices || n_splits > 256) return MHC_ERR_INVALID_ARG;
  if (n_splits == 0 && T > 0) {
    int stag = -1;
    const int t = tuned_splits(T, n, D, dt, boundary, &stag);
    if (t != 0 && make_pre_plan(T, n, D, t, dt, p, boundary) == MHC_OK) {
      p->rstag = stag;
      return MHC_OK;
    }
  }
  PrePlan q{};
  q.T = T;
  q.D = D;
  q.n = n;
  q.K = (int64_t)n * D;
  q.N = n * (n + 2);
  q.NP = (q.N + 1 + 3) / 4 * 4;
  q.dt = dt;
  // One "k-step" is 32 hidden elements for the MFMA path, 64 for the VALU path.
  const int kstep = dt == MHC_BF16 ? 32 : 64;
  q.ksteps = (int)((q.K + kstep - 1) / kstep);
  if (dt == MHC_BF16) {
    q.NCB = pack_blocks(n);
    if (n == 8) {   // 11 column blocks, four waves. From 128 tokens on, two 16-token tiles per wave
                    // (each B fragment from L2 serves 32 tokens; one tile per wave measured 21 % slower
                    // at T = 2048, D = 7168; four tiles' LDS wave sums, 181 KB, would not fit); below
                    // that one tile per wave, which keeps more workgroups (2.3 us faster at T = 16)
      q.MT = T >= 128 ? 2 : 1;
      q.NW = 4;
    } else if (n_splits == 1) {  // one split: a tall workgroup of 16 waves per 16 tokens keeps the k-loop parallel
      q.MT = 1;
      q.NW = 16;
    } else {
      q.MT = 4;
      q.NW = 4;
    }
    q.tok_per_wg = 16 * q.MT;
  } else {
    q.NCB = 0;
    q.MT = 0;
    q.NW = 1;
    q.tok_per_wg = 4;
  }
  const int64_t groups = T > 0 ? (T + q.tok_per_wg - 1) / q.tok_per_wg : 1;
  int S = n_splits;
  if (S <= 0) {
    // Library choice: about 512 workgroups, each split at least one k-step per wave.
    int64_t want = (512 + groups - 1) / groups;
    int64_t cap = q.ksteps / q.NW;
    if (cap < 1) cap = 1;
    if (cap > 64) cap = 64;
    S = (int)(want < 1 ? 1 : (want > cap ? cap : want));
  }
  if (S > q.ksteps) S = q.ksteps;
  q.steps_per_split = (q.ksteps + S - 1) / S;
  q.S = (q.ksteps + q.steps_per_split - 1) / q.steps_per_split;  // no empty split
  q.off_fnp = kStatusBytes;
  q.fnp_bytes = dt == MHC_BF16 ? (size_t)q.ksteps * q.NCB * 64 * 16 : 0;
  q.off_part = align_up(q.off_fnp + q.fnp_bytes, 256);
  q.part_bytes = (size_t)q.S * (size_t)T * q.NP * sizeof(float);
  size_t total2 = align_up(q.off_part + q.part_bytes, 256);
  // Single-pass path: the library's choice when the shape allows it, or on
  // request (n_splits = -1, or -S for S slices). Layout: status, packed fn (as
  // above), then the tagged exchange words: partials [rS][T][N + 1] and pre
  // [T][4], 8 bytes each.
  ResidentChoice rc{};
  const int want_S = n_splits < kSplitsSinglePass ? -n_splits : 0;
  const bool res_ok = n_splits <= 0 && resident_choose(T, n, D, dt, &rc, boundary, want_S);
  if (n_splits < 0 && !res_ok) return MHC_ERR_UNSUPPORTED;
  q.res = res_ok;
  q.rstag = -1;
  q.total_bytes = total2;
  if (q.res) {
    q.rS = rc.S;
    q.rcps = rc.cps;
    q.rper = rc.per;
    q.rTB = rc.TB;
    q.off_fpart = align_up(q.off_fnp + q.fnp_bytes, 256);
    q.off_pre = align_up(q.off_fpart + (size_t)q.rS * (size_t)T * (q.N + 1) * 8, 256);
    q.off_tags_end = align_up(q.off_pre + (size_t)T * 4 * 8, 256);
    // also enough for the two-pass path, which a call with an fn that is not
    // 16-byte aligned takes instead
    q.total_bytes = q.off_tags_end > total2 ? q.off_tags_end : total2;
  }
  *p = q;
  return MHC_OK;
}

namespace {

// The pre step once the plan is made and the arguments are checked.
int run_pre(const PrePlan& p, float* post, float* comb, void* y, const void* residual, const float* fn,
            const float* hc_scale, const float* bias, int sinkhorn_repeat, float eps, void* workspace,
            hipStream_t s) {
  hipError_t e;
  if (p.res && aligned(fn, 16)) {
    e = launch_pre_resident(p, residual, fn, hc_scale, bias, post, comb, y, workspace, sinkhorn_repeat, eps, s);
    return e == hipSuccess ? MHC_OK : hip_fail(e);
  }
  // Two-pass path.
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + p.off_part);
  void* fnp = ws + p.off_fnp;
  if (p.dt == MHC_BF16) {
    e = launch_pack_fn(p, fn, fnp, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  e = launch_pre_gemm(p, residual, fnp, fn, part, s);
  if (e != hipSuccess) return hip_fail(e);
  e = launch_pre_epilogue(p, residual, part, hc_scale, bias, post, comb, y, sinkhorn_repeat, eps,
                          reinterpret_cast<unsigned long long*>(ws), s);
  if (e != hipSuccess) return hip_fail(e);
  return MHC_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// A buffer an entry point touches: its address and the bytes the call reads
// or writes there (null: an optional buffer that is absent).
struct Span {
  const void* p;
  size_t bytes;
};

// True when a written buffer overlaps another written buffer or a read one.
// The kernels read inputs and write outputs from many workgroups in no fixed
// order, so such an overlap would make the results depend on the schedule.
bool outputs_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    if (!o->p) continue;
    for (auto q = o + 1; q != outs.end(); ++q)
      if (q->p && overlaps(o->p, o->bytes, q->p, q->bytes)) return true;
    for (const Span& i : ins)
      if (i.p && overlaps(o->p, o->bytes, i.p, i.bytes)) return true;
  }
  return false;
}

size_t elem_bytes(mhc_dtype dt) { return dt == MHC_BF16 ? 2 : 4; }

}  // namespace

int pre_call(float* post, float* comb, void* y, const void* residual, mhc_dtype dt, const float* fn,
             const float* hc_scale, const float* bias, int64_t T, int n, int64_t D, int sinkhorn_repeat, float eps,
             int n_splits, void* workspace, size_t workspace_bytes, hipStream_t s, WorkspaceProvider provider) {
  PrePlan p;
  int st = make_pre_plan(T, n, D, n_splits, dt, &p);
  if (st != MHC_OK) return st;
  if (sinkhorn_repeat < 1 || !(eps > 0.0f) || !std::isfinite(eps)) return MHC_ERR_INVALID_ARG;
  if (T == 0) return MHC_OK;
  if (!post || !comb || !y || !residual || !fn || !hc_scale || !bias) return MHC_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(residual, 16)) return MHC_ERR_MISALIGNED;
  if (!aligned(post, 4) || !aligned(comb, 4) || !aligned(fn, 4) || !aligned(hc_scale, 4) || !aligned(bias, 4))
    return MHC_ERR_MISALIGNED;
  if (provider) {   // the workspace comes from the provider, after every other check
    if (workspace_bytes < p.total_bytes) return MHC_ERR_WORKSPACE;
  } else if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.total_bytes) {
    return MHC_ERR_WORKSPACE;
  }
  if (p.res && !aligned(fn, 16) && n_splits < 0) return MHC_ERR_MISALIGNED;
  {
    const size_t e = elem_bytes(dt), N = (size_t)n * (n + 2);
    if (outputs_overlap({{post, (size_t)T * n * 4}, {comb, (size_t)T * n * n * 4}, {y, (size_t)T * D * e},
                         {provider ? nullptr : workspace, p.total_bytes}},
                        {{residual, (size_t)T * n * D * e}, {fn, (size_t)n * D * N * 4}, {hc_scale, 3 * 4},
                         {bias, N * 4}}))
      return MHC_ERR_INVALID_ARG;
  }
  if (provider) {
    st = provider(s, &workspace);
    if (st != MHC_OK) return st;
  }
  return run_pre(p, post, comb, y, residual, fn, hc_scale, bias, sinkhorn_repeat, eps, workspace, s);
}

}  // namespace mhc

using namespace mhc;

extern "C" {

MHC_API const char* mhc_status_string(int status) {
  switch (status) {
    case MHC_OK: return "MHC_OK";
    case MHC_ERR_INVALID_ARG: return "MHC_ERR_INVALID_ARG: null pointer, negative size or invalid knob";
    case MHC_ERR_UNSUPPORTED: return "MHC_ERR_UNSUPPORTED: shape not supported by the GPU kernels";
    case MHC_ERR_MISALIGNED: return "MHC_ERR_MISALIGNED: D not a multiple of the vector width, or pointer misaligned";
    case MHC_ERR_WORKSPACE: return "MHC_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MHC_ERR_HIP: return "MHC_ERR_HIP: a HIP launch failed (see mhc_last_error)";
    default: return "unknown mhc status";
  }
}

MHC_API const char* mhc_last_error(void) { return g_last_error; }

MHC_API int mhc_pre_splits(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt) {
  PrePlan p;
  const int st = make_pre_plan(T, n, D, n_splits, dt, &p);
  return st != MHC_OK ? st : (p.res ? p.rS : p.S);
}

MHC_API size_t mhc_pre_workspace_bytes(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt) {
  PrePlan p, q;
  if (T == 0 || make_pre_plan(T, n, D, n_splits, dt, &p) != MHC_OK) return 0;
  // the same workspace serves mhc_post_pre, whose single-pass tiling may differ
  if (make_pre_plan(T, n, D, n_splits, dt, &q, true) == MHC_OK && q.total_bytes > p.total_bytes) return q.total_bytes;
  return p.total_bytes;
}

MHC_API int mhc_post_pre_fused(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt) {
  PrePlan p;
  const int st = make_pre_plan(T, n, D, n_splits, dt, &p, true);
  return st != MHC_OK ? st : (p.res ? 1 : 0);
}

MHC_API int mhc_pre_plan_info(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt, int boundary, int* info) {
  if (info == nullptr) return MHC_ERR_INVALID_ARG;
  PrePlan p;
  const int st = make_pre_plan(T, n, D, n_splits, dt, &p, boundary != 0);
  if (st != MHC_OK) return st;
  if (p.res) {
    const int64_t tiles = (T + kResidentTile - 1) / kResidentTile;
    info[0] = 1;
    info[1] = p.rS;
    info[2] = p.rcps;
    info[3] = (int)(p.rper > 0 ? (tiles + p.rper - 1) / p.rper : 0);
    info[4] = resident_stagger(p, boundary != 0);
  } else {
    info[0] = 0;
    info[1] = p.S;
    info[2] = 0;
    info[3] = 0;
    info[4] = -1;
  }
  return MHC_OK;
}

MHC_API int mhc_pre(float* post, float* comb, void* y, const void* residual, mhc_dtype dt, const float* fn,
                    const float* hc_scale, const float* bias, int64_t T, int n, int64_t D, int sinkhorn_repeat,
                    float eps, int n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return pre_call(post, comb, y, residual, dt, fn, hc_scale, bias, T, n, D, sinkhorn_repeat, eps, n_splits, workspace,
                  workspace_bytes, static_cast<hipStream_t>(stream), nullptr);
}

MHC_API int mhc_post_pre(void* out, float* post_next, float* comb_next, void* y_next, const void* h,
                         const void* residual, const float* post, const float* comb, mhc_dtype dt, const float* fn,
                         const float* hc_scale, const float* bias, int64_t T, int n, int64_t D, int sinkhorn_repeat,
                         float eps, int n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  PrePlan fp, pp;
  int st = make_pre_plan(T, n, D, n_splits, dt, &fp, true);
  if (st != MHC_OK) return st;
  st = make_pre_plan(T, n, D, n_splits, dt, &pp);
  if (st != MHC_OK) return st;
  if (sinkhorn_repeat < 1 || !(eps > 0.0f) || !std::isfinite(eps)) return MHC_ERR_INVALID_ARG;
  if (T == 0) return MHC_OK;
  if (!out || !post_next || !comb_next || !y_next || !h || !residual || !post || !comb || !fn || !hc_scale || !bias)
    return MHC_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(h, 16) || !aligned(residual, 16) || !aligned(y_next, 16))
    return MHC_ERR_MISALIGNED;
  if (!aligned(post_next, 4) || !aligned(comb_next, 4) || !aligned(post, 4) || !aligned(comb, 4) ||
      !aligned(fn, 4) || !aligned(hc_scale, 4) || !aligned(bias, 4))
    return MHC_ERR_MISALIGNED;
  const size_t need = fp.total_bytes > pp.total_bytes ? fp.total_bytes : pp.total_bytes;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return MHC_ERR_WORKSPACE;
  if (fp.res && !aligned(fn, 16) && n_splits < 0) return MHC_ERR_MISALIGNED;
  {
    const size_t e = elem_bytes(dt), N = (size_t)n * (n + 2);
    if (outputs_overlap({{out, (size_t)T * n * D * e}, {post_next, (size_t)T * n * 4},
                         {comb_next, (size_t)T * n * n * 4}, {y_next, (size_t)T * D * e}, {workspace, need}},
                        {{h, (size_t)T * D * e}, {residual, (size_t)T * n * D * e}, {post, (size_t)T * n * 4},
                         {comb, (size_t)T * n * n * 4}, {fn, (size_t)n * D * N * 4}, {hc_scale, 3 * 4},
                         {bias, N * 4}}))
      return MHC_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fp.res && aligned(fn, 16)) {
    const hipError_t er = launch_post_pre_resident(fp, h, residual, post, comb, out, fn, hc_scale, bias, post_next,
                                                   comb_next, y_next, workspace, sinkhorn_repeat, eps, s);
    return er == hipSuccess ? MHC_OK : hip_fail(er);
  }
  // the two calls in sequence
  const hipError_t er = launch_post(h, residual, post, comb, out, dt, T, n, D, s);
  if (er != hipSuccess) return hip_fail(er);
  return run_pre(pp, post_next, comb_next, y_next, out, fn, hc_scale, bias, sinkhorn_repeat, eps, workspace, s);
}

MHC_API int mhc_pre_sync_timeouts(const void* workspace, size_t workspace_bytes, int64_t T, int n, int64_t D,
                                  int n_splits, mhc_dtype dt, void* stream) {
  PrePlan p;
  const int st = make_pre_plan(T, n, D, n_splits, dt, &p);
  if (st != MHC_OK) return st;
  if (!p.res || T == 0) return 0;
  if (!workspace || workspace_bytes < p.total_bytes) return MHC_ERR_WORKSPACE;
  unsigned long long v[2] = {0, 0};   // kStEpoch, kStTimeout
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipMemcpy(v, workspace, sizeof v, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  return v[0] != 0 && v[1] == v[0] ? 1 : 0;
}

MHC_API int mhc_post(void* out, const void* h, const void* residual, const float* post, const float* comb,
                     mhc_dtype dt, int64_t T, int n, int64_t D, void* stream) {
  int st = check_shape(T, n, D, dt);
  if (st != MHC_OK) return st;
  if (T == 0) return MHC_OK;
  if (!out || !h || !residual || !post || !comb) return MHC_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(h, 16) || !aligned(residual, 16)) return MHC_ERR_MISALIGNED;
  if (!aligned(post, 4) || !aligned(comb, 4)) return MHC_ERR_MISALIGNED;
  {
    const size_t e = elem_bytes(dt);
    if (outputs_overlap({{out, (size_t)T * n * D * e}},
                        {{h, (size_t)T * D * e}, {residual, (size_t)T * n * D * e}, {post, (size_t)T * n * 4},
                         {comb, (size_t)T * n * n * 4}}))
      return MHC_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_post(h, residual, post, comb, out, dt, T, n, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHC_OK : hip_fail(e);
}

MHC_API int mhc_post_combine_norm(void* normalized, void* out_residual, const void* h, const void* residual,
                                  const float* post, const float* comb, const float* combine_w,
                                  const float* norm_weight, float norm_eps, mhc_dtype dt, int64_t T, int n,
                                  int64_t D, void* stream) {
  int st = check_shape(T, n, D, dt);
  if (st != MHC_OK) return st;
  if (!(norm_eps > 0.0f) || !std::isfinite(norm_eps)) return MHC_ERR_INVALID_ARG;
  if (D / vec_elems(dt) > pcn_max_vectors(n)) return MHC_ERR_UNSUPPORTED;
  if (T == 0) return MHC_OK;
  if (!normalized || !h || !residual || !post || !comb || !combine_w || !norm_weight) return MHC_ERR_INVALID_ARG;
  if (!aligned(normalized, 16) || !aligned(h, 16) || !aligned(residual, 16) ||
      (out_residual && !aligned(out_residual, 16)))
    return MHC_ERR_MISALIGNED;
  if (!aligned(post, 4) || !aligned(comb, 4) || !aligned(combine_w, 4) || !aligned(norm_weight, 4))
    return MHC_ERR_MISALIGNED;
  {
    const size_t e = elem_bytes(dt);
    if (outputs_overlap({{normalized, (size_t)T * D * e}, {out_residual, (size_t)T * n * D * e}},
                        {{h, (size_t)T * D * e}, {residual, (size_t)T * n * D * e}, {post, (size_t)T * n * 4},
                         {comb, (size_t)T * n * n * 4}, {combine_w, (size_t)T * n * 4}, {norm_weight, (size_t)D * 4}}))
      return MHC_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_post_combine_norm(normalized, out_residual, h, residual, post, comb, combine_w,
                                                norm_weight, norm_eps, dt, T, n, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MHC_OK : hip_fail(e);
}

}  // extern "C"
