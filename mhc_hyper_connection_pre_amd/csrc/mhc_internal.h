// Host-side plan and launcher declarations shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mhc.h"

namespace mhc {

// Tiling of the pre GEMM (residual [T, K] x fn [K, N], K = n*D, N = n(n+2)).
// bf16: MFMA 16x16x32 tiles; B = [fn_hi | fn_lo | fn_lo2 of the pre columns]
// packed into fragment order, NCB column blocks of 16. f32: a VALU dot-product kernel, no packing.
struct PrePlan {
  int64_t T, D, K;
  int n, N, NP;          // NP = per-token partial stride of the two-pass path (N sums + 1, padded)
  mhc_dtype dt;
  int ksteps;            // bf16: K / 32 rounded up; f32: K / 64 rounded up
  // two-pass path
  int S;                 // split-K partials written
  int steps_per_split;
  int MT, NW;            // bf16: 16-row token tiles per wave, waves per workgroup
  int NCB;               // bf16: 16-column blocks of [fn_hi | fn_lo | fn_lo2]
  int tok_per_wg;
  size_t off_fnp, fnp_bytes, off_part, part_bytes;
  // single-pass ("resident") path, bf16: 128-token tiles x S slices of the
  // hidden axis, 32 * cps positions per stream each; `rper` tiles resident at
  // once (one generation)
  bool res;
  int rS, rcps, rper, rTB;
  int rstag;             // single-pass instance from the tile table: 0 in step, 1 per wave, -1 the library's rule
  size_t off_fpart, off_pre, off_tags_end;  // tagged exchange words [off_fpart, off_tags_end)
  size_t total_bytes;    // enough for whichever path runs
};

// Status words at offset 0 of every workspace (kStatusBytes), as uint64. The
// single-pass path keeps its exchange state here between calls; the two-pass
// path clears kStMarker and kStTimeout.
constexpr size_t kStatusBytes = 256;
constexpr int kStEpoch = 0;     // epoch of the last finished single-pass call (0: none)
constexpr int kStTimeout = 1;   // epoch of the last single-pass call whose polls timed out
constexpr int kStMarker = 2;    // shape marker: the tag region was zeroed for this shape
constexpr int kStDone = 16;     // finished workgroups of the running call (own 128-byte line)
constexpr int kStArrive = 24;   // first-use barrier arrivals of the running call (own 128-byte line)

// n_splits value that asks for the single-pass path with the library's tiling;
// n_splits = -S (2 <= S <= kMaxSlices) asks for it with S slices of the hidden
// axis (a tile table or tuner picks among them).
constexpr int kSplitsSinglePass = -1;
constexpr int kMaxSlices = 256;

// The tile table's n_splits for the shape (0 when no entry covers it); with
// `stagger`, also the entry's single-pass kernel instance (0: workgroup in
// step, 1: one pipeline per wave, -1: the library's rule; -1 when no entry).
int tuned_splits(int64_t T, int n, int64_t D, mhc_dtype dt, bool boundary, int* stagger = nullptr);

// Fills `p`; returns MHC_OK or the status mhc_pre would return for the sizes.
// n_splits = 0 takes the tile table's entry when one covers the shape and is
// valid for it, and the heuristic below otherwise.
// boundary: plan the layer-boundary call (mhc_post_pre), whose single-pass
// kernel also keeps the block output in registers.
int make_pre_plan(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt, PrePlan* p, bool boundary = false);

// Launchers (stream-ordered, no synchronisation). Return the launch error.
hipError_t launch_pack_fn(const PrePlan& p, const float* fn, void* fnp, hipStream_t s);
hipError_t launch_pre_gemm(const PrePlan& p, const void* residual, const void* fnp, const float* fn,
                           float* part, hipStream_t s);
hipError_t launch_pre_epilogue(const PrePlan& p, const void* residual, const float* part,
                               const float* hc_scale, const float* bias, float* post, float* comb,
                               void* y, int repeat, float eps, unsigned long long* status, hipStream_t s);
hipError_t launch_pre_resident(const PrePlan& p, const void* residual, const float* fn, const float* hc_scale,
                               const float* bias, float* post, float* comb, void* y, void* workspace, int repeat,
                               float eps, hipStream_t s);
// The same kernel at the layer boundary: out = mhc_post(h, residual, post_in,
// comb_in) is formed in registers, stored, and is the residual of the pre step.
hipError_t launch_post_pre_resident(const PrePlan& p, const void* h, const void* residual, const float* post_in,
                                    const float* comb_in, void* out, const float* fn, const float* hc_scale,
                                    const float* bias, float* post, float* comb, void* y, void* workspace,
                                    int repeat, float eps, hipStream_t s);
// The single-pass kernel instance a call with plan `p` runs: 1 one pipeline
// per wave, 0 the workgroup's waves in step (the tile table's choice, else
// a rule on the number of generations; MHC_STAGGER = 0 / 1 overrides).
int resident_stagger(const PrePlan& p, bool boundary);
// Single-pass tiling for the shape on the current device (or a 256-CU MI355X
// when no device is visible): false if the shape is not supported. want_S > 0
// restricts the choice to that many slices of the hidden axis.
struct ResidentChoice {
  int cps, S, per, TB;
};
bool resident_choose(int64_t T, int n, int64_t D, mhc_dtype dt, ResidentChoice* c, bool boundary = false,
                     int want_S = 0);
constexpr int kResidentTile = 128;

hipError_t launch_post(const void* h, const void* residual, const float* post, const float* comb,
                       void* out, mhc_dtype dt, int64_t T, int n, int64_t D, hipStream_t s);
hipError_t launch_post_combine_norm(void* normalized, void* out, const void* h, const void* residual,
                                    const float* post, const float* comb, const float* combine_w,
                                    const float* norm_weight, float eps, mhc_dtype dt, int64_t T, int n,
                                    int64_t D, hipStream_t s);

// Records a HIP error as this thread's last error text and returns MHC_ERR_HIP.
int hip_fail(hipError_t e);
// Records `text` as this thread's last error text and returns `status`.
int fail_with(int status, const char* text);

// Supplies a workspace address for a pre call once its arguments have passed
// every check (the static-scratch entry point).
typedef int (*WorkspaceProvider)(hipStream_t s, void** workspace);

// mhc_pre's checks and launches. With a provider, `workspace` is ignored and
// `workspace_bytes` is the provider's capacity: the provider is called only
// after every argument check has passed, right before the launches.
int pre_call(float* post, float* comb, void* y, const void* residual, mhc_dtype dt, const float* fn,
             const float* hc_scale, const float* bias, int64_t T, int n, int64_t D, int sinkhorn_repeat, float eps,
             int n_splits, void* workspace, size_t workspace_bytes, hipStream_t s, WorkspaceProvider provider);

// Threads per workgroup of the fused combine+norm kernel, and the longest row
// (in 16-byte vectors) it keeps in registers: threads x 4 vectors.
template <int NS>
constexpr int kPcnThreads = NS > 4 ? 512 : 1024;
constexpr int64_t pcn_max_vectors(int n) { return n > 4 ? 512 * 4 : 1024 * 4; }

}  // namespace mhc
