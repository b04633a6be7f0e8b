// Host-side plan and launcher declarations shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mhc.h"

namespace mhc {

// Tiling of the pre GEMM (residual [T, K] x fn [K, N], K = n*D, N = n(n+2)).
// bf16: MFMA 16x16x32 tiles; B = [fn_hi | fn_lo] packed into fragment order,
// NCB column blocks of 16. f32: a VALU dot-product kernel, no packing.
struct PrePlan {
  int64_t T, D, K;
  int n, N, NP;          // NP = per-token partial stride (N sums + 1 sum of squares, padded)
  mhc_dtype dt;
  int ksteps;            // bf16: K / 32 rounded up; f32: K / 256 rounded up
  int S;                 // split-K partials actually written
  int steps_per_split;
  int MT, NW;            // bf16: 16-row token tiles per wave, waves per workgroup
  int NCB;               // bf16: 16-column blocks of [fn_hi | fn_lo]
  int tok_per_wg;
  size_t off_fnp, fnp_bytes, off_part, part_bytes, total_bytes;
};

// Fills `p`; returns MHC_OK or the status mhc_pre would return for the sizes.
int make_pre_plan(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt, PrePlan* p);

// Launchers (stream-ordered, no synchronisation). Return the launch error.
hipError_t launch_pack_fn(const PrePlan& p, const float* fn, void* fnp, hipStream_t s);
hipError_t launch_pre_gemm(const PrePlan& p, const void* residual, const void* fnp, const float* fn,
                           float* part, hipStream_t s);
hipError_t launch_pre_epilogue(const PrePlan& p, const void* residual, const float* part,
                               const float* hc_scale, const float* bias, float* post, float* comb,
                               void* y, int repeat, float eps, hipStream_t s);
hipError_t launch_post(const void* h, const void* residual, const float* post, const float* comb,
                       void* out, mhc_dtype dt, int64_t T, int n, int64_t D, hipStream_t s);
hipError_t launch_post_combine_norm(void* normalized, void* out, const void* h, const void* residual,
                                    const float* post, const float* comb, const float* combine_w,
                                    const float* norm_weight, float eps, mhc_dtype dt, int64_t T, int n,
                                    int64_t D, hipStream_t s);

// Largest D the fused combine+norm kernel keeps in registers: 1024 threads x 4 vectors.
constexpr int64_t kPcnMaxVectors = 1024 * 4;

}  // namespace mhc
