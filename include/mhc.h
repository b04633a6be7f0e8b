/*
 * mhc.h - C ABI of the MI355X (gfx950) library for multi-stream
 * hyper-connection (mHC) pre/post mixing.
 *
 * Sources, cited by page title and section:
 *  [P1] "[sglang] AMD ROCm DeepSeek-V4 performance optimisation: Aiter MHC
 *       kernel integration analysis" (sglang PR #24355), section 2
 *       "DeepSeek-V4 model-layer kernel swap" (the pre call returning post,
 *       comb and y; the post call writing into a tensor allocated like the
 *       residual) and section 3 "TileLang kernel tuning" (the pre GEMM is a
 *       split-K GEMM fused with a sum of squares, tiled over the hidden axis).
 *  [P2] "[sglang] DeepSeek-V4.1 performance optimisation: mHC and metadata
 *       overhead analysis" (sglang PR #39704), section 1 "mHC
 *       Post/Combine/RMSNorm fusion (prefill)" and section 2 "All-reduce
 *       kernel extension and fusion" (post mix, next-layer combine and
 *       RMSNorm in one pass, result stored as `normalized`).
 *
 * Conventions shared by every entry point
 *  - All tensors are dense, row-major (last index fastest), caller-owned
 *    device memory. The library never allocates, frees or synchronises, and
 *    keeps no pointer after a call returns. Calls are asynchronous on
 *    `stream` (a hipStream_t; NULL = the default stream).
 *  - `dt` is the storage type of the residual-shaped tensors (residual, h,
 *    y, out, normalized). post, comb, fn, hc_scale, bias, combine_w and
 *    norm_weight are always float32.
 *  - Supported on the GPU: 1 <= n <= 4 and n = 8; D a multiple of 8 (bf16)
 *    or 4 (f32); residual-shaped pointers 16-byte aligned; float32 pointers
 *    4-byte aligned. T = 0 is a successful no-op.
 *  - Errors: argument problems return a negative status before anything is
 *    launched, and no output is touched. A failed launch returns
 *    MHC_ERR_HIP; mhc_last_error() then describes it. Nothing is printed and
 *    no C++ exception crosses the boundary.
 *  - Arithmetic: fp32 accumulation; every stored bf16 value is rounded once,
 *    to nearest even. Results are deterministic: the same inputs and knobs
 *    give the same bits (no floating-point atomics).
 */
#ifndef MHC_H_
#define MHC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_API __attribute__((visibility("default")))

typedef enum {
  MHC_OK = 0,
  MHC_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad eps/repeat/dtype */
  MHC_ERR_UNSUPPORTED = -2,  /* valid mathematically but not built (n = 5..7 or > 8, D too large) */
  MHC_ERR_MISALIGNED = -3,   /* D not a multiple of the vector width, or a pointer misaligned */
  MHC_ERR_WORKSPACE = -4,    /* workspace missing, misaligned or smaller than required */
  MHC_ERR_HIP = -5           /* a HIP launch failed */
} mhc_status;

/* Element type of residual, h, y and out. The two range markers make the
 * type span every int (C++ gives an enum only the values its enumerators'
 * bits cover), so a caller's out-of-range value is well defined and is
 * rejected with MHC_ERR_INVALID_ARG; they are not element types. */
typedef enum {
  MHC_BF16 = 0,
  MHC_F32 = 1,
  MHC_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  MHC_DTYPE_RANGE_MAX_ = 2147483647
} mhc_dtype;

/* Human-readable name of a status code (static string, never NULL). */
MHC_API const char* mhc_status_string(int status);

/* Text of the last HIP error seen by this thread (static storage, "" if none). */
MHC_API const char* mhc_last_error(void);

/* Number of split-K partials (slices of the hidden axis) mhc_pre uses for
 * these sizes: `n_splits` itself when positive (capped at K / 32), S for
 * n_splits = -S, otherwise the library's choice for the shape. Returns a
 * negative status for arguments mhc_pre would reject. */
MHC_API int mhc_pre_splits(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt);

/* Bytes of device workspace mhc_pre and mhc_post_pre need for these sizes and
 * knobs (0 when T = 0, and 0 for arguments mhc_pre would reject: the call
 * itself then reports the error). One workspace of this size serves both. */
MHC_API size_t mhc_pre_workspace_bytes(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt);

/*
 * mhc_pre - [P1] section 2 (the pre call), section 3 (split-K GEMM with sum of
 * squares), and the closing list of [P1] (fused Sinkhorn and normalisation).
 *
 * For every token t, with x = residual[t] flattened stream-major
 * (x[k] = residual[t][k / D][k % D], K = n*D) and N = n*(n+2):
 *   r      = 1 / sqrt(sum_k x[k]^2 / K + eps)
 *   m[c]   = sum_k x[k] * fn[k][c]                              c < N
 *   z[c]   = hc_scale[g(c)] * (r * m[c]) + bias[c]   g = 0 (c < n), 1 (c < 2n), 2
 *   pre[i] = sigmoid(z[i]);  post[t][i] = sigmoid(z[n + i])
 *   comb[t] = Sinkhorn(exp(Z)), Z[i][j] = z[2n + i*n + j], `sinkhorn_repeat`
 *            repeats of (normalise every row to sum 1, then every column)
 *   y[t][d] = sum_i pre[i] * residual[t][i][d]
 *
 * Outputs (first, in the order the page's call returns them):
 *   post  float32 [T, n]        comb float32 [T, n, n] (comb[t][i][j]: stream i -> j)
 *   y     dt      [T, D]
 *   They must not overlap one another, an input or the workspace bytes the
 *   call uses (MHC_ERR_INVALID_ARG).
 * Inputs:
 *   residual dt [T, n, D]; fn float32 [n*D, N]; hc_scale float32 [3]
 *   (pre, post, comb); bias float32 [N].
 * Knobs: sinkhorn_repeat >= 1; eps > 0; n_splits = split-K partials over the
 *   hidden axis: 0 = library choice; 1..256 = that many partials on the
 *   two-pass path; -1 = the single-pass path with the library's tiling, -S
 *   (2 <= S <= 256) = the single-pass path with S slices of the hidden axis
 *   (D = 32 * cps * S with cps one of 1 to 8 or 14), or an error for
 *   either (MHC_ERR_UNSUPPORTED for a shape or slice count it does not cover,
 *   MHC_ERR_MISALIGNED for an fn that is not 16-byte aligned); tile tables
 *   and tuners choose among these values. Any value gives the same result
 *   up to fp32 reassociation, and a fixed value is bitwise repeatable.
 * Paths: the single-pass kernel (one launch; the residual is read once and
 *   stays in registers; the workgroups of a token tile exchange partial sums
 *   through the workspace) covers bf16, n <= 4, D a multiple of 32 for which a
 *   slice tiling fits (mhc_pre_splits(..., -1, ...) > 0) and a 16-byte
 *   aligned fn; n_splits = 0 takes it when it can. Otherwise the two-pass
 *   path runs (pack fn, split-K GEMM, then an epilogue that reads the
 *   residual again for y). The single-pass kernel either keeps each
 *   workgroup's waves in step or runs one pipeline per wave; the tile table
 *   picks per shape (measured), else a rule on the number of generations of
 *   resident tiles; the environment variable MHC_STAGGER (0 or 1, read at
 *   each launch) forces either, as a test hook.
 * Co-residency: the single-pass kernel's workgroups wait for one another, so
 *   the launch is sized to what the device holds at once (workgroups per CU
 *   from the occupancy query times the CUs). Work that holds CUs while it
 *   runs (kernels on other streams or in other processes, CU masking) can
 *   keep some workgroups from starting; the waiting ones then give up after
 *   100 ms (see mhc_pre_sync_timeouts). Every output that depends on an
 *   exchange that did not complete is written as NaN (post, comb and y of
 *   that token; at the layer boundary post_next, comb_next and y_next, while
 *   out, which does not depend on the exchange, is still right), so a
 *   timed-out call cannot pass for a good one.
 * Workspace: device memory of at least mhc_pre_workspace_bytes(...) bytes,
 *   256-byte aligned, owned by the caller, not shared by concurrent calls.
 *   Its first 256 bytes are status words that the single-pass path keeps
 *   between calls: they must be zero before the first call on a workspace
 *   (and again if anything other than mhc_pre wrote the workspace since);
 *   the rest may hold anything.
 */
MHC_API int mhc_pre(float* post, float* comb, void* y,
                    const void* residual, mhc_dtype dt,
                    const float* fn, const float* hc_scale, const float* bias,
                    int64_t T, int n, int64_t D,
                    int sinkhorn_repeat, float eps, int n_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * 1 if the last mhc_pre call on `workspace` hit an exchange time-out, else 0
 * (synchronises `stream`, then copies 16 bytes to the host). The single-pass
 * path exchanges partial sums between the workgroups of a token tile through
 * the workspace; a workgroup that waits longer than 100 ms gives up (so the
 * call always finishes), marks the call and writes NaN into the outputs that
 * depend on the missing values.
 * Always 0 after a two-pass call. The sizes and knobs must be those of that
 * call. For tests and health checks: it blocks the host. The environment
 * variable MHC_POLL_TICKS (read at each launch) replaces the 100 ms limit by
 * that many ticks of the 100 MHz wall clock; 0 makes every wait that its first
 * read does not satisfy give up, and -1 makes the call publish every
 * exchanged value with a stale tag, so that every wait gives up (test hooks
 * for this path; the outputs of the tokens concerned are then NaN, and the
 * next call on the workspace is unaffected).
 */
MHC_API int mhc_pre_sync_timeouts(const void* workspace, size_t workspace_bytes, int64_t T, int n, int64_t D,
                                  int n_splits, mhc_dtype dt, void* stream);

/*
 * mhc_pre_static - mhc_pre for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results as mhc_pre with the
 * same n_splits (the same bits), but the workspace is a device array inside
 * the library, MHC_PRE_STATIC_SCRATCH_BYTES (32 MiB) per GPU, held from the
 * library's load until the process ends. The call allocates nothing.
 *   Limit: sizes whose mhc_pre_workspace_bytes(T, n, D, n_splits, dt) exceeds
 *   the array return MHC_ERR_WORKSPACE (mhc_last_error() says so) before any
 *   launch; at n = 4, D = 7168 that covers T up to 2048 (the single-pass
 *   exchange takes 200 bytes per token per slice), and T = 0 is a no-op.
 *   Sharing: every call on a GPU uses that GPU's one array, which keeps the
 *   last call's contents (the exchange state in its status words carries
 *   over by design). Calls that overlap on one GPU (other streams, other host
 *   threads) race on it and must not be made. Arguments are checked as
 *   mhc_pre checks them, before anything is launched; the first accepted call
 *   on a device also launches a one-block kernel on `stream`, ahead of its
 *   own, that clears the array's status words.
 */
#define MHC_PRE_STATIC_SCRATCH_BYTES (32u << 20)
MHC_API int mhc_pre_static(float* post, float* comb, void* y,
                           const void* residual, mhc_dtype dt,
                           const float* fn, const float* hc_scale, const float* bias,
                           int64_t T, int n, int64_t D,
                           int sinkhorn_repeat, float eps, int n_splits, void* stream);

/*
 * mhc_post - [P1] section 2 (the post call, into a tensor shaped like the
 * residual):
 *   out[t][j][d] = post[t][j] * h[t][d] + sum_i comb[t][i][j] * residual[t][i][d]
 * Output: out dt [T, n, D] (must not overlap an input: MHC_ERR_INVALID_ARG).
 * Inputs: h dt [T, D] (the block output); residual dt [T, n, D];
 *   post float32 [T, n]; comb float32 [T, n, n] as mhc_pre writes them.
 */
MHC_API int mhc_post(void* out, const void* h, const void* residual,
                     const float* post, const float* comb, mhc_dtype dt,
                     int64_t T, int n, int64_t D, void* stream);

/*
 * mhc_post_pre - the layer boundary: mhc_post of the finished layer, then
 * mhc_pre of the next layer on its result. [P1] section 2: a layer ends with
 * the post call, whose result (shaped like the residual) is the next
 * layer's residual, and the next layer begins with the pre call on it; [P2]
 * section 1 fuses the post mix with the next layer's input processing to
 * save memory traffic, and the closing paragraph of [P2] names that saving.
 *   out                       = mhc_post(h, residual, post, comb), rounded to dt
 *   post_next, comb_next, y_next = mhc_pre(out, fn, hc_scale, bias, ...)
 * exactly as the two calls in sequence (the same bits as mhc_post followed by
 * mhc_pre with the same knobs, when both run the same pre path).
 * Outputs: out dt [T, n, D]; post_next float32 [T, n]; comb_next float32
 *   [T, n, n]; y_next dt [T, D]. They must not overlap one another, an
 *   input or the workspace bytes the call uses (MHC_ERR_INVALID_ARG).
 * Inputs: h, residual, post, comb as mhc_post (post and comb of the finished
 *   layer); fn, hc_scale, bias of the next layer as mhc_pre.
 * Knobs, workspace and errors: as mhc_pre (same workspace size and status
 *   words). When the single-pass kernel covers the shape (see
 *   mhc_post_pre_fused) the call is one launch that reads h and the residual
 *   once, forms out in registers, writes out and y_next, and never reads out
 *   back; otherwise it launches mhc_post's kernel and then mhc_pre's path on
 *   out.
 */
MHC_API int mhc_post_pre(void* out, float* post_next, float* comb_next, void* y_next,
                         const void* h, const void* residual, const float* post, const float* comb,
                         mhc_dtype dt, const float* fn, const float* hc_scale, const float* bias,
                         int64_t T, int n, int64_t D, int sinkhorn_repeat, float eps, int n_splits,
                         void* workspace, size_t workspace_bytes, void* stream);

/* 1 if mhc_post_pre runs as one launch for these sizes and knobs (given a
 * 16-byte aligned fn), 0 if it runs mhc_post and mhc_pre's kernels in
 * sequence, or a negative status for arguments it would reject. */
MHC_API int mhc_post_pre_fused(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt);

/*
 * The plan of an mhc_pre (boundary = 0) or mhc_post_pre (boundary = 1) call
 * with these sizes on the current device (given a 16-byte aligned fn), for
 * tests and tuning ([P1] section 3: the hidden-axis tiling is chosen per
 * shape). info must hold 5 ints: info[0] = 1 for the single-pass kernel, 0 for
 * the two-pass path; info[1] = its slices of the hidden axis, or the two-pass
 * split count; info[2] = 32-wide columns per slice (single-pass, else 0);
 * info[3] = generations of resident token tiles (single-pass, else 0);
 * info[4] = the single-pass kernel's instance, 1 for one pipeline per wave,
 * 0 for the workgroup's waves in step (-1 for the two-pass path). Returns
 * MHC_OK, MHC_ERR_INVALID_ARG for a NULL info, or the status the call would
 * return for the sizes; info is written only on MHC_OK.
 */
MHC_API int mhc_pre_plan_info(int64_t T, int n, int64_t D, int n_splits, mhc_dtype dt, int boundary, int* info);

/*
 * mhc_post_combine_norm - [P2] section 1 (post mix, combine into one bf16
 * row, RMSNorm, one row per workgroup) and section 2 (the row is stored as
 * `normalized`):
 *   o_j[d]        = mhc_post result, rounded to dt
 *   c[d]          = sum_j combine_w[t][j] * o_j[d], rounded to dt
 *   normalized[d] = (c[d] / sqrt(sum_d c[d]^2 / D + norm_eps)) * norm_weight[d], rounded to dt
 * Outputs: normalized dt [T, D]; out_residual dt [T, n, D] receives o (pass
 *   NULL to skip writing it). They must not overlap each other or an input
 *   (MHC_ERR_INVALID_ARG).
 * Inputs: as mhc_post, plus combine_w float32 [T, n] and norm_weight float32
 *   [D]; norm_eps > 0. D <= 32768 (bf16) or 16384 (f32); at n = 8,
 *   D <= 16384 (bf16) or 8192 (f32).
 */
MHC_API int mhc_post_combine_norm(void* normalized, void* out_residual,
                                  const void* h, const void* residual,
                                  const float* post, const float* comb,
                                  const float* combine_w, const float* norm_weight,
                                  float norm_eps, mhc_dtype dt,
                                  int64_t T, int n, int64_t D, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H_ */
