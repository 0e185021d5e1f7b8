/*
 * fused_boundary.h -- C ABI of the fused post-experts boundary for MI355X (gfx950).
 *
 * One kernel launch performs, per token row t (rows are independent):
 *
 *   x_t      = sum_{r<R} P_r[t]                         partial sums
 *            + sum_{k<K, idx valid} w[t,k] * E[idx[t,k]]  MoE finalize
 *            + s_t * S[t]                               shared expert, added once
 *            + X[t]                                     residual
 *   residual_out[t] = bf16(x_t)
 *   normed_out[t]   = bf16( x_t * rsqrt(mean_h(x_t^2) + eps) * (gamma + weight_bias) )
 *
 * Sources (sglang pull-request pages):
 *  - "Share the CuTe DSL AR fusion core and wire it for DeepSeek-V3 / GLM-5.x"
 *    (PR #37196), Motivation: the MoE finalize, the shared-expert add and the
 *    post-experts reduction are folded into the next layer's input RMSNorm.
 *    Modifications part 1: the kernel scales by (gamma + weight_bias); the
 *    handoff record and a workspace handle shared by every MoE layer.
 *    Modifications part 2: the finalize replaces a separate deferred-finalize
 *    call; the DeepSeek/GLM shared expert carries no gate while Qwen3.5's is
 *    sigmoid-gated; the shared expert must be counted exactly once.
 *  - "fuse trailing TP all-reduce with final RMSNorm" (PR #37104), Motivation:
 *    the residual RMSNorm boundary; Changes: fail loudly without a residual,
 *    and a runtime decline after which the caller performs the owed work itself.
 *  - ROCm fused all-reduce + mHC post (PR #42020), Summary: the fused kernel
 *    declines inputs it cannot take and the layer falls back to the split path.
 *
 * Numerics.  Sums are accumulated in fp32 registers in a fixed order: partials
 * 0..R-1, expert slots 0..K-1 (product w*E rounded to fp32, then added), the
 * shared term (s_t*S rounded to fp32, then added), the residual; no fused
 * multiply-add in that chain.  residual_out is exactly the bf16 rounding (to
 * nearest, ties to even) of that fp32 sum.  The norm reads the unrounded fp32
 * sum; its reduction order is unspecified, so normed_out may differ from an
 * exact evaluation by about one bf16 ulp.  s_t = fp32(1/(1+exp(-g_t))) evaluated
 * in fp64 when gate logits are given, else 1.  Inf and NaN inputs propagate as
 * IEEE fp32 arithmetic does (an Inf element zeroes the rest of its normed row
 * and a NaN makes it NaN); a skipped slot's row is never read into the sum.
 *
 * Layouts.  All activations are bf16, row-major, contiguous:
 *   P_r, X, S, normed_out, residual_out: [T, H];  E: [N, H];  gamma: [H].
 *   expanded_row_idx: int32 [T, K], token-major, value = row of E;
 *   topk_weights: fp32 [T, K];  shared_gate_logits: fp32 [T].
 * Every bf16 base pointer must be 16-byte aligned and H a multiple of 8
 * (128-bit loads of 8 elements); otherwise the call is declined.
 *
 * Ownership.  The caller owns all memory.  Device pointers stay owned by the
 * caller; the host array `partials` is read during the call only (its pointers
 * are copied into the launch) and may be freed on return.  The library
 * allocates nothing, does not synchronise, and launches exactly one kernel on
 * `stream` (a hipStream_t; NULL = the null stream), so calls may be captured
 * in a HIP graph.  The launch plan is chosen for the calling thread's current
 * HIP device (its CU count and LDS size), which must be the device that owns
 * `stream` and the buffers.
 *
 * Errors.  Argument checks run on the host before any HIP call; on any
 * non-OK return the outputs are untouched.
 *   FB_INVALID_ARGUMENT  a required pointer is NULL, a size is negative or out
 *                        of range, eps or weight_bias is not finite (or
 *                        eps < 0), an output overlaps an input (other than
 *                        residual_out == residual_in exactly, see
 *                        residual_out below) or the workspace.
 *   FB_DECLINED          a valid request this library does not take: H % 8 != 0,
 *                        H > FB_MAX_HIDDEN, or a bf16 pointer not 16-byte
 *                        aligned.  The caller falls back to an unfused path.
 *   FB_HIP_ERROR         the launch failed (see fused_boundary_last_hip_error).
 * num_tokens == 0 returns FB_OK without launching once the sizes and scalars
 * check out; the [T, ...] pointers may then be NULL.  Index values are not
 * checked on the host: a slot whose index is < 0 or >= num_expanded_rows is
 * skipped (it contributes nothing, whatever its weight), never read out of
 * bounds; every kernel applies exactly this rule (with num_expanded_rows of
 * 2^31 or more, every non-negative int32 index is valid).
 *
 * Workspace.  Optional.  Given (>= fused_boundary_workspace_bytes(T, H) bytes,
 * 16-byte aligned, zero-filled once before its first use), small-T calls split
 * each row over several workgroups that combine their sums of squares through
 * it (a 256-byte header plus 512 bytes per token row); without it every row
 * runs in one workgroup.  The library leaves the
 * workspace ready for the next call, so it is zeroed only once, and it may be
 * reused across calls with any T and H that fit.  Calls that may run
 * concurrently (different streams) need distinct workspaces.
 *
 * Bounded wait.  A split row's workgroups exchange their sums of squares and
 * wait for each other; if they cannot all run at once (another kernel holds the
 * GPU) the wait gives up after about a second.  The workgroup then takes the
 * sums its siblings have published by then and computes the others itself from
 * the inputs, in the same order, so the outputs are exactly what a normal call
 * gives, also with residual_out == residual_in (a split row's workgroup
 * overwrites an in-place residual only once its own sum is visible to its
 * siblings).  It sets bit 0 of the status word (the first uint32 of the
 * workspace, FB_WS_STATUS_WAIT_TIMEOUT), which stays set until the caller
 * zero-fills the workspace again; nothing else persists, and later calls on the
 * workspace exchange normally.  The status word is a diagnostic only: no output
 * is ever wrong or undefined because of a time-out.
 */
#ifndef FUSED_BOUNDARY_H_
#define FUSED_BOUNDARY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  FB_OK = 0,
  FB_INVALID_ARGUMENT = 1,
  FB_DECLINED = 2,
  FB_HIP_ERROR = 3,
  FB_TOO_MANY_ROWS = 4, /* allocation-free entry point only: T > FB_NOALLOC_MAX_ROWS */
};

#define FB_MAX_PARTIALS 16 /* R: up to a TP16 group (PR #37196, Known gaps: TP8/TP16 profiles) */
#define FB_MAX_TOP_K 16
#define FB_MAX_HIDDEN 16384

/* Workspace status word bits (first uint32 of the workspace). */
#define FB_WS_STATUS_WAIT_TIMEOUT 1u

/*
 * Partial sums + residual + RMSNorm, no MoE finalize (PR #37104: the trailing
 * reduction fused with the residual RMSNorm).
 *   partials      host array of num_partials device pointers, bf16 [T, H] each;
 *                 num_partials in [1, FB_MAX_PARTIALS].
 *   residual_in   bf16 [T, H], required.
 *   gamma         bf16 [H]; the norm scales by (gamma + weight_bias).
 *   weight_bias   finite; eps finite and >= 0 (added to the mean inside the root).
 *   num_tokens    T >= 0;  hidden  H, a multiple of 8, in [8, FB_MAX_HIDDEN].
 *   normed_out    bf16 [T, H].
 *   residual_out  bf16 [T, H]; may equal residual_in (in place; a partial or
 *                 shared_out that is that same buffer is then read in place
 *                 too), may not otherwise overlap any input (expert_out, whose
 *                 rows are gathered at any index, included).
 *   workspace     optional (NULL, 0): see above.
 *   stream        hipStream_t.
 */
int fused_reduce_rmsnorm(const void* const* partials, int32_t num_partials,
                         const void* residual_in, const void* gamma, float weight_bias,
                         float eps, int64_t num_tokens, int64_t hidden, void* normed_out,
                         void* residual_out, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Partial sums + MoE finalize (+ optional shared expert, optionally gated)
 * + residual + RMSNorm (PR #37196: the handoff's contents become these
 * arguments).
 *   partials            as above but num_partials in [0, FB_MAX_PARTIALS]
 *                       (partials may be NULL when num_partials == 0).
 *   expert_out          bf16 [num_expanded_rows, H]: unfinalized expert output
 *                       rows; may be NULL only if num_expanded_rows == 0.
 *   num_expanded_rows   N in [0, 2^40].
 *   expanded_row_idx    int32 [T, top_k], token-major; the row of expert_out
 *                       holding token t's slot k; outside [0, N) = skip the slot.
 *   topk_weights        fp32 [T, top_k], applied as given.
 *   top_k               K in [1, FB_MAX_TOP_K].
 *   shared_out          bf16 [T, H] or NULL (no shared expert).
 *   shared_gate_logits  fp32 [T] or NULL (ungated: scale 1); ignored when
 *                       shared_out is NULL.
 *   remaining arguments as in fused_reduce_rmsnorm.
 */
int fused_moe_finalize_rmsnorm(const void* const* partials, int32_t num_partials,
                               const void* expert_out, int64_t num_expanded_rows,
                               const int32_t* expanded_row_idx, const float* topk_weights,
                               int32_t top_k, const void* shared_out,
                               const float* shared_gate_logits, const void* residual_in,
                               const void* gamma, float weight_bias, float eps,
                               int64_t num_tokens, int64_t hidden, void* normed_out,
                               void* residual_out, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Allocation-free variant of fused_moe_finalize_rmsnorm, for callers that
 * cannot allocate device memory or hand over a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  It takes
 * the same arguments minus the workspace, plus top_k == 0 for a call without
 * the MoE finalize (then expert_out, expanded_row_idx, topk_weights,
 * shared_out and shared_gate_logits are ignored, num_partials must be >= 1,
 * and the call is exactly fused_reduce_rmsnorm's); outputs are identical to
 * those entry points' with a workspace.
 *
 * Split rows exchange through a static device array inside the library, one
 * copy per GPU, held until the process ends: 256 bytes plus 512 per token row,
 * for up to FB_NOALLOC_MAX_ROWS rows (512 KiB + 256 bytes).  Calls with more
 * token rows return FB_TOO_MANY_ROWS before launching (outputs untouched).
 * The array starts zero-filled and the split-row protocol keeps it consistent
 * across calls of any shape, so nothing needs clearing.  Every call on a GPU
 * uses that GPU's one array: calls that may overlap on one GPU (different
 * streams, concurrent graph replays) race and must not be made.  A bounded
 * wait that gives up (see above) marks rows in the array for good: their calls
 * stay exact but recompute (slower) until the process ends.  The first call on
 * each device looks up the array's device address (no allocation).  No
 * hipMalloc, hipFree or other allocation, no synchronisation, one launch.
 */
#define FB_NOALLOC_MAX_ROWS 1024
int fused_moe_finalize_rmsnorm_noalloc(const void* const* partials, int32_t num_partials,
                                       const void* expert_out, int64_t num_expanded_rows,
                                       const int32_t* expanded_row_idx,
                                       const float* topk_weights, int32_t top_k,
                                       const void* shared_out, const float* shared_gate_logits,
                                       const void* residual_in, const void* gamma,
                                       float weight_bias, float eps, int64_t num_tokens,
                                       int64_t hidden, void* normed_out, void* residual_out,
                                       void* stream);

/*
 * Split (unfused) boundary: the two-launch flow the fused entry points replace,
 * and the fallback after they return FB_DECLINED.  The pages compare the fused
 * kernel against this flow: the reduction (and the MoE finalize) materialised
 * as a bf16 [T, H] tensor, then a separate residual RMSNorm (PR #37104,
 * Motivation and Performance table; the owed reduction is materialised before
 * the ordinary norm when the fused runtime declines, PR #37104 Changes; the
 * standalone deferred finalize, PR #37196 Modifications part 2).
 * Both stages take any H in [1, FB_MAX_HIDDEN] and 2-byte aligned bf16
 * pointers (4-byte for int32/fp32); 128-bit kernels run when every pointer is
 * 16-byte aligned and H % 8 == 0.  Errors as for the fused entry points
 * (FB_DECLINED only for H > FB_MAX_HIDDEN).  One launch per stage on `stream`,
 * no allocation.
 *
 * Stage 1: sum_out[t] = bf16( sum_r P_r[t] + sum_k fl32(w[t,k] * E[idx[t,k]])
 *                              + fl32(s_t * S[t]) ), fp32 in that order.
 *   Arguments as fused_moe_finalize_rmsnorm; top_k may be 0 (no finalize:
 *   expert_out, expanded_row_idx and topk_weights are then ignored) and
 *   num_partials may be 0.  sum_out: bf16 [T, H], overlapping no input.
 */
int fused_boundary_split_sum(const void* const* partials, int32_t num_partials,
                             const void* expert_out, int64_t num_expanded_rows,
                             const int32_t* expanded_row_idx, const float* topk_weights,
                             int32_t top_k, const void* shared_out,
                             const float* shared_gate_logits, int64_t num_tokens, int64_t hidden,
                             void* sum_out, void* stream);

/* Stage 2: x = fl32(0 + x_in) + residual_in (fp32), residual_out = bf16(x),
 * normed_out = bf16(x * rsqrt(mean(x^2) + eps) * (gamma + weight_bias)).
 * residual_out may equal residual_in exactly. */
int fused_boundary_split_residual_rmsnorm(const void* x_in, const void* residual_in,
                                          const void* gamma, float weight_bias, float eps,
                                          int64_t num_tokens, int64_t hidden, void* normed_out,
                                          void* residual_out, void* stream);

/*
 * Diagnostic: the boundary's memory traffic without its arithmetic, to measure
 * what the part attains for it.  One workgroup per token row, the stream
 * kernel's shape (vec_per_thread 1, 2, 4 or 8 16-byte vectors per lane, so
 * ceil(H / (8 * vec_per_thread)) lanes rounded up to whole waves, at most 512;
 * at most workgroups_per_cu (<= 16) resident per CU, 0 = no limit), the row's
 * gather indices read once into lanes, nontemporal loads of
 * num_direct bf16 [T, H] rows at the row's offset (<= FB_MAX_PARTIALS + 2) and
 * of num_gathered rows of `gathered` ([N, H], N = num_gathered_rows) through
 * gather_idx (int32 [T, num_gathered]; an index outside [0, N) is skipped), then
 * nontemporal stores of num_outputs (<= 2) [T, H] rows: output d holds the XOR
 * of every 32-bit word read for that row, XOR d (a check value, not a result).  All pointers 16-byte aligned, H % 8 == 0,
 * H <= FB_MAX_HIDDEN.  Returns FB_OK, FB_INVALID_ARGUMENT or FB_HIP_ERROR (see
 * fused_boundary_probe_last_hip_error).  One launch on `stream`.
 */
int fused_boundary_bandwidth_probe(const void* const* direct, int32_t num_direct,
                                   const void* gathered, int64_t num_gathered_rows,
                                   const int32_t* gather_idx, int32_t num_gathered,
                                   void* const* outputs, int32_t num_outputs, int64_t num_tokens,
                                   int64_t hidden, int32_t vec_per_thread,
                                   int32_t workgroups_per_cu, void* stream);

/* hipError_t of the most recent FB_HIP_ERROR of a bandwidth-probe call on the
 * calling thread (0 if none). */
int fused_boundary_probe_last_hip_error(void);

/*
 * Diagnostic: how many workgroups of `block` lanes (a multiple of 64, <= 1024)
 * a CU holds at once for kernels that keep different numbers of scalar
 * registers per wave.  Launches `grid` (1..65536) workgroups of a probe kernel
 * built at sgpr_level 0, 1 or 2 (about 20, 88 and 104 SGPRs per wave); the
 * first lane of workgroup g writes out[3g] = XCC id << 32 | HW_ID (the CU's
 * hardware ids), out[3g+1] and out[3g+2] = the realtime counter before and
 * after sleeping sleep_ticks (<= 1e6) of it.  No workgroup waits on another.
 * `out`: device memory of 3 * grid uint64, 8-byte aligned, owned by the
 * caller.  Counting the overlapping intervals per CU gives the workgroups it
 * held at once; the planner's residency rule (a wave holds its SGPR count
 * plus 16, rounded up to 16, of 800 per SIMD) is checked against it.  Returns
 * FB_OK, FB_INVALID_ARGUMENT or FB_HIP_ERROR.  One launch on `stream`.
 */
int fused_boundary_residency_probe(int32_t sgpr_level, int32_t grid, int32_t block,
                                   uint64_t sleep_ticks, void* out, void* stream);

/* hipError_t of the most recent FB_HIP_ERROR of a split-stage call on the
 * calling thread (0 if none). */
int fused_boundary_split_last_hip_error(void);

/* Bytes of workspace that let every call with these sizes use split rows.
 * Returns 0 for negative sizes.  Pure host function. */
size_t fused_boundary_workspace_bytes(int64_t num_tokens, int64_t hidden);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char* fused_boundary_status_string(int status);

/* hipError_t of the most recent FB_HIP_ERROR on the calling thread (0 if none). */
int fused_boundary_last_hip_error(void);

/* Test hook: the number of polls a split row's workgroup makes before it gives
 * up, for subsequent calls on the calling thread; 0 restores the default (about
 * a second of polling) and FB_WAIT_NO_POLL makes every split row give up
 * without polling.  A row that gives up sets status bit
 * FB_WS_STATUS_WAIT_TIMEOUT and takes or recomputes its siblings' sums
 * (outputs unchanged, see "Bounded wait" above).  Lets tests force the
 * time-out path from the host while every kernel still exits normally. */
#define FB_WAIT_NO_POLL 0xFFFFFFFFu
void fused_boundary_set_wait_limit(uint32_t polls);

/* Diagnostic: workgroups of `block` lanes per CU that the planner counts on
 * for the latency kernel (units_per_wave 0) or the balanced kernel with
 * num_partials R and top_k K (*planned) -- its streamed form when
 * sources_per_batch is 2 (units_per_wave 1), else 0 -- and what the runtime's
 * occupancy query reports for that kernel on the current device (*device).
 * The planner launches split-row and balanced grids no larger than CUs x
 * *planned, so *planned must never exceed *device.  The runtime's query
 * counts registers and LDS but not the 16 scalar registers per wave that
 * MI355X sets aside (fused_boundary_residency_probe measures it), so it can
 * overstate what fits; the planner's table is also held to that tighter
 * bound.  Returns FB_OK, FB_INVALID_ARGUMENT, or FB_HIP_ERROR (no device;
 * *device = -1). */
int fused_boundary_resident_workgroups(int32_t num_partials, int32_t top_k,
                                       int32_t units_per_wave, int32_t sources_per_batch,
                                       int32_t block, int32_t* planned, int32_t* device);

/* Test hook: while on (non-zero), the two fused entry points return FB_DECLINED
 * on the calling thread for every call that passes argument validation and
 * has T > 0, before anything is launched, as a runtime decline would (the
 * decline path of PR #37104, Changes, and its mocked-decline regression test,
 * Correctness; PR #42020, Summary).  Lets tests drive a caller's fallback on
 * ordinary shapes. */
void fused_boundary_set_force_decline(int on);

/*
 * Launch plan: how a call with these sizes is laid out on the GPU.  Used by
 * benchmarks and tests; the entry points pick it themselves.
 *   block              threads per workgroup (a multiple of 64, <= 1024)
 *   vec_per_thread     16-byte vectors (8 bf16) each thread owns per row: 1, 2, 4 or 8
 *   split              workgroups per row (1 = whole row in one workgroup);
 *                      balanced kernel: units per row, ceil(H / 512)
 *   grid               workgroups launched (num_tokens * split; balanced
 *                      kernel: ceil(waves / (block / 64)))
 *   sources_per_batch  0: latency kernel (one vector per thread, every source
 *                      in flight at once, rows may be split) or balanced
 *                      kernel;  1, 2, 4 or 8: stream kernel (whole rows,
 *                      sources fetched this many at a time with streaming
 *                      loads);  2 with units_per_wave 1: the balanced
 *                      kernel's streamed form (each wave's unit fetches its
 *                      sources two at a time)
 *   workgroups_per_cu  stream and balanced kernels: at most this many
 *                      workgroups resident on a CU (the launch reserves LDS
 *                      to hold it there), 1..16; 0 = as many as registers
 *                      allow.  Fewer rows in flight keep HBM streaming more
 *                      efficiently.  0 for the latency kernel.
 *   units_per_wave     0: not the balanced kernel.  1, 2, 3, 4, 6 or 8: the
 *                      balanced kernel, which cuts rows into units of 512
 *                      elements (64 lanes x 8), gives each of
 *                      workgroups_per_cu (0 = 1) workgroups per CU an equal
 *                      run of units and each wave at most this many; the whole
 *                      grid is resident at once.
 *   waves              balanced kernel: waves launched (grid * block / 64).
 */
typedef struct fused_boundary_plan {
  int32_t block;
  int32_t vec_per_thread;
  int32_t split;
  int32_t grid;
  int32_t sources_per_batch;
  int32_t workgroups_per_cu;
  int32_t units_per_wave;
  int32_t waves;
} fused_boundary_plan;

/* The plan a call would use for these sizes (num_partials R, top_k K = 0 for
 * the reduce entry point, has_shared 0/1) with a workspace of workspace_bytes
 * (0 = none).  Returns FB_OK, FB_INVALID_ARGUMENT or FB_DECLINED.  Host only,
 * apart from a cached device-attribute query. */
int fused_boundary_get_plan(int64_t num_tokens, int64_t hidden, int32_t num_partials,
                            int32_t top_k, int32_t has_shared, size_t workspace_bytes,
                            fused_boundary_plan* plan);

/* Force (block, vec_per_thread, sources_per_batch, workgroups_per_cu,
 * units_per_wave) for subsequent calls on the calling thread; split, grid and
 * waves follow from the sizes.  NULL restores the
 * automatic choice.  Returns FB_INVALID_ARGUMENT for an unsupported
 * combination.  A call whose forced plan does not fit (a stream plan shorter
 * than the row, a split plan without a large enough workspace, a latency
 * block too wide for its R and K, a balanced grid larger than can be resident
 * at once, with more than units_per_wave units for some wave or more rows per
 * workgroup than its routing lanes hold) returns
 * FB_INVALID_ARGUMENT.  Latency blocks may be up to 1024 threads for R <= 8
 * with K = 0 or K <= 8, up to 512 for R <= 8 with K <= 12, and up to 256
 * otherwise. */
int fused_boundary_set_plan_override(const fused_boundary_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* FUSED_BOUNDARY_H_ */
