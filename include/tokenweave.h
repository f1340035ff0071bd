/*
 * tokenweave.h -- C ABI of the MI355X (gfx950) fused reduce + residual-add +
 * RMSNorm library and its wave-aware split planner.
 *
 * Sources, by page title and section:
 *   [Blog]  "TokenWeave: Why Hiding Tensor-Parallel Communication Needs Wave
 *           Arithmetic, Not Finer Tiles" -- sections "The overlap trap",
 *           "Fix one: split at wave boundaries, unequally" and "Fix two:
 *           RMSNorm was never insignificant" (the per-CTA kernel sketch).
 *   [Guide] "TokenWeave Guide: Compute-Communication Overlap for LLMs" --
 *           section "Fused AllReduce-RMSNorm: Bypassing Global Memory" (the
 *           RMSNorm equation).
 *
 * The header uses only C types: streams are opaque `void*` (a hipStream_t,
 * NULL for the null stream), so it can be included without HIP headers and
 * loaded with ctypes.
 *
 * Ownership and threading
 *   - The caller owns all memory.  The library never allocates, frees or
 *     synchronizes device memory; kernels are enqueued on the caller's stream
 *     and the call returns after the enqueue.
 *   - Device faults surface at the caller's next synchronization; launch
 *     errors come back as TW_ERR_DEVICE.
 *   - The only global state is a thread-local last-error string and the
 *     process-wide pointer-check switch (an atomic), so calls from several
 *     host threads are safe.
 *
 * Errors: every argument is checked before any HIP call is made, so an
 * argument error never touches the device.
 */
#ifndef TOKENWEAVE_H_
#define TOKENWEAVE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TW_OK = 0,
  TW_ERR_INVALID_ARG = 1,   /* argument out of its documented range */
  TW_ERR_UNSUPPORTED = 2,   /* valid, but outside what the kernels handle */
  TW_ERR_DEVICE = 3         /* the HIP runtime reported an error */
} tw_status;

typedef enum {
  TW_F32 = 0,               /* IEEE binary32 */
  TW_BF16 = 1               /* bfloat16: the upper 16 bits of a binary32 */
} tw_dtype;

#define TW_MAX_PARTIALS 16        /* tensor-parallel degree N handled */
#define TW_MAX_ROW_BYTES 131072   /* largest hidden * sizeof(dtype): h <= 65536
                                     for bf16, h <= 32768 for fp32 */
#define TW_MAX_TOKENS 2147483647  /* largest num_tokens */

#define TW_ABI_VERSION 2

/* Version of this ABI (TW_ABI_VERSION of the built library). */
int32_t tw_abi_version(void);

/*
 * tw_set_pointer_checks -- opt-in verification of tensor pointers (default:
 * off).  When enabled, every entry that launches a kernel also asks the HIP
 * runtime, after the argument checks, whether each tensor is device (or
 * managed) memory and whether its whole byte range lies inside one
 * allocation; if not, the call returns TW_ERR_INVALID_ARG and launches
 * nothing.  This turns a host pointer or a short buffer into an error instead
 * of a device memory fault, for a few runtime queries per call.  The setting
 * is process-wide and may be changed from any thread.
 *   enabled   nonzero: on; 0: off
 */
void tw_set_pointer_checks(int32_t enabled);

/*
 * tw_fused_reduce_rmsnorm -- the fused step for every token row.
 *
 * [Blog] "Fix two", kernel sketch, and [Guide] RMSNorm equation.  For each
 * row t < num_tokens, in float32 arithmetic:
 *     x      = sum_{i<N} partials[i][t,:] + residual[t,:]
 *     rs     = 1 / sqrt( (sum_j x_j^2) / hidden + eps )
 *     out[t,:]          = round_dtype( (x * rs) * weight )
 *     residual_out[t,:] = round_dtype( x )
 * The N partials stand for the row-parallel GEMM outputs of N tensor-parallel
 * ranks (on the pages the NVSwitch reduces them; here they are N buffers in
 * this GPU's memory).  The partial sum is a compensated (error-free
 * transformation) float32 sum; rounding to bf16 is round-to-nearest-even.
 * NaN and infinite inputs propagate to their row.  A row whose sum of
 * squares overflows float32 (|x| above about 1.8e19) gets rs = 0 and out = 0
 * (NaN where x is infinite); residual_out is still x rounded.
 * The order of the sum of squares depends only on hidden, dtype and N, so a
 * row's results are bit-identical whichever entry point or batch size
 * computes it (how a launch schedules its loads changes no bit).  The same
 * inputs in another order of the partials may differ in the last bit of out,
 * except where the sums are exact.
 *
 * Arguments
 *   partials      host array of num_partials device pointers, each to a
 *                 row-major [num_tokens, hidden] tensor of `dtype`
 *   num_partials  N, 1..TW_MAX_PARTIALS
 *   residual      device [num_tokens, hidden] `dtype`
 *   weight        device [hidden] `dtype` (the RMSNorm gamma)
 *   out           device [num_tokens, hidden] `dtype`, written
 *   residual_out  device [num_tokens, hidden] `dtype`, written; may equal
 *                 `residual` exactly (in-place update)
 *   num_tokens    T >= 0; T == 0 is a no-op returning TW_OK
 *   hidden        h >= 1; must be a multiple of 16/sizeof(dtype), with
 *                 h * sizeof(dtype) <= TW_MAX_ROW_BYTES
 *   eps           finite, >= 0, added to the mean of squares under the root
 *   dtype         element type of every tensor
 *   stream        hipStream_t to enqueue on, NULL for the null stream
 *
 * Errors
 *   TW_ERR_INVALID_ARG  N out of range, T < 0, h < 1, eps negative or not
 *                       finite, a NULL pointer when T > 0, an output range
 *                       overlapping an input or the other output (except
 *                       residual_out == residual), an unknown dtype value
 *   TW_ERR_UNSUPPORTED  a pointer not 16-byte aligned, h not a multiple of
 *                       16/sizeof(dtype), h * sizeof(dtype) > TW_MAX_ROW_BYTES,
 *                       num_tokens > TW_MAX_TOKENS
 *   TW_ERR_DEVICE       the launch failed (see tw_last_error())
 */
tw_status tw_fused_reduce_rmsnorm(const void* const* partials, int32_t num_partials,
                                  const void* residual, const void* weight,
                                  void* out, void* residual_out,
                                  int64_t num_tokens, int64_t hidden, float eps,
                                  tw_dtype dtype, void* stream);

/*
 * tw_fused_reduce_rmsnorm_grid -- the fused step on a fixed number of
 * workgroups.
 *
 * [Blog] "Fix two", kernel sketch: each CTA of the grid takes
 * ceil(num_tokens / grid) consecutive tokens; [Blog] "What it buys": the
 * pages' kernel runs near-optimally on about 8 SMs and is deployed on 2-8, so
 * that the GEMM it overlaps keeps the rest.  Workgroup b processes rows
 * [b*ceil(T/G), min(T, (b+1)*ceil(T/G))) one after another, G =
 * num_workgroups.  Results are bit-identical to tw_fused_reduce_rmsnorm (the
 * per-row code is the same); only how many CUs the launch can occupy changes.
 *
 * Arguments are those of tw_fused_reduce_rmsnorm plus
 *   num_workgroups  G >= 1 (else TW_ERR_INVALID_ARG); G >= T runs one
 *                   workgroup per row, as tw_fused_reduce_rmsnorm does.
 */
tw_status tw_fused_reduce_rmsnorm_grid(const void* const* partials, int32_t num_partials,
                                       const void* residual, const void* weight,
                                       void* out, void* residual_out,
                                       int64_t num_tokens, int64_t hidden, float eps,
                                       tw_dtype dtype, int32_t num_workgroups, void* stream);

/*
 * tw_shard_rmsnorm -- the fused step on one rank's token shard.
 *
 * [Blog] "Fix two": after a ReduceScatter split at token boundaries each of
 * the N ranks owns complete rows for 1/N of the tokens and normalizes only
 * those.  Shard k covers rows [floor(k*T/N), floor((k+1)*T/N)) with N =
 * num_partials.  Every tensor argument is the FULL [num_tokens, hidden]
 * buffer; only the shard's rows are read (of partials and residual) and
 * written (of out and residual_out), at their own row offsets, and all other
 * rows are left untouched.  Per-row arithmetic is bit-identical to
 * tw_fused_reduce_rmsnorm.
 *
 * Arguments are those of tw_fused_reduce_rmsnorm plus
 *   shard_index   k, 0 <= k < num_partials (else TW_ERR_INVALID_ARG)
 * An empty shard (T < N) is a no-op returning TW_OK.
 */
tw_status tw_shard_rmsnorm(const void* const* partials, int32_t num_partials,
                           const void* residual, const void* weight,
                           void* out, void* residual_out,
                           int64_t num_tokens, int64_t hidden, float eps,
                           tw_dtype dtype, int32_t shard_index, void* stream);

/*
 * Unfused comparator (not on the fused path).  [Blog] "What it buys" measures
 * the fused kernel against a standalone AllReduce followed by a standalone
 * RMSNorm; [Blog] "Fix two" describes the standard RMSNorm as reading the
 * tensor twice (once for the variance, once to scale) and writing it once.
 * These two calls are that sequence on one GPU, for timing against
 * tw_fused_reduce_rmsnorm: (N+3) reads and 3 writes of [T, h] against the
 * fused kernel's (N+1) reads and 2 writes.
 *
 * tw_reduce_partials -- the AllReduce result:
 *     reduced[t,:] = round_dtype( sum_{i<N} partials[i][t,:] )
 * with the fused kernel's compensated float32 sum.
 *   partials, num_partials, num_tokens, hidden, dtype, stream: as for
 *                 tw_fused_reduce_rmsnorm
 *   reduced       device [num_tokens, hidden] `dtype`, written; must not
 *                 overlap a partial
 * Errors: those of tw_fused_reduce_rmsnorm that apply to these arguments.
 */
tw_status tw_reduce_partials(const void* const* partials, int32_t num_partials, void* reduced,
                             int64_t num_tokens, int64_t hidden, tw_dtype dtype, void* stream);

/*
 * tw_add_rmsnorm -- standard two-pass residual-add + RMSNorm.  Per row:
 *   pass 1: x = input + residual (compensated float32), residual_out =
 *           round_dtype(x), s = sum_j x_j^2 of the unrounded x;
 *   pass 2: re-read residual_out, out = round_dtype((x' * rs) * weight) with
 *           x' the stored (rounded) value and rs = 1/sqrt(s/hidden + eps).
 * Arguments as for tw_fused_reduce_rmsnorm with one partial (`input`);
 * residual_out may equal residual exactly.  Same errors.
 */
tw_status tw_add_rmsnorm(const void* input, const void* residual, const void* weight, void* out,
                         void* residual_out, int64_t num_tokens, int64_t hidden, float eps,
                         tw_dtype dtype, void* stream);

/*
 * Split planner: [Blog] "The overlap trap" and "Fix one".  A GEMM over M
 * token rows launches ceil(M / tokens_per_cta) * ctas_per_token_tile CTAs;
 * a wave holds num_cus * ctas_per_cu of them; waves(M) = ceil(CTAs / that).
 * The batch of T tokens is split in two, prefix = floor(T/2) + offset and
 * suffix = T - prefix, with the first offset (in the given order) below
 * floor(T/2) for which waves(prefix) + waves(suffix) <= waves(T).  No split
 * when T == 0, when T < min_split_tokens, when waves(T) <= 1, or when no
 * offset qualifies; then prefix = T, suffix = 0, offset = -1.
 */
typedef struct {
  int64_t num_tokens;           /* T = B * L, >= 0 */
  int64_t tokens_per_cta;       /* GEMM tile rows (M-tile), >= 1 */
  int64_t ctas_per_token_tile;  /* GEMM tiles across the output features, >= 1 */
  int32_t num_cus;              /* compute units (256 on MI355X), >= 1 */
  int32_t ctas_per_cu;          /* resident CTAs per CU in one wave, >= 1 */
  int64_t min_split_tokens;     /* split threshold, >= 0 (0 disables it) */
  const int32_t* offsets;       /* candidate offsets, strictly ascending,
                                   >= 0; NULL selects {0,64,128,192,256,512} */
  int32_t num_offsets;          /* length of offsets (0 when offsets is NULL) */
} tw_split_problem;

#define TW_PLAN_SPLIT 0
#define TW_PLAN_BELOW_THRESHOLD 1
#define TW_PLAN_SINGLE_WAVE 2
#define TW_PLAN_NO_FEASIBLE_OFFSET 3
#define TW_PLAN_EMPTY 4
#define TW_PLAN_MEASURED_SPLIT 5        /* tw_split_plan_measured: the table's offset */
#define TW_PLAN_MEASURED_UNSPLIT 6      /* tw_split_plan_measured: the table keeps T whole */
#define TW_PLAN_MEASURED_OVER_WAVES 7   /* tw_split_plan_measured: the table's offset breaks
                                           the wave condition, so T stays whole */

typedef struct {
  int64_t prefix_tokens;
  int64_t suffix_tokens;
  int32_t offset;               /* -1 when not split */
  int32_t waves_unsplit;
  int32_t waves_prefix;
  int32_t waves_suffix;
  int32_t reason;               /* one of TW_PLAN_* */
} tw_split_plan_result;
/* A plan splits exactly when suffix_tokens > 0 (reasons TW_PLAN_SPLIT and
 * TW_PLAN_MEASURED_SPLIT); then prefix_tokens = floor(T/2) + offset. */

/*
 * tw_split_plan -- host only, integer arithmetic, no device call.
 *   in, out       non-NULL (else TW_ERR_INVALID_ARG)
 * Errors: TW_ERR_INVALID_ARG for a field out of range or offsets not
 * strictly ascending; TW_ERR_UNSUPPORTED when num_tokens exceeds 2^40,
 * ctas_per_token_tile exceeds 2^20 or a wave count does not fit in int32.
 */
tw_status tw_split_plan(const tw_split_problem* in, tw_split_plan_result* out);

/*
 * Measured split table.  [Blog] "Fix one" chooses the offset per shape by
 * timing the two GEMMs offline and keeps the winner in a lookup table keyed
 * by the shape.  One entry of such a table:
 */
typedef struct {
  int64_t num_tokens;           /* T the entry applies to, >= 1 */
  int32_t offset;               /* the measured winner: 0 <= offset < floor(T/2),
                                   or -1 when the whole batch was fastest */
} tw_split_entry;

/*
 * tw_split_plan_measured -- tw_split_plan with a measured table consulted
 * first.  host only, integer arithmetic, no device call.
 *   in            the problem, as for tw_split_plan (its offsets serve the
 *                 analytic search of counts the table does not list)
 *   table         table_len entries, token counts strictly ascending; the
 *                 caller keeps ownership (the library keeps no pointer)
 *   table_len     >= 0; 0 (table may be NULL) gives exactly tw_split_plan
 *   out           non-NULL
 * In the pages' order: T == 0, T < min_split_tokens and waves(T) <= 1 keep
 * the batch whole, as in tw_split_plan, before the table is read.  A T the
 * table lists then takes the table's offset: -1 keeps it whole
 * (TW_PLAN_MEASURED_UNSPLIT); an offset whose pieces take no more waves than
 * the whole batch splits at prefix = floor(T/2) + offset
 * (TW_PLAN_MEASURED_SPLIT); an offset whose pieces take more keeps it whole
 * (TW_PLAN_MEASURED_OVER_WAVES), since the planner never exceeds the
 * unsplit wave count.  A T the table does not list gets tw_split_plan's
 * analytic plan.  The wave fields always describe the returned pieces.
 * Errors: those of tw_split_plan; TW_ERR_INVALID_ARG also for table_len < 0,
 * a NULL table with table_len > 0, token counts not >= 1 and strictly
 * ascending, or an offset outside [0, floor(num_tokens/2)) other than -1.
 */
tw_status tw_split_plan_measured(const tw_split_problem* in, const tw_split_entry* table,
                                 int32_t table_len, tw_split_plan_result* out);

/*
 * tw_fused_launch_info -- how tw_fused_reduce_rmsnorm would launch a call
 * (host only; runtime queries, no launch).  A round is the workgroups
 * resident at once on the CUs the stream may use: the device's CU count, or
 * the CUs of the stream's CU mask when fewer.  The launch rules (which kernel
 * a dispatch runs) depend on the row count against that round; they never
 * change a result bit.  A long call is cut into dispatches of consecutive
 * rows, each taking its own kernel for its row count; `kernel` is that of
 * the first dispatch (of rows_per_dispatch rows).
 *   num_partials, num_tokens, hidden, dtype, stream: as for
 *                 tw_fused_reduce_rmsnorm (a shard or split launch passes its
 *                 own row count)
 *   out           non-NULL (else TW_ERR_INVALID_ARG)
 * Errors: those of tw_fused_reduce_rmsnorm that apply to the scalars.
 */
#define TW_KERNEL_ALL_AT_ONCE 0   /* one workgroup per row, all loads issued at once */
#define TW_KERNEL_SEQUENCED 1     /* one workgroup per row, tensors loaded in sequence */
#define TW_KERNEL_STRIDED 2       /* one round of workgroups, each taking every round-th row */
#define TW_KERNEL_BOTH_SLOTS 3    /* one workgroup per row, both vector slots' loads at once */
typedef struct {
  int32_t num_cus;                /* CUs counted for the stream */
  int32_t threads_per_workgroup;
  int32_t vectors_per_thread;     /* 16-byte vectors of a row per thread */
  int32_t kernel;                 /* TW_KERNEL_* of the first dispatch; -1 when T == 0 */
  int64_t round_rows;             /* workgroups resident at once */
  int64_t rows_per_dispatch;      /* 0 when T == 0 */
  int64_t dispatches;             /* 0 when T == 0 */
} tw_launch_info;

tw_status tw_fused_launch_info(int32_t num_partials, int64_t num_tokens, int64_t hidden,
                               tw_dtype dtype, void* stream, tw_launch_info* out);

/* Static description of a status code. */
const char* tw_status_string(tw_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* tw_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKENWEAVE_H_ */
