/*
 * rowred.h -- fused FP32 row reductions on AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every entry point is extern "C", takes plain pointers and sizes,
 * returns an int status (enum rowred_status) and never throws.
 *
 * Layout: every matrix is row-major FP32, `rows` x `width`, row stride equal
 * to `width` elements, contiguous.  All matrix pointers are device pointers
 * and must be 4-byte aligned; 16-byte alignment is not required.  x is read
 * 16 bytes at a time; r and y are read / written 16 bytes at a time when
 * they share x's address modulo 16, otherwise 4 bytes at a time (equally
 * valid results, lower bandwidth).
 *
 * Reads: each row is fetched as the run of whole 16-byte granules that
 * contain it, so a call may read up to 12 bytes before the first element and
 * after the last element of x (and r), always inside the 16-byte granules
 * that hold valid elements.  Those extra values are never used and never
 * written.
 *
 * Writes: exactly the rows*width elements of y, each once.
 *
 * Ownership: the caller owns all memory.  The library allocates nothing,
 * keeps no per-call state and is safe to call from several host threads.
 *
 * Asynchrony: work is enqueued on `stream` (NULL = the default stream) and
 * the call returns without synchronising, so calls can be captured into a
 * HIP graph.  ROWRED_ERR_HIP reports a failed launch; a fault during the
 * kernel surfaces at the caller's next synchronisation.
 *
 * Aliasing: y must not overlap x or r (checked on the host,
 * ROWRED_ERR_ALIAS); x and r may overlap each other (both are only read).
 * The kernels keep each row in registers between its phases, so an in-place
 * call would be computable, but the no-overlap rule follows the pages'
 * requirement that the caller guarantee noalias and that a packed row tail
 * never reads and writes one buffer ("Immutable input reuse in Metal
 * reductions", section "What the transformation actually preserves";
 * "Cooperating-program packing: implementation and fixed-plan evidence",
 * section "Implementation boundary").
 *
 * Sizes: rows < 0 or width < 0 -> ROWRED_ERR_INVALID_ARG.  rows == 0 or
 * width == 0 -> ROWRED_OK with nothing launched (pointers may then be NULL).
 * A NULL or misaligned pointer otherwise -> ROWRED_ERR_INVALID_ARG.  A row
 * whose 16-byte slot window (ceil((width + misalignment) / 4)) is at most
 * 8192 (width <= 32768 for 16-byte-aligned rows) is held in registers across
 * the phases and read once.  LayerNorm, RMSNorm and softmax rows wider than
 * that (up to 64 segments of 4096 slots, about a million columns; LayerNorm
 * 128), and in calls of 128 MiB or more per input also LayerNorm rows of
 * 2049-8192 slots and RMSNorm / softmax rows of 4097-8192 (rows off 16-byte
 * boundaries: 512 MiB), are cut into segments of one workgroup each that
 * hold their part in registers (and LDS) and swap their statistics through
 * words kept in y's own row (ROWRED_POLICY_EXCHANGE on a row plan): read
 * once, no workspace.  That needs the device to hold twice a row's
 * segments at once.  Where it does not, for wider rows, and for affine
 * LayerNorm beyond 8192 slots with 256 rows or more (where the exchange is
 * slower): RMSNorm and softmax rows of up to 16384 slots are held in
 * registers and LDS (ROWRED_POLICY_LDS_STRIPE), wider ones have their first
 * 16384 slots held
 * that way, wider LayerNorm rows x and r of their first 8192, and the rest
 * is walked twice (ROWRED_POLICY_LDS_STRIPE | ROWRED_POLICY_LOOPED).  Wider
 * row sum and min/max rows are walked once by one workgroup
 * (ROWRED_POLICY_LOOPED); for few of them the _ws entry points at the end
 * split each row over many workgroups.  width > ROWRED_MAX_WIDTH ->
 * ROWRED_ERR_UNSUPPORTED.
 *
 * eps must be finite and >= 0, else ROWRED_ERR_INVALID_ARG.  eps = 0 is
 * accepted; a LayerNorm row with zero variance then gives NaN (0/0), as
 * IEEE arithmetic does.  NaN and infinite inputs propagate with no special
 * case.
 *
 * Determinism: for a fixed plan (see rowred_plan_query) results are bitwise
 * reproducible from run to run.
 */
#ifndef ROWRED_H
#define ROWRED_H

#include <stddef.h>
#include <stdint.h>

/* Widest row any entry point takes: 2^31 - 2^20 - 1 floats.  The kernels
 * index a row's elements, and the 16-byte granules past its end that their
 * last tile or segment covers, in 32-bit integers; this keeps every such
 * index below 2^31. */
#define ROWRED_MAX_WIDTH 2146435071LL

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (identical to the typedef in hip_runtime_api.h). */
struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

enum rowred_status {
  ROWRED_OK = 0,
  ROWRED_ERR_INVALID_ARG = 1, /* bad size, pointer, eps or plan */
  ROWRED_ERR_ALIAS = 2,       /* y overlaps an input */
  ROWRED_ERR_UNSUPPORTED = 3, /* a size beyond the limits stated below (32-bit widths, launch grid) */
  ROWRED_ERR_HIP = 4          /* the HIP runtime refused the launch */
};

enum rowred_op {
  ROWRED_OP_LAYERNORM_RESIDUAL = 0,
  ROWRED_OP_RMSNORM = 1,
  ROWRED_OP_SOFTMAX = 2,
  ROWRED_OP_ROW_SUM = 3,
  ROWRED_OP_ROW_MINMAX = 4
};

/*
 * Residual LayerNorm without affine parameters, per row i:
 *   c = x_i + r_i;  mean = sum(c) / width;  d = c - mean;
 *   var = sum(d^2) / width  (biased, second pass over d);
 *   y_i = d / sqrt(var + eps).
 * Defined by the residual LayerNorm program in "Residual LayerNorm
 * shared-Tile materialization search", section "Structural finding"; the
 * pages use eps = 1e-5.  Only y is written (the combined row is not).
 * x, r: inputs (rows x width); r must be non-NULL.  y: output.
 */
int rowred_layernorm_residual(const float *x, const float *r, float *y,
                              int64_t rows, int64_t width, float eps,
                              hipStream_t stream);

/*
 * LayerNorm with an optional residual and optional affine vectors, per row i:
 *   c = x_i (+ r_i);  mean, d, var as above;  y_ij = d_j / sqrt(var + eps)
 *   (* gamma_j) (+ beta_j).
 * r, gamma and beta may each be NULL: r = NULL is plain LayerNorm, the form
 * timed next to softmax and RMSNorm in "Immutable input reuse in Metal
 * reductions", section "Fixed-width GPU and dispatch results"; gamma/beta
 * are the affine form named in the tolerance list of "Cooperating-program
 * packing: implementation and fixed-plan evidence", section "Predeclared
 * comparison and measurement".  gamma and beta hold `width` floats each
 * (4-byte aligned, read only, must not overlap y), never read beyond
 * their `width` elements.  With all three NULL this is the no-affine
 * LayerNorm of the same page's "Validation" section.  With gamma or beta,
 * rows of 6145-8192 granules (24577-32768 floats for 16-byte aligned rows)
 * take the exchange kernels in large calls (see Sizes above) and the looped
 * kernels otherwise (gamma/beta need registers the wider register-resident
 * kernels do not have), wider rows the head+tail kernels (the exchange
 * kernels below 256 rows).
 */
int rowred_layernorm(const float *x, const float *r, const float *gamma,
                     const float *beta, float *y, int64_t rows, int64_t width,
                     float eps, hipStream_t stream);

/*
 * RMSNorm without weight, per row i:  y_i = x_i / sqrt(sum(x_i^2)/width + eps).
 * "Immutable input reuse in Metal reductions", section "What the
 * transformation actually preserves", gives its phases (one sum-of-squares
 * reduction, then an output map over the same input); the formula is the
 * plain definition.  Typical eps = 1e-6.
 */
int rowred_rmsnorm(const float *x, float *y, int64_t rows, int64_t width,
                   float eps, hipStream_t stream);

/*
 * Softmax with max subtraction, per row i:
 *   m = max_j x_ij;  e_j = exp(x_ij - m);  y_ij = e_j / sum_j e_j.
 * Phases as in "Immutable input reuse in Metal reductions", section "What
 * the transformation actually preserves" (max, then exp-sum over a computed
 * stripe, then normalise).  -inf entries get weight 0; a row that is all
 * -inf gives NaN (-inf - -inf).  The normaliser is applied as one
 * reciprocal per row times each e_j.
 */
int rowred_softmax(const float *x, float *y, int64_t rows, int64_t width,
                   hipStream_t stream);

/*
 * Row sum: out[i] = sum_j x_ij, accumulated in FP64 and rounded once to FP32.
 * Paired row min/max: out_min[i] = min_j x_ij, out_max[i] = max_j x_ij,
 * exact; NaN entries are skipped (IEEE minNum/maxNum), so an all-NaN row
 * gives (+inf, -inf).  Sum is the identical-source control and min/max one of
 * the four operators of "Cooperating-program packing: implementation and
 * fixed-plan evidence", section "Validation"; "Immutable input reuse in Metal
 * reductions", section "Fixed-width GPU and dispatch results", times sum.
 * out, out_min, out_max hold `rows` floats (4-byte aligned) and must not
 * overlap x or each other.  A row needs at least one element: width == 0 with
 * rows > 0 -> ROWRED_ERR_INVALID_ARG.  Same loads, geometry and width cap as
 * the entry points above; the outputs are written by one lane per row.
 */
int rowred_row_sum(const float *x, float *out, int64_t rows, int64_t width,
                   hipStream_t stream);
int rowred_row_minmax(const float *x, float *out_min, float *out_max,
                      int64_t rows, int64_t width, hipStream_t stream);

/*
 * Launch geometry.  A row is owned by `lanes_per_row` (L) consecutive lanes
 * of one workgroup; `rows_per_group` = threads / L rows share a workgroup
 * (several short rows per wavefront when L < 64, one or more wavefronts per
 * row when L >= 64).  Lane l of a row holds, for chunk c < chunks, the 16-byte
 * slot c*L + l of the row's window, so each input element is read once and
 * stays in registers through every phase of the reduction.  This is the
 * packing geometry of "Cooperating-program packing: implementation and
 * fixed-plan evidence", section "Implementation boundary", and the element
 * ownership map of "Immutable input reuse in Metal reductions", section
 * "What the transformation actually preserves", with 4 elements per slot.
 * The last workgroup's surplus row slots recompute the last row and store
 * nothing.
 */
typedef struct rowred_plan {
  int32_t lanes_per_row;  /* L: power of two, 1..1024 */
  int32_t rows_per_group; /* threads / L (ROWRED_POLICY_EXCHANGE: 1) */
  int32_t chunks;         /* 16-byte slots per lane: 1..8, 10, 12 or 16 (affine LayerNorm: <= 12) */
  int32_t threads;        /* workgroup size: multiple of 64, <= 1024 (<= 512 when chunks > 8,
                             and for affine LayerNorm when chunks >= 7) */
  int64_t grid;           /* workgroups launched: ceil(rows / rows_per_group)
                             (ROWRED_POLICY_EXCHANGE: rows * segments per row) */
  int32_t vector_io;      /* 1: r and y share x's address modulo 16 (all accesses 16 bytes) */
  int32_t window;         /* largest number of 16-byte granules a row of x spans (L*chunks covers it;
                             ROWRED_POLICY_EXCHANGE: segments of L*chunks do) */
  int32_t policy;         /* memory policy: ROWRED_POLICY_* bits */
  int32_t reserved;       /* 0 */
} rowred_plan;

/* Policy bits of a plan.  They change speed; all but ROWRED_POLICY_ONLINE
 * leave the results bit for bit unchanged. */
enum rowred_policy {
  ROWRED_POLICY_NT_LOADS = 1,   /* loads carry the non-temporal (streaming) hint */
  ROWRED_POLICY_NT_STORES = 2,  /* stores carry the non-temporal hint */
  ROWRED_POLICY_XCD_REMAP = 4,  /* each XCD walks one contiguous range of row blocks */
  ROWRED_POLICY_STAGE_STORES = 8, /* a workgroup's outputs (its rows are consecutive) are
                                     assembled in LDS and stored as whole 16-byte granules by
                                     consecutive threads; needs y at x's 16-byte phase,
                                     threads <= 512 and chunks <= 4 */
  ROWRED_POLICY_RELOAD = 16,      /* diagnostic: every phase after the first reads x (and r)
                                     again instead of keeping the row in registers, and
                                     recomputes what it derives from them (the per-phase
                                     reload of the reference design in "Immutable input reuse
                                     in Metal reductions", section "What the transformation
                                     actually preserves").  Same arithmetic, same results,
                                     more reads.  Matrix operators only (LayerNorm without
                                     gamma/beta, RMSNorm, softmax), chunks <= 8, LayerNorm at
                                     7-8 chunks with threads <= 512; never chosen by the
                                     entry points */
  ROWRED_POLICY_REVERSE = 32,     /* split plans (rowred_split_plan): the apply kernel walks
                                     the (row, segment) pairs in reverse order, so that it
                                     first reads again what the statistics kernel read last;
                                     head+tail row plans (LOOPED | LDS_STRIPE, below): the
                                     second walk takes the tail last tile first.  Measured
                                     no faster, never chosen */
  ROWRED_POLICY_LOOPED = 64,      /* rows of any width: lanes_per_row == threads, one row per
                                     workgroup, which walks the row in tiles of threads * chunks
                                     granules (chunks 2 or 4; LayerNorm 2) twice -- statistics
                                     with cached loads, then map and store (row sum and min/max:
                                     once).  NT_LOADS / NT_STORES apply to the second walk,
                                     XCD_REMAP to the row order; no other bit may be set.  The
                                     entry points choose it for row sum and min/max rows wider
                                     than 8192 granules.  With LDS_STRIPE (rows wider than the
                                     held head): RMSNorm and softmax with chunks 16 hold the
                                     first 16384 granules as LDS_STRIPE holds them, LayerNorm
                                     with chunks 8 holds x and r of the first 8192 (4 register
                                     and 4 LDS slots of each), and the rest is walked twice in
                                     tiles; REVERSE then walks the tail last tile first in the
                                     second walk and maps the head after it (measured within
                                     3% either way, not chosen) */
  ROWRED_POLICY_EXCHANGE = 128,   /* LayerNorm / RMSNorm / softmax.  Split plans: one kernel
                                     instead of three.  Each (row, segment) workgroup keeps its
                                     segment in registers, publishes its statistics to the
                                     workspace and waits for the row's other segments, so x (and
                                     r) are read once.  Needs S <= 128 and S <= threads;
                                     chunks may also be 8
                                     (threads <= 512; not LayerNorm).
                                     NT_LOADS / NT_STORES apply to its loads and stores;
                                     REVERSE may not be set.
                                     Row plans (lanes_per_row == threads, beside it only
                                     NT_LOADS, NT_STORES and LDS_STRIPE): the same kernels with
                                     the geometry of the split plan of these threads, chunks and
                                     policy (S segments of threads * chunks granules per row,
                                     grid = rows * S), the statistics swapped through 8-byte
                                     words in y's own row, from its first 16-byte boundary: 2S +
                                     1 for LayerNorm, S + 1 otherwise, which must end within the
                                     first segment's outputs (16 * threads * chunks - 12 bytes;
                                     LayerNorm: within the granules of its first slot, 16 *
                                     threads - 12 bytes) and within the row (else
                                     ROWRED_ERR_INVALID_ARG).  A small kernel zeroes them first.
                                     RMSNorm and softmax: the first segment writes its outputs
                                     over them once every segment of the row has read them.
                                     LayerNorm: the first segment leaves its granules over the
                                     words unstored, and the workgroup that is the last of the
                                     row to finish reading them computes and stores those.  The
                                     device must hold 2S of these workgroups at once, else
                                     ROWRED_ERR_UNSUPPORTED at run time.  Waits are bounded
                                     (about a second); a wait that gives up leaves its segment
                                     of the row NaN (there is no status word).  Same results bit
                                     for bit as the split plan */
  ROWRED_POLICY_LDS_STRIPE = 256, /* row plans: RMSNorm and softmax, lanes_per_row == threads
                                     == 1024, chunks 5-16: slots 0-3 (from 9 chunks on 0-7)
                                     of each lane stay in registers and the rest are loaded
                                     straight into LDS (16-byte loads that write LDS).  At
                                     5-8 chunks two workgroups then fit a CU, with the
                                     register kernel's arithmetic in the same order (same
                                     bits); at 9-16 chunks rows of up to 16384 granules are
                                     read once.  NT_LOADS / NT_STORES / XCD_REMAP (and for
                                     softmax ONLINE) apply; no other bit may be set.
                                     split plans (with EXCHANGE only): 256 threads, chunks 8
                                     (4 in registers + 4 in LDS), 12 (8 + 4) or 16 (8 + 8),
                                     x (and r) of the LDS slots go
                                     straight into LDS */
  ROWRED_POLICY_FLAT = 512        /* row plans, RMSNorm and softmax, width >= 4: a workgroup of
                                     `threads` (64-512) lanes takes rows_per_group consecutive
                                     rows as one run of 16-byte granules, lane after lane
                                     (chunks 1, 2 or 4 granules per lane), so no lane slot
                                     idles past a row's end; each granule's partial
                                     statistics (its two rows' parts) are folded per row in
                                     LDS, and whole granules are stored.  Derived:
                                     rows_per_group = min(threads, (4 * threads * chunks - 3)
                                     / width), lanes_per_row = the lanes that fold one
                                     row (the largest power of two <= threads / rows_per_group,
                                     at most 64).  NT_LOADS / NT_STORES / XCD_REMAP apply; no
                                     other bit may be set */,
  ROWRED_POLICY_ONLINE = 1024     /* row plans, softmax only, with the register kernels (no
                                     RELOAD, LOOPED or FLAT) or LDS_STRIPE at 5-16 chunks: the
                                     row max and the exponential sum take one workgroup
                                     collective instead of two.  Each lane keeps the max m of
                                     its own elements and the sum of exp(x - m) over them; the
                                     row max M is taken and every sum restated under it
                                     (multiplied by exp(m - M)) before they are added, and
                                     output element x of a lane with max m is exp(x - m) *
                                     (exp(m - M) / S) for the row's M and S.  Same operator,
                                     other rounding (within the softmax tolerance, not bit for
                                     bit equal to the two-collective order); register and LDS
                                     stripes of the same chunks still agree bit for bit */
};

/* Bits 12-15 of a row plan's policy (register kernels only, not FLAT, LOOPED or
 * LDS_STRIPE): n = ROWRED_POLICY_CU_GROUPS_OF(policy), 1-14, caps the
 * workgroups that share a compute unit at n by reserving for each
 * floor(160 KiB / n) of LDS (rounded down to 1 KiB), most of it unused; 0
 * sets no cap (register and LDS use alone decide).  A cap means fewer waves
 * per SIMD.  Speed only; 15 is rejected. */
#define ROWRED_POLICY_CU_GROUPS_SHIFT 12
#define ROWRED_POLICY_CU_GROUPS(n) ((int32_t)(n) << ROWRED_POLICY_CU_GROUPS_SHIFT)
#define ROWRED_POLICY_CU_GROUPS_OF(policy) (((policy) >> ROWRED_POLICY_CU_GROUPS_SHIFT) & 15)

/*
 * Host-only: fill *out with the plan the matching entry point would launch
 * for these arguments (x, r, y are only inspected for their alignment; r may
 * be NULL: for ROWRED_OP_LAYERNORM_RESIDUAL that is the plan of
 * rowred_layernorm without a residual; for ROWRED_OP_ROW_SUM and
 * ROWRED_OP_ROW_MINMAX, y is out / out_min and r is out_max, vectors of
 * `rows` floats).  No device work, callable without a GPU.  Returns the
 * status the entry point would return before launching.  Exchange plans
 * depend on how many workgroups the current device holds at once (a host
 * query of the HIP runtime); without a device the plan is the one the entry
 * point would take where they do not fit.
 */
int rowred_plan_query(int op, const float *x, const float *r, const float *y,
                      int64_t rows, int64_t width, rowred_plan *out);

/*
 * Run one operator with an explicit plan instead of the chooser's (for
 * tuning sweeps and tests of every geometry).  lanes_per_row, chunks,
 * threads and policy are read from *plan; grid, rows_per_group, vector_io and
 * window are derived.  A plan that breaks a constraint listed in rowred_plan, or
 * whose lanes_per_row * chunks does not cover the row window, ->
 * ROWRED_ERR_INVALID_ARG.
 * eps is ignored for softmax.  Same contract as the entry points above.
 */
int rowred_run_plan(int op, const float *x, const float *r, float *y,
                    int64_t rows, int64_t width, float eps,
                    const rowred_plan *plan, hipStream_t stream);

/* Row sum (op ROWRED_OP_ROW_SUM, out1 unused) or row min/max (op
 * ROWRED_OP_ROW_MINMAX, out0 = min, out1 = max) with an explicit plan (as
 * rowred_run_plan; ROWRED_POLICY_STAGE_STORES does not apply). */
int rowred_row_reduce_run_plan(int op, const float *x, float *out0, float *out1,
                               int64_t rows, int64_t width,
                               const rowred_plan *plan, hipStream_t stream);

/* Host-only: the plan rowred_layernorm would launch for these arguments
 * (pointers are only inspected for alignment and overlap; r, gamma, beta may
 * be NULL).  Affine LayerNorm (gamma or beta given) has geometry rules of its
 * own, so rowred_plan_query does not cover it.  Same status as
 * rowred_layernorm would return before launching. */
int rowred_layernorm_plan_query(const float *x, const float *r, const float *gamma, const float *beta,
                                const float *y, int64_t rows, int64_t width, rowred_plan *out);

/* rowred_layernorm with an explicit plan (as rowred_run_plan). */
int rowred_layernorm_run_plan(const float *x, const float *r, const float *gamma,
                              const float *beta, float *y, int64_t rows,
                              int64_t width, float eps, const rowred_plan *plan,
                              hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *rowred_status_string(int status);

/*
 * Measurement aid: y[i] = x[i] for i < n, with the same 16-byte streaming
 * loads and stores as the reductions, to measure the bandwidth a plain copy
 * reaches and to calibrate traffic counters.  x and y must not overlap; both
 * 16-byte aligned, n a multiple of 4, else ROWRED_ERR_INVALID_ARG.
 */
int rowred_copy(const float *x, float *y, int64_t n, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Any width, and rows split across workgroups: the _ws entry points.
 *
 * The entry points above split wide LayerNorm, RMSNorm and softmax rows over
 * workgroups only where the device holds a row's segments twice over and
 * the row takes at most 64 segments of 4096 granules (RMSNorm, softmax:
 * about a million columns; LayerNorm 128, about two million); row sum
 * and min/max rows, and wider rows, get one workgroup each, which walks
 * rows wider than 8192 16-byte granules twice, and a matrix of few such
 * rows keeps few compute units busy.  "Immutable input reuse
 * in Metal reductions" leaves rows beyond the private stripe open (section
 * "Next decisions and open questions": mixed cache/reload choices) and times
 * few-row shapes such as 7x1537 (section "Fixed-width GPU and dispatch
 * results").  The _ws entry points compute the same operators, same
 * arguments, for any width:
 *   - when the row fits the register-resident kernels they run those;
 *   - otherwise each row's window of 16-byte granules is cut into segments
 *     of T*C granules, one workgroup per (row, segment).  LayerNorm, RMSNorm
 *     and softmax rows that take at most 64 segments (up to about a million
 *     columns) run the exchange kernels (ROWRED_POLICY_EXCHANGE): each
 *     workgroup keeps its segment in registers, and the row's workgroups
 *     swap their statistics through the workspace, so x (and r) are read
 *     once;
 *   - other rows wider than the register-resident window, with at least
 *     2048 rows, run the looped kernels (ROWRED_POLICY_LOOPED) -- the
 *     workspace is then not touched;
 *   - the rest run three kernels: per-segment statistics into the
 *     workspace, a fixed-order merge per row, and (LayerNorm, RMSNorm,
 *     softmax) an apply kernel that reads its segment again and writes it.
 *     x (and r) are read twice, the second time from cache where it fits
 *     (the first pass uses cached loads).
 * Merges: LayerNorm combines per-segment (sum, sum of squares about the
 * segment mean) with the pairwise update of Chan, Golub and LeVeque, which is
 * exactly the biased two-pass variance about the row mean of "Residual
 * LayerNorm shared-Tile materialization search", section "Structural
 * finding"; softmax combines (max m_k, sum of exp(x - m_k)) as
 * m = max m_k, s = sum s_k exp(m_k - m); RMSNorm and row sum add, min/max
 * take min and max.  Results agree with the entry points above within the
 * same tolerance (different summation order); for a fixed plan they are
 * bitwise reproducible.  IEEE special cases behave as above (an all -inf
 * softmax row is NaN, a NaN poisons its row, min/max skip NaN).
 *
 * workspace: device memory of at least rowred_workspace_size() bytes,
 * 16-byte aligned, owned by the caller, not overlapping any operand; its
 * contents need no initialisation (the exchange kernels' words are zeroed by
 * a small kernel of their own, enqueued first) and are garbage afterwards.
 * Calls that run concurrently need separate workspaces.  An exchange
 * workgroup waits only for workgroups of its own row, which the hardware
 * dispatches no later than those of later rows, so every wait ends; each is
 * bounded all the same (2^20 polls, a second or so), and one that gives up
 * (not observed) writes NaN to its segment of the row and a nonzero value to
 * the workspace's first 8 bytes (zeroed once per call).  An explicit plan
 * (rowred_split_run_plan) may set a smaller bound, for tests of that path.
 * A row's segments must all be resident on the device at once: when the
 * current device (its compute units times the exchange kernel's occupancy)
 * cannot hold twice a row's segments, the entry points run the three
 * split kernels instead, and an explicit exchange plan gets
 * ROWRED_ERR_UNSUPPORTED.  A NULL,
 * misaligned or short workspace -> ROWRED_ERR_INVALID_ARG when the split
 * kernels are needed;
 * overlap -> ROWRED_ERR_ALIAS.  Everything else as for the entry points
 * above (sizes, alignment, aliasing, eps, stream, no allocation).
 * ------------------------------------------------------------------------ */

/* Workspace bytes enough for the _ws entry point of `op` (enum rowred_op;
 * ROWRED_OP_LAYERNORM_RESIDUAL stands for rowred_layernorm_ws) at any
 * alignment of x: rows * (S + 1) * 16 with S segments per row.  0 when
 * rows or width is 0.  Host only. */
int rowred_workspace_size(int op, int64_t rows, int64_t width, size_t *bytes);

int rowred_layernorm_ws(const float *x, const float *r, const float *gamma, const float *beta, float *y,
                        int64_t rows, int64_t width, float eps, void *workspace, size_t workspace_bytes,
                        hipStream_t stream);
int rowred_rmsnorm_ws(const float *x, float *y, int64_t rows, int64_t width, float eps, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);
int rowred_softmax_ws(const float *x, float *y, int64_t rows, int64_t width, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);
int rowred_row_sum_ws(const float *x, float *out, int64_t rows, int64_t width, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);
int rowred_row_minmax_ws(const float *x, float *out_min, float *out_max, int64_t rows, int64_t width,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Geometry of the split kernels: workgroups of `threads` lanes, each lane
 * holding `chunks` 16-byte slots of its segment, so a segment is
 * threads * chunks granules. */
typedef struct rowred_split_plan {
  int32_t threads;         /* 64, 128, 256, 512 or 1024 */
  int32_t chunks;          /* 1, 2 or 4 (8 with ROWRED_POLICY_EXCHANGE) */
  int32_t policy;          /* ROWRED_POLICY_NT_LOADS / NT_STORES (apply kernel), ROWRED_POLICY_REVERSE */
  int32_t window;          /* derived: largest granule window of a row */
  int64_t block_rows;      /* rows per pass of the kernels (0: all rows in one pass, which the
                              _ws entry points use); passes run one after another on the stream,
                              so a block's second read can find its first in the last-level cache */
  int64_t segments;        /* derived: S = ceil(window / (threads * chunks)) */
  int64_t grid;            /* derived: block_rows * S workgroups per kernel launch */
  int64_t workspace_bytes; /* derived: (block_rows * S + block_rows) * 16 */
  int32_t wait_polls;      /* exchange plans run by rowred_split_run_plan: polls of an empty slot
                              after which a wait gives up (0: the default bound, 2^20 polls).
                              For tests of the give-up path; the _ws entry points always use
                              the default */
  int32_t reserved;        /* 0 */
} rowred_split_plan;

/* Host only.  threads == 0 in *plan: fill in the plan the _ws entry points
 * use when they split; otherwise check the given threads / chunks / policy
 * (ROWRED_ERR_INVALID_ARG if not allowed) and fill the derived fields. */
int rowred_split_plan_query(int op, const float *x, int64_t rows, int64_t width, rowred_split_plan *plan);

/* Run the split kernels with an explicit plan, at any width (for sweeps and
 * tests).  op: enum rowred_op; r, gamma, beta only with
 * ROWRED_OP_LAYERNORM_RESIDUAL (each optional); y2 only with
 * ROWRED_OP_ROW_MINMAX (y = out_min, y2 = out_max); y = out for
 * ROWRED_OP_ROW_SUM. */
int rowred_split_run_plan(int op, const float *x, const float *r, const float *gamma, const float *beta, float *y,
                          float *y2, int64_t rows, int64_t width, float eps, const rowred_split_plan *plan,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory at all -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * _ws entry points with a workspace that the library itself holds, a static
 * device array of ROWRED_STATIC_WORKSPACE_BYTES on each GPU, kept from the
 * first call on that GPU until the process ends.  Nothing is allocated per
 * call.
 *
 * op (enum rowred_op) selects the operator; the arguments are those of
 * rowred_split_run_plan without plan and workspace (r, gamma, beta only with
 * ROWRED_OP_LAYERNORM_RESIDUAL, each optional: rowred_layernorm_ws; y2 only
 * with ROWRED_OP_ROW_MINMAX: y = out_min, y2 = out_max; y = out for
 * ROWRED_OP_ROW_SUM; eps only where the operator has one).  Plans and results
 * are those of the matching _ws entry point (bitwise, for the same device).
 * Call it with the stream's device current: the first call on a device looks
 * up that device's copy of the array.
 *
 * A call whose plan needs more workspace than the array holds (rows * (S + 1)
 * * 16 bytes with S segments per row, see rowred_workspace_size) returns
 * ROWRED_ERR_UNSUPPORTED before anything is enqueued; calls whose rows fit
 * the register-resident or looped kernels use no workspace and have no such
 * limit.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind: calls that may overlap in time on one GPU (several
 * streams, several host threads) race and must be serialised by the caller.
 */
#define ROWRED_STATIC_WORKSPACE_BYTES (8LL << 20)
int rowred_static_ws(int op, const float *x, const float *r, const float *gamma, const float *beta, float *y,
                     float *y2, int64_t rows, int64_t width, float eps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROWRED_H */
