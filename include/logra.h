/*
 * logra.h - C ABI of the LoGRA low-rank gradient-sketching hot path on
 * AMD Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [LoGRA] wispaper.ai research summary of "LoGRA: Scaling LLM
 *           Reinforcement Learning with Low-Rank Gradient Sketches";
 *           sections Sketch (how the sketch replaces the full gradient
 *           buffer), Sync (the same sketch also compresses policy sync),
 *           PKL (predicted-KL control), Rank (projection rank vs. refresh).
 *   [SALMON11] Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3",
 *           SC'11 (Philox4x64-10).
 *
 * Notation: a linear layer computes Y = X W^T with W of shape d x k
 * (d = out features, k = in features).  X (T x k) is the saved layer input
 * and dY (T x d) the gradient of the layer output for one microbatch of T
 * tokens.  G = dY^T X is the d x k weight gradient, A the r x k projection,
 * S = G A^T the d x r sketch.
 *
 * Conventions (every entry point):
 *   - All matrices are row-major.  bf16 values are passed as uint16_t bit
 *     patterns (IEEE-style bfloat16).  "ld" arguments are row strides in
 *     elements; they must be >= the row length and a multiple of 8, and the
 *     base pointer of a bf16 matrix must be 16-byte aligned.
 *   - Buffers are device pointers owned by the caller.  The library never
 *     allocates or frees device memory and keeps no state between calls
 *     (apart from the test-only kernel choice of logra_set_kernel_choice).
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream);
 *     scalar results are written to device memory, so no call synchronises.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call returns a negative status and enqueues nothing.
 *   - NaN / Inf inside the data propagate; they are not errors.
 *   - Calls that share an output buffer (S, W) must be ordered by the caller
 *     (same stream or events).  Two concurrent calls must not share a
 *     workspace.
 */
#ifndef LOGRA_H
#define LOGRA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOGRA_ABI_VERSION 1

/* Status codes. */
#define LOGRA_OK 0
#define LOGRA_EINVAL (-1)     /* invalid argument: null pointer, bad size,
                                 bad stride/alignment, bad kind, bad scalar */
#define LOGRA_EWORKSPACE (-2) /* workspace missing or smaller than required */
#define LOGRA_EHIP (-3)       /* a HIP launch failed (see logra_status_str) */

/* Projection kinds ([LoGRA] Sketch, Rank). */
#define LOGRA_RADEMACHER 0 /* iid signs scaled by 1/sqrt(r) (default basis) */
#define LOGRA_GAUSSIAN 1   /* iid N(0, 1/r), stored as bf16 values */

#define LOGRA_MAX_RANK 256

/* Version of this ABI (LOGRA_ABI_VERSION). */
int logra_abi_version(void);

/* Static text for a status code.  For LOGRA_EHIP it also names the last HIP
 * error seen by this thread.  Never returns NULL. */
const char* logra_status_str(int status);

/*
 * logra_regen_A - materialise the projection A (r x k, fp32, row-major,
 * contiguous) exactly as the sketch and merge kernels regenerate it.
 * [LoGRA] Sketch: A is r x k, independent of the batch, fixed while S
 * accumulates and never learned; its default entries are random signs scaled
 * by 1/sqrt(r).  [LoGRA] Sync: the rollout side rebuilds A from the seed.
 * [LoGRA] Rank: per-step refreshed and Gaussian bases are also studied.
 *
 * Generator: Philox4x64-10 [SALMON11] with key (seed, stream); `stream` is
 * the refresh index (0 for a fixed basis).
 *   Rademacher: counter (j >> 8, i, 0, 0); entry (i, j) takes bit (j & 63) of
 *     output word ((j >> 6) & 3); a set bit gives -c, a clear bit +c, with
 *     c = 1/sqrt(r) computed in double and rounded once to float.
 *   Gaussian: counter (j >> 2, i, 1, 0); each output word w gives the uniform
 *     u = (2 (w >> 41) + 1) 2^-24; Box-Muller on (u0, u1) gives columns 4q and
 *     4q+1 (R cos, R sin with R = sqrt(-2 ln u0), angle 2 pi u1), (u2, u3)
 *     gives 4q+2 and 4q+3; the entry is z / sqrt(r) rounded to bf16 (RNE),
 *     written widened to float.
 *
 * A: device float[r * k].  1 <= r <= 256, k >= 1.  A must be 4-byte aligned.
 * Returns LOGRA_OK, LOGRA_EINVAL or LOGRA_EHIP.
 */
int logra_regen_A(uint64_t seed, uint64_t stream, int kind, int32_t r,
                  int64_t k, float* A, hipStream_t s);

/*
 * logra_set_kernel_choice - force one of two equivalent kernels of the sketch
 * entry points, for tests and measurements (not part of the method).  By
 * default each call picks its kernels from the shapes; results of the
 * alternatives agree to fp32 rounding.
 *
 * which: LOGRA_CHOICE_PROJECT_TILE - the projection tile (only considered
 *            for r > 32); mode 1 forces its 64-token form, mode 2 its
 *            128-token form where r > 64 (the 64-token form below);
 *        LOGRA_CHOICE_ACC_WIDE - the work-group-wide accumulate kernel (only
 *            considered for r > 64).  It changes the workspace size, so it
 *            must not change between logra_sketch_ws_bytes (or
 *            logra_sketch_shared_ws_bytes) and the call that workspace serves.
 * mode:  LOGRA_CHOICE_AUTO (the default), 0 (never) or 1 (always), and 2
 *        for the projection tile as above.
 * The setting is process-wide: it applies to every later sketch call on any
 * thread until it is set again.  This is the library's only state.
 * Returns LOGRA_OK, or LOGRA_EINVAL for an unknown `which` or `mode`.
 */
#define LOGRA_CHOICE_PROJECT_TILE 0
#define LOGRA_CHOICE_ACC_WIDE 1
#define LOGRA_CHOICE_AUTO (-1)
int logra_set_kernel_choice(int which, int mode);

/* Bytes of workspace logra_sketch_accumulate needs for these sizes (either
 * projection kind).  Returns 0 for invalid sizes. */
size_t logra_sketch_ws_bytes(int64_t T, int64_t d, int64_t k, int32_t r);

/* Flags of the sketch entry points. */
#define LOGRA_SKETCH_OVERWRITE 1 /* S = dY^T (X A^T): start the accumulation */
#define LOGRA_SKETCH_DEFER 2     /* keep the contribution in the workspace, S untouched */
#define LOGRA_SKETCH_PENDING 4   /* the workspace holds deferred contributions: add them */

/*
 * logra_sketch_accumulate - S += dY^T (X A^T), one microbatch.
 * [LoGRA] Sketch: each microbatch's contribution to S = G A^T is accumulated
 * in fp32 by projecting the inputs of the weight-gradient product first and
 * then multiplying with the backward derivatives, so the d x k gradient is
 * never formed.  The contribution is added as is (no 1/n scaling; any loss
 * scale is already inside dY).
 *
 * X:  device bf16[T x ldx], row-major, ldx >= k, ldx % 8 == 0, 16-B aligned.
 * dY: device bf16[T x ldd], row-major, ldd >= d, ldd % 8 == 0, ldd < 2^26,
 *     16-B aligned.
 * S:  device float[d x r], contiguous, in/out, 4-B aligned.
 * seed, stream, kind: select A as in logra_regen_A.
 * flags: 0, or LOGRA_SKETCH_OVERWRITE for the first microbatch of an
 *     optimizer step: S = dY^T (X A^T), S's contents on entry are ignored
 *     (they need not be initialised), which spares the caller a zero fill of
 *     S and the kernels a read of it.
 *   Deferred chains (the microbatches of one optimizer step): a call with
 *     LOGRA_SKETCH_DEFER does not touch S; its contribution stays in the
 *     workspace, in the per-split partial sums the kernels keep anyway.  A
 *     later call with LOGRA_SKETCH_PENDING adds its own contribution to
 *     those; the chain ends with a call that has PENDING but not DEFER, which
 *     adds everything to S (or, with OVERWRITE, stores it) and runs the one
 *     split reduction of the chain instead of one per call.  Typical step:
 *     DEFER, DEFER|PENDING, ..., PENDING|OVERWRITE.  Rules: every call of a
 *     chain uses the same ws, T, d, k, r, seed, stream and kind (and kernel
 *     choice), and T >= 1; DEFER with OVERWRITE, or either flag with T == 0,
 *     is LOGRA_EINVAL; a PENDING call after anything but a DEFER call with
 *     the same workspace gives undefined values (never out-of-bounds
 *     accesses).  Other bits: LOGRA_EINVAL.
 * ws: device scratch of at least logra_sketch_ws_bytes(T, d, k, r) bytes,
 *     256-B aligned, owned by the caller; its contents on entry do not
 *     matter (except with LOGRA_SKETCH_PENDING, above).  The result is
 *     deterministic (fixed summation order).
 * T == 0 is a no-op (returns LOGRA_OK; X, dY and ws are not inspected);
 *     with LOGRA_SKETCH_OVERWRITE it sets S to zero.
 * Constraints: d, k >= 1, T >= 0, 1 <= r <= 256, d, k, T < 2^31.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_sketch_accumulate(const uint16_t* X, int64_t ldx, const uint16_t* dY,
                            int64_t ldd, int64_t T, int64_t d, int64_t k,
                            int32_t r, uint64_t seed, uint64_t stream, int kind,
                            int32_t flags, float* S, void* ws, size_t ws_bytes,
                            hipStream_t s);

/* Bytes of library-owned scratch behind logra_sketch_accumulate_noalloc
 * (one copy per GPU, held until the process ends). */
#define LOGRA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * logra_sketch_accumulate_noalloc - logra_sketch_accumulate without a
 * workspace argument and without any device allocation, for callers that
 * cannot allocate: code under stream capture, tight loops that must not call
 * the allocator, harnesses that forbid it.  The scratch the kernels need
 * lives in a device array inside the library, LOGRA_NOALLOC_SCRATCH_BYTES per
 * GPU, whose address is looked up once per device on the first call there.
 * The call itself allocates and frees nothing.
 *
 * Arguments, result and ordering as in logra_sketch_accumulate (same kernels,
 * so the same bits), except that the deferral flags (LOGRA_SKETCH_DEFER,
 * LOGRA_SKETCH_PENDING) are refused with LOGRA_EINVAL: the scratch is shared
 * by every call on the GPU, so nothing may be left pending in it.  The
 * stream's device (the current device for the null stream) selects which
 * GPU's scratch is used.
 * Limit: the call needs logra_sketch_ws_bytes(T, d, k, r) bytes of scratch;
 *     beyond LOGRA_NOALLOC_SCRATCH_BYTES it returns LOGRA_EWORKSPACE and
 *     enqueues nothing (d = k = 4096 at r = 64 needs 10.5 MiB for T = 8192;
 *     the r = 256 layers need more and must use logra_sketch_accumulate).
 * Concurrency: every call on one GPU shares that GPU's scratch, so calls
 *     that may overlap on one GPU (different streams without ordering, or
 *     different threads) race and give wrong results; order them.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_sketch_accumulate_noalloc(const uint16_t* X, int64_t ldx, const uint16_t* dY,
                                    int64_t ldd, int64_t T, int64_t d, int64_t k, int32_t r,
                                    uint64_t seed, uint64_t stream, int kind, int32_t flags,
                                    float* S, hipStream_t s);

/* Largest number of outputs one logra_sketch_accumulate_shared call takes. */
#define LOGRA_MAX_SHARED 4

/* Bytes of workspace logra_sketch_accumulate_shared needs for these sizes
 * (d: host int64[n_out]).  Returns 0 for invalid sizes. */
size_t logra_sketch_shared_ws_bytes(int64_t T, int64_t k, int32_t r, int32_t n_out,
                                    const int64_t* d);

/*
 * logra_sketch_accumulate_shared - S_o += dY_o^T (X A^T) for up to
 * LOGRA_MAX_SHARED outputs o that share the input X and the projection A.
 * [LoGRA] Sketch: the inputs used in the weight-gradient computation are
 * projected before they meet the backward derivatives, so projections of
 * one layer that read the same input (q/k/v, or gate/up) and use the same A
 * (same seed, stream, kind and k) need X A^T only once; each output then
 * streams its own dY.  One projection pass and one accumulate launch over
 * the d groups of every output.  Equal to n_out logra_sketch_accumulate
 * calls up to fp32 summation order.
 *
 * X, ldx, T, k, r, seed, stream, kind, flags: as in logra_sketch_accumulate
 *     (every flag applies to every S[o]; a deferred chain keeps the same
 *     outputs in the same order).
 * dY, ldd, d, S: host arrays of n_out entries (1 <= n_out <= LOGRA_MAX_SHARED);
 *     dY[o] device bf16[T x ldd[o]] (same rules as dY above), S[o] device
 *     float[d[o] x r]; no two S ranges overlap.
 * ws: device scratch of logra_sketch_shared_ws_bytes(T, k, r, n_out, d)
 *     bytes, 256-B aligned.
 * T == 0 is a no-op (X, dY and ws are not inspected); with
 *     LOGRA_SKETCH_OVERWRITE it sets every S[o] to zero.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_sketch_accumulate_shared(const uint16_t* X, int64_t ldx, int64_t T, int64_t k,
                                   int32_t r, uint64_t seed, uint64_t stream, int kind,
                                   int32_t flags, int32_t n_out, const uint16_t* const* dY,
                                   const int64_t* ldd, const int64_t* d, float* const* S,
                                   void* ws, size_t ws_bytes, hipStream_t s);

/* Limits of logra_sketch_accumulate_layer: input groups per call, and
 * outputs per call over all groups. */
#define LOGRA_MAX_GROUPS 4
#define LOGRA_MAX_LAYER_OUT 8

/* One input group of logra_sketch_accumulate_layer: X (device bf16[T x ldx],
 * rules as in logra_sketch_accumulate) with k columns and A from (seed,
 * stream), feeding n_out (1..LOGRA_MAX_SHARED) outputs: dY[o] (device
 * bf16[T x ldd[o]]) with d[o] columns into S[o] (device float[d[o] x r]).
 * Entries past n_out are ignored.  A plain C struct, passed in host memory. */
typedef struct logra_sketch_group {
  const uint16_t* X;
  int64_t ldx;
  int64_t k;
  uint64_t seed;
  uint64_t stream;
  int32_t n_out;
  const uint16_t* dY[LOGRA_MAX_SHARED];
  int64_t ldd[LOGRA_MAX_SHARED];
  int64_t d[LOGRA_MAX_SHARED];
  float* S[LOGRA_MAX_SHARED];
} logra_sketch_group;

/* Bytes of workspace logra_sketch_accumulate_layer needs (only k, n_out and
 * d of the groups are read).  Returns 0 for invalid sizes. */
size_t logra_sketch_layer_ws_bytes(int64_t T, int32_t r, int32_t n_groups,
                                   const logra_sketch_group* groups);

/*
 * logra_sketch_accumulate_layer - the sketches of a whole layer set for one
 * microbatch: S_o += dY_o^T (X_g A_g^T) for every output o of every input
 * group g, in one projection launch (every group's token blocks, largest k
 * first) and one accumulate launch (every output's column groups), plus one
 * split reduction at the end of a call or chain.
 * [LoGRA] Sketch (wispaper.ai summary): each weight's sketch is accumulated
 * input-first per microbatch; the cloud.baidu.com evaluation guide, section
 * on the evaluated objects (first bullet), sketches selected attention and
 * MLP projections of each decoder layer: q/k/v (one input), o, gate/up (one
 * input) and down are four input groups with seven outputs.  Equal, output by
 * output, to logra_sketch_accumulate_shared per group up to fp32 summation
 * order.
 *
 * T, r, kind, flags: as in logra_sketch_accumulate; T is every group's token
 *     count, and every flag applies to every output (a deferred chain keeps
 *     the same groups and outputs in the same order).
 * groups: host array of n_groups (1..LOGRA_MAX_GROUPS) entries with
 *     LOGRA_MAX_LAYER_OUT outputs at most in all; no two S ranges overlap.
 * ws: device scratch of logra_sketch_layer_ws_bytes(T, r, n_groups, groups)
 *     bytes, 256-B aligned (each group's projected input, the partial sums).
 * T == 0 is a no-op (no X, dY or ws inspected); with LOGRA_SKETCH_OVERWRITE
 *     it sets every S to zero.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_sketch_accumulate_layer(int64_t T, int32_t r, int kind, int32_t flags,
                                  int32_t n_groups, const logra_sketch_group* groups, void* ws,
                                  size_t ws_bytes, hipStream_t s);

/*
 * The sketch in two calls: logra_sketch_project computes the projected input
 * P = X A^T into a buffer of the caller's, and logra_sketch_accumulate_p adds
 * dY^T P to S.  [LoGRA] Sketch: the inputs are projected before they meet
 * the backward derivatives; the projection needs only X (available from the
 * forward pass) and the accumulation only P and dY, so the two halves can
 * run at different times or on different streams: the projection of the
 * next microbatch may overlap the accumulation of this one.  Run back to
 * back on one stream with the same T, k, r, seed, stream, kind and outputs,
 * the pair launches the kernels of logra_sketch_accumulate (or
 * logra_sketch_accumulate_shared) on the same tiling, and S receives the same
 * bits.
 *
 * P layout (bf16, logra_sketch_p_bytes(T, r) bytes): with rp = r rounded up
 * to 16, 32, 64, 128 or 256 and steps = ceil(max(T, 1) / 32), P holds steps
 * x (rp / 16) x 2 blocks of 512 bf16 values, block (step, b, h) at element
 * offset ((step (rp / 16) + b) 2 + h) 512.  Element 8 (16 g + n) + e of a
 * block is token 32 step + 8 g + e (g < 4, e < 8) and column 16 b + n
 * (n < 16) of p = c X A^T, split as p = hi + lo with hi = RNE_bf16(p) in the
 * block with h = 0 and lo = RNE_bf16(p - hi) in h = 1; c = 1 / sqrt(r) for
 * signs and 1 for the Gaussian basis (whose entries already carry it).
 * Tokens past T hold zeros; columns r .. rp - 1 hold values that the
 * accumulation ignores.
 */

/* Bytes of P for T tokens at rank r.  Returns 0 for invalid sizes. */
size_t logra_sketch_p_bytes(int64_t T, int32_t r);

/* Bytes of scratch logra_sketch_project needs for the Gaussian basis (the
 * bf16 basis written once per call); the sign basis needs none.  Returns 0
 * for invalid sizes. */
size_t logra_sketch_project_ws_bytes(int64_t k, int32_t r);

/*
 * logra_sketch_project - P = X A^T for one microbatch, in the layout above.
 * X, ldx, T, k, r, seed, stream, kind: as in logra_sketch_accumulate.
 * P: device bf16 buffer of p_bytes >= logra_sketch_p_bytes(T, r) bytes,
 *     16-B aligned, written (its contents on entry do not matter).
 * ws: for kind == LOGRA_GAUSSIAN, device scratch of
 *     logra_sketch_project_ws_bytes(k, r) bytes, 256-B aligned, owned by
 *     the caller; for signs it is not used (may be NULL).
 * T == 0 is a no-op (returns LOGRA_OK; X, P and ws are not inspected).
 * X, P and ws must not overlap.
 * Returns LOGRA_OK, LOGRA_EINVAL (also for a P smaller than required),
 * LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_sketch_project(const uint16_t* X, int64_t ldx, int64_t T, int64_t k, int32_t r,
                         uint64_t seed, uint64_t stream, int kind, uint16_t* P, size_t p_bytes,
                         void* ws, size_t ws_bytes, hipStream_t s);

/* Bytes of workspace logra_sketch_accumulate_p needs (the per-split partial
 * sums; d: host int64[n_out]).  Returns 0 for invalid sizes. */
size_t logra_sketch_accumulate_p_ws_bytes(int64_t T, int32_t r, int32_t n_out, const int64_t* d);

/*
 * logra_sketch_accumulate_p - S_o += dY_o^T P for up to LOGRA_MAX_SHARED
 * outputs o, with P made by logra_sketch_project for the same T and r.
 * P, p_bytes: as written by logra_sketch_project (p_bytes >=
 *     logra_sketch_p_bytes(T, r), 16-B aligned); read only.
 * T, r, flags, n_out, dY, ldd, d, S: as in logra_sketch_accumulate_shared,
 *     including the deferred chains (every call of a chain uses the same
 *     ws, T, r and outputs; P may differ from call to call, which is how a
 *     chain covers the microbatches of a step).
 * ws: device scratch of logra_sketch_accumulate_p_ws_bytes(T, r, n_out, d)
 *     bytes, 256-B aligned, owned by the caller (same kernel-choice rule as
 *     logra_sketch_ws_bytes).
 * T == 0 is a no-op (P, dY and ws are not inspected); with
 *     LOGRA_SKETCH_OVERWRITE it sets every S[o] to zero.
 * P, dY, S and ws must not overlap.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_sketch_accumulate_p(const uint16_t* P, size_t p_bytes, int64_t T, int32_t r,
                              int32_t flags, int32_t n_out, const uint16_t* const* dY,
                              const int64_t* ldd, const int64_t* d, float* const* S, void* ws,
                              size_t ws_bytes, hipStream_t s);

/*
 * logra_merge - W <- RNE_bf16(W - alpha * eta * S A), in place.
 * [LoGRA] Sketch: the update is W <- W - alpha eta U A with U = S in the basic
 * SGD variant, merged directly into the weights (no adapter branch).
 * [LoGRA] Sync: the rollout engine applies the same merge to the received
 * alpha*eta*U after rebuilding A from the seed (pass alpha*eta*U as S with
 * alpha = eta = 1).
 *
 * The product S A is accumulated in fp32, scaled by (float)alpha *
 * (float)eta (and by c for the sign basis) and subtracted from the fp32 value
 * of W; the result is rounded once to bf16, ties to even.
 *
 * W: device bf16[d x ldw], in/out, ldw >= k, ldw % 8 == 0, 16-B aligned.
 * S: device float[d x r], contiguous, 4-B aligned (read only).
 * alpha, eta: finite.  Constraints as for logra_sketch_accumulate.
 * Returns LOGRA_OK, LOGRA_EINVAL or LOGRA_EHIP.
 */
int logra_merge(uint16_t* W, int64_t ldw, const float* S, int64_t d, int64_t k,
                int32_t r, uint64_t seed, uint64_t stream, int kind,
                float alpha, float eta, hipStream_t s);

/* Largest number of weights one logra_merge_many call takes. */
#define LOGRA_MAX_MERGE 8

/* One weight of logra_merge_many: W (device bf16[d x ldw]) and its sketch S
 * (device float[d x r]), A from (seed, stream); rules as in logra_merge. */
typedef struct logra_merge_item {
  uint16_t* W;
  int64_t ldw;
  const float* S;
  int64_t d;
  int64_t k;
  uint64_t seed;
  uint64_t stream;
} logra_merge_item;

/*
 * logra_merge_many - logra_merge for n (1..LOGRA_MAX_MERGE) weights that
 * share r, kind, alpha and eta (the weights of one layer set), in one launch.
 * [LoGRA] Sketch: every sketched weight takes W <- W - alpha eta U A after the
 * step; the step size alpha comes from the one predicted-KL controller.
 * Bit-identical, weight by weight, to n logra_merge calls (the same tiles
 * and arithmetic; only the launch is shared).
 *
 * items: host array of n entries.  No W's rows may overlap another W's or
 *     any S (W is written in place while every S is read).
 * Returns LOGRA_OK, LOGRA_EINVAL or LOGRA_EHIP.
 */
int logra_merge_many(int32_t n, const logra_merge_item* items, int32_t r, int kind,
                     float alpha, float eta, hipStream_t s);

/* Sketch-space update rules for logra_sketch_update. */
#define LOGRA_UPDATE_SGD 0      /* U = S */
#define LOGRA_UPDATE_MOMENTUM 1 /* m <- beta1 m + S; U = m */
#define LOGRA_UPDATE_ADAM 2     /* Adam on the sketch (see below) */

/*
 * logra_sketch_update - the update factor U from the sketch S and the state
 * of a sketch-space optimizer, entrywise over d x r.
 * [LoGRA] Sketch: the update is W <- W - alpha eta U A, with U = S in the
 * basic SGD variant; stateful sketch optimizers keep state of their own
 * (the pages do not define one).  The stateful rules are the textbook ones on
 * the d x r sketch instead of the d x k gradient:
 *   LOGRA_UPDATE_SGD       U = S
 *   LOGRA_UPDATE_MOMENTUM  m <- beta1 m + S;  U = m          (heavy ball)
 *   LOGRA_UPDATE_ADAM      m <- beta1 m + (1 - beta1) S
 *                          v <- beta2 v + (1 - beta2) S^2
 *                          U = (m / b1) / (sqrt(v / b2) + eps)
 *                          b1 = 1 - beta1^step, b2 = 1 - beta2^step
 *                          (Kingma & Ba, ICLR 2015, Algorithm 1)
 * U then goes to logra_merge in place of S (and to the rollout payload).
 * Arithmetic is fp32 per entry; b1, b2 are formed in double on the host and
 * rounded to float.  With eps = 0 an entry whose m and v are both 0 gives NaN.
 *
 * S: device float[d x r] (read only).  m, v: device float[d x r] state,
 *     in/out (m for MOMENTUM and ADAM, v for ADAM; otherwise ignored and may
 *     be NULL); start them at zero.  U: device float[d x r], written.
 * U may be S itself, and for MOMENTUM also m itself; no other pair of the
 * arrays may overlap.  All arrays contiguous and 4-byte aligned.
 * beta1, beta2 in [0, 1); eps >= 0 and finite; step >= 1 (ADAM: the 1-based
 * step number).  d >= 1, 1 <= r <= LOGRA_MAX_RANK.
 * Returns LOGRA_OK, LOGRA_EINVAL or LOGRA_EHIP.
 */
int logra_sketch_update(int rule, const float* S, float* m, float* v, float* U,
                        int64_t d, int32_t r, float beta1, float beta2, float eps,
                        int64_t step, hipStream_t s);

/* Bytes of workspace logra_predicted_kl needs when kl_tok is NULL (0 when
 * kl_tok is given).  Returns 0 for invalid sizes. */
size_t logra_kl_ws_bytes(int64_t n_tok, int64_t vocab);

/*
 * logra_predicted_kl - q(D) and the step size alpha.
 * [LoGRA] PKL: on a small sample of responses, the current and the proposed
 * model's vocabulary distributions are compared at one common temperature;
 * the mean predicted KL scales as alpha^2 q(D); for a KL budget delta the
 * controller sets alpha = min(alpha_max, sqrt(delta / q(D))).
 *
 * Computed: for every row t (a sampled token position),
 *   KL_t = KL(softmax(z_cur[t] / tau) || softmax(z_prop[t] / tau))
 * (forward KL, z_prop = logits after the alpha = 1 proposal), in one pass
 * over both rows; q = mean_t KL_t (equal weight per row);
 * alpha = min(alpha_max, sqrt(kl_budget / q)); q <= 0 gives alpha_max; a NaN
 * q gives a NaN alpha; q = +inf gives alpha = 0.
 * Masked tokens: a logit of -inf is a token of probability zero.  One with
 * z_cur = -inf adds nothing to KL_t (its proposed mass, if any, still enters
 * the proposal's normaliser); one with finite z_cur and z_prop = -inf
 * (p > 0, p' = 0) makes KL_t = +inf.  A row with no finite z_cur, and NaN or
 * +inf logits, give a NaN KL_t.  Rows with a -inf logit take a second pass
 * over their data, and so do rows whose one-pass result would be a small
 * difference of large terms (a proposal offset that the row's first 64
 * tokens do not carry): that pass is centred on the p-weighted mean of
 * z_prop - z_cur.
 *
 * z_cur, z_prop: device bf16[n_tok x ld], ld >= vocab, ld % 8 == 0, 16-B
 *     aligned.
 * q_alpha_out: device float[2] <- {q, alpha}.
 * kl_tok: device float[n_tok] <- KL_t, or NULL.
 * ws: device scratch of logra_kl_ws_bytes(n_tok, vocab) bytes (256-B
 *     aligned) when kl_tok is NULL; ignored otherwise.
 * tau > 0, kl_budget > 0, alpha_max >= 0, all finite; n_tok, vocab >= 1.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_predicted_kl(const uint16_t* z_cur, const uint16_t* z_prop,
                       int64_t n_tok, int64_t vocab, int64_t ld, float tau,
                       float kl_budget, float alpha_max, float* q_alpha_out,
                       float* kl_tok, void* ws, size_t ws_bytes, hipStream_t s);

/* Largest number of step multipliers one logra_predicted_kl_sweep call takes. */
#define LOGRA_MAX_SWEEP 8

/* Bytes of workspace logra_predicted_kl_sweep needs when kl_tok is NULL (0
 * when kl_tok is given).  Returns 0 for invalid sizes. */
size_t logra_kl_sweep_ws_bytes(int64_t n_tok, int32_t n_alpha);

/*
 * logra_predicted_kl_sweep - the predicted KL at several step multipliers,
 * in one pass over the current logits and the update direction.
 * [LoGRA] PKL: the current and the proposed model's vocabulary distributions
 * are compared at one common temperature, and the mean predicted KL grows as
 * alpha^2 q(D).  Here the proposal at multiplier alpha_i is z + alpha_i delta,
 * formed in fp32 and never rounded to bf16, so the alpha^2 law holds on the
 * inputs as given.
 *
 * Computed: for every row t and multiplier i,
 *   KL_t(alpha_i) = KL(softmax(z[t] / tau) || softmax((z[t] + alpha_i delta[t]) / tau))
 * (forward KL), and kl_mean[i] = sum_t w_t KL_t(alpha_i) / sum_t w_t in fp64
 * (w_t = weight[t], or 1 when weight is NULL; a token mask or per-response
 * averaging is a choice of weights; a row of weight zero is left out whatever
 * its KL_t, e.g. a padded position with every logit -inf; a zero weight sum
 * gives NaN).
 * Masked tokens: a current logit of -inf is a token of probability zero and
 * stays masked in every proposal, whatever its delta entry (NaN and inf
 * included); a row with no finite z gives NaN, and so do NaN or +inf logits.
 * A non-finite delta at an unmasked token is not specified (NaN or +-inf).
 * Rows with a -inf logit take a second pass over their data, and so do rows
 * whose one-pass result would be a small difference of large terms (a
 * direction offset that the row's first 64 tokens do not carry): that pass
 * is centred on the p-weighted mean of delta.
 * Per element the cost does not depend on n_alpha: the multipliers enter
 * through weighted moments of delta (see kl_sweep.hip); the relative
 * truncation of that expansion is below 1.1e-5.
 *
 * z, delta: device bf16[n_tok x ld], ld >= vocab, ld % 8 == 0, 16-B aligned.
 * alphas: host float[n_alpha], 1 <= n_alpha <= LOGRA_MAX_SWEEP, finite.
 * weight: device float[n_tok] (>= 0), 4-B aligned, or NULL.
 * kl_mean: device float[n_alpha] <- the weighted means.
 * kl_tok: device float[n_alpha x n_tok] (multiplier-major) <- KL_t(alpha_i),
 *     or NULL.
 * ws: device scratch of logra_kl_sweep_ws_bytes(n_tok, n_alpha) bytes (256-B
 *     aligned) when kl_tok is NULL; ignored otherwise.
 * tau > 0 and finite; n_tok, vocab >= 1.
 * Returns LOGRA_OK, LOGRA_EINVAL, LOGRA_EWORKSPACE or LOGRA_EHIP.
 */
int logra_predicted_kl_sweep(const uint16_t* z, const uint16_t* delta, int64_t n_tok,
                             int64_t vocab, int64_t ld, const float* alphas,
                             int32_t n_alpha, float tau, const float* weight,
                             float* kl_mean, float* kl_tok, void* ws, size_t ws_bytes,
                             hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* LOGRA_H */
