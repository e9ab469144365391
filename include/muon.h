/*
 * muon.h - C ABI of libmuon.so, the MI355X (gfx950) hot path of the Muon
 * optimizer: Nesterov momentum followed by quintic Newton-Schulz
 * orthogonalisation (NS5) iterated in bfloat16.
 *
 * Source of the method: Synced (机器之心) report on Modded-NanoGPT, section
 * "Muon optimizer" - the printed function zeroth_power_via_newtonschulz5 and
 * the summary paragraph that follows it (Nesterov momentum, orthogonalise
 * after momentum, run the iteration in bfloat16).
 *
 * Conventions for every entry point
 *  - Matrices are dense, row-major and contiguous (leading dimension = cols),
 *    in device memory.  The caller owns every buffer, including the
 *    workspace; the library allocates no device memory and keeps no data
 *    between calls (muon_momentum_ns5_batched_static alone uses a device
 *    array the library holds as its workspace).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is ordered on it and the call returns without synchronising.  A
 *    batched call over a large single-group batch (at least 5e11 nominal
 *    NS5 flops and 2 matrices per part) runs as 2 or 3 parts, every part but
 *    the first on a side stream the library creates once per device (default
 *    priority, not synchronising with the null stream), forked from and
 *    joined back into `stream` with events, so the work still begins after
 *    everything enqueued on `stream` before the call and ends before
 *    anything enqueued after it; this holds under graph capture too.
 *    Results do not depend on the split.  Batched calls enqueue under a
 *    process-wide lock.
 *  - Matrices whose short side is at most 64 and long side at most 256 run
 *    their whole step in one launch (one workgroup per matrix) in every
 *    entry point; the workspace sizes keep their share, unused.
 *  - Arguments are validated before anything is enqueued; a validation error
 *    returns a non-zero status and enqueues nothing.  A HIP launch error is
 *    reported as MUON_ERR_HIP; faults during execution surface at the
 *    caller's next synchronisation.
 *  - muon_last_error() returns a per-thread message describing the most
 *    recent non-zero status.
 *  - Calls that share a workspace must not overlap in time (enqueue them on
 *    one stream, or give each stream its own workspace).
 *  - NaN and Inf inputs are not checked; they propagate to the outputs.
 */
#ifndef MUON_H
#define MUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
    MUON_OK = 0,
    MUON_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, bad count  */
    MUON_ERR_UNSUPPORTED = 2,  /* a size beyond the documented limits         */
    MUON_ERR_WORKSPACE = 3,    /* workspace null or smaller than required     */
    MUON_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed  */
} muon_status;

/* Element type of G and out in muon_ns5 / muon_ns5_grouped: float32, or
 * bfloat16 (uint16_t bit patterns).  The iteration is bf16 either way. */
typedef enum muon_dtype {
    MUON_F32 = 0,
    MUON_BF16 = 1
} muon_dtype;

/* Quintic coefficients of p(x) = a x + b x^3 + c x^5 (the printed listing);
 * the kernels use their float32 values. */
#define MUON_NS5_A 3.4445f
#define MUON_NS5_B (-4.7750f)
#define MUON_NS5_C 2.0315f
#define MUON_NS5_DEFAULT_STEPS 5
#define MUON_NS5_DEFAULT_EPS 1e-7f

/* Largest number of matrices one launch covers; larger groups and batches
 * are processed in passes of at most this many, reusing the workspace. */
#define MUON_NS5_MAX_GROUP 128
/* Matrices per launch of muon_momentum_nesterov_grouped. */
#define MUON_NESTEROV_MAX_GROUP 64
/* Largest supported min(rows, cols) and max(rows, cols). */
#define MUON_NS5_MAX_SHORT 16384
#define MUON_NS5_MAX_LONG (1 << 20)

/*
 * Nesterov momentum, one step (summary paragraph of the Muon section, which
 * names Nesterov momentum as the first stage of the update but whose formula
 * did not survive in the page; the plain SGD-Nesterov form without dampening
 * is used):
 *     buf[i] <- mu * buf[i] + g[i]
 *     u[i]   <- g[i] + mu * buf[i]          (new buf)
 * each computed as one float32 fused multiply-add (one rounding).
 *  g    : [numel] float32, read.
 *  buf  : [numel] float32, read and overwritten in place (the optimizer state).
 *  u    : [numel] float32, written; may alias g (in-place update of the
 *         gradient), must not alias buf.
 *  numel: >= 0; 0 enqueues nothing and returns MUON_OK.
 * Errors: MUON_ERR_INVALID_ARG for a null pointer with numel > 0 or
 * numel < 0, or u == buf.
 */
int muon_momentum_nesterov(const float* g, float* buf, float* u, int64_t numel, float mu,
                           void* stream);

/*
 * Nesterov momentum over a list of matrices (or any float32 arrays) in one
 * launch per MUON_NESTEROV_MAX_GROUP of them: for each i, the update of
 * muon_momentum_nesterov on g[i], buf[i], u[i] with numel[i] elements.
 *  g, buf, u : host arrays of `count` device pointers (float32); u[i] may
 *          alias g[i], must not alias buf[i]; distinct i must not overlap.
 *  numel  : host array of `count` element counts, each >= 0 (0: skipped,
 *          its pointers may be null).
 *  count  : >= 0; 0 enqueues nothing and returns MUON_OK.
 * Asynchronous on `stream`; the caller owns every buffer.
 * Errors: MUON_ERR_INVALID_ARG for count < 0, a null array, a negative
 * numel[i], a null pointer of a non-empty entry, or u[i] == buf[i]; nothing
 * is enqueued then.
 */
int muon_momentum_nesterov_grouped(const float* const* g, float* const* buf, float* const* u, const int64_t* numel,
                                   int64_t count, float mu, void* stream);

/*
 * Bytes of workspace muon_ns5 / muon_ns5_grouped need for `count` matrices of
 * rows x cols (larger groups than MUON_NS5_MAX_GROUP reuse one pass's
 * workspace, so the size stops growing there).  Returns 0 for invalid sizes.  The workspace
 * must be device memory aligned to 256 bytes; its contents on entry do not
 * matter.
 */
size_t muon_ns5_workspace_size(int64_t rows, int64_t cols, int64_t count);

/*
 * NS5 of one matrix (the printed zeroth_power_via_newtonschulz5):
 *     X = bf16( bf16(G) / (||G||_F + eps) )         norm of the input
 *     if rows > cols: X = X^T                        iterate on the short side
 *     repeat `steps` times:
 *         A = bf16( X X^T )                          bf16 MFMA, fp32 accumulate
 *         B = bf16( b A + c A A )
 *         X = bf16( a X + B X )
 *     out = (G's type)( rows > cols ? X^T : X )
 * with (a, b, c) = (MUON_NS5_A, MUON_NS5_B, MUON_NS5_C).
 *  G    : [rows x cols] of `dtype`, read only.
 *  out  : [rows x cols] of `dtype`, written; may alias G.  float32: every
 *         value is bf16-representable; bfloat16: the last iterate as is (the
 *         same values).  For bfloat16 G the first cast is exact, and the norm
 *         is that of the bf16 values.
 *  rows, cols : >= 1, min <= MUON_NS5_MAX_SHORT, max <= MUON_NS5_MAX_LONG.
 *  dtype: MUON_F32 or MUON_BF16.
 *  steps: >= 0 (0 returns the normalised, bf16-rounded input).
 *  eps  : > 0 is typical; any finite value is accepted.
 *  workspace, workspace_bytes: >= muon_ns5_workspace_size(rows, cols, 1)
 *         (the same for either dtype).
 * Errors: MUON_ERR_INVALID_ARG (null pointer, rows/cols < 1, an unknown
 * dtype, steps < 0, eps not finite), MUON_ERR_UNSUPPORTED (sizes beyond the
 * limits), MUON_ERR_WORKSPACE (workspace null, misaligned or too small).
 */
int muon_ns5(const void* G, void* out, int64_t rows, int64_t cols, muon_dtype dtype, int steps, float eps,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * NS5 of `count` independent matrices of the same shape and type, batched so
 * that each kernel launch covers every matrix of a pass (up to
 * MUON_NS5_MAX_GROUP).
 *  G, out : host arrays of `count` device pointers to `dtype` matrices;
 *           out[i] may alias G[i]; distinct i must not overlap.
 *  count  : >= 1.
 *  Everything else as in muon_ns5, with workspace_bytes >=
 *  muon_ns5_workspace_size(rows, cols, count).
 * Errors: as muon_ns5, plus MUON_ERR_INVALID_ARG for count < 1 or a null
 * entry in G or out.
 */
int muon_ns5_grouped(const void* const* G, void* const* out, int64_t count, int64_t rows, int64_t cols,
                     muon_dtype dtype, int steps, float eps, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Bytes of workspace muon_ns5_batched needs for `count` matrices of shapes
 * rows[i] x cols[i].  Returns 0 for invalid sizes (a null array, count < 1,
 * a dimension < 1 or beyond the limits).  Same alignment rule as above.
 */
size_t muon_ns5_batched_workspace_size(const int64_t* rows, const int64_t* cols, int64_t count);

/*
 * NS5 of `count` independent matrices of arbitrary shapes, each exactly as
 * muon_ns5 computes it.  Matrices of equal shape are batched together, and
 * every product of every NS5 step is one launch over all matrices whose
 * short side takes the same tile size (up to MUON_NS5_MAX_GROUP matrices and
 * 8 distinct shapes per launch; beyond that the batch runs in passes that
 * reuse the workspace).  Use this for a whole optimizer step: the launches
 * are few and large instead of many and small.
 *  G, out     : host arrays of `count` device pointers (float32, row-major
 *               rows[i] x cols[i]); out[i] may alias G[i]; distinct i must not
 *               overlap.
 *  rows, cols : host arrays of `count` sizes, each >= 1 and within the
 *               limits of muon_ns5.
 *  count      : >= 1.
 *  steps, eps, stream : as in muon_ns5.
 *  workspace, workspace_bytes: >= muon_ns5_batched_workspace_size(rows, cols,
 *               count).
 * Errors: as muon_ns5_grouped, per matrix.
 */
int muon_ns5_batched(const float* const* G, float* const* out, const int64_t* rows, const int64_t* cols,
                     int64_t count, int steps, float eps, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * The batched iteration of muon_ns5_batched with caller-chosen coefficients:
 * each of the `steps` steps is X <- a X + (b A + c A A) X with A = X X^T, in
 * the same precision, rounding points and layout as NS5.  The Muon section of
 * the Synced report on Modded-NanoGPT explains its quintic as coefficients
 * picked for the steepest slope at zero, at the price of converging to a band
 * around 1 rather than to 1; this entry point also runs the alternatives that
 * contrast implies, such as the classic cubic Newton-Schulz iteration
 * (a, b, c) = (1.5, -0.5, 0), whose singular values converge to 1.
 *  coeffs : host array of 3 floats (a, b, c), each finite.
 *  Everything else as muon_ns5_batched (same workspace requirement);
 *  coefficients (MUON_NS5_A, MUON_NS5_B, MUON_NS5_C) give exactly
 *  muon_ns5_batched's result.
 * Errors: as muon_ns5_batched, plus MUON_ERR_INVALID_ARG for a null or
 * non-finite coefficient.
 */
int muon_newton_schulz_batched(const float* const* G, float* const* out, const int64_t* rows, const int64_t* cols,
                               int64_t count, int steps, const float* coeffs, float eps, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Workspace bytes for muon_newton_schulz_f32_batched on these shapes (0 if a
 * shape is invalid or beyond MUON_NS5_MAX_SHORT / MUON_NS5_MAX_LONG).
 */
size_t muon_newton_schulz_f32_workspace_size(const int64_t* rows, const int64_t* cols, int64_t count);

/*
 * The iteration carried in float32 instead of bfloat16: the contrast the
 * summary paragraph of the Muon section (Synced report on Modded-NanoGPT)
 * draws when it notes that the Newton-Schulz iteration stays stable in bf16,
 * unlike methods that need float32.  The steps of the printed
 * zeroth_power_via_newtonschulz5 with float32 in place of bf16: no bf16 cast
 * of the input, X0 = G / (||G||_F + eps) rounded once to float32 (the quotient
 * formed in float64), transposed when rows > cols; then `steps` times
 * A = X X^T, B = b A + c A A, X = a X + B X, each stored matrix rounded once
 * to float32 (float32 MFMA products with float32 accumulation); the result in
 * G's orientation.  For comparison with the bf16 path: about 16 times the
 * MFMA time per flop (float32 dense peak 157.3 TFLOP/s against 2.5 PFLOP/s).
 *  G, out, rows, cols, count, steps, eps : as muon_ns5_batched (float32,
 *          device pointers, host arrays; out may alias G).
 *  coeffs : host array of 3 finite floats (a, b, c), or NULL for NS5's
 *          (MUON_NS5_A, MUON_NS5_B, MUON_NS5_C).
 *  workspace : device memory of at least
 *          muon_newton_schulz_f32_workspace_size(rows, cols, count) bytes,
 *          256-byte aligned, owned by the caller; contents on entry are
 *          ignored and on return undefined.  Same-shaped matrices run in
 *          passes of up to MUON_NS5_MAX_GROUP, one launch per product and
 *          step; shapes run one after another.
 * Errors: as muon_ns5_batched, plus MUON_ERR_INVALID_ARG for a non-finite
 * coefficient.
 */
int muon_newton_schulz_f32_batched(const float* const* G, float* const* out, const int64_t* rows,
                                   const int64_t* cols, int64_t count, int steps, const float* coeffs, float eps,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * NS5 of bfloat16 matrices, returning bfloat16 (as muon_ns5_batched, whose
 * inputs and outputs are float32).  The printed listing of the Muon section
 * (Synced report on Modded-NanoGPT) casts G to bfloat16 before the iteration
 * and returns the result in G's dtype, so for a bfloat16 G the cast is exact
 * and the output is the last iterate X itself, transposed back for a tall G,
 * with no further rounding.  The norm is taken over G's bfloat16 values in
 * float64, as for float32 inputs.
 *  G, out : host arrays of `count` device pointers to bfloat16 bit patterns,
 *           row-major rows[i] x cols[i]; out[i] may alias G[i]; distinct i
 *           must not overlap.
 *  Everything else as muon_ns5_batched (same workspace requirement).
 * Errors: as muon_ns5_batched.
 */
int muon_ns5_batched_bf16(const uint16_t* const* G, uint16_t* const* out, const int64_t* rows, const int64_t* cols,
                          int64_t count, int steps, float eps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One whole Muon step over a batch: Nesterov momentum (as
 * muon_momentum_nesterov, per matrix) followed by NS5 of the momentum
 * output u (as muon_ns5_batched), with the first pass of the norm fused into
 * the momentum pass.  u is never stored in float32: the fused pass writes the
 * new buffer, bf16(u) into the workspace and the norm's partial sums, so the
 * step reads g and buf once.  The result equals momentum followed by NS5 up
 * to the summation order of the float64 norm.
 *  g    : host array of `count` device pointers, float32 rows[i] x cols[i]
 *         gradients, read only.
 *  buf  : host array of `count` device pointers, the float32 momentum
 *         buffers (same shapes), read and overwritten with mu*buf + g.
 *  out  : host array of `count` device pointers, float32 orthogonalised
 *         updates; out[i] may alias g[i], must not alias buf[i].
 *  mu   : momentum coefficient.
 *  Everything else as muon_ns5_batched; the workspace requirement is
 *  muon_ns5_batched_workspace_size(rows, cols, count).
 * Errors: as muon_ns5_batched, plus MUON_ERR_INVALID_ARG for a null buf
 * array or entry, or out[i] == buf[i].
 */
int muon_momentum_ns5_batched(const float* const* g, float* const* buf, float* const* out, const int64_t* rows,
                              const int64_t* cols, int64_t count, float mu, int steps, float eps, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The Muon step with its parameter update: as muon_momentum_ns5_batched, then
 * p <- p - lr * O with the orthogonalised O, applied in the epilogue of the
 * last iteration step, so O itself is never stored.  The Muon section of the
 * Synced report on Modded-NanoGPT orders the step as momentum,
 * orthogonalisation, update; its update formula did not survive, and this is
 * the plain reading: a learning rate and no other scaling, with one float32
 * rounding (fused multiply-add).  A momentum warmup, which the page lists
 * among the speedrun's techniques, is a schedule of mu over calls.
 *  p    : host array of `count` device pointers, the float32 parameters
 *         (rows[i] x cols[i]), read and overwritten; p[i] must not alias g[i]
 *         or buf[i].
 *  lr   : learning rate, finite.
 *  Everything else as muon_momentum_ns5_batched (same workspace
 *  requirement).
 * Errors: as muon_momentum_ns5_batched (with p in place of out), plus
 * MUON_ERR_INVALID_ARG for a null p array, p[i] == g[i] or a non-finite lr.
 */
int muon_momentum_ns5_apply_batched(const float* const* g, float* const* buf, float* const* p, const int64_t* rows,
                                    const int64_t* cols, int64_t count, float mu, float lr, int steps, float eps,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement support: muon_ns5_batched (buf == NULL) or
 * muon_momentum_ns5_batched (buf != NULL, with coefficient mu), which in
 * addition records caller-created hipEvent_t pairs on `stream` around the
 * launches of the a X + B X product of the non-final steps (the dominant
 * kernel of the iteration): events[2*i] just before and events[2*i+1] just
 * after the i-th such launch, for i < n_event_pairs.  *recorded (if non-null)
 * receives the number of pairs recorded.  With events == NULL it is the plain
 * call.
 * Errors: as the plain call, plus MUON_ERR_INVALID_ARG for n_event_pairs < 0
 * or events == NULL with n_event_pairs > 0.
 */
int muon_ns5_batched_timed(const float* const* G, float* const* out, float* const* buf, float mu,
                           const int64_t* rows, const int64_t* cols, int64_t count, int steps, float eps,
                           void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                           int n_event_pairs, int* recorded);

/* Largest min(rows, cols) of muon_polar_svd_grouped. */
#define MUON_POLAR_MAX_SHORT 4096

/*
 * Bytes of workspace muon_polar_svd_grouped needs for `count` matrices of
 * rows x cols (passes of MUON_NS5_MAX_GROUP reuse it); 0 for invalid sizes
 * or a short side above MUON_POLAR_MAX_SHORT.  256-byte aligned device
 * memory; contents on entry do not matter.
 */
size_t muon_polar_svd_workspace_size(int64_t rows, int64_t cols, int64_t count);

/*
 * U V^T of each G = U S V^T, computed through an SVD on the GPU: the
 * orthogonalisation that NS5 approximates, and that the Muon section of the
 * Synced report on Modded-NanoGPT calls too slow for the optimizer; this
 * entry point exists to measure that claim against NS5 on the same matrices.
 * Block one-sided Jacobi on the rows of the short-side-first W (G or G^T):
 * float32 storage, float64 arithmetic; a sweep pairs every two blocks of 32
 * rows once, diagonalising each pair's 64 x 64 Gram matrix by cyclic Jacobi
 * and rotating the pair's rows, until every two rows are orthogonal to a
 * cosine of 1e-6 or max_sweeps sweeps have run.  The result has G's shape and
 * orientation; for a rank-deficient G (singular values below 1e-6 of the
 * largest) it is U_r V_r^T over the nonzero singular values.
 *  G, out : host arrays of `count` device pointers, float32 rows x cols; out[i]
 *           may alias G[i].
 *  max_sweeps : 1 .. 64 (12 is ample for the workloads here).
 *  workspace, workspace_bytes : >= muon_polar_svd_workspace_size(rows, cols,
 *           count).
 * Errors: MUON_ERR_INVALID_ARG (null pointers, sizes < 1, count < 1,
 * max_sweeps out of range), MUON_ERR_UNSUPPORTED (short side above
 * MUON_POLAR_MAX_SHORT or long side above MUON_NS5_MAX_LONG),
 * MUON_ERR_WORKSPACE.
 */
int muon_polar_svd_grouped(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols,
                           int max_sweeps, void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The Muon
 * step of muon_momentum_ns5_batched, with the workspace taken from a device
 * array the library holds instead of a caller argument: MUON_STATIC_WORKSPACE_BYTES
 * per GPU, allocated when the library's code is loaded on that GPU and kept
 * until the process ends.  The call itself allocates no device memory (its
 * host-side planning uses small host containers).
 *  g, buf, out, rows, cols, count, mu, steps, eps, stream : as
 *         muon_momentum_ns5_batched (device pointers in host arrays; the
 *         caller owns them).
 * Results are bitwise those of muon_momentum_ns5_batched.  A batch whose
 * workspace exceeds MUON_STATIC_WORKSPACE_BYTES runs in more launch groups
 * (each fitting in it), one after another; a matrix whose own workspace
 * exceeds it (muon_ns5_workspace_size(rows, cols, 1) > the size: a square
 * matrix of side above 5632, or 4096 x 16384) is rejected.
 * Every call on one GPU uses that GPU's single array: calls that overlap in
 * time on one GPU (different streams, threads or processes' graphs replayed
 * concurrently) race and give undefined results; order them on one stream.
 * Errors: as muon_momentum_ns5_batched, plus MUON_ERR_UNSUPPORTED for a
 * matrix too large for the static workspace, and MUON_ERR_HIP if no device
 * is current or the array's address cannot be found; nothing is enqueued
 * then.
 */
#define MUON_STATIC_WORKSPACE_BYTES (256u << 20)
int muon_momentum_ns5_batched_static(const float* const* g, float* const* buf, float* const* out,
                                     const int64_t* rows, const int64_t* cols, int64_t count, float mu, int steps,
                                     float eps, void* stream);

/* Static description of a status code ("ok", "invalid argument", ...). */
const char* muon_status_string(int status);

/* Per-thread description of the most recent failing call ("" if none). */
const char* muon_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_H */
