/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan library
 *               (libssmscan.so).
 *
 * Sources (web pages; cited by title and section/equation):
 *   [SPEC]      "ТЕХНИЧЕСКОЕ ЗАДАНИЕ: Реализовать selective scan (Mamba)"
 *               (aivaro.ru practice task 53)
 *   [EXPLAINED] "Mamba CUDA 实现解析" (mamba-code-explained README)
 *   [BLELLOCH]  "从顺序到并行用PyTorch实现Blelloch算法加速Mamba状态空间模型"
 *               (lpnh.cn news 821471)
 *   [CUTILE]    "Прорыв в оптимизации SSM-моделей" (aikraft.ru digest of the
 *               cuTile Mamba-2 forward kernels)
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to dense, contiguous,
 *     row-major memory owned by the caller.  The library never frees them
 *     and keeps no reference after the enqueued work completes.
 *   - Calls only enqueue work on `stream` and return; they never
 *     synchronise the host.  Results are ready when the stream reaches them.
 *   - Outputs must not alias inputs.
 *   - Errors are reported by status code only; nothing is thrown across the
 *     ABI.  All argument checks run before any HIP call, so a rejected call
 *     has no side effect.  ssm_last_error_message() describes the most
 *     recent failure on the calling thread.
 *   - Every tensor base pointer must be 16-byte aligned (any allocation
 *     from hipMalloc or PyTorch is).
 *   - Floating-point inputs are either all float32 or all bfloat16
 *     (`in_dtype`), except the parameters documented as float32.
 *     Arithmetic is float32 throughout (bf16 inputs are widened exactly).
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle type (identical to the typedef in the HIP headers). */
typedef struct ihipStream_t *hipStream_t;

typedef enum ssm_status {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or enum value */
  SSM_ERR_UNSUPPORTED = 2, /* valid request outside the documented limits,
                              or a device that is not gfx950 */
  SSM_ERR_HIP = 3          /* a HIP runtime call failed */
} ssm_status;

typedef enum ssm_dtype {
  SSM_F32 = 0,  /* IEEE float32 */
  SSM_BF16 = 1  /* bfloat16 (upper half of a float32) */
} ssm_dtype;

typedef struct ssm_scan_context *ssm_handle;

/* Static text for a status code (never NULL). */
const char *ssm_status_string(ssm_status status);

/* Human-readable reason for the most recent non-OK status returned on the
 * calling thread ("" if none).  Valid until the next call on this thread. */
const char *ssm_last_error_message(void);

/* Create a handle bound to HIP device `hip_device`.  Reads the device
 * properties once, rejects non-gfx950 devices with SSM_ERR_UNSUPPORTED and
 * fixes the per-shape launch table.  Allocates no per-call memory.  The
 * handle is immutable afterwards and may be used from several threads and
 * streams at once.  *out is set to NULL on failure. */
ssm_status ssm_scan_create(ssm_handle *out, int hip_device);

/* Destroy a handle (NULL is accepted).  The handle owns no device memory,
 * so destroying it while work enqueued with it is still in flight is safe. */
ssm_status ssm_scan_destroy(ssm_handle handle);

/*
 * Mamba-1 selective scan, forward ([SPEC] Stage 1 items 3-4; [EXPLAINED]
 * eqs. (4)-(12); [BLELLOCH] section 4.1).  For every row (b, d) and time t,
 * with the state h[b,d,:] starting at zero:
 *
 *   delta_t = delta[b,d,t] + delta_bias[d]       (bias optional)
 *   delta_t = softplus(delta_t)                   if delta_softplus != 0
 *   h[n]    = exp(delta_t * A[d,n]) * h[n] + delta_t * B[b,n,t] * u[b,d,t]
 *   y[b,d,t] = sum_n C[b,n,t] * h[n]  +  D[d] * u[b,d,t]   (D optional)
 *   y[b,d,t] *= silu(z[b,d,t])                    (z optional)
 *   last_state[b,d,n] = h[n] after t = seqlen-1   (optional output)
 *
 * The recurrence is evaluated as an associative scan over (a, v) pairs with
 * the combine operator of [EXPLAINED] eq. (10); the result equals the plain
 * sequential loop up to float32 rounding.
 *
 * Layouts (row-major):
 *   u, delta, z, y : [batch, dim, seqlen]      element type in_dtype
 *   B, C           : [batch, dstate, seqlen]   element type in_dtype
 *   A              : [dim, dstate]             float32
 *   D, delta_bias  : [dim]                     float32
 *   last_state     : [batch, dim, dstate]      float32
 * Nullable: D, z, delta_bias, last_state.  y has the input element type.
 *
 * Limits: batch, dim, seqlen >= 1; 1 <= dstate <= 64 ([SPEC] Definition of
 * Done asks for documented limits; there is no seqlen limit).  batch*dim
 * and seqlen must each fit in 2^31-1.  Sizes <= 0 return
 * SSM_ERR_INVALID_ARG without touching the device ([SPEC] Definition of
 * Done: batch=0 must not crash).  The initial state is zero (see
 * ssm_selective_scan_fwd_with_state for a given one).
 *
 * Performance: when the rows are too few to give every SIMD a wave (e.g.
 * batch 2, dim 1536), this call splits each time chunk across the waves of
 * one workgroup only (73 us at batch 2, dim 1536, dstate 16, seqlen 2048,
 * float32); ssm_selective_scan_fwd_ws with a workspace also splits the
 * sequence across workgroups (63 us there, and far faster for a single
 * short row block such as batch 1, dim 256: 16 against 68 us).
 */
ssm_status ssm_selective_scan_fwd(ssm_handle handle, const void *u,
                                  const void *delta, const float *A,
                                  const void *B, const void *C, const float *D,
                                  const void *z, const float *delta_bias,
                                  int delta_softplus, void *y,
                                  float *last_state, int64_t batch,
                                  int64_t dim, int64_t dstate, int64_t seqlen,
                                  ssm_dtype in_dtype, hipStream_t stream);

/*
 * ssm_selective_scan_fwd with an initial state: h[b,d,:] starts at
 * initial_state[b,d,:] instead of zero (the v_0 term of the closed form in
 * [EXPLAINED] eqs. (8)-(9)).  A sequence split into pieces and scanned piece
 * by piece, each call given the last_state of the previous one, gives the
 * same y and last_state as one call over the whole sequence (up to float32
 * rounding).
 *
 *   initial_state : [batch, dim, dstate] float32, nullable (NULL = zero,
 *                   which is ssm_selective_scan_fwd).  16-byte aligned.
 *                   It may be the same pointer as last_state (the state is
 *                   then updated in place); any other overlap with an
 *                   output returns SSM_ERR_INVALID_ARG.
 * Every other argument, layout, limit and error is as for
 * ssm_selective_scan_fwd.
 */
ssm_status ssm_selective_scan_fwd_with_state(
    ssm_handle handle, const void *u, const void *delta, const float *A,
    const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, const float *initial_state,
    void *y, float *last_state, int64_t batch, int64_t dim, int64_t dstate,
    int64_t seqlen, ssm_dtype in_dtype, hipStream_t stream);

/*
 * ssm_selective_scan_fwd_with_state with B and C given per group of
 * channels: channel d reads B[b, g, :, :] and C[b, g, :, :] with
 * g = d / (dim / ngroups).  ngroups = 1 is ssm_selective_scan_fwd_with_state;
 * ngroups = dim gives every channel its own B and C, the per-channel form
 * of the [SPEC] reference kernel (B and C indexed by batch, channel and
 * step, one state per channel there).
 *
 *   B, C    : [batch, ngroups, dstate, seqlen] in_dtype, 16-byte aligned
 *   ngroups : >= 1 and a divisor of dim, else SSM_ERR_INVALID_ARG
 * Every other argument, layout, limit and error is as for
 * ssm_selective_scan_fwd_with_state.  When dim / ngroups is a multiple of
 * the rows one workgroup handles (64 to 256), B and C are staged once per
 * workgroup as for one group; otherwise each row reads its own B and C.
 */
ssm_status ssm_selective_scan_fwd_grouped(
    ssm_handle handle, const void *u, const void *delta, const float *A,
    const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, const float *initial_state,
    void *y, float *last_state, int64_t batch, int64_t dim, int64_t dstate,
    int64_t seqlen, int64_t ngroups, ssm_dtype in_dtype, hipStream_t stream);

/*
 * Bytes of workspace that ssm_selective_scan_fwd_ws can use for these
 * sizes: 0 when the (batch, channel) rows alone give every SIMD of the
 * device a wave (with per-row B, C, see below: every CU a wave), or when
 * the sequence is too short to split (fewer than 8 time chunks of the
 * kernel); then no workspace is needed.  Else the room
 * for one aggregate (prod a, v) per (segment, row, state) of a time split
 * ([EXPLAINED] eqs. (10)-(11)).  Same size checks as
 * ssm_selective_scan_fwd_grouped; touches no device memory.
 */
ssm_status ssm_selective_scan_fwd_workspace_size(ssm_handle handle,
                                                 int64_t batch, int64_t dim,
                                                 int64_t dstate, int64_t seqlen,
                                                 int64_t ngroups,
                                                 size_t *bytes);

/*
 * ssm_selective_scan_fwd_grouped with a caller-owned device workspace.
 * When the workspace size above is non-zero and workspace is given, the
 * sequence is cut into time segments: a first launch scans every segment
 * from the identity and stores its aggregate (prod a, v) per (row, state)
 * in the workspace; a second launch folds, for each segment, the
 * aggregates before it onto the initial state with the combine operator
 * of [EXPLAINED] eq. (10) and rescans the segment from that carry-in,
 * writing y.  This fills the device for small batches and long sequences.
 * The result equals the unsplit call's up to float32 rounding.
 *
 *   workspace       : device memory, 16-byte aligned, nullable (NULL = no
 *                     split: the call is ssm_selective_scan_fwd_grouped);
 *                     overwritten; must not overlap any input or output.
 *   workspace_bytes : its size; below the size above (with workspace
 *                     given and a split planned) is SSM_ERR_INVALID_ARG.
 * No split is made when initial_state is last_state (in place).  When a
 * group of channels does not cover whole workgroups (64 to 256 rows), each
 * row reads its own B, C rows and the split is made only when the rows
 * give fewer waves than the device has CUs (the aggregate launch reads the
 * B rows a second time).  Every other argument, layout, limit and error is as for
 * ssm_selective_scan_fwd_grouped.
 */
ssm_status ssm_selective_scan_fwd_ws(
    ssm_handle handle, const void *u, const void *delta, const float *A,
    const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, const float *initial_state,
    void *y, float *last_state, int64_t batch, int64_t dim, int64_t dstate,
    int64_t seqlen, int64_t ngroups, void *workspace, size_t workspace_bytes,
    ssm_dtype in_dtype, hipStream_t stream);

/*
 * ssm_selective_scan_fwd_ws for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc.  It takes no workspace and allocates nothing; when the
 * time split applies, its aggregates go to a scratch array of
 * SSM_NOALLOC_SCRATCH_BYTES that the library keeps on each GPU it runs on
 * (a file-scope device array, held until the process ends).  Every plan of
 * the time split on a 256-CU gfx950 device fits in it; a plan that would
 * not returns SSM_ERR_UNSUPPORTED before any device work.
 *
 * The scratch is shared by every call on the same GPU and keeps the last
 * call's contents; no part of it needs to start at zero (a call writes
 * every entry it reads).  Calls on one GPU whose device work overlaps in
 * time (different streams, different threads, different handles) race on
 * it and must be serialised by the caller, e.g. by issuing them on one
 * stream.  Arguments, layouts, limits, results and every other error are
 * those of ssm_selective_scan_fwd_ws (with the workspace it would use).
 */
#define SSM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ssm_status ssm_selective_scan_fwd_noalloc(
    ssm_handle handle, const void *u, const void *delta, const float *A,
    const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, const float *initial_state,
    void *y, float *last_state, int64_t batch, int64_t dim, int64_t dstate,
    int64_t seqlen, int64_t ngroups, ssm_dtype in_dtype, hipStream_t stream);

/*
 * Workspace size in bytes needed by ssm_selective_scan_bwd for these sizes
 * (caller-allocated).  Same size checks as ssm_selective_scan_bwd.
 */
ssm_status ssm_selective_scan_bwd_workspace_size(ssm_handle handle,
                                                 int64_t batch, int64_t dim,
                                                 int64_t dstate, int64_t seqlen,
                                                 size_t *bytes);

/*
 * Mamba-1 selective scan, backward ([SPEC]: the backward-pass stage asks
 * for the gradients of every input; [EXPLAINED] eqs. (5)-(7): the
 * recurrence differentiated).  Given the forward inputs of
 * ssm_selective_scan_fwd_with_state and the upstream gradients dy (of y)
 * and dlast_state (of last_state), computes the gradient of
 *   sum(dy * y) + sum(dlast_state * last_state)
 * with respect to u, delta (the raw delta, before bias and softplus), A, B,
 * C, D, z, delta_bias and initial_state.  The forward is recomputed inside
 * the call (a state saved every 16 steps in the workspace); nothing needs
 * to be kept from the forward call.
 *
 * Layouts (row-major):
 *   u, delta, z, dy, du, ddelta, dz : [batch, dim, seqlen]  in_dtype
 *   B, C                            : [batch, dstate, seqlen] in_dtype
 *   dB, dC                          : [batch, dstate, seqlen] float32
 *   A, dA                           : [dim, dstate]  float32
 *   D, delta_bias, dD, ddelta_bias  : [dim]          float32
 *   initial_state, dlast_state, dinitial_state : [batch, dim, dstate] float32
 * Nullable: D, z, delta_bias, initial_state (zero), dlast_state (zero),
 * dD, ddelta_bias, dinitial_state (not computed); dz is required when z
 * is given.  workspace: ssm_selective_scan_bwd_workspace_size bytes.
 * Pointers 16-byte aligned; outputs and the workspace must not overlap
 * each other or any input.  Every output is overwritten (nothing is
 * accumulated into).  The result is deterministic (partial sums are added
 * in a fixed order).
 *
 * Limits: as ssm_selective_scan_fwd (dstate <= 64; SSM_ERR_UNSUPPORTED
 * above).  For dstate > 16 the states are taken in blocks of 16, each a
 * backward pass of its own whose per-step sums over its states are added
 * up across blocks (the workspace then also holds three float32
 * [batch, dim, seqlen] accumulators); the result is the same.
 */
ssm_status ssm_selective_scan_bwd(
    ssm_handle handle, const void *u, const void *delta, const float *A,
    const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, const float *initial_state,
    const void *dy, const float *dlast_state, void *du, void *ddelta,
    float *dA, float *dB, float *dC, float *dD, void *dz,
    float *ddelta_bias, float *dinitial_state, void *workspace,
    size_t workspace_bytes, int64_t batch, int64_t dim, int64_t dstate,
    int64_t seqlen, ssm_dtype in_dtype, hipStream_t stream);

/*
 * Workspace size of ssm_selective_scan_bwd_grouped (as
 * ssm_selective_scan_bwd_workspace_size, for ngroups groups of B and C).
 * Same size and group checks as ssm_selective_scan_bwd_grouped.
 */
ssm_status ssm_selective_scan_bwd_grouped_workspace_size(ssm_handle handle,
                                                        int64_t batch, int64_t dim,
                                                        int64_t dstate, int64_t seqlen,
                                                        int64_t ngroups, size_t *bytes);

/*
 * ssm_selective_scan_bwd for B and C given per group of channels, as in
 * ssm_selective_scan_fwd_grouped ([SPEC] backward-pass stage; channel d
 * reads group d / (dim / ngroups)):
 *   B, C   : [batch, ngroups, dstate, seqlen] in_dtype
 *   dB, dC : [batch, ngroups, dstate, seqlen] float32, each group's
 *            gradient summed over its channels only
 *   workspace: ssm_selective_scan_bwd_grouped_workspace_size bytes.
 * ngroups >= 1 must divide dim (else SSM_ERR_INVALID_ARG); any such value
 * is supported.  When dim / ngroups is a multiple of the channels one
 * workgroup of the shared-B/C backward kernels handles (64 for dstate
 * 9..64, 128 for 5..8, 256 for 1..4), those kernels run and sum dB, dC
 * over whole workgroups; otherwise (per-channel B and C, ngroups = dim,
 * down to groups of a few channels) a kernel with one state per lane reads
 * each row's own B and C, and for groups of more than one channel writes
 * per-row dB, dC to the workspace (2 * batch * dim * dstate * seqlen floats
 * of it) that a second kernel adds up per group, in channel order; at small
 * batches it cuts the sequence in time as the shared-B/C kernels do (the
 * workspace then also holds the segments' aggregates).  Both are
 * deterministic.  ngroups = 1 is ssm_selective_scan_bwd.  Every other
 * argument, layout, limit and error is as for ssm_selective_scan_bwd.
 */
ssm_status ssm_selective_scan_bwd_grouped(
    ssm_handle handle, const void *u, const void *delta, const float *A,
    const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, const float *initial_state,
    const void *dy, const float *dlast_state, void *du, void *ddelta,
    float *dA, float *dB, float *dC, float *dD, void *dz,
    float *ddelta_bias, float *dinitial_state, void *workspace,
    size_t workspace_bytes, int64_t batch, int64_t dim, int64_t dstate,
    int64_t seqlen, int64_t ngroups, ssm_dtype in_dtype, hipStream_t stream);

/*
 * One decode step of the Mamba-1 recurrence ([SPEC] Stage 1 items 3-4;
 * [EXPLAINED] eqs. (5)-(7); [BLELLOCH] section 1: the sequential form for
 * online inference).  For every row (b, d), with the state updated in place:
 *
 *   delta   = delta[b,d] + delta_bias[d];  softplus if delta_softplus != 0
 *   state[b,d,n] = exp(delta * A[d,n]) * state[b,d,n] + delta * B[b,n] * u[b,d]
 *   y[b,d]  = (sum_n C[b,n] * state[b,d,n] + D[d] * u[b,d]) * silu(z[b,d])
 *
 * This is ssm_selective_scan_fwd_with_state for seqlen = 1 with the state
 * updated in place (same result), with a kernel sized for one step.
 *
 * Layouts (row-major):
 *   u, delta, z, y : [batch, dim]       element type in_dtype
 *   B, C           : [batch, dstate]    element type in_dtype
 *   A              : [dim, dstate]      float32
 *   D, delta_bias  : [dim]              float32
 *   state          : [batch, dim, dstate] float32, read and written
 * Nullable: D, z, delta_bias.  Pointers 16-byte aligned; state and y must
 * not overlap each other or any input (SSM_ERR_INVALID_ARG).
 * Limits: batch, dim >= 1; 1 <= dstate <= 64; batch*dim <= 2^40.
 */
ssm_status ssm_selective_state_update(ssm_handle handle, float *state,
                                      const void *u, const void *delta,
                                      const float *A, const void *B,
                                      const void *C, const float *D,
                                      const void *z, const float *delta_bias,
                                      int delta_softplus, void *y, int64_t batch,
                                      int64_t dim, int64_t dstate,
                                      ssm_dtype in_dtype, hipStream_t stream);

/*
 * ssm_selective_state_update with B and C given per group of channels, as
 * in ssm_selective_scan_fwd_grouped ([SPEC] reference kernel's per-channel
 * B, C at ngroups = dim): channel d reads group g = d / (dim / ngroups),
 *   B, C : [batch, ngroups, dstate] in_dtype.
 * ngroups >= 1 must divide dim (else SSM_ERR_INVALID_ARG); ngroups = 1 is
 * ssm_selective_state_update.  Calling it token after token equals
 * ssm_selective_scan_fwd_grouped over the tokens with the state carried
 * (up to float32 rounding).  Every other argument, layout, limit and error
 * is as for ssm_selective_state_update.
 */
ssm_status ssm_selective_state_update_grouped(
    ssm_handle handle, float *state, const void *u, const void *delta,
    const float *A, const void *B, const void *C, const float *D, const void *z,
    const float *delta_bias, int delta_softplus, void *y, int64_t batch,
    int64_t dim, int64_t dstate, int64_t ngroups, ssm_dtype in_dtype,
    hipStream_t stream);

/*
 * One decode step of the Mamba-2 (SSD) recurrence: one new token per
 * (batch, head), the state updated in place ([CUTILE]: the recurrence with
 * a scalar A per head; [EXPLAINED] eq. (2): the skip term).  For every
 * (b, head h) with group g = h / (nheads/ngroups) and every p, n:
 *
 *   dt = dt[b,h] + dt_bias[h];  softplus if dt_softplus != 0
 *   state[b,h,p,n] = exp(dt * A[h]) * state[b,h,p,n] + dt * x[b,h,p] * B[b,g,n]
 *   y[b,h,p] = sum_n C[b,g,n] * state[b,h,p,n] + D[h] * x[b,h,p]
 *
 * This equals ssd_chunk_scan_fwd_with_state over a sequence of one token
 * with initial_state = state and final_state = state; calling it token
 * after token gives the chunked scan's y and final state (up to float32
 * rounding).
 *
 * Layouts (row-major):
 *   state       : [batch, nheads, headdim, dstate] float32, read and written
 *   x, y        : [batch, nheads, headdim]         in_dtype
 *   dt          : [batch, nheads]                  in_dtype
 *   B, C        : [batch, ngroups, dstate]         in_dtype
 *   A, D, dt_bias : [nheads]                       float32
 * Nullable: D, dt_bias.  Pointers 16-byte aligned; y and state must not
 * overlap each other or any input.
 *
 * Limits: all sizes >= 1; nheads a multiple of ngroups; dstate <= 256;
 * batch*nheads*headdim <= 2^40.
 */
ssm_status ssd_state_update(ssm_handle handle, float *state, const void *x,
                            const void *dt, const float *A, const void *B,
                            const void *C, const float *D,
                            const float *dt_bias, int dt_softplus, void *y,
                            int64_t batch, int64_t nheads, int64_t headdim,
                            int64_t dstate, int64_t ngroups,
                            ssm_dtype in_dtype, hipStream_t stream);

/*
 * Workspace size in bytes needed by ssd_chunk_scan_fwd for these sizes
 * (the caller allocates it, so the library never allocates device memory).
 * Returns SSM_ERR_INVALID_ARG / SSM_ERR_UNSUPPORTED for sizes that
 * ssd_chunk_scan_fwd would reject.
 */
ssm_status ssd_chunk_scan_workspace_size(ssm_handle handle, int64_t batch,
                                         int64_t seqlen, int64_t nheads,
                                         int64_t headdim, int64_t dstate,
                                         int64_t ngroups, int64_t chunk_size,
                                         size_t *bytes);

/*
 * Mamba-2 (SSD) chunked scan, forward ([CUTILE]: chunk cumulative sums of
 * the log-decay, chunk states advanced with the jump formula, fused output
 * with causal mask and skip connection).  For every (b, head h) with group
 * g = h / (nheads/ngroups) and state S[b,h,:,:] starting at zero:
 *
 *   dt_t  = dt[b,t,h] + dt_bias[h];  softplus if dt_softplus != 0
 *   S[p,n] = exp(dt_t * A[h]) * S[p,n] + dt_t * x[b,t,h,p] * B[b,t,g,n]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] * S[p,n] + D[h] * x[b,t,h,p]
 *   final_state[b,h,p,n] = S[p,n] after t = seqlen-1
 *
 * computed chunk by chunk (chunk_size tokens) with matrix products.
 *
 * Layouts (row-major):
 *   x, y        : [batch, seqlen, nheads, headdim]   in_dtype
 *   dt          : [batch, seqlen, nheads]            in_dtype
 *   B, C        : [batch, seqlen, ngroups, dstate]   in_dtype
 *   A, D, dt_bias : [nheads]                         float32
 *   final_state : [batch, nheads, headdim, dstate]   float32
 * Nullable: D, dt_bias, final_state.  `workspace` must hold at least
 * ssd_chunk_scan_workspace_size() bytes (16-byte aligned device memory,
 * caller-owned, contents need not be initialised; it is overwritten).
 *
 * Limits: nheads % ngroups == 0; chunk_size in {64, 128, 256};
 * 1 <= headdim <= 128; 1 <= dstate <= 256; bf16 inputs only (in_dtype
 * SSM_F32 returns SSM_ERR_UNSUPPORTED).  The kernels' tiles cover headdim
 * 32, 64, 128 and dstate 32, 64, 128, 256; other sizes run on zero-padded
 * copies of x, B, C (and the initial state) in the workspace, whose size
 * then includes them; the result is the same.
 */
ssm_status ssd_chunk_scan_fwd(ssm_handle handle, const void *x, const void *dt,
                              const float *A, const void *B, const void *C,
                              const float *D, const float *dt_bias,
                              int dt_softplus, void *y, float *final_state,
                              void *workspace, size_t workspace_bytes,
                              int64_t batch, int64_t seqlen, int64_t nheads,
                              int64_t headdim, int64_t dstate, int64_t ngroups,
                              int64_t chunk_size, ssm_dtype in_dtype,
                              hipStream_t stream);

/*
 * ssd_chunk_scan_fwd with an initial state: S[b,h,:,:] starts at
 * initial_state[b,h,:,:] instead of zero (the v_0 term of the closed form in
 * [EXPLAINED] eqs. (8)-(9), carried across chunks by the same jump formula
 * as every chunk state).  Scanning a sequence in pieces, each call given the
 * final_state of the previous one, gives the same y and final_state as one
 * call (up to rounding; the carried state passes through bf16 between
 * chunks as in ssd_chunk_scan_fwd).
 *
 *   initial_state : [batch, nheads, headdim, dstate] float32, nullable
 *                   (NULL = zero, which is ssd_chunk_scan_fwd).  16-byte
 *                   aligned.  It may be the same pointer as final_state (an
 *                   in-place update); any other overlap with an output
 *                   returns SSM_ERR_INVALID_ARG.
 * Every other argument, layout, limit and error is as for ssd_chunk_scan_fwd.
 */
ssm_status ssd_chunk_scan_fwd_with_state(
    ssm_handle handle, const void *x, const void *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    int dt_softplus, const float *initial_state, void *y, float *final_state,
    void *workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen,
    int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
    int64_t chunk_size, ssm_dtype in_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
