/*
 * mamba_scan.h -- C ABI of the MI355X (gfx950) selective-scan (S6) library.
 *
 * The library computes, for every channel (b, d) independently, the selective
 * state space recurrence of Mamba (Gu & Dao, "Mamba: Linear-Time Sequence
 * Modeling with Selective State Spaces"):
 *
 *   delta_t = softplus(delta_raw_t + delta_bias[d])        (or without softplus)
 *   Abar_t[n] = exp(delta_t * A[d,n])
 *   Bbar_t[n] = (exp(delta_t*A[d,n]) - 1) / A[d,n] * B[b,n,t]    (ZOH)
 *             =  delta_t * B[b,n,t]                             (EULER)
 *   h_t[n]  = Abar_t[n] * h_{t-1}[n] + Bbar_t[n] * u_t,   h_{-1} = h0 (or 0)
 *   y_t     = sum_n C[b,n,t] * h_t[n] + D[d] * u_t
 *   out_t   = y_t * z_t * sigmoid(z_t)                      (when z is given)
 *
 * Definitions on the pages this follows:
 *   - ZOH rule and recurrence: chapterpal.com page of the paper, Knowl 1
 *     "Selective State Space Layer (S6)", steps 3 and 4 (diagonal A, so the
 *     matrix exponential is elementwise).
 *   - delta = tau_Delta(Parameter + s_Delta(x)) with tau_Delta = softplus:
 *     same Knowl, step 2; delta_bias is that Parameter.
 *   - B and C shared by all D channels, shape (B, L, N); A of shape (D, N):
 *     trishampatil.com essay, Part II §6 "S6: the selective SSM", Algorithm 2.
 *   - h_0 = 0: same essay, Part II §4.
 *   - Fused scan, chunks carrying the scan state across chunk boundaries,
 *     recomputation of the states in the backward: paper-graph-ui.vercel.app
 *     summary, section 3.4, "Hardware-Aware Scan Algorithm (Section 3.3)".
 *   - SiLU gate: chapterpal page, Knowl 3 "Mamba Block Architecture" items
 *     4-5 (the gate branch multiplies the SSM output).
 * The D skip term, the gate fused into the scan, the Euler variant of Bbar
 * and the initial state h0 are part of this library's specification, not of
 * the pages.
 *
 * Layouts: every array is dense, row-major, with no strides.
 *   u, delta, z, out, dout, du, ddelta, dz   (batch, dim, seqlen)
 *   B, C, dB, dC                             (batch, dstate, seqlen)
 *   A, dA                                    (dim, dstate)
 *   D, dD, delta_bias, ddelta_bias           (dim)
 *   h0, dh0, last_state, state               (batch, dim, dstate)
 *   state_update per-step tensors: u, delta, z, out (batch, dim);
 *                                  B, C (batch, dstate)
 * Dtypes: `dt` selects the element type of u, delta, B, C, z, out and dout
 * (MAMBA_F32 or MAMBA_BF16, bfloat16 stored as 16-bit words).  A, D,
 * delta_bias, h0, last_state, state and every gradient are float32.  All
 * arithmetic is float32; bf16 inputs are widened exactly, bf16 outputs are
 * rounded to nearest even.
 *
 * Pointers: every array pointer is a DEVICE pointer (hipMalloc'ed or
 * equivalent memory visible to the GPU) with at least 16-byte alignment.
 * `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *
 * Ownership: the caller allocates and frees every buffer, including the
 * workspace sized by the *_workspace_size queries.  The library never
 * allocates, frees or synchronizes, keeps no global mutable state, and only
 * enqueues work on `stream`.  Inputs are read only.  Outputs are fully
 * overwritten (gradients are never accumulated into caller memory); the
 * library clears whatever it accumulates into on `stream` itself.  Calls on
 * distinct streams with distinct output and workspace buffers may run
 * concurrently.
 *
 * Errors: functions return a mamba_status and never abort.  Arguments are
 * checked before anything is enqueued; on any error nothing is enqueued and
 * outputs are untouched.  A failed kernel launch returns MAMBA_ERR_HIP.
 * Faults inside kernels surface at the caller's next synchronization, as
 * for any HIP call.  Limits: batch >= 1, dim >= 1, 1 <= dstate <= 64,
 * seqlen >= 1, batch*dim*seqlen < 2^62; otherwise MAMBA_ERR_UNSUPPORTED
 * (MAMBA_ERR_SHAPE for non-positive sizes).
 */
#ifndef MAMBA_SCAN_H_
#define MAMBA_SCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MAMBA_SCAN_ABI_VERSION 2

typedef enum {
  MAMBA_OK = 0,
  MAMBA_ERR_NULL_PTR = 1,     /* a required pointer is NULL                 */
  MAMBA_ERR_SHAPE = 2,        /* a size is zero or negative                 */
  MAMBA_ERR_DTYPE = 3,        /* unknown dtype or discretization value      */
  MAMBA_ERR_ALIGNMENT = 4,    /* a pointer is not 16-byte aligned           */
  MAMBA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required    */
  MAMBA_ERR_UNSUPPORTED = 6,  /* sizes outside the supported limits         */
  MAMBA_ERR_HIP = 7,          /* a HIP runtime call or launch failed        */
  MAMBA_ERR_INVALID = 8,      /* inconsistent optional arguments            */
  MAMBA_ERR_SCRATCH_LIMIT = 9 /* more scratch than mamba_scan_bwd_noalloc's
                                 fixed device array holds                   */
} mamba_status;

typedef enum { MAMBA_F32 = 0, MAMBA_BF16 = 1 } mamba_dtype;

typedef enum { MAMBA_DISC_ZOH = 0, MAMBA_DISC_EULER = 1 } mamba_disc;

/* Version of this ABI (MAMBA_SCAN_ABI_VERSION). */
int mamba_abi_version(void);

/* Static description of a status code; never NULL. */
const char* mamba_status_string(mamba_status status);

/* Bytes of device workspace mamba_scan_fwd needs for these sizes (may be 0;
 * then workspace may be NULL).  Returns SIZE_MAX for unsupported sizes.
 * It is non-zero when the sequence spans at least 8 chunks of 128 steps and
 * the channels alone give at most 256 workgroups of 16 channels (batch *
 * ceil(dim/16) <= 256), too few to fill the GPU: the forward then splits the
 * sequence into segments that run in parallel, joined by an exact carry of the state
 * (the associative scan composition of trishampatil essay, Part III §2, with
 * the chunking of its Part III §4).  The workspace holds, per channel and
 * segment, the segment's end state, its entering state (float32, dstate
 * each) and its delta sum.  mamba_scan_fwd given a smaller workspace (or
 * NULL) still works, in one pass over the sequence (slower for such shapes). */
size_t mamba_scan_fwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                     mamba_dtype dt);

/* Bytes of device workspace mamba_scan_bwd needs (SIZE_MAX if unsupported).
 * It holds the state entering every 128-step chunk (batch, dim,
 * ceil(seqlen/128), dstate) float32 and one int per workgroup.  When the
 * channels alone give at most 512 workgroups of 16 channels (batch *
 * ceil(dim/16) <= 512) the backward splits the sequence into segments run in
 * parallel (the reverse adjoint scan composes over segments like the state,
 * trishampatil essay, Part III §2), and the workspace adds per channel and
 * segment the state-pass buffers of the forward's segmentation and the
 * adjoint's (its value at the segment start from a zero end, the value
 * entering it, the delta sum).  mamba_scan_bwd given only the unsegmented
 * size runs in one pass over the sequence (slower for such shapes). */
size_t mamba_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                     mamba_dtype dt);

/*
 * Forward scan: writes out (batch, dim, seqlen) and, when last_state is not
 * NULL, the final state h_{seqlen-1} (batch, dim, dstate) in float32.
 * D, z, delta_bias, h0, last_state may be NULL (no skip term, no gate, zero
 * bias, zero initial state, no final state).  The expanded (B, L, D, N)
 * tensors are never written to memory: only out and last_state are.
 */
mamba_status mamba_scan_fwd(const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z,
                            const float* delta_bias, const float* h0, int delta_softplus,
                            mamba_disc disc, mamba_dtype dt, int64_t batch, int64_t dim,
                            int64_t dstate, int64_t seqlen, void* out, float* last_state,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of mamba_scan_fwd for the loss sum(dout * out): recomputes the
 * states from the inputs (none are saved by the forward) and writes float32
 * gradients du, ddelta (w.r.t. the raw delta), dA, dB, dC, and, exactly when
 * the matching input is given, dD, dz, ddelta_bias, dh0 (each must be NULL
 * when its input is NULL, else MAMBA_ERR_INVALID; dh0 may also be NULL when
 * h0 is given, to skip it).  No gradient flows into last_state.  Reductions
 * (dA, dB, dC, dD, ddelta_bias) use float32 atomics or partial sums, so the
 * backward is deterministic only up to float32 rounding order.
 */
mamba_status mamba_scan_bwd(const void* u, const void* delta, const float* A, const void* B,
                            const void* C, const float* D, const void* z,
                            const float* delta_bias, const float* h0, const void* dout,
                            int delta_softplus, mamba_disc disc, mamba_dtype dt, int64_t batch,
                            int64_t dim, int64_t dstate, int64_t seqlen, float* du,
                            float* ddelta, float* dA, float* dB, float* dC, float* dD, float* dz,
                            float* ddelta_bias, float* dh0, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * mamba_scan_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It calls no hipMalloc, hipFree or other
 * allocating routine.  The buffers mamba_scan_bwd keeps in its workspace (the
 * state at every 128-step chunk start, one flag per workgroup, and for long
 * sequences the segment summaries) live instead in a file-scope device array
 * of MAMBA_NOALLOC_SCRATCH_BYTES (32 MiB), one per GPU, held from the
 * library's first use on that GPU until the process ends.  Its address is
 * looked up once per device, on the first call made with that device
 * current; `stream` must belong to the current device.
 *
 * Arguments, layouts, results and errors are those of mamba_scan_bwd (the
 * automatic segment choice included); additionally MAMBA_ERR_SCRATCH_LIMIT
 * when the problem needs more than the array holds even in one pass, checked
 * before anything is enqueued.  The array is shared by every call on a GPU
 * and keeps the last call's contents (every value the kernels read from it
 * is written earlier in the same call): calls that overlap on one GPU, from
 * several streams or host threads, race and must be serialized by the
 * caller.
 */
#define MAMBA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
mamba_status mamba_scan_bwd_noalloc(const void* u, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z,
                                    const float* delta_bias, const float* h0, const void* dout,
                                    int delta_softplus, mamba_disc disc, mamba_dtype dt,
                                    int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                    float* du, float* ddelta, float* dA, float* dB, float* dC,
                                    float* dD, float* dz, float* ddelta_bias, float* dh0,
                                    void* stream);

/*
 * One recurrent (decode) step for every (b, d): state (batch, dim, dstate)
 * float32 is updated IN PLACE (h <- Abar*h + Bbar*u) and out (batch, dim)
 * receives y * SiLU(z).  Constant time and memory per step (the pages'
 * recurrent inference mode: paper-graph-ui.vercel.app summary, section 3.4,
 * the recurrent form "ideal for autoregressive inference").
 * D, z, delta_bias may be NULL.
 */
mamba_status mamba_state_update(float* state, const void* u, const void* delta, const float* A,
                                const void* B, const void* C, const float* D, const void* z,
                                const float* delta_bias, int delta_softplus, mamba_disc disc,
                                mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                void* out, void* stream);

/*
 * Packed variable-length sequences.  Same as mamba_scan_fwd / mamba_scan_bwd
 * plus `reset`: (batch, seqlen) bytes, required (NULL returns
 * MAMBA_ERR_NULL_PTR).  Where reset[b*seqlen + t] != 0 the state of every
 * channel of batch row b is set to zero before step t, so sequences packed
 * one after another along t run exactly as if each started alone; h0 (if
 * given) enters only where step 0 is not flagged, and the backward sends no
 * gradient across a flagged step (dh0 is 0 for rows flagged at t = 0).  This
 * is the boundary resetting the pages attribute to the selection mechanism
 * (paper-graph-ui summary, section 3.4; trishampatil essay, Part II §8),
 * done by an explicit flag instead of a learned large Delta.  last_state is
 * the state after the final step of each row.  Flags run with 16 lanes per
 * channel; the workspace rules are those of the plain calls.
 */
mamba_status mamba_scan_fwd_varlen(const void* u, const void* delta, const float* A,
                                   const void* B, const void* C, const float* D, const void* z,
                                   const float* delta_bias, const float* h0,
                                   const uint8_t* reset, int delta_softplus, mamba_disc disc,
                                   mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                   int64_t seqlen, void* out, float* last_state, void* workspace,
                                   size_t workspace_bytes, void* stream);

mamba_status mamba_scan_bwd_varlen(const void* u, const void* delta, const float* A,
                                   const void* B, const void* C, const float* D, const void* z,
                                   const float* delta_bias, const float* h0, const void* dout,
                                   const uint8_t* reset, int delta_softplus, mamba_disc disc,
                                   mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                   int64_t seqlen, float* du, float* ddelta, float* dA,
                                   float* dB, float* dC, float* dD, float* dz,
                                   float* ddelta_bias, float* dh0, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Complex-valued forward: diagonal complex A, complex B, C and state (the
 * S4D-Lin parameterization, printed as A_n = -1/2 + n i in the paper-graph-ui
 * summary, section 5 (Table 8 discussion); section 3.4 "Real vs. Complex"
 * and the trishampatil essay, Part III, name complex states for audio).  Abar = exp(delta A); Bbar = (Abar - 1)/A B (ZOH, delta B at
 * A = 0) or delta B (Euler); h_t = Abar h_{t-1} + Bbar u_t;
 * y_t = Re(sum_n C_t[n] h_t[n]) + D u_t; out = y * SiLU(z).  The pages fix no
 * output convention for a complex state: the real part is this library's
 * reading (a caller that pairs each state with its conjugate may double it).
 * Complex arrays are interleaved (re, im) float32 pairs: A (dim, dstate),
 * B and C (batch, dstate, seqlen), h0 and last_state (batch, dim, dstate),
 * both nullable.  u, delta, z, out follow mamba_scan_fwd (float32 or
 * bfloat16); D, delta_bias float32.  dstate <= 16 (MAMBA_ERR_UNSUPPORTED
 * otherwise).  Errors as for mamba_scan_fwd.  The workspace, of
 * mamba_scan_fwd_complex_workspace_size bytes (0 when not needed; then it
 * may be NULL), plays the part it does for mamba_scan_fwd: for long
 * sequences over few channels the sequence is split into segments run in
 * parallel, joined by an exact carry of the complex state (per channel,
 * segment and state: the end state from zero, the entering state and the
 * segment's product of Abar).  Given less, the call runs in one pass.
 */
size_t mamba_scan_fwd_complex_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                             int64_t seqlen);

mamba_status mamba_scan_fwd_complex(const void* u, const void* delta, const float* A,
                                    const float* B, const float* C, const float* D,
                                    const void* z, const float* delta_bias, const float* h0,
                                    int delta_softplus, mamba_disc disc, mamba_dtype dt,
                                    int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                                    void* out, float* last_state, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * One recurrent (decode) step of the complex-valued model, in place on the
 * complex state (batch, dim, dstate) interleaved (re, im) float32 pairs: the
 * body of mamba_scan_fwd_complex's step loop on a stored state (autoregressive
 * generation; paper-graph-ui summary, section 3.4, recurrent mode).  u,
 * delta, z, out are (batch, dim) float32 or bfloat16; A complex (dim,
 * dstate); B, C complex (batch, dstate); D, delta_bias float32 (dim),
 * nullable; dstate <= 16.  Continuing a forward's last_state with this call
 * gives the outputs of a forward over the longer sequence.  Errors as for
 * mamba_state_update.
 */
mamba_status mamba_state_update_complex(float* state, const void* u, const void* delta,
                                        const float* A, const float* B, const float* C,
                                        const float* D, const void* z, const float* delta_bias,
                                        int delta_softplus, mamba_disc disc, mamba_dtype dt,
                                        int64_t batch, int64_t dim, int64_t dstate, void* out,
                                        void* stream);

/*
 * Backward of mamba_scan_fwd_complex for the loss sum(dout * out): the
 * states are recomputed chunkwise (one state per 128-step chunk is
 * recomputed into the workspace first).  The gradient of a complex input w
 * is dL/dRe(w) + i dL/dIm(w): dA (dim, dstate), dB, dC (batch, dstate,
 * seqlen) and dh0 (batch, dim, dstate; NULL unless h0 is given) are complex
 * (interleaved pairs); du, ddelta, dz (batch, dim, seqlen) and dD,
 * ddelta_bias (dim) are real float32.  Null-pairing rules, dtypes and errors
 * follow mamba_scan_bwd; the workspace is
 * mamba_scan_bwd_complex_workspace_size bytes: the chunk states, plus,
 * where the sequence is split into segments (the shapes mamba_scan_bwd
 * splits), the state pass's segment buffers and the adjoint's (its value at
 * each segment's start from a zero end, the value entering the segment, and
 * the segment's product of conj(Abar)).  Given only the unsegmented size it
 * runs in one pass.  Reductions use float32 atomics (deterministic up to
 * rounding order).
 */
size_t mamba_scan_bwd_complex_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                             int64_t seqlen);

mamba_status mamba_scan_bwd_complex(const void* u, const void* delta, const float* A,
                                    const float* B, const float* C, const float* D,
                                    const void* z, const float* delta_bias, const float* h0,
                                    const void* dout, int delta_softplus, mamba_disc disc,
                                    mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                                    int64_t seqlen, float* du, float* ddelta, float* dA,
                                    float* dB, float* dC, float* dD, float* dz,
                                    float* ddelta_bias, float* dh0, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Short causal depthwise convolution + SiLU, the stage that feeds the SSM
 * in the Mamba block (chapterpal.com page, Knowl 3 "Mamba Block
 * Architecture": a width-4 temporal convolution, then SiLU; trishampatil
 * essay, Part II §8).  Per channel (b, d), with W = width taps (1..4):
 *   pre_t = b[d] + sum_{k<W} w[d*W + k] * x_{t-(W-1)+k},  u_t = pre_t*sigmoid(pre_t)
 * x before t = 0 counts as zero, and so does x before the start of the
 * current packed sequence when `reset` (nullable, (batch, seqlen) bytes, as
 * for mamba_scan_fwd_varlen) flags sequence starts.
 * Layouts: x, u (batch, dim, seqlen) in `dt`; w (dim, width) and b (dim,
 * nullable) float32.  u is overwritten.
 *
 * The backward takes du (float32, the gradient at u) and writes dx
 * (float32, same layout), dw (dim, width) and db (dim; NULL iff b is NULL),
 * recomputing pre from x rather than reading a stored copy (trishampatil
 * essay, Part III §4: the block's cheap activations and the short
 * convolution are recomputed in the backward, not saved).  dw and db are
 * zeroed on the stream, then summed with float32 atomics (deterministic up to
 * rounding order).  Errors as for the scan calls; width outside 1..4 is
 * MAMBA_ERR_UNSUPPORTED.
 */
mamba_status mamba_conv1d_silu_fwd(const void* x, const float* w, const float* b,
                                   const uint8_t* reset, int64_t width, mamba_dtype dt,
                                   int64_t batch, int64_t dim, int64_t seqlen, void* u,
                                   void* stream);

mamba_status mamba_conv1d_silu_bwd(const void* x, const float* w, const float* b,
                                   const uint8_t* reset, const float* du, int64_t width,
                                   mamba_dtype dt, int64_t batch, int64_t dim, int64_t seqlen,
                                   float* dx, float* dw, float* db, void* stream);

/*
 * Tuning and timing variants.  Identical to the calls above (reset may be
 * NULL here: no flags) except for:
 *  - lanes_per_channel: the number of lanes each channel's scan is spread
 *    over (16, 32 or 64 for the forward; 0 picks the default the plain calls
 *    use; the backward accepts 0 and 16 only).  The result does not depend on
 *    the choice beyond float32 rounding order; tests and launch-shape sweeps
 *    use it.  mamba_scan_bwd_ex needs the workspace reported by
 *    mamba_scan_bwd_workspace_size_ex for the same lanes and segments values.
 *  - segments: 0 = automatic (as mamba_scan_fwd / mamba_scan_bwd), 1 = one
 *    pass over the sequence, k >= 2 = split the sequence into k segments of
 *    whole 128-step chunks (fewer when there are fewer chunks, or when k does
 *    not divide them evenly).  Segmented runs need the workspace reported by
 *    mamba_scan_fwd_workspace_size_ex / mamba_scan_bwd_workspace_size_ex for
 *    the same lanes and segments values (MAMBA_ERR_WORKSPACE otherwise) and
 *    16 lanes per channel; a segments value below 0 is
 *    MAMBA_ERR_UNSUPPORTED.
 *  - checkpoints (forward: float* output, backward: const float* input;
 *    NULL = none): the state entering every 128-step chunk, (batch, dim,
 *    ceil(seqlen/128), dstate) float32, mamba_scan_checkpoint_size bytes.
 *    A forward given the buffer writes it (with 16 lanes per channel); a
 *    backward given it uses it instead of recomputing those states in a
 *    separate pass, and then needs only the part of its workspace past the
 *    states (the query's size still suffices).  The backward still replays
 *    every state inside each chunk from its checkpoint: only 1/128 of the
 *    (B, L, D, N) states is ever stored (paper-graph-ui summary, section
 *    3.4, and trishampatil essay, Part III §4: the full states are
 *    recomputed, not saved).  Checkpoints must come from a forward over the
 *    same inputs.
 *  - timing_begin, timing_end: hipEvent_t handles (NULL = none).  When given,
 *    they are recorded on `stream` immediately before and after the main
 *    scan kernel of the call (the forward's output kernel; in a segmented
 *    run its first launch, which runs every segment from a zero state, before
 *    the carry and the launch that corrects each segment's first chunks; the
 *    backward's reverse-scan kernel, after its state-recompute, adjoint-carry
 *    and zeroing kernels have been enqueued), so a
 *    caller can time that kernel alone with hipEventElapsedTime.  The caller
 *    owns the events; failure to record one returns MAMBA_ERR_HIP.
 */
size_t mamba_scan_fwd_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                        int64_t seqlen, mamba_dtype dt, int lanes_per_channel,
                                        int segments);

mamba_status mamba_scan_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                               const void* C, const float* D, const void* z,
                               const float* delta_bias, const float* h0, const uint8_t* reset,
                               int delta_softplus, mamba_disc disc, mamba_dtype dt,
                               int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                               void* out, float* last_state, void* workspace,
                               size_t workspace_bytes, void* stream, int lanes_per_channel,
                               int segments, float* checkpoints, void* timing_begin,
                               void* timing_end);

size_t mamba_scan_bwd_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                        int64_t seqlen, mamba_dtype dt, int lanes_per_channel,
                                        int segments);

mamba_status mamba_scan_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                               const void* C, const float* D, const void* z,
                               const float* delta_bias, const float* h0, const void* dout,
                               const uint8_t* reset, int delta_softplus, mamba_disc disc,
                               mamba_dtype dt, int64_t batch, int64_t dim, int64_t dstate,
                               int64_t seqlen, float* du, float* ddelta, float* dA, float* dB,
                               float* dC, float* dD, float* dz, float* ddelta_bias, float* dh0,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int lanes_per_channel, int segments, const float* checkpoints,
                               void* timing_begin, void* timing_end);

/* Bytes of the checkpoint buffer of the _ex calls (SIZE_MAX for unsupported
 * sizes). */
size_t mamba_scan_checkpoint_size(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen);

/*
 * The complex-valued forward and backward with chunk checkpoints, as the
 * real _ex calls have them (same argument meaning as mamba_scan_fwd_complex
 * and mamba_scan_bwd_complex, plus the buffer):
 *  - checkpoints (forward: float* output, backward: const float* input;
 *    NULL = none, and the calls then behave exactly as the plain ones): the
 *    complex state entering every 128-step chunk, (batch, dim,
 *    ceil(seqlen/128), dstate) interleaved (re, im) float32 pairs,
 *    mamba_scan_complex_checkpoint_size bytes, 16-byte aligned.  A backward
 *    given the buffer skips its state-recompute pass and needs only the
 *    workspace's segment buffers (none in one pass: workspace may then be
 *    NULL, workspace_bytes 0).  The backward still replays
 *    every state inside each chunk from its checkpoint (paper-graph-ui
 *    summary, section 3.4, and trishampatil essay, Part III §4: only the
 *    chunk-boundary states are kept).  Checkpoints must come from a forward
 *    over the same inputs.
 *  - segments: as for the real _ex calls (0 = automatic, 1 = one pass, k =
 *    k segments of whole chunks); explicit segments need the workspace the
 *    _ex size queries report for the same count (MAMBA_ERR_WORKSPACE
 *    otherwise).
 *  - reset (nullable, (batch, seqlen) bytes): packed sequences, as for
 *    mamba_scan_fwd_varlen / mamba_scan_bwd_varlen: the complex state
 *    entering each flagged step is zero (and no gradient passes back across
 *    it).
 */
size_t mamba_scan_complex_checkpoint_size(int64_t batch, int64_t dim, int64_t dstate,
                                          int64_t seqlen);

size_t mamba_scan_fwd_complex_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                                int64_t seqlen, int segments);

size_t mamba_scan_bwd_complex_workspace_size_ex(int64_t batch, int64_t dim, int64_t dstate,
                                                int64_t seqlen, int segments);

mamba_status mamba_scan_fwd_complex_ex(const void* u, const void* delta, const float* A,
                                       const float* B, const float* C, const float* D,
                                       const void* z, const float* delta_bias, const float* h0,
                                       const uint8_t* reset, int delta_softplus, mamba_disc disc,
                                       mamba_dtype dt,
                                       int64_t batch, int64_t dim, int64_t dstate,
                                       int64_t seqlen, void* out, float* last_state,
                                       float* checkpoints, void* workspace,
                                       size_t workspace_bytes, void* stream, int segments);

mamba_status mamba_scan_bwd_complex_ex(const void* u, const void* delta, const float* A,
                                       const float* B, const float* C, const float* D,
                                       const void* z, const float* delta_bias, const float* h0,
                                       const void* dout, const uint8_t* reset,
                                       int delta_softplus, mamba_disc disc,
                                       mamba_dtype dt, int64_t batch, int64_t dim,
                                       int64_t dstate, int64_t seqlen, float* du, float* ddelta,
                                       float* dA, float* dB, float* dC, float* dD, float* dz,
                                       float* ddelta_bias, float* dh0, const float* checkpoints,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       int segments);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H_ */
