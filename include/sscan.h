/*
 * sscan.h -- C ABI of the MI355X (gfx950) selective scan (S6) library, libsscan.so.
 *
 * The operation (pages: "The loop that beats attention" eqs. (1)-(2) and
 * "Selectivity" eq. (4); "Mamba and State Space Models", "Mamba: making the
 * state selective"; "State space models and Mamba", continuous form with D;
 * "Mamba matches the Transformer...", "Selection makes the recurrence read
 * the token" and "The scan that pays for selection"):
 *
 *   for every batch row b, channel d and state n, with h = 0 before token 0:
 *     Abar  = exp(delta[b,t,d] * A[d,n])                       zero-order hold
 *     Bbar  = (exp(delta*A[d,n]) - 1) / A[d,n] * B[b,t,n]        (delta*B when A = 0)
 *     h[n]  = Abar * h[n] + Bbar * x[b,t,d]                     linear recurrence
 *     y[b,t,d] = sum_n C[b,t,n] * h[n] + Dskip[d] * x[b,t,d]    readout + skip
 *
 * delta, x are per (b, t, d); B, C per (b, t, n), shared by every channel;
 * A is diagonal per channel, (dim, N).  The per-token Abar/Bbar tensor of
 * shape (batch, L, dim, N) is never written to memory.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers (hipMalloc / torch CUDA tensors) owned by the
 *     caller.  The library keeps no reference after the call returns, except
 *     that the enqueued work reads and writes them until it completes.
 *   - All arrays are dense, row-major, contiguous, naturally aligned for their
 *     element type.  io_dtype selects the element type of x, delta, B, C, y
 *     (and of x_t, delta_t, B_t, C_t, y_t); A, Dskip and states are always fp32.
 *     bf16 outputs are rounded to nearest, ties to even.  All arithmetic and the
 *     state are fp32.
 *   - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t; NULL
 *     is the default stream) and the call returns.  Errors found while the
 *     kernels run surface at the caller's next synchronisation.
 *   - Arguments are validated before anything is enqueued; on a validation error
 *     nothing is touched and a negative status is returned.  There is no fallback
 *     path of any kind: the kernels below run, or the call fails.
 *   - Values are not checked: delta <= 0, A >= 0, NaN and Inf are computed by the
 *     formula and propagate (A > 0 grows, as an eigenvalue above 1 would).
 *   - Any tensor with zero elements may be passed as NULL.
 *   - Calls on different streams may run concurrently; each call owns the
 *     stream-ordered scratch memory it allocates (hipMallocAsync) and frees it on
 *     the same stream.  The exception is sscan_forward_noalloc, which allocates
 *     nothing and shares one static scratch array per GPU among its calls.
 */
#ifndef SSCAN_H
#define SSCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSCAN_ABI_VERSION 1
#define SSCAN_MAX_DSTATE 16 /* N = 1 .. 16 */
#define SSCAN_MAX_DCONV 4   /* front-end convolution width d_conv = 1 .. 4 */

/* Activation after the front-end convolution. */
#define SSCAN_ACT_NONE 0
#define SSCAN_ACT_SILU 1

typedef enum { SSCAN_F32 = 0, SSCAN_BF16 = 1 } sscan_dtype;

typedef enum {
    SSCAN_OK = 0,
    SSCAN_ERR_NULL = -1,        /* a required pointer is NULL (its tensor is non-empty) */
    SSCAN_ERR_SHAPE = -2,       /* a size is negative, or a byte size overflows int64   */
    SSCAN_ERR_UNSUPPORTED = -3, /* dstate outside 1..SSCAN_MAX_DSTATE, bad io_dtype, or a
                                   shape beyond a launch limit (see sscan_forward_plan) */
    SSCAN_ERR_ALIAS = -4,       /* an output overlaps an input or another output         */
    SSCAN_ERR_HIP = -5          /* a HIP call (allocation, launch) failed; see last error */
} sscan_status;

/*
 * Whole-sequence forward pass (prefill / training forward).
 *
 *   x, delta     [in]  (batch, seqlen, dim), io_dtype.  delta is the step size
 *                      after its softplus (the pages' Delta_t), not the raw projection.
 *   A            [in]  (dim, dstate) fp32, the diagonal continuous-time A.
 *   B, C         [in]  (batch, seqlen, dstate), io_dtype.
 *   Dskip        [in]  (dim) fp32, or NULL for no skip term.
 *   y            [out] (batch, seqlen, dim), io_dtype.  Must not overlap any input.
 *   final_state  [out] (batch, dim, dstate) fp32 state after the last token, or NULL.
 *                      With seqlen == 0 it receives zeros.  Same layout as the
 *                      `state` of sscan_step, so a prefill hands over directly.
 *   batch, seqlen, dim >= 0; 1 <= dstate <= SSCAN_MAX_DSTATE.
 *   stream       hipStream_t to enqueue on.
 * Returns SSCAN_OK or a negative sscan_status.
 */
int sscan_forward(const void *x, const void *delta, const float *A, const void *B, const void *C,
                  const float *Dskip, void *y, float *final_state, int64_t batch, int64_t seqlen,
                  int64_t dim, int64_t dstate, int io_dtype, void *stream);

/*
 * Whole-sequence forward pass that starts from a given state instead of zero:
 * resuming a sequence from a snapshot, or prefilling it in pieces ("Mamba and
 * State Space Models", failure mode 2: an SSM resumes a shared prefix by
 * snapshotting and restoring its state).  Running [0, L1) with sscan_forward and
 * then [L1, L) with this call from the first call's final_state gives the same
 * result as one call over [0, L), up to rounding.
 *
 *   initial_state [in] (batch, dim, dstate) fp32 state h before the first token, or
 *                      NULL for zero (then identical to sscan_forward).  It may not
 *                      overlap final_state or any other argument (use two buffers).
 *   All other arguments as for sscan_forward.  With seqlen == 0 final_state
 *   receives a copy of initial_state.
 */
int sscan_forward_from_state(const void *x, const void *delta, const float *A, const void *B,
                             const void *C, const float *Dskip, const float *initial_state,
                             void *y, float *final_state, int64_t batch, int64_t seqlen,
                             int64_t dim, int64_t dstate, int io_dtype, void *stream);

/*
 * sscan_forward_from_state for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  It makes no allocation of any kind (no hipMalloc, hipMallocAsync or
 * hipFree); its scratch (staged B/C rows, tile flags, segment aggregates) is a
 * static array of 64 MiB that the library holds on each GPU it runs on until the
 * process ends.  Every call on one GPU uses that GPU's array: calls that overlap in
 * time on one GPU (on different streams, or from several threads) race and give
 * wrong results; serialise them.  Nothing in the array needs to start at zero.
 *
 *   Arguments and results exactly as for sscan_forward_from_state; on the segment
 *   path it may cut the sequence into fewer segments than sscan_forward_plan
 *   reports, so that their aggregates fit the array (the same result to rounding).
 * Returns SSCAN_ERR_UNSUPPORTED, before anything is enqueued, when the call needs more
 * than 64 MiB of scratch even so (sscan_forward_plan reports the allocating call's
 * scratch_bytes: 128 bytes per (batch row, token) at dstate 9..16, fewer below, plus
 * the segment aggregates of the segment kernels), or SSCAN_ERR_HIP if the array's
 * address cannot be obtained.
 */
int sscan_forward_noalloc(const void *x, const void *delta, const float *A, const void *B,
                          const void *C, const float *Dskip, const float *initial_state, void *y,
                          float *final_state, int64_t batch, int64_t seqlen, int64_t dim,
                          int64_t dstate, int io_dtype, void *stream);

/*
 * One recurrent decode step (generation: constant work and memory per token;
 * "The loop that beats attention", section "Going back to the baton";
 * "State space models and Mamba", cost table, generation per token O(1)).
 *
 *   state        [in/out] (batch, dim, dstate) fp32, h_{t-1} on entry, h_t on
 *                      return; updated in place.  Must not overlap any other argument.
 *   x_t, delta_t [in]  (batch, dim), io_dtype.
 *   A            [in]  (dim, dstate) fp32.
 *   B_t, C_t     [in]  (batch, dstate), io_dtype.
 *   Dskip        [in]  (dim) fp32, or NULL.
 *   y_t          [out] (batch, dim), io_dtype.
 *   batch, dim >= 0; 1 <= dstate <= SSCAN_MAX_DSTATE.
 * Returns SSCAN_OK or a negative sscan_status.
 */
int sscan_step(float *state, const void *x_t, const void *delta_t, const float *A,
               const void *B_t, const void *C_t, const float *Dskip, void *y_t, int64_t batch,
               int64_t dim, int64_t dstate, int io_dtype, void *stream);

/*
 * Backward pass of the whole-sequence scan: gradients of a scalar loss through
 * sscan_forward_from_state, given dLoss/dy and dLoss/d(final_state).  The pages
 * name the backward pass and its recomputation of the states from the inputs
 * ("Mamba and State Space Models", the hardware-aware implementation; "Mamba
 * matches the Transformer...", "Fuse the kernel and recompute"); the formulas
 * are the chain rule through the forward definition above:
 *   lam_t     = C_t dy_t + Abar_{t+1} lam_{t+1}   (lam_{L-1} = C dy + dfinal_state)
 *   dx        = Dskip dy + sum_n lam Bbar           ddelta = sum_n lam (A h_t + B x)
 *   dA[d,n]   = sum_{b,t} lam (delta Abar h_{t-1} + (delta Abar - gain)/A B x)
 *   dB[b,t,n] = sum_d lam gain x                    dC[b,t,n] = sum_d dy h_t
 *   dDskip[d] = sum_{b,t} dy x                      dinitial_state = Abar_0 lam_0
 * with gain = (exp(delta A) - 1)/A (delta when A = 0).  The states are recomputed
 * on chip; nothing from the forward pass is needed.
 *
 *   x, delta, A, B, C, Dskip, initial_state  [in]  as for sscan_forward_from_state
 *                      (Dskip, initial_state may be NULL: zero).
 *   dy           [in]  (batch, seqlen, dim), io_dtype: dLoss/dy.
 *   dfinal_state [in]  (batch, dim, dstate) fp32 dLoss/d(final_state), or NULL (zero).
 *   dx, ddelta   [out] (batch, seqlen, dim), io_dtype.
 *   dA           [out] (dim, dstate) fp32, summed over batch and time.
 *   dB, dC       [out] (batch, seqlen, dstate) fp32 (not io_dtype), summed over channels.
 *   dDskip       [out] (dim) fp32, or NULL if not wanted.
 *   dinitial_state [out] (batch, dim, dstate) fp32, or NULL if not wanted.
 * dim may be at most 2^24 (SSCAN_ERR_UNSUPPORTED above).
 * Outputs are overwritten, not accumulated, and must not overlap any argument.
 * Every sum is taken in a fixed order: results are bitwise reproducible.  With
 * seqlen == 0, dinitial_state receives a copy of dfinal_state (zeros if NULL) and
 * dA, dDskip zeros; with dim == 0, dB and dC are zeros.
 * Scratch (stream-ordered): about 4*dstate*(seqlen/32)*batch*dim bytes of saved
 * states plus 128*batch*seqlen*ceil(dim/64) bytes of dB/dC partials (dstate
 * rounded up to a power of two).
 */
int sscan_backward(const void *x, const void *delta, const float *A, const void *B, const void *C,
                   const float *Dskip, const float *initial_state, const void *dy,
                   const float *dfinal_state, void *dx, void *ddelta, float *dA, float *dB,
                   float *dC, float *dDskip, float *dinitial_state, int64_t batch, int64_t seqlen,
                   int64_t dim, int64_t dstate, int io_dtype, void *stream);

/*
 * Forward pass with the front end fused in: the scan input and the step size are
 * formed inside the scan kernels from their raw forms, so neither is written to or
 * read back from memory.  Step size ("Mamba and State Space Models", the selective
 * pseudocode; knowledge-base entry on Mamba, section 3.2, algorithm 2):
 *     delta[b,t,d] = softplus(delta_raw[b,t,d] + delta_bias[d]),  softplus(v) = log(1 + e^v)
 * Scan input: the short causal convolution in front of the SSM ("Mamba and State
 * Space Models", "How this shows up in practice", d_conv), per channel,
 *     c[b,t,d] = conv_bias[d] + sum_{k<d_conv} conv_weight[d,k] * x[b, t-d_conv+1+k, d]
 *     u[b,t,d] = c (activation SSCAN_ACT_NONE) or c / (1 + e^-c) (SSCAN_ACT_SILU),
 * with the inputs before token 0 taken from conv_state_in.  Then exactly
 * sscan_forward_from_state on (u, delta): y = C.h + Dskip * u.
 *
 *   x              [in]  (batch, seqlen, dim), io_dtype: the convolution's input.
 *   conv_weight    [in]  (dim, d_conv) fp32 (a depthwise conv1d weight without its
 *                        middle axis).
 *   conv_bias      [in]  (dim) fp32, or NULL (0).
 *   d_conv              1 .. SSCAN_MAX_DCONV.
 *   activation          SSCAN_ACT_NONE or SSCAN_ACT_SILU.
 *   conv_state_in  [in]  (batch, d_conv-1, dim), io_dtype: the raw inputs of the
 *                        d_conv-1 tokens before token 0, oldest first; NULL = zeros.
 *   delta_raw      [in]  (batch, seqlen, dim), io_dtype.
 *   delta_bias     [in]  (dim) fp32, or NULL (0).
 *   A, B, C, Dskip, initial_state, y, final_state: as for sscan_forward_from_state.
 *   conv_state_out [out] (batch, d_conv-1, dim), io_dtype, or NULL: the raw inputs of
 *                        the last d_conv-1 tokens (with seqlen < d_conv-1, partly the
 *                        carried ones), the conv_state_in of a following call or of
 *                        sscan_step_fused.  Must not overlap conv_state_in or x.
 * Returns SSCAN_OK or a negative sscan_status (SSCAN_ERR_UNSUPPORTED for a bad
 * d_conv or activation).
 */
int sscan_forward_fused(const void *x, const float *conv_weight, const float *conv_bias, int d_conv,
                        int activation, const void *conv_state_in, const void *delta_raw,
                        const float *delta_bias, const float *A, const void *B, const void *C,
                        const float *Dskip, const float *initial_state, void *y, float *final_state,
                        void *conv_state_out, int64_t batch, int64_t seqlen, int64_t dim,
                        int64_t dstate, int io_dtype, void *stream);

/*
 * One decode step with the front end fused in (the recurrent form of
 * sscan_forward_fused): x_t and delta_raw_t are the raw token inputs.
 *
 *   state          [in/out] as for sscan_step.
 *   conv_state     [in/out] (batch, d_conv-1, dim), io_dtype: the raw inputs of the
 *                        d_conv-1 previous tokens, oldest first; shifted by one token
 *                        in place (x_t appended).  May be NULL only when d_conv == 1.
 *   x_t, delta_raw_t [in] (batch, dim), io_dtype.
 *   conv_weight, conv_bias, d_conv, activation, delta_bias: as for sscan_forward_fused.
 *   A, B_t, C_t, Dskip, y_t, batch, dim, dstate, io_dtype, stream: as for sscan_step.
 */
int sscan_step_fused(float *state, void *conv_state, const void *x_t, const float *conv_weight,
                     const float *conv_bias, int d_conv, int activation, const void *delta_raw_t,
                     const float *delta_bias, const float *A, const void *B_t, const void *C_t,
                     const float *Dskip, void *y_t, int64_t batch, int64_t dim, int64_t dstate,
                     int io_dtype, void *stream);

/*
 * Scalar-A-per-head selective scan (Mamba-2's state space model), computed in its
 * chunked matrix form.  The state space duality ("Mamba and State Space Models";
 * "Mamba matches the Transformer...", the duality section): with A a scalar per
 * head the scan is a lower-triangular structured (semiseparable) matrix applied to
 * x, evaluated here chunk by chunk with dense block products.  Per batch row b,
 * head h, channel p < headdim, state n < dstate, with group g = h / (nheads/ngroups):
 *     Abar = exp(delta[b,t,h] * A[h]),  gain = (Abar - 1)/A[h]   (delta when A[h] = 0)
 *     h[p][n] = Abar * h[p][n] + gain * B[b,t,g,n] * x[b,t,h,p]
 *     y[b,t,h,p] = sum_n C[b,t,g,n] * h[p][n] + Dskip[h] * x[b,t,h,p]
 * (the zero-order hold of sscan_forward, with A[d,n] = A[h] for every state).
 *
 *   x, y          (batch, seqlen, nheads, headdim), io_dtype.
 *   delta         (batch, seqlen, nheads), io_dtype, after its softplus.
 *   A             (nheads) fp32.   Dskip (nheads) fp32 or NULL.
 *   B, C          (batch, seqlen, ngroups, dstate), io_dtype.
 *   initial_state, final_state  (batch, nheads, headdim, dstate) fp32, or NULL.
 *   headdim == 64; dstate 64 or 128; nheads a multiple of ngroups.
 * Products run on the matrix cores with fp32 accumulation: for SSCAN_BF16 on bf16
 * operands, where the operands computed in fp32 (the masked scores, w x and the
 * state) enter as two bf16 parts each (high part + remainder); for SSCAN_F32 on
 * fp32 operands.  The carried state is fp32.
 * Returns SSCAN_OK or a negative sscan_status.
 */
int sscan_ssd_forward(const void *x, const void *delta, const float *A, const void *B, const void *C,
                      const float *Dskip, const float *initial_state, void *y, float *final_state,
                      int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups,
                      int64_t dstate, int io_dtype, void *stream);

/*
 * One decode step of the scalar-A-per-head scan: the recurrence of
 * sscan_ssd_forward for a single token, with the state read and written in place
 * (the state of the duality's recurrent form: "Mamba matches the Transformer...",
 * the duality section; generation at constant work per token, "State space
 * models and Mamba", cost table).  Per batch row b, head h (group g as above):
 *     state[b,h,p,n] = exp(delta A[h]) state[b,h,p,n] + gain B[b,g,n] x[b,h,p]
 *     y[b,h,p] = sum_n C[b,g,n] state[b,h,p,n] + Dskip[h] x[b,h,p]
 * so that running it over the tokens of a sequence from the final_state of a
 * sscan_ssd_forward prefill continues that sequence.
 *
 *   state         [in/out] (batch, nheads, headdim, dstate) fp32.  Must not overlap any
 *                      other argument.
 *   x_t, y_t      (batch, nheads, headdim), io_dtype.
 *   delta_t       (batch, nheads), io_dtype, after its softplus.
 *   A             (nheads) fp32.   Dskip (nheads) fp32 or NULL.
 *   B_t, C_t      (batch, ngroups, dstate), io_dtype.
 *   headdim == 64; dstate 64 or 128; nheads a multiple of ngroups.
 * All arithmetic is fp32 (no matrix instructions: one token is a rank-1 update).
 * Returns SSCAN_OK or a negative sscan_status.
 */
int sscan_ssd_step(float *state, const void *x_t, const void *delta_t, const float *A, const void *B_t,
                   const void *C_t, const float *Dskip, void *y_t, int64_t batch, int64_t nheads,
                   int64_t headdim, int64_t ngroups, int64_t dstate, int io_dtype, void *stream);

/*
 * How sscan_forward (and the _from_state and _fused variants) would split a
 * problem of this shape, computed on the host without touching the GPU: which
 * kernel scans the sequence (either takes tiles of any A), how the sequence is
 * cut, and the device scratch the call allocates.  This makes the chosen path visible to the caller
 * (the pages warn that a benchmark is only meaningful once it is confirmed that
 * the fused kernel is the one running: "Mamba and State Space Models", failure
 * modes).
 *
 * Launch limits, checked here and by every forward call (SSCAN_ERR_UNSUPPORTED
 * beyond them): the kernels address x, delta and y through buffer descriptors
 * with 32-bit offsets, so one token row (dim * element size) may be at most 2^27
 * bytes, and the segment kernels cut the sequence so that a segment's rows span
 * below 2^31 bytes; a launch has fewer than 2^32 work items.
 *
 * Testing hook: with the environment variable SSCAN_FORCE_SEGMENTS=n (n > 0) set,
 * every forward of the process plans the segment path with n segments (at most one
 * per token, at least what the descriptor bound needs), so that one shape can be
 * scanned through differently cut decompositions and the results compared; unset
 * or 0, the plan is automatic.  It is read at each call.
 *
 *   batch, seqlen, dim, dstate, io_dtype  as for sscan_forward.
 *   out          [out] the plan (host memory, caller-owned).
 * Returns SSCAN_OK, or a negative sscan_status with *out zeroed.
 */
#define SSCAN_PLAN_LOCKSTEP 1 /* one workgroup per 64-channel tile over the whole sequence */
#define SSCAN_PLAN_SEGMENT 2  /* one wave per (64-channel tile, time segment): a scan from  */
                              /* zero, a carry of the segment end states, a correction      */
typedef struct {
    int32_t kernel;        /* SSCAN_PLAN_LOCKSTEP or SSCAN_PLAN_SEGMENT                    */
    int32_t segments;      /* time segments per tile (1 for the lockstep kernel)           */
    int64_t seg_len;       /* tokens per segment, the last shorter (lockstep: seqlen)      */
    int64_t tiles;         /* batch * ceil(dim / 64)                                       */
    int64_t chunk_tokens;  /* lockstep: tokens per chunk (waves x run length); else 0      */
    int64_t scratch_bytes; /* device scratch one call allocates (stream-ordered)           */
} sscan_plan_info;
int sscan_forward_plan(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int io_dtype,
                       sscan_plan_info *out);

/* Static text for a status code (never NULL). */
const char *sscan_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). Valid until the
 * next call on this thread. */
const char *sscan_last_error(void);

/* SSCAN_ABI_VERSION of the loaded library. */
int sscan_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSCAN_H */
