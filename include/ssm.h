/*
 * ssm.h - C ABI of the MI355X (gfx950) selective-scan library (libssm.so).
 *
 * The operation is Mamba's selective state-space scan.  For batch b, time t,
 * channel d and state n:
 *
 *   Delta[b,t,d] = softplus(delta[b,t,d] + delta_bias[d])   (or without softplus)
 *   h[b,t,d,n]   = exp(Delta * A[d,n]) * h[b,t-1,d,n] + Delta * B[b,t,n] * u[b,t,d]
 *   y[b,t,d]     = (sum_n C[b,t,n] * h[b,t,d,n] + Dskip[d] * u[b,t,d]) * silu(z[b,t,d])
 *
 * with h[b,-1] = 0 and silu(z) = z / (1 + exp(-z)).  Sources: the recurrence and
 * its readout follow the "Selective scan pseudo-code" of the interview-prep
 * page on Mamba (vanos001.github.io) and the "Mamba selective" listing of the
 * slide deck (brendanjameslynskey.github.io, Arch_02_Mamba_SSM): decay
 * exp(Delta*A), input term Delta*B (the simplified zero-order hold).  The
 * softplus of a biased projection is that page's "Discretization and
 * initialization details"; the skip term D*u is the deck's S4 output equation;
 * the SiLU(z) gate is the lecture notes' §6 "The block".
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HBM), row-major, densely packed.
 *  - Activations (u, delta, z, y, B, C) use the activation dtype `dt`:
 *    SSM_F32 = float32, SSM_BF16 = bfloat16 (raw 16-bit patterns; y is
 *    rounded to nearest even).  Parameters A, Dskip, delta_bias and every
 *    state buffer are always float32.  Arithmetic is float32.
 *  - Calls are asynchronous and stream-ordered on `stream` (a hipStream_t;
 *    NULL = the null stream).  They never synchronise.  Argument errors are
 *    returned before anything is enqueued and leave outputs untouched.
 *    Device faults surface at the caller's next synchronisation.
 *  - The library never allocates or frees device memory; the caller owns
 *    every buffer.  NaN/Inf inputs are not checked and propagate.
 *  - Results are deterministic: same inputs, shapes and device give
 *    bitwise-identical outputs.
 *  - Alignment: every pointer must be aligned to its element size.  16-byte
 *    aligned pointers and L a multiple of 8 select the vectorised scan; other
 *    shapes run a slower path with the same results.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = 1,  /* null required pointer, negative size, misalignment, aliasing */
  SSM_ERR_UNSUPPORTED = 2,  /* N outside [1, 64], unknown dtype or variant */
  SSM_ERR_HIP = 3,          /* no usable device, launch failure, or missing gfx950 code */
  SSM_ERR_TOO_LARGE = 4     /* the call needs more scratch than the allocation-free entry point holds */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

#define SSM_MAX_N 64
#define SSM_MAX_CONV_WIDTH 4

/*
 * Selective scan, forward (prefill / training forward): the interview-prep page's
 * "Selective scan pseudo-code" (inputs u, Delta, A, B, C; B_t and C_t of shape
 * (L, N) per sequence) with the D skip term, the SiLU(z) gate and the biased
 * softplus of Delta described above.
 *
 *   u, delta, z  : [batch][D][L] act   (each channel's time series is contiguous)
 *   A            : [D][N] float32      (the diagonal state matrix, one row per channel)
 *   Bm, Cm       : [batch][L][N] act   (the pages' order: a token's N values are
 *                                       contiguous; shared by all D channels of a row)
 *   Dskip        : [D] float32 or NULL (NULL means 0)
 *   z            : NULL means no gate
 *   delta_bias   : [D] float32 or NULL (NULL means 0); added before the softplus
 *   delta_softplus: 0 or 1
 *   y            : out [batch][D][L] act
 *   final_state  : out [batch][D][N] float32, h[b, L-1, d, :], or NULL
 *   batch, L, D  : >= 0 (a zero size is a no-op; with L == 0 the final state is 0)
 *   N            : 1..64
 *   workspace    : device scratch owned by the caller, 16-byte aligned, of
 *                  workspace_bytes >= ssm_selective_scan_workspace_size(...) bytes;
 *                  may be NULL when that size is 0.  Its contents on entry do not
 *                  matter and on return are unspecified; calls sharing one
 *                  workspace must not overlap in time.
 *
 * The pages write u, Delta and z as (batch, L, D); the library stores them
 * channel-major, [batch][D][L], so that each channel's series is read as coalesced
 * vectors along L.  The values are the same.
 *
 * Errors: SSM_ERR_INVALID_ARG for a NULL required pointer, a negative size, a
 * misaligned pointer, y / final_state overlapping any input or each other, or a
 * workspace that is too small, misaligned or overlaps another argument;
 * SSM_ERR_UNSUPPORTED for N outside [1, 64] or a bad dtype; SSM_ERR_HIP when no
 * device is usable or the launch fails.
 */
ssm_status ssm_selective_scan_fwd(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    void *y, float *final_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Bytes of workspace a forward scan (ssm_selective_scan_fwd, _from_state, _variant)
 * of this shape needs; 0 when it needs none (then workspace may be NULL).  Every
 * kernel of this version walks a channel's whole sequence in one wave and keeps its
 * carry in registers, so the size is 0 for every shape; callers that pass the
 * queried size keep working when a shape starts to use one.  Returns 0 for invalid
 * sizes or dtypes (the scan call reports those).  Host-only: touches no device.
 */
size_t ssm_selective_scan_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt);

/*
 * The same scan started from a given state instead of zero: h[b, -1, d, :] =
 * initial_state[b, d, :] (the lecture notes' §2.1 solves the system from a zero
 * initial state; this takes any).  Scanning a sequence in pieces, each piece
 * from the previous piece's final state, gives the result of one scan over the
 * whole sequence: chunked prefill, the carry step of a sequence split across
 * devices, and the state-level prefix reuse of the interview-prep page's
 * "Common Pitfalls" (the state after a shared prefix is resumed).
 *
 *   initial_state : [batch][D][N] float32, or NULL (= zero, as ssm_selective_scan_fwd)
 *   final_state   : may be the same pointer as initial_state (updated in place)
 *                   but must not otherwise overlap it
 * Other arguments and errors as for ssm_selective_scan_fwd; with L == 0 the
 * final state is the initial state.
 */
ssm_status ssm_selective_scan_fwd_from_state(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, void *y, float *final_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Same operation with an explicit kernel choice, for testing that every
 * implementation agrees: SSM_SCAN_AUTO picks the fastest valid one (measured: the
 * token-sequential kernel for N == 16 from 32768 channels batch * D; else the
 * chunked kernel; else the sequential one);
 * SSM_SCAN_SEQUENTIAL runs one thread per (b, d) channel stepping through time
 * (the plain recurrence); SSM_SCAN_CHUNKED runs the chunked wave-scan kernel
 * (returns SSM_ERR_UNSUPPORTED when the shape does not fit it); SSM_SCAN_TOKSEQ
 * runs the token-sequential kernel, whose lanes own states and walk the tokens in
 * order (N == 16, L % 8 == 0, 16-byte aligned activations, B and C; else
 * SSM_ERR_UNSUPPORTED).  `tokens_per_lane` (0 = default) selects the chunked
 * kernel's tokens per lane (8, 12 or 16; 12 is built without the full ZOH and the
 * fused conv), and for SSM_SCAN_TOKSEQ the states per lane (4 or 2).  Other arguments as in ssm_selective_scan_fwd_from_state.
 */
typedef enum {
  SSM_SCAN_AUTO = 0,
  SSM_SCAN_SEQUENTIAL = 1,
  SSM_SCAN_CHUNKED = 2,
  SSM_SCAN_TOKSEQ = 3,
  /* Flag, OR-ed into any of the above: allow the arithmetic-progression decay path.
   * With it, the bfloat16 scan kernels with N == 16 and the simplified input term
   * (the chunked kernel in its 12-wave vector-load form, the token-sequential kernel
   * at 4 states per lane) check each channel's A row and, where it is an exact
   * non-increasing arithmetic progression, A[d, n] == A[d, 0] + n * b in float32 with
   * b = A[d, 1] - A[d, 0] <= 0 (the S4D-real -(n+1) and the HiPPO-derived -(2n+1)
   * rows of the interview-prep page's "Discretization and initialization details"),
   * form exp(Delta A[d, n]) as exp(Delta A[d, n0]) * exp(Delta b)^(n - n0) with
   * n - n0 < 8: multiplies in place of most exponentials, within a few float32
   * roundings of the direct values.  Other rows, other kernels, float32 and the full
   * zero-order hold compute every exp(Delta A) directly (the general path), as every
   * call without the flag does. */
  SSM_SCAN_AP = 16
} ssm_scan_variant;

ssm_status ssm_selective_scan_fwd_variant(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, void *y, float *final_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
    void *workspace, size_t workspace_bytes, void *stream,
    int variant, int tokens_per_lane);

/*
 * The kernel a forward scan of this shape (L > 0) with 16-byte-aligned buffers runs:
 * SSM_SCAN_SEQUENTIAL, SSM_SCAN_CHUNKED or SSM_SCAN_TOKSEQ; or a negative
 * ssm_status when such a call would be rejected.  `gate` nonzero when z is given;
 * `zoh` nonzero for ssm_selective_scan_fwd_zoh, `conv_width` > 0 for
 * ssm_selective_scan_fwd_conv (those two take variant SSM_SCAN_AUTO only);
 * otherwise the call is ssm_selective_scan_fwd_variant(variant, tokens_per_lane).
 * Host-only: touches no device.
 */
int ssm_selective_scan_fwd_kernel(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt, int gate, int zoh,
                                  int conv_width, int variant, int tokens_per_lane);

/*
 * One recurrent decode step (the O(1)-state generation mode): advances the
 * state of `batch` sequences by one token with the same arithmetic as one step
 * of the scan, started from state_in instead of zero.  This is the recurrent
 * mode of the slide deck's introduction and "Where SSMs win" section (one state
 * update of fixed size per generated token, no cache that grows with the
 * sequence) and of the lecture notes' §5 "Inference": h_t = exp(Delta A) h_{t-1}
 * + Delta B_t u_t, y_t = C_t h_t (+ D u_t, gated as above).
 *
 *   state_in     : [batch][D][N] float32
 *   state_out    : [batch][D][N] float32; may equal state_in (in place) but must
 *                  not partially overlap it
 *   u_t, delta_t, z_t : [batch][D] act (z_t NULL = no gate)
 *   A            : [D][N] float32
 *   B_t, C_t     : [batch][N] act
 *   Dskip, delta_bias : [D] float32 or NULL
 *   y_t          : out [batch][D] act
 *
 * Errors as for the scan; y_t overlapping any input or the state is invalid.
 */
ssm_status ssm_state_update(
    const float *state_in, float *state_out,
    const void *u_t, const void *delta_t, const float *A,
    const void *B_t, const void *C_t,
    const float *Dskip, const void *z_t, const float *delta_bias, int delta_softplus,
    void *y_t,
    int64_t batch, int64_t D, int64_t N, ssm_dtype dt, void *stream);

/*
 * The scan and the decode step with the full zero-order-hold discretization: the
 * input term is (exp(Delta*A) - 1)/A * B * u instead of Delta * B * u, the
 * (Delta A)^-1 (exp(Delta A) - I) Delta B of the slide deck's S4 section and the
 * lecture notes' §3 "Discretisation" for a diagonal A (the exact step of
 * x' = A x + B u with u and B held for a time Delta).  The decay exp(Delta*A), the
 * readout, the skip term and the gate are unchanged.
 *
 * Arguments, layouts, outputs and errors as in ssm_selective_scan_fwd_from_state
 * (without a workspace) and ssm_state_update.  A state with A[d, n] == 0 takes the
 * term's limit Delta * B * u (the simplified term: with no decay the state
 * integrates its input).  The scan runs the chunked kernel at 8 tokens per lane or,
 * from 32768 channels with N == 16, the token-sequential kernel.
 */
ssm_status ssm_selective_scan_fwd_zoh(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, void *y, float *final_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt, void *stream);

ssm_status ssm_state_update_zoh(
    const float *state_in, float *state_out, const void *u_t, const void *delta_t,
    const float *A, const void *B_t, const void *C_t,
    const float *Dskip, const void *z_t, const float *delta_bias, int delta_softplus,
    void *y_t,
    int64_t batch, int64_t D, int64_t N, ssm_dtype dt, void *stream);

/*
 * Causal depthwise convolution along L, optionally followed by SiLU: the branch of
 * the Mamba block in front of the selective scan (dileepadev "Mamba
 * Architecture", SSM block internals: depthwise conv, then SiLU, then the SSM;
 * vanos001 "The Mamba Block" and its model card's d_conv = 4).
 *
 *   out[b,d,t] = act( sum_{k<K} conv_w[d,k] * x[b,d,t-K+1+k] + conv_b[d] ),  x = 0 before t = 0
 *
 *   x, out       : [batch][D][L] act (distinct buffers)
 *   conv_w       : [D][K] float32; conv_w[d, K-1] weighs the current token
 *   conv_b       : [D] float32 or NULL (= 0)
 *   conv_width K : 1..SSM_MAX_CONV_WIDTH
 *   apply_silu   : 1 = SiLU(z) = z / (1 + e^-z) on the result, 0 = none
 * Errors: SSM_ERR_INVALID_ARG for NULL required pointers, negative sizes,
 * misalignment or out overlapping an input; SSM_ERR_UNSUPPORTED for K outside
 * 1..4 or a bad dtype; SSM_ERR_HIP when no device is usable or the launch fails.
 */
ssm_status ssm_causal_conv1d_fwd(
    const void *x, const float *conv_w, const float *conv_b, int64_t conv_width, int apply_silu,
    void *out, int64_t batch, int64_t D, int64_t L, ssm_dtype dt, void *stream);

/*
 * The scan with the causal conv1d + SiLU of ssm_causal_conv1d_fwd applied to its
 * input on the fly: u = SiLU(conv(x)) is computed inside the scan kernel, so the
 * block's input branch reads x once instead of writing and re-reading u.
 *
 *   x            : [batch][D][L] act, the conv input (in place of u)
 *   conv_w, conv_b, conv_width : as in ssm_causal_conv1d_fwd
 *   u_out        : [batch][D][L] act, receives u (what a backward pass needs), or NULL
 *   tokens_per_lane : 0 (default), 8 or 16
 * Other arguments, outputs and errors as in ssm_selective_scan_fwd_from_state
 * (initial_state may be NULL).  The convolution starts from zeros at t = 0.
 */
ssm_status ssm_selective_scan_fwd_conv(
    const void *x, const float *conv_w, const float *conv_b, int64_t conv_width,
    const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, void *u_out, void *y, float *final_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt, void *stream, int tokens_per_lane);

/*
 * Selective scan, backward pass: the gradients of
 *     loss = sum(dy * y) + sum(dfinal_state * final_state)
 * for (y, final_state) = ssm_selective_scan_fwd_from_state(...) with the same
 * inputs.  The forward states are recomputed from the inputs, not stored (the
 * recomputation of the slide deck on Mamba's fused kernel and of the "Hardware-
 * Aware Parallel Scan" sections of the dileepadev and vanos001 pages); the state
 * gradient is the same recurrence run backwards in time,
 *     lam_t = dy_t silu(z_t) C_t + exp(Delta_{t+1} A) lam_{t+1},
 * scanned with the forward pass's associative operator (the slide deck's
 * "Parallel scan" section).
 *
 * Inputs (as in ssm_selective_scan_fwd_from_state): u, delta, A, Bm, Cm, Dskip,
 * z, delta_bias, delta_softplus, initial_state (NULL = zero), and
 *   dy            : [batch][D][L] act, the gradient of y
 *   dfinal_state  : [batch][D][N] float32, the gradient of the final state, or NULL (= 0)
 * Outputs (each overwritten, never accumulated into):
 *   du, ddelta    : [batch][D][L] act; ddelta is w.r.t. the raw delta (before bias and softplus)
 *   dA            : [D][N] float32
 *   dB, dC        : [batch][L][N] act (the layout of B and C)
 *   dD            : [D] float32 or NULL (not computed); the gradient at Dskip (0 if Dskip is NULL)
 *   dz            : [batch][D][L] act or NULL; must be NULL when z is NULL
 *   ddelta_bias   : [D] float32 or NULL; the gradient at delta_bias (0 if NULL)
 *   dinitial_state: [batch][D][N] float32 or NULL; the gradient at the initial state
 * Workspace: `workspace_bytes` >= ssm_selective_scan_bwd_workspace_size(...)
 * bytes of device memory, 16-byte aligned, owned by the caller; its contents on
 * entry do not matter and on return are unspecified.  Calls that share a
 * workspace must not overlap in time.
 *
 * Determinism: every output, including the sums over channels (dB, dC, dA, dD,
 * ddelta_bias), is formed in a fixed order and is bitwise reproducible.
 * Errors: SSM_ERR_INVALID_ARG for a NULL required pointer (u, delta, A, Bm, Cm,
 * dy, du, ddelta, dA, dB, dC, workspace where the size is nonzero), a negative
 * size, misalignment, a too-small workspace, dz without z, or any output
 * overlapping an input, another output or the workspace; SSM_ERR_UNSUPPORTED for
 * N outside [1, 64] or a bad dtype; SSM_ERR_HIP when no device is usable or a
 * launch fails.  With L == 0 the sums (dA, dD, ddelta_bias) are zero and
 * dinitial_state = dfinal_state.
 */
size_t ssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt);

ssm_status ssm_selective_scan_bwd(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, const void *dy, const float *dfinal_state,
    void *du, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
    float *ddelta_bias, float *dinitial_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training pair with saved chunk states: a forward scan that also stores the state
 * entering every SSM_SAVE_CHUNK-token chunk, and a backward pass that reads those
 * states instead of recomputing them.  The recomputation trade of the slide deck on
 * Mamba's fused kernel (keep the inputs, rebuild the states) is kept inside each
 * chunk; across chunks the backward pass starts from the stored states, so it no
 * longer needs a pass over the whole sequence to find them.  The stored states are
 * batch * D * ceil(L / 512) * N floats: at N = 16 a sixteenth of the size of u in
 * bfloat16 (8 MB for batch 8, D 4096, L 2048).
 *
 * ssm_selective_scan_fwd_save: as ssm_selective_scan_fwd_from_state (same inputs,
 * outputs and errors), plus
 *   chunk_states : out [batch][D][ceil(L / SSM_SAVE_CHUNK)][N] float32, 16-byte
 *                  aligned, owned by the caller; entry c is the state entering
 *                  token c * SSM_SAVE_CHUNK (entry 0: initial_state, or zeros).
 *                  NULL is invalid for a nonempty call; it must not overlap any
 *                  other buffer.
 * N above 16 is SSM_ERR_UNSUPPORTED.  y and final_state are the ones
 * ssm_selective_scan_fwd_from_state gives (the same kernels' arithmetic; the
 * chunked kernel runs at 8 tokens per lane).
 *
 * ssm_selective_scan_bwd_saved: as ssm_selective_scan_bwd (same inputs, outputs,
 * determinism and errors), plus
 *   chunk_states : [batch][D][ceil(L / SSM_SAVE_CHUNK)][N] float32, what
 *                  ssm_selective_scan_fwd_save wrote for these same inputs (the
 *                  call cannot check this; other contents give wrong gradients).
 *                  NULL is invalid for a nonempty call.
 * Workspace: ssm_selective_scan_bwd_saved_workspace_size(...) bytes.  With
 * N <= 16 and batch * D >= 16384 (enough channels to fill the device without
 * splitting the sequence) the pass walks each channel's chunks from the last to
 * the first, one read of every input; other shapes ignore chunk_states and run the
 * ssm_selective_scan_bwd decomposition.  The gradients match ssm_selective_scan_bwd's
 * to float32 rounding (the states are summed in a different order), not bitwise.
 */
#define SSM_SAVE_CHUNK 512

ssm_status ssm_selective_scan_fwd_save(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, void *y, float *final_state, float *chunk_states,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
    void *workspace, size_t workspace_bytes, void *stream);

size_t ssm_selective_scan_bwd_saved_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt);

ssm_status ssm_selective_scan_bwd_saved(
    const void *u, const void *delta, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const void *z, const float *delta_bias, int delta_softplus,
    const float *initial_state, const void *dy, const float *dfinal_state, const float *chunk_states,
    void *du, void *ddelta, float *dA, void *dB, void *dC, float *dD, void *dz,
    float *ddelta_bias, float *dinitial_state,
    int64_t batch, int64_t L, int64_t D, int64_t N, ssm_dtype dt,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Mamba-2 SSD scan: a scalar decay per head (the slide deck's "Mamba-2" table; the
 * interview-prep page's "Mamba-2 and State Space Duality").  For batch b, time t,
 * head h, head channel p and state n:
 *
 *   Delta[b,t,h] = softplus(dt[b,t,h] + dt_bias[h])    (or without softplus)
 *   H[b,t,h,p,n] = exp(Delta*A[h]) * H[b,t-1,h,p,n] + Delta * x[b,t,h,p] * B[b,t,n]
 *   y[b,t,h,p]   = sum_n C[b,t,n] * H[b,t,h,p,n] + Dskip[h] * x[b,t,h,p]
 *
 * computed in its chunk-parallel form on the matrix cores (chunks of 64 tokens: the
 * masked quadratic form inside a chunk, the P x N state carried between chunks).
 *
 *   x, y          : [batch][L][H][P] bf16 (the pages' (batch, L, D) order, D = H*P)
 *   dt            : [batch][L][H] bf16 (raw; bias and softplus applied inside)
 *   A             : [H] float32 (nonpositive in the models)
 *   Bm, Cm        : [batch][L][N] bf16, shared by all heads
 *   Dskip, dt_bias: [H] float32 or NULL (= 0)
 *   initial_state : [batch][H][P][N] float32 or NULL (= 0)
 *   final_state   : out [batch][H][P][N] float32 or NULL; may be the initial_state
 *                   pointer (updated in place) but must not otherwise overlap it
 * Supported: dtype SSM_BF16, P == 64, N in {64, 128}, H <= 65536 (SSM_ERR_UNSUPPORTED
 * otherwise).
 * x, y, Bm, Cm, the states and the workspace must be 16-byte aligned.  The products
 * run in bfloat16 with float32 accumulation and a float32 state (the carried-state
 * product uses the state as two bfloat16 terms); y is rounded to bfloat16.
 *
 * Workspace: with workspace_bytes >= ssm_ssd_scan_workspace_size(...) (owned by the
 * caller, contents irrelevant) the sequences are cut into segments that run in
 * parallel (a pre-pass computes each segment's end state); with NULL / 0 each
 * sequence runs as one segment (slower at few heads x batch rows, same results up to
 * rounding).  A size query of 0 means no workspace helps for that shape.
 * Errors as for ssm_selective_scan_fwd; also SSM_ERR_INVALID_ARG for a workspace
 * overlapping any other argument.  Deterministic for a given workspace size.
 */
size_t ssm_ssd_scan_workspace_size(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, ssm_dtype dtype);

ssm_status ssm_ssd_scan_fwd(
    const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const float *dt_bias, int dt_softplus,
    const float *initial_state, void *y, float *final_state,
    int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, ssm_dtype dtype,
    void *workspace, size_t workspace_bytes, void *stream);

/*
 * The SSD scan for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same operation,
 * arguments (without the workspace), layouts, errors and results as ssm_ssd_scan_fwd
 * given a workspace of ssm_ssd_scan_workspace_size(...) bytes: the segment states
 * live in a library-owned
 * device array of SSM_SSD_NOALLOC_SCRATCH_BYTES per GPU (allocated when the library's
 * code is loaded on that GPU, held until the process ends), so the call allocates
 * nothing.  A shape whose workspace size exceeds that array returns SSM_ERR_TOO_LARGE
 * (no supported shape does: the segment rule keeps it under ~51 MB).  The first call
 * on a device looks up the array's address there (thread-safe).  Calls on one GPU
 * share the array: two calls that overlap in time on the same GPU (on different
 * streams, or captured into graphs that run concurrently) race on it and give wrong
 * results; calls in one stream order are safe.  Nothing in the array needs clearing:
 * each call writes every entry it reads.
 */
#define SSM_SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

ssm_status ssm_ssd_scan_fwd_noalloc(
    const void *x, const void *dt, const float *A, const void *Bm, const void *Cm,
    const float *Dskip, const float *dt_bias, int dt_softplus,
    const float *initial_state, void *y, float *final_state,
    int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, ssm_dtype dtype, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *ssm_status_string(ssm_status s);

/* Library version as major * 10000 + minor * 100 + patch. */
int ssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
