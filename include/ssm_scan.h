/*
 * ssm_scan.h -- C ABI of the MI355X (gfx950) selective-scan library
 * (libssmscan.so).
 *
 * The operation is the Mamba selective-scan forward pass as the pages below
 * define it, plus the bare scan of affine pairs it is built on.
 *
 * Pages cited:
 *   [Scan page]    "Hardware-aware parallel associative scan for Mamba"
 *                  (http://www.pwwt.cn/news/6375169/)
 *   [Mamba-2 page] "Mamba (part 2): parallel scan and hardware-aware
 *                  optimisation" (https://scwacadex.pages.dev/posts/blog8_mamba_parallel_scan/)
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller, dense and
 *   row-major in the layouts stated per argument.  The library never frees
 *   or keeps them.  Pointers must be 16-byte aligned.
 * - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *   on it and the call returns without waiting; results are ready when the
 *   stream is.  Faults inside a kernel therefore surface at the caller's
 *   next synchronisation of that stream.
 * - Every argument is validated on the host before any HIP call is made, so
 *   a bad argument never reaches the GPU.
 * - Return value: one of the SSM_* status codes below.  On failure a
 *   description is available from ssm_last_error() on the same thread.
 * - Outputs must not overlap inputs unless an entry point says otherwise.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define SSM_OK           0  /* enqueued successfully */
#define SSM_EINVAL       1  /* null required pointer, size <= 0, misaligned
                               pointer, overlapping output, bad flag value */
#define SSM_EUNSUPPORTED 2  /* valid request this build does not implement
                               (dtype, d_state > 16, too many chunks) */
#define SSM_EHIP         3  /* the HIP runtime reported an error */
#define SSM_ENOMEM       4  /* the two-pass workspace could not be allocated */

/* Storage type of u, delta, B, C, z and y.  A, D, delta_bias and
 * last_state are always float32; all arithmetic is float32. */
#define SSM_F32  0
#define SSM_BF16 1

/* Plans of ssm_scan_fwd_plan. */
#define SSM_PLAN_AUTO    0  /* what ssm_scan_fwd uses (see ssm_scan_plan_for) */
#define SSM_PLAN_CARRY   1  /* one launch; each workgroup carries the state
                               over the whole length L */
#define SSM_PLAN_TWOPASS 2  /* chunk aggregates -> scan over chunks -> fix-up */
#define SSM_PLAN_MIXED   3  /* carry plan in one launch that mixes blocks of two
                               16-channel groups at two states per lane with
                               blocks of one group at one state per lane, so
                               that every SIMD carries the same number of
                               (channel, state) chains when the channel groups
                               number about three per CU */
#define SSM_PLAN_LPAR    4  /* L-parallel single pass: workgroups of 4
                               channels; each tile is cut into 16 time
                               segments (one per lane of a row of 16) that
                               fold thread-serially, are joined by a wave64
                               DPP scan of their (prod a, h) pairs and refold
                               from registers ([Scan page] §2.1, §3.2, §3.3) */

/*
 * ssm_scan_fwd -- selective-scan forward pass ([Scan page] §1.1-§1.2,
 * §2.3; [Mamba-2 page] §2.1 and §4.1).
 *
 * For every batch row b < batch, channel d < d_inner and step t < L, with
 * the state h[b,d,:] starting at zero:
 *     x     = delta[b,d,t] + delta_bias[d]          (delta_bias NULL -> 0)
 *     Delta = softplus(x) if delta_softplus else x
 *     a_n   = exp(Delta * A[d,n])
 *     h_n   = a_n * h_n + Delta * B[b,n,t] * u[b,d,t]
 *     y     = sum_n C[b,n,t] * h_n + D[d] * u[b,d,t] (D NULL -> 0)
 *     y    *= silu(z[b,d,t])                         (z NULL -> no gate)
 *     y[b,d,t] = y  (rounded to nearest even when stored as bfloat16)
 * and last_state[b,d,n] = h_n after step L-1.
 *
 * Arguments (all device pointers):
 *   u, delta, z : [batch, d_inner, L], dtype `dtype`, L contiguous.
 *   A           : [d_inner, d_state] float32 (the diagonal state matrix;
 *                 negative values give decays in (0, 1)).
 *   B, C        : [batch, d_state, L], dtype `dtype`, shared by all channels.
 *   D, delta_bias : [d_inner] float32, nullable.
 *   delta_softplus : 0 or 1.
 *   y           : [batch, d_inner, L], dtype `dtype`, output; must not
 *                 overlap any input.
 *   last_state  : [batch, d_inner, d_state] float32 output, nullable.
 *   batch, d_inner, d_state, L : sizes, all > 0; d_state <= 16.
 *   dtype       : SSM_F32 or SSM_BF16.
 *   stream      : hipStream_t.
 * Errors: SSM_EINVAL (bad pointer/size/flag), SSM_EUNSUPPORTED (dtype,
 * d_state > 16), SSM_EHIP, SSM_ENOMEM (two-pass workspace).
 * The two-pass plan allocates its workspace with hipMallocAsync on `stream`
 * and frees it with hipFreeAsync on the same stream.
 */
int ssm_scan_fwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int delta_softplus,
                 void *y, float *last_state,
                 int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                 int dtype, void *stream);

/*
 * ssm_scan_fwd_noalloc -- ssm_scan_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It calls no hipMalloc, hipFree,
 * hipMallocAsync or other allocating routine: the two-pass plan's workspace
 * (chunk aggregates and chunk start states, 12 * batch * d_inner * d_state
 * * K bytes for K chunks) lives in a fixed per-device scratch array of
 * 8 MiB (8388608 bytes) that the library holds on every GPU it runs on
 * until the process ends.  Its device address is looked up once per device,
 * on the first call with that device current.
 *   Arguments, semantics and results: as ssm_scan_fwd (the same plan, the
 *   same kernels, bit for bit the same outputs).
 *   Errors: as ssm_scan_fwd, plus SSM_EUNSUPPORTED when the plan's
 *   workspace would exceed the scratch (never for the automatic plan, whose
 *   two-pass split stays below 7.1 MB), and SSM_EHIP if the scratch's
 *   address cannot be looked up.
 *   Concurrency: every call on one GPU uses that GPU's one scratch array;
 *   calls whose work overlaps on one GPU (other streams, other host
 *   threads) race on it.  Calls ordered on one stream do not.  Each call
 *   writes every word of the scratch it reads, so nothing needs clearing.
 */
int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A, const void *B, const void *C,
                         const float *D, const void *z, const float *delta_bias, int delta_softplus,
                         void *y, float *last_state,
                         int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                         int dtype, void *stream);

/*
 * ssm_scan_fwd_plan -- ssm_scan_fwd with an explicit plan
 * ([Scan page] §2.2 and §3.3 describe both decompositions).
 *   plan            : SSM_PLAN_AUTO, SSM_PLAN_CARRY, SSM_PLAN_TWOPASS,
 *                     SSM_PLAN_MIXED or SSM_PLAN_LPAR (states_per_lane and
 *                     chunk ignored by the last two).
 *   states_per_lane : how many of the d_state states one lane carries for
 *                     its channel (1, 2 or 4; 0 = automatic).  A workgroup
 *                     covers 16 channels and 16 states with 4/states_per_lane
 *                     wavefronts.
 *   chunk           : two-pass chunk length in steps, a multiple of 64
 *                     (0 = automatic; ignored by the carry plan).
 * Same semantics, arguments and errors as ssm_scan_fwd otherwise; results of
 * the plans agree to float32 rounding, not bit for bit.
 */
int ssm_scan_fwd_plan(const void *u, const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, int delta_softplus,
                      void *y, float *last_state,
                      int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                      int dtype, int plan, int states_per_lane, int64_t chunk, void *stream);

/*
 * ssm_scan_fwd_states -- ssm_scan_fwd from a given start state, keeping the
 * state at every chunk boundary.  Starting from any h_0 is the
 * h_t = A_t h_0 + B_t form of [Scan page] §2.1; the boundary states are the
 * checkpoints that the chunked recomputation of [Mamba-2 page] §4.3 keeps
 * (h_0, h_c, h_2c, ...), from which any chunk can be recomputed alone.
 *   h0           : [batch, d_inner, d_state] float32 start state, nullable
 *                  (zero).  An input: must not overlap any output.
 *   chunk_states : [batch, K, d_inner, d_state] float32 output, nullable,
 *                  K = ceil(L / state_chunk).  Entry k is the state after
 *                  step min((k+1)*state_chunk, L) - 1, so entry K-1 equals
 *                  last_state.
 *   state_chunk  : steps between saved states, a positive multiple of 32
 *                  when chunk_states is given (ignored otherwise).
 *   plan         : as for ssm_scan_fwd_plan (states per lane and chunk are
 *                  chosen automatically).
 * Other arguments, semantics and errors as ssm_scan_fwd.
 */
int ssm_scan_fwd_states(const void *u, const void *delta, const float *A, const void *B, const void *C,
                        const float *D, const void *z, const float *delta_bias, int delta_softplus,
                        const float *h0, void *y, float *last_state, float *chunk_states, int64_t state_chunk,
                        int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype, int plan,
                        void *stream);

/*
 * ssm_scan_plan_for -- the plan, states per lane and chunk length that
 * SSM_PLAN_AUTO picks for a problem size (host only, no HIP call);
 * states per lane is 0 for SSM_PLAN_MIXED (it uses 2 and 1).
 * Any output pointer may be NULL.  Returns SSM_OK or SSM_EINVAL.
 */
int ssm_scan_plan_for(int64_t batch, int64_t d_inner, int64_t d_state, int64_t L, int dtype,
                      int *plan, int *states_per_lane, int64_t *chunk);

/*
 * ssm_scan_fwd_conv -- ssm_scan_fwd_states with the causal depthwise conv1d
 * and SiLU of the Mamba block fused in front of the scan ([Mamba-2 page]
 * §4.1: Conv1D, the SSM scan and SiLU in one kernel so the intermediate
 * never goes to HBM).  The scan's input u is computed in the kernel:
 *     u[b,d,t] = silu(conv_b[d] + sum_{k<K} conv_w[d,k] * x[b,d,t-(K-1)+k]),
 * x at steps before 0 being zero (a causal convolution with K-1 steps of
 * left padding; conv_w[d, K-1] multiplies the current step).
 *   x      : [batch, d_inner, L], dtype `dtype`, the conv's input.
 *   conv_w : [d_inner, conv_k] float32; conv_k = 1 .. 4.
 *   conv_b : [d_inner] float32, nullable (zero).
 *   u_out  : [batch, d_inner, L], dtype `dtype`, output of u, nullable (u is
 *            then never written; it is recomputed from x wherever needed).
 * Other arguments, semantics and errors as ssm_scan_fwd_states (with
 * SSM_EUNSUPPORTED for conv_k outside 1..4).  u enters the scan at float32:
 * with SSM_BF16 it is not rounded to bfloat16 first (u_out is).
 */
int ssm_scan_fwd_conv(const void *x, const float *conv_w, const float *conv_b, int conv_k,
                      const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, int delta_softplus,
                      const float *h0, void *y, float *last_state, void *u_out,
                      float *chunk_states, int64_t state_chunk,
                      int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                      int dtype, int plan, void *stream);

/*
 * ssm_scan_bwd -- gradients of ssm_scan_fwd by chunked recomputation
 * ([Scan page] §4.2: the forward keeps only the state at every chunk
 * boundary, the backward re-runs each chunk from its boundary state and
 * walks it back; [Mamba-2 page] §4.3 on recomputing chunk by chunk).
 * The loss is taken as sum(dy * y) + sum(dlast * last_state), so dy and
 * dlast are the incoming gradients of the forward's outputs.  With
 * s_t = C_t . h_t + D u_t (y = s silu(z), or s without a gate) and
 * g_t = dLoss/dh_t:
 *     gs_t = dy_t silu(z_t);   g_t = C_t gs_t + a_{t+1} g_{t+1},  g_L = dlast
 *     du     = D gs + Delta sum_n g B            ddelta = dDelta * sigmoid(x)
 *     dDelta = u sum_n g B + sum_n g a h_{t-1} A     (without softplus: ddelta = dDelta)
 *     dz     = dy s silu'(z)                     dA[d,n] = sum_{b,t} g a h_{t-1} Delta
 *     dB[b,n,t] = sum_d g Delta u                dC[b,n,t] = sum_d gs h
 *     dD[d]  = sum_{b,t} gs u                    ddelta_bias[d] = sum_{b,t} ddelta
 *     dh0    = a_0 g_0
 *   u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0 : the forward's
 *                  inputs, as for ssm_scan_fwd_states (h0 nullable: zero).
 *   chunk_states : [batch, K, d_inner, d_state] float32, K = ceil(L /
 *                  state_chunk), as written by ssm_scan_fwd_states for the
 *                  same inputs and state_chunk (required).
 *   state_chunk  : a multiple of 32, at most 512.
 *   dy           : [batch, d_inner, L], dtype `dtype`, gradient of y.
 *   dlast        : [batch, d_inner, d_state] float32, gradient of last_state,
 *                  nullable (zero).
 *   du, ddelta   : [batch, d_inner, L], dtype `dtype`, outputs.
 *   dz           : [batch, d_inner, L], dtype `dtype`, output; required if
 *                  and only if z is given.
 *   dA           : [d_inner, d_state] float32 output.
 *   dB, dC       : [batch, d_state, L] float32 outputs (float32 for either
 *                  dtype: they are sums over d_inner channels).
 *   dD, ddelta_bias : [d_inner] float32 outputs, nullable (not computed); the
 *                  gradient is that at the given value, or at zero when D or
 *                  delta_bias is NULL.
 *   dh0          : [batch, d_inner, d_state] float32 output, nullable.
 *   states_per_lane : 1, 2 or 4 (0 = automatic), as for ssm_scan_fwd_plan.
 * Outputs must not overlap each other or any input.  dA, dB, dC, dD and
 * ddelta_bias are sums over workgroups taken with float32 atomic adds: their
 * rounding depends on the order in which workgroups finish, so repeated runs
 * agree to float32 rounding, not bit for bit.  The library clears them on
 * `stream` before accumulating.  No memory is allocated.
 * Errors: SSM_EINVAL (bad pointer, size, flag or state_chunk; overlap;
 * misaligned pointer), SSM_EUNSUPPORTED (dtype, d_state > 16), SSM_EHIP.
 */
int ssm_scan_bwd(const void *u, const void *delta, const float *A, const void *B, const void *C,
                 const float *D, const void *z, const float *delta_bias, int delta_softplus,
                 const float *h0, const float *chunk_states, int64_t state_chunk,
                 const void *dy, const float *dlast,
                 void *du, void *ddelta, float *dA, float *dB, float *dC, float *dD, void *dz,
                 float *ddelta_bias, float *dh0,
                 int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                 int dtype, int states_per_lane, void *stream);

/*
 * ssm_scan_bwd_conv -- gradients of ssm_scan_fwd_conv (the causal conv1d +
 * SiLU fused in front of the scan) by the same chunked recomputation as
 * ssm_scan_bwd.  u = silu(pre) is recomputed from x; with du the scan's
 * gradient of u (as ssm_scan_bwd computes it) and pre_t = conv_b +
 * sum_k conv_w[k] x_{t-(K-1)+k}:
 *     dpre_t = du_t silu'(pre_t),   silu'(p) = sig(p) (1 + p (1 - sig(p)))
 *     dx_t   = sum_k conv_w[k] dpre_{t+(K-1)-k}          (dpre past L is zero)
 *     dconv_w[d,k] = sum_{b,t} dpre_t x_{t-(K-1)+k},  dconv_b[d] = sum_{b,t} dpre_t
 *   x, conv_w, conv_b, conv_k : as for ssm_scan_fwd_conv; chunk_states must
 *                  come from ssm_scan_fwd_conv with the same inputs.
 *   dx           : [batch, d_inner, L], dtype `dtype` (in place of du).
 *   dconv_w      : [d_inner, conv_k] float32 output; dconv_b: [d_inner]
 *                  float32 output, nullable.
 * Other arguments, semantics (sums by float32 atomic adds) and errors as
 * ssm_scan_bwd.
 */
int ssm_scan_bwd_conv(const void *x, const float *conv_w, const float *conv_b, int conv_k,
                      const void *delta, const float *A, const void *B, const void *C,
                      const float *D, const void *z, const float *delta_bias, int delta_softplus,
                      const float *h0, const float *chunk_states, int64_t state_chunk,
                      const void *dy, const float *dlast,
                      void *dx, float *dconv_w, float *dconv_b, void *ddelta, float *dA, float *dB, float *dC,
                      float *dD, void *dz, float *ddelta_bias, float *dh0,
                      int64_t batch, int64_t d_inner, int64_t d_state, int64_t L,
                      int dtype, int states_per_lane, void *stream);

/*
 * ssm_step -- one recurrent step of the selective scan for every (batch,
 * channel): the constant-time inference form of the recurrence
 * ([Mamba-2 page] §7; the step itself is [Scan page] §1.2):
 *     x     = delta[b,d] + delta_bias[d];  Delta = softplus(x) or x
 *     h_n   = exp(Delta * A[d,n]) * h_n + Delta * B[b,n] * u[b,d]
 *     y     = sum_n C[b,n] * h_n + D[d] * u[b,d];  y *= silu(z[b,d])
 * i.e. one step t of ssm_scan_fwd with h taken from state_in.
 *   u, delta, z : [batch, d_inner], dtype `dtype`; z nullable (no gate).
 *   A           : [d_inner, d_state] float32.
 *   B, C        : [batch, d_state], dtype `dtype`.
 *   D, delta_bias : [d_inner] float32, nullable.
 *   state_in    : [batch, d_inner, d_state] float32, the state before the step.
 *   state_out   : [batch, d_inner, d_state] float32, the state after the step;
 *                 may equal state_in (updated in place) or be disjoint from it.
 *   y           : [batch, d_inner], dtype `dtype`, output.
 * Errors as ssm_scan_fwd (d_state <= 16).
 */
int ssm_step(const void *u, const void *delta, const float *A, const void *B, const void *C,
             const float *D, const void *z, const float *delta_bias, int delta_softplus,
             const float *state_in, float *state_out, void *y,
             int64_t batch, int64_t d_inner, int64_t d_state, int dtype, void *stream);

/*
 * ssm_step_conv -- ssm_step with the causal conv1d + SiLU in front, the
 * decode-time form of ssm_scan_fwd_conv: the conv keeps the K-1 previous
 * inputs of every channel as its state.  For every (batch, channel):
 *     window = (conv_state[b,d,0 .. K-2], x[b,d])          oldest first
 *     u      = silu(conv_b[d] + sum_k conv_w[d,k] * window[k])
 *     conv_state <- (window[1 .. K-1])                     x enters, the oldest leaves
 * then the step of ssm_step with u.  T calls over x_1 .. x_T from a zero conv
 * state and a zero SSM state reproduce ssm_scan_fwd_conv over those T steps.
 *   x            : [batch, d_inner], dtype `dtype`.
 *   conv_w       : [d_inner, conv_k] float32, conv_k = 1 .. 4; conv_b: [d_inner]
 *                  float32, nullable.
 *   conv_state_in, conv_state_out : [batch, d_inner, conv_k-1] float32 (unused
 *                  and may be NULL when conv_k = 1); out may equal in (updated
 *                  in place) or be disjoint from it.
 *   u_out        : [batch, d_inner], dtype `dtype`, nullable: u of this step.
 * Other arguments and errors as ssm_step (SSM_EUNSUPPORTED for conv_k outside
 * 1..4).
 */
int ssm_step_conv(const void *x, const float *conv_w, const float *conv_b, int conv_k,
                  const float *conv_state_in, float *conv_state_out,
                  const void *delta, const float *A, const void *B, const void *C,
                  const float *D, const void *z, const float *delta_bias, int delta_softplus,
                  const float *state_in, float *state_out, void *y, void *u_out,
                  int64_t batch, int64_t d_inner, int64_t d_state, int dtype, void *stream);

/*
 * ssm_out_proj -- the Linear projection after the gated scan, the last
 * operator of the fused chain ([Mamba-2 page] §4.1: Conv1D, SSM, SiLU gate,
 * Linear), on the matrix cores:
 *     out[b, t, m] = sum_k W[m, k] * y[b, k, t]
 * with float32 accumulation.  y is read in the layout the scan writes; the
 * result is token-major.
 *   y     : [batch, d_inner, L], dtype `dtype` (the scan's y).
 *   W     : [d_model, d_inner], dtype `dtype` (a Linear layer's weight).
 *   out   : [batch, L, d_model], dtype `dtype`, output (bfloat16 rounded to
 *           nearest even from the float32 sum); must not overlap y or W.
 * Sizes: all positive; each of y's batch rows, W and each of out's batch
 * rows must be under 2^31 bytes (else SSM_EUNSUPPORTED).  Any d_inner, L and
 * d_model are accepted; the fastest path needs d_inner and L multiples of 8
 * (bfloat16) or 4 (float32) and d_model a multiple of 4.
 * Errors: SSM_EINVAL (NULL pointer, size <= 0, misalignment, overlap),
 * SSM_EUNSUPPORTED (dtype, sizes), SSM_EHIP (launch).
 */
int ssm_out_proj(const void *y, const void *W, void *out, int64_t batch, int64_t d_inner, int64_t d_model,
                 int64_t L, int dtype, void *stream);

/*
 * ssm_out_proj_bwd -- gradients of ssm_out_proj for an incoming gradient
 * dout of its output (the chain rule of the same Linear), on the matrix
 * cores with float32 accumulation:
 *     dy[b, k, t] = sum_m W[m, k] * dout[b, t, m]
 *     dW[m, k]    = sum_{b, t} dout[b, t, m] * y[b, k, t]
 *   y     : [batch, d_inner, L], dtype `dtype` (the forward's input).
 *   W     : [d_model, d_inner], dtype `dtype`.
 *   dout  : [batch, L, d_model], dtype `dtype`.
 *   dy    : [batch, d_inner, L], dtype `dtype`, output, nullable (not computed).
 *   dW    : [d_model, d_inner], dtype `dtype`, output, nullable (not computed);
 *           at least one of dy and dW must be given.  dW is summed in a fixed
 *           order, so repeated calls give identical bits.
 * When the d_model x d_inner tiles of dW alone would leave the GPU idle,
 * the sum over batch rows is split over several workgroups whose float32
 * partials sit in a workspace the call allocates and frees stream-ordered
 * (hipMallocAsync / hipFreeAsync; SSM_ENOMEM if that fails).
 * Sizes: as ssm_out_proj, and W in float32 under 2^31 bytes.  Outputs must
 * not overlap the inputs or each other.
 * Errors: SSM_EINVAL, SSM_EUNSUPPORTED, SSM_ENOMEM, SSM_EHIP.
 */
int ssm_out_proj_bwd(const void *y, const void *W, const void *dout, void *dy, void *dW, int64_t batch,
                     int64_t d_inner, int64_t d_model, int64_t L, int dtype, void *stream);

/*
 * affine_scan -- inclusive scan of affine pairs along each row
 * ([Scan page] §1.2 and §2.1; [Mamba-2 page] §2.2).
 * A pair (a, b) is the map h -> a*h + b; composition, later step first, is
 *     (a2, b2) o (a1, b1) = (a2*a1, a2*b1 + b2),  identity (1, 0).
 * For each row r and step t:
 *     out_a[r,t] = a[r,t] * out_a[r,t-1],   out_b[r,t] = a[r,t]*out_b[r,t-1] + b[r,t]
 * starting from (1, 0), i.e. out_b is h_t with h_0 = 0.
 *   a, b         : [rows, L] float32 inputs.
 *   out_a        : [rows, L] float32 output, nullable (products not written).
 *   out_b        : [rows, L] float32 output.
 *   Each output may equal its own input (in place) or be disjoint from all
 *   inputs; partial overlap is SSM_EINVAL.
 * Rounding: float32 with a fused multiply-add for a*b + c, evaluated in the
 * fixed association order that affine_scan_order() describes, so results are
 * reproducible bit for bit from run to run and by any replay of that order.
 * That order, with T = items per lane, 64 lanes per wave, W waves per block
 * and chunk = 64*W*T:
 *   chunks of each row are taken in order with a carry starting at (1, 0);
 *   item j of lane l of wave w of chunk k is step k*chunk + (w*64 + l)*T + j,
 *   steps past L being identities.  (1) each lane folds its T items left to
 *   right from its first item; (2) the lane totals are scanned inside each
 *   wave in rounds d = 1, 2, 4, 8 (lane l takes lane l-d if l mod 16 >= d),
 *   then 16 (lanes with bit 4 set take lane 16*floor(l/16)-1) and 32 (lanes
 *   >= 32 take lane 31), every lane composing own o taken with the identity
 *   where it takes nothing; (3) lane l's exclusive prefix is lane l-1's
 *   inclusive value; (4) acc = carry folded with the totals of waves
 *   0..w-1 in order; a lane starts from (exclusive o acc), lane 0 from acc;
 *   the next carry folds all W totals; (5) each lane re-folds its items from
 *   its start, writing every prefix.
 */
int affine_scan(const float *a, const float *b, float *out_a, float *out_b,
                int64_t rows, int64_t L, void *stream);

/*
 * affine_scan_order -- the constants of affine_scan's association order
 * (host only).  Any pointer may be NULL.  Returns SSM_OK.
 */
int affine_scan_order(int *items_per_lane, int *lanes, int *waves, int *chunk);

/*
 * ssm_last_error -- text of the last failure on the calling thread
 * ("" if none).  The pointer stays valid until that thread's next call.
 */
const char *ssm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
