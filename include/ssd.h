/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 SSD forward pass.
 *
 * The operation (per sequence s and head h, group g = h / (nheads/ngroups)):
 *
 *   state <- initial_state[s, h]  (headdim x dstate, fp32), or zeros
 *   for each token t of s:
 *     state[p, n] = exp(dt[t, h] * A[h]) * state[p, n] + dt[t, h] * x[t, h, p] * B[t, g, n]
 *     y[t, h, p]  = sum_n C[t, g, n] * state[p, n] + D[h] * x[t, h, p]
 *   final_state[s, h] <- state
 *
 * Sources: the selective SSM with per-token step size, B and C and the decay
 * exp(step * A) (tj-hxxt.cn long read of "Mamba: Linear-Time Sequence Modeling
 * with Selective State Spaces", part III, sub-sections (2) and 3); the
 * equivalence of this recurrence with a masked-attention product by a
 * semiseparable matrix, and its evaluation by block-decomposed matrix products
 * (QbitAI "Mamba-2" article, srwj168 repost, sections "Unifying SSM and
 * attention" and "Mamba-2: stronger learning, faster training and inference",
 * which also names variable sequence lengths); the state reset between packed
 * sequences (same long read, part III item 2.3 "Boundary Resetting").
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or synchronises; ssd_forward only enqueues kernels
 *    on the given HIP stream and returns.
 *  - Tensors are dense, row-major (C-contiguous) in the shapes listed, with
 *    the token index flattened as t = b * seqlen + l (dense batch) or the
 *    packed position (varlen). Every pointer must be 16-byte aligned.
 *  - x, dt, B, C and y share one element type (ssd_dtype). A, D, the initial
 *    and final states and all internal states are fp32; accumulation is fp32.
 *  - Errors are reported by return code; no exception crosses the ABI.
 *    Argument errors are detected before anything is enqueued. A thread-local
 *    message with details is available from ssd_last_error_detail().
 *  - The library keeps no state between calls and is safe to call from
 *    several host threads at once (on different workspaces).
 */
#ifndef SSD_MI355X_H_
#define SSD_MI355X_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
  SSD_OK = 0,
  SSD_ERR_INVALID_ARG = 1, /* malformed shape, pointer, size or cu_seqlens */
  SSD_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported set */
  SSD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  SSD_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} ssd_status;

typedef enum ssd_dtype {
  SSD_DTYPE_F32 = 0,  /* IEEE fp32 */
  SSD_DTYPE_BF16 = 1  /* bfloat16; y rounded to nearest even */
} ssd_dtype;

/* Flags for ssd_problem.flags. */
#define SSD_FLAG_GENERIC_KERNELS 1u /* use the plain FMA kernels even where the
                                       MFMA kernels apply (testing aid) */
#define SSD_FLAG_UNFUSED 2u         /* one kernel per step of the method
                                       (cumsum, chunk state, state passing,
                                       chunk scan) with per-chunk states in
                                       the workspace, instead of the fused
                                       kernel that bf16 problems use by
                                       default */
#define SSD_FLAG_PER_SEQUENCE 4u    /* fused kernel with one workgroup per
                                       (sequence, head) walking its chunks in
                                       order, instead of the default one
                                       workgroup per (chunk, head) chained
                                       through the state hand-off */

/*
 * Problem description.
 *   batch      dense batch rows (>= 1); must be 1 in varlen mode
 *   seqlen     tokens per batch row; in varlen mode the total packed tokens
 *   nheads     H >= 1
 *   headdim    P: 16, 32, 64 or 128
 *   dstate     N: a multiple of 16, 16 <= N <= 256
 *   ngroups    G >= 1 with H % G == 0; head h reads B and C of group
 *              h / (H / G), so consecutive heads share a group
 *   chunk_size Q: 64, 128 or 256 (the result does not depend on Q beyond
 *              rounding)
 *   num_seqs   0 = dense batch; > 0 = varlen with that many packed sequences
 *   dtype      ssd_dtype of x, dt, B, C, y
 *   flags      0 or SSD_FLAG_* bits
 */
typedef struct ssd_problem {
  int32_t batch;
  int32_t seqlen;
  int32_t nheads;
  int32_t headdim;
  int32_t dstate;
  int32_t ngroups;
  int32_t chunk_size;
  int32_t num_seqs;
  int32_t dtype;
  uint32_t flags;
} ssd_problem;

/* Check a problem description (host only, no device access).
 * Returns SSD_OK, SSD_ERR_INVALID_ARG (null, non-positive or inconsistent
 * sizes, H % G != 0, batch != 1 with num_seqs > 0, sizes whose element
 * counts overflow int32 indexing) or SSD_ERR_UNSUPPORTED (headdim, dstate,
 * chunk_size or dtype outside the supported set). */
ssd_status ssd_validate(const ssd_problem *prob);

/* Check host-resident cu_seqlens (num_seqs + 1 int32 values) against a
 * varlen problem: cu[0] == 0, non-decreasing, cu[num_seqs] == seqlen.
 * Zero-length sequences are allowed (their final state is their initial
 * state). Host only. */
ssd_status ssd_validate_cu_seqlens(const ssd_problem *prob,
                                   const int32_t *host_cu_seqlens);

/* Bytes of device workspace ssd_forward needs for this problem (host only).
 * The size depends only on the problem (never on the cu_seqlens values):
 * fp32 per-chunk states (chunks x H x P x N), per-chunk decay prefixes
 * (chunks x H x Q) and the chunk table, where chunks = batch * ceil(seqlen/Q)
 * (dense) or floor(seqlen/Q) + num_seqs (varlen upper bound). */
ssd_status ssd_workspace_size(const ssd_problem *prob, size_t *bytes);

/*
 * Run the SSD forward pass.
 *   x              (batch, seqlen, H, P)     dtype
 *   dt             (batch, seqlen, H)        dtype; step sizes as given
 *                                            (already positive; no bias,
 *                                            softplus or clamp applied here)
 *   A              (H)                       fp32 (decay exp(dt*A); A <= 0
 *                                            expected, not required)
 *   B, C           (batch, seqlen, G, N)     dtype
 *   D              (H)                       fp32, NULL = no skip term
 *   initial_state  (batch | num_seqs, H, P, N) fp32, NULL = zeros
 *   cu_seqlens     (num_seqs + 1)            int32 device array, varlen only
 *                                            (NULL in dense mode). Values must
 *                                            satisfy ssd_validate_cu_seqlens;
 *                                            they are not read by the host.
 *                                            Invalid device values never
 *                                            cause an out-of-bounds access,
 *                                            but y and final_state are then
 *                                            unspecified.
 *   y              (batch, seqlen, H, P)     dtype, written (out)
 *   final_state    (batch | num_seqs, H, P, N) fp32 (out), NULL = not written
 *   workspace      device buffer of at least ssd_workspace_size() bytes,
 *                  256-byte aligned; its contents on entry do not matter
 *   stream         a hipStream_t (NULL = the default stream)
 * Inputs and outputs must not overlap. Returns SSD_OK once all kernels are
 * enqueued; SSD_ERR_HIP if a launch fails.
 * The chained kernel (the default for bf16) bounds each of its waits for a
 * predecessor's state by one second; a wait that runs out sets the int32
 * error word chain_sync[1] of the workspace (ssd_get_workspace_layout) and
 * that pass's y and final_state are wrong. The word is cleared at the start
 * of every pass; a caller that must know reads it after the stream has
 * completed (no kernel of this library ever waits on another stream, so the
 * bound is only reached if the device stalls).
 */
ssd_status ssd_forward(const ssd_problem *prob, const void *x, const void *dt,
                       const float *A, const void *B, const void *C,
                       const float *D, const float *initial_state,
                       const int32_t *cu_seqlens, void *y, float *final_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ssd_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same operation, arguments, layouts and
 * kernels as ssd_forward; the workspace is instead a fixed scratch area of
 * 64 MiB that the library keeps in device memory on every GPU it runs on
 * (held until the process ends; its address is looked up on the first call
 * on a device, with that device current). The current device must be the
 * stream's device. Nothing is allocated, freed or synchronised.
 * Where the default bf16 path would give its chained kernel one state slot
 * and one aggregate per (chunk, head) (grids of up to 1536 one-chunk units)
 * and those do not fit, it uses the two slots per (sequence, head) of larger
 * grids instead, with the same outputs. Returns SSD_ERR_WORKSPACE, before
 * anything is enqueued, for problems whose workspace still exceeds 64 MiB;
 * use ssd_forward for those. On the default bf16 path the state hand-off
 * takes 64 KiB per (sequence, head) at P = 64, N = 128 and the C B^T and B^T
 * tiles about 136 KiB per (chunk, group) at chunk 256, so the 2.7B-shaped
 * batch (8 sequences of 2048 tokens, 80 heads: about 51 MB) fits and the
 * 64-sequence packed batch does not.
 * All calls on one GPU share its scratch area, and each pass clears what it
 * needs cleared itself: calls that may overlap on one GPU (on different
 * streams, or from several host threads) race and give wrong results; order
 * them on one stream. */
ssd_status ssd_forward_noalloc(const ssd_problem *prob, const void *x, const void *dt,
                               const float *A, const void *B, const void *C,
                               const float *D, const float *initial_state,
                               const int32_t *cu_seqlens, void *y, float *final_state,
                               void *stream);

/* ssd_forward with the step activation fused in: dt_raw holds the step's
 * pre-activation and every kernel uses
 *   dt[t, h] = softplus(dt_raw[t, h] + dt_bias[h]),  softplus(v) = log(1 + e^v)
 * in fp32 (not rounded to the dtype), which is how the selection mechanism
 * produces the step (tj-hxxt.cn long read of the Mamba-1 paper, part III (2):
 * the step passes through the softplus activation tau_delta). dt_bias is
 * (H) fp32 on the device, NULL = no offset; there is no clamp. Every other
 * argument, the layouts, the workspace and the errors are those of
 * ssd_forward. */
ssd_status ssd_forward_dt_softplus(const ssd_problem *prob, const void *x, const void *dt_raw,
                                   const float *dt_bias, const float *A, const void *B,
                                   const void *C, const float *D, const float *initial_state,
                                   const int32_t *cu_seqlens, void *y, float *final_state,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Per-kernel timing of the same launch sequence (a measurement aid).
 * Runs `iterations` back-to-back forward passes exactly as ssd_forward would
 * enqueue them, with a HIP event recorded before the first kernel and after
 * every kernel, then SYNCHRONISES the stream and reports, per kernel, the
 * summed event-to-event time (kernel duration plus launch gap) in `ms`, and
 * the first-to-last event time in `total_ms`. Same arguments, outputs and
 * errors as ssd_forward; creates and destroys its own events. */
#define SSD_MAX_STAGES 12
typedef struct ssd_stage_times {
  int32_t num_stages;
  int32_t iterations;
  char names[SSD_MAX_STAGES][24];
  float ms[SSD_MAX_STAGES];
  float total_ms;
} ssd_stage_times;
ssd_status ssd_forward_timed(const ssd_problem *prob, const void *x, const void *dt,
                             const float *A, const void *B, const void *C,
                             const float *D, const float *initial_state,
                             const int32_t *cu_seqlens, void *y, float *final_state,
                             void *workspace, size_t workspace_bytes, void *stream,
                             int32_t iterations, ssd_stage_times *times);

/* Where ssd_forward leaves its intermediates inside the workspace (byte
 * offsets), for inspection after the stream has completed:
 * The per-chunk intermediates exist only when the per-step kernels run
 * (fp32 problems, shapes the fused kernel does not cover, SSD_FLAG_UNFUSED);
 * the fused kernel keeps them on chip and the workspace has no room for them.
 *   chunk_cumsum  fp32 (chunks, H, Q): inclusive prefix of dt*A*log2(e)
 *                 inside each chunk, i.e. the base-2 logarithm of the decay
 *                 from the chunk's start through each token (entries past a
 *                 partial chunk's end are unspecified)
 *   chunk_states  fp32 (chunks, H, P, N): the state entering each chunk
 *   chunk_table   int32 (varlen only): [0] = number of chunks, [1] = nonzero
 *                 if the device cu_seqlens were invalid, [2 .. num_seqs+2] =
 *                 first chunk of each sequence followed by the total, then
 *                 from int offset chunk_records one (sequence, first token,
 *                 length, index in sequence) record per chunk
 *   chunk_records int32 offset of the records inside chunk_table
 *   max_chunks    chunks the layout has room for
 * Host only. */
typedef struct ssd_workspace_layout {
  size_t chunk_cumsum;
  size_t chunk_states;
  size_t chunk_table;
  int64_t chunk_records;
  int64_t max_chunks;
  size_t chain_sync;        /* int32 words of the chained kernel: [1] is
                               nonzero after a pass in which a workgroup
                               gave up waiting for its predecessor's state
                               (outputs then wrong); 0 = no chained kernel */
  int64_t chain_sync_words; /* number of those words (0 = none) */
  int64_t chain_chunks_per_unit; /* consecutive chunks of one (sequence, head)
                               that one workgroup of the chained kernel walks,
                               passing the state between them on chip; the
                               state goes through the workspace only between
                               such units (0 = no chained kernel) */
  int64_t chain_ranges;     /* > 0: the chained kernel's workgroups each take
                               one of this many balanced ranges of the
                               (sequence, head, chunk) order instead (dense
                               input with at least as many (sequence, head)
                               pairs as the current device holds such
                               workgroups); the state goes through the
                               workspace where a range starts inside a
                               sequence */
} ssd_workspace_layout;
ssd_status ssd_get_workspace_layout(const ssd_problem *prob,
                                    ssd_workspace_layout *layout);

/* One decode step: every sequence of a dense batch advances by one token,
 * its fp32 state updated in place (the recurrent mode of the same layer).
 *
 * Per sequence b and head h, with group g = h / (nheads/ngroups):
 *   state[b, h, p, n] = exp(dt[b, h] * A[h]) * state[b, h, p, n]
 *                       + dt[b, h] * x[b, h, p] * B[b, g, n]
 *   y[b, h, p]        = sum_n C[b, g, n] * state[b, h, p, n] + D[h] * x[b, h, p]
 * i.e. one iteration of the recurrence ssd_forward evaluates, so a sequence
 * may be prefilled with ssd_forward (final_state) and continued token by
 * token here. Source: the discretised SSM evaluated as a recurrence
 * (tj-hxxt.cn long read of the Mamba-1 paper, part II (1), "from continuous
 * systems to discrete modelling") and the state cache that makes generation
 * linear in length (same page, part IV (5), "computational efficiency", the
 * inference-speed item).
 *
 * Arguments (device pointers owned by the caller, 16-byte aligned):
 *   prob   batch = sequences (0 = nothing to do), seqlen must be 1,
 *          num_seqs must be 0, flags must be 0; chunk_size is ignored.
 *          nheads, headdim, dstate, ngroups and dtype as for ssd_forward
 *          (headdim in {16, 32, 64, 128}, dstate a multiple of 16 up to 256).
 *   x      (batch, H, P)   dtype
 *   dt     (batch, H)      dtype, used as given (already positive)
 *   A      (H)             fp32
 *   B, C   (batch, G, N)   dtype
 *   D      (H)             fp32, NULL = no skip term
 *   state  (batch, H, P, N) fp32, read and overwritten with the new state
 *   y      (batch, H, P)   dtype (out)
 *   stream a hipStream_t (NULL = the default stream)
 * The state must not overlap the other tensors. Errors: SSD_ERR_INVALID_ARG
 * (malformed sizes, NULL or misaligned pointers), SSD_ERR_UNSUPPORTED (shape
 * or dtype outside the set above), SSD_ERR_HIP (launch failed); nothing is
 * enqueued on error. Enqueues one kernel; no allocation, no synchronisation,
 * no workspace. */
ssd_status ssd_step(const ssd_problem *prob, const void *x, const void *dt,
                    const float *A, const void *B, const void *C, const float *D,
                    float *state, void *y, void *stream);

/* The Mamba-1 selective scan: the layer that SSD is measured against. Its A
 * is a diagonal N x D matrix (one rate per channel and state index) instead
 * of one scalar per head, so it cannot use matrix products; the pages credit
 * Mamba-2's restriction with a 2-8x speed-up over this scan (QbitAI CSDN
 * repost, abstract; briefgpt TL;DR). The step, B and C depend on the input
 * and A is discretised as exp(step * A) (tj-hxxt.cn long read of the Mamba-1
 * paper, part III (2) and item 3); A's shape N x D and the step's B x L x D
 * follow the kuaisou snippet on selective SSMs as linear attention. Per
 * sequence b, channel d and state index n:
 *   h[b, d, n] <- exp(delta[b, t, d] * A[d, n]) * h[b, d, n]
 *                 + delta[b, t, d] * B[b, t, n] * x[b, t, d]
 *   y[b, t, d]  = sum_n C[b, t, n] * h[b, d, n] + D[d] * x[b, t, d]
 * With A[d, n] = A_h for the channels of head h and delta shared by them it
 * is the SSD operation above.
 *
 * Problem: batch >= 0 (0 = nothing to do), seqlen >= 0, dim a multiple of 64,
 * dstate in {16, 32, 64, 128, 256}, batch <= 65535, flags 0.
 * Arguments (device pointers owned by the caller, 16-byte aligned):
 *   x, delta       (batch, seqlen, dim)   dtype; delta used as given (> 0)
 *   A              (dim, dstate) fp32
 *   B, C           (batch, seqlen, dstate) dtype (one set for all channels)
 *   D              (dim) fp32, NULL = no skip term
 *   initial_state  (batch, dim, dstate) fp32, NULL = zeros
 *   y              (batch, seqlen, dim) dtype (out)
 *   final_state    (batch, dim, dstate) fp32 (out), NULL = not written
 *   stream         a hipStream_t (NULL = the default stream)
 * Errors: SSD_ERR_INVALID_ARG (malformed sizes, NULL or misaligned
 * pointers), SSD_ERR_UNSUPPORTED (outside the set above), SSD_ERR_HIP;
 * nothing is enqueued on error. One kernel, no allocation, no workspace. */
typedef struct ssd_scan_problem {
  int32_t batch, seqlen, dim, dstate;
  int32_t dtype;      /* an ssd_dtype value (int32_t so that any value can be checked) */
  uint32_t flags;
} ssd_scan_problem;
ssd_status ssd_selective_scan(const ssd_scan_problem *prob, const void *x, const void *delta,
                              const float *A, const void *B, const void *C, const float *D,
                              const float *initial_state, void *y, float *final_state,
                              void *stream);

/* The backward pass: gradients of a loss L with respect to every input of
 * ssd_forward, given dL/dy and dL/d(final state). Training recomputes the
 * states instead of storing them (tj-hxxt.cn long read of the Mamba-1 paper,
 * part III (3), the efficient implementation); the gradients are those of the
 * recurrence above, through the same chunked decomposition ([QbitAI "Mamba-2"
 * article, srwj168 repost], "Mamba-2: stronger learning, faster training and
 * inference"). Per sequence and head, with G_t = dL/dh_t walked backwards from
 * dL/d(final state):
 *   G_t  += dy_t C_t^T;  dx_t = D dy_t + dt_t G_t B_t;  dB_t += dt_t G_t^T x_t
 *   dC_t += h_t^T dy_t;  ddt_t = <G_t, x_t B_t^T> + A exp(dt_t A) <G_t, h_{t-1}>
 *   dA   += dt_t exp(dt_t A) <G_t, h_{t-1}>;  dD += <dy_t, x_t>;  G_{t-1} = exp(dt_t A) G_t
 * and dL/d(initial state) = G before the first token (dB, dC summed over the
 * heads of a group). The states are recomputed from the forward inputs; the
 * forward output is not needed.
 *
 * Problem: as for ssd_forward, with flags 0, dtype BF16, headdim 64, dstate
 * 64 or 128 and chunk_size 128 or 256 (SSD_ERR_UNSUPPORTED otherwise).
 * Arguments (device pointers owned by the caller, 16-byte aligned unless
 * noted; shapes as in ssd_forward):
 *   x, dt, A, B, C, D, initial_state, cu_seqlens   the forward inputs
 *   dy             (tokens, H, P) bf16: dL/dy
 *   dfinal_state   (batch | num_seqs, H, P, N) fp32, NULL = zero
 *   dx             (tokens, H, P) bf16 (out)
 *   ddt            (tokens, H) bf16 (out, any alignment), NULL = not written
 *   dA             (H) fp32 (out, any alignment)
 *   dB, dC         (tokens, G, N) bf16 (out)
 *   dD             (H) fp32 (out, any alignment), NULL = not written; without D
 *                  it is the gradient at D = 0
 *   dinitial_state (batch | num_seqs, H, P, N) fp32 (out), NULL = not written;
 *                  without an initial state it is the gradient at zero
 *   workspace      at least ssd_backward_workspace_size() bytes, 256-byte
 *                  aligned; contents on entry do not matter
 *   stream         a hipStream_t (NULL = the default stream)
 * Outputs must not overlap inputs or each other. Enqueues the kernels and
 * returns; no allocation, no synchronisation. Errors as for ssd_forward. */
ssd_status ssd_backward_workspace_size(const ssd_problem *prob, size_t *bytes);
ssd_status ssd_backward(const ssd_problem *prob, const void *x, const void *dt, const float *A,
                        const void *B, const void *C, const float *D,
                        const float *initial_state, const int32_t *cu_seqlens,
                        const void *dy, const float *dfinal_state, void *dx, void *ddt,
                        float *dA, void *dB, void *dC, float *dD, float *dinitial_state,
                        void *workspace, size_t workspace_bytes, void *stream);

/* ssd_backward `iterations` times back to back with a HIP event after every
 * kernel; synchronises the stream and returns per-kernel times (ms summed
 * over the iterations) in `times`. For measurement. */
ssd_status ssd_backward_timed(const ssd_problem *prob, const void *x, const void *dt,
                              const float *A, const void *B, const void *C, const float *D,
                              const float *initial_state, const int32_t *cu_seqlens,
                              const void *dy, const float *dfinal_state, void *dx, void *ddt,
                              float *dA, void *dB, void *dC, float *dD, float *dinitial_state,
                              void *workspace, size_t workspace_bytes, void *stream,
                              int32_t iterations, ssd_stage_times *times);

/* The convolution front that produces the SSD layer's x, B and C: a causal
 * depthwise 1-D convolution over the packed channels [x | B | C] of each
 * token, followed by SiLU. In the Mamba-2 model one part of the input
 * projection passes through a 1-D convolution that captures local
 * dependencies without looking ahead (CSDN csdn_xmj page, related-article
 * snippet on implementing the Mamba-2 model), and the Mamba block uses an
 * activation where H3 had a gate (tj-hxxt.cn long read of the Mamba-1 paper,
 * part III, the closing paragraph on the selection mechanism). With
 * ch = x_dim + 2 bc_dim and K = width, per sequence and channel c, the K - 1
 * inputs before the first token being the sequence's history rows (or zeros):
 *   pre[t, c] = bias[c] + sum_{k < K} weight[c, k] * u[t - (K - 1) + k, c]
 *   out[t, c] = pre[t, c] / (1 + exp(-pre[t, c]))
 * (weight[c, K - 1] multiplies the current token). Channels [0, x_dim) of out
 * go to x, the next bc_dim to B and the last bc_dim to C. Packed sequences
 * never see each other's tokens. The history of a sequence is its last K - 1
 * inputs, oldest first: history_out of one call is history_in of the next
 * call over the same sequences (chunked prefill, then decode with seqlen 1).
 *
 * Problem: dense mode (num_seqs 0) has batch >= 0 rows of seqlen >= 0 tokens;
 * packed mode (num_seqs > 0) has batch 1, seqlen = the total tokens and
 * cu_seqlens. x_dim and bc_dim are multiples of 8 (x_dim = H * P and
 * bc_dim = G * N for the SSD layer), ch >= 8; width in {2, 3, 4}; in_stride
 * >= ch and a multiple of 16 bytes; dtype F32 or BF16; flags 0.
 * Arguments (device pointers owned by the caller, 16-byte aligned where
 * listed):
 *   xbc          row t at xbc + t * in_stride, channels [0, ch)   dtype, aligned
 *                (in_stride > ch reads a slice of a wider projection row)
 *   weight       (ch, width) fp32 taps
 *   bias         (ch) fp32, NULL = none
 *   history_in   (batch | num_seqs, width - 1, ch) dtype, aligned, NULL = zeros
 *   cu_seqlens   (num_seqs + 1) int32, packed mode only (NULL in dense mode):
 *                0 = cu[0] <= cu[1] <= ... <= cu[num_seqs] = seqlen; zero
 *                lengths allowed. Invalid device values never cause an
 *                out-of-bounds access, but the outputs are then unspecified.
 *   x            (tokens, x_dim) dtype (out), aligned
 *   B, C         (tokens, bc_dim) dtype (out), aligned
 *   history_out  (batch | num_seqs, width - 1, ch) dtype (out), aligned,
 *                NULL = not written; must not overlap history_in
 *   stream       a hipStream_t (NULL = the default stream)
 * Arithmetic is fp32; bf16 outputs are rounded to nearest even; histories
 * copy inputs exactly. Outputs must not overlap inputs. Errors:
 * SSD_ERR_INVALID_ARG (malformed sizes, NULL or misaligned pointers),
 * SSD_ERR_UNSUPPORTED (outside the set above), SSD_ERR_HIP; nothing is
 * enqueued on error. No allocation, no workspace. */
typedef struct ssd_conv_problem {
  int32_t batch, seqlen, num_seqs;
  int32_t x_dim, bc_dim, width, in_stride;
  int32_t dtype;      /* an ssd_dtype value (int32_t so that any value can be checked) */
  uint32_t flags;
} ssd_conv_problem;
ssd_status ssd_conv1d_silu(const ssd_conv_problem *prob, const void *xbc, const float *weight,
                           const float *bias, const void *history_in,
                           const int32_t *cu_seqlens, void *x, void *B, void *C,
                           void *history_out, void *stream);

/* Static text for a status code. */
const char *ssd_status_string(ssd_status status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char *ssd_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H_ */
