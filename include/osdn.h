/*
 * libosdn -- Online Scaled DeltaNet (OSDN) forward and decode step for AMD gfx950 (MI355X).
 *
 * The operation (OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
 * Attention, technical summary, section 2.1, with the per-token loss of section 1): for every
 * (batch b, head h) sequence, token by token,
 *
 *     S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) (d_t (.) k_t)^T ,
 *     o_t = S_t q_t ,
 *
 * i.e. one delta-rule write whose gradient step is right-preconditioned by diag(d_t), which
 * the summary shows is the same as scaling the write-side key to k~_t = d_t (.) k_t while the
 * residual keeps the plain key.  The optional per-head scalar decay alpha_t is the
 * gated-delta form (Erase-then-Delta Attention, section 2.2, eq. 4); it multiplies the old
 * state before the residual is formed.  The read-out is taken after the write.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library allocates
 *     nothing, keeps no per-call state, and never synchronises the stream.  Work is enqueued
 *     on `stream` (a hipStream_t; NULL = the default stream) and is complete when that
 *     stream reaches it.  Calls on different streams may run concurrently.
 *   - Layouts are dense row-major, head-major:  q, k, d [B,H,T,dk];  v, o [B,H,T,dv];
 *     beta, alpha [B,H,T];  states [B,H,dk,dv] holding M = S^T (row i = key feature,
 *     column j = value feature), always float32.
 *   - q, k, v and o share one element type (`qkv`: OSDN_F32 or OSDN_BF16); d has its own
 *     (`d_dtype`); beta, alpha and states are float32.  bf16 outputs are rounded to nearest
 *     even.
 *   - q, k, v, d, o and the state pointers must be 16-byte aligned; beta and alpha 4-byte.
 *   - Validation happens on the host before anything is enqueued.  On any error the call
 *     returns the status and touches no memory.  NaN/Inf in the inputs are not checked;
 *     they propagate to the outputs.
 *   - The same inputs give bitwise-identical outputs on every run (no atomics, fixed
 *     reduction orders).
 */
#ifndef OSDN_H
#define OSDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSDN_ABI_VERSION 6

typedef enum osdn_status {
    OSDN_OK = 0,
    OSDN_ERR_NULL = -1,        /* a required pointer is NULL                                 */
    OSDN_ERR_SHAPE = -2,       /* a size is negative, or an element count would overflow     */
    OSDN_ERR_UNSUPPORTED = -3, /* dk / dv / chunk / dtype combination not implemented        */
    OSDN_ERR_ALIGN = -4,       /* a pointer violates the alignment rule above                */
    OSDN_ERR_ALIAS = -5,       /* an output overlaps memory it must not overlap              */
    OSDN_ERR_LAUNCH = -6,      /* the HIP runtime rejected the launch (e.g. no gfx950 device) */
    OSDN_ERR_SCRATCH = -7,     /* the no-allocation entry point: the problem needs more scratch
                                  than OSDN_NOALLOC_SCRATCH_BYTES                             */
} osdn_status;

typedef enum osdn_dtype { OSDN_F32 = 0, OSDN_BF16 = 1 } osdn_dtype;

/*
 * Chunkwise-parallel forward over whole sequences (OSDN technical summary, section 2.1: the
 * scaled key takes the place of the stored key in the chunk Gram matrix and in the
 * intra-chunk scores; the chunk algebra itself is derived from the token step above).
 *
 *   q, k   [B,H,T,dk] qkv     queries and keys (the write-side key is d (.) k)
 *   v      [B,H,T,dv] qkv     values
 *   beta   [B,H,T]    f32     scalar write gate
 *   d      [B,H,T,dk] d_dtype per-token, per-feature preconditioner diagonal
 *   alpha  [B,H,T]    f32     per-token, per-head decay; NULL means alpha == 1 (no decay)
 *   S0     [B,H,dk,dv] f32    initial state M0 = S0^T; NULL means zero
 *   o      [B,H,T,dv] qkv     output, o_t = S_t q_t (written for every t < T)
 *   S_T    [B,H,dk,dv] f32    final state, NULL means not written.  S_T may be the same
 *                             pointer as S0 (in-place carry); any other overlap is an error.
 *   B, H, T >= 0              T == 0 writes S_T = S0 (or zeros); B*H == 0 does nothing.
 *   dk, dv in {64, 128}
 *   chunk                     rows per chunk: 64 for OSDN_BF16; 16, 32 or 64 for OSDN_F32.
 *                             The result does not depend on it beyond rounding.  T need
 *                             not be a multiple of it (the last chunk is masked).
 *   qkv                       OSDN_F32 (fp32 arithmetic throughout) or OSDN_BF16 (bf16
 *                             matrix-core operands, fp32 accumulation and fp32 state)
 *   d_dtype                   OSDN_F32 or OSDN_BF16
 *   o must not overlap any input or S_T.
 */
osdn_status osdn_chunk_fwd(const void *q, const void *k, const void *v, const float *beta,
                           const void *d, const float *alpha, const float *S0, void *o,
                           float *S_T, int64_t B, int64_t H, int64_t T, int32_t dk,
                           int32_t dv, int32_t chunk, osdn_dtype qkv, osdn_dtype d_dtype,
                           void *stream);

/*
 * One recurrent decode step for every (b,h) (the token step above, applied once):
 *   q, k   [B,H,dk] qkv;  v [B,H,dv] qkv;  beta [B,H] f32;  d [B,H,dk] d_dtype;
 *   alpha  [B,H] f32 or NULL (no decay);
 *   S      [B,H,dk,dv] f32, read as M_{t-1} and overwritten in place with M_t;
 *   o      [B,H,dv] qkv, o = M_t^T q.
 *   dk, dv in {64, 128}.  o must not overlap S or any input; S must not overlap an input.
 */
osdn_status osdn_step(const void *q, const void *k, const void *v, const float *beta,
                      const void *d, const float *alpha, float *S, void *o, int64_t B,
                      int64_t H, int32_t dk, int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype,
                      void *stream);

/*
 * Phase-1 preconditioner scan: the per-token diagonal d_t that osdn_chunk_fwd takes, produced
 * from the key stream (OSDN technical summary, section 2.2: d is moved by online gradient
 * descent on the hypergradient surrogate h_t, whose closed form depends only on k_t and
 * beta_t; section 2.3: the APF retention gate r multiplies the preconditioner state).  For
 * every (b,h), token by token, with x_t = k_t^2 (elementwise):
 *
 *     token t writes with d_t;
 *     d_{t+1} = r_t d_t + eta beta_t (1 - beta_t <d_t, x_t>) x_t / ||k_t||^2
 *             = r_t d_t - eta grad_d h_t(d_t);
 *
 * a zero key takes no gradient step (d_{t+1} = r_t d_t).
 *
 *   k      [B,H,T,dk] k_dtype  keys (the same k that osdn_chunk_fwd takes)
 *   beta   [B,H,T]    f32      scalar write gate
 *   r      [B,H,T]    f32      retention gate, expected in (0, 1]; NULL means r == 1
 *   d1     [B,H,dk]   f32      preconditioner of each sequence's first token; NULL means 1
 *   eta                        meta step size
 *   d      [B,H,T,dk] d_dtype  output: d_t for every t < T
 *   d_next [B,H,dk]   f32      output: the preconditioner after the last token, NULL means not
 *                              written; it may be the same pointer as d1 (in-place carry)
 *   B, H, T >= 0;  dk in {64, 128}
 *   chunk                      1: token-serial scan (any k_dtype; one wave per sequence).
 *                              64: chunkwise form (k_dtype must be OSDN_BF16): the step is affine
 *                              in d, so each 64-token chunk is one small triangular solve plus
 *                              bf16 matrix-core products with fp32 accumulation.  The two agree
 *                              to rounding; for ln r below -80 the chunkwise form uses -80.
 *   d must not overlap any input or d_next; d_next may overlap d1 only exactly.
 */
osdn_status osdn_precond_scan(const void *k, const float *beta, const float *r,
                              const float *d1, float eta, void *d, float *d_next, int64_t B,
                              int64_t H, int64_t T, int32_t dk, int32_t chunk,
                              osdn_dtype k_dtype, osdn_dtype d_dtype, void *stream);

/*
 * One decode token of the scan above, for every (b,h):
 *   k [B,H,dk] k_dtype;  beta [B,H] f32;  r [B,H] f32 or NULL;
 *   dstate [B,H,dk] f32, read as d_t and overwritten in place with d_{t+1};
 *   d_out  [B,H,dk] d_dtype, receives d_t (the diagonal this token writes with: osdn_step's d);
 *          NULL means not written.
 *   d_out must not overlap dstate or an input; dstate must not overlap an input.
 */
osdn_status osdn_precond_step(const void *k, const float *beta, const float *r, float *dstate,
                              void *d_out, float eta, int64_t B, int64_t H, int32_t dk,
                              osdn_dtype k_dtype, osdn_dtype d_dtype, void *stream);

/*
 * Chunkwise forward with the channel-wise (Kimi Delta Attention) gate in place of the scalar
 * one (Erase-then-Delta Attention, section 2.2, eq. 5, and section 3.2, eq. 7, with the OSDN
 * write key of section 2.1 of the OSDN technical summary).  For every (b,h), token by token,
 * in the storage convention M = S^T:
 *
 *     M_t = Diag(a_t) M_{t-1} + beta_t k~_t (v_t - (Diag(a_t) M_{t-1})^T k_t)^T ,
 *     o_t = M_t^T q_t ,      k~_t = d_t (.) k_t ,
 *
 * i.e. each key feature (row of M) has its own retention factor a_t[i].
 *
 *   alpha_ch  [B,H,T,dk] f32   per-token, per-key-feature retention in [0, 1], any size
 *                              (Erase-then-Delta Attention sets no lower bound): the decay
 *                              enters only as products of these factors, never divided;
 *                              16-byte aligned (OSDN_ERR_ALIGN otherwise)
 *   workspace                  bf16 inputs: caller-owned device memory of at least
 *                              osdn_chunk_fwd_kda_workspace(B, H, T, dk, chunk, qkv) bytes,
 *                              256-byte aligned; its contents on entry are ignored and on
 *                              return unspecified; it must not overlap any other argument.
 *                              fp32 inputs need none (the size is 0; may be NULL)
 *   workspace_bytes            its size
 *   every other argument       as for osdn_chunk_fwd (there is no scalar alpha here)
 * bf16 inputs: two kernels run on `stream`.  The first forms, for every chunk in parallel, the
 * gate-scaled q o G, k o G, k~ o (G_C / G) (G the running product of the gates from the chunk
 * start, G_C its value at the chunk's end, each formed as a product), G_C, the score matrix and
 * the pieces of the chunk's UT transform, into the workspace; the chunkwise forward then reads
 * them.  fp32 inputs: one kernel, at chunk min(chunk, 32).
 */
int64_t osdn_chunk_fwd_kda_workspace(int64_t B, int64_t H, int64_t T, int32_t dk,
                                     int32_t chunk, osdn_dtype qkv); /* -1 if invalid */

osdn_status osdn_chunk_fwd_kda(const void *q, const void *k, const void *v, const float *beta,
                               const void *d, const float *alpha_ch, const float *S0, void *o,
                               float *S_T, void *workspace, int64_t workspace_bytes,
                               int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                               int32_t chunk, osdn_dtype qkv, osdn_dtype d_dtype,
                               void *stream);

/*
 * One decode step with the channel-wise gate (the token step above, applied once):
 *   alpha_ch [B,H,dk] f32; every other argument as for osdn_step (no scalar alpha).
 */
osdn_status osdn_step_kda(const void *q, const void *k, const void *v, const float *beta,
                          const void *d, const float *alpha_ch, float *S, void *o, int64_t B,
                          int64_t H, int32_t dk, int32_t dv, osdn_dtype qkv,
                          osdn_dtype d_dtype, void *stream);

/*
 * Gradients of the chunkwise forward (osdn_chunk_fwd with the same inputs) for a scalar loss
 * whose gradients with respect to the outputs are grad_o [B,H,T,dv] (qkv dtype) and grad_S_T
 * [B,H,dk,dv] fp32 (NULL: zero).  The pages give no backward pass; the gradients are those of
 * the token step (OSDN technical summary, section 2.1; decay as in Erase-then-Delta Attention,
 * section 2.2, eq. 4), computed in a chunk form derived from the forward's.
 *
 *   grad_q, grad_k [B,H,T,dk], grad_v [B,H,T,dv]   out, qkv dtype
 *   grad_beta [B,H,T] fp32, grad_d [B,H,T,dk] d dtype   out
 *   grad_alpha [B,H,T] fp32   out; ignored when alpha is NULL, may be NULL (not written)
 *   grad_S0 [B,H,dk,dv] fp32  out, the gradient with respect to the initial state (whether or
 *                             not S0 is given); NULL: not written
 *   workspace                 caller-owned device memory of at least
 *                             osdn_chunk_bwd_workspace(B, H, T, dk, dv, qkv) bytes, 256-byte
 *                             aligned; contents on entry ignored, on return unspecified
 * Every other argument as for osdn_chunk_fwd; the chunk size is the library's (64 rows for
 * bf16 inputs, 32 for fp32).  Outputs must not overlap each other, an input or the workspace.
 * Kernels run on `stream`: the forward recording the state at every chunk start (the same
 * forward osdn_chunk_fwd runs for this input type), for bf16 inputs the inverse (I + A)^{-1},
 * the scores and k~ of every chunk, a reverse pass over chunks for the state gradient, and the
 * per-chunk gradients.
 * The workspace holds the state and state-gradient checkpoints (per sequence and chunk a dk x dv
 * matrix; bf16 for bf16 inputs, the precision the matrix products take them in, stored as dv/16
 * contiguous dk x 16 column tiles, [B,H,nchunks,dv/16,dk,16]; fp32 [B,H,nchunks,dk,dv] for fp32
 * inputs)
 * and, for bf16 inputs, per chunk three bf16 64 x 64 planes (the inverse (I + A)^{-1} as hi and
 * lo parts, and the intra-chunk scores) and k~ = d (.) k as 64 x dk bf16, then the per-row
 * pseudo-values U (from the forward) and their gradient dR (from the reverse pass), bf16, per
 * 64-row chunk dv/16 contiguous 64 x 16 column tiles, [B,H,nchunks,dv/16,64,16] each (the last
 * chunk padded).
 */
int64_t osdn_chunk_bwd_workspace(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                 osdn_dtype qkv); /* -1 if invalid */

osdn_status osdn_chunk_bwd(const void *q, const void *k, const void *v, const float *beta,
                           const void *d, const float *alpha, const float *S0,
                           const void *grad_o, const float *grad_S_T, void *grad_q,
                           void *grad_k, void *grad_v, float *grad_beta, void *grad_d,
                           float *grad_alpha, float *grad_S0, void *workspace,
                           int64_t workspace_bytes, int64_t B, int64_t H, int64_t T, int32_t dk,
                           int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype, void *stream);

/*
 * The training pair: the forward that also keeps the state at every chunk start, and the
 * backward that takes those states instead of recomputing them (the first of its launches).
 *
 * osdn_chunk_fwd_states: as osdn_chunk_fwd with the backward's chunk size (64 rows for bf16
 * inputs, 32 for fp32), and in addition
 *   states   out, osdn_chunk_states_bytes(B, H, T, dk, dv, qkv) bytes, 16-byte aligned,
 *            overlapping no other argument: the state before chunk c's first row in slot c,
 *            for bf16 inputs in bf16 (the precision the backward's products take them in) as
 *            dv/16 contiguous dk x 16 column tiles, [B,H,nchunks,dv/16,dk,16], then, from the
 *            next 256-byte boundary, the pseudo-values U of every row, bf16, per 64-row chunk
 *            dv/16 contiguous 64 x 16 column tiles, [B,H,nchunks,dv/16,64,16]; for
 *            fp32 inputs fp32 [B,H,nchunks,dk,dv]
 * o and S_T are bitwise those of osdn_chunk_fwd with that chunk size.
 *
 * osdn_chunk_bwd_states: as osdn_chunk_bwd, with `states` (input) from osdn_chunk_fwd_states on
 * the same inputs; it may not overlap an output or the workspace.  The gradients are bitwise
 * those of osdn_chunk_bwd.  The workspace holds only what the states do not (the state gradient
 * at every chunk end, the chunk planes and, for bf16 inputs, dR):
 * osdn_chunk_bwd_states_workspace(B, H, T, dk, dv, qkv) bytes, 256-byte aligned.
 */
int64_t osdn_chunk_states_bytes(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                osdn_dtype qkv); /* -1 if invalid */
int64_t osdn_chunk_bwd_states_workspace(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                        osdn_dtype qkv); /* -1 if invalid */

osdn_status osdn_chunk_fwd_states(const void *q, const void *k, const void *v,
                                  const float *beta, const void *d, const float *alpha,
                                  const float *S0, void *o, float *S_T, void *states, int64_t B,
                                  int64_t H, int64_t T, int32_t dk, int32_t dv, osdn_dtype qkv,
                                  osdn_dtype d_dtype, void *stream);

osdn_status osdn_chunk_bwd_states(const void *q, const void *k, const void *v,
                                  const float *beta, const void *d, const float *alpha,
                                  const float *S0, const void *states, const void *grad_o,
                                  const float *grad_S_T, void *grad_q, void *grad_k,
                                  void *grad_v, float *grad_beta, void *grad_d,
                                  float *grad_alpha, float *grad_S0, void *workspace,
                                  int64_t workspace_bytes, int64_t B, int64_t H, int64_t T,
                                  int32_t dk, int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype,
                                  void *stream);

/*
 * Gradients of the forward with the channel-wise gate (osdn_chunk_fwd_kda with the same
 * inputs) for a scalar loss whose gradients with respect to the outputs are grad_o and
 * grad_S_T, as for osdn_chunk_bwd.  The pages give no backward pass; these are the gradients of
 * the token step M_t = Diag(a_t) M_{t-1} + beta_t k~_t (v_t - (Diag(a_t) M_{t-1})^T k_t)^T
 * (Erase-then-Delta Attention, section 2.2, eq. 5, with the OSDN write key of section 2.1 of
 * the OSDN technical summary), computed in a chunk form derived from the gated chunk algebra.
 *
 *   alpha_ch        [B,H,T,dk] f32   the gate, in (0, 1]: the gate's own gradient is formed as
 *                                    d(ln a)/a, so a gate of exactly 0 gives a non-finite
 *                                    grad_alpha_ch there (the other gradients stay finite);
 *                                    16-byte aligned
 *   grad_alpha_ch   [B,H,T,dk] f32   out; NULL: not written
 *   workspace       caller-owned device memory of at least osdn_chunk_bwd_kda_workspace(B, H,
 *                   T, dk, dv, qkv) bytes, 256-byte aligned: the state at every chunk start and
 *                   the state gradient at every chunk end, [B,H,nchunks,dk,dv] fp32 each, then
 *                   every chunk's gated score tiles and the inverse formed from them,
 *                   [B,H,nchunks,3,32,32] fp32 (AS, P and (I + diag(beta) AS)^{-1})
 *   every other argument   as for osdn_chunk_bwd (there is no scalar alpha here)
 * All arithmetic is fp32 for either input type, with 32-row chunks (the products of the two
 * gradient passes on the fp32 matrix cores, the rest on the vector ALUs); the per-feature decays
 * inside the chunk's score products are e to differences of running sums of ln a kept in double
 * precision, so every factor is at most 1.  Four kernels run on `stream`: the score tiles of
 * every chunk (in parallel), the fp32 forward with the gate recording the state at every chunk
 * start, a reverse pass over chunks for the state gradient, and the per-chunk gradients.
 */
int64_t osdn_chunk_bwd_kda_workspace(int64_t B, int64_t H, int64_t T, int32_t dk, int32_t dv,
                                     osdn_dtype qkv); /* -1 if invalid */

osdn_status osdn_chunk_bwd_kda(const void *q, const void *k, const void *v, const float *beta,
                               const void *d, const float *alpha_ch, const float *S0,
                               const void *grad_o, const float *grad_S_T, void *grad_q,
                               void *grad_k, void *grad_v, float *grad_beta, void *grad_d,
                               float *grad_alpha_ch, float *grad_S0, void *workspace,
                               int64_t workspace_bytes, int64_t B, int64_t H, int64_t T,
                               int32_t dk, int32_t dv, osdn_dtype qkv, osdn_dtype d_dtype,
                               void *stream);

/*
 * osdn_chunk_fwd_kda with no workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The caller passes inputs and outputs as for osdn_chunk_fwd_kda; the bf16 path's gate-scaled
 * operands and chunk planes go into a library-owned device array of
 * OSDN_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU the library runs on, held until the process
 * ends.  No call allocates or frees memory.
 *   - A problem whose workspace (osdn_chunk_fwd_kda_workspace) exceeds the array returns
 *     OSDN_ERR_SCRATCH before anything is enqueued (at dk = 128: about 67 k head-tokens,
 *     B * H * T, per call).  fp32 inputs need no scratch.
 *   - Every call on one GPU shares that GPU's array; it keeps the last call's contents, which
 *     no call reads before writing them.  Calls that overlap in time on one GPU (other
 *     streams, other host threads) race on it: serialise them.
 *   - The first call on a device looks up the array's address on that device (current device);
 *     a failure there returns OSDN_ERR_LAUNCH.
 * Outputs are bitwise those of osdn_chunk_fwd_kda (the same kernels).
 */
#define OSDN_NOALLOC_SCRATCH_BYTES (64ll << 20)
osdn_status osdn_chunk_fwd_kda_noalloc(const void *q, const void *k, const void *v,
                                       const float *beta, const void *d, const float *alpha_ch,
                                       const float *S0, void *o, float *S_T, int64_t B,
                                       int64_t H, int64_t T, int32_t dk, int32_t dv,
                                       int32_t chunk, osdn_dtype qkv, osdn_dtype d_dtype,
                                       void *stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char *osdn_status_string(osdn_status s);

/* OSDN_ABI_VERSION of the built library. */
int32_t osdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OSDN_H */
