/*
 * eda.h -- C ABI of the MI355X (gfx950) Erase-then-Delta Attention forward.
 *
 * The operation (EDA paper, Sec. 3.3, Eq. (8); reading slides, frame "EDA
 * preserves the delta write after cleanup"): every head keeps a state
 * S in R^{d_k x d_v} (rows are key channels, fp32) and for each token t
 *
 *     S_t = (I - beta_t k_t k_t^T)(I - gamma_t e_t e_t^T) Diag(alpha_t) S_{t-1}
 *           + beta_t k_t v_t^T,                 o_t = S_t^T q_t,
 *
 * i.e. decay the retained key channels, erase along the cleanup address
 * e_t, then the delta-rule corrected write along k_t (Eqs. (9)-(13)); the
 * readout uses the post-update state and no query scale.
 *
 * Conventions shared by every entry point:
 *  - All tensor arguments are DEVICE pointers to contiguous row-major
 *    arrays owned by the caller.  q, k, e, v, alpha, beta, gamma need only
 *    their element alignment (2 or 4 bytes); states and the chunked path's
 *    o must be 16-byte aligned (decode's o: element alignment).
 *  - Token inputs use the layout [B, T, H, d] (batch, time, head, channel);
 *    per-token scalars [B, T, H]; states [B, H, d_k, d_v].
 *  - q, k, e, v and o share one storage type (`eda_dtype_t`); alpha, beta,
 *    gamma and the states are always fp32.  Arithmetic on the state is fp32.
 *  - Inputs are not range-checked (they are device data): the results are
 *    defined for alpha in (0, 1], beta and gamma in [0, 1] and finite
 *    values; q, k, e are used exactly as given (the layer normalises them,
 *    paper Fig. 1).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued; no call synchronises, allocates memory or keeps state between
 *    calls, so concurrent calls on different streams are safe.
 *  - Every check below happens before anything is enqueued; a call that
 *    returns an error has touched no memory.  A failed kernel launch
 *    returns EDA_ERR_HIP.  Nothing is printed and no exception crosses the
 *    ABI.
 */
#ifndef EDA_H
#define EDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EDA_OK = 0,
    EDA_ERR_NULL = 1,        /* a required pointer is NULL                        */
    EDA_ERR_SHAPE = 2,       /* a size is <= 0 or too large                       */
    EDA_ERR_DTYPE = 3,       /* unknown eda_dtype_t                               */
    EDA_ERR_ALIGN = 4,       /* a pointer is misaligned (see conventions)          */
    EDA_ERR_UNSUPPORTED = 5, /* head dims or chunk size outside the supported set */
    EDA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required        */
    EDA_ERR_ALIAS = 7,       /* an output overlaps an input it may not overlap     */
    EDA_ERR_HIP = 8,         /* a HIP launch failed                               */
    EDA_ERR_SCRATCH = 9      /* eda_fwd_chunked_noalloc: the problem needs more
                                workspace than EDA_NOALLOC_SCRATCH_BYTES          */
} eda_status_t;

typedef enum { EDA_F32 = 0, EDA_BF16 = 1 } eda_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char *eda_status_string(eda_status_t s);

/*
 * Bytes of device workspace eda_fwd_chunked needs for these sizes (0 for an
 * unsupported combination).  `chunk` is the number of tokens per chunk (0
 * selects the default, 64).  The workspace holds every chunk's
 * state-independent factors between the two kernels of the chunked forward.
 * For bf16 inputs those are the chunk's affine state map (S -> Lambda S +
 * Phi S + Psi V, O = Qhat S + Phat V): with d_k = d_v = 128 that is 74240
 * bytes per 64-token chunk and head (1.16 KB per token and head), 51712 per
 * 32-token chunk and 46592 per 16-token chunk.  With few heads and a long
 * sequence (B*H*d/16 < 256 with d = 64 or 128, and at least 256 chunks), the
 * bf16 state pass walks P segments of each head at the same time, and the
 * workspace also holds B*H*(P-1)*d_k*(d_k + 2 d_v) fp32 values: the segment
 * maps and start states.  fp32 inputs compute chunk 64 as 32-token chunks (a
 * 64-token chunk's fp32 operands exceed one compute unit's LDS) and need the
 * same workspace as chunk 32.
 */
size_t eda_fwd_chunked_workspace_size(int B, int T, int H, int d_k, int d_v,
                                      eda_dtype_t dtype, int chunk);

/*
 * Chunk-parallel (prefill) forward over a whole sequence.
 *
 * Computes, for all B*H heads, o_t for t = 0..T-1 and the final state,
 * exactly the recurrence above up to floating-point rounding.  The sequence
 * is cut into chunks of `chunk` tokens; each token is treated as two rank-1
 * sub-steps, an erase (key e_t, gate gamma_t, decay alpha_t, no write) then
 * a delta write (key k_t, gate beta_t, no decay, value v_t), which is the
 * doubled-sequence form of the paper's Sec. 3.4 (Eqs. (17)-(18); slides
 * frame "Two virtual steps recover a standard delta recurrence").  Within a
 * chunk the sub-steps are solved with a triangular (UT/WY-type) transform
 * and dense bf16/fp32 matrix-core products; the state is carried across
 * chunks in fp32.  The chunk size does not change the exact result.
 *
 *   q, k, e : [B, T, H, d_k]  dtype          v : [B, T, H, d_v]  dtype
 *   alpha   : [B, T, H, d_k]  fp32 retention per key channel
 *   beta, gamma : [B, T, H]   fp32 write gate and erase gate
 *   S0      : [B, H, d_k, d_v] fp32 initial state, or NULL for zeros
 *   o       : [B, T, H, d_v]  dtype, written (fp32 accumulation, then
 *             round-to-nearest-even for bf16)
 *   S_final : [B, H, d_k, d_v] fp32 final state, or NULL (not written);
 *             may be the same pointer as S0 (updated in place)
 *   workspace : device scratch of at least
 *             eda_fwd_chunked_workspace_size(...) bytes, 256-byte aligned;
 *             its contents on entry are ignored and on return undefined
 *
 * Supported: 1 <= d_k, d_v <= 128; chunk in {0, 16, 32, 64}; B, T, H >= 1 with
 * B*T*H*max(d_k, d_v) < 2^31.  o may not overlap any input; S_final may
 * overlap S0 only as the identical pointer.
 */
eda_status_t eda_fwd_chunked(const void *q, const void *k, const void *e, const void *v,
                             const float *alpha, const float *beta, const float *gamma,
                             const float *S0, void *o, float *S_final,
                             int B, int T, int H, int d_k, int d_v, eda_dtype_t dtype,
                             int chunk, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * eda_fwd_chunked, additionally recording three caller-created HIP events
 * (hipEvent_t values passed as void *) on `stream`: events[0] before the
 * chunk-factor kernel, events[1] between it and the state pass, events[2]
 * after the state pass, so a caller can time the two kernels separately
 * (benchmarks and profiling).  `events` may be NULL, which makes the call
 * identical to eda_fwd_chunked; otherwise all three must be valid events of
 * the stream's device.  Events are recorded only once every argument check
 * has passed.
 */
eda_status_t eda_fwd_chunked_timed(const void *q, const void *k, const void *e, const void *v,
                                   const float *alpha, const float *beta, const float *gamma,
                                   const float *S0, void *o, float *S_final,
                                   int B, int T, int H, int d_k, int d_v, eda_dtype_t dtype,
                                   int chunk, void *workspace, size_t workspace_bytes,
                                   void *stream, void *const *events);

/*
 * eda_fwd_chunked for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results as eda_fwd_chunked, without the
 * workspace arguments: the workspace is a scratch array of
 * EDA_NOALLOC_SCRATCH_BYTES (160 MiB) that the library holds on every device
 * it runs on, from the first use until the process ends.  The call makes no
 * hipMalloc, hipFree or other allocating call; the caller still passes every
 * input and output.
 *
 *   - The array of the calling thread's current device is used; `stream`
 *     must belong to that device.  Its address is looked up on the first
 *     call on each device.
 *   - A problem whose eda_fwd_chunked_workspace_size exceeds
 *     EDA_NOALLOC_SCRATCH_BYTES (bf16 at d_k = d_v = 128 and chunk 64 with 64
 *     heads fits T <= 2240, e.g. B=4, H=16, T=2048) is rejected with
 *     EDA_ERR_SCRATCH before anything is enqueued; use eda_fwd_chunked.
 *   - Every call on a device shares that device's array, which keeps the
 *     last call's contents (no call reads what an earlier call left there).
 *     Calls that can overlap in time on one device -- on different streams,
 *     or from different host threads without ordering -- race on the array
 *     and give undefined results: serialise them.
 */
#define EDA_NOALLOC_SCRATCH_BYTES ((size_t)160 << 20)
eda_status_t eda_fwd_chunked_noalloc(const void *q, const void *k, const void *e, const void *v,
                                     const float *alpha, const float *beta, const float *gamma,
                                     const float *S0, void *o, float *S_final,
                                     int B, int T, int H, int d_k, int d_v, eda_dtype_t dtype,
                                     int chunk, void *stream);

/*
 * One token of the recurrence for N independent sequences (decode).
 *
 * For each (n, h): reads S_in once, applies decay, erase and corrected write
 * for one token and writes S_out and o.  The three reductions S^T e, S^T k,
 * S^T q are taken in the same pass over S (the paper's Sec. 3.5 notes that
 * decoding is dominated by reading and writing the state).
 *
 *   q, k, e : [N, H, d_k] dtype   v : [N, H, d_v] dtype
 *   alpha   : [N, H, d_k] fp32    beta, gamma : [N, H] fp32
 *   S_in    : [N, H, d_k, d_v] fp32, or NULL for zeros
 *   S_out   : [N, H, d_k, d_v] fp32, required; may equal S_in (in place)
 *   o       : [N, H, d_v] dtype
 *
 * Supported: 1 <= d_k, d_v <= 128, N, H >= 1.  S_out may overlap S_in only
 * as the identical pointer; o may not overlap any input.
 */
eda_status_t eda_fwd_recurrent_step(const void *q, const void *k, const void *e, const void *v,
                                    const float *alpha, const float *beta, const float *gamma,
                                    const float *S_in, float *S_out, void *o,
                                    int N, int H, int d_k, int d_v, eda_dtype_t dtype,
                                    void *stream);

/*
 * Layer form: the same recurrence with the layer's prologue fused in (EDA
 * paper Fig. 1 and Eqs. (14)-(15); slides frames on the layer structure and
 * on the safe decay parameterization), for H_v value heads that share H_k
 * key heads (H_v a multiple of H_k; value head h reads key head
 * h / (H_v / H_k), as in the paper's models with 8/16 and 16/32 heads):
 *
 *   q, k, e <- x / max(||x||_2, 1e-6)       per token and key head (raw inputs)
 *   alpha    = exp(g),  g = l + (-l) exp(-(A / |l|) softplus(a + b)),
 *              A = exp(A_log), b = dt_bias, l = -5, per key channel,
 *
 * so e^-5 < alpha <= 1.  beta, gamma, v, o and the states are per value head.
 *
 *   q, k, e, a : [B, T, H_k, d_k]  dtype (a: the decay gate's input)
 *   A_log, dt_bias : [H_k, d_k]    fp32
 *   v : [B, T, H_v, d_v] dtype;  beta, gamma : [B, T, H_v] fp32
 *   S0, S_final : [B, H_v, d_k, d_v] fp32;  o : [B, T, H_v, d_v] dtype
 *
 * Everything else (chunk, workspace, aliasing, errors) is as for
 * eda_fwd_chunked, with the workspace sized by
 * eda_fwd_chunked_layer_workspace_size.  H_v not a multiple of H_k (or a
 * head count < 1) returns EDA_ERR_SHAPE.
 */
size_t eda_fwd_chunked_layer_workspace_size(int B, int T, int H_k, int H_v, int d_k, int d_v,
                                            eda_dtype_t dtype, int chunk);

eda_status_t eda_fwd_chunked_layer(const void *q, const void *k, const void *e, const void *v,
                                   const void *a, const float *A_log, const float *dt_bias,
                                   const float *beta, const float *gamma, const float *S0, void *o,
                                   float *S_final, int B, int T, int H_k, int H_v, int d_k, int d_v,
                                   eda_dtype_t dtype, int chunk, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * One decode token in layer form: as eda_fwd_recurrent_step with the prologue
 * above.  q, k, e, a : [N, H_k, d_k] dtype;  A_log, dt_bias : [H_k, d_k] fp32;
 * v : [N, H_v, d_v];  beta, gamma : [N, H_v];  S_in, S_out : [N, H_v, d_k, d_v];
 * o : [N, H_v, d_v].  Same checks and aliasing rules as eda_fwd_recurrent_step.
 */
eda_status_t eda_fwd_recurrent_step_layer(const void *q, const void *k, const void *e, const void *v,
                                          const void *a, const float *A_log, const float *dt_bias,
                                          const float *beta, const float *gamma, const float *S_in,
                                          float *S_out, void *o, int N, int H_k, int H_v, int d_k,
                                          int d_v, eda_dtype_t dtype, void *stream);

/*
 * Second workload: the rank-1 DPLR update of GDN-2 and QED (QED slides,
 * frames "GDN-2 separates decay, erase, and write" and "QED adds a query
 * term to the erase vector"), per head and token
 *
 *     Sbar_t = Diag(alpha_t) S_{t-1},   S_t = Sbar_t + k_t (v_t - Sbar_t^T a_t)^T,   o_t = S_t^T q_t,
 *
 * i.e. S_t = (I - k_t a_t^T) Diag(alpha_t) S_{t-1} + k_t v_t^T: decay, then a
 * rank-1 edit that reads along the erase vector a_t and writes along k_t.
 * The caller forms a_t (GDN-2: b_t o k_t; QED: b_t o k_t + lambda d_t with
 * d_t the gated query projected off k_t) and passes the gated value w_t o v_t
 * as v.  It runs on the same two chunked kernels as eda_fwd_chunked, with a
 * non-symmetric decayed Gram.
 *
 *   q, k, a : [B, T, H, d_k] dtype   v : [B, T, H, d_v] dtype
 *   alpha   : [B, T, H, d_k] fp32
 *   S0, S_final, o, chunk, workspace : as for eda_fwd_chunked (same
 *             workspace size, eda_fwd_chunked_workspace_size)
 *
 * Results are defined for finite inputs and alpha in (0, 1]; a and k are not
 * required to be unit or related.  Checks, aliasing rules and errors as for
 * eda_fwd_chunked.
 */
eda_status_t eda_fwd_chunked_dplr(const void *q, const void *k, const void *a, const void *v,
                                  const float *alpha, const float *S0, void *o, float *S_final,
                                  int B, int T, int H, int d_k, int d_v, eda_dtype_t dtype,
                                  int chunk, void *workspace, size_t workspace_bytes, void *stream);

/*
 * One decode token of the DPLR update above for N independent sequences:
 * q, k, a : [N, H, d_k] dtype;  v : [N, H, d_v];  alpha : [N, H, d_k] fp32;
 * S_in, S_out, o as for eda_fwd_recurrent_step (same checks and aliasing rules).
 */
eda_status_t eda_fwd_recurrent_step_dplr(const void *q, const void *k, const void *a, const void *v,
                                         const float *alpha, const float *S_in, float *S_out,
                                         void *o, int N, int H, int d_k, int d_v, eda_dtype_t dtype,
                                         void *stream);

/*
 * Backward pass of the recurrence above (training; the EDA paper trains its
 * models in BF16 with AdamW, Sec. 4).  Given the forward's inputs, the
 * gradient dO of the outputs and the gradient dS_final of the final state,
 * computes the gradients of L = <o, dO> + <S_T, dS_final> with respect to
 * q, k, e, v, alpha, beta, gamma and S0.  Each stage's adjoint:
 *
 *   dq = S_t dO_t,  w = G^T k,  dv = beta w,  dbeta = w.(v - r_k),
 *   dk = beta (G (v - r_k) - St w),  de = -gamma (dSt r_e + Sh z),  dgamma = -z.r_e,
 *   dalpha = rowsum(dSh o S_{t-1}),  dS_{t-1} = Diag(alpha) dSh,
 *
 * with G = dL/dS_t, Sh, St, r_e, r_k the decayed and erased states and reads
 * of the forward, dSt = G - beta k w^T, z = dSt^T e, dSh = dSt - gamma e z^T.
 * The states are recomputed from fp32 checkpoints (every 8 tokens) and the
 * per-token column sums of a first forward sweep, kept in the workspace; all
 * arithmetic is fp32.
 *
 *   q, k, e : [B, T, H, d_k] dtype;  v, dO : [B, T, H, d_v] dtype
 *   alpha : [B, T, H, d_k] fp32;  beta, gamma : [B, T, H] fp32
 *   S0, dS_final : [B, H, d_k, d_v] fp32 or NULL (zeros)
 *   dq, dk, de, dalpha : [B, T, H, d_k] fp32;  dv : [B, T, H, d_v] fp32
 *   dbeta, dgamma : [B, T, H] fp32;  dS0 : [B, H, d_k, d_v] fp32 or NULL
 *   workspace : eda_bwd_workspace_size(...) bytes, 256-byte aligned (about
 *               3.4 GB for B = 4, T = 2048, H = 16, d = 128)
 *
 * Supported: 1 <= d_k, d_v <= 128.  No output may overlap an input, the
 * workspace or another output.  Errors as for eda_fwd_chunked.
 */
size_t eda_bwd_workspace_size(int B, int T, int H, int d_k, int d_v);

eda_status_t eda_bwd(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                     const float *beta, const float *gamma, const float *S0, const void *dO,
                     const float *dS_final, float *dq, float *dk, float *de, float *dv, float *dalpha,
                     float *dbeta, float *dgamma, float *dS0, int B, int T, int H, int d_k, int d_v,
                     eda_dtype_t dtype, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EDA_H */
