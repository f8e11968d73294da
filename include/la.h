/*
 * la.h -- C ABI of liblinattn: causal kernelized linear attention in
 * fast-weight form on AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h, tokens i = 0..N-1):
 *
 *   S_i = lambda_h * S_{i-1} + phi(k_i) v_i^T          state,      [F x d_v]
 *   z_i = lambda_h * z_{i-1} + phi(k_i)                normaliser, [F]
 *   y_i = phi(q_i)^T S_i / (phi(q_i)^T z_i + eps)
 *
 * The state is updated with token i before it is queried by token i.
 * Sources: "Attention is also an FFN" (kwkr.cn/news/587576) sec. 2.1 (fast
 * weight state and its outer-product recurrence), sec. 3.2 (decay lambda),
 * sec. 4.2 (normaliser z, eps, decay applied to z as well); "From standard
 * attention to linear attention" (tqpw.cn/news/561043) sec. 3 (S and Z,
 * non-causal form), sec. 4.1 (elu+1), sec. 4.2 (random cos/sin features),
 * sec. 6 (state layout, autoregressive step).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are row-major and contiguous: q, k [B,H,N,d_k]; v, y [B,H,N,d_v];
 *    state S [B,H,F,d_v] fp32 and z [B,H,F] fp32.  F = d_k for LA_PHI_ELU1 and
 *    LA_PHI_RELU, F = 2m for the random-feature maps.  Every device pointer
 *    must be 16-byte aligned.
 *  - The caller owns and allocates every device buffer, including the
 *    workspace sized by la_workspace_size().  The library never allocates,
 *    frees or synchronises.  Descriptors and lambda_h are host memory, read
 *    only during the call.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    null stream).  For fixed shapes the result is bitwise deterministic.
 *  - Validation happens on the host before anything is enqueued.  On failure
 *    a non-zero la_status is returned, la_last_error() describes it, and
 *    nothing is enqueued.  A failed launch returns LA_ERR_HIP.  Device faults
 *    surface at the caller's next synchronisation.
 *  - Support matrix: d_k, d_v in {64, 128}; random features with m in {32, 64,
 *    128} (F = 2m) and d_k * m <= 8192; in_dtype LA_BF16 or LA_F32; out_dtype
 *    equal to in_dtype or LA_F32.  m = 256 (F = 512, the last point of the
 *    m sweep in "From standard attention to linear attention" sec. 7) is
 *    supported by the causal forward entry points (fixed, masked, packed and
 *    no-allocation) for bf16 inputs with d_k = d_v = 64: the library runs it as
 *    two halves of 128 directions and the workspace also holds d_v + 1 floats
 *    per output row.  Other valid shapes return LA_ERR_UNSUPPORTED.
 *  - H <= LA_MAX_HEADS; lambda_h values must lie in [0, 1] (0^0 is taken as 1);
 *    eps must be finite and >= 0.
 */
#ifndef LA_H_
#define LA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream handle (hipStream_t); NULL selects the null stream. */
typedef struct ihipStream_t* la_stream_t;

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARGUMENT = 1,  /* malformed call: null pointer, bad size, lambda or eps */
    LA_ERR_UNSUPPORTED = 2,       /* valid but outside the support matrix                */
    LA_ERR_WORKSPACE = 3,         /* workspace missing or smaller than la_workspace_size */
    LA_ERR_HIP = 4                /* a HIP launch failed; la_last_error() has the text   */
} la_status;

enum { LA_F32 = 0, LA_BF16 = 1 };             /* element types of q, k, v, y */
/* feature maps */
enum {
    LA_PHI_ELU1 = 0,
    LA_PHI_TRIG_RF = 1,
    LA_PHI_RELU = 2,
    LA_PHI_TRIG_RF_PLAIN = 3,
    LA_PHI_TRIG_RF_SOFTMAX = 4
};

#define LA_MAX_HEADS 256

/* Feature map descriptor.
 *  LA_PHI_ELU1   : phi(x)_f = x_f + 1 if x_f > 0, else exp(x_f)  ("From standard
 *                  attention to linear attention" sec. 4.1: elu with alpha 1, plus
 *                  one).  m = 0, omega = NULL, qk_scale must be 1.
 *  LA_PHI_TRIG_RF: x' = qk_scale * x, u = omega x',
 *                  phi(x) = exp(-|x'|^2 / 2) / sqrt(m) [cos u_1..u_m, sin u_1..u_m]
 *                  (same page, sec. 4.2).  omega is a device pointer to an fp32
 *                  [m, d_k] row-major matrix supplied by the caller (the random
 *                  directions are an input: draw them once from a fixed seed and
 *                  share them).  qk_scale is typically d_k^(-1/4).
 *  LA_PHI_RELU   : phi(x)_f = max(x_f, 0)  ("Attention is also an FFN", sec. 5.1,
 *                  beside elu+1 as a map with a controlled range).  m = 0,
 *                  omega = NULL, qk_scale must be 1.  A query whose features are
 *                  all zero has output 0 (numerator 0, denominator eps).
 *  LA_PHI_TRIG_RF_PLAIN, LA_PHI_TRIG_RF_SOFTMAX: as LA_PHI_TRIG_RF with the
 *                  prefactor 1/sqrt(m) (the section's exp(|x|^2/2) h(x) with
 *                  h = exp(-|x|^2/2): a Gaussian-kernel estimate) or
 *                  exp(+|x'|^2/2)/sqrt(m) (h = 1: an estimate of exp(x'.y')).  */
typedef struct {
    int32_t kind;
    int32_t m;
    const float* omega;
    float qk_scale;
} la_phi;

/* Problem shape and element types.  For la_decode_step N is the number of
 * tokens per head-state, 1 <= N <= LA_DECODE_MAX_TOKENS. */
#define LA_DECODE_MAX_TOKENS 64
typedef struct {
    int64_t B, H, N;
    int32_t d_k, d_v;
    int32_t in_dtype, out_dtype;
} la_shape;

/* Zero the state: S[B,H,F,d_v] = 0 and z[B,H,F] = 0 (fp32, device memory).
 * "Attention is also an FFN" sec. 4.1 and "From standard attention to linear
 * attention" sec. 6: the recurrent state starts at zero.  Implemented with a
 * fill kernel (no hipMemset node), so it may be recorded into a HIP graph.
 * Either pointer may be NULL to skip that buffer. */
la_status la_init_state(float* S, float* z, int64_t B, int64_t H, int32_t F, int32_t d_v,
                        la_stream_t stream);

/* Identity-initialised state ("Attention is also an FFN" sec. 6: start S at
 * the identity or near it, a default history, rather than at zero):
 * S[b,h,f,d] = alpha if f == d else 0 (a rectangular identity when F != d_v)
 * and z[b,h,f] = alpha for f < min(F, d_v), else 0 -- the state left by
 * min(F, d_v) virtual tokens with phi(k) = e_f and v = e_f at weight alpha, so
 * that numerator and normaliser describe the same history.  alpha must be
 * finite.  Fill kernel, no hipMemset node (graph-capturable).  Either pointer
 * may be NULL to skip that buffer. */
la_status la_init_state_identity(float* S, float* z, int64_t B, int64_t H, int32_t F, int32_t d_v,
                                 float alpha, la_stream_t stream);

/* Bytes of device workspace that la_forward_causal (causal != 0) or
 * la_forward_noncausal (causal == 0) needs for this shape; 0 when none is
 * needed.  Returns 0 for shapes that fail validation as well. */
size_t la_workspace_size(const la_shape* shape, const la_phi* phi, int32_t causal);

/* Causal forward over [B,H,N,d].
 * q, k, v: device inputs of shape->in_dtype; y: device output [B,H,N,d_v] of
 * shape->out_dtype, must not alias q, k or v.  lambda_h: host array [H] of
 * per-head decays, NULL means lambda = 1 for every head.  S_in [B,H,F,d_v] /
 * z_in [B,H,F]: optional initial state (both NULL = zero state; both or none).
 * S_out / z_out: optional final state (both or none); S_out may equal S_in and
 * z_out may equal z_in for an in-place carry.  N = 0 copies S_in to S_out (or
 * zeroes S_out) and returns LA_OK.
 * Method ("Attention is also an FFN" sec. 4.1 and sec. 5.2: cut the sequence
 * into chunks, parallel inside a chunk, carried across chunks): the sequence
 * is cut into chunks of C tokens; inside a chunk the decayed, masked scores
 * phi(Q) phi(K)^T and their product with V run on matrix cores, the chunk
 * reads the carried state, and the state is carried forward as
 * S <- lambda^n S + sum_j lambda^(n-1-j) phi(k_j) v_j^T.  Long sequences are
 * additionally split into segments whose states are combined by a scan. */
la_status la_forward_causal(const void* q, const void* k, const void* v, void* y,
                            const la_shape* shape, const la_phi* phi,
                            const float* lambda_h, float eps,
                            const float* S_in, const float* z_in,
                            float* S_out, float* z_out,
                            void* workspace, size_t workspace_bytes, la_stream_t stream);

/* la_forward_causal for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and arguments without the workspace.  The
 * segment states live in a static device array of LA_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every device it runs on until the process
 * ends; the call allocates nothing.  The number of segments is capped so that
 * their states fit it (fewer segments: less parallelism, the same result up
 * to rounding order).  A window carry state (LA_WINDOWS > 1) that does not fit
 * on its own is LA_ERR_WORKSPACE.  All calls on one device share its array:
 * calls that overlap on one device (several streams or threads) race and must
 * be serialised by the caller. */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)
la_status la_forward_causal_noalloc(const void* q, const void* k, const void* v, void* y,
                                    const la_shape* shape, const la_phi* phi,
                                    const float* lambda_h, float eps,
                                    const float* S_in, const float* z_in,
                                    float* S_out, float* z_out, la_stream_t stream);

/* Non-causal forward ("From standard attention to linear attention" sec. 3
 * and sec. 6): S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j) over the whole
 * sequence (no decay), then y_i = phi(q_i)^T S / (phi(q_i)^T z + eps).
 * Arguments as for la_forward_causal.  N must be >= 1. */
la_status la_forward_noncausal(const void* q, const void* k, const void* v, void* y,
                               const la_shape* shape, const la_phi* phi, float eps,
                               void* workspace, size_t workspace_bytes, la_stream_t stream);

/* Causal forward with a key padding mask ("From standard attention to linear
 * attention" sec. 6 gives the forward a key padding mask).  As
 * la_forward_causal, plus key_padding_mask: device bytes [B,N]; a nonzero
 * byte drops key n of batch b from every sum -- its term phi(k_n) v_n^T and
 * phi(k_n) never enter S or z, in the outputs or the final state.  Positions
 * keep their indices: the decay between two kept keys is still
 * lambda^(distance).  A query whose kept history is empty reads only the
 * initial state (y = 0 from a zero state).  Workspace: la_workspace_size with
 * causal = 1.  A NULL mask is LA_ERR_INVALID_ARGUMENT (use la_forward_causal). */
la_status la_forward_causal_masked(const void* q, const void* k, const void* v, void* y,
                                   const la_shape* shape, const la_phi* phi,
                                   const float* lambda_h, float eps,
                                   const uint8_t* key_padding_mask,
                                   const float* S_in, const float* z_in,
                                   float* S_out, float* z_out,
                                   void* workspace, size_t workspace_bytes, la_stream_t stream);

/* Causal forward over packed sequences of different lengths.
 * shape->B is the number of sequences, shape->N the packed token count T:
 * q, k: [H,T,d_k], v: [H,T,d_v], y: [H,T,d_v] (one row of T tokens per head),
 * and sequence b holds tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 of every
 * head's row.  cu_seqlens: device int32 [B+1], non-decreasing from 0 and at
 * most T (the kernels clamp every offset to [0, T], so other values cannot
 * address memory outside the rows, but their results are unspecified).  Each
 * sequence is an independent causal problem (the recurrence of
 * la_forward_causal restarted at its first token) with its own initial state
 * S_in[b] / z_in[b] and final state S_out[b] / z_out[b] ([B,H,F,d_v] and
 * [B,H,F]; same rules as la_forward_causal).  Output rows outside every
 * sequence are not written.  max_seqlen (host, 0 <= max_seqlen <= T): the
 * longest sequence; it sizes the segment split and the workspace
 * (la_workspace_size_varlen, never 0 for T > 0: it holds the table of work
 * items) -- results do not depend on it, only speed. */
size_t la_workspace_size_varlen(const la_shape* shape, int64_t max_seqlen, const la_phi* phi);
la_status la_forward_causal_varlen(const void* q, const void* k, const void* v, void* y,
                                   const int32_t* cu_seqlens, int64_t max_seqlen,
                                   const la_shape* shape, const la_phi* phi,
                                   const float* lambda_h, float eps,
                                   const float* S_in, const float* z_in,
                                   float* S_out, float* z_out,
                                   void* workspace, size_t workspace_bytes, la_stream_t stream);

/* Cross attention, non-causal ("From standard attention to linear attention"
 * sec. 2: N queries against M keys and values; sec. 3 and sec. 6 for the
 * form): per (b,h), S = sum_j phi(k_j) v_j^T and z = sum_j phi(k_j) over the
 * n_kv keys that key_padding_mask keeps, then y_i = phi(q_i)^T S /
 * (phi(q_i)^T z + eps) for the shape->N queries.  q: [B,H,N,d_k], k:
 * [B,H,n_kv,d_k], v: [B,H,n_kv,d_v], y: [B,H,N,d_v]; key_padding_mask: NULL or
 * device bytes [B,n_kv], nonzero = the key is ignored.  N >= 1, n_kv >= 1.
 * Workspace: la_workspace_size_cross (sized by n_kv). */
size_t la_workspace_size_cross(const la_shape* shape, int64_t n_kv, const la_phi* phi);
la_status la_forward_cross(const void* q, const void* k, const void* v, void* y,
                           const la_shape* shape, int64_t n_kv,
                           const uint8_t* key_padding_mask, const la_phi* phi, float eps,
                           void* workspace, size_t workspace_bytes, la_stream_t stream);

/* Gradients of la_forward_causal (training: "Attention is also an FFN"
 * sec. 4.1 and 5.2 train with the chunked form).  For the loss
 *   L = sum_i dy_i . y_i + <dS_out, S_final> + <dz_out, z_final>
 * writes dq, dk [B,H,N,d_k] and dv [B,H,N,d_v] (input type), and, if given,
 * dS_in [B,H,F,d_v] / dz_in [B,H,F] fp32, the gradient of the initial state.
 * q, k, v, y, dy: device inputs of shape->in_dtype; y is the forward's output
 * for the same q, k, v, lambda_h, eps, key_padding_mask and S_in / z_in, and
 * shape->out_dtype must equal shape->in_dtype.  dS_out / dz_out: optional
 * gradient of the final state (both or none; NULL = 0).  Outputs must not
 * alias inputs or each other.  Feature maps: all kinds.  The random-feature
 * kinds ("From standard attention to linear attention" sec. 4.2) run the
 * same sweeps on phi(q), phi(k) computed first (F = 2m in the role of d_k,
 * supported for F * d_v <= 256 * 128 with bf16 inputs and F <= 128 with fp32
 * inputs) and map the resulting d phi back through omega:
 * dx = s (omega^T g + sigma x' (phi . d phi)), g_r = c (cos u_r d phi_{m+r} -
 * sin u_r d phi_r), with x' = s x, u = omega x', c the prefactor and sigma its
 * sign (-1, 0, +1 by kind).  dlambda: optional device fp32 [H], the
 * gradient of lambda_h summed over the batch (NULL = not computed; not
 * available for fp32 inputs with d_k = d_v = 128, LA_ERR_UNSUPPORTED).
 * Method: with dnum_i = dy_i / den_i and dden_i = -(dy_i . y_i) / den_i,
 * dq comes from a chunked sweep in token order that carries the forward
 * state (d phi(q_i) = S_i dnum_i + z_i dden_i), dk and dv from a chunked
 * sweep in reverse order that carries the adjoint
 * U_j = sum_{i>=j} lambda^(i-j) phi(q_i) dnum_i^T (d phi(k_j) = U_j v_j + u_j,
 * dv_j = U_j^T phi(k_j)); long rows are cut into segments joined by scans.
 * dlambda follows the product rule through the chunks: the dq sweep also
 * carries T = dS/dlambda, and a reduction joins the segments.
 * Workspace: la_workspace_size_backward bytes (8 bytes per token plus the
 * segment states; random features add phi(q), phi(k), d phi(q) and
 * d phi(k) in the input type, B*H*N*2m values each). */
size_t la_workspace_size_backward(const la_shape* shape, const la_phi* phi);
la_status la_backward_causal(const void* q, const void* k, const void* v,
                             const void* y, const void* dy,
                             void* dq, void* dk, void* dv,
                             const la_shape* shape, const la_phi* phi,
                             const float* lambda_h, float eps,
                             const uint8_t* key_padding_mask,
                             const float* S_in, const float* z_in,
                             const float* dS_out, const float* dz_out,
                             float* dS_in, float* dz_in, float* dlambda,
                             void* workspace, size_t workspace_bytes, la_stream_t stream);

/* Gradients of la_forward_cross (and of la_forward_noncausal: n_kv = N with
 * the same rows for keys and queries).  Training with the non-causal form:
 * "From standard attention to linear attention" sec. 3 and 6 for the form,
 * "Attention is also an FFN" sec. 4.1 and 5.2 for training it.  For the loss
 * L = sum_i dy_i . y_i, with S, z the sums over the kept keys and
 * dnum_i = dy_i / den_i, dden_i = -(dy_i . y_i) / den_i:
 *   dq_i: J_phi(q_i)^T (S dnum_i + z dden_i),
 *   U = sum_i phi(q_i) dnum_i^T, u = sum_i phi(q_i) dden_i over the queries,
 *   dk_j: J_phi(k_j)^T (U v_j + u),  dv_j = U^T phi(k_j)
 * (a padded key gets dk = dv = 0).  q, y, dy, dq: [B,H,N,d_*]; k, v, dk, dv:
 * [B,H,n_kv,d_*]; all device, in shape->in_dtype (out_dtype must equal it);
 * y is la_forward_cross's output for the same q, k, v, key_padding_mask and
 * eps.  Outputs must not alias inputs or each other.  Feature maps: all
 * kinds; the random-feature kinds as in la_backward_causal (the sweeps run on
 * phi(q), phi(k), d phi returns through omega).  N >= 1, n_kv >= 1.
 * Method: three passes -- the state sums over the keys (as the forward), a
 * sweep over the queries that writes dq and sums the adjoint per segment, a
 * sweep over the keys that reads the total adjoint -- with two small
 * reductions joining the segments.  Workspace:
 * la_workspace_size_backward_cross bytes (segment states; random features
 * add phi and d phi of the queries and keys, as la_backward_causal). */
size_t la_workspace_size_backward_cross(const la_shape* shape, int64_t n_kv, const la_phi* phi);
la_status la_backward_cross(const void* q, const void* k, const void* v,
                            const void* y, const void* dy,
                            void* dq, void* dk, void* dv,
                            const la_shape* shape, int64_t n_kv,
                            const uint8_t* key_padding_mask, const la_phi* phi, float eps,
                            void* workspace, size_t workspace_bytes, la_stream_t stream);

/* Recurrent decode steps, in place ("From standard attention to linear
 * attention" sec. 6 autoregressive step, with the decay of "Attention is also
 * an FFN" sec. 3.2): per (b,h), for each of the N tokens in order
 *   S <- lambda_h S + phi(k) v^T,  z <- lambda_h z + phi(k),
 *   y  = phi(q)^T S / (phi(q)^T z + eps).
 * q, k: [B,H,N,d_k]; v: [B,H,N,d_v]; y: [B,H,N,d_v]; S [B,H,F,d_v] and
 * z [B,H,F] fp32 are read once and overwritten once.  1 <= shape->N <=
 * LA_DECODE_MAX_TOKENS (longer runs: la_forward_causal with S_in = S_out).
 * With bf16 inputs, an elementwise map and at least 10 tokens (11 where
 * F * d_v >= 128 * 128) the call runs the causal forward's kernels over its
 * tokens from S back into S (the same result up to rounding: the state's
 * contribution to the outputs is then read from a bf16 copy, as in
 * la_forward_causal); other calls run the recurrent decode kernel, whose
 * state stays fp32 throughout. */
la_status la_decode_step(const void* q, const void* k, const void* v, void* y,
                         float* S, float* z, const la_shape* shape, const la_phi* phi,
                         const float* lambda_h, float eps, la_stream_t stream);

/* Measurement hooks (for benchmarks; not needed to compute anything).
 * Between la_profile_begin() and la_profile_end(), every kernel this library
 * launches from the calling thread records its own dispatch start and end
 * timestamps into a pair of HIP events (hipExtLaunchKernelGGL), so each
 * launch's device time can be read back.  A call that launches nothing (an
 * empty copy) records nothing.
 * la_profile_begin creates 2*max_launches events (host-side runtime objects;
 * no device memory); launches beyond max_launches are not recorded.
 * la_profile_end waits for the last recorded event, writes up to `capacity`
 * (kernel id, milliseconds) pairs in launch order, sets *count to the number
 * recorded, destroys the events and turns recording off.  Calling
 * la_profile_begin twice without la_profile_end is LA_ERR_INVALID_ARGUMENT. */
enum {
    LA_KERNEL_FWD_LOCAL = 0,   /* segment-local state pass of a forward        */
    LA_KERNEL_FWD_CAUSAL = 1,  /* chunked causal output pass                   */
    LA_KERNEL_FWD_QUERY = 2,   /* non-causal output pass                       */
    LA_KERNEL_SCAN = 3,        /* segment state scan / reduction               */
    LA_KERNEL_DECODE = 4,      /* recurrent decode step                        */
    LA_KERNEL_FILL = 5,        /* zero fill (la_init_state, empty forward)     */
    LA_KERNEL_COPY = 6,        /* state copy (empty forward)                   */
    LA_KERNEL_BWD_Q = 7,       /* backward: dq sweep                           */
    LA_KERNEL_BWD_RLOCAL = 8,  /* backward: adjoint segment sums               */
    LA_KERNEL_BWD_KV = 9,      /* backward: dk, dv sweep                       */
    LA_KERNEL_BWD_DLAM = 10,   /* backward: lambda-gradient reduction          */
    LA_KERNEL_VARLEN_ITEMS = 11, /* packed sequences: table of work items      */
    LA_KERNEL_BWD_NCQ = 12,    /* non-causal backward: dq and adjoint sums     */
    LA_KERNEL_BWD_NCKV = 13,   /* non-causal backward: dk, dv                  */
    LA_KERNEL_RF_FEATURES = 14, /* random-feature backward: phi(q), phi(k)     */
    LA_KERNEL_RF_VJP = 15      /* random-feature backward: dq, dk from d phi   */
};
la_status la_profile_begin(int32_t max_launches);
la_status la_profile_end(int32_t* kernel_ids, float* ms, int32_t capacity, int32_t* count);
/* Name of a kernel id: the device function's symbol prefix, or for the three
 * forward passes, which run different kernels by shape, the pass ("segment
 * state pass", "causal output pass", "non-causal output pass"). */
const char* la_kernel_name(int32_t kernel_id);

/* Static description of a status code. */
const char* la_status_string(la_status status);

/* Thread-local detail of the last non-OK status returned on this thread
 * ("" when none).  The pointer stays valid until the next call on the thread. */
const char* la_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LA_H_ */
