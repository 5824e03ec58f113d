/*
 * kda.h -- C ABI of the KDA (gated delta-rule linear attention) library for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer keeps a d_k x d_v memory S per (sequence, head) and, for every
 * token t, applies
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * with a per-key-channel forget gate alpha_t in [0,1]^{d_k} and a scalar
 * write strength beta_t.  (KDA update rule: "Hybrid Linear Attention
 * Architectures: Breaking Through the Long-Context Engineering Bottleneck in
 * LLMs", Core Module Design, Stage 3; "Linear Attention KDA Gating in a 3:1
 * Hybrid Architecture: Principles and Implementation Guide", section 2,
 * item 5: decay each key channel first, then overwrite along k.)  The rows
 * of S are key channels; the write is beta k v^T and the read-out S^T q is
 * taken after the token's own write (token i sees tokens j <= i: same page,
 * section 3.2).  No query scaling is applied.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, owned by the caller, row-major
 *    and contiguous, 16-byte aligned (beta: 4-byte aligned).  The library never allocates, never
 *    frees and keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; nothing synchronises the host.
 *    Calls on different streams with disjoint outputs may run concurrently.
 *  - Argument errors (NULL pointer, bad size, misalignment, unsupported
 *    dtype or head size, workspace too small) are detected on the host
 *    before anything is launched; the call then returns the status and has
 *    launched nothing.  A failed kernel launch returns KDA_ERROR_LAUNCH.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Data VALUES are not validated.  Preconditions: alpha in [0, 1] (any
 *    value, exact 0 included: each (chunk, head) of the chunkwise forward
 *    runs either a direct form whose rescaled operands are checked to stay
 *    in range, or a general form in which every decay factor is a product of
 *    alpha over a run of tokens, never above 1; decode uses products of
 *    alpha only; so fast forgetting only underflows toward its exact limit),
 *    beta in [0, 1]; for 16-bit activations every |q|, |k|, |v| and every
 *    state entry stays below 6.0e4 (half-precision range of the matrix-core
 *    operands);
 *    cu_seqlens is non-decreasing with cu_seqlens[0] = 0 and
 *    cu_seqlens[N] = T.  kda_chunk_bwd has a narrower gate precondition,
 *    stated at its declaration.
 *  - Supported: d_k in {64, 128}, d_v in {64, 128}; chunk_size 64 for
 *    every call, and also 32 or 128 for the chunkwise forward (a generic
 *    path with every product in fp32; at chunk size 128 with 16-bit
 *    activations it keeps the state entering each chunk and U' in fp16 in
 *    the workspace; the result is the same recurrence, the chunk size only
 *    changes how the work is cut).
 *    Activations (q, k, v) are either all fp32 or all bf16; alpha, beta and
 *    every state are fp32.  The output o is fp32, or bf16 when the
 *    activations are bf16 (rounded once, to nearest-even, from the fp32
 *    accumulator).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KDA_API __attribute__((visibility("default")))
#else
#define KDA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,      /* NULL pointer, negative or inconsistent size, misalignment */
    KDA_ERROR_NOT_SUPPORTED = 2,      /* head size, chunk size or dtype combination not built    */
    KDA_ERROR_WORKSPACE_TOO_SMALL = 3,
    KDA_ERROR_LAUNCH = 4              /* a kernel launch failed (hipGetLastError)                */
} kda_status;

typedef enum {
    KDA_DTYPE_F32 = 0,
    KDA_DTYPE_BF16 = 1
} kda_dtype;

/*
 * Form of the forget gate passed to the *_gated entry points.
 *   KDA_GATE_ALPHA          alpha itself: fp32, one value per key channel
 *                           ([..., Dk]), in [0, 1].  The plain entry points
 *                           take this form.
 *   KDA_GATE_SOFTPLUS_BF16  the gate's pre-activation x: bf16, one value per
 *                           key channel ([..., Dk]), with
 *                           log alpha = -softplus(x) = -log(1 + e^x), so
 *                           alpha = 1 / (1 + e^x) lies in (0, 1).  Half the
 *                           gate bytes of KDA_GATE_ALPHA; the kernels form
 *                           alpha (or log alpha) from x without rounding
 *                           alpha to fp32 first.
 *   KDA_GATE_SCALAR         alpha fp32, ONE value per token and head
 *                           ([..., 1], i.e. the layout of beta), in [0, 1],
 *                           applied to every key channel: the coarse scalar
 *                           gate of Gated DeltaNet ("Hybrid Linear Attention
 *                           Architectures...", Core Module Design, Stage 2).
 * The pages compute the gating parameters inside each chunk from the layer
 * inputs ("Hybrid Linear Attention Architectures...", Hardware-Aware
 * Chunkwise Parallelism, implementation checklist; "Linear Attention KDA
 * Gating...", section 3.3); they print no activation function, and
 * -softplus is the log-sigmoid form with alpha in (0, 1).
 */
typedef enum {
    KDA_GATE_ALPHA = 0,
    KDA_GATE_SOFTPLUS_BF16 = 1,
    KDA_GATE_SCALAR = 2
} kda_gate;

/* Human-readable name of a status code (static string, never NULL). */
KDA_API const char *kda_status_string(kda_status s);

/*
 * Workspace size, in bytes, that kda_chunk_fwd needs for this problem.
 * Same arguments as kda_chunk_fwd (num_seqs is ignored when `varlen` is 0).
 * Returns 0 for argument combinations kda_chunk_fwd would reject.
 * The workspace holds the chunk table and the per-(chunk, head)
 * intermediates; it must be 256-byte aligned and its contents need not be
 * initialised.  One workspace must not be shared by calls that may overlap.
 */
KDA_API size_t kda_chunk_fwd_workspace_bytes(int B, int64_t T, int H, int Dk, int Dv,
                                     int varlen, int num_seqs, int chunk_size,
                                     kda_dtype act_dtype);

/*
 * Chunkwise-parallel forward (prefill / training forward).
 *
 * Follows the chunked algorithm of "Linear Attention KDA Gating in a 3:1
 * Hybrid Architecture", section 3 (inter-chunk state transition 3.1 and
 * masked intra-chunk output 3.2) and the "Hardware-Aware Chunkwise
 * Parallelism" section of "Hybrid Linear Attention Architectures...": the
 * sequence is cut into chunks of `chunk_size` tokens; inside a chunk the
 * work is dense matrix products, and only the d_k x d_v state passes from
 * one chunk to the next.  The result equals the token-by-token recurrence
 * above up to rounding.
 *
 * Layout (contiguous):
 *   q, k       [B, T, H, Dk]   act_dtype
 *   v          [B, T, H, Dv]   act_dtype
 *   alpha      [B, T, H, Dk]   fp32, in [0, 1]
 *   beta       [B, T, H]       fp32, in [0, 1]
 *   o          [B, T, H, Dv]   out_dtype (written for every token)
 *   initial_state [N, H, Dk, Dv] fp32, or NULL for zeros
 *   final_state   [N, H, Dk, Dv] fp32, or NULL (not written); it may be the
 *                 same pointer as initial_state (updated in place).
 * Sequences:
 *   cu_seqlens == NULL: N = B independent sequences of length T.
 *   cu_seqlens != NULL: device int32 [num_seqs + 1] prefix offsets of
 *                 num_seqs sequences packed along T; B must be 1 and
 *                 N = num_seqs.  Zero-length sequences are allowed (their
 *                 final state equals their initial state).  Chunks never
 *                 cross a sequence boundary.
 * T may be 0 (then only final_state := initial_state is written).
 */
KDA_API kda_status kda_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta,
                         const float *initial_state, float *final_state,
                         const int32_t *cu_seqlens, int num_seqs,
                         void *o,
                         int B, int64_t T, int H, int Dk, int Dv, int chunk_size,
                         kda_dtype act_dtype, kda_dtype out_dtype,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * kda_chunk_fwd with the forget gate in any form of kda_gate: `gate` takes
 * the place of `alpha` (layouts: [B, T, H, Dk] for KDA_GATE_ALPHA and
 * KDA_GATE_SOFTPLUS_BF16, [B, T, H] for KDA_GATE_SCALAR; alignment 16, 8
 * and 4 bytes).  Everything else is as for kda_chunk_fwd, which is this call
 * with KDA_GATE_ALPHA.  Any finite pre-activation x is allowed for
 * KDA_GATE_SOFTPLUS_BF16.
 */
KDA_API kda_status kda_chunk_fwd_gated(const void *q, const void *k, const void *v,
                         const void *gate, kda_gate gate_kind, const float *beta,
                         const float *initial_state, float *final_state,
                         const int32_t *cu_seqlens, int num_seqs,
                         void *o,
                         int B, int64_t T, int H, int Dk, int Dv, int chunk_size,
                         kda_dtype act_dtype, kda_dtype out_dtype,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * kda_chunk_fwd_gated for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): there is no workspace argument; the workspace is a static
 * device array of KDA_STATIC_WORKSPACE_BYTES inside the library, one copy per
 * GPU, reserved when the library's code is loaded on that GPU and held until
 * the process ends.  The call allocates nothing.  Arguments, layouts,
 * preconditions and results are those of kda_chunk_fwd_gated; `stream`
 * selects the GPU (the current GPU for the null stream).
 *   - A problem whose kda_chunk_fwd_workspace_bytes exceeds
 *     KDA_STATIC_WORKSPACE_BYTES is rejected with
 *     KDA_ERROR_WORKSPACE_TOO_SMALL before anything is launched (64 MiB:
 *     e.g. 900 chunk-heads of 64 tokens at d = 128 with bf16 activations).
 *   - Every call on one GPU uses that GPU's one array, whatever the stream:
 *     calls that may overlap on one GPU (other streams, other host threads)
 *     race and must be ordered by the caller.  The array needs no clearing:
 *     every value a call uses from it, the same call has written first.
 *   - The first call on a GPU looks up that GPU's copy of the array
 *     (hipGetSymbolAddress); KDA_ERROR_LAUNCH if that lookup fails.
 */
#define KDA_STATIC_WORKSPACE_BYTES (64u << 20)

KDA_API kda_status kda_chunk_fwd_static(const void *q, const void *k, const void *v,
                         const void *gate, kda_gate gate_kind, const float *beta,
                         const float *initial_state, float *final_state,
                         const int32_t *cu_seqlens, int num_seqs,
                         void *o,
                         int B, int64_t T, int H, int Dk, int Dv, int chunk_size,
                         kda_dtype act_dtype, kda_dtype out_dtype,
                         void *stream);

/*
 * Workspace size, in bytes, that kda_chunk_bwd needs for this problem (same
 * arguments as kda_chunk_fwd_workspace_bytes).  Returns 0 for argument
 * combinations kda_chunk_bwd would reject.  256-byte alignment; contents
 * need not be initialised; not to be shared by calls that may overlap.
 * Per (chunk, head), with C = chunk_size: (3 C d_k + 3 C d_v + 2 d_k d_v +
 * 2 C^2 + d_k) * 4 bytes for fp32 activations, 14 C d_k + 8 C d_v +
 * 4 d_k d_v + 6 C^2 + 4 d_k bytes for bf16 (each rounded up to 256), plus
 * 8 bytes (the list of chunks that take the general form, and a flag).
 */
KDA_API size_t kda_chunk_bwd_workspace_bytes(int B, int64_t T, int H, int Dk, int Dv,
                                     int varlen, int num_seqs, int chunk_size,
                                     kda_dtype act_dtype);

/*
 * Chunkwise backward (training): the gradients of
 *     L = sum(dout * o) + sum(dfinal_state * S_T)
 * with respect to every input of kda_chunk_fwd_gated, for the same inputs.
 * The pages present the chunk algorithm as the training form ("Hybrid
 * Linear Attention Architectures...", Hardware-Aware Chunkwise Parallelism;
 * "Linear Attention KDA Gating in a 3:1 Hybrid Architecture", section 3);
 * this is the chain rule through that chunked forward, chunk by chunk from
 * the last, carrying only the state gradient between chunks.  The forward
 * is recomputed inside the call (nothing has to be kept from it).
 *
 * Inputs, as for kda_chunk_fwd_gated (same layouts, alignment, sequences,
 * preconditions): q, k, v, gate (form gate_kind), beta, initial_state
 * (NULL = zeros), cu_seqlens / num_seqs.  Gate precondition of this call:
 * alpha in (0, 1], any decay strength.  A (chunk, head) in which every
 * channel's decay over the chunk stays within 2^-64 runs in the direct
 * form (Gamma and 1/Gamma of the chunk as fp32 factors); any other in the
 * general form, whose decay factors never exceed 1.  The gate gradient is
 * formed from dL/dlog(alpha): dL/dalpha = dL/dlog(alpha) / alpha, whose
 * absolute error is that of dL/dlog(alpha) times 1/alpha, while the
 * softplus form's dL/dx = -sigmoid(x) dL/dlog(alpha) keeps the accuracy of
 * dL/dlog(alpha) at every alpha.  Upstream gradients:
 *   dout          [B, T, H, Dv]  act_dtype
 *   dfinal_state  [N, H, Dk, Dv] fp32, or NULL for zeros
 * Outputs (written for every token; none may overlap an input):
 *   dq, dk        [B, T, H, Dk]  act_dtype (bf16: rounded once, nearest-even)
 *   dv            [B, T, H, Dv]  act_dtype
 *   dgate         fp32, the shape of gate: dL/dalpha for KDA_GATE_ALPHA,
 *                 dL/dx for KDA_GATE_SOFTPLUS_BF16, dL/da for KDA_GATE_SCALAR
 *   dbeta         [B, T, H]      fp32
 *   dinitial_state [N, H, Dk, Dv] fp32 dL/dS_0, or NULL (not written)
 * q, k, v, dout, dq, dk, dv, the states and their gradients are 16-byte
 * aligned; dgate and dbeta 4-byte aligned.  Accumulation is fp32
 * throughout; with fp32 activations every operand is fp32, with bf16 the
 * products of the two state passes and of the value-side contractions take
 * fp16 operands; the key-side products keep fp32 operands (the largest run
 * on the bf16 matrix cores with each operand split into bf16 hi + lo).
 */
KDA_API kda_status kda_chunk_bwd(const void *q, const void *k, const void *v,
                         const void *gate, kda_gate gate_kind, const float *beta,
                         const float *initial_state,
                         const int32_t *cu_seqlens, int num_seqs,
                         const void *dout, const float *dfinal_state,
                         void *dq, void *dk, void *dv, float *dgate, float *dbeta,
                         float *dinitial_state,
                         int B, int64_t T, int H, int Dk, int Dv, int chunk_size,
                         kda_dtype act_dtype,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * One recurrent decode step: every one of N sequences consumes one token and
 * its fp32 state is updated in place ("recurrent kernels for linear
 * attention" of "Linear Attention + Sparse Attention: The Hybrid
 * Architecture Trade-off for Large Models", section 6; the token-by-token
 * mode of "Linear Attention KDA Gating...", section 3).  Each state is read
 * once and written once.
 *
 * Layout (contiguous):
 *   q, k   [N, H, Dk]  act_dtype      v [N, H, Dv] act_dtype
 *   alpha  [N, H, Dk]  fp32           beta [N, H] fp32
 *   state  [N, H, Dk, Dv] fp32, read and overwritten
 *   o      [N, H, Dv]  out_dtype
 * N may be 0 (nothing is launched); N * H must stay below 2^30.
 */
KDA_API kda_status kda_recurrent_step(const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta,
                              float *state, void *o,
                              int N, int H, int Dk, int Dv,
                              kda_dtype act_dtype, kda_dtype out_dtype,
                              void *stream);

/*
 * kda_recurrent_step with the forget gate in any form of kda_gate (layouts
 * [N, H, Dk], or [N, H] for KDA_GATE_SCALAR; alignment 16, 8 and 4 bytes).
 * kda_recurrent_step is this call with KDA_GATE_ALPHA.  N * H must stay
 * below 2^30.
 */
KDA_API kda_status kda_recurrent_step_gated(const void *q, const void *k, const void *v,
                              const void *gate, kda_gate gate_kind, const float *beta,
                              float *state, void *o,
                              int N, int H, int Dk, int Dv,
                              kda_dtype act_dtype, kda_dtype out_dtype,
                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
