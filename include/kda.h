/*
 * kda.h -- C ABI of libkda, the Kimi Delta Attention (KDA) operator for
 * AMD Instinct MI355X (gfx950).
 *
 * KDA is a gated delta-rule linear attention ("Kimi K3" explainer, "Across
 * the sequence"): per head it keeps a fixed-size state S[d_k][d_v] and, for
 * each token t in order,
 *     S   <- Diag(exp(g_t)) S                 channel-wise forgetting
 *     u_t  = beta_t (v_t - S^T k_t)
 *     S   <- S + k_t u_t^T
 *     o_t  = S^T q_t
 * with the bounded log-decay g_t = KDA_G_MIN * sigmoid(theta_t)
 * ("Architecture Deep Dive: Kimi K3...", section 3.2, equation 1; "Kimi K3
 * Deep Dive...", "The Design: Putting a Lower Bound on Log-Decay").
 *
 * Conventions shared by every call:
 *  - Pointers are DEVICE pointers into memory the caller owns (for instance
 *    torch tensors).  The library never allocates, frees or retains them.
 *    Its only global state is a thread-local error string and, for
 *    kda_chunk_fwd_noalloc, one static device scratch array per device.
 *  - Tensors are dense and row-major in the layouts stated per argument; the
 *    innermost dimension is contiguous.  Every pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued asynchronously on it; KDA_OK means "validated and
 *    enqueued".  Faults inside kernels surface at the caller's next
 *    synchronisation of that stream.
 *  - All argument checks run on the host before any HIP call, so every error
 *    return leaves device memory untouched and enqueues nothing.
 *  - Non-finite inputs are not checked; they propagate into the outputs.
 *  - Results are deterministic run to run (no floating-point atomics).
 *  - Supported head sizes: d_k = d_v in {16, 32, 64, 128}.
 *  - dtype of q, k, v and o: KDA_BF16 (bf16 storage, bf16 matrix-core
 *    operands, fp32 accumulation and fp32 state) or KDA_F32 (fp32 storage and
 *    fp32 arithmetic throughout; a validation mode).  fp16 is not offered:
 *    exp(16 * 5) = 5.5e34 exceeds its range.  theta, beta and the states are
 *    always fp32.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tokens per chunk of the chunked evaluation (the pages' 16-token tile). */
#define KDA_CHUNK 16
/* Fixed lower bound of the log-decay g (the pages set it to -5). */
#define KDA_G_MIN (-5.0f)
/* Version of this ABI; bumped on any incompatible change. */
#define KDA_ABI_VERSION 1

typedef enum kda_dtype { KDA_BF16 = 0, KDA_F32 = 1 } kda_dtype;

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,       /* a required pointer is NULL                         */
    KDA_ERR_SHAPE = 2,      /* a size is out of range or unsupported              */
    KDA_ERR_DTYPE = 3,      /* unknown dtype code                                 */
    KDA_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned                   */
    KDA_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required         */
    KDA_ERR_ALIAS = 6,      /* an output overlaps memory it must not overlap      */
    KDA_ERR_HIP = 7         /* the HIP runtime reported an error at launch        */
} kda_status;

/* ---------------------------------------------------------------------------
 * kda_chunk_fwd: chunked prefill ("Kimi K3 Deep Dive...", "The Problem: The
 * Diagonal-Block Dilemma": 16-token chunks with intra-chunk (diagonal) and
 * inter-chunk causal paths; the bounded gate lets both run as dense matrix
 * products, "Architecture Deep Dive", section 3.2).
 *
 * Runs the recurrence over T tokens for every (batch, head) from the start
 * state S0 and returns every output o_t and the final state S_T.
 *
 *   dtype        KDA_BF16 or KDA_F32 (storage of q, k, v, o)
 *   B, T, H      batch, tokens (T >= 1), heads; B, H >= 1
 *   dk, dv       head sizes, equal, in {16, 32, 64, 128}
 *   segments     how many pieces each sequence is cut into along T for
 *                parallel evaluation (each piece's affine state map is
 *                composed afterwards); 0 = the library's choice, which is
 *                what kda_chunk_fwd_auto_segments returns.  Any value from 1
 *                to ceil(T/16) gives the same result up to rounding.
 *   q, k         [B, T, H, dk]   dtype
 *   v            [B, T, H, dv]   dtype
 *   theta        [B, T, H, dk]   fp32; the gate applies KDA_G_MIN*sigmoid
 *   beta         [B, T, H]       fp32, used as given (no sigmoid applied)
 *   S0           [B, H, dk, dv]  fp32 start state, or NULL for zero
 *   o            [B, T, H, dv]   dtype, written
 *   S_T          [B, H, dk, dv]  fp32 final state, written; or NULL to skip.
 *                S_T may be the same pointer as S0 (in-place update); any
 *                other overlap between an output and an input is rejected.
 *   workspace    device scratch of at least kda_chunk_fwd_workspace_size
 *                bytes (may be NULL when that size is 0); contents on entry
 *                are ignored, on exit unspecified.
 *   stream       hipStream_t as void*
 * Returns a kda_status.
 * ------------------------------------------------------------------------- */
int kda_chunk_fwd(int dtype, int B, int T, int H, int dk, int dv, int segments,
                  const void* q, const void* k, const void* v,
                  const float* theta, const float* beta, const float* S0,
                  void* o, float* S_T,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch that kda_chunk_fwd_noalloc holds per device. */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)

/* ---------------------------------------------------------------------------
 * kda_chunk_fwd_noalloc: kda_chunk_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  It takes no workspace: a segmented call uses a static
 * device array of KDA_NOALLOC_SCRATCH_BYTES (128 MiB) that each device the
 * library runs on holds from its first call there until the process ends.
 * The call itself allocates and frees nothing.
 *
 *   Every argument and the result are those of kda_chunk_fwd, without
 *   workspace and workspace_bytes.  The scratch is the one of the calling
 *   thread's current device; `stream` must belong to that device.
 *   Errors: those of kda_chunk_fwd, and KDA_ERR_WORKSPACE when the segment
 *   count (given, or the automatic one for segments = 0) needs more than
 *   KDA_NOALLOC_SCRATCH_BYTES (kda_chunk_fwd_workspace_size gives the need;
 *   one segment needs none).  The 64K-token prefill of 16 heads at d = 128
 *   with its automatic 16 segments needs 110 MiB and fits.
 *   The scratch holds nothing that must start at zero and keeps the last
 *   call's contents.  Every call on one device shares that device's scratch:
 *   calls that overlap in time on one device (several streams or threads)
 *   race and give undefined results; serialise them.
 * ------------------------------------------------------------------------- */
int kda_chunk_fwd_noalloc(int dtype, int B, int T, int H, int dk, int dv, int segments,
                          const void* q, const void* k, const void* v,
                          const float* theta, const float* beta, const float* S0,
                          void* o, float* S_T, void* stream);

/* ---------------------------------------------------------------------------
 * kda_chunk_fwd_gated: kda_chunk_fwd with the output gate applied to o
 * ("Kimi K3" explainer, "Across the sequence": in the model, the attention
 * output is multiplied channel by channel, token by token, by a sigmoid of a
 * pre-activation computed from the layer's input):
 *     o_t[j] = sigmoid(z_t[j]) * (S_t^T q_t)[j]
 * The gate acts on the output only; S_T is the same as kda_chunk_fwd's.
 *
 *   z            [B, T, H, dv]   dtype, the gate's pre-activation; must be
 *                non-NULL and 16-byte aligned, and must not overlap o, S_T or
 *                the workspace.
 *   Every other argument, the workspace size and the errors are those of
 *   kda_chunk_fwd.  The ungated output is rounded to dtype, multiplied by the
 *   gate in fp32 and rounded again.
 * ------------------------------------------------------------------------- */
int kda_chunk_fwd_gated(int dtype, int B, int T, int H, int dk, int dv, int segments,
                        const void* q, const void* k, const void* v,
                        const float* theta, const float* beta, const float* S0,
                        const void* z, void* o, float* S_T,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * kda_chunk_fwd_unbounded: the ablation of the bound.  The same recurrence
 * with the conventional unbounded log-decay that the bounded gate replaces
 * ("Kimi K3 Deep Dive...", "The Design: Putting a Lower Bound on Log-Decay"):
 *     g = -softplus(theta) = -ln(1 + e^theta),   range (-inf, 0)
 * instead of KDA_G_MIN*sigmoid(theta).  The inverse cumulative decay inside a
 * chunk is then unbounded and can overflow any floating-point type, so the two
 * diagonal tiles are formed position by position in fp32 ("Architecture Deep
 * Dive...", section 3.1) instead of as matrix products; everything else is the
 * chunked evaluation of kda_chunk_fwd.  It exists to measure what the bound
 * buys, not for use in a model.
 *
 *   Arguments as kda_chunk_fwd, without segments (always one: no workspace),
 *   with the same validation and errors.  Where the unbounded gate drives a
 *   decay below fp32's range the result is the limit (the state forgets).
 * ------------------------------------------------------------------------- */
int kda_chunk_fwd_unbounded(int dtype, int B, int T, int H, int dk, int dv,
                            const void* q, const void* k, const void* v,
                            const float* theta, const float* beta, const float* S0,
                            void* o, float* S_T, void* stream);

/* ---------------------------------------------------------------------------
 * kda_chunk_bwd: the backward pass of kda_chunk_fwd.  For the scalar
 *     L = sum_t <do_t, o_t> + <dS_T, S_T>
 * it writes the gradients of L with respect to q, k, v, theta, beta and S0, by
 * the chain rule through the recurrence taken chunk by chunk (the chunk form of
 * "Kimi K3 Deep Dive...", "The Problem: The Diagonal-Block Dilemma", run in
 * reverse; the training step the pages' kernel design serves, "Architecture
 * Deep Dive...", section 3.2).  dtheta includes the gate's derivative
 * KDA_G_MIN * sigmoid(theta) (1 - sigmoid(theta)).
 *
 *   dtype, B, T, H, dk, dv, q, k, v, theta, beta, S0   as kda_chunk_fwd
 *   do           [B, T, H, dv]   dtype, gradient of L with respect to o
 *   dS_T         [B, H, dk, dv]  fp32, gradient with respect to S_T, or NULL (zero)
 *   dq, dk       [B, T, H, dk]   fp32, written
 *   dv           [B, T, H, dv]   fp32, written
 *   dtheta       [B, T, H, dk]   fp32, written
 *   dbeta        [B, T, H]       fp32, written
 *   dS0          [B, H, dk, dv]  fp32, written; or NULL to skip
 *   workspace    kda_chunk_bwd_workspace_size bytes of device memory (every
 *                chunk's start state, and at dk = 64 and 128 its U and
 *                V - K+ S tiles and the segment maps and boundary values, fp32);
 *                contents on entry do not matter
 *   stream       hipStream_t the work is enqueued on
 * Returns KDA_OK once enqueued.  Errors (before any HIP call): as kda_chunk_fwd;
 * every gradient output must not overlap an input, another output or the
 * workspace.  One workgroup per (batch, head) walks the chunks in order; with
 * at most 64 (batch, head) pairs and at least 64 chunks (dk = 64 and 128) each
 * sequence is split into segments joined by their affine maps, as in the
 * forward.  Results are deterministic run to run.
 * ------------------------------------------------------------------------- */
int kda_chunk_bwd(int dtype, int B, int T, int H, int dk, int dv,
                  const void* q, const void* k, const void* v,
                  const float* theta, const float* beta, const float* S0,
                  const void* do_, const float* dS_T,
                  float* dq, float* dk_, float* dv_, float* dtheta, float* dbeta, float* dS0,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace kda_chunk_bwd needs.  Writes *bytes; returns a kda_status. */
int kda_chunk_bwd_workspace_size(int B, int T, int H, int dk, int dv, size_t* bytes);

/* Bytes of workspace kda_chunk_fwd needs for these sizes and this segment
 * count (0 = automatic).  Writes *bytes; returns a kda_status. */
int kda_chunk_fwd_workspace_size(int B, int T, int H, int dk, int dv, int segments,
                                 size_t* bytes);

/* The segment count kda_chunk_fwd uses when passed 0 (depends on sizes only,
 * never on the device).  Returns it, or a value <= 0 for invalid sizes. */
int kda_chunk_fwd_auto_segments(int B, int T, int H, int dk, int dv);

/* ---------------------------------------------------------------------------
 * kda_decode_step: one token of the recurrence for every (batch, head), with
 * the fixed-size state updated in place ("Kimi K3" explainer, "Across the
 * sequence": the state does not grow with context length).
 *
 *   dtype        KDA_BF16 or KDA_F32 (storage of q, k, v, o)
 *   B, H         >= 1;  dk, dv as for kda_chunk_fwd
 *   q, k         [B, H, dk]      dtype
 *   v            [B, H, dv]      dtype
 *   theta        [B, H, dk]      fp32
 *   beta         [B, H]          fp32
 *   S            [B, H, dk, dv]  fp32, read and overwritten with the new state
 *   o            [B, H, dv]      dtype, written; must not overlap any input
 *   stream       hipStream_t as void*
 * Returns a kda_status.
 * ------------------------------------------------------------------------- */
int kda_decode_step(int dtype, int B, int H, int dk, int dv,
                    const void* q, const void* k, const void* v,
                    const float* theta, const float* beta,
                    float* S, void* o, void* stream);

/* ---------------------------------------------------------------------------
 * kda_decode_step_gated: kda_decode_step with the output gate of
 * kda_chunk_fwd_gated, o[j] = sigmoid(z[j]) * (S'^T q)[j], formed in fp32 and
 * rounded once to dtype.
 *
 *   z            [B, H, dv]      dtype; non-NULL, 16-byte aligned, and not
 *                overlapping o or S.
 *   Every other argument and the errors are those of kda_decode_step; the
 *   state update is the same.
 * ------------------------------------------------------------------------- */
int kda_decode_step_gated(int dtype, int B, int H, int dk, int dv,
                          const void* q, const void* k, const void* v,
                          const float* theta, const float* beta,
                          float* S, const void* z, void* o, void* stream);

/* ---------------------------------------------------------------------------
 * kda_gate: the bounded gate on its own ("Architecture Deep Dive", section 3.2,
 * equation 1; "Kimi K3 Deep Dive", illustrative code of the lower-bounded
 * log-decay).
 *
 *   B, T, H, dk  sizes (dk in {16, 32, 64, 128}), T >= 1
 *   theta        [B, T, H, dk] fp32
 *   g            [B, T, H, dk] fp32 or NULL: g = KDA_G_MIN * sigmoid(theta)
 *   g_cum        [B, T, H, dk] fp32 or NULL: inclusive prefix sum of g along T
 *                restarted at every 16-token chunk (t = 0, 16, 32, ...)
 *   At least one of g, g_cum must be non-NULL; neither may overlap theta or
 *   each other.
 * Returns a kda_status.
 * ------------------------------------------------------------------------- */
int kda_gate(int B, int T, int H, int dk, const float* theta, float* g, float* g_cum,
             void* stream);

/* Static description of a status code (never NULL). */
const char* kda_status_string(int status);

/* Thread-local detail about the last non-OK return on this thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
