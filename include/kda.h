/*
 * kda.h - C ABI of the Kimi Delta Attention (KDA) operator for MI355X (gfx950).
 *
 * The operator (Kimi Linear review notes, research-notes-dl6.pages.dev,
 * section "Method / from Linear Attention to KDA", the KDA recurrence):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,      alpha_t = exp(g_t) in [0,1]^dk,
 *
 * computed per sequence and head, with a dk x dv fp32 state S per (sequence,
 * head).  The same page's "Training and Inference" section routes long
 * prompts to the chunkwise kernel and single decode steps to the fused
 * recurrent kernel, with the recurrent state cached between calls; both are
 * exported here.  `scale` is 1 in the pages' formula.
 *
 * General conventions for every entry point:
 *  - Every tensor pointer is a DEVICE pointer to contiguous row-major memory
 *    with the layout given below, aligned to 16 bytes.  The caller owns all
 *    memory, including the workspace; the library never allocates, frees,
 *    synchronises or keeps a pointer after the call returns.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  The call returns after enqueueing.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    any error nothing is launched and a status other than KDA_OK is
 *    returned (no exception crosses the ABI).  kda_last_error() then gives a
 *    thread-local message.  Values inside tensors are not validated: g <= 0
 *    (alpha <= 1), finite inputs and a non-decreasing cu_seqlens are
 *    preconditions, and violating them gives unspecified numbers (never an
 *    out-of-bounds access: every index the kernels form is clamped to the
 *    sizes passed here).
 *  - Results are deterministic (no atomics in any reduction): the same
 *    inputs give the same bits on every run.
 *  - Functions are thread-safe; concurrent calls on different streams are
 *    independent.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7

/*
 * Optional input transforms, applied inside the kernels to every token before
 * the recurrence (`flags` of both argument structs; 0 applies none).  The
 * Kimi Linear review notes' parameterization table has the Q/K L2
 * normalization fused into the KDA kernel, and the public tests it lists
 * cover a fused gate (section "Code Verification").
 *
 * KDA_FLAG_QK_L2NORM: q_t and k_t are divided by sqrt(sum_i x_i^2 + 1e-6)
 *   over their dk channels, per token and head, in fp32 (the pages give no
 *   epsilon; 1e-6 is this library's).
 * KDA_FLAG_GATE_SOFTPLUS: g holds gate logits z and the log-gate used is
 *   -gate_scale * softplus(z), softplus(z) = log(1 + exp(z)), so that
 *   alpha = (1 + e^z)^-gate_scale.  gate_scale must be finite and >= 0.
 * KDA_FLAG_SCALAR_GATE: g holds one value per token and head, [B, T, H]
 *   ([N, H] for a decode step), applied to every key channel: the scalar
 *   forget gate of Gated DeltaNet, which the review notes' "Method" section
 *   names as the case KDA refines channel by channel.  Combines with the
 *   other flags.
 *
 * Structs of ABI version 1 (struct_size equal to the offset of `flags`) are
 * still accepted and apply no transform.
 */
#define KDA_FLAG_QK_L2NORM 1u
#define KDA_FLAG_GATE_SOFTPLUS 2u
#define KDA_FLAG_SCALAR_GATE 4u
#define KDA_L2NORM_EPS 1e-6f

typedef enum {
    KDA_DTYPE_BF16 = 0, /* bfloat16, round-to-nearest-even on output */
    KDA_DTYPE_FP32 = 1
} kda_dtype;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1,        /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,           /* a size is negative or inconsistent */
    KDA_ERR_UNSUPPORTED = 3,         /* dk/dv/dtype/chunk size not supported */
    KDA_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes below what is required */
    KDA_ERR_BAD_STRUCT = 5,          /* struct_size does not match this library */
    KDA_ERR_HIP = 6,                 /* a HIP launch failed; see kda_last_error() */
    KDA_ERR_ALIAS = 7                /* the output overlaps an input */
} kda_status;

/*
 * Chunkwise-parallel prefill (Kimi Linear review notes, section "Chunkwise
 * Algorithm"; jxzklqfsx.com article, section on the hardware-efficient
 * chunkwise algorithm): the sequence is cut into chunks of `chunk_size`
 * tokens that never straddle two sequences; inside a chunk the decayed
 * K K^T and Q K^T blocks, the UT-transform inverse and the WY factors are
 * formed in parallel, and only the fp32 state crosses chunk boundaries.
 *
 * Shapes (N = number of sequences):
 *   q, k : [B, T, H, dk]  in_dtype
 *   v    : [B, T, H, dv]  in_dtype
 *   g    : [B, T, H, dk]  fp32, log of the per-channel forget gate (alpha = exp(g)),
 *                         or gate logits with KDA_FLAG_GATE_SOFTPLUS; [B, T, H]
 *                         with KDA_FLAG_SCALAR_GATE
 *   beta : [B, T, H]      in_dtype, the per-token, per-head write strength
 *   initial_state : [N, H, dk, dv] fp32, or NULL for zeros
 *   final_state   : [N, H, dk, dv] fp32, or NULL to skip; may equal initial_state
 *                   (each state slice is read before it is written)
 *   o    : [B, T, H, dv]  out_dtype; must not overlap any input
 *   cu_seqlens : NULL for B fixed-length sequences of T tokens (N = B), or a
 *                DEVICE int32 array [N+1] of token offsets for packed
 *                variable-length input (then B must be 1, cu_seqlens[0] = 0,
 *                cu_seqlens[N] = T, non-decreasing; empty sequences allowed,
 *                their final state equals their initial state).
 *   dk, dv : 64 or 128 (dk may differ from dv).
 *   chunk_size : 64 (16 and 32 are accepted as well).
 *   workspace : device scratch of at least kda_chunk_fwd_workspace_bytes()
 *               bytes (may be NULL when that is 0); its contents on entry
 *               are ignored and on exit are unspecified.  Two calls in
 *               flight at once must not share a workspace.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(kda_chunk_fwd_args) */
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const void *beta;
    const float *initial_state;
    float *final_state;
    void *o;
    const int32_t *cu_seqlens;
    int32_t B, T, H, dk, dv, num_seqs; /* num_seqs = N (must equal B when cu_seqlens is NULL) */
    float scale;
    kda_dtype in_dtype;  /* dtype of q, k, v, beta */
    kda_dtype out_dtype; /* dtype of o */
    int32_t chunk_size;
    void *workspace;
    size_t workspace_bytes;
    void *stream;     /* hipStream_t */
    uint32_t flags;   /* KDA_FLAG_* input transforms (ABI version 2) */
    float gate_scale; /* used with KDA_FLAG_GATE_SOFTPLUS */
} kda_chunk_fwd_args;

/* Bytes of workspace kda_chunk_fwd needs for these arguments (host-only, no
 * HIP call, only the size fields are read).  Returns (size_t)-1 when the
 * arguments are invalid. */
size_t kda_chunk_fwd_workspace_bytes(const kda_chunk_fwd_args *args);

kda_status kda_chunk_fwd(const kda_chunk_fwd_args *args);

/*
 * Multi-token fused recurrent forward (Kimi Linear review notes, section
 * "Training and Inference": segments of at most 64 tokens, as well as single
 * decode steps, go to the fused recurrent kernel, which keeps the recurrent
 * state in registers for the whole segment).  The same recurrence as
 * kda_chunk_fwd, computed token by token in order: per (sequence, head,
 * 16-column slice of dv) one wave reads its state slice once, applies every
 * token of the sequence, and writes the slice once.  Fixed-length input of one
 * token per sequence runs as a decode step, with the same result bit for bit
 * as kda_recurrent_step.  Meant for short appends
 * (speculative decoding, a few tokens per sequence): on MI355X it is the
 * faster path up to about 16 new tokens per sequence, and kda_chunk_fwd from
 * about 64 on.
 *
 * Arguments, shapes, dtypes, aliasing rules and errors are those of
 * kda_chunk_fwd; chunk_size is ignored.  The workspace is optional: when
 * workspace is given with at least kda_chunk_fwd_workspace_bytes() bytes for
 * chunk size 64 and the call carries more than 16 tokens per sequence on
 * average, it runs kda_chunk_fwd (chunk 64) instead, the faster path there;
 * its results then carry kda_chunk_fwd's rounding.  Without a workspace (or
 * a large enough one) the call always runs token by token.
 */
kda_status kda_recurrent_fwd(const kda_chunk_fwd_args *args);

/*
 * One recurrent decode step for N independent sequences (Kimi Linear review
 * notes, section "Training and Inference": the fused recurrent kernel serves
 * single steps and keeps the fixed-size recurrent state in the cache).
 * Per (n, h): S~ = Diag(exp(g)) S;  S' = S~ + beta k (v - S~^T k)^T;
 * o = scale * S'^T q.  Each state slice is read once and written once.
 *
 * Shapes:
 *   q, k : [N, H, dk] in_dtype;  v : [N, H, dv] in_dtype;  g : [N, H, dk] fp32
 *          (log-gate, or gate logits with KDA_FLAG_GATE_SOFTPLUS; [N, H] with
 *          KDA_FLAG_SCALAR_GATE)
 *   beta : [N, H] in_dtype
 *   initial_state : [N, H, dk, dv] fp32, or NULL for zeros
 *   final_state   : [N, H, dk, dv] fp32, required; may equal initial_state
 *                   (in-place update of the cached state)
 *   o : [N, H, dv] out_dtype
 *   dk, dv : 64 or 128.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(kda_recurrent_step_args) */
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const void *beta;
    const float *initial_state;
    float *final_state;
    void *o;
    int32_t N, H, dk, dv;
    float scale;
    kda_dtype in_dtype;
    kda_dtype out_dtype;
    void *stream;     /* hipStream_t */
    uint32_t flags;   /* KDA_FLAG_* input transforms (ABI version 2) */
    float gate_scale; /* used with KDA_FLAG_GATE_SOFTPLUS */
} kda_recurrent_step_args;

kda_status kda_recurrent_step(const kda_recurrent_step_args *args);

/*
 * Gradients of the recurrence (the backward pass of kda_chunk_fwd and
 * kda_recurrent_fwd, with the same input transforms): for the loss gradients
 * grad_o = dL/do and grad_final_state = dL/dS_T, the gradients of L with
 * respect to q, k, v, g, beta and the initial state.  Reverse-mode
 * differentiation of the recurrence of the Kimi Linear review notes
 * (section "Method", the KDA recurrence): going backwards through the tokens
 * with dS = dL/dS_t,
 *     dS += scale q do^T,  dq = scale S_t do,  u = v - S~^T k,  du = beta dS^T k,
 *     dv = du,  dbeta = k^T dS u,  dk = beta dS u - S~ du,
 *     dS~ = dS - k du^T,  dg = rowsum(S~ .* dS~),  dS <- Diag(exp(g)) dS~,
 * with S~ = Diag(exp(g_t)) S_{t-1}; the initial-state gradient is the final dS.
 *
 * Computed in fp32.  Long sequences are cut into segments as in
 * kda_chunk_fwd: a token-by-token fp32 pass gives each segment's transition
 * and local state, which kda_chunk_fwd's combine chains into the state
 * entering each segment, and the state-gradient recurrence, which needs no
 * forward state, is chained backwards over the segments through the
 * transposed segment transitions.  Every segment then runs token by token in parallel
 * (one workgroup per segment and head, one wave per 16 columns of dv); its
 * forward states are recomputed, not read from the forward pass: every 8th
 * one is stored in the workspace on a first sweep, and each group of 8 is
 * rebuilt from it on the way back.
 *
 * Shapes (N = number of sequences):
 *   q, k, v, g, beta, initial_state, cu_seqlens, B, T, H, dk, dv, num_seqs,
 *           scale, in_dtype : as in kda_chunk_fwd (g: [B, T, H, dk] log-gates,
 *           or [B, T, H] with KDA_FLAG_SCALAR_GATE)
 *   grad_o : [B, T, H, dv] in_dtype
 *   grad_final_state : [N, H, dk, dv] fp32, or NULL for zeros
 *   grad_q, grad_k : [B, T, H, dk] fp32;  grad_g : the shape of g, fp32
 *   grad_v : [B, T, H, dv] fp32;  grad_beta : [B, T, H] fp32
 *   grad_initial_state : [N, H, dk, dv] fp32, or NULL to skip; may equal
 *           initial_state or grad_final_state (each slice is read before it
 *           is written); must not overlap anything else.
 *   The other gradients must not overlap any input, the workspace or each
 *   other.  Every gradient element of every token is written.
 *   workspace : device scratch of at least kda_recurrent_bwd_workspace_bytes()
 *               bytes, about (B*T / 8 + 3 B*T / 64) * H * dk * dv * 4 (one
 *               stored state per 8 tokens, plus state-sized buffers for the
 *               segment chain); contents on entry ignored, on exit
 *               unspecified.
 *   flags, gate_scale : the KDA_FLAG_* input transforms of the forward call.
 *           KDA_FLAG_SCALAR_GATE: g and grad_g are [B, T, H] (the scalar gate's
 *           gradient is the sum over key channels).  KDA_FLAG_QK_L2NORM and
 *           KDA_FLAG_GATE_SOFTPLUS: grad_q, grad_k and grad_g are gradients of
 *           the raw q, k and gate logits, carried back through the L2 norm
 *           (dx = (dx^ - x^ (x^ . dx^)) / r) and through -gate_scale softplus
 *           (dz = dloggate * (-gate_scale sigmoid(z))); the workspace then also
 *           holds fp32 copies of the transformed inputs.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(kda_recurrent_bwd_args) */
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const void *beta;
    const float *initial_state;
    const void *grad_o;
    const float *grad_final_state;
    float *grad_q;
    float *grad_k;
    float *grad_v;
    float *grad_g;
    float *grad_beta;
    float *grad_initial_state;
    const int32_t *cu_seqlens;
    int32_t B, T, H, dk, dv, num_seqs;
    float scale;
    kda_dtype in_dtype; /* dtype of q, k, v, beta and grad_o */
    void *workspace;
    size_t workspace_bytes;
    void *stream; /* hipStream_t */
    uint32_t flags;
    float gate_scale; /* used with KDA_FLAG_GATE_SOFTPLUS */
} kda_recurrent_bwd_args;

/* Bytes of workspace kda_recurrent_bwd needs (host-only; only the size fields
 * are read).  Returns (size_t)-1 when the arguments are invalid. */
size_t kda_recurrent_bwd_workspace_bytes(const kda_recurrent_bwd_args *args);

kda_status kda_recurrent_bwd(const kda_recurrent_bwd_args *args);

/*
 * The same gradients by the chunk path (Kimi Linear review notes, section
 * "Training and Inference": training always runs the chunkwise kernels; the
 * gradients are those of the recurrence above), recomputing the forward
 * chunk by chunk on matrix cores.  Per chunk of 64 tokens with entering
 * state S, leaving-state gradient dS' and output gradient dO, the chunk form
 * of kda_chunk_fwd differentiates to
 *     dV_new = A_qk^T dO + Kd dS',   dS = gamma * dS' + Q^T dO - W^T dV_new,
 * (Q = scale exp(G) q, Kd = exp(G_last - G) k, W and A_qk as in the forward
 * chunk form) and the remaining gradients are products local to the chunk:
 * through V_new = U - W S, the WY factors [W | U] = T beta [exp(G) k | v],
 * T = (I + A_kk)^{-1}, and the decayed Gram products A_kk, A_qk, with a
 * reverse cumulative sum inside the chunk for dg.
 *
 * Passes: kda_chunk_fwd's operand packs, local pass and combine; a forward
 * replay keeping every chunk's entering state and V_new; the state-gradient
 * recurrence walked backwards over the chunks with its own segmented scan
 * (the transposed segment transitions carry it across segments); then one
 * workgroup per chunk and head for everything local to the chunk.  The
 * state recurrences run on fp16 operands with fp32 accumulation like
 * kda_chunk_fwd; the chunk-local products in fp32.
 *
 * Arguments: as kda_recurrent_bwd, with in_dtype = KDA_DTYPE_BF16,
 * dk = dv = 128 and flags = 0 (no input transforms); anything else returns
 * KDA_ERR_UNSUPPORTED (kda_recurrent_bwd covers it).  grad_initial_state may
 * equal initial_state or grad_final_state.  workspace : at least
 * kda_chunk_bwd_workspace_bytes() bytes, about 3.2 KiB per token and head
 * (the operand packs, and per chunk the state, V_new, the state gradient and
 * dV_new in fp32); contents on entry ignored, on exit unspecified.  Every
 * gradient element of every token is written.
 */
size_t kda_chunk_bwd_workspace_bytes(const kda_recurrent_bwd_args *args);

kda_status kda_chunk_bwd(const kda_recurrent_bwd_args *args);

/*
 * The general diagonal-plus-low-rank (DPLR) recurrence, token by token.  The
 * Kimi Linear review notes (section "Chunkwise Algorithm") give KDA's
 * transition as a DPLR matrix with D = Diag(alpha_t), a_t = beta_t k_t and
 * b_t = k_t .* alpha_t; this entry point runs the family's general member,
 * with a_t and b_t free, per sequence and head:
 *
 *     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,
 *     o_t = scale * S_t^T q_t,          alpha_t = exp(g_t).
 *
 * KDA is the case a = beta k, b = alpha .* k with write key beta k.  Computed
 * in fp32 by one wave per (sequence, head, 16 columns of dv), which reads its
 * state slice once and writes it once; meant, like kda_recurrent_fwd, for
 * short segments.
 *
 * Shapes (N = number of sequences):
 *   q, k, a, b : [B, T, H, dk] in_dtype;  v : [B, T, H, dv] in_dtype
 *   g    : [B, T, H, dk] fp32 log-decay (alpha = exp(g) <= 1)
 *   initial_state, final_state, o, cu_seqlens, B, T, H, dk, dv, num_seqs,
 *   scale, out_dtype: as in kda_chunk_fwd (final_state may equal
 *   initial_state; o must not overlap any input).
 * No workspace.  No input transform.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(kda_dplr_args) */
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const void *a;
    const void *b;
    const float *initial_state;
    float *final_state;
    void *o;
    const int32_t *cu_seqlens;
    int32_t B, T, H, dk, dv, num_seqs;
    float scale;
    kda_dtype in_dtype;  /* dtype of q, k, v, a, b */
    kda_dtype out_dtype; /* dtype of o */
    void *stream;        /* hipStream_t */
} kda_dplr_args;

kda_status kda_dplr_recurrent_fwd(const kda_dplr_args *args);

/*
 * The same general DPLR recurrence in chunkwise-parallel form, on fp32
 * matrix cores, in the harness of kda_chunk_fwd's fp32 path (same segment
 * table, local and output passes, combine).  The Kimi Linear review notes
 * (section "Chunkwise Algorithm") time KDA's chunk operator against general
 * DPLR's at about half the time; the jxzklqfsx.com article's efficiency
 * section puts the difference in the chunk algorithm: four secondary-chunk
 * products for the general form against two for KDA, and three more matrix
 * products.  Here, per chunk of C rows with cumulative log decay G
 * (G_{-1} = 0) and entering state S:
 *
 *   B_k[r,i] = b_r.(k_i e^{G_{r-1}-G_i}), B_a[r,i] = b_r.(a_i e^{G_{r-1}-G_i})   (i <  r)
 *   A_qk[r,i]= q_r.(k_i e^{G_r-G_i}),     A_qa[r,i]= q_r.(a_i e^{G_r-G_i})       (i <= r)
 *   X = (I + B_a)^{-1} ((b e^{G_{r-1}}) S + B_k V)       (the rows x_r = S_{r-1}^T b_r)
 *   O = scale ((q e^G) S + A_qk V - A_qa X)
 *   S <- e^{G_L} S + (e^{G_L - G} k)^T V - (e^{G_L - G} a)^T X
 *
 * Chunks of 32 tokens: five [C][dk] fp32 operands sit in LDS at once, which
 * at dk = 128 fits only C = 32.  Results equal kda_dplr_recurrent_fwd's up
 * to rounding.
 *
 * Arguments as kda_dplr_args, plus a workspace of at least
 * kda_dplr_chunk_fwd_workspace_bytes() bytes (contents on entry ignored, on
 * exit unspecified; must not overlap any input or output).  final_state may
 * equal initial_state.
 */
typedef struct {
    uint32_t struct_size; /* = sizeof(kda_dplr_chunk_args) */
    const void *q;
    const void *k;
    const void *v;
    const float *g;
    const void *a;
    const void *b;
    const float *initial_state;
    float *final_state;
    void *o;
    const int32_t *cu_seqlens;
    int32_t B, T, H, dk, dv, num_seqs;
    float scale;
    kda_dtype in_dtype;  /* dtype of q, k, v, a, b */
    kda_dtype out_dtype; /* dtype of o */
    void *workspace;
    size_t workspace_bytes;
    void *stream; /* hipStream_t */
} kda_dplr_chunk_args;

/* Bytes of workspace kda_dplr_chunk_fwd needs (host-only; only the size
 * fields are read).  Returns (size_t)-1 when the arguments are invalid. */
size_t kda_dplr_chunk_fwd_workspace_bytes(const kda_dplr_chunk_args *args);

kda_status kda_dplr_chunk_fwd(const kda_dplr_chunk_args *args);

/*
 * kda_chunk_fwd without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results, aliasing
 * rules and errors as kda_chunk_fwd, except that `workspace` and
 * `workspace_bytes` are ignored: the scratch lives in a device array of
 * KDA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  Nothing is allocated, freed or synchronised.
 *
 * Limit: problems whose kda_chunk_fwd_workspace_bytes() exceeds
 * KDA_NOALLOC_SCRATCH_BYTES are rejected with KDA_ERR_WORKSPACE_TOO_SMALL
 * before any launch.  With bf16 inputs and dk = dv = 128 the operand packs
 * bound it: 2,048 tokens x 16 heads fit, 2,560 do not.  The fp32 path keeps
 * only segment states there: 65,536 tokens x 16 heads at dk = dv = 128 fit.
 *
 * Every call on one GPU uses that GPU's array: calls that overlap in time on
 * the same GPU (different streams or host threads) race and must be
 * serialised by the caller.  The array keeps the last call's contents; none
 * of it needs to start at zero.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunk_fwd_noalloc(const kda_chunk_fwd_args *args);
/* KDA_NOALLOC_SCRATCH_BYTES of the loaded library. */
size_t kda_chunk_fwd_noalloc_max_workspace_bytes(void);

/* Static text for a status code. */
const char *kda_status_string(kda_status s);
/* Thread-local text describing the last failure on this thread ("" if none):
 * for KDA_ERR_HIP the failing launch and HIP's own error string, for every
 * other status the argument that was rejected.  Valid until the next call
 * on the same thread. */
const char *kda_last_error(void);
/* The same text under the name the boundary's specification uses for the
 * HIP error behind KDA_ERR_HIP. */
const char *kda_last_hip_error(void);
/* KDA_ABI_VERSION of the loaded library. */
int kda_abi_version(void);
/* The same number under the specification's name. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
