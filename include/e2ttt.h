/*
 * e2ttt.h -- C ABI of the MI355X (gfx950) E2-TTT chunk-update library.
 *
 * Operation ("Rethinking Expressivity and Efficiency in Test-Time Training",
 * E2-TTT; abstract, and the atlas summary's "Approach"): the fast weight W of
 * every (batch, head) is updated token by token with per-token learning rate
 * eta_t, momentum beta_t and decay alpha_t,
 *
 *     M_t = beta_t * M_{t-1} + eta_t * g_t,     W_t = alpha_t * W_{t-1} - M_t,
 *
 * where g_t is the gradient of token t's fast-weight loss taken at the weights
 * the token's chunk started with.  The library evaluates the closed-form
 * chunk transition that gives the exact chunk-end (W, M) of that recurrence
 * (a momentum kernel and a weight kernel from log-space suffix sums of
 * log alpha and log beta, then two coefficient-weighted gradient
 * aggregations) and the chunk output y_t = f_{W_chunk_start}(q_t) (arxivlens
 * "Limitations": the output stays fixed within a chunk).
 *
 * Fast weights (per head; k, q, v are D-vectors):
 *   E2TTT_LINEAR  y = W k                         W [D][D]
 *   E2TTT_MLP     y = W2 silu(W1 k)               W1 [Hd][D], W2 [D][Hd]
 *   E2TTT_SWIGLU  y = (silu(k W1) * (k W3)) W2    W1, W3 [D][Hd], W2 [Hd][D]
 * Losses: E2TTT_LOSS_MSE 0.5*||y - v||^2, E2TTT_LOSS_NEGDOT -<y, v>.
 * The per-(b,h) parameter vector packs the matrices in the order listed,
 * each row-major fp32: P = D*D, 2*D*Hd or 3*D*Hd floats.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises.  Work is queued on
 *     `stream` (a hipStream_t; NULL = the null stream) and runs
 *     asynchronously.
 *   - Return values report argument validation synchronously; a failed
 *     kernel launch returns E2TTT_ERR_HIP.  No exception crosses the ABI.
 *   - NaN/Inf in the inputs propagate; the hot path performs no checks.
 *   - The library keeps no mutable global state other than the scratch of
 *     e2ttt_chunk_forward_noalloc; calls on different streams may run
 *     concurrently as long as they do not share output or workspace buffers
 *     (or, for e2ttt_chunk_forward_noalloc, the GPU).  Path 4 (see
 *     e2ttt_path) needs all its workgroups resident at once: concurrent
 *     path-4 calls whose grids together exceed the device's compute units
 *     can hold part of each other's grid; their waits then end after 10 s
 *     and the affected final states are NaN.
 */
#ifndef E2TTT_H
#define E2TTT_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define E2TTT_API __attribute__((visibility("default")))
#else
#define E2TTT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { E2TTT_LINEAR = 0, E2TTT_MLP = 1, E2TTT_SWIGLU = 2 } e2ttt_kind;
typedef enum { E2TTT_LOSS_MSE = 0, E2TTT_LOSS_NEGDOT = 1 } e2ttt_loss;
typedef enum { E2TTT_F32 = 0, E2TTT_BF16 = 1 } e2ttt_dtype; /* dtype of q, k, v, out */

typedef enum {
    E2TTT_OK = 0,
    E2TTT_ERR_INVALID_ARG = 1, /* bad enum or flag, negative size, null or misaligned pointer */
    E2TTT_ERR_UNSUPPORTED = 2, /* shape outside what any kernel handles (e.g. D > 256, Hd > 1024) */
    E2TTT_ERR_ALIAS = 3,       /* an output overlaps an input or another output */
    E2TTT_ERR_WORKSPACE = 4,   /* workspace null or smaller than e2ttt_workspace_size() */
    E2TTT_ERR_HIP = 5,         /* a kernel launch failed */
    E2TTT_ERR_SCRATCH_LIMIT = 6 /* e2ttt_chunk_forward_noalloc: the call needs more than
                                   E2TTT_NOALLOC_SCRATCH_BYTES of scratch */
} e2ttt_status;

/* flags */
#define E2TTT_FLAG_FORCE_GENERIC 1 /* run the portable fp32 kernel even where the MFMA path applies */
/* No momentum: the recurrence W_t = alpha_t W_{t-1} - eta_t g_t (the official
 * code's token weights without momentum, as named on the codewithpapers page
 * of "Rethinking Expressivity and Efficiency in Test-Time Training").  beta,
 * M0 and M_end are not used and may be NULL; the chunk transition is
 * W_end = prod(alpha) W0 - sum_t alpha(t:end] eta_t g_t. */
#define E2TTT_FLAG_NO_MOMENTUM 2
/* Chunk average: the chunk-averaged ablation of the same paper (atlas summary,
 * "Surprising findings"), read as: the per-token momentum and weight kernels
 * m_t, w_t are replaced by their mean over the chunk; each token keeps its
 * own eta_t, and the chunk scalars prod alpha, prod beta, gamma are
 * unchanged.  Combines with NO_MOMENTUM. */
#define E2TTT_FLAG_CHUNK_AVG 4
/* Save states for the backward (training): with this flag the forward and
 * the backward share one workspace, sized by e2ttt_workspace_size() ==
 * e2ttt_backward_workspace_size() for the flagged desc.  The forward leaves
 * in it what the backward needs (scalar kernels and every chunk's start
 * state); a following e2ttt_chunk_backward with the same desc (flag
 * included), the same inputs and the untouched workspace skips its forward
 * recompute.  Unsupported (E2TTT_ERR_UNSUPPORTED) where the backward is. */
#define E2TTT_FLAG_SAVE_STATES 8
/* Precise operands on the SwiGLU MFMA path (e2ttt_path 2).  The default MFMA
 * path rounds the chunk-start weights (grad operands) and the
 * coefficient-scaled per-token factors (aggregation operands) to bf16, 8
 * significant bits.  While the state decays fast (the stated gates with a
 * strongly driven momentum) the chunk-to-chunk transition amplifies those
 * roundings: over 3-4 chunks the output error can pass 2e-2 at any hidden
 * width.  With this flag each such operand is a hi/lo bf16 pair (16 bits)
 * summed by two MFMAs into the fp32 accumulator; the state then stays within
 * about 1e-4 of the exact recurrence.  About twice the MFMA work, on 32-unit
 * hidden slices.  The chunk outputs still come from bf16 chunk-start
 * weights.  The backward of a precise call runs the portable fp32 backward,
 * so E2TTT_FLAG_SAVE_STATES is unsupported with it.  No effect on the
 * portable path, which computes in fp32. */
#define E2TTT_FLAG_PRECISE 16

typedef struct {
    int32_t kind;     /* e2ttt_kind */
    int32_t loss;     /* e2ttt_loss */
    int32_t io_dtype; /* e2ttt_dtype of q, k, v, out */
    int32_t flags;    /* E2TTT_FLAG_* */
    int64_t B, H, T;  /* batch, heads, tokens per sequence */
    int64_t D;        /* head dim (k, q, v, out width) */
    int64_t Hd;       /* hidden width of MLP / SwiGLU fast weights; ignored for LINEAR */
    int64_t chunk;    /* tokens per chunk; the last chunk holds the remaining T mod chunk tokens */
} e2ttt_desc;

/* Floats per (b, h) in the packed fast-weight vector; -1 for a bad desc. */
E2TTT_API int64_t e2ttt_param_count(const e2ttt_desc* desc);

/* Bytes of scratch e2ttt_chunk_forward needs for `desc` (0 when B*H*T == 0,
 * (size_t)-1 for a bad desc).  Contents need not be initialised. */
E2TTT_API size_t e2ttt_workspace_size(const e2ttt_desc* desc);

/* Which device path e2ttt_chunk_forward takes: 0 = portable fp32 kernel,
 * 1 = SwiGLU bf16 MFMA path (SWIGLU, LOSS_NEGDOT, BF16, D == 128, Hd a
 * multiple of 64 up to 4096, chunk a multiple of 64, T * D * 2 < 2^31),
 * 2 = the same shapes with E2TTT_FLAG_PRECISE (hi/lo bf16 operands),
 * 3 = fp32 MFMA path for LINEAR / MLP with F32 I/O (D a multiple of 16 up to
 * 64, Hd a multiple of 16, a head's state within 32 16x16 tiles per matrix),
 * 4 = the same for an MLP split over 16-unit hidden slices (B*H*Hd/16 <= 256,
 * 32 <= Hd <= 128, chunk <= 64; the slices of a head synchronise through device memory once
 * per chunk, so all B*H*Hd/16 workgroups run at once, one per compute unit:
 * on a device with fewer compute units the call runs path 3's kernel);
 * negative e2ttt_status for a bad desc. */
E2TTT_API int e2ttt_path(const e2ttt_desc* desc);

/*
 * Host-only validation of a call, touching no device memory (usable without
 * a GPU).  ptrs[] holds, in order: q, k, v, eta, alpha, beta, W0, M0, out,
 * W_end, M_end.  Returns E2TTT_OK or the first problem found:
 *   - sizes: B, H, T >= 0; D >= 1; 1 <= chunk <= 2^31 - 1; Hd >= 1 for MLP / SWIGLU;
 *     enums and flags in range (E2TTT_ERR_INVALID_ARG);
 *   - pointers: non-null when the tensor is non-empty, 16-byte aligned
 *     (eta, alpha, beta: 4-byte aligned) (E2TTT_ERR_INVALID_ARG); with
 *     E2TTT_FLAG_NO_MOMENTUM, beta, M0 and M_end are not checked;
 *   - shape support: E2TTT_ERR_UNSUPPORTED when neither device path handles
 *     the shape (portable path: D <= 256 and Hd <= 1024);
 *   - aliasing: W_end may equal W0 and M_end may equal M0 exactly (in-place
 *     update); any other byte overlap between an output and an input or two
 *     outputs is E2TTT_ERR_ALIAS.
 */
E2TTT_API int e2ttt_validate(const e2ttt_desc* desc, const void* const ptrs[11]);

/*
 * The chunk update over whole sequences (the hot path).  "Rethinking
 * Expressivity and Efficiency in Test-Time Training": abstract (gradients at
 * the chunk-start weights, closed-form transition to the exact chunk-end
 * fast weight and momentum), atlas summary "Approach" (momentum and weight
 * kernels from log-space sums, two weighted gradient aggregations), arxivlens
 * "Limitations" (the chunk output from the chunk-start weights).
 *   q, k, v   [B][H][T][D]  io_dtype, contiguous
 *   eta, alpha, beta [B][H][T] fp32 (domain: eta >= 0, alpha, beta in [0, 1])
 *   W0, M0    [B][H][P] fp32 chunk-0 fast weight and momentum
 *   out       [B][H][T][D]  io_dtype: out_t = f_{W at t's chunk start}(q_t)
 *   W_end, M_end [B][H][P] fp32 state after the last chunk (may be W0 / M0)
 *   workspace device scratch of >= e2ttt_workspace_size(desc) bytes, 256-byte
 *             aligned; clobbered.
 * T == 0 copies W0 -> W_end and M0 -> M_end; B*H == 0 does nothing.
 * A ragged tail (T % chunk != 0) is a shorter last chunk of T mod chunk
 * tokens with the same closed form over its tokens (the official code's
 * tail-length helper, named on the codewithpapers page, suggests one).
 */
E2TTT_API int e2ttt_chunk_forward(const e2ttt_desc* desc,
                        const void* q, const void* k, const void* v,
                        const float* eta, const float* alpha, const float* beta,
                        const float* W0, const float* M0,
                        void* out, float* W_end, float* M_end,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * e2ttt_chunk_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * (e.g. one chunk per call on a carried state), harnesses that forbid
 * allocation.  It allocates nothing and calls no allocating routine.  Its
 * scratch is a device array built into the library, E2TTT_NOALLOC_SCRATCH_BYTES
 * per GPU, present on every GPU the library runs on until the process ends.
 * Arguments, layouts, results and aliasing rules as e2ttt_chunk_forward
 * (results are identical to it bit for bit).  Errors:
 *   - E2TTT_ERR_SCRATCH_LIMIT when e2ttt_workspace_size(desc) exceeds
 *     E2TTT_NOALLOC_SCRATCH_BYTES (checked before any device call; e.g. one
 *     256-token chunk of a B = 8, H = 16, D = 128, Hd = 256 SwiGLU layer needs
 *     25.4 MB and fits, its whole 2048-token sequence needs 203 MB and does not);
 *   - E2TTT_ERR_INVALID_ARG with E2TTT_FLAG_SAVE_STATES (a saved state would
 *     not survive the next call on the GPU);
 *   - the others as e2ttt_chunk_forward.
 * Every call on a GPU uses that GPU's one scratch array: calls that overlap in
 * time on one GPU (other streams, other host threads) race and give wrong
 * results.  Calls on one stream are ordered and safe.  Nothing in the scratch
 * needs to start at zero, and nothing is kept from one call to the next.
 */
#define E2TTT_NOALLOC_SCRATCH_BYTES (64u << 20)
E2TTT_API int e2ttt_chunk_forward_noalloc(const e2ttt_desc* desc,
                        const void* q, const void* k, const void* v,
                        const float* eta, const float* alpha, const float* beta,
                        const float* W0, const float* M0,
                        void* out, float* W_end, float* M_end, void* stream);

/*
 * e2ttt_chunk_forward plus per-stage timing for profilers and benchmarks.
 * `events` holds 4 hipEvent_t created by the caller (hipEventCreate); they
 * are recorded on `stream` before the scalar-kernel launch, after it, after
 * the chunk-loop launch and after the output launch, so
 * hipEventElapsedTime(events[1], events[2]) is the chunk-loop kernel's
 * duration.  events == NULL behaves exactly like e2ttt_chunk_forward.
 */
E2TTT_API int e2ttt_chunk_forward_events(const e2ttt_desc* desc,
                        const void* q, const void* k, const void* v,
                        const float* eta, const float* alpha, const float* beta,
                        const float* W0, const float* M0,
                        void* out, float* W_end, float* M_end,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* const events[4]);

/*
 * The scalar-kernel step alone (per-subsystem parity): the momentum and weight
 * kernels of "Rethinking Expressivity and Efficiency in Test-Time Training"
 * (atlas summary "Approach"; the log-space suffix sums the arxivlens
 * "Results" section counts as the method's overhead).  For every chunk of
 * every (b, h), from log-space suffix sums of log alpha and log beta:
 *   cM[b][h][t] = eta_t * m_t,  m_t = prod_{s after t in its chunk} beta_s
 *   cW[b][h][t] = eta_t * w_t,  w_t = sum_{tau >= t} alpha(tau:end] * beta(t:tau]
 *   scal[b][h][c][0..3] = { prod alpha, prod beta, gamma = beta_first * w_first, 0 }
 * eta, alpha, beta, cM, cW: [B][H][T] fp32; scal: [B][H][ceil(T/chunk)][4] fp32
 * (a shorter last chunk takes the same sums over its tokens).
 * Only desc->B, H, T, chunk and flags are read: E2TTT_FLAG_NO_MOMENTUM takes
 * beta = 0 (beta may be NULL), E2TTT_FLAG_CHUNK_AVG replaces m_t and w_t by
 * their chunk means.  E2TTT_ERR_INVALID_ARG for negative sizes, chunk outside
 * [1, 2^31 - 1], unknown flag bits, or a null or misaligned pointer (for a
 * non-empty call).  The outputs must not overlap the inputs.
 */
E2TTT_API int e2ttt_logscan(const e2ttt_desc* desc, const float* eta, const float* alpha, const float* beta,
                  float* cM, float* cW, float* scal, void* stream);

/*
 * Backward pass of the chunk update (the gradients a training step needs).
 * It is the vector-Jacobian product of e2ttt_chunk_forward: given cotangents
 * dout, dW_end, dM_end of its outputs, it returns
 *   dX = d/dX [ <dout, out> + <dW_end, W_end> + <dM_end, M_end> ]
 * for X in q, k, v, eta, alpha, beta, W0, M0 -- the derivative of the chunk
 * update that "Rethinking Expressivity and Efficiency in Test-Time Training"
 * trains with (abstract; atlas summary "Approach").  The forward is
 * recomputed inside the call (scalar kernels and chunk loop, keeping each
 * chunk's start state); nothing needs to be saved from the forward call.
 *
 * Paths, chosen like the forward's: the SwiGLU MFMA backward for its shapes
 * (SWIGLU, LOSS_NEGDOT, BF16 I/O, D == 128, Hd a multiple of 64 up to 4096,
 * chunk a multiple of 64, T*D*2 < 2^31), else (or with
 * E2TTT_FLAG_FORCE_GENERIC) a portable fp32 backward for every kind and loss
 * with D <= 256, Hd <= 1024.  chunk <= 2048 on both (else
 * E2TTT_ERR_UNSUPPORTED).  E2TTT_FLAG_NO_MOMENTUM and E2TTT_FLAG_CHUNK_AVG
 * are honoured and a ragged last chunk is allowed.
 *
 *   q, k, v, dout        [B][H][T][D] io_dtype (dout: cotangent of out)
 *   eta, alpha, beta     [B][H][T] fp32
 *   W0, M0               [B][H][P] fp32 (the forward's initial state)
 *   dW_end, dM_end       [B][H][P] fp32 cotangents of W_end, M_end
 *   dq, dk, dv           [B][H][T][D] io_dtype outputs
 *   deta, dalpha, dbeta  [B][H][T] fp32 outputs
 *   dW0, dM0             [B][H][P] fp32 outputs (packed like W0)
 *   workspace            >= e2ttt_backward_workspace_size(desc) bytes,
 *                        256-byte aligned; clobbered
 * Without momentum, beta, M0, dM_end, dbeta and dM0 are not used (may be NULL).
 * Every output must be disjoint from every other buffer (no in-place form).
 * T == 0 copies dW_end -> dW0 and dM_end -> dM0; B*H == 0 does nothing.
 */
E2TTT_API size_t e2ttt_backward_workspace_size(const e2ttt_desc* desc);

/* Host-only validation of a backward call; ptrs[] holds, in order: q, k, v,
 * eta, alpha, beta, W0, M0, dout, dW_end, dM_end, dq, dk, dv, deta, dalpha,
 * dbeta, dW0, dM0.  Same rules as e2ttt_validate (16-byte alignment; eta,
 * alpha, beta, deta, dalpha, dbeta 4-byte), and no output may overlap any
 * other tensor (E2TTT_ERR_ALIAS). */
E2TTT_API int e2ttt_validate_backward(const e2ttt_desc* desc, const void* const ptrs[19]);

E2TTT_API int e2ttt_chunk_backward(const e2ttt_desc* desc,
                        const void* q, const void* k, const void* v,
                        const float* eta, const float* alpha, const float* beta,
                        const float* W0, const float* M0,
                        const void* dout, const float* dW_end, const float* dM_end,
                        void* dq, void* dk, void* dv,
                        float* deta, float* dalpha, float* dbeta,
                        float* dW0, float* dM0,
                        void* workspace, size_t workspace_bytes, void* stream);

/* e2ttt_chunk_backward plus timing: `events` (4 hipEvent_t, or NULL) are
 * recorded before the forward recompute, after it, after the reverse chunk
 * loop and after the scalar kernels' backward. */
E2TTT_API int e2ttt_chunk_backward_events(const e2ttt_desc* desc,
                        const void* q, const void* k, const void* v,
                        const float* eta, const float* alpha, const float* beta,
                        const float* W0, const float* M0,
                        const void* dout, const float* dW_end, const float* dM_end,
                        void* dq, void* dk, void* dv,
                        float* deta, float* dalpha, float* dbeta,
                        float* dW0, float* dM0,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* const events[4]);

/* Static, human-readable name of a status code. */
E2TTT_API const char* e2ttt_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* E2TTT_H */
