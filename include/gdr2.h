/*
 * gdr2.h -- C ABI of the Gated DeltaNet-2 library for AMD MI355X
 * (gfx950).  Plain C: no C++ or HIP types.  Streams are passed as void*
 * holding a hipStream_t (NULL = the default stream).
 *
 * The operation (page "Gated DeltaNet-2: 선형 어텐션에서 삭제와 쓰기 게이트
 * 분리", section "Gated Delta Rule-2 업데이트 수식", the update equation and
 * its symbol table), for every batch row b and head h independently:
 *
 *     S_t = (I - k_t (b_t * k_t)^T) D_t S_{t-1} + k_t (w_t * v_t)^T
 *     o_t = S_t^T q_t
 *
 *   S_t    d_k x d_v memory state (fp32 here), row index = key channel
 *   k_t    key (the pages take it L2-normalised; the caller normalises, the
 *          library computes the formula for any k)
 *   b_t    erase gate, per key channel (width d_k) or one scalar (width 1)
 *   w_t    write gate, per value channel (width d_v) or one scalar (width 1)
 *   D_t    diag(exp(g_t)): per-key-channel decay, passed as its logarithm g_t
 *          (fp32, width d_k or 1; g <= 0 is expected but not required)
 *   o_t    readout after the update at t, without scaling (the pages give no
 *          readout; this is the usual linear-attention convention)
 *   '*'    elementwise product
 *
 * Width-1 gates broadcast over their channels: b = w = one scalar beta is
 * KDA, and a scalar decay on top is Gated DeltaNet (same section).
 *
 * Optional initial state S0: a learned prefilled memory (page "[논문리뷰]
 * Sparse Delta Memory: Scaling the State of Linear RNNs through Sparsity",
 * section 3, the learned initial state M_0).  S_out of one call may be passed
 * as S0 of the next to continue a sequence segment by segment (page "Memory
 * Caching(MC): ...", section "체크포인트를 캐싱할까, 독립 압축기를 쓸까?");
 * the result equals one call over the whole sequence up to rounding.
 *
 * Chunked prefill: fixed-size chunks (page "Gated DeltaNet-2 ...", section
 * "효율적 구현": a chunkwise algorithm with a WY form that absorbs the
 * cumulative per-channel decay into the rank-1 erase factors).  The decode
 * step is the pure recurrent mode of the same page (section "개요"): one
 * token per sequence, state updated in place.
 *
 * Common rules for every entry point
 *   Ownership : the caller allocates and frees every device buffer (inputs,
 *               outputs, workspace).  The library allocates no device memory,
 *               does not synchronise, and keeps no pointer after returning.
 *               Work is enqueued on `stream` and runs asynchronously.
 *   Errors    : arguments are validated on the host before any launch; on
 *               error the call returns a non-zero gdr2_status, records a
 *               message for gdr2_last_error() in the calling thread, launches
 *               nothing and leaves every output untouched.  A failed HIP
 *               launch returns GDR2_ERR_HIP with the HIP error text.  NaN or
 *               Inf inputs are not checked; they propagate.
 *   Layout    : every tensor is dense, row-major, contiguous, in device memory,
 *               16-byte aligned.
 *   Threads   : calls are reentrant; calls on different streams run
 *               concurrently as long as their buffers do not overlap.
 */
#ifndef GDR2_H
#define GDR2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR2_ABI_VERSION 6

typedef enum gdr2_status {
    GDR2_OK = 0,
    GDR2_ERR_INVALID_ARG = 1,  /* null / misaligned / overlapping pointer, bad size */
    GDR2_ERR_UNSUPPORTED = 2,  /* valid but outside the supported set below */
    GDR2_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
    GDR2_ERR_HIP = 4,          /* the HIP runtime reported an error */
    GDR2_STATUS_RANGE_ = 0x7fffffff  /* not a status: makes every 32-bit value a
                                        valid gdr2_status, so an unknown code
                                        passed to gdr2_status_string is defined */
} gdr2_status;

/* Element type of q, k, v, b, w and o.  g, S0, S_out and state are fp32. */
typedef enum gdr2_dtype {
    GDR2_F32 = 0,
    GDR2_BF16 = 1  /* bfloat16; o is rounded to nearest-even once, at store */
} gdr2_dtype;

/*
 * Optional input prologue, fused into the kernels (bit flags; 0 = inputs are
 * used as given).  The page "Gated DeltaNet-2 ..." (section "Gated Delta
 * Rule-2 업데이트 수식", symbol table) takes the key L2-normalised, the
 * erase and write gates in [0, 1] and the decay in (0, 1); these bits let a
 * caller pass raw projections instead of normalising and activating them in
 * a separate pass over HBM.  The pages name no activation function: the
 * logistic sigmoid and the log-sigmoid decay below are this library's choice.
 *   NORM_QK  q and k are scaled per token and head to unit L2 norm over the
 *            d_k channels: x <- x (sum x_i^2 + 1e-6)^(-1/2)
 *   GATES    b <- sigmoid(b), w <- sigmoid(w) (applied to the scalar of a
 *            width-1 gate), and g carries a pre-activation x whose log-decay
 *            is -softplus(x) = log sigmoid(-x)
 * The backward's gradients are then with respect to the raw inputs.
 */
typedef enum gdr2_prologue {
    GDR2_PROLOGUE_NORM_QK = 1,
    GDR2_PROLOGUE_GATES = 2
} gdr2_prologue;

/* Algorithm of the chunked forward. */
typedef enum gdr2_algo {
    GDR2_ALGO_AUTO = 0,    /* the library picks */
    GDR2_ALGO_STAGED = 1,  /* intra-chunk kernel writes per-chunk factors to the
                              workspace; a propagation kernel carries the state
                              through the chunks and writes o */
    GDR2_ALGO_SEGMENTED = 2, /* STAGED with the chunks of each sequence cut into
                              segments that run in parallel: a span kernel
                              forms each segment's chunk product and local
                              state, a fold kernel chains the segments' start
                              states, and the propagation kernel runs every
                              segment from its start (a two-level scan of the
                              chunk recurrence, for few sequences x heads and
                              many chunks).  AUTO takes it when one pass would
                              leave most of the GPU idle.  Same results as
                              STAGED up to rounding order. */
    GDR2_ALGO_FUSED = 3    /* one kernel per (sequence, head, 64 value
                              columns): each workgroup forms every chunk's
                              factors in LDS and carries the state through
                              the chunks, so nothing per chunk goes through
                              device memory and no workspace is needed.
                              bf16 only (GDR2_ERR_UNSUPPORTED otherwise), and
                              only with GDR2_STAGE_ALL.  AUTO takes it for
                              bf16 at Dk = 64 when B*H is at least the GPU's
                              compute-unit count (there it is faster than
                              STAGED; at Dk = 128 each head's two column
                              workgroups would repeat the chunk's factors).
                              Same results as STAGED up to rounding order. */
} gdr2_algo;

/* Which kernels of GDR2_ALGO_STAGED one call runs.  Two calls on the same
 * stream, PREP then STATE, with identical arguments (workspace included),
 * give exactly the result of one GDR2_STAGE_ALL call; the split exists so the
 * two kernels can be timed or scheduled separately.  A STATE call reads the
 * per-chunk factors the PREP call left in the workspace. */
typedef enum gdr2_stage {
    GDR2_STAGE_ALL = 0,
    GDR2_STAGE_PREP = 1,   /* intra-chunk kernel only (writes the workspace) */
    GDR2_STAGE_STATE = 2   /* propagation/output kernel only (reads it) */
} gdr2_stage;

/*
 * Arguments of the chunked forward.
 *   q, k   [B, T, H, Dk]        dtype
 *   v      [B, T, H, Dv]        dtype
 *   b      [B, T, H, b_width]   dtype, b_width in {1, Dk}
 *   w      [B, T, H, w_width]   dtype, w_width in {1, Dv}
 *   g      [B, T, H, g_width]   fp32 log-decay, g_width in {1, Dk}
 *   S0     [B, H, Dk, Dv]       fp32, may be NULL (zero initial state)
 *   o      [B, T, H, Dv]        dtype, written
 *   S_out  [B, H, Dk, Dv]       fp32, written, may be NULL; may be the same
 *                               pointer as S0 (in-place continuation), must
 *                               not otherwise overlap anything
 *   S_chunks [B, H, NC, Dk, Dv] fp32, NC = ceil(T / chunk), may be NULL:
 *                               written with the state at the start of every
 *                               chunk (S_chunks[b, h, n] = the state before
 *                               token n*chunk; n = 0 gives S0 or zeros), the
 *                               segment-boundary memory checkpoints of the
 *                               page "Memory Caching(MC): 길이에 따라
 *                               메모리가 커지는 RNN에 대한 연구", section
 *                               "체크포인트를 캐싱할까, 독립 압축기를
 *                               쓸까?".  Written by the STATE stage; must
 *                               not overlap anything else.
 *   o must not overlap any input.
 * Supported set: Dk == Dv in {64, 128}; chunk in {32, 64}; dtype F32 or BF16;
 * B, T, H >= 0 (T need not be a multiple of chunk; T == 0 writes S0, or
 * zeros, to S_out).  Anything else returns GDR2_ERR_UNSUPPORTED.  The chunked
 * form is exact for every chunk size, so the chunk changes results only by
 * rounding; F32 with Dk = 128 and chunk 64 is evaluated in chunks of 32 (a
 * 64 x 128 fp32 chunk does not fit the intra-chunk kernel's LDS), with
 * S_chunks still sampled every 64 tokens.
 */
typedef struct gdr2_fwd_args {
    int64_t B, T, H, Dk, Dv;
    int32_t chunk;
    int32_t dtype;        /* gdr2_dtype */
    int32_t algo;         /* gdr2_algo */
    int32_t stage;        /* gdr2_stage */
    int32_t b_width, w_width, g_width;
    int32_t prologue;     /* gdr2_prologue bits */
    const void *q, *k, *v, *b, *w;
    const float *g;
    const float *S0;
    void *o;
    float *S_out;
    void *workspace;      /* device memory, >= gdr2_forward_workspace_size() bytes */
    size_t workspace_bytes;
    float *S_chunks;      /* optional chunk-start states (see above) */
} gdr2_fwd_args;

/*
 * Arguments of one batched decode step: N sequences x H heads, one token each.
 *   q, k   [N, H, Dk]   dtype        v  [N, H, Dv]   dtype
 *   b      [N, H, b_width]           w  [N, H, w_width]       (dtype)
 *   g      [N, H, g_width] fp32
 *   state  [N, H, Dk, Dv] fp32, read and overwritten in place with S_t
 *   o      [N, H, Dv] dtype, written; must not overlap any other buffer
 * Supported set: Dk == Dv in {64, 128}; dtype F32 or BF16; N, H >= 0.
 */
typedef struct gdr2_decode_args {
    int64_t N, H, Dk, Dv;
    int32_t dtype;        /* gdr2_dtype */
    int32_t b_width, w_width, g_width;
    const void *q, *k, *v, *b, *w;
    const float *g;
    float *state;
    void *o;
    int32_t prologue;     /* gdr2_prologue bits */
    int32_t reserved;     /* must be 0 */
} gdr2_decode_args;

/*
 * Arguments of the chunked backward: the gradients of a loss L with respect
 * to every input of the chunked forward, given dL/do and dL/dS_final.  The
 * derivatives are those of the update and readout above (page "Gated
 * DeltaNet-2 ...", section "Gated Delta Rule-2 업데이트 수식"), taken
 * through the chunked WY form of section "효율적 구현"; the state at every
 * chunk start comes from the forward (S_chunks), so no state is recomputed.
 *   q, k, v, b, w, g   the forward's inputs, same shapes, dtype and widths
 *   S_chunks [B, H, NC, Dk, Dv] fp32, NC = ceil(T / 64): the chunk-start
 *                      states the forward wrote with chunk = 64 (any exact
 *                      source of the states before tokens 0, 64, 128, ...
 *                      serves); S_chunks[:, :, 0] is the forward's S0
 *   dO       [B, T, H, Dv]  dtype  dL/do
 *   dS_final [B, H, Dk, Dv] fp32   dL/dS_final, may be NULL (zero)
 * Outputs, all fp32, written in full (no accumulation into them):
 *   dq, dk   [B, T, H, Dk]     dv [B, T, H, Dv]
 *   db       [B, T, H, b_width]   dw [B, T, H, w_width]   dg [B, T, H, g_width]
 *            (a width-1 gate gets the sum over the channels it broadcasts to)
 *   dS0      [B, H, Dk, Dv], may be NULL: dL/dS0
 * No output may overlap any input, another output or the workspace.
 * Supported set: Dk == Dv in {64, 128}; chunk == 64; dtype F32 or BF16;
 * B, T, H >= 0 (T == 0 writes dS_final, or zeros, to dS0).  Anything else
 * returns GDR2_ERR_UNSUPPORTED.  Accumulation is fp32; with bf16 inputs the
 * matrix-core operands are bf16, as in the forward.  The result does not
 * depend on scheduling: every sum runs in a fixed order (no atomics), so a
 * call repeated on the same arguments gives the same bits.
 */
typedef struct gdr2_bwd_args {
    int64_t B, T, H, Dk, Dv;
    int32_t chunk;        /* must be 64 */
    int32_t dtype;        /* gdr2_dtype of q, k, v, b, w, dO */
    int32_t b_width, w_width, g_width;
    int32_t prologue;     /* gdr2_prologue bits, as given to the forward */
    const void *q, *k, *v, *b, *w;
    const float *g;
    const float *S_chunks;
    const void *dO;
    const float *dS_final;
    float *dq, *dk, *dv, *db, *dw, *dg;
    float *dS0;
    void *workspace;      /* device memory, >= gdr2_backward_workspace_size() bytes */
    size_t workspace_bytes;
    int32_t algo;         /* gdr2_algo of the reverse scan over the chunks:
                             STAGED one pass per (b, h), SEGMENTED the
                             two-level scan over chunk segments (a span
                             kernel, the segment fold and the scan per
                             segment, as in the forward), AUTO the library
                             picks (the two-level scan when one pass would
                             leave most of the GPU idle) */
    int32_t reserved;     /* must be 0 */
} gdr2_bwd_args;

/* Bytes of device workspace gdr2_forward_chunked needs for these arguments
 * (pointers are not read).  0 when none is needed or the arguments are
 * invalid or unsupported. */
size_t gdr2_forward_workspace_size(const gdr2_fwd_args *args);

/* Chunked forward: o for every token and the final state S_out. */
gdr2_status gdr2_forward_chunked(const gdr2_fwd_args *args, void *stream);

/* Bytes of device workspace gdr2_backward_chunked needs for these
 * arguments (pointers are not read).  0 when none is needed or the arguments
 * are invalid or unsupported. */
size_t gdr2_backward_workspace_size(const gdr2_bwd_args *args);

/* Chunked backward: every input gradient and dS0. */
gdr2_status gdr2_backward_chunked(const gdr2_bwd_args *args, void *stream);

/* One recurrent decode step for every (sequence, head) state. */
gdr2_status gdr2_decode_step(const gdr2_decode_args *args, void *stream);

/* Bytes of the library's static device scratch used by
 * gdr2_forward_chunked_noalloc (one copy per device, held until the process
 * ends). */
#define GDR2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* The chunked forward for callers that cannot allocate device memory: code
 * under HIP stream/graph capture, tight serving loops, hosts that forbid
 * hipMalloc.  Same arguments, results and checks as gdr2_forward_chunked,
 * except that args->workspace and args->workspace_bytes are ignored: the
 * workspace is the library's static device scratch of
 * GDR2_NOALLOC_SCRATCH_BYTES bytes.  The call allocates nothing (no
 * hipMalloc, no hipFree).  Arguments whose workspace
 * (gdr2_forward_workspace_size) exceeds the scratch return
 * GDR2_ERR_WORKSPACE and launch nothing.  Every call on one device shares
 * that device's scratch: calls that may overlap in time on one device (other
 * streams, other threads) race and must be serialised by the caller.  The
 * scratch's address is looked up on the first call on each device (a HIP
 * error then returns GDR2_ERR_HIP). */
gdr2_status gdr2_forward_chunked_noalloc(const gdr2_fwd_args *args, void *stream);

/* Static text for a status code (never NULL). */
const char *gdr2_status_string(gdr2_status status);

/* Message of the last failed call in this thread ("" if none). */
const char *gdr2_last_error(void);

/* GDR2_ABI_VERSION of the built library. */
int gdr2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR2_H */
