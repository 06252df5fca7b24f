/*
 * ssm.h -- C ABI of libssm, the MI355X (gfx950) selective state-space scan.
 *
 * Two operations, both from the Mamba selective-scan pages:
 *
 *   ssm_scan_fwd      the fused prefill scan.  Per token it forms the step
 *                     size delta_t = softplus(delta + delta_bias) (SSM
 *                     engineering essay, discosf.com, §1.3; ufo.work article
 *                     "Mamba hardware-aware operator fusion and selective-scan
 *                     parallelisation", §2.1), discretises dA = exp(delta_t A),
 *                     dBu = delta_t B_t u_t (ufo.work article §1.1; "From
 *                     FlashAttention to Mamba", kj168168, §三.1), runs the
 *                     diagonal recurrence h_t = dA h_{t-1} + dBu (ufo.work
 *                     article §1.1) and emits y_t = C_t . h_t + D u_t (essay
 *                     §1.1, skip term D), optionally multiplied by silu(z_t).
 *                     Long sequences are cut into chunks joined by transfer
 *                     operators (ufo.work article §3.1).
 *
 *   ssm_state_update  the single-token update of a persistent state
 *                     h_new = exp(delta A) h_old + delta B u (ufo.work article
 *                     §4.1), with the same output rule.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc'd or from an
 *     allocator built on it); the descriptor itself is host memory.  The
 *     caller owns every buffer; the library never allocates device memory
 *     and keeps no pointer after the call returns.
 *   - Layouts are dense, row-major, last index fastest:
 *       u, delta, z, y       (batch, d_inner, seqlen)     [scan]
 *       B, C                 (batch, d_state, seqlen)     [scan]
 *       u, delta, z, y       (batch, d_inner)             [update]
 *       B, C                 (batch, d_state)             [update]
 *       A                    (d_inner, d_state)  float32
 *       D, delta_bias        (d_inner)           float32
 *       state, last_state    (batch, d_inner, d_state) float32
 *     B and C are shared by all channels of a batch row.
 *   - io_dtype selects the element type of u, delta, z, B, C and y
 *     (float32 or bfloat16).  A, D, delta_bias and the states are always
 *     float32; all arithmetic is float32.  bf16 results are rounded to
 *     nearest, ties to even.
 *   - All work is enqueued on `stream` (NULL = the default stream).  Calls
 *     are asynchronous: they return once the kernels are queued, never
 *     synchronise, and a device fault surfaces at the caller's next
 *     synchronisation.
 *   - Arguments are validated before anything is launched; on an error
 *     nothing is launched and no buffer is touched.  Input values are not
 *     inspected: NaN and Inf propagate.
 *   - No buffer may overlap another, except where stated.
 *   - Thread safety: calls are reentrant; concurrent calls must not share a
 *     workspace or an output.
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t, so a hipStream_t can be passed unchanged. */
typedef struct ihipStream_t *ssm_stream_t;

typedef enum {
    SSM_OK = 0,
    SSM_ERR_NULL_ARG = 1,     /* a required pointer (or the descriptor) is NULL        */
    SSM_ERR_BAD_SHAPE = 2,    /* a negative dimension, or a bad chunk_size            */
    SSM_ERR_UNSUPPORTED = 3,  /* d_state outside 1..256, seqlen > SSM_MAX_SEQLEN, an unknown io_dtype, or more chunks than a grid holds */
    SSM_ERR_MISALIGNED = 4,   /* a pointer not aligned to its element size            */
    SSM_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than ssm_scan_workspace_bytes */
    SSM_ERR_HIP = 6           /* a HIP launch error (hipGetLastError after launching) */
} ssm_status;

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype;

#define SSM_MAX_D_STATE 256
/* Widest causal convolution ssm_scan_fwd_conv fuses (taps per channel). */
#define SSM_MAX_CONV_WIDTH 4
/* Longest sequence ssm_scan_fwd accepts (token offsets inside one row of the
 * packed B/C workspace stay within 32 bits). */
#define SSM_MAX_SEQLEN (1LL << 25)

typedef struct ssm_desc {
    int64_t batch;            /* >= 0 */
    int64_t d_inner;          /* >= 0, channels */
    int64_t d_state;          /* N, 1..256 */
    int64_t seqlen;           /* L >= 0; ignored by ssm_state_update */
    int32_t io_dtype;         /* ssm_dtype */
    int32_t chunk_size;       /* scan only: tokens per chunk; 0 = chosen by the
                                 library, else a positive multiple of 16.  A chunk
                                 covers tokens [kK, min((k+1)K, L)). */
    void *workspace;          /* scan only: device scratch, >= workspace_bytes */
    size_t workspace_bytes;   /* scan only */
    void *profile_begin;      /* scan only, optional hipEvent_t (timing enabled): when */
    void *profile_end;        /* both are set, the scan's first kernel dispatch
                                 records profile_begin at its start and its last
                                 dispatch profile_end at its end, so that
                                 hipEventElapsedTime gives the execution time of
                                 every pass of the scan together (measurement hook) */
    uint32_t flags;           /* SSM_FLAG_* bits; unknown bits: SSM_ERR_UNSUPPORTED */
    uint32_t reserved;        /* must be 0 */
} ssm_desc;

/* Zero-order-hold discretisation of the input term (SSM engineering essay,
 * §1.2: the input is held constant over the step): the state update becomes
 * h = exp(dt A) h + (exp(dt A) - 1) / A * B u, with the A = 0 limit dt B u,
 * instead of the default Euler term dt B u.  Scan and single-token update. */
#define SSM_FLAG_ZOH 1u

/* Scheduling flag of ssm_scan_fwd / _ex / _conv, no effect on the result
 * bits.  With d_state <= 16, 2..32 chunks and chunks of 1024 tokens or more,
 * one launch runs the whole chunked scan: each chunk publishes its transfer
 * operator (ufo.work article
 * "Accelerating state-space models ...", §3.1) in the workspace, waits for
 * those of the chunks before it for a bounded time, and computes any that
 * have not arrived by then itself.  With this flag no chunk waits: each
 * computes the operators of all chunks before it itself (work grows with
 * the square of the chunk count).  Meant for testing that path, and for
 * callers whose other work on the GPU could keep a chunk's predecessors
 * from running for long.  Accepted and ignored by the other entry points. */
#define SSM_FLAG_INDEPENDENT_CHUNKS 2u

/* Bytes of device workspace that ssm_scan_fwd needs for this descriptor
 * (its shapes, io_dtype and chunk_size; the workspace fields are ignored).
 * Returns 0 for an invalid descriptor.  Host-only, never touches the GPU. */
size_t ssm_scan_workspace_bytes(const ssm_desc *desc);

/* Chunk length that ssm_scan_fwd uses for this descriptor (chunk_size, or
 * the library's choice when it is 0); seqlen means a single chunk.  Returns
 * -1 for an invalid descriptor.  Host-only. */
int64_t ssm_scan_chunk_size(const ssm_desc *desc);

/* The schedule that ssm_scan_fwd runs for this descriptor, as a short
 * static string (for example "one chunk", or "two passes, 64 chunks, carry
 * kernel"), for logs and measurements; "invalid" for an invalid
 * descriptor.  Host-only. */
const char *ssm_scan_plan(const ssm_desc *desc);

/* Fused selective-scan forward pass.
 *   u, delta       (batch, d_inner, L) io_dtype; delta is the raw step size
 *   A              (d_inner, N) float32
 *   B, C           (batch, N, L) io_dtype
 *   D              (d_inner) float32 or NULL (no skip term)
 *   z              (batch, d_inner, L) io_dtype or NULL (no gate)
 *   delta_bias     (d_inner) float32 or NULL (zero); added before softplus
 *   softplus_flag  nonzero: delta_t = softplus(delta + bias); zero: delta + bias
 *   y              (batch, d_inner, L) io_dtype, written
 *   last_state     (batch, d_inner, N) float32, written with h_{L-1}
 *                  (zeros when L == 0), or NULL
 * The state starts at zero.  Needs desc->workspace of at least
 * ssm_scan_workspace_bytes(desc) bytes (may be NULL when that is 0); its
 * contents on entry do not matter and are garbage afterwards. */
ssm_status ssm_scan_fwd(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                        const void *B, const void *C, const float *D, const void *z,
                        const float *delta_bias, int softplus_flag, void *y, float *last_state,
                        ssm_stream_t stream);

/* ssm_scan_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, result and errors as ssm_scan_fwd, except that the
 * descriptor's workspace fields are ignored: the chunked schedules use a
 * scratch array that the library holds in device memory, one copy of
 * SSM_NOALLOC_SCRATCH_BYTES (32 MiB) on every GPU it runs on, until the
 * process ends.  Nothing is allocated by the call.  A descriptor whose plan
 * needs more than that (ssm_scan_workspace_bytes of a plain call above the
 * limit, for example 65536 tokens of 2048 channels in chunks of 512) returns
 * SSM_ERR_WORKSPACE before anything is launched.  All calls on one GPU share
 * its array: calls that may overlap on one GPU (different streams, or other
 * host threads) race and must be serialised by the caller; calls in order on
 * one stream are safe, whatever the array holds from the last call (the
 * schedules never read state they have not written in the same call). */
#define SSM_NOALLOC_SCRATCH_BYTES (32u << 20)
ssm_status ssm_scan_fwd_noalloc(const ssm_desc *desc, const void *u, const void *delta,
                                const float *A, const void *B, const void *C, const float *D,
                                const void *z, const float *delta_bias, int softplus_flag,
                                void *y, float *last_state, ssm_stream_t stream);

/* The same scan with explicit start states and, optionally, several
 * variable-length sequences packed along the token axis (packed-sequence
 * batching with a cu_seqlens offset table, the state reset at every sequence
 * boundary: ufo.work article, §4.2; a persistent start state: §4.1).
 *   initial_state  float32 or NULL (zeros): the state h_{-1} of every sequence
 *   cu_seqlens     NULL: every batch row is one sequence; initial_state and
 *                  last_state are (batch, d_inner, N).
 *                  Else a DEVICE int32 array of n_seqs + 1 token offsets,
 *                  cu_seqlens[0] = 0, nondecreasing, cu_seqlens[n_seqs] =
 *                  seqlen, and desc->batch must be 1: sequence s is the token
 *                  range [cu_seqlens[s], cu_seqlens[s+1]) of the single row;
 *                  at its first token the state is reset to initial_state[s]
 *                  (or 0); initial_state and last_state are (n_seqs, d_inner, N)
 *                  and last_state[s] is the state after the sequence's last
 *                  token (initial_state[s] or 0 for an empty sequence).
 *   n_seqs         number of sequences (>= 1) when cu_seqlens is given;
 *                  ignored otherwise.
 * The offsets are read on the device and not validated: a table that breaks
 * the rules above gives unspecified values of y and last_state, but every
 * memory access stays inside the buffers described here.  Needs the same
 * workspace as ssm_scan_fwd for the same descriptor.  Every other argument is
 * as for ssm_scan_fwd, which is this call with initial_state = NULL and
 * cu_seqlens = NULL.  Extra errors: SSM_ERR_BAD_SHAPE if cu_seqlens is given
 * with batch != 1 or n_seqs < 1. */
ssm_status ssm_scan_fwd_ex(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                           const void *B, const void *C, const float *D, const void *z,
                           const float *delta_bias, int softplus_flag, const float *initial_state,
                           const int32_t *cu_seqlens, int64_t n_seqs, void *y, float *last_state,
                           ssm_stream_t stream);

/* The scan with the short depthwise causal convolution that precedes it in
 * the Mamba layer fused in front ("From FlashAttention to Mamba": the SSM
 * layer is a 1-D convolution followed by the scan, §三.3; convolution and scan
 * merged into one kernel, §四.3).  The scan input is computed on the fly and
 * is not read from memory:
 *   u[b,d,t] = act(conv_bias[d] + sum_k conv_weight[d,k] x[b,d,t-(W-1)+k])
 * with W = conv_width (1..SSM_MAX_CONV_WIDTH) and act = silu when conv_silu
 * is nonzero, identity otherwise.  It feeds both the recurrence (dt u B) and
 * the skip term (D u).
 *   x            (batch, d_inner, L) io_dtype: the convolution's input
 *   conv_weight  (d_inner, W) float32; column W-1 multiplies the current token
 *   conv_bias    (d_inner) float32 or NULL (zero)
 *   conv_state   float32 (rows, d_inner, W-1) or NULL (zeros): the inputs
 *                before each sequence's first token, conv_state[s,d,W-2] being
 *                the one just before it; rows as for initial_state
 *   u_out        (batch, d_inner, L) io_dtype or NULL: written with u
 * Sequences (batch rows, or cu_seqlens ranges) never see each other's inputs
 * through the convolution.  All other arguments as for ssm_scan_fwd_ex.
 * Extra errors: SSM_ERR_UNSUPPORTED for conv_width outside 1..4,
 * SSM_ERR_NULL_ARG for a NULL conv_weight. */
ssm_status ssm_scan_fwd_conv(const ssm_desc *desc, const void *x, const float *conv_weight,
                             const float *conv_bias, int conv_width, int conv_silu,
                             const float *conv_state, const void *delta, const float *A,
                             const void *B, const void *C, const float *D, const void *z,
                             const float *delta_bias, int softplus_flag,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int64_t n_seqs, void *y, float *last_state, void *u_out,
                             ssm_stream_t stream);

/* Single-token update of a persistent state, in place.
 *   state  (batch, d_inner, N) float32, read and overwritten with
 *          exp(delta A) state + delta B u
 *   u, delta (batch, d_inner) io_dtype; delta is the FINAL step size
 *          (no bias, no softplus)
 *   A (d_inner, N) float32;  B, C (batch, N) io_dtype
 *   D (d_inner) float32 or NULL;  z (batch, d_inner) io_dtype or NULL
 *   y (batch, d_inner) io_dtype, written: (C . state_new + D u) silu(z)
 * desc->seqlen, chunk_size and the workspace fields are ignored. */
ssm_status ssm_state_update(const ssm_desc *desc, float *state, const void *u, const void *delta,
                            const float *A, const void *B, const void *C, const float *D,
                            const void *z, void *y, ssm_stream_t stream);

/* Bytes of device workspace that ssm_scan_bwd needs for this descriptor;
 * 0 for an invalid or unsupported descriptor.  Host-only. */
size_t ssm_scan_bwd_workspace_bytes(const ssm_desc *desc);

/* The schedule that ssm_scan_bwd (with_ckpt 0) or ssm_scan_bwd_ex given the
 * forward pass's checkpoints (with_ckpt 1; no packed sequences) runs for this
 * descriptor, as a short static string (for example "one chunk", or "the
 * blocks of a whole round in one chunk, the rest in chunks"), for logs and
 * measurements; "invalid" for an invalid or unsupported descriptor.
 * Host-only. */
const char *ssm_scan_bwd_plan(const ssm_desc *desc, int with_ckpt);

/* Backward pass of the scan: the gradients of the loss
 *   sum(dy * y) + sum(dlast * last_state)
 * with respect to every input, for upstream gradients dy (of y) and dlast
 * (of last_state).  It keeps states only at 8-token boundaries and recomputes
 * the rest while walking back (ufo.work article, §2.2: fine-grained
 * checkpoints, recompute inside the chunk); the reverse recurrence of the
 * state gradient is joined across chunks by transfer operators like the
 * forward one (§3.1).
 * Supported: d_state 1 .. 256, Euler or, with SSM_FLAG_ZOH in desc->flags,
 * the zero-order-hold input term; the fused convolution has no backward here
 * (its input u is an input of this call).  Above 16 states the pass runs once
 * per group of 16 states (their recurrences are independent, §3.2) and the
 * groups' per-token sums (du, ddelta, dz, ddelta_bias) are added in a fixed
 * order; when one group's channel blocks leave most of the GPU idle and
 * chunk_size is 0, up to four groups run side by side, each over the whole
 * sequence, and the workspace then also holds their per-token sums.
 * Packed sequences: see ssm_scan_bwd_ex.
 * Inputs: as ssm_scan_fwd_ex (initial_state may be NULL), plus
 *   dy             (batch, d_inner, L) io_dtype
 *   dlast          (batch, d_inner, N) float32 or NULL (zero)
 * Outputs, all float32, all overwritten (none is accumulated into):
 *   du, ddelta     (batch, d_inner, L); ddelta is the gradient of the raw
 *                  delta (before delta_bias and softplus)
 *   dA             (d_inner, N)
 *   dB, dC         (batch, N, L)
 *   dD             (d_inner) or NULL (not written)
 *   dz             (batch, d_inner, L); required when z is given
 *   ddelta_bias    (d_inner) or NULL (not written)
 *   dh0            (batch, d_inner, N) or NULL: gradient of initial_state
 * Needs desc->workspace of ssm_scan_bwd_workspace_bytes(desc) bytes.  All
 * sums run in a fixed order: results are identical from run to run. */
ssm_status ssm_scan_bwd(const ssm_desc *desc, const void *u, const void *delta, const float *A,
                        const void *B, const void *C, const float *D, const void *z,
                        const float *delta_bias, int softplus_flag, const float *initial_state,
                        const void *dy, const float *dlast, float *du, float *ddelta, float *dA,
                        float *dB, float *dC, float *dD, float *dz, float *ddelta_bias,
                        float *dh0, ssm_stream_t stream);

/* ssm_scan_bwd for sequences packed along L (ufo.work article, §4.2), the
 * backward of ssm_scan_fwd_ex: batch must be 1 and cu_seqlens holds n_seqs + 1
 * device int32 token offsets (as in ssm_scan_fwd_ex).  The state gradient
 * starts over at each sequence's last token from that sequence's row of
 * dlast, and stops at its first token, where it gives that sequence's row of
 * dh0.  initial_state, dlast and dh0 are (n_seqs, d_inner, N); an empty
 * sequence's dh0 is its dlast.  ckpt: the checkpoints written by
 * ssm_scan_fwd_ckpt for the same call, or NULL (the backward recomputes them
 * in its workspace).  Both need d_state <= 16 (SSM_ERR_UNSUPPORTED above).
 * With cu_seqlens and ckpt NULL this is ssm_scan_bwd.
 * Errors as ssm_scan_bwd, and SSM_ERR_BAD_SHAPE for packing with batch != 1
 * or n_seqs < 1.  A malformed offset table gives unspecified gradients but
 * no access out of bounds. */
ssm_status ssm_scan_bwd_ex(const ssm_desc *desc, const void *u, const void *delta,
                           const float *A, const void *B, const void *C, const float *D,
                           const void *z, const float *delta_bias, int softplus_flag,
                           const float *initial_state, const int32_t *cu_seqlens, int64_t n_seqs,
                           const float *ckpt, const void *dy, const float *dlast, float *du,
                           float *ddelta, float *dA, float *dB, float *dC, float *dD, float *dz,
                           float *ddelta_bias, float *dh0, ssm_stream_t stream);

/* The forward pass that also keeps what the backward pass would otherwise
 * recompute (ufo.work article "Accelerating state-space models ...", §2.2:
 * the forward keeps states at fine-grained boundaries, the backward
 * recomputes the rest): as ssm_scan_fwd_ex, and in addition writes ckpt, the
 * state entering every 8-token tile of every row,
 *   ckpt           (batch, d_inner, ceil(L / 8), 16) float32, written; states
 *                  n >= N of each 16 are zero; ssm_scan_ckpt_bytes(desc) bytes,
 *                  16-byte aligned.  With packed sequences the entry of a tile
 *                  whose first token starts a sequence is unspecified (the
 *                  backward starts that tile from the sequence's initial state)
 * Given to ssm_scan_bwd_ex with the same descriptor (shapes, io_dtype, flags)
 * and inputs, it spares the backward pass its forward recompute; with other
 * inputs the gradients are unspecified.  d_state <= 16 only
 * (SSM_ERR_UNSUPPORTED otherwise); ckpt NULL: SSM_ERR_NULL_ARG. */
ssm_status ssm_scan_fwd_ckpt(const ssm_desc *desc, const void *u, const void *delta,
                             const float *A, const void *B, const void *C, const float *D,
                             const void *z, const float *delta_bias, int softplus_flag,
                             const float *initial_state, const int32_t *cu_seqlens,
                             int64_t n_seqs, void *y, float *last_state, float *ckpt,
                             ssm_stream_t stream);

/* Bytes of the checkpoint array of ssm_scan_fwd_ckpt for this descriptor
 * (0 when invalid or d_state > 16).  Host-only. */
size_t ssm_scan_ckpt_bytes(const ssm_desc *desc);

/* Static, NUL-terminated name of a status code ("unknown status" otherwise). */
const char *ssm_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int ssm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSM_H */
