/* gdn.h — C-ABI of libgdn: the bounded-decay gated delta rule on MI355X (gfx950).
 *
 * The layer.  Per sequence and head, a fixed-size state S (d_k x d_v, fp32) is
 * updated once per token, and each token reads the updated state:
 *
 *     S_t = diag(alpha_t) S_{t-1} + beta_t k_t (v_t - (diag(alpha_t) S_{t-1})^T k_t)^T
 *     o_t = S_t^T q_t,            alpha_t = exp(g_t)   (one value per key channel)
 *
 * i.e. the state is decayed first, then the value the decayed state returns for
 * k_t is replaced by v_t in proportion beta_t.  This is the fixed-size state
 * with correct-on-write updates and a position-dependent decay gate of
 * "How to Think About Trillion-Parameter Sparse Multimodal LLMs", section 2.2;
 * the log-decay g is the lower-bounded quantity of "Trillion-Parameter MoE
 * Multimodal LLMs: How to Evaluate the New Generation", section 3.1, eq. 1
 * (g = g_min * sigmoid(.), g_min = -5), so its domain is [-5, 0].  No scale is
 * applied to q.
 *
 * Conventions shared by every entry point
 *   - Pointers named as device pointers must address memory of the current
 *     HIP device; pointers named as host pointers must address host memory.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns without waiting; results are ready
 *     when the stream reaches that point.  Apart from the side streams of the
 *     time split (see gdn_prefill) and the fixed scratch array of
 *     gdn_prefill_noalloc, the library keeps no state between calls; it frees
 *     no caller memory and prints nothing.
 *   - Every call returns a gdn_status.  Argument errors are reported before any
 *     memory is touched or any work is enqueued.  GDN_ERR_HIP means a HIP call
 *     (allocation aside) or a kernel launch failed; a fault inside a kernel
 *     surfaces at the caller's next synchronisation, as for any HIP kernel.
 *   - Inputs with NaN or Inf are not masked: they propagate into the outputs.
 *   - Element types: q, k, v, o share one dtype (GDN_F32 or GDN_BF16); g, beta
 *     and all states are always fp32.  With GDN_BF16 the contractions run on
 *     bf16 matrix cores with fp32 accumulation and an fp32 state; with GDN_F32
 *     all arithmetic is fp32.  fp32 -> bf16 conversions round to nearest even.
 *   - Supported sizes: d_k and d_v each 64 or 128; H >= 1.
 *   - Alignment: q, k, v, o, g, states and the workspace must be 16-byte
 *     aligned; beta and cu_seqlens 4-byte aligned.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, short workspace */
    GDN_ERR_UNSUPPORTED = 2, /* d_k or d_v not in {64, 128}, unknown dtype */
    GDN_ERR_DOMAIN = 3,      /* validation mode only: g outside [-5, 0], bad cu_seqlens */
    GDN_ERR_OOM = 4,         /* device allocation failed */
    GDN_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed */
    GDN_ERR_SCRATCH_LIMIT = 6 /* gdn_prefill_noalloc: the call needs more scratch
                                 than GDN_NOALLOC_SCRATCH_BYTES */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Gate of the logit entry points (gdn_prefill_logits, gdn_decode_logits): the
 * log-decay of each (token, head, key channel) is computed inside the kernels
 * from a bf16 logit z and a scalar parameter p, so the gate costs 2 bytes per
 * channel instead of 4.
 *   GDN_GATE_SCALED_SIGMOID  g = p * sigmoid(z), p = g_min in [-5, 0]: the
 *       lower-bounded scaled-sigmoid decay of "Trillion-Parameter MoE
 *       Multimodal LLMs: How to Evaluate the New Generation", section 3.1,
 *       eq. 1 (there g_min = -5); g lies in [g_min, 0].
 *   GDN_GATE_ALPHA_MIN       g = log(p + (1 - p) * sigmoid(z)), p = a_min in
 *       [e^-5, 1]: the decay factor alpha = e^g bounded below by a_min
 *       instead; g lies in [log a_min, 0].
 * Either way g stays inside [-5, 0] for every z (z = -inf and +inf give the
 * endpoints).  GDN_GATE_LOG (g given in fp32) is what gdn_prefill and
 * gdn_decode take. */
typedef enum gdn_gate { GDN_GATE_LOG = 0, GDN_GATE_SCALED_SIGMOID = 1, GDN_GATE_ALPHA_MIN = 2 } gdn_gate;

/* Static English description of a status code (never NULL).  A utility of
 * this library: no passage of the pages defines it. */
const char* gdn_status_string(int32_t status);

/* Bytes of a state tensor [num_seqs, H, d_k, d_v] fp32 (d_v fastest); 0 for
 * negative arguments, SIZE_MAX when the product does not fit a size_t.  A
 * utility of this library: the pages define the state (see gdn_state_alloc)
 * but no such call. */
size_t gdn_state_bytes(int64_t num_seqs, int32_t H, int32_t d_k, int32_t d_v);

/* Allocates a zero-filled state tensor [num_seqs, H, d_k, d_v] fp32 on the
 * current device, ordered on `stream` (the zero fill is enqueued there).
 * *out receives the device pointer (NULL when the size is 0); the caller
 * releases it with gdn_state_free.  GDN_ERR_OOM when the device cannot
 * provide the memory, or when the size does not fit a size_t (then no device
 * call is made).  The fixed-size state replaces a key-value cache: its size
 * does not depend on the sequence length (section 5.3 of "Trillion-Parameter
 * MoE Multimodal LLMs: How to Evaluate the New Generation"). */
int32_t gdn_state_alloc(int64_t num_seqs, int32_t H, int32_t d_k, int32_t d_v, float** out, void* stream);

/* Releases memory from gdn_state_alloc, ordered on `stream`.  NULL is a no-op.
 * A utility of this library: no passage of the pages defines it. */
int32_t gdn_state_free(float* state, void* stream);

/* Device scratch bytes gdn_prefill needs for these sizes (may be 0).  The
 * bound depends only on the arguments, never on the lengths inside
 * cu_seqlens, so no device-to-host copy is needed to size it.  The scratch
 * holds the time split's segment maps and, with more than one sequence when
 * the split runs or when num_seqs * H exceeds the 256 compute units, an int32
 * table of num_seqs entries: the order (longest sequence first) in which the
 * workgroups take the sequences, written by the call itself.  Both are this
 * library's design: no passage of the pages defines this call. */
size_t gdn_prefill_workspace_bytes(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_k, int32_t d_v);

/* Chunked prefill over packed variable-length sequences.
 *
 *   q, k        device, [T_total, H, d_k], dtype
 *   v           device, [T_total, H, d_v], dtype
 *   g           device, [T_total, H, d_k] fp32, log-decay in [-5, 0]
 *   beta        device, [T_total, H] fp32
 *   cu_seqlens  device, int32 [num_seqs + 1]: sequence n is tokens
 *               cu_seqlens[n] .. cu_seqlens[n+1]-1; cu_seqlens[0] = 0,
 *               non-decreasing, cu_seqlens[num_seqs] = T_total.  Zero-length
 *               sequences are allowed (their final state is their initial
 *               state).  The contents are trusted unless the environment
 *               variable GDN_VALIDATE=1 is set, which copies them to the host
 *               (and g, to range-check it) and returns GDN_ERR_DOMAIN on a
 *               violation.
 *   initial_state  device, [num_seqs, H, d_k, d_v] fp32, or NULL for zeros.
 *   final_state    device, [num_seqs, H, d_k, d_v] fp32, or NULL to skip;
 *                  may be the same pointer as initial_state (updated in place).
 *   o           device, [T_total, H, d_v], dtype; written for every token.
 *   workspace   device scratch of at least
 *               gdn_prefill_workspace_bytes(T_total, num_seqs, H, d_k, d_v)
 *               bytes (may be NULL when that is 0).  Owned by the caller; its
 *               contents on entry are ignored and on return are unspecified.
 *               Two calls in flight at once need two workspaces.
 *
 * Method: each sequence is cut into chunks (32 tokens with GDN_BF16, 64 with
 * GDN_F32), long sequences also into segments run in parallel and joined
 * through the affine map of the state.  The segment length is planned from the
 * arguments alone: for sequences of the mean length, and, when those need no
 * split but (sequence, head) units outnumber the 256 compute units, so that
 * any sequence longer than T_total / (256 / H + 1) tokens is split (a
 * balanced batch then has none, and runs as unsplit).  A split call runs the first segment's
 * output pass on a side stream, forked from and joined back into `stream` by
 * events (also when a later step of the call fails), so the call stays
 * ordered on `stream` and can be captured into a graph.  The library creates
 * one side stream (default priority) and two events per caller stream, on
 * first use, and keeps them until the process ends: calls on different caller
 * streams do not serialise on a shared side stream while at most 16 caller
 * streams per device are in use (beyond that an idle side stream that is not
 * being captured is reused, or a new one is made).  Host threads may call
 * concurrently, on different streams; two captures in progress at once use
 * different side streams.  Inside a chunk the decay
 * is carried as a local cumulative log-decay (the cumulative decay factor of
 * "Architecture Evolution and Training Engineering for Trillion-Scale Sparse
 * Multimodal Models", section 3.2), the causal intra-chunk products run as
 * dense matrix-core tiles, and chunks are linked through the carried state.
 * Results agree with the token-by-token recurrence up to rounding. */
int32_t gdn_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                    const float* initial_state, float* final_state, void* o,
                    int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* gdn_prefill for packed batches whose lengths are skewed (say one long
 * sequence among many short ones), with a host-side bound on the lengths.
 *   max_seqlen  >= cu_seqlens[n+1] - cu_seqlens[n] for every n; 0 = unknown
 *               (then exactly gdn_prefill).  Negative: GDN_ERR_INVALID_ARG.
 *               With GDN_VALIDATE=1 a sequence longer than the bound is
 *               GDN_ERR_DOMAIN.
 *   workspace   at least gdn_prefill_workspace_bytes_maxlen(T_total,
 *               num_seqs, max_seqlen, H, d_k, d_v) bytes.
 * Everything else is as for gdn_prefill.  gdn_prefill plans the time split
 * (which sequences are cut into segments run in parallel) from the mean
 * length, since the lengths stay on the device; a bound lets it cut the long
 * sequences of a skewed batch, whose serial chains would otherwise be the
 * whole call's critical path.  A bound that is too large or too small changes
 * the plan, never the result (up to rounding).  This is this library's
 * scheduling of the pages' chunked form: no passage of the pages defines the
 * call. */
int32_t gdn_prefill_maxlen(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total, int64_t max_seqlen,
                           const float* initial_state, float* final_state, void* o,
                           int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Device scratch bytes of gdn_prefill_maxlen (0 for invalid arguments); a
 * function of the arguments only, like gdn_prefill_workspace_bytes, which it
 * equals for max_seqlen = 0. */
size_t gdn_prefill_workspace_bytes_maxlen(int64_t T_total, int32_t num_seqs, int64_t max_seqlen, int32_t H,
                                          int32_t d_k, int32_t d_v);

/* Bytes of the fixed device scratch of gdn_prefill_noalloc (64 MiB). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_prefill that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The arguments and the result are gdn_prefill's, without
 * the workspace: its scratch is a device array of GDN_NOALLOC_SCRATCH_BYTES
 * inside the library, which each GPU the library runs on holds from the first
 * call until the process ends.
 *   - Returns GDN_ERR_SCRATCH_LIMIT, before any work is enqueued, when
 *     gdn_prefill_workspace_bytes(T_total, num_seqs, H, d_k, d_v) exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES (one 65,536-token sequence x 32 heads at
 *     d = 128 needs 32 MiB; four 8,192-token sequences x 32 heads, 44 MiB).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (on different streams, or from different host threads)
 *     race on it and their results are undefined.  Calls ordered on one
 *     stream, or separated by synchronisation, are safe.
 *   - It calls no hipMalloc or hipFree.  The first call on a device looks up
 *     the array's address; a split call on a caller stream the library has not
 *     seen creates that stream's side stream and events (see gdn_prefill), as
 *     gdn_prefill does.  GDN_VALIDATE=1 adds host buffers and a
 *     synchronisation, as for gdn_prefill. */
int32_t gdn_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                            const float* initial_state, float* final_state, void* o,
                            int32_t H, int32_t d_k, int32_t d_v, int32_t dtype, void* stream);

/* gdn_prefill with one log-decay per (token, head), shared by the key
 * channels: the gate g_th of "How to Think About Trillion-Parameter Sparse
 * Multimodal LLMs", section 3 item 3, written per token t and head h.
 *   g   device, [T_total, H] fp32, log-decay in [-5, 0], 4-byte aligned
 *   dtype GDN_BF16 only (GDN_F32: GDN_ERR_UNSUPPORTED)
 * Everything else, the workspace size included, is as for gdn_prefill, and
 * the result equals gdn_prefill with g broadcast over the d_k channels, up to
 * rounding.  With one gate per head the decay of a token pair is a scalar, so
 * the kernels scale the products instead of the operands (no exponential per
 * element and no exponent budget). */
int32_t gdn_prefill_head_gate(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                              const float* initial_state, float* final_state, void* o, int32_t H, int32_t d_k,
                              int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* gdn_prefill with the gate given as bf16 logits (see gdn_gate):
 *   z           device, [T_total, H, d_k] bf16, 16-byte aligned (replaces g)
 *   gate        GDN_GATE_SCALED_SIGMOID or GDN_GATE_ALPHA_MIN, else
 *               GDN_ERR_INVALID_ARG
 *   gate_param  g_min in [-5, 0], or a_min in [e^-5, 1]; outside the range
 *               GDN_ERR_DOMAIN
 *   dtype       GDN_BF16 only (GDN_F32: GDN_ERR_UNSUPPORTED)
 * Every other argument, the workspace size and the result are as for
 * gdn_prefill with g = the parameterisation of z (computed in fp32 from the
 * bf16 logits). */
int32_t gdn_prefill_logits(const void* q, const void* k, const void* v, const void* z, int32_t gate,
                           float gate_param, const float* beta, const int32_t* cu_seqlens, int32_t num_seqs,
                           int64_t T_total, const float* initial_state, float* final_state, void* o, int32_t H,
                           int32_t d_k, int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/* One decode step: one new token for each of N sequences, state updated in
 * place (the recurrent form of "How to Think About Trillion-Parameter Sparse
 * Multimodal LLMs", section 2.2, whose inference cost does not grow with the
 * context).
 *
 *   q, k   device, [N, H, d_k], dtype        v, o   device, [N, H, d_v], dtype
 *   g      device, [N, H, d_k] fp32          beta   device, [N, H] fp32
 *   state  device, [N, H, d_k, d_v] fp32, read and overwritten in place.
 * N = 0 is a no-op.  A decode step equals a one-token gdn_prefill from the
 * same state, up to rounding. */
int32_t gdn_decode(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   float* state, void* o, int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                   void* stream);

/* gdn_decode with one log-decay per (sequence, head): g [N, H] fp32 in
 * [-5, 0], 4-byte aligned; dtype GDN_F32 or GDN_BF16. */
int32_t gdn_decode_head_gate(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             float* state, void* o, int32_t N, int32_t H, int32_t d_k, int32_t d_v, int32_t dtype,
                             void* stream);

/* gdn_decode with the gate given as bf16 logits z [N, H, d_k] (16-byte
 * aligned), gate and gate_param as for gdn_prefill_logits; dtype GDN_BF16
 * only. */
int32_t gdn_decode_logits(const void* q, const void* k, const void* v, const void* z, int32_t gate,
                          float gate_param, const float* beta, float* state, void* o, int32_t N, int32_t H,
                          int32_t d_k, int32_t d_v, int32_t dtype, void* stream);

/* Device scratch bytes gdn_prefill_backward needs: one state per 16-token
 * sub-chunk and head in the input dtype, (T_total / 16 + num_seqs) * H * d_k
 * * d_v * (2 for GDN_BF16, 4 for GDN_F32), rounded up to 256; with a time
 * split of segment length L (below), also gdn_prefill's split workspace for
 * segments of L tokens and (T_total / L + num_seqs) * H * d_k * d_v * 4 bytes,
 * for GDN_BF16 with d_k = d_v also min(num_seqs, T_total / (L + 1)) * H * d_k
 * * d_k * 4 bytes (the last segments' transitions) and T_total * H * d_k * 2
 * bytes (a bf16 buffer of q^ below), each rounded up to 256, and with more
 * than one sequence two int32 tables
 * (the order of the sequences, longest first, and their segment counts) of
 * num_seqs and num_seqs + 1 entries; without the split, that order alone when
 * num_seqs * H exceeds 256.  Depends on the arguments and on
 * GDN_BACKWARD_SEGMENT only; 0 for invalid arguments.  The checkpoints and
 * the split are this library's design: no passage of the pages defines this
 * call. */
size_t gdn_prefill_backward_workspace_bytes(int64_t T_total, int32_t num_seqs, int32_t H, int32_t d_k,
                                            int32_t d_v, int32_t dtype);

/* Gradients of gdn_prefill.  The method is trained by back-propagation
 * ("Architecture Evolution and Training Engineering for Trillion-Scale Sparse
 * Multimodal Models", section 3.3; "What a Trillion-Parameter MoE Model
 * Reveals About the Next Stage of LLM Scaling", section 3.2); given the
 * gradient of a loss with respect to every output o and to the final states,
 * this returns its gradient with respect to q, k, v, g, beta and the initial
 * states: the exact adjoint of the recurrence above, up to rounding.
 *
 *   q, k, v, g, beta, cu_seqlens, num_seqs, T_total, initial_state, H, d_k,
 *   d_v, dtype     as for gdn_prefill (the forward inputs; initial_state may
 *                  be NULL for zeros)
 *   d_o            device, [T_total, H, d_v], dtype: dL/do
 *   d_final_state  device, [num_seqs, H, d_k, d_v] fp32: dL/d(final state),
 *                  or NULL for zero
 *   dq, dk         device, [T_total, H, d_k], dtype (written)
 *   dv             device, [T_total, H, d_v], dtype (written)
 *   dg             device, [T_total, H, d_k] fp32 (written)
 *   dbeta          device, [T_total, H] fp32, 4-byte aligned (written)
 *   d_initial_state  device, [num_seqs, H, d_k, d_v] fp32 (written), or NULL
 *                  when not wanted; written also when initial_state is NULL
 *                  (the gradient at a zero initial state)
 *   workspace      device scratch of at least
 *                  gdn_prefill_backward_workspace_bytes(...) bytes, 16-byte
 *                  aligned, owned by the caller; contents on entry ignored,
 *                  on return unspecified.  Two calls in flight at once need
 *                  two workspaces.
 * Outputs must not alias inputs.  Alignment and validation (GDN_VALIDATE=1)
 * as for gdn_prefill.
 *
 * Method: a forward sweep stores the state at the start of every 16-token
 * sub-chunk; a reverse sweep carries dL/dS from the last sub-chunk to the
 * first and forms each sub-chunk's gradients from its start state with
 * dense matrix-core tiles.  The cumulative decay inside a 16-token window is
 * referred to the window's middle token, so every factor stays within
 * e^-40 .. e^40 for g in [-5, 0] (the 16-token tile bound of
 * "Trillion-Parameter MoE Multimodal LLMs: How to Evaluate the New
 * Generation", section 3.1).
 * Time split: when few (sequence, head) pairs leave compute units idle
 * (num_seqs * H <= 144) and sequences are long, each sequence is cut into
 * segments of L tokens (a multiple of 64) swept in parallel; when there are
 * more pairs than the 256 compute units and more than one sequence, every
 * sequence longer than L = T_total / (256 / H + 1) tokens is (when L >= 16384),
 * so that one long sequence among short ones does not set the call's time.  The state map
 * of a segment is affine, S_end = M S_start + N, and its adjoint
 * dS_start = M^T dS_end + D, where D, the gradient of the segment's outputs
 * o_t = (M_t S_start + N_t)^T q_t with respect to its start state, is the sum
 * over its tokens of q^_t dO_t^T, q^_t = M_t^T q_t (M_t: the transition
 * through token t).  gdn_prefill's own time split gives M, N and every
 * segment's start state; for GDN_BF16 with d_k = d_v its transition pass also
 * forms q^ and one streaming pass D, otherwise per-segment reverse sweeps give
 * D; a sequential fold gives every segment's end gradient; then both sweeps
 * run per segment.
 * Same results up to rounding.  GDN_BACKWARD_SEGMENT=L forces the length
 * (rounded up to a multiple of 64), 0 turns the split off; it must not
 * change between the workspace query and the call. */
int32_t gdn_prefill_backward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                             const float* initial_state, const void* d_o, const float* d_final_state, void* dq,
                             void* dk, void* dv, float* dg, float* dbeta, float* d_initial_state, int32_t H,
                             int32_t d_k, int32_t d_v, int32_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/* The two ways of forming the intra-tile ("diagonal tile") pair terms that
 * gdn_prefill_tiles offers (see there). */
typedef enum gdn_tile_path { GDN_TILES_DENSE = 0, GDN_TILES_PAIRS = 1 } gdn_tile_path;

/* Prefill in 16-token windows with a choice of diagonal-tile path: the
 * comparison the pages describe between a bounded and an unbounded log-decay
 * ("How to Think About Trillion-Parameter Sparse Multimodal LLMs", section 3;
 * "What a Trillion-Parameter MoE Model Reveals About the Next Stage of LLM
 * Scaling", section 3.2).  Inside a window the pair terms carry the decay
 * e^{G_t - G_s} between two of its tokens (G the window's cumulative
 * log-decay).
 *   GDN_TILES_DENSE  the decay is split into a row factor e^{G_t - m} and a
 *       column factor e^{m - G_s} about the window's middle token m and the
 *       pair terms are dense matrix-core products.  Needs g in [-5, 0] (the
 *       lower-bounded gate of "Trillion-Parameter MoE Multimodal LLMs: How to
 *       Evaluate the New Generation", section 3.1, which keeps both factors
 *       within e^-40 .. e^40); with a steeper gate the factors overflow and
 *       the results are not finite.
 *   GDN_TILES_PAIRS  each pair's decay is formed position by position on the
 *       vector units: valid for any finite g <= 0, e.g. the unbounded
 *       negative-softplus gate the pages replace.
 * Arguments, layouts and the result are as for gdn_prefill (no workspace;
 * final_state may alias initial_state), except g's domain: [-5, 0] for
 * GDN_TILES_DENSE, any finite g <= 0 for GDN_TILES_PAIRS (checked under
 * GDN_VALIDATE=1, GDN_ERR_DOMAIN).  An unknown tile_path is
 * GDN_ERR_INVALID_ARG.  For bounded gates gdn_prefill is the faster path;
 * this call exists for unbounded gates and for measuring what the
 * position-pair path costs. */
int32_t gdn_prefill_tiles(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, int32_t num_seqs, int64_t T_total,
                          const float* initial_state, float* final_state, void* o, int32_t H, int32_t d_k,
                          int32_t d_v, int32_t dtype, int32_t tile_path, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
