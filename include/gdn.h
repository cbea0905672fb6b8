/*
 * gdn.h -- C ABI of the gated delta-rule (Gated DeltaNet) sequence mixer for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the gated delta rule of "Long-Context Aware Upcycling: A
 * New Frontier for Hybrid LLM Scaling" (arXiv:2604.24715), App. A.3 "GDN Layer
 * Architecture", Eqs. 16-19.  Per sequence n and head h a fixed-size fp32
 * state S (d_v x d_k) replaces the KV cache; each token t does
 *
 *     S_t = e^{g_t} S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * which is Eqs. 16-18 (decay, delta correction, write) with the decay and the
 * correction multiplied out, and Eq. 19 (read of the updated state).  The
 * paper's state is d_k x d_v with o = S^T q; this library stores its
 * transpose, row i = value index, so every state row is one contiguous d_k
 * vector.  g_t <= 0 is the log forget gate (alpha_t = e^{g_t}) and
 * beta_t in (0, 1) the write strength, as stated under Eq. 21.
 *
 * Optional q/k L2 normalisation (qk_l2norm != 0) replaces x by
 * x / sqrt(sum(x^2) + 1e-6) per (token, head) before use.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers unless the name ends in _host.
 *   - The caller owns and allocates every buffer (including the workspace);
 *     the library never allocates device memory and keeps no process-wide
 *     state.  The only HIP objects it creates are those of an execution
 *     context (gdn_context_create), which the caller owns and destroys.
 *   - Work is enqueued on `stream` (and, for the _ctx calls, on the streams
 *     of the context, forked from and joined back to `stream`) and runs
 *     asynchronously; no call synchronises the device (unless
 *     GDN_DEBUG_SYNC=1 is set, which makes each call wait for its kernels and
 *     report launch/device errors).  Every call may be captured into a HIP
 *     graph, the first one included: nothing a call enqueues is a memset, a
 *     copy or a synchronisation.
 *   - Argument errors are detected on the host before anything is launched
 *     and returned as a gdn_status; nothing is written in that case.
 *   - Results are deterministic: no atomics, fixed reduction order.
 *   - Calls on different streams with disjoint buffers may run concurrently.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,     /* a required pointer is NULL                                  */
    GDN_ERR_BAD_SHAPE = 2,    /* negative / zero sizes, or sizes that disagree              */
    GDN_ERR_UNSUPPORTED = 3,  /* (dtype, d_k, d_v, chunk) combination not built             */
    GDN_ERR_BAD_SEQLENS = 4,  /* cu_seqlens not 0 = c_0 <= c_1 <= ... <= c_N = total_tokens  */
    GDN_ERR_ALIGNMENT = 5,    /* q/k/v/o/state not 16-byte, g/beta not 4-byte aligned       */
    GDN_ERR_WORKSPACE = 6,    /* workspace NULL or too small (see gdn_prefill_workspace_size)  */
    GDN_ERR_LAUNCH = 7,       /* a kernel launch failed (or, under GDN_DEBUG_SYNC, faulted) */
    GDN_ERR_CONTEXT = 8       /* context creation failed, or the context belongs to another device */
} gdn_status;

/* Element type of q, k, v and o.  Gates, beta and states are always fp32. */
typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/*
 * Supported combinations (anything else returns GDN_ERR_UNSUPPORTED):
 *   GDN_F32 : d_k, d_v in {16, 32, 64, 128, 256}, chunk in {16, 32, 64}
 *   GDN_BF16: d_k in {64, 128, 256}, d_v in {64, 128, 256, 512}, chunk = 64
 * gdn_decode_step has no chunk and accepts any d_k, d_v in the lists above.
 */

/*
 * Bytes of device workspace gdn_chunk_prefill needs for these sizes.
 * Returns 0 for an unsupported or invalid combination.  The workspace holds
 * per-chunk intermediates of the chunked (WY) evaluation and is fully
 * rewritten by every call; its contents between calls are meaningless.
 */
size_t gdn_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk,
                                  int32_t dv, int32_t chunk, gdn_dtype dt);

/*
 * Smallest workspace gdn_chunk_prefill (and the _ctx, _gated and _frontend
 * forms) accept for these sizes: room for the chunk table, the per-sequence
 * fp32 state carry (num_seqs x H x dv x dk) and one chunk's intermediates.
 * Between this and gdn_prefill_workspace_size, the call processes the chunks
 * in the largest windows that fit, one window after another on its stream
 * (each stage over the window, each sequence's state carried from window to
 * window in fp32); results are bit-identical to a full-size workspace's, the
 * overlap of the stages is given up, and a sequence cut by window boundaries
 * runs its chain in pieces.  (gdn_chunk_prefill_staged with a subset of the
 * stages needs the full size.)  Returns 0 for an unsupported combination.
 */
size_t gdn_prefill_workspace_min_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk,
                                      int32_t dv, int32_t chunk, gdn_dtype dt);

/*
 * Chunked prefill over packed variable-length sequences (App. A.3, last
 * paragraph: the sequence is cut into chunks of `chunk` tokens, the delta
 * corrections inside a chunk are batched through the WY representation and
 * the state is carried from chunk to chunk).  The result equals the
 * token-by-token recurrence above up to floating-point rounding.
 *
 *   q, k        [total_tokens, H, dk]   dt, contiguous, 16-byte aligned
 *   v           [total_tokens, H, dv]   dt
 *   g, beta     [total_tokens, H]       fp32 (log forget gate, write strength),
 *               4-byte aligned
 *   init_state  [num_seqs, H, dv, dk]   fp32, or NULL for zeros
 *   cu_seqlens  device int32 [num_seqs + 1], sequence n owns tokens
 *               [cu_seqlens[n], cu_seqlens[n+1]); NULL means one sequence
 *               (num_seqs must then be 1).
 *   cu_seqlens_host  optional host mirror of cu_seqlens (same values).  When
 *               given it is validated on the host (GDN_ERR_BAD_SEQLENS) and
 *               used to schedule sequences; when NULL the device copy is
 *               trusted: invalid contents are clamped so no access leaves its
 *               buffer, and the outputs are then unspecified.
 *   scale       read scale of Eq. 19; scale <= 0 selects 1/sqrt(dk)
 *   qk_l2norm   nonzero: L2-normalise q and k per (token, head)
 *   o           [total_tokens, H, dv]   dt (written)
 *   final_state [num_seqs, H, dv, dk]   fp32 (written), may be NULL, may
 *               alias init_state exactly (in-place carry)
 *   workspace   device buffer, 256-byte aligned, of gdn_prefill_workspace_size(...)
 *               bytes, or of fewer but at least gdn_prefill_workspace_min_size(...)
 *               (then processed in windows of chunks, see there)
 * Sequences of length 0 are allowed: their final state equals the initial.
 */
gdn_status gdn_chunk_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             const float* init_state, const int32_t* cu_seqlens,
                             const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens,
                             int32_t H, int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                             int32_t qk_l2norm, void* o, float* final_state, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * The stages of gdn_chunk_prefill, for callers that schedule or time them
 * separately.  Same arguments and rules as gdn_chunk_prefill, plus `stages`,
 * a bit set of:
 *   GDN_STAGE_PREPARE    per-chunk work, fully parallel over (chunk, head):
 *                        chunk table, q/k norms, cumulative log-decay, the
 *                        triangular solve, the WY factors W and U and the
 *                        intra-chunk scores P, written into the workspace
 *                        (reads q, k, v, g, beta; writes only the workspace);
 *   GDN_STAGE_PROPAGATE  the sequential pass over each sequence's chunks (the
 *                        state carry): reads the workspace left by PREPARE and
 *                        init_state; writes final_state and, into the
 *                        workspace, the state entering every chunk and the
 *                        chunk's corrected values;
 *   GDN_STAGE_OUTPUT     the outputs of every chunk, fully parallel over
 *                        (chunk, head), from the workspace left by PREPARE and
 *                        PROPAGATE; writes o;
 *   GDN_STAGE_ALL        all three, in order (what gdn_chunk_prefill does).
 * Stages of one prefill must be enqueued in order on one stream (or ordered
 * by the caller) with the same workspace and the same inputs and sizes.
 */
#define GDN_STAGE_PREPARE 1
#define GDN_STAGE_PROPAGATE 2
#define GDN_STAGE_OUTPUT 4
#define GDN_STAGE_ALL 7
gdn_status gdn_chunk_prefill_staged(const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, const float* init_state, const int32_t* cu_seqlens,
                                    const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens,
                                    int32_t H, int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                    int32_t qk_l2norm, void* o, float* final_state, void* workspace,
                                    size_t workspace_bytes, int32_t stages, hipStream_t stream);

/*
 * Execution context of the overlapped (pipelined) prefill.  Opaque and owned
 * by the caller, like a library handle: gdn_context_create makes, on the
 * device that is current, the streams and events that let one prefill call
 * overlap its three stages -- one stream for the sequential state chain,
 * CU-masked to `chain_cus_per_xcd` compute units of every XCD (the chain of
 * the 64K-token workload, B=1, H=6, d=256, needs 16), and two streams for the
 * per-chunk preparation and output kernels on the other CUs -- and
 * gdn_context_destroy waits for the context's streams and releases them.
 *
 *   chain_cus_per_xcd  CUs reserved for the chain on each XCD, 1..31; 0 or
 *                      less selects the default (16).  On a device that is not
 *                      a 256-CU MI355X the streams are created without masks.
 *
 * A context serves calls on its own device only (GDN_ERR_CONTEXT otherwise);
 * calls that share a context are ordered on the host by a lock inside it
 * (they may come from several threads).  It must not be destroyed while a
 * call that uses it is being enqueued or captured, nor while a captured graph
 * that contains its streams' work is still to be replayed.
 * Errors: GDN_ERR_NULL_ARG (ctx == NULL), GDN_ERR_BAD_SHAPE
 * (chain_cus_per_xcd > 31), GDN_ERR_CONTEXT (a stream or event could not be
 * created; nothing is left allocated).
 */
typedef struct gdn_context* gdn_context_t;
gdn_status gdn_context_create(int32_t chain_cus_per_xcd, gdn_context_t* ctx);
gdn_status gdn_context_destroy(gdn_context_t ctx);

/*
 * gdn_chunk_prefill with an execution context: when the sequences' state
 * chains fit in the context's CU reservation and the batch is long enough for
 * the overlap to pay (at least 576 chunks), the chunks are cut into segments
 * and the chain of each segment runs on the context's chain stream while the
 * preparation of later segments and the outputs of earlier ones run beside
 * it; otherwise, and with ctx == NULL, it is exactly gdn_chunk_prefill.  The
 * results are bit-identical to gdn_chunk_prefill's either way.  The context's
 * streams wait for `stream` on entry and `stream` waits for them before the
 * call's last kernel, so the call is ordered on `stream` like any other.
 */
gdn_status gdn_chunk_prefill_ctx(gdn_context_t ctx, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* init_state, const int32_t* cu_seqlens,
                                 const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens, int32_t H,
                                 int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                 int32_t qk_l2norm, void* o, float* final_state, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory -- code being captured into
 * a HIP graph, serving loops that must not call hipMalloc, harnesses that
 * forbid it: gdn_chunk_prefill without a workspace argument.  The workspace is
 * a device array inside the library, GDN_NOALLOC_SCRATCH_BYTES (256 MiB) on
 * every GPU the library is used on, held from the library's first use on that
 * device until the process ends; the call itself allocates nothing.  When the
 * call's workspace (gdn_prefill_workspace_size) is larger, the chunks are
 * processed in windows that fit, one after another on `stream`, each
 * sequence's state carried from window to window in fp32; the results are
 * bit-identical to gdn_chunk_prefill's.  Sizes whose fixed part (chunk table
 * and the num_seqs x H x dv x dk fp32 carry) leaves no room for even one chunk
 * are rejected with GDN_ERR_WORKSPACE before anything is launched.
 * Every call on one GPU uses the same array and leaves its contents behind
 * (nothing in it needs to start at zero): calls that can overlap on one GPU --
 * on different streams, or from several threads without ordering -- race on
 * it and must be serialised by the caller.  Arguments and every other rule as
 * for gdn_chunk_prefill.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
gdn_status gdn_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const float* init_state, const int32_t* cu_seqlens,
                                     const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens,
                                     int32_t H, int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                     int32_t qk_l2norm, void* o, float* final_state, hipStream_t stream);

/*
 * One recurrent decode step for N independent sequences (the token-level
 * recurrence above with one token per sequence; the serving form of the
 * fixed-size state described in App. A.3 and the HyLo-Qwen GDN model card).
 *
 *   q, k   [N, H, dk]  dt;   v [N, H, dv] dt (16-byte aligned);
 *   g, beta [N, H] fp32 (4-byte aligned)
 *   state  [N, H, dv, dk] fp32, read and updated IN PLACE
 *   o      [N, H, dv]  dt (written)
 * Each state row is streamed from HBM exactly once (read, update, write).
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           float* state, int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt,
                           float scale, int32_t qk_l2norm, void* o, hipStream_t stream);

/*
 * Gated RMSNorm read-out (App. A.3, Eq. 20: the read of the updated state is
 * normalised and gated by a projection of the layer input before the output
 * projection of Eq. 21).  Same as gdn_chunk_prefill / gdn_decode_step, except
 * that every output row -- one token and head, d_v values -- becomes
 *
 *     y = o / sqrt(mean_v(o_v^2) + norm_eps) * norm_weight * silu(gate)
 *
 * with o the read of Eq. 19 (scale included) and silu(x) = x / (1 + e^{-x}).
 *
 *   gate        [tokens (or N), H, dv]  dt, the gate input W_G x_t (the
 *               projection itself is the caller's), 16-byte aligned; required
 *               when there is at least one token
 *   norm_weight [dv] fp32 per-channel weight shared by all heads, 4-byte
 *               aligned, or NULL for ones
 *   norm_eps    >= 0 and finite (GDN_ERR_BAD_SHAPE otherwise)
 *
 * The prefill applies the norm to the fp32 outputs inside its output stage.
 * The decode step applies it in a second small kernel to the row as stored in
 * o (rounded to bf16 when dt is GDN_BF16), since one head's rows are spread
 * over several workgroups.
 */
gdn_status gdn_chunk_prefill_gated(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                   const float* init_state, const int32_t* cu_seqlens,
                                   const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens, int32_t H,
                                   int32_t dk, int32_t dv, int32_t chunk, gdn_dtype dt, float scale,
                                   int32_t qk_l2norm, const void* gate, const float* norm_weight, float norm_eps,
                                   void* o, float* final_state, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* gdn_chunk_prefill_gated with an execution context (see gdn_chunk_prefill_ctx). */
gdn_status gdn_chunk_prefill_gated_ctx(gdn_context_t ctx, const void* q, const void* k, const void* v,
                                       const float* g, const float* beta, const float* init_state,
                                       const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                       int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                                       gdn_dtype dt, float scale, int32_t qk_l2norm, const void* gate,
                                       const float* norm_weight, float norm_eps, void* o, float* final_state,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

gdn_status gdn_decode_step_gated(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 float* state, int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt,
                                 float scale, int32_t qk_l2norm, const void* gate, const float* norm_weight,
                                 float norm_eps, void* o, hipStream_t stream);

/*
 * Front end of the mixer (App. A.3): the short convolution with SiLU applied
 * to Q, K and V before the recurrence (the paragraph under Table 8: kernel
 * size 4), and the gates of the paragraph after Eq. 21:
 *
 *     q_t[c] = silu(sum_{j=0..3} w[c][j] xq_{t-3+j}[c])       (likewise k, v)
 *     g_t    = -exp(A_log[h]) * softplus(a_t[h] + dt_bias[h])
 *     beta_t = sigmoid(b_t[h])
 *
 * The convolution is causal and depthwise (each channel mixes only its own
 * past three inputs and the current one; tap 3 multiplies the current token)
 * and has no bias.  silu(u) = u / (1 + e^{-u}), softplus(u) = log(1 + e^u),
 * sigmoid(u) = 1 / (1 + e^{-u}); the arithmetic is fp32, the outputs q, k, v
 * are rounded to dt (round to nearest even).  The projections W_Q x, W_K x,
 * W_V x, W_alpha x, W_beta x are the caller's: their results are the inputs.
 *
 * Channel axis: the channels of q, k and v are numbered as one axis of
 * ctot = 2 H dk + H dv channels -- q's H*dk (head-major), then k's, then v's.
 *
 *   xq, xk        [tokens, H, dk]  dt;  xv [tokens, H, dv] dt (16-byte aligned)
 *   conv_weight   [ctot][4] fp32 taps, oldest first (16-byte aligned)
 *   a, b          [tokens, H] fp32: W_alpha x_t and W_beta x_t
 *   A_log, dt_bias [H] fp32
 *   q, k, v       outputs shaped like xq, xk, xv (dt); g, beta [tokens, H] fp32
 *   conv state    [num_seqs (or N), 3, ctot] dt: the three inputs before the
 *                 next token of each sequence, oldest first.  dk and dv must
 *                 be multiples of 8.
 *
 * Prefill: sequence n of cu_seqlens (as for gdn_chunk_prefill; NULL = one
 * sequence) starts from conv_state_in[n] (NULL: zeros) and nothing crosses a
 * sequence boundary.  conv_state_out (may be NULL; may alias conv_state_in
 * exactly) receives the last three inputs of every sequence, reaching into
 * conv_state_in for sequences shorter than three tokens.  The outputs q, k,
 * v, g, beta are the inputs of gdn_chunk_prefill.
 * Decode: one token per sequence; conv_state is read and updated in place.
 * The outputs are the inputs of gdn_decode_step.
 */
gdn_status gdn_frontend_prefill(const void* xq, const void* xk, const void* xv, const float* conv_weight,
                                const float* a, const float* b, const float* A_log, const float* dt_bias,
                                const void* conv_state_in, const int32_t* cu_seqlens, int32_t num_seqs,
                                int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, void* q,
                                void* k, void* v, float* g, float* beta, void* conv_state_out, hipStream_t stream);

gdn_status gdn_frontend_decode(const void* xq, const void* xk, const void* xv, const float* conv_weight,
                               const float* a, const float* b, const float* A_log, const float* dt_bias,
                               void* conv_state, int32_t N, int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, void* q,
                               void* k, void* v, float* g, float* beta, hipStream_t stream);

/*
 * The front end folded into the chunked prefill: the same result as
 * gdn_frontend_prefill followed by gdn_chunk_prefill_ctx, bit for bit, without
 * the round trip of q, k, v, g and beta through device memory.  The paragraph
 * under Table 8 of App. A.3 puts the short convolution with SiLU directly
 * before the recurrence; here it runs inside the per-chunk preparation: each
 * chunk's preparation reads the projections of its tokens plus the three
 * before them (or the sequence's conv state), convolves, applies SiLU, rounds
 * to bf16 as the front end does, and computes g and beta from a and b.
 *
 *   ctx, init_state, cu_seqlens, cu_seqlens_host, num_seqs, total_tokens, H,
 *   dk, dv, chunk, scale, qk_l2norm, o, final_state, workspace,
 *   workspace_bytes, stream      as for gdn_chunk_prefill_ctx (ctx may be NULL)
 *   xq, xk, xv, conv_weight, a, b, A_log, dt_bias, conv_state_in,
 *   conv_state_out               as for gdn_frontend_prefill
 * Supported: dt = GDN_BF16, chunk 64 (the combinations of gdn_chunk_prefill
 * for bf16); anything else returns GDN_ERR_UNSUPPORTED.  conv_state_out may
 * alias conv_state_in exactly; it is written after every read of it.
 */
gdn_status gdn_chunk_prefill_frontend(gdn_context_t ctx, const void* xq, const void* xk, const void* xv,
                                      const float* conv_weight, const float* a, const float* b, const float* A_log,
                                      const float* dt_bias, const void* conv_state_in, const float* init_state,
                                      const int32_t* cu_seqlens, const int32_t* cu_seqlens_host, int32_t num_seqs,
                                      int64_t total_tokens, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                                      gdn_dtype dt, float scale, int32_t qk_l2norm, void* o, float* final_state,
                                      void* conv_state_out, void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/*
 * Bytes of device workspace gdn_chunk_prefill_backward needs for these sizes
 * (0 for an unsupported or invalid combination).  It holds per-chunk
 * intermediates in 4-byte slots, among them the state entering every chunk
 * and the state gradient after it: max_chunks * H * (2 dv dk + 64 (10 dk +
 * 8 dv) + 7 * 64 * 64 + 5 * 64) * 4 bytes plus the chunk table and 256-byte
 * alignment, max_chunks = total_tokens / 64 + num_seqs.
 */
size_t gdn_prefill_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t H, int32_t dk,
                                           int32_t dv);

/*
 * Gradients of the chunked prefill.  Training evaluates the mixer in chunks
 * (App. A.3, the paragraph after Eq. 21), so this differentiates the chunked
 * (WY) form of gdn_chunk_prefill with chunk 64: given the cotangents d_o of
 * the outputs and d_final_state of the final states, it returns the
 * gradients of  L = sum <d_o, o> + sum <d_final_state, final_state>  with
 * respect to q, k, v, g, beta and the initial state, through the optional
 * q/k L2 normalisation.  It recomputes the forward from the inputs (nothing
 * of a previous gdn_chunk_prefill call is reused).
 *
 *   q, k, v, g, beta, init_state, cu_seqlens, cu_seqlens_host, num_seqs,
 *   total_tokens, H, dk, dv, dt, scale, qk_l2norm
 *               as for gdn_chunk_prefill
 *   d_o         [total_tokens, H, dv]  dt
 *   d_final_state [num_seqs, H, dv, dk] fp32, or NULL for zeros
 *   grad_q, grad_k [total_tokens, H, dk]  fp32 (written)
 *   grad_v      [total_tokens, H, dv]  fp32 (written)
 *   grad_g, grad_beta [total_tokens, H] fp32 (written)
 *   grad_init_state [num_seqs, H, dv, dk] fp32 (written), or NULL
 *   workspace   at least gdn_prefill_backward_workspace_size(...) bytes,
 *               256-byte aligned
 * Supported: dt in {GDN_F32, GDN_BF16}, dk and dv in {64, 128, 256}.
 * Intermediates and sums are fp32; the per-chunk products run on the fp32
 * matrix cores, the two state recurrences on the bf16 ones with every fp32
 * operand split into bf16 hi and lo parts (three products per pair; a bf16
 * input row is exact in its hi part).  Every gradient stays within 1e-4 of
 * the rms of an fp64 evaluation on the tested workloads.  Gradient buffers must not overlap the
 * inputs or each other; for grad_init_state against init_state and
 * d_final_state this is checked (GDN_ERR_BAD_SHAPE).  With an invalid device cu_seqlens (and no host
 * mirror) no chunk is processed and the gradients are unspecified.
 */
gdn_status gdn_chunk_prefill_backward(const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const float* init_state, const void* d_o,
                                      const float* d_final_state, const int32_t* cu_seqlens,
                                      const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens,
                                      int32_t H, int32_t dk, int32_t dv, gdn_dtype dt, float scale,
                                      int32_t qk_l2norm, float* grad_q, float* grad_k, float* grad_v,
                                      float* grad_g, float* grad_beta, float* grad_init_state, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* gdn_status_string(gdn_status s);

/* Library version as major*10000 + minor*100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
