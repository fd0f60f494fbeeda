/*
 * liger_attn.h - C ABI of the Liger Attention layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer (paper-notes page "Liger: Linearizing Large Language Models to
 * Gated Recurrent Structures", sections on the unified gated linear
 * recurrence and on Liger Attention) mixes two token mixers inside one
 * attention layer:
 *
 *   GRM  S_t = G_t (.) S_{t-1} + phi(k_t)^T v_t ,   o_t = phi(q_t) S_t
 *   SWA  softmax attention of q_t over the last `window` keys (self included)
 *   out  o_t = alpha * GRM + (1 - alpha) * SWA
 *
 * phi is a softmax over the head dimension applied to q and k separately;
 * G_t is a parameter-free pooling of the raw key k_t squashed by a sigmoid
 * (the key projection reused as the gate, section on the gate built from the
 * key projection). The pages say only "pooling, e.g. mean"; the two pooled
 * gates offered here are:
 *   LIGER_GATE_SCALAR_MEAN     g_t = sigmoid(mean_c k_t[c]) on every entry of S
 *   LIGER_GATE_VECTOR_AVGPOOL4 g_t[c] = sigmoid(mean of k_t[c-1 .. c+2] over the
 *                              in-range channels), applied to row c (d_k) of S
 * The state starts at zero for prefill. The GRM output of token t uses the
 * state that already holds token t. SWA uses the raw q and k, scale 1/sqrt(d).
 * Query head h reads key/value head h / (H_q / H_kv).
 *
 * Layouts (row-major, contiguous, device memory unless stated otherwise):
 *   q, o   [B, T, H_q,  d]          dtype of the shape (fp32 or bf16)
 *   k, v   [B, T, H_kv, d]          same dtype
 *   S, S_T [B, H_kv, d, d]          float32, row index d_k, column index d_v
 *   ring   k, v [N, H_kv, window, d] input dtype; token t in slot t mod window
 *          pos  [N] int64: tokens consumed so far
 *          sync [N] uint32: arrival counters, zero between calls
 *
 * Conventions for every call:
 *   - Returns LIGER_OK (0) or a negative liger_status. liger_last_error()
 *     then returns a message (thread-local; valid until the next call on the
 *     same thread).
 *   - All arguments are validated before any HIP call; an invalid call
 *     launches nothing and touches no memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL means the default
 *     stream). The library never synchronises: results are valid once the
 *     caller has synchronised with the stream.
 *   - The caller owns every buffer. The library keeps no pointer after
 *     returning, allocates nothing and frees nothing. Device pointers must be
 *     16-byte aligned. Output buffers must not overlap the input buffers
 *     or each other (their byte ranges, from the shape, are checked:
 *     LIGER_E_INVALID_ARG); inputs may overlap one another.
 *   - No global mutable state: calls on different streams may run
 *     concurrently as long as their buffers do not overlap.
 *   - Floating-point inputs are not sanitised: NaN or Inf propagate.
 */
#ifndef LIGER_ATTN_H
#define LIGER_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum liger_status {
    LIGER_OK = 0,
    LIGER_E_INVALID_ARG = -1, /* bad pointer, size, enum or range            */
    LIGER_E_UNSUPPORTED = -2, /* valid but not built (e.g. d not in {64,128}) */
    LIGER_E_HIP = -3,         /* a HIP call or kernel launch failed           */
    LIGER_E_WORKSPACE = -4    /* workspace missing or too small               */
} liger_status;

typedef enum liger_gate_mode {
    LIGER_GATE_SCALAR_MEAN = 0,
    LIGER_GATE_VECTOR_AVGPOOL4 = 1
} liger_gate_mode;

typedef enum liger_dtype {
    LIGER_F32 = 0,
    LIGER_BF16 = 1
} liger_dtype;

/* Problem shape. B is the batch (number of sequences; N for decode), T the
 * sequence length (prefill; ignored by decode), d the head size (64 or 128),
 * dtype a liger_dtype for q, k, v, o and the ring. */
typedef struct liger_shape {
    int64_t B;
    int64_t T;
    int32_t H_q;
    int32_t H_kv;
    int32_t d;
    int32_t dtype;
} liger_shape;

/* Sliding-window KV ring of the decode state (all device pointers). */
typedef struct liger_kv_ring {
    void* k;        /* [N, H_kv, window, d], input dtype                     */
    void* v;        /* [N, H_kv, window, d], input dtype                     */
    int64_t* pos;   /* [N] tokens consumed; advanced by one per decode step  */
    uint32_t* sync; /* [N] arrival counters; zero before and after each call */
    int32_t window; /* 1 .. 64                                               */
} liger_kv_ring;
/*
 * The decode state of sequence n is (S[n], ring k/v of sequence n, pos[n]);
 * sync[n] holds nothing between calls: it is zero whenever no call on the
 * sequence is in flight (liger_kv_ring_fill and liger_attn_prefill_continue
 * set it to zero; a completed decode step leaves it zero). A snapshot of
 * (S, ring k/v, pos) taken between calls, with sync set to zero, is a
 * complete decode state. A decode step that finds sync[n] non-zero on entry
 * (memory never cleared, a snapshot restored without clearing it, a step
 * that did not complete) cannot tell when every workgroup of the sequence
 * has read pos[n]: it sets bit 31 of sync[n], which stays set, and from then
 * on pos[n] is not advanced. After synchronising, sync[n] != 0 reports this;
 * restore (S, ring, pos) from a snapshot and clear sync (or rebuild the ring
 * with liger_kv_ring_fill) to recover.
 */

/*
 * Meta-memory tokens ("attention sinks", Japanese summary page of Lizard,
 * section "アンカーウィンドウアテンション"): n extra key/value pairs per key/value
 * head that the sliding-window softmax of every query also sees, with the
 * same 1/sqrt(d) scale and no causal or window mask; they do not enter the
 * recurrence. Device pointers, dtype of the shape, 16-byte aligned, read only.
 */
typedef struct liger_sinks {
    const void* k;  /* [H_kv, n, d] */
    const void* v;  /* [H_kv, n, d] */
    int32_t n;      /* 1 .. 16      */
} liger_sinks;

/*
 * Defined by: the chunked ("right-multiplication", linear in T) evaluation
 * of the recurrence (news article on Liger, 手法の説明); the segments of
 * that evaluation need the carried states below.
 * Bytes of device workspace liger_attn_prefill needs for `shape`: the state
 * carried into each segment of the chunked scan and a running-state slot per
 * segment (fp32 at d = 128 also a state-operand slot per segment and 64
 * window-halo key and value rows per (b, kv head)). Returns 0 when the shape
 * is invalid. `chunks_per_segment` selects the segment length
 * in 64-token chunks; 0 picks it from the shape (the same choice the
 * prefill call makes when given 0).
 */
size_t liger_attn_prefill_workspace_size(const liger_shape* shape);
size_t liger_attn_prefill_workspace_size_ex(const liger_shape* shape,
                                            int32_t chunks_per_segment);

/*
 * Prefill: whole sequences from a zero state.
 * Defined by: paper-notes page "Liger: Linearizing Large Language Models to
 * Gated Recurrent Structures", sections 统一的门控线性循环框架 (the gated
 * recurrence and its output), Liger Attention：层内混合注意力 (the alpha/beta
 * mix with window-64 softmax attention) and 核心思想：Key 投影复用构建门控 (the
 * gate pooled from the key); one of the two calls of this boundary.
 * Inputs q, k, v (layouts above). Outputs o [B, T, H_q, d] (dtype of q) and
 * S_T [B, H_kv, d, d] float32, the state after the last token.
 * window in 1..64, alpha in [0, 1] (beta = 1 - alpha).
 * workspace: device memory of at least liger_attn_prefill_workspace_size
 * bytes (may be NULL when that size is 0); its contents on entry are
 * ignored and on return are unspecified.
 * Supported: d in {64, 128} for bf16 and for fp32.
 */
liger_status liger_attn_prefill(const void* q, const void* k, const void* v,
                                int32_t gate_mode, int32_t window, float alpha,
                                const liger_shape* shape, void* o, float* S_T,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* As liger_attn_prefill with an explicit segment length (0 = automatic);
 * every segment length gives the same result up to float32 rounding.
 * Defined by: the same sections as liger_attn_prefill (a tuning extension
 * of that call). */
liger_status liger_attn_prefill_ex(const void* q, const void* k, const void* v,
                                   int32_t gate_mode, int32_t window, float alpha,
                                   const liger_shape* shape, void* o, float* S_T,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t chunks_per_segment, void* stream);

/*
 * liger_attn_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and result as liger_attn_prefill, with
 * the workspace taken from scratch memory the library holds instead of a
 * caller buffer. The scratch is one static block of
 * liger_attn_prefill_noalloc_max_workspace() bytes (32 MiB) on each GPU the
 * library runs on, kept until the process ends; the call allocates and
 * frees nothing. It runs on the current device (hipGetDevice), which must
 * be the device of `stream`.
 *   Shapes whose liger_attn_prefill_workspace_size exceeds that size are
 *   rejected with LIGER_E_WORKSPACE before anything is launched.
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (different streams or threads, without ordering between
 *   them) race and give undefined results. Calls ordered on one stream are
 *   safe: nothing in the scratch needs to start at zero and every byte read
 *   is written earlier in the same call.
 * Other arguments, layouts and errors as for liger_attn_prefill.
 */
size_t liger_attn_prefill_noalloc_max_workspace(void);
liger_status liger_attn_prefill_noalloc(const void* q, const void* k, const void* v,
                                        int32_t gate_mode, int32_t window, float alpha,
                                        const liger_shape* shape, void* o, float* S_T,
                                        void* stream);

/*
 * Defined by: the same sections as liger_attn_prefill (a profiling
 * extension of that call: it computes nothing else).
 * Profiling aid: enqueue only the prefill kernels chosen by stage_mask, in
 * pipeline order: LIGER_STAGE_SEGMENT_STATES (local end state of every
 * segment but the last), LIGER_STAGE_CARRY_SCAN (states entering each
 * segment, in the workspace) and LIGER_STAGE_OUTPUT (o and S_T). Enqueuing
 * mask 3 and then mask 4 on one stream with the same workspace is the same
 * work as one liger_attn_prefill_ex call. Other arguments as for
 * liger_attn_prefill_ex; stage_mask must be in 1..7.
 */
#define LIGER_STAGE_SEGMENT_STATES 1
#define LIGER_STAGE_CARRY_SCAN 2
#define LIGER_STAGE_OUTPUT 4
liger_status liger_attn_prefill_stages(const void* q, const void* k, const void* v,
                                       int32_t gate_mode, int32_t window, float alpha,
                                       const liger_shape* shape, void* o, float* S_T,
                                       void* workspace, size_t workspace_bytes,
                                       int32_t chunks_per_segment, int32_t stage_mask,
                                       void* stream);

/*
 * Prefill continuation: T = shape->T more tokens for each of B sequences
 * after the kv_ring->pos[b] tokens already consumed, from the state S0 and
 * the KV ring those tokens left (after liger_attn_prefill + liger_kv_ring_fill,
 * decode steps or an earlier continuation). The result equals one prefill of
 * the concatenated sequence restricted to the new tokens, and T decode steps
 * (the fixed-size decoding state of the recurrence; paper-notes page "Liger:
 * Linearizing Large Language Models to Gated Recurrent Structures", unified
 * gated linear recurrence; news article on Liger, 実験分析: constant-memory
 * decoding).
 *   q [B, T, H_q, d], k, v [B, T, H_kv, d] (dtype of the shape); o as q.
 *   S0 [B, H_kv, d, d] float32, read only; S_T [B, H_kv, d, d] float32,
 *   written; they must not overlap.
 *   kv_ring: window = kv_ring->window (1..64) is the attention window; the
 *   ring is read, then the last min(T, window) new tokens are written to
 *   slots (pos + t) mod window, older slots keep their tokens, pos[b] += T
 *   and sync[b] = 0. Entries of pos may differ between sequences.
 *   workspace as for liger_attn_prefill (liger_attn_prefill_workspace_size).
 * gate_mode and alpha must be those that produced S0. Errors as for
 * liger_attn_prefill; a NULL ring, pos or sync is LIGER_E_INVALID_ARG.
 */
liger_status liger_attn_prefill_continue(const void* q, const void* k, const void* v,
                                        const float* S0, const liger_kv_ring* kv_ring,
                                        int32_t gate_mode, float alpha,
                                        const liger_shape* shape, void* o, float* S_T,
                                        void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * Decode step: one new token for each of N = shape->B sequences.
 * Defined by: paper-notes page "Liger: Linearizing Large Language Models to
 * Gated Recurrent Structures", 统一的门控线性循环框架 (the recurrence taken
 * one token at a time: S_t from S_{t-1}) and Liger Attention：层内混合注意力
 * (the window of the most recent tokens); news article on Liger, 実験分析
 * (decoding with a fixed-size state instead of a growing cache). The second
 * call of this boundary.
 * q [N, H_q, d], k, v [N, H_kv, d] (dtype of the shape); o [N, H_q, d].
 * S [N, H_kv, d, d] float32 is updated in place to G (.) S + phi(k)^T v.
 * The ring is updated in place: the new k, v go to slot pos mod window, the
 * window of `window` most recent tokens (the new one included) is attended
 * to, and pos advances by one. gate_mode and alpha must be those of the
 * prefill that produced the state. shape->T is ignored.
 * o, S, the ring's k, v, pos and sync are written: their byte ranges must be
 * pairwise disjoint and must not overlap q, k, v or the sink tokens
 * (LIGER_E_INVALID_ARG). sync must be zero on entry (see liger_kv_ring).
 */
liger_status liger_attn_decode_step(const void* q, const void* k, const void* v,
                                    float* S, const liger_kv_ring* kv_ring,
                                    int32_t gate_mode, float alpha,
                                    const liger_shape* shape, void* o,
                                    void* stream);

/*
 * Defined by: paper-notes page "Liger: Linearizing Large Language Models to
 * Gated Recurrent Structures", Liger Attention：层内混合注意力 (the softmax
 * attention sees only the last `window` tokens, so only those are kept) and
 * news article on Liger, 実験分析 (fixed-size decoding state).
 * Ring set-up after a prompt: copies the last min(T, window) tokens of
 * k, v [B, T, H_kv, d] to slots t mod window, zeroes the other slots,
 * sets pos = T and sync = 0. (Together with S_T from the prefill this is the
 * complete decode state.) The ring's k, v, pos and sync must be pairwise
 * disjoint and must not overlap k or v (LIGER_E_INVALID_ARG).
 */
liger_status liger_kv_ring_fill(const void* k, const void* v,
                                const liger_shape* shape,
                                const liger_kv_ring* kv_ring, void* stream);

/*
 * The hybrid's standard softmax attention layer (paper-notes page "Liger:
 * Linearizing Large Language Models to Gated Recurrent Structures", section
 * "Liger 整体架构": a softmax attention block after every few Liger blocks):
 *   o_t = sum_{j <= t} softmax_j(q_t . k_j / sqrt(d)) v_j
 * for every query head h, which reads key/value head h / (H_q / H_kv).
 * q, o [B, T, H_q, d]; k, v [B, T, H_kv, d]; contiguous, device memory,
 * 16-byte aligned, bf16 only (fp32 is LIGER_E_UNSUPPORTED), d in {64, 128},
 * H_q / H_kv in {1, 2, 4, 8}. o must not overlap the inputs. No workspace;
 * enqueued on `stream` (NULL: the default stream), nothing is synchronised.
 */
liger_status liger_attn_full_causal(const void* q, const void* k, const void* v,
                                    const liger_shape* shape, void* o, void* stream);

/*
 * The three calls above with meta-memory tokens (liger_sinks) prepended to
 * every sliding window: o's window part becomes softmax over
 * [sink keys; window keys] applied to [sink values; window values]. The
 * same arguments as liger_attn_prefill, liger_attn_prefill_continue and
 * liger_attn_decode_step; `sinks` must not be NULL and sinks->n must be in
 * 1..16 (else LIGER_E_INVALID_ARG). A decode or a continuation must be given
 * the sinks its prefill used.
 */
liger_status liger_attn_prefill_sinks(const void* q, const void* k, const void* v,
                                      const liger_sinks* sinks, int32_t gate_mode,
                                      int32_t window, float alpha,
                                      const liger_shape* shape, void* o, float* S_T,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);
liger_status liger_attn_prefill_continue_sinks(const void* q, const void* k, const void* v,
                                              const float* S0, const liger_kv_ring* kv_ring,
                                              const liger_sinks* sinks, int32_t gate_mode,
                                              float alpha, const liger_shape* shape,
                                              void* o, float* S_T, void* workspace,
                                              size_t workspace_bytes, void* stream);
liger_status liger_attn_decode_step_sinks(const void* q, const void* k, const void* v,
                                          float* S, const liger_kv_ring* kv_ring,
                                          const liger_sinks* sinks, int32_t gate_mode,
                                          float alpha, const liger_shape* shape, void* o,
                                          void* stream);

/*
 * Backward of liger_attn_prefill (training): the gradients of
 * L = sum(o * dO) with respect to q, k and v, for o the prefill output of
 * q, k, v from a zero state (paper-notes page "Liger: Linearizing Large
 * Language Models to Gated Recurrent Structures": unified gated linear
 * recurrence, Liger Attention, and the gate built from the key projection;
 * the gradient flows through phi, the pooled sigmoid gate and both token
 * mixers).
 *   q, dO [B, T, H_q, d]; k, v [B, T, H_kv, d]: bf16 only (fp32 is
 *   LIGER_E_UNSUPPORTED), d in {64, 128}, any H_q / H_kv.
 *   dq [B, T, H_q, d], dk, dv [B, T, H_kv, d]: float32, written (not
 *   accumulated); pairwise disjoint and not overlapping any input.
 *   gate_mode, window (1..64) and alpha as given to the prefill.
 *   workspace: at least liger_attn_prefill_backward_workspace_size bytes of
 *   device memory (chunk-start states, chunk adjoints, per-row gate
 *   gradients and window statistics); contents on entry ignored, on return
 *   unspecified.
 * Meta-memory sink tokens are not part of this call.
 */
size_t liger_attn_prefill_backward_workspace_size(const liger_shape* shape);
liger_status liger_attn_prefill_backward(const void* q, const void* k, const void* v,
                                         const void* dO, int32_t gate_mode, int32_t window,
                                         float alpha, const liger_shape* shape,
                                         float* dq, float* dk, float* dv,
                                         void* workspace, size_t workspace_bytes,
                                         void* stream);

/* Message of the last failed call on this thread ("" if none). A helper of
 * the boundary: it reports errors and computes nothing. */
const char* liger_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIGER_ATTN_H */
