/*
 * gdn.h -- C ABI of libgdn.so, the MI355X (gfx950) Gated DeltaNet library.
 *
 * A Gated DeltaNet (GDN) layer mixes tokens through a fixed-size recurrent
 * state per head instead of a per-token key/value cache (flozi.net,
 * "Qwen3.8-Flash-Next architecture": the stack table, 48 token-mixing layers
 * of which 36 are GDN, and "Der Weg eines Tokens durch das Modell", item 1).
 * The pages give no formula; the recurrence computed here, per value head with
 * an fp32 state S of shape d_v x d_k, is the gated delta rule
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,                 alpha_t = exp(g_t),
 *
 * with the output read after the token's own write, no query scaling and no
 * normalisation of q or k inside the library (except in the *_raw entry
 * points, which take the raw projections; see below).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller; the library
 *   keeps no pointer after the call returns.  Work is enqueued on `stream`
 *   (a hipStream_t; NULL = the null stream) and the call returns without
 *   waiting: the caller synchronises before reading results.
 * - Layouts are dense row-major, token-major:
 *     q, k         [tokens, num_qk_heads, head_dim_k]   element type `dtype`
 *     v, out       [tokens, num_v_heads,  head_dim_v]   element type `dtype`
 *     g, beta      [tokens, num_v_heads]                fp32 (g = log alpha <= 0, beta in [0, 1])
 *     state        [num_seqs, num_v_heads, head_dim_v, head_dim_k]  fp32
 *   Value head h reads q/k head floor(h * num_qk_heads / num_v_heads)
 *   (grouped value heads: contiguous groups share one q/k head).
 * - Alignment: q, k, v, out and states 16-byte aligned; g, beta 4-byte.
 * - Supported: head_dim_k, head_dim_v in {64, 128}; num_v_heads a multiple of
 *   num_qk_heads; dtype fp32 or bf16.  Other well-formed shapes return
 *   GDN_ERROR_NOT_SUPPORTED.
 * - Every host-checkable argument is validated before any HIP call; on an
 *   error nothing is enqueued.  No call throws or aborts.  The text of the
 *   last error on the calling thread is available from gdn_last_error().
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum gdn_status {
    GDN_SUCCESS = 0,
    GDN_ERROR_INVALID_VALUE = 1,  /* malformed argument (NULL, negative size, misaligned ...) */
    GDN_ERROR_NOT_SUPPORTED = 2,  /* well-formed shape the library has no kernel for */
    GDN_ERROR_LAUNCH = 3,         /* a HIP launch or enqueue failed */
    GDN_ERROR_OUT_OF_MEMORY = 4   /* the pool workspace could not be allocated (non-_ws forms) */
} gdn_status;

typedef enum gdn_dtype {
    GDN_DTYPE_F32 = 0,            /* q, k, v, out are fp32 */
    GDN_DTYPE_BF16 = 1            /* q, k, v, out are bf16 (out rounded to nearest even) */
} gdn_dtype;

/* Problem shape.
 * num_seqs   N >= 0 sequences.
 * num_tokens total tokens in q/k/v/out (prefill: sum of the lengths;
 *            gdn_decode_step: num_seqs, one token per sequence;
 *            gdn_decode_tokens / _slots: num_seqs * tokens_per_seq).
 * Without cu_seqlens the N sequences have equal length num_tokens / N
 * (num_tokens must be a multiple of N), stored one after another. */
typedef struct gdn_shape {
    int32_t num_seqs;
    int64_t num_tokens;
    int32_t num_qk_heads;
    int32_t num_v_heads;
    int32_t head_dim_k;
    int32_t head_dim_v;
    gdn_dtype dtype;
} gdn_shape;

/*
 * Workspace.  Every prefill entry point needs device scratch memory: per
 * 64-token chunk and value head the chunk's triangular factor and gates
 * (about 6 KB for bf16, 13 KB for fp32), and, when sequences are cut into
 * parts, per part and value head its transition, offset and start state
 * ((dk + 2 dv) * dk * 4 bytes).  Sequences are cut when there are fewer
 * (sequence, value head) pairs than compute units (every sequence, into parts
 * of about one compute unit's share), and on packed bf16 input with
 * dk = dv and up to twice as many pairs as compute units (only the sequences
 * longer than one share, so that the long ones do not leave the others' compute
 * units idle).  Each entry point comes in two forms:
 *   gdn_prefill*_ws  take a caller-owned workspace and allocate nothing;
 *   gdn_prefill*     take it from the current device's default stream-ordered
 *                    memory pool (hipMallocAsync / hipFreeAsync on `stream`,
 *                    GDN_ERROR_OUT_OF_MEMORY if that fails).  The pool's
 *                    settings are the caller's: the library changes none.
 * Both forms run the same kernels and give bit-identical results.  Apart from
 * the device address of gdn_prefill_static's scratch array, which it looks up
 * once per device, the library keeps no state between calls.
 *
 * A caller workspace is DEVICE memory, 256-byte aligned, not NULL and
 * overlapping no other argument.  It needs no initialisation; its contents are
 * undefined afterwards.  It is in use until the call's work on `stream`
 * completes, so calls that share one must be ordered (for instance, on one
 * stream).  workspace_bytes must be at least what gdn_prefill_workspace_size
 * returns for the same shape, flags and device, else GDN_ERROR_INVALID_VALUE
 * (nothing enqueued).
 */
#define GDN_WS_PACKED 1u   /* the call passes cu_seqlens                        */
#define GDN_WS_RAW 2u      /* for gdn_prefill_raw_ws                             */
#define GDN_WS_AFFINE 4u   /* for gdn_prefill_affine_ws (excludes GDN_WS_RAW)    */

/*
 * gdn_prefill_workspace_size -- bytes of workspace a prefill call with this
 * shape needs on the current device (the part length L depends on the
 * device's compute-unit count).  flags: GDN_WS_PACKED if the call passes
 * cu_seqlens, plus GDN_WS_RAW or GDN_WS_AFFINE for those entry points
 * (gdn_prefill_ws and gdn_prefill_snapshots_ws need neither).  Writes 0 when
 * num_seqs is 0.  Host-only: launches nothing and allocates nothing.
 */
gdn_status gdn_prefill_workspace_size(const gdn_shape* shape, uint32_t flags, size_t* bytes);

/*
 * gdn_prefill -- run the recurrence over whole sequences (packed varlen).
 *
 * Computes o_t for every token of every sequence and, if final_state is not
 * NULL, the state after each sequence's last token.  The chunk-wise WY / UT
 * form (chunks of 64 tokens, restarting at every sequence start) is used on
 * the GPU; the result equals the token-by-token recurrence up to rounding.
 * Decay horizon: when a sequence is cut into parts and every token of a part
 * contracts the state (g_t <= 0 and 0 <= beta_t |k_t|^2 <= 2, so that the
 * token's factor exp(g_t) (I - beta_t k_t k_t^T) has norm <= exp(g_t)), the
 * part's summary starts at the latest chunk from which the gates to the
 * part's end multiply to at most 2^-160, and the next part's start state
 * drops the earlier state's contribution (scaled by at most that factor,
 * below fp32 resolution).  Results are unchanged to rounding; a NaN or inf
 * input stays within its own part there instead of reaching later parts.
 *
 * init_state  [N, Hv, dv, dk] fp32 or NULL (zero initial state).  It may be
 *             the same buffer as final_state (each sequence's slice is read
 *             before it is written); partial overlap is not allowed.
 * cu_seqlens  DEVICE int32 [N + 1] token offsets or NULL (equal lengths).
 *             Precondition (not checked, it lives on the device):
 *             cu[0] = 0, non-decreasing, cu[N] = num_tokens.  Empty sequences
 *             are allowed: their final state equals their initial state.
 * out         [num_tokens, Hv, dv] in `dtype`.
 * final_state [N, Hv, dv, dk] fp32 or NULL.
 * Workspace from the default pool (see above).
 */
gdn_status gdn_prefill(const gdn_shape* shape, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* init_state,
                       const int32_t* cu_seqlens, void* out, float* final_state,
                       void* stream);

/* gdn_prefill_ws -- gdn_prefill on a caller-owned workspace (flags
 * GDN_WS_PACKED if cu_seqlens is given); allocates nothing. */
gdn_status gdn_prefill_ws(const gdn_shape* shape, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const float* init_state,
                          const int32_t* cu_seqlens, void* out, float* final_state,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_static -- gdn_prefill for callers that cannot allocate device
 * memory at all (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc) and have no workspace to pass: it runs on a static
 * scratch array of GDN_STATIC_SCRATCH_BYTES that the library holds on every
 * device it runs on, from the load of its code onto that device until the
 * process ends.  It calls no allocator.  Same arguments, kernels and results
 * as gdn_prefill_ws.
 *
 * A shape whose workspace (gdn_prefill_workspace_size) exceeds
 * GDN_STATIC_SCRATCH_BYTES is rejected with GDN_ERROR_NOT_SUPPORTED before
 * anything is enqueued; on a 256-CU device, at 16 value heads and d = 128 in
 * bf16, that admits one sequence of up to 8,192 tokens.
 * Every call on one device shares that device's array and leaves its contents
 * behind (the kernels need none of them): calls whose work may overlap on one
 * device, on different streams or from different threads, race on the array
 * and must be ordered by the caller.
 */
#define GDN_STATIC_SCRATCH_BYTES (64u << 20)
gdn_status gdn_prefill_static(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              const float* g, const float* beta, const float* init_state,
                              const int32_t* cu_seqlens, void* out, float* final_state, void* stream);

/*
 * gdn_prefill_affine -- the state map of each whole sequence.  Over its tokens
 * the recurrence maps any start state S to S M + B: every token's update is
 * affine in the state, so their composition is too (a property of the
 * recurrence itself, which keeps one fixed-size state per head: flozi.net,
 * "Qwen3.8-Flash-Next architecture", "Der Weg eines Tokens durch das
 * Modell", item 1).  This is the per-device half of a sequence-sharded
 * prefill: each device summarises its range of tokens, the maps are gathered
 * and composed, and each device reruns gdn_prefill on its range from the
 * composed start state.
 *
 * k, v, g, beta, cu_seqlens as for gdn_prefill (q is not needed).
 * transition  [N, Hv, dk, dk] fp32, M (the identity for an empty sequence).
 * offset      [N, Hv, dv, dk] fp32, B (the state reached from zero).
 * The two must not overlap.  Workspace from the default pool (see above).
 */
gdn_status gdn_prefill_affine(const gdn_shape* shape, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu_seqlens, float* transition, float* offset,
                              void* stream);

/* gdn_prefill_affine_ws -- gdn_prefill_affine on a caller-owned workspace
 * (flags GDN_WS_AFFINE, plus GDN_WS_PACKED if cu_seqlens is given). */
gdn_status gdn_prefill_affine_ws(const gdn_shape* shape, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* cu_seqlens, float* transition, float* offset,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_snapshots -- gdn_prefill that also writes the state at every
 * snapshot_chunks * 64 tokens of each sequence (chunk-boundary snapshots for
 * prefix reuse: a later request that shares the first s * P tokens of a
 * prompt can start from snapshot s instead of recomputing them).
 *
 * snapshot_chunks  P / 64 >= 1, where P is the snapshot interval in tokens.
 * snapshots        [slots, Hv, dv, dk] fp32, not NULL.  Snapshot s (s = 1 ..
 *                  floor(len_n / P)), the state after the first s * P tokens of
 *                  sequence n, goes to slot floor(cu[n] / P) + n + s - 1
 *                  (cu[n] = n * len without cu_seqlens).  floor(num_tokens / P)
 *                  + N slots always suffice; slots that hold no snapshot are
 *                  left as they were.  It must not overlap any other argument.
 * Everything else is as for gdn_prefill (workspace from the default pool).
 */
gdn_status gdn_prefill_snapshots(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* init_state,
                                 const int32_t* cu_seqlens, void* out, float* final_state, int32_t snapshot_chunks,
                                 float* snapshots, void* stream);

/* gdn_prefill_snapshots_ws -- gdn_prefill_snapshots on a caller-owned
 * workspace (flags as for gdn_prefill_ws); allocates nothing. */
gdn_status gdn_prefill_snapshots_ws(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const float* init_state,
                                    const int32_t* cu_seqlens, void* out, float* final_state,
                                    int32_t snapshot_chunks, float* snapshots, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * gdn_decode_step -- advance N sequences by one token each.
 *
 * Tokens = sequences: q, k [N, Hqk, dk]; v, out [N, Hv, dv]; g, beta [N, Hv].
 * state [N, Hv, dv, dk] fp32 is read and updated in place (one pass over it).
 * Needs no workspace and allocates nothing.
 */
gdn_status gdn_decode_step(const gdn_shape* shape, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state, void* out,
                           void* stream);

/*
 * gdn_decode_tokens -- advance N sequences by T tokens each in one pass over
 * the state (multi-token decode, e.g. verifying T draft tokens).  Drafting
 * several tokens at a time is what the model's multi-token-prediction module
 * is for (flozi.net, "Qwen3.8-Flash-Next architecture", the stack table, draft
 * module row); verifying them advances every GDN layer by T tokens.
 *
 * The result equals T successive gdn_decode_step calls on the sequences'
 * tokens in order (the same recurrence as gdn_prefill over N sequences of T
 * tokens), but the state is read and written once instead of T times.
 *
 * tokens_per_seq  T >= 1; shape->num_tokens must equal num_seqs * T.
 * q, k            [N * T, Hqk, dk], token t of sequence n at row n * T + t.
 * v, out          [N * T, Hv, dv];   g, beta [N * T, Hv] fp32.
 * state           [N, Hv, dv, dk] fp32, read, then overwritten with the state
 *                 after each sequence's last token.
 * token_states    [N, T, Hv, dv, dk] fp32 or NULL.  If given, receives the
 *                 state after every token (token_states[n][t] is the state
 *                 after token t of sequence n), so that a caller that accepts
 *                 only the first m tokens can copy token_states[n][m - 1] back
 *                 into state.  It must not overlap state.
 * Needs no workspace and allocates nothing.
 */
gdn_status gdn_decode_tokens(const gdn_shape* shape, int32_t tokens_per_seq, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, float* state, void* out,
                             float* token_states, void* stream);

/*
 * gdn_decode_slots -- gdn_decode_tokens over a pool of states.
 *
 * Serving engines keep the states of all live requests in one pool and pass,
 * for every batch, which pool entry each sequence uses.  Sequence n reads and
 * updates state_pool[slot_idx[n]] instead of state[n].
 *
 * state_pool   [pool_slots, Hv, dv, dk] fp32.
 * slot_idx     DEVICE int32 [N].  Entries must be distinct, except that a
 *              negative entry marks a padding row: that sequence is skipped
 *              (no state touched, its out rows and token_states left as they
 *              were).  Entries >= pool_slots are skipped the same way.
 * token_states [N, T, Hv, dv, dk] fp32 or NULL, indexed by sequence (not by
 *              slot).  It must not overlap the pool.
 * The other arguments and the result are as for gdn_decode_tokens; T = 1
 * gives a single decode step over the pool.
 */
gdn_status gdn_decode_slots(const gdn_shape* shape, int32_t tokens_per_seq, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, float* state_pool,
                            int64_t pool_slots, const int32_t* slot_idx, void* out, float* token_states,
                            void* stream);

/*
 * gdn_prefill_raw, gdn_decode_tokens_raw -- the same calls from the layer's
 * raw projections, with the steps that precede the recurrence fused into the
 * kernels (no extra pass over HBM).  q and k are taken unnormalised and g,
 * beta are replaced by logits a_gate, b_beta [tokens, Hv] fp32; per (token,
 * head) the library uses
 *     q / sqrt(|q|^2 + 1e-6),  k / sqrt(|k|^2 + 1e-6),
 *     g = -softplus(a_gate),   beta = sigmoid(b_beta).
 * (The pages name the layer -- a fixed-size recurrent state per head,
 * flozi.net, "Qwen3.8-Flash-Next architecture", "Der Weg eines Tokens durch
 * das Modell", item 1 -- but print none of these formulas; they are the usual
 * forms and give the input distributions the rest of this library is
 * measured on.)  All other arguments, layouts and rules are those of
 * gdn_prefill and gdn_decode_tokens; gdn_prefill_raw's workspace is larger by
 * (num_tokens / 64 + N) * Hv * 256 bytes (1 / |k| per token): size it with
 * GDN_WS_RAW.
 */
gdn_status gdn_prefill_raw(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* a_gate,
                           const float* b_beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                           float* final_state, void* stream);
gdn_status gdn_decode_tokens_raw(const gdn_shape* shape, int32_t tokens_per_seq, const void* q, const void* k,
                                 const void* v, const float* a_gate, const float* b_beta, float* state, void* out,
                                 float* token_states, void* stream);
/* gdn_prefill_raw_ws -- gdn_prefill_raw on a caller-owned workspace (flags
 * GDN_WS_RAW, plus GDN_WS_PACKED if cu_seqlens is given); allocates nothing. */
gdn_status gdn_prefill_raw_ws(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              const float* a_gate, const float* b_beta, const float* init_state,
                              const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Static English text for a status code (never NULL). */
const char* gdn_status_string(gdn_status status);

/* Details of the last non-success status returned on this thread ("" if none). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
