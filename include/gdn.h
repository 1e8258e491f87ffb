/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet layer library, libgdn.so.
 *
 * The layer is the gated delta rule.  No page prints the recurrence; the
 * definition in force is the layer's specification: for every sequence and
 * value head, with state S (d_v x d_k), alpha_t = exp(g_t),
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
 *
 * The pages this library follows use it as the linear-attention layer of a
 * hybrid model: the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page, section
 * 2 ("GDN prefill"), runs the prefill chunkwise with chunk length 64 in three
 * steps (intra-chunk preparation, inter-chunk state recurrence, output), the
 * entry point gdn_chunk_fwd below; its section 1 describes the speculative
 * verify step of 1 + K query tokens per request, and the "Qwen3.8-27B on one
 * RTX 3090" page keeps a fixed-size recurrent state per request plus one
 * state snapshot per speculative token (section on the 131,072-token limit),
 * the entry point gdn_recurrent_step below.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *    by the caller.  The library allocates nothing, keeps no device state and
 *    is re-entrant; calls are asynchronous on `stream` (a hipStream_t, NULL =
 *    the default stream).  A call enqueues only kernel launches on `stream`
 *    (no allocation, copy, memset or synchronisation), so it may be captured
 *    into a HIP graph and replayed; every replay reads the buffers the
 *    captured call named, with their contents at replay time.
 *  - Layouts are dense, row-major, token-major:
 *      q, k : [T, H_qk, d_k]  bfloat16      v : [T, H_v, d_v]  bfloat16
 *      g    : [T, H_v] float32 natural-log decay (alpha = exp(g), g <= 0)
 *      beta : [T, H_v] float32
 *      out  : [T, H_v, d_v] float32
 *      state: [N, H_v, d_k, d_v] float32, element [a][b] = S[b][a] (d_v contiguous)
 *    Value head h reads q/k head h / (H_v / H_qk) (contiguous groups).
 *  - Every pointer must be 16-byte aligned (GDN_ERR_MISALIGNED otherwise).
 *  - Supported sizes: d_k = d_v = 128; H_v a positive multiple of H_qk.
 *    Other head dims return GDN_ERR_NOT_SUPPORTED.
 *  - Validation reads only host values (no device reads, no synchronisation).
 *    Device-content preconditions are documented, and checked only under
 *    GDN_DEBUG_CHECKS (see gdn_check_chunk_inputs_host): cu_seqlens is
 *    nondecreasing with cu_seqlens[0] = 0 and cu_seqlens[N] = T; g <= 0; all
 *    inputs finite and, since matrix-core operands are fp16, |q|, |k|, |v|
 *    below 65504 and states and outputs well inside fp16 range.
 *  - Errors: a gdn_status is returned, no exception crosses the ABI, nothing
 *    is printed, nothing aborts.  gdn_get_last_error() gives the detail of
 *    the calling thread's last failure.  There is no fallback path: a
 *    failed launch returns GDN_ERR_LAUNCH with the HIP error text.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_SUCCESS = 0,
    GDN_ERR_INVALID_VALUE = 1, /* null pointer, negative or inconsistent size */
    GDN_ERR_NOT_SUPPORTED = 2, /* head dims other than 128 */
    GDN_ERR_MISALIGNED = 3,    /* a pointer is not 16-byte aligned */
    GDN_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
    GDN_ERR_LAUNCH = 5         /* HIP reported an error at launch */
} gdn_status;

/* Host-side problem sizes.  n_seqs and total_tokens are host copies of
 * what cu_seqlens holds on the device (N and cu_seqlens[N]).  Limits (so
 * that every launch fits the dispatch grid; GDN_ERR_INVALID_VALUE beyond
 * them): n_seqs * n_heads_v <= 2^21, n_heads_v <= 65535, and
 * n_seqs + total_tokens / 64 + 1 <= 2^24 (about 10^9 tokens). */
typedef struct {
    int32_t n_seqs;
    int64_t total_tokens;
    int32_t n_heads_qk;
    int32_t n_heads_v;
    int32_t d_k;
    int32_t d_v;
} gdn_dims;

/*
 * Workspace bytes that gdn_chunk_fwd, gdn_chunk_fwd_stages and
 * gdn_chunk_fwd_snapshots accept for `dims` (device memory the caller
 * allocates; contents undefined before and after a call).  It holds the
 * intra-chunk products of the chunkwise form that the preparation kernel
 * hands to the recurrence (Tm diag(beta), the output's intra-chunk matrix,
 * the decay vectors, and fp16 K^T and Q per q/k head), one 64-token chunk
 * slot per chunk: at most N + T/64 + 1 slots, about 28.5 KB per slot and
 * value head at two value heads per q/k head.
 */
gdn_status gdn_chunk_fwd_workspace_size(const gdn_dims* dims, size_t* bytes);

/*
 * The smallest workspace gdn_chunk_fwd and gdn_chunk_fwd_noalloc accept for
 * `dims` (gdn_chunk_fwd_workspace_size is always enough, and is what the
 * other chunked entry points need).  It is smaller only for one sequence
 * whose intermediates exceed 160 MiB, which gdn_chunk_fwd runs range by
 * range: then it holds one range's intermediates (64 chunk slots at 32
 * value / 16 q/k heads) and the fp32 state carried between ranges, e.g.
 * 62 MB instead of 1.87 GB for 131072 tokens at 32 value / 16 q/k heads.
 */
gdn_status gdn_chunk_fwd_min_workspace_size(const gdn_dims* dims, size_t* bytes);

/*
 * Chunked prefill (chunk length 64) over a packed batch of N sequences
 * (tokens cu_seqlens[n] .. cu_seqlens[n+1]-1).  Follows the three steps
 * of the "2080 Ti runs Qwen3.8-27B: a vLLM plugin" page, section 2, in two
 * kernels:
 *   gdn_chunk_prep  -- decay cumsum, masked K K^T, Tm = (I + A)^{-1} (stored
 *                      as Tm diag(beta)), and the output's intra-chunk matrix
 *                      P = M o Q K^T;
 *   gdn_chunk_state -- W and U formed on chip from Tm diag(beta), the
 *                      inter-chunk recurrence with the state held in
 *                      matrix-core accumulators and the next chunks
 *                      prefetched, and the output
 *                      O = diag(e^G) Q S_chunk + P U'.
 *  q, k, v       bf16 device tensors, layouts above.
 *  g, beta       float32 [T, H_v].
 *  cu_seqlens    int32 [N + 1], device.
 *  initial_state float32 [N, H_v, d_k, d_v] or NULL (zeros).
 *  out           float32 [T, H_v, d_v], written for every token.
 *  final_state   float32 [N, H_v, d_k, d_v] or NULL (not written); may alias
 *                initial_state (in-place state update).
 *  workspace     device buffer of at least gdn_chunk_fwd_min_workspace_size
 *                bytes (gdn_chunk_fwd_workspace_size is always enough).
 * Empty sequences are allowed (their final state equals the initial state).
 * A batch of one sequence whose intermediates exceed 160 MiB runs range by
 * range: prep and the recurrence alternate over ranges of chunks (as many
 * as one full round of prep workgroups covers), the state handed from range
 * to range in fp32 through the workspace, so that each range's
 * intermediates stay in the last-level cache; the workspace then needs room
 * for one range only.  The results are bit for bit those of the single
 * pass (gdn_chunk_fwd_stages with mask 1, then 2).
 */
gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const int32_t* cu_seqlens,
                         const float* initial_state,
                         float* out,
                         float* final_state,
                         const gdn_dims* dims,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Number of chunk-state slots of a batch: n_seqs + floor(total_tokens / 64)
 * + 1, the first dimension of gdn_chunk_fwd_snapshots' chunk_states.  Host
 * only.
 */
gdn_status gdn_chunk_state_slots(const gdn_dims* dims, int64_t* n_slots);

/*
 * gdn_chunk_fwd that also exports the state at every chunk boundary, for a
 * prefix cache that keeps the recurrent state (the "Qwen3.8-27B on one RTX
 * 3090" page, section "Pourquoi cela convient aux agents harness": the prefix
 * cache of the hybrid model stores the DeltaNet state as well as the
 * attention KV).
 *  chunk_states  float32 [n_slots, H_v, d_k, d_v], n_slots from
 *                gdn_chunk_state_slots.  The state after chunk c of sequence
 *                n, i.e. after its first min(64 (c + 1), len_n) tokens, goes
 *                to slot n + floor(cu_seqlens[n] / 64) + c for c = 0 ..
 *                ceil(len_n / 64) - 1 (the last one equals the final state).
 *                Slots of different sequences never overlap; slots no chunk
 *                maps to are not written.  Required (non-NULL) when N > 0.
 * Other arguments, results and errors as gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_snapshots(const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const int32_t* cu_seqlens,
                                   const float* initial_state,
                                   float* out,
                                   float* final_state,
                                   float* chunk_states,
                                   const gdn_dims* dims,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Workspace bytes of gdn_chunk_fwd_segmented: gdn_chunk_fwd's plus, per
 * segment slot and value head, the affine map (2 x 64 KiB) and the incoming
 * state (64 KiB) of a segment; n_seqs + (n_seqs + floor(T / 64) + 1) /
 * segment_chunks + 1 segment slots.  Host only.
 */
gdn_status gdn_chunk_fwd_segmented_workspace_size(const gdn_dims* dims, int32_t segment_chunks, size_t* bytes);

/*
 * gdn_chunk_fwd with the inter-chunk recurrence parallel over segments of
 * segment_chunks chunks (a chunk-parallel affine scan; the pages run the
 * recurrence serially, "2080 Ti runs Qwen3.8-27B: a vLLM plugin", section 2).
 * Over a segment the recurrence is affine in its incoming state, H_end = Phi
 * H_start + R, and such maps compose associatively.  Three launches after
 * prep: every segment but the last of each sequence computes (Phi, R) from
 * its own chunks; an fp32 scan over segments chains them into each segment's
 * incoming state; every segment then runs the state recurrence with the
 * output from its incoming state.  About three times the recurrence's work,
 * for parallelism when one long sequence gives fewer workgroups than CUs.
 * Results agree with gdn_chunk_fwd to the same tolerance (not bitwise).
 *  segment_chunks  >= 1; GDN_ERR_INVALID_VALUE otherwise.
 *  workspace       at least gdn_chunk_fwd_segmented_workspace_size bytes.
 * Other arguments, results and errors as gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   const int32_t* cu_seqlens,
                                   const float* initial_state,
                                   float* out,
                                   float* final_state,
                                   int32_t segment_chunks,
                                   const gdn_dims* dims,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * Runs only the selected stages of gdn_chunk_fwd, for callers that time or
 * schedule the stages one by one.  stage_mask bits: 1 = gdn_chunk_prep,
 * 2 = gdn_chunk_state with the output (3 = gdn_chunk_fwd).  The second stage
 * reads what the first left in the same workspace; run them in order, on the
 * same inputs and workspace, or the results are undefined (memory accesses
 * stay in bounds regardless, since every index comes from cu_seqlens and the
 * launch grid, never from workspace contents).  Arguments as gdn_chunk_fwd;
 * a mask outside 1..3 returns GDN_ERR_INVALID_VALUE.
 */
gdn_status gdn_chunk_fwd_stages(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const int32_t* cu_seqlens,
                                const float* initial_state,
                                float* out,
                                float* final_state,
                                const gdn_dims* dims,
                                void* workspace, size_t workspace_bytes,
                                int stage_mask,
                                void* stream);

/*
 * Per-token recurrent update for decode (tokens_per_request = 1) and
 * speculative verify (1 + K tokens per request).  Requests are packed
 * request-major: token i of request r is row r * tokens_per_request + i of
 * q, k, v, g, beta and out.  dims->n_seqs must equal n_requests and
 * dims->total_tokens must equal n_requests * tokens_per_request.
 *  state_in            float32 [R, H_v, d_k, d_v]; read only.
 *  state_out           float32 [R, H_v, d_k, d_v], the state after the last
 *                      token; may alias state_in; may be NULL only when
 *                      save_intermediate_states is nonzero.
 *  out                 float32 [R * n, H_v, d_v].
 *  intermediate_states float32 [R, n, H_v, d_k, d_v]: slot [r][i] is the
 *                      state right after token i of request r, the rollback
 *                      point if the verifier accepts exactly i + 1 tokens.
 *                      Required iff save_intermediate_states is nonzero.
 */
gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              int32_t n_requests, int32_t tokens_per_request,
                              const float* state_in,
                              float* state_out,
                              float* out,
                              float* intermediate_states,
                              int save_intermediate_states,
                              const gdn_dims* dims,
                              void* stream);

/* Storage type of the recurrent states in a slot pool. */
typedef enum {
    GDN_STATE_F32 = 0,
    GDN_STATE_F16 = 1
} gdn_state_dtype;

/*
 * Per-token recurrent update over a pool of state slots: speculative verify
 * with a variable number of tokens per request, rollback and commit by slot
 * index, and fp32 or fp16 state storage.
 *
 * The "Qwen3.8-27B on one RTX 3090" page keeps a fixed-size state per request
 * in fp16 (section "Exploiter l'architecture hybride") and eight speculative
 * state slots per request (section on the 131,072-token limit); the "2080 Ti
 * runs Qwen3.8-27B: a vLLM plugin" page verifies 1 + K query tokens per
 * request (section "vLLM on old cards").  The arithmetic is the update of
 * gdn_recurrent_step, in fp32 registers, whatever the storage type.
 *
 *  cu_tokens     int32 [R + 1], device: request r owns token rows
 *                cu_tokens[r] .. cu_tokens[r+1] - 1 of q, k, v, g, beta and
 *                out; between 0 and max_tokens rows each.
 *  state_pool    [pool_slots, H_v, d_k, d_v], float32 or float16
 *                (state_dtype), d_v contiguous; read and written in place.
 *  slot_table    int32 [R, max_tokens + 1], device.  Column c > 0 of row r
 *                names the slot that receives the state right after token
 *                c - 1 of request r (negative: not stored).  The incoming
 *                state is read from column num_accepted[r] (column 0 when
 *                num_accepted is NULL).  So a serving loop that keeps one row
 *                per request passes the previous call's accepted-token count
 *                to roll back to the last accepted state with no copy; column
 *                0 holds the committed state of a fresh request.
 *  num_accepted  int32 [R], device, or NULL.
 *  out           float32 [T, H_v, d_v], T = dims->total_tokens.
 *  dims          n_seqs = R; total_tokens = T rows of the token arrays.
 *
 * A request may name its own incoming slot among its write slots (the update
 * holds the whole state before it stores any snapshot); slots named by two
 * different requests race.  Device-content checks, done before any access
 * they guard: a request whose token range is not inside [0, T) or holds more
 * than max_tokens rows is skipped (nothing written); a request whose incoming
 * column or slot, or any write slot, is outside the table or pool gets NaN
 * outputs and no state read or written.  Host-side errors as for
 * gdn_recurrent_step; state_dtype outside the enum is GDN_ERR_INVALID_VALUE.
 */
gdn_status gdn_recurrent_step_slots(const void* q, const void* k, const void* v,
                                    const float* g, const float* beta,
                                    const int32_t* cu_tokens,
                                    int32_t n_requests, int32_t max_tokens,
                                    void* state_pool, int32_t state_dtype, int64_t pool_slots,
                                    const int32_t* slot_table,
                                    const int32_t* num_accepted,
                                    float* out,
                                    const gdn_dims* dims,
                                    void* stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The workspace is a fixed array of GDN_NOALLOC_SCRATCH_BYTES in the
 * library's device code, one per GPU, held until the process ends; the call
 * itself allocates nothing (no hipMalloc or hipFree, no allocating library
 * routine).  Batches whose gdn_chunk_fwd_min_workspace_size exceeds it
 * return GDN_ERR_WORKSPACE (128 MiB: batches up to about 9,100 tokens at 32
 * value / 16 q-k heads, 4000 tokens using 57 MiB, and one sequence of any
 * length, which runs range by range in 62 MB).  The first call on a device looks up the
 * array's address there.  Every call on one GPU uses that GPU's single copy:
 * calls that overlap on one GPU (two streams, two threads) race and give
 * undefined results; serialise them.  Arguments, results and other errors as
 * gdn_chunk_fwd.
 */
#define GDN_NOALLOC_SCRATCH_BYTES (128u << 20)
gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const int32_t* cu_seqlens,
                                 const float* initial_state,
                                 float* out,
                                 float* final_state,
                                 const gdn_dims* dims,
                                 void* stream);

/*
 * Device-content preconditions, checked on HOST copies of the inputs: a
 * debugging aid, and what every entry point runs on copies of its device
 * inputs when the environment variable GDN_DEBUG_CHECKS is set (to anything
 * but "" or "0"; the call then synchronises its stream, allocates host
 * memory and is not fit for timing or graph capture).  No page states these
 * conditions; they are what the arithmetic above needs: the decay
 * alpha = exp(g) must lie in (0, 1], the chunk boundaries must be ordered,
 * and fp16 matrix-core operands cannot hold magnitudes above 65504.
 *
 * gdn_check_chunk_inputs_host (the prefill entry points): cu_seqlens
 * nondecreasing with cu_seqlens[0] = 0 and cu_seqlens[N] = total_tokens;
 * g finite and <= 0; beta finite; q, k, v (bf16 bits) finite with
 * |x| <= 65504; initial_state (NULL allowed) finite with |x| <= 65504.
 * gdn_check_step_inputs_host (the recurrent steps): the same token checks,
 * and state_in ([n_states, H_v, d_k, d_v], NULL allowed) finite.
 * Every pointer is a host pointer with the layout of the corresponding
 * device argument.  The first violation returns GDN_ERR_INVALID_VALUE and
 * names the offending element in gdn_get_last_error(); invalid dims return
 * what the entry points return for them.
 */
gdn_status gdn_check_chunk_inputs_host(const void* q, const void* k, const void* v,
                                       const float* g, const float* beta,
                                       const int32_t* cu_seqlens,
                                       const float* initial_state,
                                       const gdn_dims* dims);
gdn_status gdn_check_step_inputs_host(const void* q, const void* k, const void* v,
                                      const float* g, const float* beta,
                                      const float* state_in, int64_t n_states,
                                      const gdn_dims* dims);

/* Static text for a status code. */
const char* gdn_status_string(gdn_status s);

/* Detail of the calling thread's last failing call ("" if none). */
const char* gdn_get_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
