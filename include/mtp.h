/*
 * mtp.h — C ABI of the MI355X (gfx950) Multi-Token-Prediction draft / verify / rollback path.
 *
 * One MTP draft step (speculators user guide, "MTP (Multi-Token Prediction)",
 * How It Works > Architecture): the verifier's hidden state and the shared token
 * embedding are RMS-normalised separately, concatenated, projected 2H -> H, run
 * through one standard decoder layer (attention over the MTP layer's own
 * single-layer KV cache + SwiGLU MLP), and a final norm plus the shared lm_head
 * gives the draft token by argmax. The layer output feeds the next step, K times.
 * Greedy verification (OpenVINO GenAI docs, "Speculative Decoding", Overview)
 * accepts the longest prefix of drafts that the target's own argmax tokens
 * reproduce and takes the target's token at the first mismatch as the bonus.
 * The MTP cache is then cut back to the committed prefix (devnotes, "How
 * OpenVINO MTP Speculative Decoding Works Internally", "Stateful execution").
 *
 * Conventions
 *  - Every pointer argument that names a tensor is DEVICE memory owned by the
 *    caller. The library keeps no reference past a call, except the weight
 *    pointers, which must stay valid and unchanged for the handle's lifetime.
 *  - Matrices are row-major [out, in]; y = W x. Weights, gains, embedding,
 *    hidden states and the KV cache use the configuration's dtype
 *    (MTP_F32: float, MTP_BF16: bfloat16 bit patterns). Accumulation is fp32.
 *  - `stream` is a hipStream_t passed as void*. NULL means the default stream.
 *    The three hot calls only enqueue work on it: no host synchronisation and
 *    no device-to-host copy. Calls on one handle must be ordered on one stream.
 *  - Argument problems that the host can see are reported synchronously, before
 *    anything is enqueued. Conditions only the device can see (a token id
 *    outside [0, vocab), a cache that would overflow its capacity, an accepted
 *    length outside [0, K]) set a device error word and the kernels stay in
 *    bounds (clamping the offending value); mtp_get_error() reports it.
 *  - No C++ exception crosses this interface.
 */
#ifndef MTP_H
#define MTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MTP_OK = 0,
  MTP_ERR_INVALID_ARG = 1, /* null pointer, null handle, bad enum value            */
  MTP_ERR_SHAPE = 2,       /* inconsistent or non-positive dimensions               */
  MTP_ERR_DTYPE = 3,       /* unknown dtype                                         */
  MTP_ERR_CAPACITY = 4,    /* B > max_batch, K > max_k, workspace or cache too small */
  MTP_ERR_UNSUPPORTED = 5, /* a shape the kernels do not handle (see mtp_create)     */
  MTP_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed             */
  MTP_ERR_DEVICE = 7       /* the device error word was set (see mtp_get_error)      */
} mtp_status;

typedef enum { MTP_F32 = 0, MTP_BF16 = 1 } mtp_dtype;

/* Device error-word bits reported by mtp_get_error(). */
#define MTP_DEVERR_TOKEN 1u    /* a token id (last_tokens or a draft) was outside [0, vocab) */
#define MTP_DEVERR_CAPACITY 2u /* len + K exceeded the cache capacity                   */
#define MTP_DEVERR_ACCEPT 4u   /* an accepted_len entry was outside [0, K]              */
#define MTP_DEVERR_COUNT 8u    /* a prefill row count or per-sequence draft length was out of range */

/* Shape of the MTP head. rope_theta: RoPE base; rms_eps: RMSNorm epsilon. */
typedef struct {
  int32_t hidden;     /* H                                            */
  int32_t n_q_heads;  /* query heads                                  */
  int32_t n_kv_heads; /* key/value heads (n_q_heads % n_kv_heads == 0) */
  int32_t head_dim;   /* d: 64 or 128                                  */
  int32_t ffn;        /* SwiGLU inner size F                          */
  int32_t vocab;      /* V, shared with the verifier                  */
  float rope_theta;
  float rms_eps;
  int32_t dtype;      /* mtp_dtype                                    */
} mtp_config;

/*
 * Weights (device pointers, configuration dtype, row-major [out, in]):
 *   g_h, g_e      [H]        gains of the two separate input RMSNorms (hidden, embedding)
 *   w_eh          [H, 2H]    projection of concat(norm(h), norm(e)); columns 0..H-1 take norm(h)
 *   g_attn        [H]        pre-attention RMSNorm gain
 *   w_q           [n_q*d, H], w_k, w_v [n_kv*d, H], w_o [H, n_q*d]
 *   g_mlp         [H]        pre-MLP RMSNorm gain
 *   w_gate, w_up  [F, H],    w_down [H, F]
 *   g_final       [H]        final RMSNorm gain (feeds the lm_head only)
 *   embed         [V, H]     the verifier's token embedding (read-only, shared)
 *   lm_head       [V, H]     the verifier's output projection (read-only, shared)
 */
typedef struct {
  const void *g_h, *g_e, *w_eh, *g_attn, *w_q, *w_k, *w_v, *w_o, *g_mlp, *w_gate, *w_up, *w_down,
      *g_final, *embed, *lm_head;
} mtp_weights;

/*
 * The MTP layer's own single-layer cache (devnotes page, "KV cache").
 *   k, v  [batch, n_kv, capacity, d] configuration dtype; keys are stored after RoPE.
 *   len   [batch] int32 device: valid slots per sequence (slots 0..len-1 are attended).
 *   pos   [batch] int32 device: RoPE position of the hidden state handed to the next draft.
 */
typedef struct {
  void *k, *v;
  int32_t *len, *pos;
  int32_t batch, capacity;
} mtp_kv;

typedef struct mtp_handle mtp_handle;

/* Bytes of device workspace a handle needs for up to max_batch sequences, up to
 * max_k steps per call and caches of up to max_capacity slots. Host only. For bf16
 * configurations with max_batch >= 3 this includes a copy of the eh_proj, attention,
 * MLP and lm_head matrices laid out for the matrix-core kernels (about the size of those
 * weights: 1.7 GB for a Qwen3-8B-shaped head). */
mtp_status mtp_workspace_size(const mtp_config* cfg, int32_t max_batch, int32_t max_k,
                              int32_t max_capacity, size_t* bytes);

/* Create a handle. `workspace` is caller-owned device memory of at least
 * mtp_workspace_size() bytes, 256-byte aligned, used only by this handle; it is
 * zeroed here (synchronously), and for bf16 configurations with max_batch >= 3 it receives
 * the re-laid-out copy of the weights: later changes to the weights are not seen by batches
 * of 3 or more sequences until mtp_refresh_weights (or use mtp_create_ex with
 * MTP_CREATE_NO_PACKED_COPY). Supported shapes: head_dim 64 or 128,
 * n_q_heads / n_kv_heads <= 8, hidden and ffn multiples of 8, max_k <= 100,
 * max_capacity <= 262144 (256 attention splits of up to 1024 slots).
 * On success *out receives the handle; on failure *out is NULL. */
mtp_status mtp_create(const mtp_config* cfg, const mtp_weights* w, int32_t max_batch,
                      int32_t max_k, int32_t max_capacity, void* workspace, size_t workspace_bytes,
                      mtp_handle** out);

/*
 * Flags of mtp_workspace_size_ex / mtp_create_ex (0 gives mtp_workspace_size / mtp_create).
 *
 * MTP_CREATE_NO_PACKED_COPY: keep no re-laid-out copy of the weights. The MTP head then
 * reads the verifier's lm_head and embedding, and its own matrices, only where the caller
 * keeps them (devnotes "How OpenVINO MTP Speculative Decoding Works Internally", "Shared
 * embeddings reduce duplication"; speculators "MTP (Multi-Token Prediction)", How It Works >
 * Training Process: embed_tokens and lm_head are shared with the verifier). The workspace
 * shrinks by mtp_info.packed_weight_bytes of the default handle (1.7 GB for a
 * Qwen3-8B-shaped head); batches of 3 or more sequences take the matrix-core kernels on the
 * row-major weights instead, which are slower (the lm_head at 32 sequences by about 15%).
 * Later changes to the weights are then seen by every call without mtp_refresh_weights.
 * Unknown flag bits give MTP_ERR_INVALID_ARG.
 */
#define MTP_CREATE_NO_PACKED_COPY 1u

mtp_status mtp_workspace_size_ex(const mtp_config* cfg, int32_t max_batch, int32_t max_k,
                                 int32_t max_capacity, uint32_t flags, size_t* bytes);
mtp_status mtp_create_ex(const mtp_config* cfg, const mtp_weights* w, int32_t max_batch,
                         int32_t max_k, int32_t max_capacity, uint32_t flags, void* workspace,
                         size_t workspace_bytes, mtp_handle** out);

/*
 * Rebuild the handle's re-laid-out weight copy from the weights given at creation, after
 * the caller changed their values in place (devnotes "How OpenVINO MTP Speculative Decoding
 * Works Internally", "Shared embeddings reduce duplication": the lm_head and embedding are
 * the verifier's own tensors, so the verifier may update them). Enqueued on `stream` (null:
 * the default stream); work on other streams that uses the handle must be ordered after it
 * by the caller, and the weights must not change while it runs. A handle without the copy
 * (mtp_info.packed_weight_bytes == 0) reads the weights directly: then this enqueues
 * nothing and returns MTP_OK. Errors: MTP_ERR_INVALID_ARG (null handle), MTP_ERR_HIP.
 */
mtp_status mtp_refresh_weights(mtp_handle* h, void* stream);

/*
 * K recursive draft steps for B sequences (speculators page, Architecture;
 * forceinjection "MTP 深度解析", 4.4: each step consumes the token drafted before it).
 *   hidden       [B, H] config dtype: verifier hidden state at position pos[b]
 *   last_tokens  [B] int32: the latest committed token (input of step 1)
 *   kv           cache; step k (1-based) writes slot len[b]+k-1 at RoPE position pos[b]+k-1
 *                and attends over slots 0..len[b]+k-1. On return len and pos are advanced by K.
 *   draft_tokens [B, K] int32 output.
 * 0 <= K <= max_k (K = 0 enqueues nothing), 1 <= B <= min(max_batch, kv->batch),
 * kv->capacity <= max_capacity. Must be followed by exactly one mtp_kv_rollback with the same K.
 */
mtp_status mtp_draft(mtp_handle* h, const void* hidden, const int32_t* last_tokens, mtp_kv* kv,
                     int32_t B, int32_t K, int32_t* draft_tokens, void* stream);

/*
 * Same kernels as mtp_draft, with diagnostic outputs (any may be NULL):
 *   hidden_out   [K, B, H] fp32: each step's layer output h^(k) (before the final norm)
 *   top2_out     [K, B, 2] fp32: the largest logit of each step (the drafted token's) and
 *                the largest among the other vocabulary rows, i.e. the margin by which the
 *                greedy choice won (0 when two rows tie). The second value comes from a
 *                second pass of the same fused lm_head argmax kernel with the drafted token
 *                left out, so asking for it doubles the lm_head traffic of the call.
 *                Near-ties matter because greedy drafts that differ only in rounding order
 *                may pick different tokens where the top two logits are this close
 *                (OpenVINO GenAI "Speculative Decoding", Overview).
 *   logits_out   [K, B, V] fp32: every logit of each step
 */
mtp_status mtp_draft_debug(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                           mtp_kv* kv, int32_t B, int32_t K, int32_t* draft_tokens,
                           float* hidden_out, float* top2_out, float* logits_out,
                           void* stream);

/*
 * Greedy verification (OpenVINO GenAI "Speculative Decoding", Overview).
 *   target_logits [B, K+1, vocab] fp32: row j scores the token after input j of
 *                 [last_token, d_1 .. d_K].
 *   draft_tokens  [B, K] int32 (ignored when K = 0)
 *   accepted_len  [B] int32 out: a = largest n <= K with d_i == argmax(row i-1) for all i <= n
 *   next_token    [B] int32 out: argmax(row a) — the bonus token. Ties take the lowest index.
 * Tokens per iteration are a + 1 ("Measuring Effectiveness" on the same page).
 */
mtp_status mtp_verify(mtp_handle* h, const float* target_logits, const int32_t* draft_tokens,
                      int32_t B, int32_t K, int32_t* accepted_len, int32_t* next_token,
                      void* stream);

/*
 * Cut the MTP cache back to the committed prefix after a K-step draft (devnotes, "How
 * OpenVINO MTP Speculative Decoding Works Internally", "Stateful execution": the MTP
 * layer's cache follows the committed sequence; OpenVINO GenAI "Speculative Decoding",
 * "How Tree Drafting Works": after verification the caches are advanced to the accepted
 * prefix only):
 *   len[b] += min(a+1, K) - K,  pos[b] += a + 1 - K,  a = accepted_len[b] (device).
 * Slot k was computed from the token committed iff k <= a+1; no KV data moves.
 * K = 0 advances pos by 1 (the bonus token) and leaves len. Errors: host checks as
 * mtp_draft; an accepted length outside [0, K] sets MTP_DEVERR_ACCEPT and is clamped.
 */
mtp_status mtp_kv_rollback(mtp_handle* h, mtp_kv* kv, const int32_t* accepted_len, int32_t B,
                           int32_t K, void* stream);

/*
 * Speculative length per sequence (OpenVINO GenAI "Speculative Decoding", Backend
 * Differences: the draft length follows each request's recent acceptance; forceinjection
 * "MTP 深度解析", 7.3: depth adapted to the live acceptance rate). These are mtp_draft,
 * mtp_verify and mtp_kv_rollback with sequence b running k_seq[b] (0 <= k_seq[b] <= K_max)
 * steps instead of K; the batch still runs K_max steps in lock step and the steps of a
 * sequence past its own length are masked: they read and write no cache slot, need no
 * capacity, and leave unspecified (valid) token ids in draft_tokens[b, k_seq[b]..K_max-1].
 *   k_seq [B] device int32, the same array for the draft, its verification and its rollback
 *   mtp_draft_seqk:   len[b], pos[b] advance by k_seq[b]; slots len..len+k_seq[b]-1 written
 *   mtp_verify_seqk:  target_logits [B, K_max+1, V]; only rows 0..k_seq[b] of sequence b are
 *                     read; accepted_len[b] in [0, k_seq[b]], next_token[b] = argmax of row
 *                     accepted_len[b]
 *   mtp_kv_rollback_seqk: as mtp_kv_rollback with K = k_seq[b] per sequence
 * Errors: as the uniform calls (K_max takes K's limits); a k_seq entry outside [0, K_max]
 * sets MTP_DEVERR_COUNT in the draft and is clamped everywhere.
 */
mtp_status mtp_draft_seqk(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                          mtp_kv* kv, const int32_t* k_seq, int32_t B, int32_t K_max,
                          int32_t* draft_tokens, void* stream);
mtp_status mtp_verify_seqk(mtp_handle* h, const float* target_logits, const int32_t* draft_tokens,
                           const int32_t* k_seq, int32_t B, int32_t K_max, int32_t* accepted_len,
                           int32_t* next_token, void* stream);
mtp_status mtp_kv_rollback_seqk(mtp_handle* h, mtp_kv* kv, const int32_t* accepted_len,
                                const int32_t* k_seq, int32_t B, int32_t K_max, void* stream);

/*
 * Greedy verification from the target's hidden states instead of its logits
 * (OpenVINO GenAI "Speculative Decoding", Overview; speculators "MTP (Multi-Token
 * Prediction)", Architecture: the LM head is shared with the verifier). For every
 * sequence b and verified input j (0..K) the target's token is
 *   argmax_v (lm_head . RMSNorm(target_hidden[b, j]; target_norm))_v, lowest index on ties,
 * computed by the fused norm + lm_head + argmax kernels without writing logits; drafts are
 * then accepted as in mtp_verify.
 *   target_hidden [B, K+1, hidden] config dtype, 16-byte aligned: the target's last-layer
 *                 outputs before its final norm at inputs [last_token, d_1 .. d_K]
 *   target_norm   [hidden] config dtype, 16-byte aligned: the target's final-norm gain
 *   draft_tokens, accepted_len, next_token: as mtp_verify.
 * Rows are processed in groups of up to 128 for bf16 heads (hidden <= 8192), else of up to 64
 * (each group streams the lm_head once; groups of more than 64 rows on a tiled matrix-core
 * contraction of the row-major lm_head); a bf16 head without the re-laid-out weight copy,
 * with hidden <= 4096 and B (K+1) <= 16, does the whole call in one launch.
 * Errors: as mtp_verify.
 */
mtp_status mtp_verify_hidden(mtp_handle* h, const void* target_hidden, const void* target_norm,
                             const int32_t* draft_tokens, int32_t B, int32_t K,
                             int32_t* accepted_len, int32_t* next_token, void* stream);

/*
 * Exact MTP-cache catch-up, used instead of mtp_kv_rollback after verification (devnotes
 * "How OpenVINO MTP Speculative Decoding Works Internally", Stateful execution; speculators
 * "MTP (Multi-Token Prediction)", Architecture). Draft step k >= 2 wrote its slot from the
 * head's own hidden state, and with all K drafts accepted the pair (h_{t+K}, d_K) was never
 * processed. For every sequence b and committed pair j = 1..a_b this runs
 * (target_hidden[b, j-1], d_j) through the layer's input side (embedding gather, separate
 * RMSNorms, eh_proj, attention RMSNorm, K/V projections, RoPE at position pos - K + j) and
 * writes slot len - K + j in the cache dtype; then len and pos advance to the committed
 * prefix: len += a + 1 - K, pos += a + 1 - K (values on entry: after the K-step draft).
 *   target_hidden [B, K+1, hidden] config dtype, 16-byte aligned: the target's last-layer
 *                 outputs before its final norm at inputs [last_token, d_1 .. d_K]
 *   draft_tokens [B, K], accepted_len [B] device int32 (accepted_len from mtp_verify /
 *                 mtp_verify_hidden).
 * Requires 1 <= K <= max_k. Device conditions: a slot outside the capacity sets
 * MTP_DEVERR_CAPACITY (the slot is skipped); an accepted length outside 0..K sets
 * MTP_DEVERR_ACCEPT and is clamped. Other errors: as mtp_kv_rollback.
 */
mtp_status mtp_kv_catchup(mtp_handle* h, mtp_kv* kv, const void* target_hidden,
                          const int32_t* draft_tokens, const int32_t* accepted_len, int32_t B,
                          int32_t K, void* stream);

/*
 * Prompt prefill of the MTP cache (devnotes "How OpenVINO MTP Speculative Decoding Works
 * Internally", "KV cache" and "Stateful execution": the MTP layer keeps its own one-layer
 * cache, filled for every position it has processed; speculators "MTP (Multi-Token
 * Prediction)", Architecture: the layer's input at position s pairs the verifier's hidden
 * state at s with the embedding of the token after s). For every sequence b and prompt row
 * s < n_valid[b] (all n rows when n_valid is NULL), the pair (target_hidden[b, s],
 * tokens[b, s]) runs through the layer's input side (embedding gather, separate RMSNorms,
 * eh_proj, attention RMSNorm, K/V projections, RoPE at position pos[b] + s) and is written
 * to slot len[b] + s in the cache dtype; then len[b] and pos[b] advance by that count.
 * After a prompt of P tokens (rows 0 .. P-2 paired with tokens 1 .. P-1, from an empty
 * cache) the first mtp_draft takes the hidden state at position P-1 and the target's first
 * generated token, and writes slot P-1.
 *   target_hidden [B, n, hidden] config dtype, 16-byte aligned: the target's last-layer
 *                 outputs before its final norm at positions pos[b] .. pos[b]+n-1
 *   tokens        [B, n] device int32: the token after each of those positions
 *   n_valid       [B] device int32 rows to take per sequence (0..n), or NULL for n
 * 0 <= n <= kv->capacity (n = 0 enqueues nothing), 1 <= B <= min(max_batch, kv->batch).
 * Rows run in groups, each streaming eh_proj and the K/V projections once: on bf16 heads (hidden
 * <= 8192) up to 2048 rows (at most max_batch x max_capacity), groups of more than 64 rows
 * on a tiled matrix-core contraction; else up to 64.
 * Device conditions: a slot outside the capacity sets MTP_DEVERR_CAPACITY (the row is
 * skipped); a token outside [0, vocab) sets MTP_DEVERR_TOKEN (row 0 of the embedding is
 * used); an n_valid entry outside [0, n] sets MTP_DEVERR_COUNT and is clamped.
 */
mtp_status mtp_kv_prefill(mtp_handle* h, mtp_kv* kv, const void* target_hidden,
                          const int32_t* tokens, const int32_t* n_valid, int32_t B, int32_t n,
                          void* stream);

/*
 * K recursive draft steps that SAMPLE each token at temperature T instead of taking the
 * argmax (OpenVINO GenAI "Speculative Decoding", Overview: at temperature > 0 the drafts
 * are verified by the standard sampling scheme, see mtp_verify_sample). Step k+1 draws
 * d_{k+1} from softmax(z_k / T), z_k = lm_head . RMSNorm(h^(k); g_final), by the
 * Gumbel-max rule argmax_v (z_k[v] / T + G_v) inside the fused lm_head kernel, and
 * writes z_k (before the temperature) to draft_logits. Everything else is mtp_draft.
 *   temperature  > 0 and finite
 *   seeds [B]    device uint64: each sequence's random stream
 *   offset       the iteration's counter: every (seed, offset) pair draws fresh numbers
 *   draft_tokens [B, K] device int32 (out)
 *   draft_logits [B, K, V] device fp32 (out): row (b, k) holds z_k of sequence b
 * Random numbers: Philox4x64-10 (Salmon et al., SC'11) with key (seeds[b], 0) and counter
 * (v >> 2, k, 0, offset); entry v takes word v & 3 as U = ((w >> 40) | 1) * 2^-24 and
 * G_v = -log(-log U).
 * Errors: as mtp_draft; a non-positive or non-finite temperature, or a null seeds /
 * draft_logits with K > 0, returns MTP_ERR_INVALID_ARG.
 */
mtp_status mtp_draft_sample(mtp_handle* h, const void* hidden, const int32_t* last_tokens,
                            mtp_kv* kv, int32_t B, int32_t K, float temperature,
                            const uint64_t* seeds, uint64_t offset, int32_t* draft_tokens,
                            float* draft_logits, void* stream);

/*
 * Speculative-sampling verification at temperature T (OpenVINO GenAI "Speculative
 * Decoding", Overview: the standard scheme, whose output follows the target's own
 * distribution; the first divergent position gets the target's sample). With
 * p_j = softmax(target_logits[b, j] / T) and q_j = softmax(draft_logits[b, j] / T):
 *   draft d_{j+1} = draft_tokens[b, j] is accepted iff U_j < p_j(d) / q_j(d) (in the log
 *   domain), for j = 0, 1, ... until the first rejection; a = number accepted;
 *   next_token = a sample of max(0, p_a - q_a) (renormalised) if a < K, of p_K if a = K
 *   (of p_a if rounding leaves no positive residual).
 *   target_logits [B, K+1, V] device fp32 (finite), draft_logits [B, K, V] device fp32 as
 *   written by mtp_draft_sample, draft_tokens [B, K] device int32, seeds / offset as for the
 *   draft of the same iteration; accepted_len [B], next_token [B] device int32 (out).
 * Random numbers (Philox4x64-10, key (seeds[b], 0)): U_j is word 0 of counter
 * (0, j, 1, offset); the final draw uses Gumbel noise from counter (v >> 2, a, 2, offset),
 * word v & 3. Use mtp_kv_rollback (or mtp_kv_catchup) afterwards as with mtp_verify.
 * Errors: as mtp_verify; a draft token outside [0, V) sets MTP_DEVERR_TOKEN and is
 * rejected; bad temperature or null seeds returns MTP_ERR_INVALID_ARG.
 */
mtp_status mtp_verify_sample(mtp_handle* h, const float* target_logits, const float* draft_logits,
                             const int32_t* draft_tokens, int32_t B, int32_t K, float temperature,
                             const uint64_t* seeds, uint64_t offset, int32_t* accepted_len,
                             int32_t* next_token, void* stream);

/* Synchronise `stream` (only that stream), read and clear the device error word. *bits
 * receives the MTP_DEVERR_* bits (may be NULL). Returns MTP_ERR_DEVICE when any bit was
 * set. Not for use under stream capture. */
mtp_status mtp_get_error(mtp_handle* h, void* stream, uint32_t* bits);

/*
 * Greedy verification that allocates nothing and needs no handle, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Same arguments and results as mtp_verify, with the vocabulary size
 * passed directly; the kernels' per-row keys and per-sequence completion counters live in a
 * fixed 320 KiB device array of the library (one per GPU, held until the process ends)
 * instead of a workspace, and each call clears the part it uses with a kernel before
 * verifying. Limits: 1 <= B <= MTP_NOALLOC_MAX_BATCH, 0 <= K <= 100 (MTP_ERR_CAPACITY
 * beyond), vocab >= 1. The stream must belong to the current device. Every call on one GPU
 * uses that GPU's array: calls that overlap in time on one GPU (different streams or
 * host threads without ordering) race and give undefined results; calls ordered on one
 * stream are safe. Never calls hipMalloc or hipFree.
 */
#define MTP_NOALLOC_MAX_BATCH 256
mtp_status mtp_verify_noalloc(const float* target_logits, const int32_t* draft_tokens,
                              int32_t B, int32_t K, int32_t vocab, int32_t* accepted_len,
                              int32_t* next_token, void* stream);

/* What a handle holds and how it groups rows (host only, no device call). */
typedef struct {
  size_t workspace_bytes;       /* device workspace the handle uses (mtp_workspace_size)      */
  size_t packed_weight_bytes;   /* of which: the re-laid-out weight copy (0 when none)        */
  int32_t verify_hidden_group_rows; /* rows per lm_head pass of mtp_verify_hidden             */
  int32_t catchup_group_rows;   /* rows per pass of mtp_kv_catchup and mtp_kv_prefill          */
  int32_t matrix_core_min_batch; /* draft batches in [min, max] run the matrix-core path;     */
  int32_t matrix_core_max_batch; /* both 0 when the configuration has no such path (fp32)    */
} mtp_info;
mtp_status mtp_get_info(const mtp_handle* h, mtp_info* out);

/*
 * Kernel timing with HIP events, for measurement only. Bit i of `mask` brackets every
 * launch of kernel class i on the caller's stream with a pair of events:
 *   0 embedding gather + norms + eh_proj   1 attention norm + QKV   2 attention
 *   3 O projection                         4 MLP norm + gate/up      5 down projection
 *   6 final norm + lm_head + argmax        7 verify                  8 rollback
 * mask = 0 (the default) records nothing. Not for use under stream capture.
 */
mtp_status mtp_set_profiling(mtp_handle* h, uint32_t mask);

/* Synchronise on the recorded events and return, per kernel class (arrays of `n`
 * entries, n <= 16), the summed duration in milliseconds and the number of launches
 * since the previous call; then forget the records. */
mtp_status mtp_get_profile(mtp_handle* h, float* total_ms, int32_t* launches, int32_t n);

/* Release the handle (host memory only; the workspace belongs to the caller). */
void mtp_destroy(mtp_handle* h);

/* Static description of a status code. */
const char* mtp_status_string(mtp_status s);

/*
 * Speculative length for the next iteration from the last one's accepted lengths (OpenVINO
 * GenAI "Speculative Decoding", Backend Differences: the stateful backend adapts
 * num_assistant_tokens per step from recent acceptance and backs off when it is low).
 * A sequence that accepted all K drafts asks for K + 1, one that accepted a < K asks for
 * a + 1; *k_next is the largest request clipped to [k_min, k_max]. Host function:
 * accepted_len is host memory [B] (values 0..K). Errors: MTP_ERR_INVALID_ARG for NULL
 * pointers or an accepted length outside 0..K, MTP_ERR_SHAPE for B < 1, K < 0,
 * k_min < 0, k_max < k_min or k_max > 100. Nothing is written on error.
 */
mtp_status mtp_adapt_k(const int32_t* accepted_len, int32_t B, int32_t K, int32_t k_min,
                       int32_t k_max, int32_t* k_next);

/*
 * Per-sequence speculative lengths from a window of recent iterations (OpenVINO GenAI
 * "Speculative Decoding", Backend Differences; forceinjection "MTP 深度解析", 7.3). Host
 * function; accepted_hist and k_hist are host [W, B] arrays (row i: one iteration's accepted
 * lengths and the lengths it used, any order of rows). Iteration i of sequence b asks for
 * k+1 when it accepted all k drafts and for a+1 otherwise; k_next[b] (host, [B]) is the mean
 * of its W requests rounded up, clipped to [k_min, k_max]. W = 1 is the per-iteration rule
 * of mtp_adapt_k applied to each sequence on its own. Errors: MTP_ERR_INVALID_ARG for NULL
 * pointers or an entry with k outside 0..100 or a outside 0..k; MTP_ERR_SHAPE for W < 1,
 * B < 1, k_min < 0, k_max < k_min or k_max > 100. Nothing is written on error.
 */
mtp_status mtp_adapt_k_seq(const int32_t* accepted_hist, const int32_t* k_hist, int32_t W,
                           int32_t B, int32_t k_min, int32_t k_max, int32_t* k_next);

/*
 * Training-loss weights of the K MTP steps, speculators user guide "MTP (Multi-Token
 * Prediction)", Step Weight Formula: out[k-1] = beta^(k-1) / sum_{j=1..K} beta^(j-1)
 * for k = 1..K (beta = 0.6, K = 3 gives 0.51, 0.31, 0.18). A host function: `out` is
 * caller-owned host memory with room for K floats; evaluated in double precision.
 * Errors: MTP_ERR_INVALID_ARG for a NULL `out` or a beta that is not finite and > 0;
 * MTP_ERR_SHAPE for K < 1 or K > 100. Nothing is written on error.
 */
mtp_status mtp_step_weights(float beta, int32_t K, float* out);

#ifdef __cplusplus
}
#endif
#endif /* MTP_H */
