/*
 * flashmap.h - C ABI of the MI355X (gfx950) FlashMap drafting step.
 *
 * The method (five news pages about FlashMap):
 *   - "FlashMap并行草拟加速大模型解码" (feinterview.poetries.top), first and
 *     second sections: K = 16 tokens drafted at once and verified by the target
 *     in one parallel pass, longest matching prefix kept; the drafter is a
 *     6-block DiT of width 2048 with 16 heads that reads target layers 1, 9,
 *     17, 25, 33 and reuses the target's frozen embedding and LM head; a flow
 *     teacher over one-hot token blocks is distilled into a flow map that goes
 *     from Gaussian noise to a whole block in one jump.
 *   - wire.sakhanda.co, "Как работает FlashMap?": the student is a denoiser
 *     with two time points; "Как развернуть FlashMap?": num_steps = 2 is an
 *     option; drafter and target share one GPU.
 *   - alphasignal.ai, "Why drafting still costs time": one cycle = propose a
 *     block, score it in parallel, accept the longest valid prefix, resume
 *     from a target token.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, unless a
 *     comment says "host".  They must stay valid until the stream reaches the
 *     call (weights: for the handle's lifetime).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work (fm_create and fm_context_sync also wait); they
 *     never allocate device memory, so a draft+verify sequence can be captured
 *     in a HIP graph, and replays of it follow the growing context.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     an error status nothing has been enqueued and no output was written;
 *     fm_last_error() describes the failure (thread-local string).
 *   - Inputs are assumed finite; NaN handling is unspecified.
 *   - Calls on one handle must not overlap on different streams.
 */
#ifndef FLASHMAP_H
#define FLASHMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fm_status {
  FM_OK = 0,
  FM_EINVAL = 1,     /* bad argument (NULL, size, alignment, order)          */
  FM_ECAPACITY = 2,  /* context or batch capacity of the handle exceeded     */
  FM_EHIP = 3,       /* a HIP runtime call or kernel launch failed           */
  FM_ESTATE = 4      /* call out of order (e.g. draft before set_weights)    */
} fm_status;

typedef enum fm_dtype {
  FM_BF16 = 0,  /* bfloat16 storage, float32 accumulation                     */
  FM_F32 = 1    /* float32 storage and arithmetic                             */
} fm_dtype;

/* Drafter shape and capacities.  Constraints checked by fm_create:
 *   K == 16; d a multiple of 128 (bf16) or 64 (f32), at most 4096; n_heads
 *   divides d with d / n_heads in {64, 128}; mlp_mult >= 1; n_ctx_layers == 5;
 *   V >= 16 and H >= 1 with V and H multiples of 8 (bf16) or 4 (f32), so
 *   every row starts 16-byte aligned;
 *   1 <= max_branches <= 4; 0 <= max_new <= 16; C_max >= 0; 1 <= max_steps <= 4,
 *   and V <= 524288 when max_steps > 1 (the softmax between jumps);
 *   1 <= max_requests <= 4, and max_branches == 1 when max_requests > 1. */
typedef struct fm_config {
  int K;             /* drafted block length (16)                            */
  int V;             /* vocabulary size (151936 for Qwen3)                    */
  int d;             /* drafter width (2048)                                  */
  int L;             /* DiT blocks (6)                                        */
  int n_heads;       /* attention heads (16)                                  */
  int mlp_mult;      /* MLP width = mlp_mult * d (4)                          */
  int H;             /* target hidden width per context layer                 */
  int n_ctx_layers;  /* target layers read (5: layers 1, 9, 17, 25, 33)       */
  int C_max;         /* context rows the cache can hold                       */
  int max_branches;  /* noise branches per draft (1, or 4 for a draft tree)   */
  int max_new;       /* context rows a single fm_draft call may append        */
  int max_steps;     /* flow-map jumps per draft (1, or 2 for num_steps = 2)  */
  fm_dtype dtype;    /* storage type of weights, features, noise              */
  int max_requests;  /* independent requests, each with its own context of up
                        to C_max rows (1, or up to 4 for batched drafting)     */
} fm_config;

/* Weights of one DiT block, all row-major [out][in], dtype = cfg.dtype:
 *   W_ada [6d][d], b_ada [6d]  adaLN: shift1, scale1, gate1, shift2, scale2, gate2
 *   W_qkv [3d][d], b_qkv [3d]  rows 0..d-1 query, d..2d-1 key, 2d..3d-1 value
 *   W_o   [d][d],  b_o   [d]
 *   W_1   [F][d],  b_1   [F]   F = mlp_mult * d
 *   W_2   [d][F],  b_2   [d]                                                 */
typedef struct fm_block_weights {
  const void *W_ada, *b_ada, *W_qkv, *b_qkv, *W_o, *b_o, *W_1, *b_1, *W_2, *b_2;
} fm_block_weights;

/* All drafter weights (device pointers, dtype = cfg.dtype, borrowed for the
 * handle's lifetime):
 *   E    [V][d]   frozen token embedding, one row per token
 *   W_lm [V][d]   frozen LM head, one row per token, no bias
 *   W_f  [d][n_ctx_layers*H], b_f [d]   context-feature fusion
 *   te_{s,t}_W1 [d][256], _b1 [d], _W2 [d][d], _b2 [d]   time embeddings of
 *                 the jump's start time s and end time t
 *   W_fa [2d][d], b_fa [2d]   final adaLN: shift, scale
 *   blocks        HOST array of L block-weight structs (copied by the call)  */
typedef struct fm_weights {
  const void *E, *W_lm, *W_f, *b_f;
  const void *te_s_W1, *te_s_b1, *te_s_W2, *te_s_b2;
  const void *te_t_W1, *te_t_b1, *te_t_W2, *te_t_b2;
  const void *W_fa, *b_fa;
  const fm_block_weights *blocks;
} fm_weights;

typedef struct fm_handle fm_handle;

/* Bytes of device workspace a handle with this configuration needs (per DiT
 * block and request a key and a value cache of ceil(C_max/32)*32 +
 * 32*max_branches positions of width d, modulation vectors, activations,
 * split-K partials and counters).  Returns 0 for an invalid configuration. */
size_t fm_workspace_bytes(const fm_config *cfg);

/* Create a handle on `device` using the caller's workspace (device memory of
 * at least fm_workspace_bytes(cfg) bytes, 256-byte aligned, owned by the
 * caller, not to be touched while the handle lives).  Enqueues a clear of the
 * workspace's counters on the null stream and waits for it.  The context
 * starts empty.  Errors: FM_EINVAL (config, NULL, alignment), FM_ECAPACITY
 * (ws_bytes too small), FM_EHIP. */
fm_status fm_create(const fm_config *cfg, void *workspace, size_t ws_bytes, int device,
                    fm_handle **out);

/* Release host state.  The workspace and weights stay the caller's. */
void fm_destroy(fm_handle *h);

/* Bind the weights (pointers are borrowed; nothing is copied on the device).
 * Must precede fm_set_schedule, fm_context_append and fm_draft.  Errors:
 * FM_EINVAL (a NULL or misaligned pointer). */
fm_status fm_set_weights(fm_handle *h, const fm_weights *w);

/* Precompute the adaLN vectors of every jump of a flow-map schedule
 * (wire.sakhanda.co, "Как работает FlashMap?": a two-time-point denoiser;
 * "Как развернуть FlashMap?": num_steps = 1 or 2).  `times` is a HOST array of
 * num_steps + 1 floats rising strictly from times[0] = 0 to times[num_steps]
 * = 1.  For each jump (s, t): c = TE_s(s) + TE_t(t); per block
 * W_ada silu(c) + b_ada; final W_fa silu(c) + b_fa, all in float32, stored in
 * the workspace.  The vectors depend only on (s, t) and the weights, so this
 * runs once per schedule, off the per-draft path.  Errors: FM_EINVAL
 * (order, num_steps outside 1..max_steps), FM_ESTATE (no weights), FM_EHIP. */
fm_status fm_set_schedule(fm_handle *h, const float *times, int num_steps, void *stream);

/* Context length.  Each request's length lives on the device, in the
 * workspace: kernels read it when the stream reaches them, and the calls that
 * append rows (fm_context_append, fm_draft, fm_draft_sample, fm_draft_batch)
 * advance it in their last kernel.  A captured HIP graph of a draft therefore
 * appends its rows and attends over the grown context on every replay (the
 * pages' cycle appends rows every cycle: alphasignal.ai, "Why drafting still
 * costs time").  The host keeps a mirror, advanced by the calls it sees (not by
 * replays), for the argument checks; fm_context_sync reloads it.  On the
 * device an append never passes C_max: the length stops there, rows past it
 * are not written, and a flag reports it to fm_context_sync. */

/* Append n rows of target hidden states to the context (prefill, or rows
 * accepted outside fm_draft).  feats: [n][n_ctx_layers][H], layers in the
 * order 1, 9, 17, 25, 33 (feinterview.poetries.top, second section).  For
 * each row: u = LN(W_f concat(feats) + b_f); for each block the row's key and
 * value (W_k u + b_k, W_v u + b_v) are written to the cache at the device
 * length and on.  Errors: FM_EINVAL, FM_ECAPACITY (mirror length + n >
 * C_max), FM_ESTATE, FM_EHIP. */
fm_status fm_context_append(fm_handle *h, const void *feats, int n, void *stream);

/* Roll the context back (or forward over rows already written) to new_len
 * rows: enqueues the write of the device length on `stream` and sets the
 * mirror.  Errors: FM_EINVAL (new_len < 0 or new_len > the highest row the
 * host has seen written), FM_EHIP. */
fm_status fm_context_truncate(fm_handle *h, int new_len, void *stream);

/* Current context length (rows) of the host mirror, or -1 for a NULL handle. */
int fm_context_length(const fm_handle *h);

/* Wait for `stream`, then load the device lengths of every request into the
 * host mirror (after graph replays).  Not for use inside a graph capture.
 * Errors: FM_EINVAL, FM_EHIP, FM_ECAPACITY (an append on the device reached
 * C_max and dropped rows since the last sync; the flag is then cleared). */
fm_status fm_context_sync(fm_handle *h, void *stream);

/* The same three calls for request `req` (0 <= req < max_requests) of a
 * handle that holds several requests; the calls above act on request 0.
 * Errors as above, plus FM_EINVAL for req out of range (length: -1). */
fm_status fm_context_append_req(fm_handle *h, int req, const void *feats, int n, void *stream);
fm_status fm_context_truncate_req(fm_handle *h, int req, int new_len, void *stream);
int fm_context_length_req(const fm_handle *h, int req);

/* One drafting step (feinterview.poetries.top, first section: the same noise
 * decides every position of the block jointly; wire.sakhanda.co, "Что такое
 * FlashMap?": K proposals from Gaussian noise in one step).
 *   noise     [B][K][V]  Gaussian noise blocks, one per branch
 *   B         branches, 1 <= B <= max_branches (B = 4: a draft tree whose
 *             branches share the context and do not see each other)
 *   new_feats [n_new][n_ctx_layers][H] context rows appended first (may be
 *             NULL when n_new == 0); they become rows length..length+n_new-1
 *   tokens    [B][K] int32 output: the draft
 *   logits    [B][K][V] float32 output of the last jump, or NULL
 *   hidden    [num_steps][L+1][B][K][d] float32 output: the residual stream
 *             after the embedding and after every block, or NULL
 * Computes, per jump (s, t) of the schedule: h = x_s E + P (P a fixed
 * sinusoidal table over the K positions), the L blocks (adaLN-modulated
 * attention of the block rows over [context; own block] keys, MLP), final
 * LN/modulation, logits = z W_lm^T; at t = 1 the tokens are the row argmax
 * of the float32 logits (lowest index among equal maxima); before t = 1 the
 * state moves by the flow map of the linear interpolant.  The new rows go to
 * the cache at the device length, the block rows attend over that length +
 * n_new rows, and the device length then advances by n_new (the mirror at
 * once).  Errors: FM_EINVAL, FM_ECAPACITY (mirror length + n_new > C_max),
 * FM_ESTATE (no weights or no schedule), FM_EHIP. */
fm_status fm_draft(fm_handle *h, const void *noise, int B, const void *new_feats, int n_new,
                   int32_t *tokens, float *logits, float *hidden, void *stream);

/* Drafting at temperature > 0 (feinterview.poetries.top, deployment list of
 * the last section, and wire.sakhanda.co, "Как развернуть FlashMap?": a
 * separate probabilistic draft-sampling mode for requests sampled at
 * temperature above 0).  The same step as fm_draft, except that row i of
 * branch b is SAMPLED from q = softmax(logits_i / temperature) instead of
 * taking the argmax: token = argmax_v (logits_iv / temperature + G), G the
 * Gumbel noise -log(-log U) of the Philox4x32-10 counter (v, i, b, 0) under
 * the key `seed` (low word, high word), U = (x + 0.5) / 2^32 for the draw x,
 * lowest index on ties.
 *   temperature  > 0 and finite (host value)
 *   seed         64-bit key (host value); the same seed gives the same draft
 *   logits       [B][K][V] float32 output, required (fm_verify_sample reads it)
 *   lse          [B][K] float32 output: log sum_v exp(logits_iv / temperature)
 * Other arguments and errors as fm_draft (hidden is not offered here). */
fm_status fm_draft_sample(fm_handle *h, const void *noise, int B, const void *new_feats, int n_new,
                          float temperature, uint64_t seed, int32_t *tokens, float *logits, float *lse,
                          void *stream);

/* One drafting step for R independent requests at once (serving with more
 * than one concurrent request; the pages measure concurrency 1 only,
 * feinterview.poetries.top, results section).  Row block r (16 rows) is
 * request r: it attends to request r's context plus its own block, exactly as
 * fm_draft with B = 1 on that request alone; the contractions stream every
 * weight once for all R * 16 rows.
 *   noise     [R][K][V]  one noise block per request
 *   R         1 <= R <= max_requests
 *   new_feats [sum n_new][n_ctx_layers][H] context rows appended first, the
 *             rows of request 0, then request 1, ... (NULL when no rows)
 *   n_new     HOST array of R counts (NULL: none), sum <= max_new
 *   tokens    [R][K] int32 output; logits [R][K][V] float32 output or NULL
 * Each request's context advances by its n_new.  fm_verify with B = R then
 * verifies the requests independently (its best output is meaningless here).
 * Errors: FM_EINVAL, FM_ECAPACITY (R > max_requests, a request's context over
 * C_max, sum n_new > max_new), FM_ESTATE, FM_EHIP. */
fm_status fm_draft_batch(fm_handle *h, const void *noise, int R, const void *new_feats, const int *n_new,
                         int32_t *tokens, float *logits, void *stream);

/* fm_draft_batch at temperature > 0 (the probabilistic draft-sampling mode of
 * feinterview.poetries.top, deployment list of the last section, for a batch
 * of requests): request r samples its rows exactly as fm_draft_sample would
 * for that request alone with seed seeds[r] and one branch, i.e. Gumbel noise
 * of Philox counter (v, i, 0, 0) under key seeds[r].
 *   temperature  > 0 and finite (host value)
 *   seeds        HOST [R] 64-bit seeds, one per request
 *   logits [R][K][V] and lse [R][K] float32 outputs, as for fm_draft_sample
 * Other arguments and errors as for fm_draft_batch; FM_EINVAL also for a
 * bad temperature or NULL seeds, logits or lse. */
fm_status fm_draft_batch_sample(fm_handle *h, const void *noise, int R, const void *new_feats,
                                const int *n_new, float temperature, const uint64_t *seeds,
                                int32_t *tokens, float *logits, float *lse, void *stream);

/* Greedy verification (feinterview.poetries.top, first section;
 * wire.sakhanda.co, "Что такое FlashMap?"; alphasignal.ai, "Why drafting
 * still costs time").  Stateless; needs no handle.
 *   target_logits [B][K+1][V] (dtype): row j is the target's prediction for
 *             draft slot j, row K the token after a fully accepted block
 *   draft     [B][K] int32
 *   emitted   [B][K+1] int32 output: draft[0..n-1], then y_n, then -1 padding
 *   accept    [B] int32 output: n = longest prefix with draft[i] == y_i,
 *             y_j = lowest-index argmax of row j
 *   best      [1] int32 output: lowest branch index with the largest n
 * Requires 1 <= B <= 64, 1 <= K <= 64, V >= 1.  Errors: FM_EINVAL, FM_EHIP. */
fm_status fm_verify(const void *target_logits, fm_dtype dtype, int B, int K, int V,
                    const int32_t *draft, int32_t *emitted, int32_t *accept, int32_t *best,
                    void *stream);

/* The same greedy verification for a handle's drafts (K = 16, V of the
 * handle's configuration), with each target row read by 16 workgroups at once
 * instead of one: the per-slice maxima go to the handle's verifier scratch and
 * one more launch merges them, so the result is the one fm_verify gives on the
 * same arguments (first maximum of each row; logits without NaN).  Rows that
 * do not start on a 16-byte boundary take fm_verify's path.  Shares the
 * scratch with fm_verify_sample: calls on one handle are ordered on one stream.
 *   target_logits [B][17][V] (dtype), draft [B][16], emitted [B][17],
 *   accept [B], best [1]: as for fm_verify.
 * Requires 1 <= B <= max(max_branches, max_requests) (branches of one
 * request, or requests).  Errors: FM_EINVAL, FM_ECAPACITY, FM_EHIP. */
fm_status fm_verify_greedy(fm_handle *h, const void *target_logits, fm_dtype dtype, int B,
                           const int32_t *draft, int32_t *emitted, int32_t *accept, int32_t *best,
                           void *stream);

/* Probabilistic verification at temperature > 0 (alphasignal.ai, "Why
 * drafting still costs time": lossless verification leaves the distribution
 * of the target's samples unchanged).  The speculative-sampling rule, with
 * p_j = softmax(target_logits_j / temperature) and q_i the drafter's
 * distribution (draft_logits_i / temperature normalised by draft_lse_i):
 *   draft i is accepted while u_i * q_i(d_i) < p_i(d_i), u_i the uniform of
 *   Philox counter (0, i, b, 2); n = accepted prefix; row n emits a sample of
 *   max(0, p_n - q_n) (renormalised) if n < K, of p_K if n = K, drawn by
 *   Gumbel-max with counters (v, n, b, 1) (lowest index on ties; a residual
 *   that is zero on every token in float32 falls back to p_n).
 *   target_logits [B][K+1][V] (dtype), draft_logits [B][K][V] and draft_lse
 *             [B][K] as written by fm_draft_sample, draft [B][K] int32 tokens
 *             in [0, V) (others give unspecified results)
 *   emitted   [B][K+1] int32 output: draft[0..n-1], the sample, then -1
 *   accept    [B] int32 output: n
 * Branches are verified independently (no branch selection: choosing among
 * sampled branches would change the output distribution).  K and V are the
 * handle's; scratch lives in the handle's workspace, so calls on one handle
 * must not overlap.  B counts branches of one request or, on a handle of
 * several requests, requests.  Errors: FM_EINVAL, FM_ECAPACITY (B above
 * max(max_branches, max_requests)), FM_EHIP. */
fm_status fm_verify_sample(fm_handle *h, const void *target_logits, fm_dtype dtype, int B,
                           const float *draft_logits, const float *draft_lse, const int32_t *draft,
                           float temperature, uint64_t seed, int32_t *emitted, int32_t *accept,
                           void *stream);

/* fm_verify_sample for the requests of a batch (alphasignal.ai, "Why
 * drafting still costs time": the verification rule leaves each request's
 * sampled output distribution unchanged): request r is verified exactly as
 * fm_verify_sample would verify it alone with seed seeds[r] as branch 0
 * (counters (0, i, 0, 2) and (v, n, 0, 1) under key seeds[r]).
 *   R         requests, 1 <= R <= max_requests; arrays as for fm_verify_sample
 *             with B = R
 *   seeds     HOST [R] 64-bit seeds, one per request
 * Errors as for fm_verify_sample; FM_EINVAL also for NULL seeds. */
fm_status fm_verify_sample_batch(fm_handle *h, const void *target_logits, fm_dtype dtype, int R,
                                 const float *draft_logits, const float *draft_lse, const int32_t *draft,
                                 float temperature, const uint64_t *seeds, int32_t *emitted,
                                 int32_t *accept, void *stream);

/* fm_verify_sample for callers that cannot allocate device memory or hold a
 * handle (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same verification, bit for bit, with its scratch
 * in a static device array of the library (160 KB per GPU, held until the
 * process ends) instead of a handle's workspace.
 *   K         must be 16; V >= 1 the vocabulary size of the logits
 *   B         1 <= B <= 4 branches (more: FM_ECAPACITY, nothing enqueued)
 *   other arguments as fm_verify_sample
 * The stream must belong to the current device.  The first call on a device
 * looks up that device's copy of the array.  Every call on one GPU shares it:
 * calls that overlap on one GPU (several streams or threads) race.  Nothing
 * in the array needs clearing between calls.  Errors: FM_EINVAL,
 * FM_ECAPACITY, FM_EHIP. */
fm_status fm_verify_sample_noalloc(const void *target_logits, fm_dtype dtype, int B, int K, int V,
                                   const float *draft_logits, const float *draft_lse, const int32_t *draft,
                                   float temperature, uint64_t seed, int32_t *emitted, int32_t *accept,
                                   void *stream);

/* Kernels a probe can bracket. */
typedef enum fm_probe_kernel {
  FM_PROBE_NONE = 0,
  FM_PROBE_EMBED = 1,    /* noise-block embedding kernel (first jump; without
                            its split-sum kernel)                             */
  FM_PROBE_LM_HEAD = 2,  /* LM head kernel with fused per-workgroup argmax keys
                            (last jump; without the merge of those keys)      */
  FM_PROBE_FC1 = 3,      /* first MLP contraction of block 0 (first jump)     */
  FM_PROBE_VERIFY = 4    /* unused by fm_draft; reserved                      */
} fm_probe_kernel;

/* Profiling hook.  While set, every fm_draft call on this handle records the
 * HIP event `ev_start` (a hipEvent_t passed as void*) on its stream right
 * before launching `kernel` and `ev_stop` right after it, so the caller can
 * read that kernel's duration with hipEventElapsedTime.  FM_PROBE_NONE clears
 * the probe.  Events are borrowed.  Errors: FM_EINVAL. */
fm_status fm_set_probe(fm_handle *h, fm_probe_kernel kernel, void *ev_start, void *ev_stop);

/* Message of the last failed call on this thread ("" if none). */
const char *fm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHMAP_H */
