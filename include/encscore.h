/*
 * encscore.h -- C ABI of the variable-length transformer scorer for MI355X
 * (gfx950).
 *
 * The library gives every sequence of a packed, variable-length batch one
 * scalar score (reward-model scoring, compact-BERT inference) and plans how to
 * group a stream of requests into batches.  The method follows:
 *   - "TurboTransformers: An Efficient GPU Serving System For Transformer
 *     Models" (review; Abstract and Proposed method): GEMMs plus per-row
 *     ("batch reduction") Softmax and LayerNorm kernels, no fixed-length
 *     padding, requests sorted by length and grouped by a dynamic-programming
 *     batch scheduler;
 *   - "Learning to summarize from human feedback" (summary; Method adaptation): a scalar
 *     head read at the end of the complete sequence, with rewards normalised
 *     so that reference sequences average zero.
 *
 * Conventions for every function:
 *   - The return value is an es_status; ES_OK is 0, errors are negative.  No
 *     C++ exception crosses this boundary.  es_last_error() gives a message
 *     for the last failure on the calling thread.
 *   - Pointers prefixed d_ are device pointers (HIP device memory of the
 *     current device), h_ are host pointers.  The caller owns every buffer it
 *     passes; the library neither frees nor keeps them after the call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Device work is
 *     enqueued on it and the call returns without waiting, unless stated.
 *   - One es_model handle runs one call at a time: its workspace is shared,
 *     so overlapping calls on one handle (from several threads, or on two
 *     streams without synchronising between them) race.  Separate handles are
 *     independent.
 */
#ifndef ENCSCORE_H
#define ENCSCORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t es_status;
enum {
  ES_OK = 0,
  ES_ERR_ARG = -1,         /* null pointer, bad count, malformed offsets       */
  ES_ERR_RANGE = -2,       /* a length outside [1, limit]                       */
  ES_ERR_CAPACITY = -3,    /* batch exceeds the workspace sized at load time    */
  ES_ERR_FORMAT = -4,      /* weight blob header or size invalid                */
  ES_ERR_IO = -5,          /* blob file unreadable                              */
  ES_ERR_HIP = -6,         /* a HIP runtime call failed (message has details)   */
  ES_ERR_DEVICE_FLAG = -7  /* a kernel saw an out-of-range token id             */
};

typedef struct es_model es_model; /* opaque: device weights + workspace */

/* Model description returned by es_model_info. */
typedef struct {
  int32_t n_layers, hidden, n_heads, head_dim, ffn, vocab, max_pos;
  int32_t pre_ln;      /* 0: post-LN encoder (embedding LN), 1: pre-LN + final LN */
  int32_t causal;      /* 0: bidirectional within a sequence, 1: causal          */
  int32_t bf16;        /* 0: fp32 weights and activations; 1: bf16 GEMM operands,
                          fp32 accumulation, fp32 residual stream and LN        */
  float eps;           /* LayerNorm epsilon                                     */
  float reward_offset; /* added to every raw reward                             */
  int64_t max_tokens;  /* capacity: tokens per es_score_batch call              */
  int32_t max_seqs;    /* capacity: sequences per call                          */
  int64_t device_bytes;/* device memory held by the handle                      */
} es_model_info_t;

/* ------------------------------------------------------------------ models */

/*
 * es_load_weights / es_load_weights_mem -- parse a weight blob, upload it to
 * the current HIP device and size the workspace for batches of up to
 * `max_tokens` packed tokens and `max_seqs` sequences.
 *
 * Blob ("ESW1", little-endian): a 64-byte header
 *   char magic[4]="ESW1"; u32 version=1; u32 n_layers, hidden, n_heads, ffn,
 *   vocab, max_pos, pre_ln, causal, act(0 = exact-erf GELU), wdtype(0 fp32,
 *   1 bf16); f32 eps, reward_offset; u32 reserved[2]
 * followed by the tensors in this order (matrices/embeddings in wdtype,
 * vectors always fp32): tok_emb[V,H], pos_emb[P,H], norm_g[H], norm_b[H]
 * (embedding LN for post-LN, final LN for pre-LN); per layer w_qkv[3H,H]
 * (rows Q|K|V, head h = rows h*d..h*d+d-1 of each part), b_qkv[3H],
 * w_o[H,H], b_o[H], ln1_g[H], ln1_b[H], w_1[F,H], b_1[F], w_2[H,F], b_2[H],
 * ln2_g[H], ln2_b[H]; then head_w[H], head_b[1].  Weight matrices are
 * [out, in] (y = x W^T + b).
 *
 * Errors: ES_ERR_IO (file), ES_ERR_FORMAT (magic/version/sizes/trailing
 * bytes), ES_ERR_ARG (max_tokens < 1, max_seqs < 1, out NULL), ES_ERR_HIP.
 * On success *out owns device memory until es_free.
 */
es_status es_load_weights(const char *blob_path, int64_t max_tokens, int32_t max_seqs,
                          es_model **out);
es_status es_load_weights_mem(const void *h_blob, int64_t nbytes, int64_t max_tokens,
                              int32_t max_seqs, es_model **out);

/* Release the handle and its device memory (synchronises the device first). */
void es_free(es_model *m);

es_status es_model_info(const es_model *m, es_model_info_t *info);

/*
 * es_blob_info -- host only (never touches HIP): validate `nbytes` bytes of a
 * weight blob exactly as es_load_weights_mem does (header fields, tensor
 * sizes, no trailing bytes) and report the model's shape in *info (the
 * capacity and device_bytes fields are 0).  Errors: ES_ERR_ARG (NULL),
 * ES_ERR_FORMAT.
 */
es_status es_blob_info(const void *h_blob, int64_t nbytes, es_model_info_t *info);

/* ----------------------------------------------------------------- scoring */

/*
 * es_score_batch -- the hot path: one forward pass over a packed batch.
 *
 *   d_token_ids  int32[h_offsets[n_seqs]] on the device, sequences back to
 *                back with no padding (TurboTransformers review, Proposed
 *                method: batches formed without fixed-length padding).
 *   h_offsets    int32[n_seqs+1] on the host, offsets[0] = 0, strictly
 *                increasing; sequence i is tokens offsets[i] .. offsets[i+1]-1
 *                and its positions restart at 0.
 *   d_rewards    float32[n_seqs] on the device; rewards[i] = w . h + b +
 *                offset, h the final hidden state of the LAST token of
 *                sequence i (after the final LayerNorm for pre-LN models)
 *                ("Learning to summarize from human feedback", Method adaptation: scalar
 *                head, reward at the end of the complete sequence).
 *
 * Precision: bf16 models run every row with bf16 GEMM operands and fp32
 * accumulation.  For pre-LN bf16 models (hidden and FFN widths multiples of
 * 64) the last row of each sequence -- the only one the
 * reward reads -- is also carried through every layer in fp32 beside that
 * pass, its GEMM operands split into hi + lo bf16 pairs and its attention
 * in fp32 over the pass's keys and values (the last-token refinement
 * kernels below); the reward is read from that row.  Its bf16 operand
 * rounding otherwise dominates the decoder's reward error.
 *
 * Host-side validation (synchronous, before any device work): n_seqs in
 * [1, max_seqs] (ES_ERR_ARG / ES_ERR_CAPACITY), offsets malformed (ES_ERR_ARG),
 * a length above max_pos (ES_ERR_RANGE), total tokens above max_tokens
 * (ES_ERR_CAPACITY).  Token ids are checked on the device: an id outside
 * [0, vocab) reads row 0 and sets a sticky flag reported by
 * es_check_device_errors.  Results are bitwise reproducible for identical
 * inputs.  The call copies its small per-batch metadata from pinned host
 * memory and may wait for the previous call's copy before reusing it.
 */
es_status es_score_batch(es_model *m, const int32_t *d_token_ids, const int32_t *h_offsets,
                         int32_t n_seqs, float *d_rewards, void *stream);

/*
 * es_score_batch_static -- es_score_batch for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, validation, kernels and
 * results (bitwise equal to es_score_batch on the same model settings); it
 * calls no hipMalloc, hipHostMalloc or hipFree.  Every intermediate -- the
 * batch metadata, activations, and (unfused attention) the score blocks --
 * lives in one fixed device array of ES_STATIC_SCRATCH_BYTES (64 MiB) that
 * the library holds on every GPU it is loaded on until the process ends.
 * A batch needing more (metadata + tensors at their lifetime-shared
 * offsets; e.g. BERT-base shapes hold about 4096 tokens with fused attention)
 * is refused with ES_ERR_CAPACITY before any device work.  The metadata is
 * copied from pageable host memory on `stream`.  All calls on one GPU share
 * that array, which keeps the previous call's contents (no kernel relies on
 * it being zero): calls that overlap in time on one GPU -- on different
 * streams, threads or handles -- race and must be serialised by the caller.
 * The current device must be the model's (else ES_ERR_ARG).
 */
#define ES_STATIC_SCRATCH_BYTES (64ll * 1024 * 1024)
es_status es_score_batch_static(es_model *m, const int32_t *d_token_ids,
                                const int32_t *h_offsets, int32_t n_seqs, float *d_rewards,
                                void *stream);

/* Plan / work summary of one es_score_requests call. */
typedef struct {
  int32_t n_batches;     /* batches the planner formed                           */
  int64_t total_cost;    /* planner objective: sum of overhead + |B| * max_len,  */
                         /* or of the cost table's entries (es_set_cost_table) */
  int64_t padded_tokens; /* sum over batches of |B| * max_len(B)                 */
  int64_t packed_tokens; /* tokens actually computed (no padding)                */
} es_stream_stats_t;

/*
 * es_score_requests -- score a whole request stream: plan, pack, forward
 * every batch, scatter the rewards back to request order.
 *
 *   d_token_ids  int32[sum h_lengths] on the device, the requests back to back
 *                in arrival order.
 *   h_lengths    int32[n] on the host, each in [1, max_pos].
 *   d_rewards    float32[n] on the device; d_rewards[i] is request i's reward.
 *
 * The planner is es_plan_batches with max_tokens = the handle's max_tokens
 * and the given batch_overhead (TurboTransformers review, Proposed method:
 * requests sorted by length and grouped by dynamic programming with minimal
 * padding).  Each batch is packed without padding: its sequences' ids are read
 * in place from d_token_ids by the embedding kernel, and the head kernel
 * writes each reward to its request slot.  Per-call metadata for all batches
 * is uploaded in one copy.  `stats` may be NULL.  Errors: as es_plan_batches
 * and es_score_batch; ES_ERR_CAPACITY if a planned batch has more sequences
 * than max_seqs.
 */
es_status es_score_requests(es_model *m, const int32_t *d_token_ids, const int32_t *h_lengths,
                            int32_t n, int64_t batch_overhead, float *d_rewards, void *stream,
                            es_stream_stats_t *stats);

/*
 * es_score_best_of_n -- best-of-N scoring with shared prompts ("Learning to
 * summarize from human feedback", Method adaptation: the reward model scores
 * N candidate summaries of a post and the highest-scoring one is kept).
 *
 *   d_token_ids     int32 on the device: the n_prompts prompts back to back,
 *                   then every candidate continuation back to back (the
 *                   candidates of prompt 0 first, then those of prompt 1, ...).
 *   h_prompt_lengths int32[n_prompts] (host), each >= 1.
 *   h_cand_lengths  int32[sum h_cand_counts] (host), each >= 1, and prompt +
 *                   candidate <= max_pos.
 *   h_cand_counts   int32[n_prompts] (host), candidates per prompt, each >= 1.
 *   d_rewards       float32[sum h_cand_counts] (device): the reward of prompt
 *                   p followed by candidate c, in candidate order.
 *   d_best          int32[n_prompts] (device): per prompt, the index within
 *                   its candidates of the largest reward; the lowest index
 *                   among equal rewards.
 *
 * The model must be causal (a token's state depends only on earlier tokens)
 * and bf16.  Each prompt is embedded and run through the layers once; its
 * candidates' tokens take positions after it and attend to its keys and
 * values, so the work is that of the prompt plus the candidates rather than
 * N copies of the prompt.  Rewards are bitwise those es_score_requests gives
 * for the concatenated prompt + candidate sequences under fused attention.
 * Prompt groups (a prompt with all its candidates) are the planner's items,
 * each as long as its tokens (es_plan_batches, budget max_tokens); grouping
 * and passes in flight apply as in es_score_requests; attention is always
 * the fused kernel here.  Asynchronous on `stream`; `stats` may be NULL
 * (packed_tokens counts each prompt once).  Errors: ES_ERR_ARG (NULL,
 * counts < 1, model not causal bf16), ES_ERR_RANGE (a length outside its
 * bounds), ES_ERR_CAPACITY (a prompt group above max_tokens tokens or
 * max_seqs - 1 candidates), ES_ERR_HIP.
 */
es_status es_score_best_of_n(es_model *m, const int32_t *d_token_ids,
                             const int32_t *h_prompt_lengths, int32_t n_prompts,
                             const int32_t *h_cand_lengths, const int32_t *h_cand_counts,
                             int64_t batch_overhead, float *d_rewards, int32_t *d_best,
                             void *stream, es_stream_stats_t *stats);

/*
 * es_forward_hidden -- diagnostic form of es_score_batch: runs the embedding
 * and the first `n_layers` layers (0 <= n_layers <= model layers) and copies
 * the fp32 residual stream into d_hidden float32[offsets[n_seqs], hidden]
 * (row t = token t of the packed batch).  Same validation as es_score_batch.
 * These are the bf16 pass's rows (no last-token refinement).
 */
es_status es_forward_hidden(es_model *m, const int32_t *d_token_ids, const int32_t *h_offsets,
                            int32_t n_seqs, int32_t n_layers, float *d_hidden, void *stream);

/*
 * es_set_concurrency -- number of planned batches es_score_requests keeps in
 * flight at once (1..4, default 1).  Each needs its own activation and score
 * workspace (allocated here, synchronously, sized like the first) and runs on
 * an internal stream forked from and joined back to the caller's stream, so
 * the call stays ordered on that stream.  Batches are still formed by the
 * planner; this only overlaps their kernels to fill the GPU.  Other entry
 * points use one workspace on the caller's stream.  With one batch in
 * flight, the last-token refinement (es_set_refinement) of a pass runs on an
 * internal stream of the model's, forked from and joined back to the pass's
 * stream (the call stays ordered on the caller's stream).  Errors:
 * ES_ERR_ARG, ES_ERR_HIP.
 */
es_status es_set_concurrency(es_model *m, int32_t batches_in_flight);

/*
 * es_set_memory_mode -- where the intermediates of a pass (residual stream,
 * GEMM inputs, Q|K|V, context, FFN middle, score blocks) live
 * (TurboTransformers review, Proposed method: a sequence-length-aware
 * allocator for variable-length inputs, balancing footprint against
 * allocation cost):
 *   ES_MEM_LENGTH_AWARE (default): per pass, sizes from the pass's own token
 *     count and score blocks, placed by es_plan_arena (tensors whose steps do
 *     not overlap share bytes) in one arena per pass in flight.  An arena
 *     grows when a pass needs more (the host waits for queued work first;
 *     1/8 headroom, 16 MiB steps) and, at a call's first pass, shrinks to the
 *     previous call's largest need (same rounding) if it holds at least
 *     twice that.
 *   ES_MEM_FIXED: one workspace per pass in flight, allocated up front for
 *     max_tokens x batches_per_pass tokens and worst-case score blocks; no
 *     allocation while scoring.
 *   ES_MEM_EXACT: per pass, an arena of exactly that pass's need, replacing
 *     the previous one after the host waits for the device -- the smallest
 *     footprint at the largest allocation cost (for comparison).
 * Rewards are bitwise the same in every mode.  Synchronises the device.
 * Errors: ES_ERR_ARG (unknown mode), ES_ERR_HIP.
 */
enum { ES_MEM_FIXED = 0, ES_MEM_LENGTH_AWARE = 1, ES_MEM_EXACT = 2 };
es_status es_set_memory_mode(es_model *m, int32_t mode);

/* Workspace memory of a handle (es_memory_stats). */
typedef struct {
  int32_t mode;            /* ES_MEM_*                                            */
  int64_t device_bytes;    /* device memory held now: weights, workspaces, arenas */
  int64_t work_bytes;      /* of which workspaces / arenas                        */
  int64_t peak_work_bytes; /* largest work_bytes since load or the last reset     */
  int64_t allocs;          /* workspace / arena allocations since then            */
  double alloc_ms;         /* host time spent in them (incl. waiting for a lane)  */
} es_memory_stats_t;

/*
 * es_memory_stats -- fill *out; reset != 0 then zeroes the allocation count
 * and time and restarts the peak from the current size.  Host only (no
 * synchronisation).  Errors: ES_ERR_ARG.
 */
es_status es_memory_stats(es_model *m, es_memory_stats_t *out, int32_t reset);

/*
 * es_set_pruning -- last-layer pruning for the scoring entry points (default
 * on).  The reward reads only the final state of each sequence's last token
 * ("Learning to summarize from human feedback", Method adaptation: the
 * reward is read at the end of the complete sequence), so the last layer runs
 * its QKV GEMM on every token (all keys and values) and the rest -- the last
 * query's attention, the output projection, the LayerNorms and the FFN -- on
 * the last token of each sequence only (with the last-token refinement of
 * es_score_batch those rows already run in the refinement, so the pruned last
 * layer stops after its QKV GEMM).  Rewards are bitwise the same either
 * way; es_forward_hidden never prunes.  enabled: 0 or 1.  Errors: ES_ERR_ARG.
 */
es_status es_set_pruning(es_model *m, int32_t enabled);

/*
 * es_set_refinement / es_get_refinement -- the last-token refinement of the
 * scoring entry points (es_score_batch: the reward row of each sequence
 * carried in fp32 with hi + lo bf16 GEMM operands).  On by default wherever
 * the model supports it: pre-LN bf16 models with hidden and FFN widths
 * multiples of 64.  0 turns it off: rewards then carry
 * the bf16 pass's operand rounding (on the 24-layer decoder up to 1.5e-2
 * from the float64 reference, against 7.3e-3 with it), and the scoring pass
 * is about 4 % faster there.  Takes effect from the next call.
 * Errors: ES_ERR_ARG (enabled not 0 / 1, or 1 on a model that does not
 * support it).
 */
es_status es_set_refinement(es_model *m, int32_t enabled);
es_status es_get_refinement(const es_model *m, int32_t *enabled);

/*
 * es_set_batch_grouping -- number of consecutive planned batches (1..8,
 * default 1) that es_score_requests packs back to back and scores in one
 * pass through the layers.  The planner's batches stay as planned
 * (TurboTransformers review, Proposed method: the DP scheduler over sorted
 * requests); grouping only makes each GEMM see the tokens of several of them
 * at once, so the matrix cores get larger problems.  Every kernel works per
 * token or per sequence, so rewards are bitwise the same for any grouping.
 * The workspaces of the batches in flight grow to hold that many planned
 * batches (allocated here, synchronously).  Combines with es_set_concurrency:
 * groups are what is kept in flight.  Errors: ES_ERR_ARG, ES_ERR_HIP.
 */
es_status es_set_batch_grouping(es_model *m, int32_t batches_per_pass);

/*
 * es_set_cost_table -- make es_score_requests plan with measured batch costs
 * (es_plan_batches_measured; TurboTransformers review, Proposed method: the
 * DP batch scheduler) instead of batch_overhead + |B| * max_len.  The table
 * has the layout es_plan_batches_measured documents and is copied; only its
 * first max_seqs rows are used, so no planned batch has more sequences than a
 * workspace holds, and batch_overhead is then ignored.  cost_table = NULL
 * goes back to the linear cost.  es_score_best_of_n keeps the linear cost
 * (its items are prompt groups, not sequences).  Errors: ES_ERR_ARG (a table
 * es_plan_batches_measured rejects, or max_len below the model's max_pos).
 */
es_status es_set_cost_table(es_model *m, const int64_t *cost_table, int32_t max_batch,
                            int32_t max_len);

/*
 * es_set_attention -- how the masked attention of each layer runs: 0 =
 * three kernels, scores to HBM, the Softmax row reduction (TurboTransformers
 * review, Proposed method), then P.V; 1 = one fused kernel per (query tile,
 * head) that keeps each score row in registers with an online softmax (same
 * result up to rounding, no score traffic).  Default: 1 for bf16 models, 0
 * for fp32 models, which support 0 only.  Shared-prompt scoring
 * (es_score_best_of_n) always runs the fused form.  Errors: ES_ERR_ARG.
 */
es_status es_set_attention(es_model *m, int32_t mode);

/* Set / read the scalar added to every reward. */
es_status es_set_reward_offset(es_model *m, float offset);
es_status es_get_reward_offset(const es_model *m, float *offset);

/*
 * es_calibrate_offset -- score a reference set (packed like es_score_batch,
 * any number of sequences; it is planned into batches internally as in
 * es_score_requests) with the offset at zero, and return
 * offset = -mean(raw rewards) (mean in double precision, stored as float) so
 * that the reference set averages zero ("Learning to summarize from human
 * feedback", Method).  Synchronises `stream`.  The model's offset is NOT
 * changed; pass the result to es_set_reward_offset.
 */
es_status es_calibrate_offset(es_model *m, const int32_t *d_token_ids, const int32_t *h_offsets,
                              int32_t n_ref, void *stream, float *offset_out);

/*
 * es_check_device_errors -- synchronise `stream`, then report and clear the
 * sticky device flag: ES_ERR_DEVICE_FLAG if any kernel since the last check
 * saw an out-of-range token id, else ES_OK.
 */
es_status es_check_device_errors(es_model *m, void *stream);

/* ---------------------------------------------------------------- planner */

/*
 * es_plan_batches -- host-only batch planner (never touches HIP).
 *
 * TurboTransformers review (Abstract; Proposed method): requests sorted by
 * length and grouped by dynamic programming with minimal padding.  Reading
 * used: minimise  sum_B ( batch_overhead + |B| * max_len(B) )  subject to
 * |B| * max_len(B) <= max_tokens, over partitions of the requests.
 *   order[n]          request indices sorted by (length, index)
 *   batch_starts[B+1] batch b is order[batch_starts[b] .. batch_starts[b+1]-1]
 *   *n_batches = B, *total_cost = the optimal cost.
 * The DP over sorted prefixes keeps the first minimising split point, so ties
 * resolve to the plan whose start list, read backwards, is smallest.
 * batch_starts must hold n+1 entries.  n = 0 gives B = 0, starts = {0}.
 * Errors: ES_ERR_ARG (n < 0, NULL pointers, max_tokens < 1,
 * batch_overhead < 0), ES_ERR_RANGE (a length < 1 or > max_tokens).
 */
es_status es_plan_batches(const int32_t *lengths, int32_t n, int64_t max_tokens,
                          int64_t batch_overhead, int32_t *order, int32_t *batch_starts,
                          int32_t *n_batches, int64_t *total_cost);

/*
 * es_plan_batches_measured -- host-only batch planner under a measured cost
 * table (never touches HIP).
 *
 * TurboTransformers review (Abstract; Proposed method): the DP batch
 * scheduler aims at throughput on variable-length requests; here the cost of
 * a batch is what it was measured to take instead of a linear formula.
 * Reading used: minimise  sum_B C[|B|-1][max_len(B)-1]  subject to
 * |B| <= max_batch and |B| * max_len(B) <= max_tokens.
 *   cost_table  int64[max_batch * max_len], row-major: entry
 *               [(b-1) * max_len + (l-1)] is the cost of b sequences whose
 *               longest has l tokens, in any unit (e.g. ns).  Every entry
 *               >= 0 and every row non-decreasing in l (then contiguous
 *               batches of the length-sorted order are optimal over all
 *               partitions).  Read only during the call.
 *   order, batch_starts, n_batches, total_cost: as es_plan_batches, with the
 *               same tie rule (first minimising split point).
 * Errors: ES_ERR_ARG (NULL pointers, n < 0, max_tokens < 1, a table of
 * fewer than 1 or more than 2^28 entries, a negative, too large or falling
 * entry), ES_ERR_RANGE (a length < 1 or above max_tokens or max_len).
 */
es_status es_plan_batches_measured(const int32_t *lengths, int32_t n, int64_t max_tokens,
                                   const int64_t *cost_table, int32_t max_batch, int32_t max_len,
                                   int32_t *order, int32_t *batch_starts, int32_t *n_batches,
                                   int64_t *total_cost);

/*
 * es_pack_offsets -- host-only: offsets[0] = 0, offsets[k+1] = offsets[k] +
 * lengths[order[begin+k]] for k < end-begin (the packed layout of one batch).
 * offsets holds end-begin+1 entries.  Errors: ES_ERR_ARG (NULL, begin > end,
 * begin < 0), ES_ERR_RANGE (a length < 1 or a sum above INT32_MAX).
 */
es_status es_pack_offsets(const int32_t *lengths, const int32_t *order, int32_t begin,
                          int32_t end, int32_t *offsets);

/*
 * es_plan_arena -- host-only offset planning for tensors with lifetimes, the
 * placement rule of ES_MEM_LENGTH_AWARE: record i holds bytes[i] (>= 0) and
 * is used from step first_step[i] to last_step[i] (inclusive).  Records are
 * placed largest first (equal sizes: lower index first), each at the lowest
 * offset, a multiple of align (a power of two), where its bytes (rounded up
 * to align) overlap no placed record whose step interval meets its own.
 * offsets[i] receives the offset (0 for empty records), *total the arena size
 * max(offset + rounded bytes).  Errors: ES_ERR_ARG (NULL, n < 0, bad align,
 * negative bytes, first_step > last_step).
 */
es_status es_plan_arena(const int64_t *bytes, const int32_t *first_step, const int32_t *last_step,
                        int32_t n, int64_t align, int64_t *offsets, int64_t *total);

/*
 * es_check_plan -- host only (never touches HIP): build every pass's
 * metadata exactly as es_score_requests (n_prompts = 0: `lengths` are the n
 * request lengths) or es_score_best_of_n (n_prompts > 0: `lengths` are the n
 * candidate lengths, prompt_lengths[n_prompts] and cand_counts[n_prompts] as
 * there) would for a model with n_heads heads, the given mask and max_pos,
 * on a handle of max_tokens / max_seqs with batches_per_pass planned batches
 * per pass, and check every index in it against the buffer it addresses:
 * packed token offsets within the pass's rows, id sources within the id
 * buffer, reward slots in range and written once, score-block bases and
 * every softmax row's score elements within the pass's score buffer, and
 * attention, softmax and last-token work items covering every query tile and
 * score row exactly once.  *n_passes, *n_checked and *n_violations receive
 * the counts.  Errors: those of es_score_requests / es_score_best_of_n's
 * host validation, ES_ERR_ARG for a bad shape, ES_ERR_FORMAT when a check
 * fails (es_last_error names the first).
 */
es_status es_check_plan(const int32_t *lengths, int32_t n, const int32_t *prompt_lengths,
                        const int32_t *cand_counts, int32_t n_prompts, int32_t n_heads,
                        int32_t causal, int32_t max_pos, int64_t max_tokens, int32_t max_seqs,
                        int64_t batch_overhead, int32_t batches_per_pass, int64_t *n_passes,
                        int64_t *n_checked, int64_t *n_violations);

/* ------------------------------------------------------- single-kernel ops */
/*
 * The kernels of the hot path on caller buffers, for per-kernel parity tests
 * and bandwidth / MFMA measurement.  All enqueue on `stream`.
 */

/*
 * es_op_layernorm -- per-row LayerNorm (TurboTransformers review, Proposed
 * method: LayerNorm as a row "batch reduction"): for each of `rows` rows of
 * `cols` floats (row stride `cols`),
 *   y = (x - mean) / sqrt(var + eps) * gamma + beta,  var biased.
 * d_y float32[rows, cols] (may be NULL), d_ybf16 bf16[rows, ld_bf16] (may be
 * NULL; columns >= cols untouched).  cols must be a multiple of 4 and at most
 * 8192; d_x and d_y may alias.  Errors: ES_ERR_ARG.
 */
es_status es_op_layernorm(const float *d_x, const float *d_gamma, const float *d_beta,
                          int64_t rows, int32_t cols, float eps, float *d_y, uint16_t *d_ybf16,
                          int32_t ld_bf16, void *stream);

/*
 * es_op_add_layernorm -- residual connection and its LayerNorm in one pass
 * (the post-LN encoder layer: LayerNorm(x + sublayer(x)); TurboTransformers
 * review, Proposed method, for the row reduction): per row,
 *   s = x + sub,  y = (s - mean) / sqrt(var + eps) * gamma + beta,
 * with the sum rounded to float32 before the statistics, so the result is
 * bitwise es_op_layernorm of the float32 sum.  d_x and d_sub float32[rows,
 * cols]; d_y (may be NULL) may alias d_x or d_sub; d_ybf16 as in
 * es_op_layernorm.  The encoder's FFN output GEMM writes the sublayer term
 * and this op adds the residual (the GEMM then reads no residual).
 * Errors: ES_ERR_ARG.
 */
es_status es_op_add_layernorm(const float *d_x, const float *d_sub, const float *d_gamma,
                              const float *d_beta, int64_t rows, int32_t cols, float eps,
                              float *d_y, uint16_t *d_ybf16, int32_t ld_bf16, void *stream);

/*
 * es_ragged_create / es_ragged_free -- ragged attention-score layout of one
 * packed batch, uploaded to the current device once (synchronous; allocates)
 * so that es_op_softmax can be launched repeatedly without host work.
 *
 * For sequence i of length n_i (h_lengths[i], 1..4096) and head h < n_heads,
 * row q < n_i of the score block starts at element
 *     base_i + h * B_i + R_i(q),  base_0 = 0, base_{i+1} = base_i + n_heads * B_i,
 * with B_i = R_i(n_i).  Bidirectional (causal = 0): R_i(q) = q * ld_i,
 * ld_i = round_up(n_i, 8), and every row holds n_i scores.  Causal: the
 * lower triangle packed, row q holding q + 1 scores in round_up(q + 1, 8)
 * elements: R(q) = sum_{r<q} round_up(r + 1, 8) = 8 (t + 1)(4 t + s) for
 * q = 8 t + s.  *n_elems (may be NULL) receives base_{n_seqs}, the element
 * count the score buffers need.
 * Errors: ES_ERR_ARG (NULL, n_seqs < 1, n_heads < 1), ES_ERR_RANGE (a length
 * outside [1, 4096]), ES_ERR_HIP.
 */
typedef struct es_ragged es_ragged;
es_status es_ragged_create(const int32_t *h_lengths, int32_t n_seqs, int32_t n_heads,
                           int32_t causal, es_ragged **out, int64_t *n_elems);
void es_ragged_free(es_ragged *r);

/*
 * es_op_softmax -- per-row softmax over the ragged score layout of `r`
 * (TurboTransformers review, Proposed method: Softmax as a row "batch
 * reduction"):  p = exp(s - max) / sum exp(s - max)  over the valid scores
 * of every row, written to the same positions of d_p (bf16 bits if
 * p_bf16 = 1, else float32).  A row of m valid scores is written in chunks
 * of 8: positions m .. round_up(m, 8) - 1 of the row (still inside its
 * stride ld_i) receive 0; no other position is written.  Asynchronous;
 * allocates nothing.  Errors: ES_ERR_ARG.
 */
es_status es_op_softmax(const es_ragged *r, const float *d_scores, void *d_p, int32_t p_bf16,
                        void *stream);

/*
 * es_op_attention -- masked multi-head attention over the ragged layout of
 * `r` in one fused pass per query tile (TurboTransformers review, Proposed
 * method: the attention scores, their Softmax row reduction and the
 * context product; here the scores never leave registers): for sequence i,
 * head h, query q
 *     ctx[t0_i + q, h d + e] = sum_k softmax_k(scale * Q_q . K_k) V_k[e]
 * over keys k < n_i (causal = 1 in `r`: k <= q).  d_qkv: bf16 bits
 * [T, ld_qkv] row-major, T = sum of the lengths, packed in sequence order;
 * row t holds Q | K | V, each n_heads * head_dim wide, head h at columns
 * h * head_dim .. of each.  d_ctx: bf16 bits [T, ld_ctx], columns
 * [0, n_heads * head_dim) written, the rest untouched.  head_dim 32, 64 or
 * 128; ld_qkv >= 3 n_heads head_dim and a multiple of 8; ld_ctx >=
 * n_heads head_dim and a multiple of 4; scale > 0 (normally 1 / sqrt(d)).
 * Probabilities are rounded to bf16 before the context product, as in a
 * scoring pass.  Asynchronous; allocates nothing; the caller owns all
 * buffers.  Errors: ES_ERR_ARG, ES_ERR_HIP.
 */
es_status es_op_attention(const es_ragged *r, const uint16_t *d_qkv, int32_t ld_qkv,
                          int32_t head_dim, float scale, uint16_t *d_ctx, int32_t ld_ctx,
                          void *stream);

/*
 * es_op_gemm_bf16 -- C = epilogue(A W^T + bias) on bf16 MFMA, fp32 accumulate.
 *   d_a  bf16[rows >= round_up(M,256), lda]  (K columns used)
 *   d_w  bf16[rows >= round_up(N,256), K]    (row n = output feature n)
 *   d_bias float32[N]
 *   epilogue 0: out bf16 = acc + bias
 *            1: out bf16 = GELU(acc + bias)            (erf form; erfc by a Chebyshev
 *                                                       fit, fractional error < 1.2e-7)
 *            2: out fp32 = acc + bias + d_res[m, n]     (d_res fp32, ld ldc)
 *            3: out fp32 = acc + bias
 *   d_out [M, ldc] (bf16 for 0/1, fp32 for 2/3); only n < N, m < M written.
 * K must be a positive multiple of 64, lda >= K and a multiple of 8, ldc >= N and a
 * multiple of 4; d_bias, d_res and d_out 16-byte aligned.
 * Rows beyond M (A) and N (W) up to the rounded sizes are read, never used.
 * Errors: ES_ERR_ARG.
 */
es_status es_op_gemm_bf16(const uint16_t *d_a, int32_t lda, const uint16_t *d_w,
                          const float *d_bias, const float *d_res, void *d_out, int32_t ldc,
                          int32_t M, int32_t N, int32_t K, int32_t epilogue, void *stream);

/*
 * es_op_gemm_bf16_tile -- es_op_gemm_bf16 with the block-tile configuration
 * forced instead of chosen from the shape (for tests and tuning): tile -1 =
 * automatic, 0 = 128x64 register-staged, 1 = 128x128 ping-pong, 2 = 256x256
 * ping-pong, 3 = 128x384 ping-pong, 4 = 32x64 register-staged, 5 = 256x256
 * software-pipelined, 6 = 32x32 per wavefront with operands loaded straight
 * into registers.  Every configuration accumulates each output over K in the
 * same order, so all give bitwise the same result.
 * Errors: as es_op_gemm_bf16, and ES_ERR_ARG for a tile outside [-1, 6].
 */
es_status es_op_gemm_bf16_tile(const uint16_t *d_a, int32_t lda, const uint16_t *d_w,
                               const float *d_bias, const float *d_res, void *d_out, int32_t ldc,
                               int32_t M, int32_t N, int32_t K, int32_t epilogue, int32_t tile,
                               void *stream);

/* ------------------------------------------- last-token refinement kernels
 *
 * For pre-LN bf16 models the scoring entry points carry the last row of every
 * sequence (the one the reward reads: "Learning to summarize from human
 * feedback", Method adaptation) through the layers in fp32 beside the bf16
 * pass of all rows.  Its GEMMs take each fp32 activation a as the bf16 pair
 * hi = bf16(a), lo = bf16(a - hi) (round to nearest even both times; a - hi
 * is exact in fp32), two bf16 MFMAs into one fp32 accumulator: 16
 * significant bits, |a - hi - lo| <= 2^-16 |a|.  Those operands live in the
 * split-operand layout: for an fp32 matrix [M, K] (K a multiple of 16), rows
 * in tiles of 32 and columns in k-steps of 16, element (m, k) half h (0 hi,
 * 1 lo) at bf16 index
 *   ((((m / 32) (K / 16) + k / 16) 2 + h) 64 + ((k / 8) % 2) 32 + m % 32) 8 + k % 8,
 * 4 * 32 ceil(M / 32) * K bytes in all.  The four entry points below run the
 * refinement's kernels on caller buffers, for per-kernel parity tests;
 * asynchronous, they allocate nothing.
 */

/* es_op_split -- fp32 rows d_a [M, lda] (K columns; lda >= K, lda % 4 == 0,
 * 16-byte aligned) into the split-operand layout d_out; rows
 * [M, 32 ceil(M/32)) are written as zeros.  Errors: ES_ERR_ARG, ES_ERR_HIP. */
es_status es_op_split(const float *d_a, int32_t lda, int32_t M, int32_t K, uint16_t *d_out,
                      void *stream);

/* es_op_layernorm_split -- per-row LayerNorm (as es_op_layernorm, fp32
 * arithmetic) of d_x float32[rows, cols] (cols a multiple of 16) into the
 * split-operand layout d_out (rows past `rows` in the last tile untouched).
 * Errors: ES_ERR_ARG, ES_ERR_HIP. */
es_status es_op_layernorm_split(const float *d_x, const float *d_gamma, const float *d_beta,
                                int32_t rows, int32_t cols, float eps, uint16_t *d_out,
                                void *stream);

/* es_op_gemm_split -- epilogue(A W^T + bias), A [M, K] in the split-operand
 * layout (d_a, 32 ceil(M/32) rows read), W bf16 bits [N, K] row-major, K a
 * positive multiple of 64, fp32 accumulation.  epilogue 3: d_out fp32
 * [M, ldc] = acc + bias; 2: d_out = acc + bias + d_res[m, n] (d_res fp32
 * [M, ldc], may be d_out); 1: GELU(acc + bias) (erf form) into d_out_split
 * in the split-operand layout with K' = N (N a multiple of 16; rows past M
 * untouched).  Only m < M, n < N written.  Errors: ES_ERR_ARG, ES_ERR_HIP. */
es_status es_op_gemm_split(const uint16_t *d_a, const uint16_t *d_w, const float *d_bias,
                           const float *d_res, float *d_out, uint16_t *d_out_split, int32_t ldc,
                           int32_t M, int32_t N, int32_t K, int32_t epilogue, void *stream);

/* es_op_attention_last -- the attention of each sequence's last query in
 * fp32 over the ragged layout of `r` (Attention Is All You Need, Scaled
 * Dot-Product Attention; the last query sees every key of its sequence,
 * causal or not): for sequence i (rows t0_i .. t0_i + n_i - 1 of d_qkv) and
 * head h,  ctx_i[h d + e] = sum_k softmax_k(scale q . K_k) V_k[e]  with q,
 * and the last key and value, from row i of d_ql (fp32 [n_seqs, ld_ql],
 * Q | K | V as in d_qkv), the other keys and values from d_qkv (bf16 bits
 * [T, ld_qkv], ld_qkv a multiple of 8).  Row i of d_ctx_split, in the
 * split-operand layout with K = kc (>= n_heads d, a multiple of 16), gets
 * columns [0, n_heads d) and zeros in [n_heads d, kc).  head_dim 32, 64 or
 * 128; sequences of at most 1024 tokens.
 * Errors: ES_ERR_ARG, ES_ERR_RANGE (a longer sequence), ES_ERR_HIP. */
es_status es_op_attention_last(const es_ragged *r, const uint16_t *d_qkv, int32_t ld_qkv,
                               const float *d_ql, int32_t ld_ql, int32_t head_dim, float scale,
                               uint16_t *d_ctx_split, int32_t kc, void *stream);

/* ------------------------------------------------------------- profiling */

/* Kernel classes of the hot path, in launch order within a layer. */
enum {
  ES_KC_EMBED = 0, ES_KC_QKV = 1, ES_KC_SCORES = 2, ES_KC_SOFTMAX = 3, ES_KC_PV = 4,
  ES_KC_OPROJ = 5, ES_KC_LAYERNORM = 6, ES_KC_FFN1 = 7, ES_KC_FFN2 = 8, ES_KC_HEAD = 9,
  ES_KC_ATTN_FUSED = 10, ES_KC_GATHER = 11, ES_KC_REFINE = 12, ES_KC_COUNT = 13
};

typedef struct {
  int32_t kernel_class; /* ES_KC_*                                                */
  int32_t launches;     /* launches recorded since the last collect               */
  double total_ms;      /* sum of HIP-event durations around those launches       */
  double flops;         /* algorithmic flops of those launches (no padding)       */
  double bytes;         /* algorithmic HBM bytes (each operand read / written once) */
} es_kernel_stat_t;

/*
 * es_profile_enable -- from the next call on, record a HIP event pair on the
 * call's stream around every launch of the classes in `class_mask`
 * (bit ES_KC_x), together with that launch's algorithmic flops and bytes.
 * While enabled, the last-token refinement runs on the pass's stream, so
 * each recorded launch runs alone.  0 disables.  Clears earlier records.
 */
es_status es_profile_enable(es_model *m, uint32_t class_mask);

/*
 * es_profile_collect -- wait for the last recorded event, then fill
 * out[ES_KC_COUNT] with per-class totals and clear the records.
 */
es_status es_profile_collect(es_model *m, es_kernel_stat_t *out);

/* Name of a kernel class ("ffn1_gemm", ...), "" if out of range. */
const char *es_kernel_class_name(int32_t kernel_class);

/* Thread-local message describing the last error on this thread ("" if none). */
const char *es_last_error(void);

/* Library version string. */
const char *es_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ENCSCORE_H */
