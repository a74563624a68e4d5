/*
 * grw.h — C ABI of the wide-beam decode-step library for AMD Instinct MI355X (gfx950).
 *
 * One decode step of wide-beam generative recommendation:
 *   beam_select       trie-masked per-beam top_k, then the global beam_width-of-pool select
 *   beam_select_gumbel the same with Gumbel-perturbed ordering keys (temperature > 0)
 *   beam_select_logits the same from raw logits, with the row log-softmax fused in
 *   beam_select_ex     every selection option at once, with a dense-or-CSR trie
 *   beam_select_noalloc beam_select of one request with no workspace (allocates nothing)
 *   beam_attn_decode  beam attention over a shared prompt KV plus per-beam decode KV
 *                     reached through parent pointers, in three stages
 *                     (shared stage, unshared stage, online-softmax merge)
 *
 * Sources of the operations (cited by page title and section):
 *   xLLM "generative recommendation design" doc, section 4.1.1 (every beam expands top_k
 *   candidates; beam_width new beams are chosen from the beam_width x top_k pool),
 *   section 4.2.1 (prompt KV stored once and shared by all beams; decode-token KV per beam
 *   at token granularity, no block copy), section 4.2.2 (shared stage, unshared stage,
 *   OnlineSoftmax merge), section 4.3 (early termination of sorting, early filtering of
 *   invalid item paths, reuse of candidate containers), section 3.2 (multi-step execution
 *   with no per-step device-to-host round trip; buffers prepared once up front);
 *   FlashRec announcement in the SGLang beam-search PR thread (a fused semantic-ID trie,
 *   dense or CSR, so illegal IDs are never candidates).
 *
 * Conventions shared by every entry point
 *   - Return value: GRW_OK or an error code (grw_status_str gives its text).
 *   - Every tensor argument is caller-owned DEVICE memory unless stated otherwise; the
 *     library never frees it.  The library allocates device memory only in grw_ws_create
 *     (and pinned host staging there); it never allocates in any other call.
 *     beam_select_noalloc uses no workspace: its scratch is a static device array.
 *   - Every call that takes a stream enqueues its work on that stream and returns
 *     without synchronising and without any device-to-host copy, except grw_ws_bind_batch
 *     (one host-to-device upload of descriptors, then a stream synchronise) and
 *     grw_ws_error (synchronises to read the device flags).
 *   - Host-checkable argument errors return GRW_EINVAL / GRW_EUNSUPPORTED with nothing
 *     enqueued.  Device-side precondition violations (a parent or node id out of range,
 *     NaN or positive log-probabilities) do not stop the kernels; they set bits in a
 *     device flag word that grw_ws_error reports.
 *   - A workspace serves one stream at a time; calls on one workspace from two streams
 *     at once race.
 *   - Streams are hipStream_t passed as void* (NULL = the default stream).
 *
 * Indexing
 *   A batch holds R requests; request r owns beam slots [boff_r, boff_r + W_r) of
 *   sumW = sum_r W_r slots (boff_r = W_0 + ... + W_{r-1}).  Requests never mix: every
 *   selection and every attention read stays inside one request.
 */
#ifndef GRW_H
#define GRW_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct grw_ws grw_ws;

enum grw_status {
  GRW_OK = 0,
  GRW_EINVAL = 1,        /* bad argument (null pointer, size beyond a limit, mismatch)  */
  GRW_ENOMEM = 2,        /* an allocation failed (device or pinned host memory in
                            grw_ws_create; host memory in the host-side calls)            */
  GRW_EDEVICE = 3,       /* a HIP runtime call failed                                    */
  GRW_EUNSUPPORTED = 4,  /* valid but unsupported shape / dtype combination              */
  GRW_ESTATE = 5         /* call order: e.g. a step call before grw_ws_bind_batch        */
};

enum grw_dtype { GRW_F32 = 0, GRW_BF16 = 1, GRW_FP8_E4M3 = 2 };

/* device flag bits reported by grw_ws_error */
enum grw_device_flag {
  GRW_FLAG_NAN_LOGPROB = 1,     /* a NaN log-probability or beam score was seen            */
  GRW_FLAG_POS_LOGPROB = 2,     /* a log-probability > 0 was seen (breaks the early exit)   */
  GRW_FLAG_BAD_NODE = 4,        /* a live beam's trie node is outside [0, n_internal)       */
  GRW_FLAG_BAD_PARENT = 8,      /* a parent pointer walk left [0, W_r)                       */
  GRW_FLAG_CHILD_MISSING = 16,  /* a selected code is not a child of its parent's node      */
  GRW_FLAG_POOL_CORRUPT = 32,   /* internal check: a pool entry names a slot outside W_r    */
  GRW_FLAG_BAD_NOISE = 64       /* a Gumbel noise value of the sampled selection is not finite */
};

/*
 * Limits fixed at workspace creation; every later call is checked against them.
 *   max_requests     R of any bound batch
 *   max_total_beams  sumW of any bound batch
 *   max_W            beam_width of any request (<= 8192)
 *   max_K            top_k of any request (<= 2048)
 *   max_C            codes per level / vocabulary of beam_select
 *   max_S            decode steps (depth of parent_idx / unshared KV), <= 64
 *   max_P            prompt length of any request
 *   Hq, Hkv, D       query heads, kv heads (Hq % Hkv == 0, Hq/Hkv in {1,2,4}),
 *                    head dim; Hkv * D must be one of 128, 256, 512, 1024
 *   q_dtype          GRW_F32 or GRW_BF16
 *   kv_dtype         GRW_F32, GRW_BF16 or GRW_FP8_E4M3 (OCP E4M3 "fn")
 *   max_splits       partial-result slots of the shared stage's split over the prompt
 *                    (1..16; 0 means 8)
 */
typedef struct grw_limits {
  int32_t max_requests;
  int32_t max_total_beams;
  int32_t max_W;
  int32_t max_K;
  int32_t max_C;
  int32_t max_S;
  int32_t max_P;
  int32_t Hq, Hkv, D;
  int32_t q_dtype, kv_dtype;
  int32_t max_splits;
} grw_limits;

/* Allocate a workspace (all device buffers the step needs, sized by the limits).
   The workspace is bound to the device current at the time of the call. */
int grw_ws_create(const grw_limits* limits, grw_ws** out);
int grw_ws_destroy(grw_ws* ws);

/*
 * Bind a batch (setup, once per batch — not per step).
 *   W_host, K_host, P_host: HOST arrays [n_requests] of beam_width, top_k and prompt
 *   length per request.  Validated against the limits, then the per-request descriptors
 *   and the shared-stage work list are uploaded with one host-to-device copy; the call
 *   synchronises the stream before returning.
 */
int grw_ws_bind_batch(grw_ws* ws, int32_t n_requests, const int32_t* W_host,
                      const int32_t* K_host, const int32_t* P_host, void* stream);

/* Level-0 beam state for the bound batch: slot boff_r of every request gets score 0 and
   trie node 0 (the root); every other slot gets score -inf and node -1.
   beam_scores [sumW] float, beam_node [sumW] int32. */
int grw_beams_init(grw_ws* ws, float* beam_scores, int32_t* beam_node, void* stream);

/*
 * beam_attn_decode — attention of every beam slot of the bound batch at decode depth
 * `step`, for one layer (xLLM design doc, sections 4.2.1 and 4.2.2).
 *
 * For slot b of request r at depth d = step the beam's key/value sequence is the P_r
 * prompt tokens followed by its d + 1 decode tokens: the tokens of its ancestors at
 * depths 0..d-1 and its own token at depth d, found by walking parent pointers
 * (j_d = b, j_{e-1} = parent_idx[e][boff_r + j_e], request-local slot ids).
 * Output = softmax(q k^T / sqrt(D)) v per query head; query head h reads kv head
 * h / (Hq / Hkv).  A slot whose parent_idx[step][slot] is negative is dead: its output
 * row is zero.
 *
 * Three stages run on `stream`: the shared stage (each prompt KV tile streamed once per
 * beam group into LDS and reused by all of the request's beams, bf16 MFMA when D = 128
 * and q is bf16), the unshared stage (wavefronts walking each beam's parent pointers: one
 * per beam slot, or two when Hkv * D = 1024, each then taking half of the slot's kv heads),
 * and the online-softmax merge of their partial outputs and log-sum-exp statistics.
 *
 *   q          [sumW][Hq][D]  q_dtype
 *   k_shared   prompt keys of this layer, requests packed back to back: request r's block
 *              is [Hkv][Pp_r][D] at element offset Hkv*D*(Pp_0 + ... + Pp_{r-1}),
 *              Pp_r = P_r rounded up to a multiple of 64 (rows >= P_r are ignored and may
 *              hold any bits, NaN included)
 *   v_shared   prompt values of this layer, same packing, each block TRANSPOSED:
 *              [Hkv][D][Pp_r] (the PV contraction streams it without a transpose); columns
 *              >= P_r are ignored like the key rows
 *   k_scale, v_scale  [Hkv] float per-head scales (GRW_FP8_E4M3 only, else NULL); the
 *              value of an fp8 code is code * scale
 *   k_unshared, v_unshared  [>= step + 1][sumW][Hkv][D]  kv_dtype: the decode token of
 *              slot b at depth e is row [e][b]
 *   parent_idx [>= step + 1][sumW] int32, request-local parent slots; row 0 only marks
 *              dead slots (negative)
 *   out        [sumW][Hq][D] float32
 */
int beam_attn_decode(grw_ws* ws, const void* q, const void* k_shared, const void* v_shared,
                     const float* k_scale, const float* v_scale, const void* k_unshared,
                     const void* v_unshared, const int32_t* parent_idx, int32_t step,
                     float* out, void* stream);

/*
 * beam_attn_decode_stages — beam_attn_decode restricted to a subset of its stages, for
 * per-stage measurement and testing.  `stages` is a bit mask: GRW_STAGE_SHARED (1) runs the
 * shared stage (partials into the workspace), GRW_STAGE_UNSHARED (2) the unshared stage,
 * GRW_STAGE_MERGE (4) the merge into `out`.  The merge reads the partials the other two
 * stages last wrote into this workspace.  Mask 7 is beam_attn_decode.  Arguments and
 * errors as for beam_attn_decode; a mask outside 1..7 is GRW_EINVAL.
 */
enum grw_stage { GRW_STAGE_SHARED = 1, GRW_STAGE_UNSHARED = 2, GRW_STAGE_MERGE = 4 };
int beam_attn_decode_stages(grw_ws* ws, const void* q, const void* k_shared,
                            const void* v_shared, const float* k_scale, const float* v_scale,
                            const void* k_unshared, const void* v_unshared,
                            const int32_t* parent_idx, int32_t step, float* out,
                            int32_t stages, void* stream);

/*
 * beam_attn_decode_overlap — beam_attn_decode with the shared and unshared stages on two
 * streams (xLLM design doc, section 4.2.2: shared, unshared and merge placed on different
 * execution units and queues as a pipeline, the two stages overlapping, with as few
 * synchronisation points as possible).  The unshared stage runs on side_stream once the work
 * enqueued on `stream` before this call is done (one event), writing its partial into the
 * workspace; the shared stage runs on `stream`; the merge runs on `stream` after both (a
 * second event).  Work enqueued on `stream` afterwards sees `out` complete; side_stream needs
 * no synchronisation by the caller.  The two events belong to the workspace, so calls on one
 * workspace must not overlap each other.  The result equals beam_attn_decode_stages with
 * GRW_STAGE_SHARED, then GRW_STAGE_UNSHARED, then GRW_STAGE_MERGE, bit for bit.  Graph
 * capture of `stream` takes side_stream into the capture through the first event.
 * side_stream must differ from stream (GRW_EINVAL otherwise, and for a NULL side_stream);
 * other arguments and errors as for beam_attn_decode.
 */
int beam_attn_decode_overlap(grw_ws* ws, const void* q, const void* k_shared, const void* v_shared,
                             const float* k_scale, const float* v_scale, const void* k_unshared,
                             const void* v_unshared, const int32_t* parent_idx, int32_t step,
                             float* out, void* stream, void* side_stream);

/*
 * beam_select — one selection step for every request of the bound batch (xLLM design doc,
 * sections 4.1.1 and 4.3; FlashRec's trie-constrained expansion).
 *
 * For every live slot b (finite beam_scores[b]) of request r, the candidates are the
 * codes c of the CSR row of its trie node beam_node[b] (every c in [0, C) when the trie
 * pointers are NULL).  key(b, c) = fl32(beam_scores[b] + logprobs[b][c]); keys equal to
 * -inf are not candidates.  Each beam keeps its K_r best candidates, the request keeps
 * the W_r best of that pool; order is key descending, ties by flat index
 * (b - boff_r) * C + c ascending (+0.0 and -0.0 compare equal).  Output slot i of request
 * r (global slot boff_r + i) holds the i-th best: token c, parent (b - boff_r), score
 * key (the exact float32 sum), node = the child of beam_node[b] reached by c (-1 when
 * unconstrained).  If the pool holds n < W_r candidates, slots n..W_r-1 become pads
 * (token -1, parent -1, score -inf, node -1).
 *
 * Early exit (section 4.3): log-probabilities must be <= 0 (log_softmax output), so no
 * key exceeds its beam's score; a beam whose score is below a proven lower bound of the
 * W_r-th best key contributes nothing and is skipped.  The result is the same as
 * without the exit whenever the precondition holds (GRW_FLAG_POS_LOGPROB reports it).
 *
 *   logprobs     [sumW][C] float32, row-major
 *   beam_scores  [sumW] float32, beam_node [sumW] int32 (ignored when unconstrained)
 *   trie_row_ptr [n_internal + 1], trie_code [n_edges] int32: breadth-first node ids
 *                with the root 0, codes ascending within a row, the child reached through
 *                edge e is node e + 1; both NULL for unconstrained selection
 *   W, K         must equal the largest W_r and the largest K_r of the bound batch
 *   C            codes per level (<= max_C); (max W_r) * C must be < 2^32
 *   out_*        [sumW] each; out_parent may alias a row of parent_idx, out_score and
 *                out_node must not alias beam_scores / beam_node
 */
int beam_select(grw_ws* ws, const float* logprobs, const float* beam_scores,
                const int32_t* beam_node, const int32_t* trie_row_ptr,
                const int32_t* trie_code, int32_t trie_n_internal, int32_t W, int32_t K,
                int32_t C, int32_t* out_token, int32_t* out_parent, float* out_score,
                int32_t* out_node, void* stream);

/*
 * beam_select_gumbel — the sampled selection step: Gumbel top-k at a positive temperature
 * (FlashRec deployment guide, request section: temperature 0 is the deterministic top-k,
 * a positive temperature a Gumbel top-k whose noise only orders the candidates; the
 * returned sequence score holds no noise).
 *
 * Same candidates, tie rules, outputs and early exit as beam_select, except that every
 * top_k and beam_width decision orders candidate (b, c) by
 *   okey(b, c) = fl32(key(b, c) + fl32(temperature * noise[b][c]))
 * (two IEEE roundings, no fused multiply-add) in place of key(b, c); a candidate whose okey
 * is -inf is dropped.  out_score is still key(b, c), so the next step's beam scores carry
 * no noise.  With temperature 0 the result equals beam_select's.  The library draws no
 * random numbers: noise is the caller's, typically standard Gumbel draws -log(-log(u)).
 * Noise can lift an ordering key above its beam's score, so the score-based skip of whole
 * beams is off; the bound on the W_r-th best ordering key still prunes candidates.
 *
 *   noise        [sumW][C] float32, row-major like logprobs; must be finite
 *                (GRW_FLAG_BAD_NOISE reports a non-finite value)
 *   temperature  finite, >= 0 (else GRW_EINVAL, nothing enqueued)
 *   other arguments as for beam_select
 */
int beam_select_gumbel(grw_ws* ws, const float* logprobs, const float* noise, float temperature,
                       const float* beam_scores, const int32_t* beam_node,
                       const int32_t* trie_row_ptr, const int32_t* trie_code,
                       int32_t trie_n_internal, int32_t W, int32_t K, int32_t C,
                       int32_t* out_token, int32_t* out_parent, float* out_score,
                       int32_t* out_node, void* stream);

/*
 * beam_select_logits — the selection step from raw logits, with the log-softmax fused in
 * (the step upstream of the selection in the xLLM design doc's device loop, section 6:
 * forward, then sampling and beam search on the device).  Saves writing the log-probability
 * rows and reading them back.
 *
 * For every live slot b the log-softmax over all C codes of its row is taken first:
 *   lse_b = fl32(ln sum_c exp(logits[b][c])), evaluated in float64 as m + ln sum exp(x - m)
 *           with m the row max, rounded once;
 *   lp(b, c) = fl32(logits[b][c] - lse_b), one float32 subtraction;
 * then the selection proceeds exactly as beam_select on lp (or as beam_select_gumbel when
 * noise is not NULL).  lp <= 0 holds by construction, so the early exit is always valid.
 * Every row's lse is computed once, by one workgroup, into the workspace.
 *
 *   logits       [sumW][C] float32, row-major; finite or -inf, at least one finite logit in
 *                every live row (NaN or +inf raise GRW_FLAG_NAN_LOGPROB)
 *   noise        NULL for the deterministic selection, else as for beam_select_gumbel
 *   temperature  used with noise only: finite, >= 0 (else GRW_EINVAL, nothing enqueued)
 *   other arguments as for beam_select; out_score is beam_scores[b] + lp(b, c)
 */
int beam_select_logits(grw_ws* ws, const float* logits, const float* noise, float temperature,
                       const float* beam_scores, const int32_t* beam_node,
                       const int32_t* trie_row_ptr, const int32_t* trie_code,
                       int32_t trie_n_internal, int32_t W, int32_t K, int32_t C,
                       int32_t* out_token, int32_t* out_parent, float* out_score,
                       int32_t* out_node, void* stream);

/*
 * The trie of beam_select_ex: the CSR arrays of beam_select, and optionally a dense child
 * bit mask for some nodes (FlashRec announcement: the fused SID trie is dense or CSR).  The
 * CSR stays complete; a mask is another view of its node's row that lets the selection read
 * the node's log-prob row in full lines, which is cheaper than gathering its children when
 * the node has many.  All pointers are device memory.
 *   dense_slot  [n_internal] int32: index of the node's mask, or -1 (CSR only); NULL: none
 *   dense_mask  [n_dense][(C + 31) / 32] uint32: bit c % 32 of word c / 32 is set when code
 *               c is a child of the node (must agree with the CSR row; a code set here but
 *               missing from the CSR row that the selection keeps raises
 *               GRW_FLAG_CHILD_MISSING, and its output node is -1)
 */
typedef struct grw_trie {
  const int32_t* row_ptr;
  const int32_t* code;
  int32_t n_internal;
  const int32_t* dense_slot;
  const uint32_t* dense_mask;
} grw_trie;

/* Options of beam_select_ex. */
typedef struct grw_select_opts {
  const float* noise;       /* Gumbel noise [sumW][C] (as for beam_select_gumbel) or NULL */
  float temperature;        /* with noise: finite, >= 0 */
  int32_t raw_logits;       /* 1: the input holds raw logits (as for beam_select_logits) */
  int32_t first_step_fanout;  /* 1: first-step fan-out — only slot boff_r of each request
                                 expands (the other slots are ignored) and it keeps its top
                                 W_r candidates instead of top_k, so one prompt beam fills the
                                 whole beam set; for the first step, from the level-0 state of
                                 grw_beams_init.  A request wider than 2048 needs
                                 C <= W_r * top_k_r (its prompt row then passes whole
                                 through its pool); GRW_EUNSUPPORTED otherwise */
} grw_select_opts;

/*
 * beam_select_ex — the selection step with every option: trie given by a grw_trie (host
 * struct; NULL for unconstrained selection), and opts (host struct; NULL for the
 * deterministic selection from log-probabilities).  beam_select, beam_select_gumbel and
 * beam_select_logits are this call with a CSR-only trie and the corresponding options;
 * results do not depend on which nodes have dense masks.  opts->first_step_fanout selects
 * the first-step fan-out (FlashRec deployment guide, wide-beam section: the beam width sets
 * the width of the fused expansion of the prompt, k x n rows): the one live prompt beam of
 * each request is expanded to its best W_r children directly.  Arguments and errors
 * otherwise as for beam_select.
 */
int beam_select_ex(grw_ws* ws, const float* input, const float* beam_scores, const int32_t* beam_node,
                   const grw_trie* trie, const grw_select_opts* opts, int32_t W, int32_t K, int32_t C,
                   int32_t* out_token, int32_t* out_parent, float* out_score, int32_t* out_node,
                   void* stream);

/*
 * grw_trie_dense_build — host-side: dense child masks for the nodes of a CSR trie with at
 * least min_fanout children.  All arguments are host memory.  Writes dense_slot[n_internal]
 * (mask index or -1) and *n_dense; with dense_mask non-NULL also the masks
 * [n_dense][(C + 31) / 32] (call once with dense_mask NULL to size it).  GRW_EINVAL for
 * NULL arguments, a decreasing row_ptr or a code outside [0, C).
 */
int grw_trie_dense_build(const int32_t* row_ptr, const int32_t* code, int32_t n_internal, int32_t C,
                         int32_t min_fanout, int32_t* dense_slot, uint32_t* dense_mask, int32_t* n_dense);

/*
 * grw_plan_batches — host-side slot-budget batching (FlashRec announcement: scheduling by a
 * beam-row slot budget, so that the rows of several requests share one step; FlashRec
 * deployment guide, wide-beam section: the slot count bounds how many wide requests run
 * together).  Packs a queue of n requests with beam widths W[0..n) into batches whose total
 * beam rows stay within slot_budget and which hold at most max_requests requests each.
 * Policy: first fit in queue order — request i joins the lowest-numbered batch that still
 * has room for it (rows and request count), else opens the next batch; batches are numbered
 * in the order they open and keep their requests in queue order.  Each batch is one
 * grw_ws_bind_batch of a workspace created with max_total_beams >= slot_budget and
 * max_requests >= max_requests.
 *   W         [n] int32 host, each in [1, slot_budget]
 *   batch_of  [n] int32 host, written: batch index of each request
 *   n_batches int32 host, written: the number of batches (0 for n == 0)
 * GRW_EINVAL for n < 0, NULL pointers (W and batch_of may be NULL when n == 0),
 * slot_budget < 1, max_requests < 1, or a width outside [1, slot_budget]; GRW_ENOMEM when
 * its host working memory (about 12 bytes per request) cannot be allocated.  O(n log n).
 */
int grw_plan_batches(int32_t n, const int32_t* W, int32_t slot_budget, int32_t max_requests,
                     int32_t* batch_of, int32_t* n_batches);

/*
 * grw_backtrack — the semantic-ID tuple of every final beam (xLLM design doc, section
 * 4.1.1: the item id is the fixed-length sequence of generated tokens).
 *   tokens, parents  [S][sumW] int32, the out_token / out_parent of steps 0..S-1
 *   sid_out          [sumW][S] int32; sid_out[b][d] is the code chosen at depth d on the
 *                    path of final slot b (all -1 for a pad slot)
 */
int grw_backtrack(grw_ws* ws, const int32_t* tokens, const int32_t* parents, int32_t S,
                  int32_t* sid_out, void* stream);

/* Synchronise the workspace's last stream and report (then clear) the device flag word
   (grw_device_flag bits) in *flags (host pointer). */
int grw_ws_error(grw_ws* ws, void* stream, int32_t* flags);

/* Number of partial-result splits the shared stage uses for request r of the bound batch
   (diagnostics; host-side, no device work). */
int grw_ws_splits(const grw_ws* ws, int32_t r, int32_t* n_splits);

/* Size of request r's candidate pool after the last beam_select call: the survivors its
   beams kept, after the per-beam top_k and the early-exit bound (xLLM design doc, section
   4.1.1 for the beam_width x top_k pool, section 4.3 for stopping early).  Synchronises
   the stream, then writes the count to *pool_size (host pointer).  Diagnostics only. */
int grw_ws_pool_size(grw_ws* ws, int32_t r, void* stream, int64_t* pool_size);

/* Bound on how long a beam workgroup of the fused pilot + per-beam selection kernel polls
   for its request's bound (the kernel used when every row has at most 8192 codes and
   W <= 1024): at most `polls` polls (default 262144, a fraction of a second).  A workgroup
   that gives up proceeds with no bound: it admits every candidate of its row and leaves a
   row with more than top_k of them to the W-of-pool stage, so the result is the same, only
   slower.  For tests of that fallback (polls = 0 forces it) and for callers that want a
   tighter bound on the wait.  Host-side; affects later beam_select* calls on this
   workspace.  GRW_EINVAL if polls < 0. */
int grw_ws_set_wait_limit(grw_ws* ws, int32_t polls);

/*
 * beam_select_noalloc — for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): beam_select of ONE request
 * with no workspace.  It calls no hipMalloc / hipFree and no allocating library routine; its
 * scratch (request descriptor, slot map, pilot descriptors and buffer, candidate pool with
 * CSR edges, survivor counts, bound, step words, flag word: about 3.2 MiB) is a static
 * device array of the library, which every GPU the library runs on holds until the process
 * ends.  The caller passes inputs and outputs only.
 *
 * Limits: 1 <= W <= 1024, 1 <= K, W * K <= 262144 (the W = K = 512 pool), 1 <= C <= 8192;
 * sizes beyond them return GRW_EUNSUPPORTED, other argument errors GRW_EINVAL, both with
 * nothing enqueued.  The selection, its tie rules, outputs and early exit are those of
 * beam_select for a batch of one request (boff = 0, so out_parent holds slots 0..W-1).
 * Each call first clears the scratch words that must start at zero (with a kernel, so a
 * captured graph replays it), so consecutive calls of any sizes are independent.  Calls on
 * one GPU share that GPU's array and the array keeps the last call's contents: calls that
 * overlap on one GPU (two streams, two threads) race.
 *   logprobs     [W][C] float32; beam_scores [W]; beam_node [W] (ignored when unconstrained)
 *   trie_*       as for beam_select (both NULL for unconstrained selection)
 *   out_*        [W] each, as for beam_select
 *   device_flags [1] int32 device word that device precondition flags (grw_device_flag bits)
 *                are OR'd into; NULL: they go to the library's own word in the scratch,
 *                which the call clears and nothing reads
 */
int beam_select_noalloc(const float* logprobs, const float* beam_scores, const int32_t* beam_node,
                        const int32_t* trie_row_ptr, const int32_t* trie_code, int32_t trie_n_internal,
                        int32_t W, int32_t K, int32_t C, int32_t* out_token, int32_t* out_parent,
                        float* out_score, int32_t* out_node, int32_t* device_flags, void* stream);

/* Self-check of the device's wave primitives: the register lane exchanges (DPP quad, row and
   wave controls, v_permlane16/32_swap), wave scans and reductions that the selection and
   attention kernels use, each compared bit for bit with the general shuffle it replaces, on
   one workgroup of 256 threads.  `scratch` is a device buffer of at least GRW_SELFTEST_WORDS
   int32 words owned by the caller (overwritten).  Enqueues on `stream`,
   synchronises it, and writes the number of (check, thread) pairs that disagree to
   *mismatches (host pointer): 0 on a correct build and device.  NULL scratch or mismatches:
   GRW_EINVAL with nothing enqueued.  Diagnostics only. */
#define GRW_SELFTEST_WORDS 3584
int grw_selftest_lanes(int32_t* scratch, void* stream, int32_t* mismatches);

const char* grw_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GRW_H */
