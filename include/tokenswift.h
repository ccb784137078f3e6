/*
 * tokenswift.h -- C ABI of the MI355X (gfx950) hot-path library libtokenswift.so.
 *
 * The library runs the per-step, data-parallel work of TokenSwift-style
 * lossless ultra-long generation on one GPU: tree-masked verification
 * attention over the full KV cache, draft attention over the partial cache,
 * the dynamic partial-KV update, the contextual-penalty logit pass, the
 * acceptance of the verified tree with its KV commit, and the n-gram draft
 * tree.
 *
 * Citations name pages and sections, not files:
 *   "TokenSwift summary"  = the paperlayer.ai source-linked summary of
 *                           "TokenSwift: Lossless Acceleration of Ultra Long
 *                           Sequence Generation" (arXiv 2502.18890v2);
 *                           section numbers are the paper's.
 *   "Reproducibility checklist" = the acmrep2026 page on the same paper.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Pointers are caller-owned DEVICE memory unless marked (host). The library
 *   never allocates, frees or synchronises device memory and keeps no mutable
 *   global state except a per-device property cache; calls on different
 *   streams may run concurrently as long as their buffers do not overlap.
 * - bf16 tensors are passed as uint16_t bit patterns.
 * - A KV cache element (g, j, c) -- KV head g, cache row j, channel c -- sits
 *   at  base[g * s_head + j * s_pos + c]  (strides in elements; channels
 *   contiguous). d <= s_pos <= 2^23; s_head >= rows * s_pos is not required but the
 *   rows of different heads must not overlap. Base pointers and strides must
 *   keep every row 16-byte aligned.
 * - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = the
 *   default stream) and runs asynchronously; the return code reports only
 *   host-side validation and launch errors.
 * - Every argument is validated on the host BEFORE anything is launched; on
 *   error nothing is enqueued, outputs are untouched, and ts_last_error()
 *   returns a message for the calling thread.
 * - Workspace: each entry point has a *_workspace_size() query that depends
 *   on shapes only (no device needed). Pass at least that many bytes, 256-byte
 *   aligned. Workspace contents need not be initialised and are scratch. The
 *   selection calls leave a histogram in their workspace at zero for the
 *   next call: a workspace reused from such a call (or zero-filled once)
 *   saves the first call a recount of each KV head's scores.
 */
#ifndef TOKENSWIFT_H
#define TOKENSWIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define TS_OK          0
#define TS_EINVAL     (-1) /* null pointer, bad stride/alignment/shape/parameter, bad parent[] */
#define TS_ENOTSUP    (-2) /* a shape the kernels do not handle (d not 64/128, T > 128, ...)  */
#define TS_EWORKSPACE (-3) /* workspace smaller than the *_workspace_size() query            */
#define TS_EHIP       (-4) /* the HIP runtime reported an error while launching               */

/* Largest tree / draft-chain size: two 64-bit ancestor words per node. */
#define TS_MAX_TREE 128

/*
 * ts_verify_attn -- tree-masked verification attention over the FULL cache.
 *
 * TokenSwift summary §3.1 (with Figure 2): the target model checks the whole
 * draft in one forward pass using the full KV cache; Appendix E "Tree-Based
 * Attention": the draft is a tree of candidate continuations and each tree
 * token attends only to its predecessors; §3.3: under GQA the query heads of
 * one KV head form a group.
 *
 * For every query head h (KV head g = h / (Hq/Hkv)) and tree node i:
 *   out[h][i][:] = sum_{j in Vis(i)} softmax_j(scale * q[h][i] . k[g][j]) * v[g][j]
 *   Vis(i) = committed rows 0..n_ctx-1  U  {n_ctx + a : a is i or an ancestor of i}
 *
 *   q       [Hq][T][d] bf16, contiguous.
 *   k, v    caches (layout above) holding n_ctx committed rows followed by the
 *           T tree nodes' own keys/values at rows n_ctx..n_ctx+T-1 (the caller
 *           writes them before the call, as in any decode step).
 *   parent  (host) [T] int32: parent[0] = -1 (root), 0 <= parent[i] < i.
 *   Hq, Hkv Hq % Hkv == 0.      d: 64 or 128.      1 <= T <= 128.  n_ctx >= 0.
 *   scale   softmax scale; <= 0 selects 1/sqrt(d).
 *   out     [Hq][T][d] float32, contiguous (row (h, i) at (h*T + i)*d).
 *   n_split number of cache chunks per KV head processed in parallel before
 *           a log-sum-exp merge; 0 = automatic. Results agree for every value
 *           up to float rounding.
 *   ws      workspace of ts_verify_attn_workspace_size(...) bytes.
 *
 * Precision: q.k in bf16 x bf16 with float32 accumulation; softmax in
 * float32; probabilities and v enter the p.v product as float16 with float32
 * accumulation. Every bf16 value of v up to 65280 in magnitude is exact in
 * float16; a value of 65536 or more (beyond the float16 range) converts to
 * +-inf, so the output rows that see it come out non-finite in that channel
 * (never a silently clamped value). The call still returns TS_OK: the
 * library does not scan v.
 */
int ts_verify_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t T,
                   const int32_t* parent, int32_t Hq, int32_t Hkv, int32_t d,
                   float scale, float* out, int32_t n_split,
                   void* ws, size_t ws_bytes, void* stream);

size_t ts_verify_attn_workspace_size(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv,
                                     int32_t d, int32_t n_split);

/*
 * ts_verify_attn_noalloc -- ts_verify_attn with no workspace argument, for
 * callers that cannot allocate device memory around the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The split partials go to a scratch array the library holds in device
 * memory (one copy per device, from the library's load until the process
 * ends, ts_verify_attn_noalloc_max_scratch() bytes); the call itself
 * allocates nothing. Every argument and the output as for ts_verify_attn;
 * the output is bitwise what ts_verify_attn writes for the same arguments.
 * A call whose ts_verify_attn_workspace_size(...) exceeds the scratch size
 * returns TS_EWORKSPACE (use ts_verify_attn with a workspace then).
 * All calls on one device share its scratch array: calls that may overlap
 * on one device (different streams without ordering) race and must not be
 * made; calls ordered on one stream are fine. Nothing in the scratch array
 * needs to start at zero.
 */
int ts_verify_attn_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t T,
                           const int32_t* parent, int32_t Hq, int32_t Hkv, int32_t d,
                           float scale, float* out, int32_t n_split, void* stream);

/* Bytes of the scratch array behind ts_verify_attn_noalloc (per device). */
size_t ts_verify_attn_noalloc_max_scratch(void);

/*
 * ts_verify_attn_scored -- ts_verify_attn that also writes the grouped key
 * scores of the committed rows, summed from the query-key products the
 * attention already forms (no second pass over the keys).
 *
 * TokenSwift summary §3.3 "Dynamic KV Cache Management": a cached pair's
 * importance is a query-key dot product and, under GQA, the products of the
 * query heads of a group are added; when the partial cache is refreshed with
 * the queries of the verification step, those are exactly the products of
 * this pass.
 *
 *   scores  [Hkv][n_ctx] float32 output (row j of head g at g*n_ctx + j):
 *           scores[g][j] = sum_{h in group g} sum_{i<T} q[h][i] . k[g][j]
 *           for j < n_ctx: raw products (no softmax scale, no tree mask),
 *           the same sigma as ts_partial_kv_select with the same q.
 *   Every other argument and output as for ts_verify_attn (same workspace
 *   query); `out` is bitwise what ts_verify_attn writes for the same call.
 *   The (Hq/Hkv)*T query rows of a KV head must fit one workgroup: at most
 *   256, else TS_ENOTSUP (use ts_partial_kv_select for the scores then).
 *
 * Precision: bf16 x bf16 products with float32 accumulation, summed over the
 * rows in float32 (in another order than ts_partial_kv_select's).
 */
int ts_verify_attn_scored(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t T,
                          const int32_t* parent, int32_t Hq, int32_t Hkv, int32_t d,
                          float scale, float* out, float* scores, int32_t n_split,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * ts_draft_attn -- draft attention over the PARTIAL cache.
 *
 * TokenSwift summary §3.1 and §3.3: drafting runs the target model with a
 * partial KV cache of fixed budget. The Tq new tokens of a drafting pass form
 * a chain: token t sees the n_part partial rows and its own rows
 * n_part..n_part+t. This is ts_verify_attn with parent[t] = t-1.
 *
 *   q               [Hq][Tq][d] bf16.
 *   k_part, v_part  partial caches (layout above; strides s_head, s_pos) with
 *                   n_part rows then the Tq new tokens' rows.
 *   1 <= Tq <= 128.  Other arguments as for ts_verify_attn.
 */
int ts_draft_attn(const uint16_t* q, const uint16_t* k_part, const uint16_t* v_part,
                  int64_t s_head, int64_t s_pos, int32_t n_part, int32_t Tq,
                  int32_t Hq, int32_t Hkv, int32_t d, float scale, float* out,
                  int32_t n_split, void* ws, size_t ws_bytes, void* stream);

size_t ts_draft_attn_workspace_size(int32_t n_part, int32_t Tq, int32_t Hq, int32_t Hkv,
                                    int32_t d, int32_t n_split);

/*
 * ts_partial_kv_select -- dynamic partial-KV update: score, select, gather.
 *
 * TokenSwift summary §3.3 "Dynamic KV Cache Management" (and §2): the
 * drafting cache has a fixed budget, always keeps the initial |S| pairs, and
 * replaces less important pairs as generation proceeds; importance is a
 * query-key dot product, and under GQA the queries of a group are kept apart
 * (keys are not replicated) and their scores added up.
 *
 *   score   sigma[g][j] = sum_{h in group g} sum_{t<T} q[h][t] . k[g][j]
 *           for committed rows j < n_ctx (float32 accumulation).
 *   C       candidates = rows [n_sink, n_ctx - n_recent) (empty if n_ctx <=
 *           n_sink + n_recent). B' = min(budget, |C|).
 *   select  per KV head, the B' candidates first in (score desc, row asc).
 *   sel_idx [Hkv][budget] int32: selected rows, ascending, then -1 padding.
 *   gather  partial rows = [0, min(n_sink, n_ctx)) U selected U
 *           [max(n_sink, n_ctx - n_recent), n_ctx), ascending; row r of the
 *           partial cache of head g (k_part/v_part, strides sp_head, sp_pos)
 *           receives that row's key and value.
 *   n_part_out (host) receives the number of partial rows (the same for every
 *           head); it is computed on the host from the scalars.
 *   scores  optional [Hkv][n_ctx] float32 output of sigma (NULL = not written).
 *
 *   q [Hq][T][d] bf16 contiguous, 1 <= T <= 128; d 64 or 128; n_sink, budget,
 *   n_recent >= 0. The partial cache must not overlap the full cache.
 */
int ts_partial_kv_select(const uint16_t* q, int32_t T, const uint16_t* k, const uint16_t* v,
                         int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t Hq, int32_t Hkv,
                         int32_t d, int32_t n_sink, int32_t budget, int32_t n_recent,
                         int32_t* sel_idx, uint16_t* k_part, uint16_t* v_part,
                         int64_t sp_head, int64_t sp_pos, int32_t* n_part_out, float* scores,
                         void* ws, size_t ws_bytes, void* stream);

size_t ts_partial_kv_select_workspace_size(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv,
                                           int32_t d, int32_t budget);

/*
 * ts_partial_kv_rows -- the number of partial-cache rows (n_part) that
 * ts_partial_kv_select and ts_partial_kv_select_scored write for these
 * scalars: min(n_sink, n_ctx) + B' + the recent rows (TokenSwift summary
 * §3.3: the initial pairs, the selected pairs, and the latest ones). A shape
 * query (no device); the partial caches k_part / v_part must hold at least
 * this many rows per head. Returns -1 when an argument is negative.
 */
int32_t ts_partial_kv_rows(int32_t n_ctx, int32_t n_sink, int32_t budget, int32_t n_recent);

/*
 * ts_partial_kv_select_scored -- the select and gather steps of
 * ts_partial_kv_select on scores the caller provides (for instance those
 * ts_verify_attn_scored wrote in the same step), so no query or key pass runs.
 *
 * TokenSwift summary §3.3 "Dynamic KV Cache Management" (as for
 * ts_partial_kv_select).
 *
 *   scores  [Hkv][n_ctx] float32, read only (row j of head g at g*n_ctx + j);
 *           only the candidate rows are read.
 *   C, B', the selection order, sel_idx, the gather into k_part / v_part and
 *   n_part_out (host) exactly as for ts_partial_kv_select, with sigma = scores.
 *   ws      ts_partial_kv_select_scored_workspace_size(...) bytes.
 */
int ts_partial_kv_select_scored(const float* scores, const uint16_t* k, const uint16_t* v,
                                int64_t s_head, int64_t s_pos, int32_t n_ctx, int32_t Hkv,
                                int32_t d, int32_t n_sink, int32_t budget, int32_t n_recent,
                                int32_t* sel_idx, uint16_t* k_part, uint16_t* v_part,
                                int64_t sp_head, int64_t sp_pos, int32_t* n_part_out,
                                void* ws, size_t ws_bytes, void* stream);

size_t ts_partial_kv_select_scored_workspace_size(int32_t n_ctx, int32_t Hkv, int32_t d,
                                                  int32_t budget);

/*
 * ts_penalty_sample -- contextual penalty, temperature, min-p and top-p.
 *
 * TokenSwift summary §3.4: a repetition penalty restricted to the tokens of
 * the most recent W positions; Appendix D.1: top-p samples from the shortest
 * probability-ordered head of the vocabulary with mass above top_p, min-p
 * from the tokens at or above min_p * max p; Reproducibility checklist,
 * Table 11: penalty 1.2, penalty length 1024, temperature 1.0, top-p 0.9,
 * min-p 0.05.
 *
 * Per row r of logits [rows][V] float32:
 *   1. for each DISTINCT id w of window[r] with 0 <= w < V (other ids are
 *      padding): x_w <- x_w / penalty if x_w > 0, else x_w * penalty;
 *   2. z = x / temperature  -> logits_out (may alias logits);
 *   3. p = softmax(z);
 *   4. keep_top(i) <=> mass of the tokens before i in (p desc, id asc) order
 *      <= top_p;  keep_min(i) <=> p_i >= min_p * max(p);  keep = both;
 *   5. probs = p * keep / sum(p * keep)          (optional output);
 *   6. token = smallest id t with sum_{i<=t} probs_i > u[r]  (optional; needs u).
 *
 *   window  [rows][W] int32 with row stride window_stride, or one row shared by
 *           every row when window_stride == 0. W may be 0.
 *   penalty > 0, temperature > 0, 0 <= top_p <= 1, 0 <= min_p <= 1.
 *   keep    [rows][V] uint8 (1 = kept) or NULL.    probs [rows][V] float32 or NULL.
 *   u       [rows] float32 in [0, 1) or NULL.       token [rows] int32 or NULL
 *           (token requires u).
 *   1 <= V <= 262144; rows >= 1.
 */
int ts_penalty_sample(const float* logits, int32_t rows, int32_t V,
                      const int32_t* window, int32_t W, int64_t window_stride,
                      float penalty, float temperature, float top_p, float min_p,
                      float* logits_out, uint8_t* keep, float* probs,
                      const float* u, int32_t* token,
                      void* ws, size_t ws_bytes, void* stream);

size_t ts_penalty_sample_workspace_size(int32_t rows, int32_t V);

/*
 * ts_penalty_sample_eta -- the same pass with eta-sampling in place of top-p
 * and min-p.
 *
 * TokenSwift summary Appendix D.1: eta-sampling's pool is the tokens whose
 * probability reaches eta, a quantity built from the distribution's entropy
 * and two constants alpha and epsilon; §D.2 reports TokenSwift under it.
 * Here eta = min(epsilon, alpha * exp(-H)), H = -sum_i p_i ln p_i (nats), and
 * the most probable token always stays:
 *   keep(i) <=> p_i >= min(eta, max p);
 * steps 1-3, 5 and 6 as for ts_penalty_sample.
 *
 *   0 < epsilon <= 1; alpha >= 0 and finite (alpha = 0 keeps every token).
 *   Other arguments, outputs and the workspace as for ts_penalty_sample.
 */
int ts_penalty_sample_eta(const float* logits, int32_t rows, int32_t V,
                          const int32_t* window, int32_t W, int64_t window_stride,
                          float penalty, float temperature, float epsilon, float alpha,
                          float* logits_out, uint8_t* keep, float* probs,
                          const float* u, int32_t* token,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * ts_tree_accept -- the accepted path of a verified token tree.
 *
 * TokenSwift summary §3.1 (with Figure 2): after the target model verifies
 * the drafted tree, the longest valid draft is accepted; Appendix A "Lossless
 * Nature of Speculative Decoding": acceptance and rejection together keep
 * the target model's sampling distribution.
 *
 * A child c of node p continues a valid draft iff node_token[c] equals
 * target[p], the target model's token at node p (its draw from the processed
 * distribution at p, e.g. ts_penalty_sample's token for that node's row, or
 * the argmax when decoding greedily). Every emitted token is then the
 * target's own draw, so the output is distributed as the target's. The path
 * ends at the deepest node all of whose edges from the root are valid (ties:
 * the smaller node index); node 0 (the root) is always accepted.
 *
 *   parent      (host) [T] int32, a tree listed parents-first as for
 *               ts_verify_attn.   1 <= T <= 128.
 *   node_token  [T] int32: the token of each node (node 0's is not read).
 *   target      [T] int32: the target model's token at each node.
 *   result      [T + 2] int32 output: result[0] = n = m + 1 nodes accepted,
 *               result[1] = target[a_m] (the next token, emitted after the
 *               accepted ones), result[2 .. 2+n) = a_0 = 0 < a_1 < ... < a_m,
 *               result[2+n .. 2+T) = -1.
 * Two waves; no workspace. The host learns n only by reading result[0].
 */
int ts_tree_accept(const int32_t* parent, int32_t T, const int32_t* node_token,
                   const int32_t* target, int32_t* result, void* stream);

/*
 * ts_kv_commit -- commit an accepted path into the full and partial caches.
 *
 * TokenSwift summary §3.1 (with Figure 2): after acceptance the accepted
 * tokens' keys and values join the KV cache; §3.3: drafting continues on the
 * partial cache, so they are appended to it as well.
 *
 * For every layer l and KV head g, with a_0..a_m the path in result (as
 * written by ts_tree_accept for the same T):
 *   row n_ctx + k of the full cache <- row n_ctx + a_k   (k = 0..m)
 *   row n_part + k of the partial cache <- the same row  (if k_part given)
 * Rows n_ctx + m + 1 .. n_ctx + T - 1 keep their contents; nothing else is
 * touched. The moves are done as a gather (all accepted rows are read before
 * any is written), so overlapping source and destination rows are fine.
 *
 *   k, v        full caches of `layers` layers: element (l, g, j, c) at
 *               l*s_layer + g*s_head + j*s_pos + c (layers and heads must not
 *               overlap), holding the tree rows n_ctx .. n_ctx+T-1.
 *   k_part, v_part  partial caches with strides sp_layer, sp_head, sp_pos, or
 *               both NULL; they hold part_rows rows per head, of which the
 *               first n_part are in use: n_part + T <= part_rows.
 *   d 64 or 128; 1 <= layers, Hkv <= 65535. One launch for all layers.
 */
int ts_kv_commit(const int32_t* result, int32_t T, uint16_t* k, uint16_t* v,
                 int64_t s_layer, int64_t s_head, int64_t s_pos, int32_t layers,
                 int32_t Hkv, int32_t d, int32_t n_ctx,
                 uint16_t* k_part, uint16_t* v_part, int64_t sp_layer, int64_t sp_head,
                 int64_t sp_pos, int32_t n_part, int32_t part_rows, void* stream);

/*
 * ts_ngram_tree -- n-gram retrieval, random n-gram choice and the draft tree.
 *
 * TokenSwift summary §3.2 "Multi-token Generation and Token Reutilization":
 * frequent 4-grams of the generated text are reused as draft candidates, at
 * most k of them (k = 20 in the reproducibility checklist's Table 11); §3.4:
 * a random choice among several valid n-grams keeps the output diverse;
 * §4.4.1 and Appendix B.2: the tree is a simple ternary [1,3,3,3] tree of the
 * draft heads' candidates, merged with the n-grams.
 *
 * The n-gram table is the multiset of 4-grams lying in `window` (the last W
 * committed tokens; the root is window[W-1]). A 4-gram is valid iff its first
 * token is the root; valid 4-grams are counted per distinct continuation
 * (the last three tokens), numbered q = 0, 1, ... by first occurrence. If more
 * than k are valid, the k with the smallest (r_q, q) are kept, r_q = output q
 * of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) started from state
 * `seed`: a uniformly random subset. Kept chains are ordered by count
 * (descending), then first occurrence.
 * Tree: node 0 = root; for level l = 1..levels, nodes 3(l-1)+1 .. 3l carry
 * head_cand[l-1][0..2] under node 0 (l = 1) or under node 3(l-2)+1; then each
 * kept chain (a, b, c) adds three nodes in a line under node 0. Nodes past
 * T_max are cut off.
 *
 *   window      [W] int32, 1 <= W <= 4096.     k >= 0.     seed: any.
 *   head_cand   [levels][3] int32 (NULL when levels == 0); 0 <= levels <= 3.
 *   T_max       1 <= T_max <= 128.
 *   parent, node_token  [T_max] int32 outputs (parents-first tree as
 *               ts_verify_attn takes it); slots past T hold -1.
 *   info        [4] int32 output: T (nodes), chains with a node in the tree,
 *               distinct valid continuations, valid occurrences.
 * One workgroup; no workspace. parent and T reach the host by a copy.
 */
int ts_ngram_tree(const int32_t* window, int32_t W, int32_t k, uint64_t seed,
                  const int32_t* head_cand, int32_t levels, int32_t T_max,
                  int32_t* parent, int32_t* node_token, int32_t* info, void* stream);

/* Message for the last non-zero return on the calling thread ("" if none). */
const char* ts_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int ts_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TOKENSWIFT_H */
