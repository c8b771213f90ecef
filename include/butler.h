/*
 * butler.h -- C ABI of libbutler, query-aware sparse decode for AMD MI355X (gfx950).
 *
 * The method (TokenButler, "Meta-Llama-3.1-8B-Instruct-Butler" model card, section
 * Method; TokenSelect README, highlights):
 *   producer layers 0, G, 2G, ... turn LN(H) into low-dimensional importance queries
 *   Q_imp = f_theta(LN(H)); every layer projects its cached post-RoPE keys to
 *   K_imp = K . W_K; a consumer layer scores every cached token with its slot of Q_imp
 *   against K_imp (or, TokenSelect style, with per-head softmax-normalised Q.K summed
 *   over the heads of a GQA group), keeps a fixed budget of top-x tokens plus a sink
 *   prefix and a recent window, and attends over that set only.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer owned by the caller (the one exception:
 *     butler_fetch_rows also reads a cache in pinned host memory).  The library never
 *     allocates or frees device memory, keeps no pointer after returning and never
 *     synchronises: all work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream).  Buffers must stay alive until the stream has passed the enqueued work.
 *   - Tensors are dense, row-major, innermost dimension contiguous, with the shapes
 *     given below.  Cache tensors are allocated with a token capacity L_cap >= L.
 *     Every tensor pointer must be 16-byte aligned.
 *   - dtype is BUTLER_BF16 or BUTLER_F32 for the key, query and value tensors; scores
 *     and attention outputs are always float32; indices, counts are int32.
 *   - Arguments are validated on the host before anything is enqueued.  On an error
 *     return nothing has been enqueued and no output has been touched.
 *   - Workspace follows a two-phase query.  workspace == NULL with ws_bytes != NULL is
 *     a size query: the required size (0 when none is needed) is written to *ws_bytes,
 *     BUTLER_OK is returned and nothing is enqueued.  The real call passes a buffer of at
 *     least that size with *ws_bytes set to its size, or workspace == NULL and
 *     ws_bytes == NULL when the required size is 0 (BUTLER_ERR_WORKSPACE otherwise).  A
 *     workspace must be zero-filled before its first use; every call leaves the
 *     accumulators in it zero again, so one buffer serves every later call with the same
 *     size arguments on one stream.  A call with other sizes may lay the workspace out
 *     differently: give it its own buffer, or zero-fill the shared one first.  Two calls
 *     that share a workspace must not run concurrently.
 *   - Results are deterministic: the same inputs give bitwise identical outputs.
 *   - Selection heads.  The model card (Method) gives Q_imp one d'-vector per attention
 *     head, and does not say whether the heads of a GQA group share one selected set.
 *     Calls that take `sel_group` let the caller choose: a selected set belongs to
 *     sel_group consecutive query heads.  sel_group = 0 means the whole group of
 *     R = Hq / Hkv query heads of a KV head (one set per (b, KV head), the default);
 *     any divisor of R is accepted, and sel_group = 1 gives every query head its own set.
 *     Hs = Hq / sel_group (Hkv when sel_group = 0) is the number of selection heads per
 *     batch entry.  Selection head j covers query heads [j*sel_group, (j+1)*sel_group) and
 *     reads KV head j*sel_group / R.  Scores, radix histograms, keep flags, index lists,
 *     bitmasks and counts are laid out per selection head ([B, Hs, ...]); caches and K_imp
 *     stay per KV head.  butler_select_topk and butler_expand_neighbors work per row and
 *     take Hs directly.
 */
#ifndef BUTLER_H
#define BUTLER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum butler_status {
  BUTLER_OK = 0,
  BUTLER_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned pointer, ...   */
  BUTLER_ERR_UNSUPPORTED = -2,  /* dtype / head dim / d' / group size not built      */
  BUTLER_ERR_WORKSPACE = -3,    /* workspace smaller than the queried size           */
  BUTLER_ERR_HIP = -4           /* a kernel launch failed (hipGetLastError)          */
};

enum butler_dtype { BUTLER_F32 = 0, BUTLER_BF16 = 1 };

enum butler_score_mode { BUTLER_SCORE_RAW = 0, BUTLER_SCORE_SOFTVOTE = 1 };

/* Human-readable name of a status code (static storage, never NULL). */
const char* butler_status_string(int status);

/* ABI version, currently 8. */
int butler_abi_version(void);

/*
 * butler_project_keys -- K_imp = K . W_K for the tokens [pos0, pos0 + n_new).
 * Model card, Method: every cached key (after RoPE) is mapped to the d'-dimensional
 * importance space by a learned D x d' matrix W_K; one row is added per generated token
 * (n_new = 1 in decode, n_new = L when a prompt is first cached).
 *
 *   k_cache [B, Hkv, L_cap, D]      dtype   cached keys (read)
 *   w_k     [D, d']                 dtype   projection of this layer, shared by all KV heads
 *   kimp    [B, Hkv, L_cap, d']     dtype   rows pos0 .. pos0+n_new-1 written, others untouched
 * Each output is the dot product accumulated in float64 and rounded once, to nearest
 * even, into dtype.  For bf16 inputs the float64 sum is exact, so the result is the
 * exactly rounded dot product; for float32 inputs the float64 sum may round (products
 * take up to 48 bits), which in rare cases moves the result by one float32 ulp.
 * D in {64, 128}; d' in {16, 32}; 0 <= pos0, n_new >= 1, pos0 + n_new <= L_cap.
 */
int butler_project_keys(void* stream, int dtype, const void* k_cache, const void* w_k,
                        void* kimp, int B, int Hkv, int L_cap, int D, int dprime,
                        int pos0, int n_new);

/*
 * butler_produce_queries -- Q_imp = f_theta(LN(H)) at a producer layer.
 * Model card, Method: a producer reads the hidden states H [B, Lq, E] and predicts
 * importance queries for itself and the next G-1 layers, (B*Hq) x G x Lq x d'.
 * f_theta is the two-layer MLP  y = relu(LN(h) . W1^T) . W2^T  without biases; LN is a
 * LayerNorm without affine parameters (biased variance, ln_eps).  The normalised row,
 * the hidden activation and y are stored as bf16 between the steps.  Column
 * (head*G + slot)*d' + i of y is Q_imp[b, head, slot, t, i].  The weights are in the
 * [out_features, in_features] layout of a PyTorch Linear (K-contiguous rows).
 *
 *   h      [B, Lq, E]         bf16
 *   w1     [F, E]             bf16
 *   w2     [Hq*G*d', F]       bf16
 *   q_imp  [B, Hq, G, Lq, d'] bf16 (written)
 * dtype must be BUTLER_BF16.  E, F multiples of 64, E <= 8192; Hq*G*d' a multiple of 64;
 * d' a multiple of 8.
 * workspace: normalised rows and hidden activations, split-K partial sums (at most 4
 * rows: the hidden activations only).
 */
int butler_produce_queries(void* stream, int dtype, const void* h, const void* w1,
                           const void* w2, void* q_imp, int B, int Lq, int E, int F, int Hq,
                           int G, int dprime, float ln_eps, void* workspace, size_t* ws_bytes);

/*
 * butler_score -- importance score of every cached token, per selection head and query row.
 *
 * BUTLER_SCORE_RAW (model card, Method: the consumer scores every cached token with its
 * slot of Q_imp against K_imp):
 *   q     = q_imp [B, Hq, G, Lq, d'], the consumer reads slot `slot`
 *   keys  = kimp  [B, Hkv, L_cap, d']
 *   score[b, j, i, t] = (sum over the query heads h of selection head j of
 *                        Q_imp[b, h, slot, i, :]) . K_imp[b, kv(j), t, :]
 *   (kv(j) = j * sel_group / R, the KV head of those query heads)
 *   computed from float64 products and float64 sums of the stored values, rounded once
 *   to float32.  For bf16 inputs every product and partial sum is exact in float64, so
 *   the score is the exactly rounded dot product whatever the summation order.  For
 *   float32 inputs a product takes up to 48 bits and the float64 sums may round, so in
 *   rare cases the result differs from the exactly rounded value.  dk = d'.
 * BUTLER_SCORE_SOFTVOTE (TokenSelect README, highlights: per-head Q.K criticality,
 * normalised by a softmax per head, summed over heads):
 *   q     = [B, Hq, Lq, D] attention queries, keys = k_cache [B, Hkv, L_cap, D]
 *   score[b, j, i, t] = sum_{h in j} softmax_t(softmax_scale * q_h . k_t), k_t of KV head kv(j)
 *   float32 arithmetic; the softmax runs over all scored tokens of the row.  dk = D,
 *   G and slot are ignored.
 * Causal rows (causal != 0): query row i sits at absolute position q_pos0 + i and scores
 * only the tokens t <= q_pos0 + i; the others are written as -inf.  Non-causal rows score
 * tokens [0, L).
 *
 *   scores     [B, Hs, Lq, L]      float32 (written)
 *   radix_hist [B, Hs, Lq, 2048]   uint32, optional (NULL = none), used by single-row
 *              (Lq == 1) calls only; multi-row calls leave it untouched.  When used, the
 *              count of every written score (t < row length) is added to bin key >> 21,
 *              where key is the score's order-preserving 32-bit key (bits of the float
 *              with -0 taken as +0 and NaN as -inf; sign set: all bits flipped, else the
 *              sign bit set).  The caller zero-fills it before its first use; passing it
 *              on to butler_select_topk spares the selection one pass over the scores, and
 *              butler_select_topk leaves it zero-filled again.
 *   keep       [B, Hs]             int32, optional (NULL = none), single-row calls only:
 *              rows of a (b, selection head) with keep != 0 are skipped -- their scores
 *              (and radix_hist) are left as they were (see butler_selection_cache).
 * sel_group: query heads per selected set (see "Selection heads" above; 0 = R).
 * RAW: d' in {16, 32}, B * Hs <= 65535; SOFTVOTE: D in {64, 128}, Lq == 1 (decode);
 * R in {1, 2, 4, 8}.
 * workspace: SOFTVOTE keeps per-token logits and per-block softmax partials.
 */
int butler_score(void* stream, int mode, int dtype, const void* q, const void* keys,
                 float* scores, uint32_t* radix_hist, const int32_t* keep, int B, int Hq,
                 int Hkv, int sel_group, int G, int slot, int Lq, int L,
                 int L_cap, int dk, int q_pos0, int causal, float softmax_scale,
                 void* workspace, size_t* ws_bytes);

/*
 * butler_project_and_score -- one decode step's projection and raw scoring in one launch:
 * the same results as butler_project_keys(pos0 = L - 1, n_new = 1) followed by
 * butler_score(BUTLER_SCORE_RAW, Lq = 1, non-causal) with the same arguments.  Model card,
 * Method: the key row of the token just appended is projected to K_imp, then every cached
 * token (this one included) is scored against the consumer's slot of Q_imp.
 *
 *   q_imp      [B, Hq, G, 1, d']    dtype (read), slot `slot` is used
 *   k_cache    [B, Hkv, L_cap, D]   dtype (read): row L - 1 is projected
 *   w_k        [D, d']              dtype (read)
 *   kimp       [B, Hkv, L_cap, d']  dtype: row L - 1 written (even for kept rows), rows
 *                                   0 .. L-2 read
 *   scores     [B, Hs, 1, L]        float32 (written)
 *   radix_hist, keep, sel_group     as in butler_score (single-row call)
 * D in {64, 128}; d' in {16, 32}; R in {1, 2, 4, 8}; B * Hs <= 65535; kimp must not alias
 * k_cache or w_k.  No workspace.
 */
int butler_project_and_score(void* stream, int dtype, const void* q_imp, const void* k_cache,
                             const void* w_k, void* kimp, float* scores, uint32_t* radix_hist,
                             const int32_t* keep, int B, int Hq, int Hkv, int sel_group, int G,
                             int slot, int L, int L_cap, int D, int dprime);

/*
 * butler_score_tokens -- raw scores of the tokens [t_begin, t_end) of single decode rows of
 * length L, optionally with the appended key row projected in the same launch.  Model
 * card, Method: a producer predicts the importance queries of itself and the next G - 1
 * layers, so a consumer's scores of the tokens already cached depend only on its
 * producer's Q_imp and on K_imp: they can be computed as soon as the producer has run,
 * before the consumer layer's own input exists, and only the token that layer appends is
 * left for its turn.  Scores and histogram counts are those of butler_score (RAW, Lq = 1,
 * non-causal) for the same tokens; the other tokens of the rows are left as they were, so
 * two calls over [0, L-1) and [L-1, L) give butler_score's or butler_project_and_score's
 * result over [0, L).
 *
 *   q_imp      [B, Hq, G, 1, d']    dtype (read), slot `slot`
 *   kimp       [B, Hkv, L_cap, d']  dtype: rows t_begin .. t_end-1 read
 *   k_cache    [B, Hkv, L_cap, D]   dtype, w_k [D, d'] dtype: both NULL, or both given with
 *                                   t_end == L, and row L - 1 of kimp is first projected
 *                                   (written) as butler_project_and_score does
 *   scores     [B, Hs, 1, L]        float32: entries t_begin .. t_end-1 of every row written
 *   radix_hist, keep, sel_group     as in butler_score (single-row call): the counts of the
 *                                   scored tokens are added
 * 0 <= t_begin < t_end <= L; d' in {16, 32}; D in {64, 128} when projecting; R in
 * {1, 2, 4, 8}; B * Hs <= 65535.  No workspace.
 */
int butler_score_tokens(void* stream, int dtype, const void* q_imp, void* kimp,
                        const void* k_cache, const void* w_k, float* scores,
                        uint32_t* radix_hist, const int32_t* keep, int B, int Hq, int Hkv,
                        int sel_group, int G, int slot, int L, int L_cap, int D, int dprime,
                        int t_begin, int t_end);

/*
 * butler_select_topk -- fixed-budget top-x + sink + window, per selection head and query row.
 * Model card, Method and Memory requirements: keep the top-x tokens under a fixed
 * budget (fixed_<N>pc keeps (100-N)% of the tokens), augmented by a sink prefix of
 * n_sink tokens (min_sparse_index) and a recent window of n_window tokens
 * (sliding_window).  For a row of length L_r (L, or q_pos0+i+1 for causal row i):
 *   x   = floor(L_r * budget_num / budget_den)
 *   F   = [0, min(n_sink, L_r))  U  [max(0, L_r - n_window), L_r)   (the forced tokens)
 *   P   = every token of the row, or, with budget_excludes_forced != 0, the tokens not in F
 *   T   = the first min(x, |P|) tokens of P ordered by (score descending, index
 *         ascending); -0 equals +0, NaN ranks as -inf
 *   S   = T  U  F
 * (budget_excludes_forced is the reading where the budget counts only the tokens outside
 * the sink and the window, so |S| = min(x, |P|) + |F|; the default ranks every token.)
 * Output: `idx` (when non-NULL) holds S in ascending order in the first count[row]
 * entries of its row, entries beyond that are left as they were; `bitmask` (when
 * non-NULL) holds bit (t % 32) of word t / 32 set iff t in S, for every word of the row;
 * count[row] = |S|.  At least one of idx, bitmask must be non-NULL.
 *
 *   scores  [B, Hs, Lq, L]           float32 (read)
 *   keep    [B, Hs]                  int32, optional (NULL = none), single-row calls only:
 *                                    rows with keep != 0 are not selected again: they keep
 *                                    the previous selection with the window re-taken at
 *                                    the current L (the cache may have grown since), i.e.
 *                                    S = {t in S_prev : t < max(0, L - n_window)}
 *                                        U [max(0, L - n_window), L).
 *                                    idx then holds the first min(|S|, cap) entries of S
 *                                    and count = min(|S|, cap): a kept row grows by one
 *                                    entry per token appended since its selection, so cap
 *                                    must leave room for them.  bitmask (laid out for the
 *                                    current L) gains the window's bits; with a bitmask and
 *                                    no idx, count is the number of bits set in the row.
 *   radix_hist [B, Hs, Lq, 2048]     uint32, optional: the histogram butler_score built for
 *                                    exactly these scores (see butler_score); it is used
 *                                    instead of a counting pass and zero-filled again.  NULL:
 *                                    the selection counts by itself.  Multi-row (Lq > 1)
 *                                    calls ignore it, as butler_score does.  It must be NULL
 *                                    when budget_excludes_forced is set (BUTLER_ERR_INVALID_ARG).
 *   idx     [B, Hs, Lq, cap]         int32   (written) -- cap >= min(L, x + n_sink + n_window)
 *   bitmask [B, Hs, Lq, ceil(L/32)]  uint32  (written)
 *   count   [B, Hs, Lq]              int32   (written)
 * Hs: selection heads per batch entry (Hkv, or Hq / sel_group; see "Selection heads").
 * 0 <= budget_num, 1 <= budget_den, n_sink >= 0, n_window >= 0.  Rows of a causal or
 * multi-row (Lq > 1) call hold at most 65536 tokens; single-row decode calls up to 2^23.
 * workspace: none for causal / multi-row calls and rows up to 4096 tokens; otherwise a
 * radix histogram, each chunk's candidate keys, per-chunk counts and coarse-bin tables
 * (about 8 bytes per token per row).  The state it carries between calls sits at the
 * start of the buffer, depends only on the number of rows B * Hs * Lq and is valid for
 * any budget and any L: one buffer sized for the longest row serves every call with the
 * same rows, whatever their budgets and lengths (a decode loop whose cache grows by a
 * token per step).  butler_select_attend lays out the same state the same way, so the
 * two calls may share one buffer too.
 */
int butler_select_topk(void* stream, const float* scores, uint32_t* radix_hist,
                       const int32_t* keep, int budget_num, int budget_den, int n_sink,
                       int n_window, int budget_excludes_forced, int32_t* idx,
                       uint32_t* bitmask, int32_t* count, int B, int Hs, int Lq, int L,
                       int cap, int q_pos0, int causal, void* workspace, size_t* ws_bytes);

/*
 * butler_sparse_decode_attn -- attention over the selected tokens only.
 * Model card, intro and Method: attention reads only the selected subset of the full
 * (never evicted) KV cache.  For query head h (selection head j = h / sel_group, KV head
 * h / R) of row i:
 *   o[b, h, i, :] = sum_{t in S} softmax_t(softmax_scale * q . k_t) v_t
 * with float32 logits, a float32 online softmax (running maximum m, normaliser
 * l = sum of the float32 probabilities p_t = exp(z_t - m)) and float32 accumulation.
 * Precision of P.V: with bf16 inputs and D = 128 (the matrix-core kernels: decode with
 * R in {1, 2, 4, 8}, prefill with R = 4) the probabilities enter the product rounded to
 * bf16 while l sums the unrounded ones.  Each p_t then carries a relative error of at
 * most 2^-8, so an output element lies within 2^-8 * sum_t p_t |v_t| / sum_t p_t
 * (<= 2^-8 * max |v|) of the float32 result.  The other kernels (float32 inputs, D = 64)
 * multiply float32 probabilities.
 *
 * Lq == 1 (decode): S comes from idx [B, Hs, 1, cap] / count [B, Hs, 1] as written by
 *   butler_select_topk (or butler_expand_neighbors); the list is split over workgroups
 *   and a second kernel merges the partial results in a fixed order.
 * Lq > 1 (chunked prefill): S of row i comes from bitmask [B, Hs, Lq, ceil(L/32)];
 *   query row i sits at absolute position q_pos0 + i; only tokens t <= q_pos0 + i may
 *   be selected.
 *
 *   q       [B, Hq, Lq, D]      dtype
 *   k_cache [B, Hkv, L_cap, D]  dtype
 *   v_cache [B, Hkv, L_cap, D]  dtype
 *   out     [B, Hq, Lq, D]      float32 (written)
 * sel_group: query heads per selected set (see "Selection heads"; 0 = R).
 * An empty selected set is an error of the caller (the window always holds the newest
 * token); its output row is written as zeros.  Selected indices must be < L <= L_cap.
 * workspace: per-split softmax partials (decode).
 */
int butler_sparse_decode_attn(void* stream, int dtype, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* idx, const int32_t* count,
                              const uint32_t* bitmask, float* out, int B, int Hq, int Hkv,
                              int sel_group, int D, int Lq, int L, int L_cap, int cap,
                              int q_pos0, float softmax_scale, void* workspace,
                              size_t* ws_bytes);

/*
 * butler_select_attend -- one decode step's selection and sparse attention in one call:
 * the same results as butler_select_topk (Lq = 1, non-causal, idx output, no keep flags)
 * followed by butler_sparse_decode_attn over that idx / count, with the same arguments.
 * Model card, Method: the step keeps the top-x tokens plus sink and window, then attends
 * only to them.  For bf16, D = 128 and rows longer than 4096 tokens the selection's
 * finishing pass attends to its own chunk of the row while the chunk's indices are still
 * on chip, and a merge kernel combines the chunks; other shapes run the two calls' kernels.
 * The attention output equals the separate calls' up to float32 rounding order; idx and
 * count are identical.
 *
 *   scores [B, Hs, 1, L] float32, radix_hist [B, Hs, 1, 2048] optional (as in
 *   butler_select_topk), idx [B, Hs, 1, cap] int32 and count [B, Hs, 1] int32 (written),
 *   q [B, Hq, 1, D], k_cache / v_cache [B, Hkv, L_cap, D] (dtype), out [B, Hq, 1, D] float32;
 *   sel_group as in butler_sparse_decode_attn.
 * Limits as in the two calls; L <= 2^23.  workspace: the selection's state and each
 * chunk's candidates, and one softmax partial per chunk (or the two calls' workspaces).
 */
int butler_select_attend(void* stream, int dtype, const float* scores, uint32_t* radix_hist,
                         int budget_num, int budget_den, int n_sink, int n_window,
                         int budget_excludes_forced, int32_t* idx, int32_t* count, const void* q,
                         const void* k_cache, const void* v_cache, float* out, int B, int Hq,
                         int Hkv, int sel_group, int D, int L, int L_cap, int cap,
                         float softmax_scale, void* workspace, size_t* ws_bytes);

/*
 * butler_select_attend_noalloc -- butler_select_attend without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, and serving
 * loops or harnesses that forbid hipMalloc.  The arguments, results, limits and error
 * codes are those of butler_select_attend; idx, count and out are bitwise the same.  The
 * call allocates nothing: its workspace is a fixed device array inside the library of
 * BUTLER_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held until the process ends.
 * A call that needs more (the size butler_select_attend's workspace query reports; about
 * 8 bytes per token per selection row, so up to ~7M tokens over all rows) returns
 * BUTLER_ERR_WORKSPACE with nothing enqueued.  Every call on a GPU uses that GPU's one
 * array: calls that may overlap on one GPU (other streams, other host threads) race and
 * must be ordered by the caller.  Each call first clears, with a kernel on `stream`, the
 * part of the array that must start at zero, so it depends on no earlier call.  The first
 * call on a device looks up that device's copy (hipGetSymbolAddress) before enqueuing.
 */
#define BUTLER_NOALLOC_SCRATCH_BYTES (64u << 20)
int butler_select_attend_noalloc(void* stream, int dtype, const float* scores,
                                 uint32_t* radix_hist, int budget_num, int budget_den,
                                 int n_sink, int n_window, int budget_excludes_forced,
                                 int32_t* idx, int32_t* count, const void* q,
                                 const void* k_cache, const void* v_cache, float* out, int B,
                                 int Hq, int Hkv, int sel_group, int D, int L, int L_cap,
                                 int cap, float softmax_scale);

/*
 * butler_selection_cache -- TokenSelect README, highlights, Selection Cache: consecutive
 * similar queries share one token selection, so selection runs less often.  For every
 * (b, selection head j) of a decode step, the cosine similarity between j's current query
 * (the D-vectors of its query heads stacked into one vector) and the reference query the
 * cached selection was made for:
 *   cos >= threshold  ->  keep[b, j] = 1: score and select skip the (b, j) rows; the
 *                         previous index list / bitmask stand, with the recent window
 *                         re-taken at the current length (see butler_select_topk);
 *   otherwise         ->  keep[b, j] = 0 and q_ref takes q for j's heads: the next score
 *                         and select recompute the selection for this query.
 * A zero vector on either side gives cos = 0.  The similarity is accumulated in float32
 * (products of the stored values, one sum per (b, g) in lane order, then a fixed tree).
 *
 *   q      [B, Hq, 1, D]   dtype (read)
 *   q_ref  [B, Hq, 1, D]   dtype (read, rows refreshed) -- caller-owned state; a first call
 *                          with threshold > 1 (or a zero-filled q_ref) refreshes every row
 *   keep   [B, Hs]         int32 (written)
 * sel_group as in butler_score.  D in {64, 128}, R = Hq / Hkv in {1, 2, 4, 8}.  No workspace.
 */
int butler_selection_cache(void* stream, int dtype, const void* q, void* q_ref, int32_t* keep,
                           int B, int Hq, int Hkv, int sel_group, int D, float threshold);

/*
 * butler_expand_neighbors -- neighbour fetching for the prediction interval.
 * TokenButler arXiv abstract: the predictor can run once per prediction interval, the
 * selection made at its last run being reused in between and widened with the tokens'
 * neighbours (neighbor fetching).  Per (b, selection head) decode row:
 *   S' = { u : |u - t| <= width for some t in S }  U  [max(0, L - n_window), L),  0 <= u < L
 * where S is the first min(count, cap_in) entries of idx (a selection made at an earlier,
 * shorter length) and the window is taken at the current length L, so the tokens appended
 * since are attended.  Indices outside [0, L) in S are ignored.  idx_out holds S' in
 * ascending order in its first count_out entries (entries beyond cap_out are dropped;
 * count_out is |S'|).
 *
 *   idx       [B, Hs, cap_in]     int32 (read), count [B, Hs] int32 (read)
 *   idx_out   [B, Hs, cap_out]    int32 (written), count_out [B, Hs] int32 (written)
 * 0 <= width <= 31; L <= 2^23; cap_out >= min(L, cap_in * (2*width + 1) + n_window); the
 * output buffers must not alias the inputs.  No workspace.
 */
int butler_expand_neighbors(void* stream, const int32_t* idx, const int32_t* count,
                            int32_t* idx_out, int32_t* count_out, int B, int Hs, int L,
                            int cap_in, int cap_out, int width, int n_window);

/*
 * butler_fetch_rows -- selected-row fetch from a KV cache kept in host memory.
 * TokenButler arXiv abstract: against dense attention with the KV cache offloaded to the
 * CPU, selection cuts decode latency, because only the selected tokens' K and V rows
 * have to cross to the GPU.  For selection head j of batch b (see "Selection heads") and
 * p < min(count[b, j], cap):
 *   k_sel[b, j, p, :] = k_cache[b, kv(j), idx[b, j, 0, p], :]   (and v_sel from v_cache)
 * so the rows of each selected set arrive packed in set order.  Slots p >= count are left
 * as they were.  butler_sparse_decode_attn then attends over them with k_sel / v_sel as
 * its caches ([B, Hs, cap, D], Hkv = Hs, sel_group = 0), positions 0 .. count-1 as its
 * index list (any ascending list of them) and the same count.
 *
 *   idx     [B, Hs, 1, cap]       int32 (device), count [B, Hs, 1] int32 (device), as
 *                                 written by butler_select_topk
 *   k_cache [B, Hkv, L_cap, D]    dtype, pinned host memory (hipHostMalloc) that the GPU
 *   v_cache [B, Hkv, L_cap, D]    maps -- the rows are read across the host link, with no
 *                                 staging copy -- or device memory
 *   k_sel   [B, Hs, cap, D]       dtype, device memory (written)
 *   v_sel   [B, Hs, cap, D]       dtype, device memory (written)
 * D in {64, 128}; R = Hq / Hkv in {1, 2, 4, 8}; indices outside [0, L_cap) are clamped.
 * The memory kind of every pointer is checked with hipPointerGetAttributes (this call's
 * validation uses the HIP runtime): pageable host memory, which no kernel may read, and
 * unknown pointers give BUTLER_ERR_INVALID_ARG.  No workspace.
 */
int butler_fetch_rows(void* stream, int dtype, const int32_t* idx, const int32_t* count,
                      const void* k_cache, const void* v_cache, void* k_sel, void* v_sel, int B,
                      int Hq, int Hkv, int sel_group, int D, int L_cap, int cap);

#ifdef __cplusplus
}
#endif

#endif /* BUTLER_H */
