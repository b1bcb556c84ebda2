/*
 * sd.h -- C ABI of one block-parallel speculative draft-and-verify step on
 * AMD Instinct MI355X (gfx950).
 *
 * The step has three parts, one entry point each:
 *   sd_draft_attn     draft-block attention over the target's paged KV cache
 *                     (whole prefix, or recent window + context summary)
 *   sd_summary_update summarise whole prefixes, or fold newly retained target
 *                     KV rows into the summary
 *   sd_schedule_draft  pre-draft estimation, joint draft / verify schedule
 *   sd_schedule_verify post-draft estimation, verification budget split
 *   sd_lm_head_probs  drafter LM head, softmax statistics, draft sampling
 *   sd_markov_sample   sequential (Markov) correction and sampling, logit fusion
 *   sd_log_prior_bias  smoothed unigram log-prior (fusion bias)
 *   sd_verify         lossless speculative-sampling verification
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees, copies to the host or synchronises; scratch
 *     memory is the caller's `workspace` (size from the matching
 *     *_workspace_size function, any alignment of at least 256 bytes).
 *   - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns at once.  The status reports host-side
 *     argument validation and launch errors only; NULL pointers, sizes out of
 *     range and a short workspace are rejected before anything is launched.
 *   - Integer arrays that live on the device (lengths, offsets, page ids,
 *     tokens) are never read on the host.  Values that break the documented
 *     contract give unspecified results but never an out-of-bounds access:
 *     kernels clamp page ids, lengths and offsets to the host-given sizes.
 *   - bf16 is IEEE binary32 truncated to its upper 16 bits (bfloat16);
 *     fp32 is IEEE binary32.  All arrays are dense, row-major, unpadded.
 *   - Re-entrant: the library holds no global state (apart from the device
 *     array of sd_draft_attn_noalloc).  Calls that share a workspace must not
 *     overlap in time.
 *
 * Randomness: every random decision uses Philox-4x32-10 (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11) keyed by
 * (seed mod 2^32, seed >> 32) with counter (v >> 2, j, req_id[b], stream):
 * word (v & 3) serves vocab entry v, j is the 1-based draft position (b_b + 1
 * for the bonus token), stream 0 = draft sampling, 1 = acceptance test
 * (word 0 of counter (0, j, req_id, 1), u = (x >> 8) * 2^-24), 2 = correction
 * or bonus token.  Tokens are Gumbel-max draws argmax_v(key_v - log(-log u_v))
 * with u = (2 (x >> 9) + 1) * 2^-24; the smallest index wins a tie.
 */
#ifndef SD_H
#define SD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sd_status;

enum {
  SD_OK = 0,
  SD_ERR_NULL = 1,      /* a required pointer is NULL                        */
  SD_ERR_SHAPE = 2,     /* a size argument is out of the supported range     */
  SD_ERR_WORKSPACE = 3, /* workspace NULL or smaller than required           */
  SD_ERR_LAUNCH = 4,    /* the HIP runtime rejected a launch                 */
  SD_ERR_DEVICE = 5,    /* no gfx950 device is current                       */
  SD_ERR_SCRATCH = 6    /* sd_draft_attn_noalloc: the call needs more scratch
                           than its fixed device array holds                  */
};

/* Attention among the draft block's own rows (sd_draft_attn block_mask). */
enum {
  SD_MASK_NONE = 0,     /* bidirectional: every block row sees every block row */
  SD_MASK_CAUSAL = 1    /* block row j sees block rows 0..j                    */
};

/* Static description of a status code (never NULL). */
const char* sd_status_str(sd_status s);

/* Library version string, e.g. "0.1.0". */
const char* sd_version(void);

/* ------------------------------------------------------------------------
 * sd_draft_attn -- draft-block attention over the target's paged KV cache.
 *
 * Defined by: "ForeSpark: Joint draft and verification budget scheduling for
 * parallel speculative decoding", sec. 1 and sec. 4.1 (each draft position
 * attends bidirectionally to every draft position and to the context, which
 * enters as extra keys and values); "LongSpark: Efficient speculative
 * decoding with a fixed-cost parallel drafter", App. A.1, Fig. 6 (one
 * attention normalisation across all sources; bidirectional among the block's
 * slots); "H-Spec: Parallel speculative decoding without a drafter-side KV
 * cache", sec. 3.3.2 (draft attention reads the target's KV cache in place;
 * head counts and dims equal the target's; block Q/K use RoPE positions that
 * continue the prefix, so q, k_blk and the cache are all post-RoPE).
 *
 * For request b with prefix length N_b = ctx_len[b] and K_b = q_off[b+1] -
 * q_off[b] draft rows, every query head h (KV head g = h / (Hq / Hkv)) of
 * every draft row r computes, with one softmax,
 *     out[r, h] = softmax(s) . [V_prefix(g); v_blk[rows of b, g]; Z_b(g)]
 *     s = softmax_scale * q[r, h] . [K_prefix(g); k_blk[rows of b, g]; U(g)]
 * where K_prefix / V_prefix are the cached rows of head g in logical token
 * order: all N_b of them (window = 0), or only the last min(W, N_b)
 * (window = W > 0).  U(g) / Z_b(g) are the n_summary context-summary keys and
 * values (absent when n_summary = 0).  With block_mask = SD_MASK_NONE there
 * is no mask; with SD_MASK_CAUSAL block row j (j = r - q_off[b]) sees block
 * keys 0..j only (prefix and summary keys stay visible).  Scores, softmax
 * and accumulation are fp32; summary values enter rounded to bf16 (nearest
 * even) like every other value row; out is rounded to bf16 (nearest even).
 *
 * Variants: the recent window plus summary is the fixed-size context of
 * "LongSpark", sec. 2.2, eq. (6) (block; recent window of W target KV rows;
 * summary queries as keys and summary values as values, under one
 * normalisation); the causal block mask and a window are the attention of
 * "H-Spec", sec. 3.3.2 (causal over the block, target KV as prefix context,
 * a sliding window over the prefix; here one window shared by the block's
 * rows).
 *
 * Arguments
 *   q        bf16 [total_q, Hq, D]   draft queries, request b owns rows
 *                                    q_off[b] .. q_off[b+1]-1
 *   k_blk    bf16 [total_q, Hkv, D]  draft-block keys (same rows)
 *   v_blk    bf16 [total_q, Hkv, D]  draft-block values
 *   k_cache  bf16 [num_pages, Hkv, D/8, page_size, 8]  target keys: dims
 *            8c..8c+7 of the token in slot t of a page are at [page, g, c, t, :]
 *   v_cache  bf16 [num_pages, Hkv, D, page_size]  target values: dim d of the
 *            token in slot t is at [page, g, d, t]
 *   page_table int32 [batch, max_pages]: logical page i of request b is
 *            physical page page_table[b*max_pages + i]; token n is slot n % 16
 *            of logical page n / 16
 *   ctx_len  int32 [batch]  N_b >= 0, N_b <= max_pages * page_size
 *   q_off    int32 [batch+1] non-decreasing, q_off[0] = 0,
 *            q_off[batch] = total_q, 0 <= K_b <= max_draft_k (a request
 *            with K_b = 0, e.g. one the scheduler gives no drafts, has no
 *            rows and no work)
 *   max_draft_k  host bound on K_b; (Hq/Hkv) * max_draft_k <= 128 (the
 *                query rows of one (request, KV head) share one read of its
 *                KV: up to 64 rows per work item with two waves, up to 128
 *                with four)
 *   num_pages    rows of the caches (page ids are clamped to it)
 *   page_size    16
 *   num_heads_q, num_heads_kv  Hq % Hkv == 0
 *   head_dim     64 or 128
 *   max_total_ctx  host upper bound on sum_b N_b (sizes the launch and the
 *                  split-K partials in the workspace).  If the lengths on the
 *                  device add up to more and their work items do not fit the
 *                  partials, nothing is computed and every output row of the
 *                  call is set to NaN (never left stale).  When every
 *                  request's streamable span (max_pages * 16 tokens, or the
 *                  window plus one page) fits one split and n_summary = 0,
 *                  each (request, KV head) is one work item that writes its
 *                  rows directly: no partials are used and the bound plays
 *                  no part
 *   split_tokens   prefix tokens per split-K work item; 0 lets the library
 *                  choose (a power of two in [2048, 32768] from batch,
 *                  num_heads_kv and max_total_ctx); otherwise a multiple of
 *                  64, at most 32768
 *   softmax_scale  > 0, usually 1/sqrt(head_dim)
 *   block_mask     SD_MASK_NONE or SD_MASK_CAUSAL
 *   window         0 (whole prefix) or W > 0 (the last W prefix tokens)
 *   summary_keys   bf16 [Hkv, n_summary, D] (U), or NULL when n_summary = 0
 *   summary_values fp32 [batch, Hkv, n_summary, D] (Z_b, as kept by
 *                  sd_summary_update), or NULL when n_summary = 0
 *   n_summary      0 .. 64
 *   out      bf16 [total_q, Hq, D]
 * ------------------------------------------------------------------------ */
size_t sd_draft_attn_workspace_size(int32_t batch, int32_t num_heads_q,
                                    int32_t num_heads_kv, int32_t head_dim,
                                    int32_t max_draft_k, int64_t max_total_ctx,
                                    int32_t split_tokens);

sd_status sd_draft_attn(const void* q, const void* k_blk, const void* v_blk,
                        const void* k_cache, const void* v_cache,
                        const int32_t* page_table, const int32_t* ctx_len,
                        const int32_t* q_off, int32_t batch, int32_t total_q,
                        int32_t max_draft_k, int32_t num_pages,
                        int32_t max_pages, int32_t page_size,
                        int32_t num_heads_q, int32_t num_heads_kv,
                        int32_t head_dim, int64_t max_total_ctx,
                        int32_t split_tokens, float softmax_scale,
                        int32_t block_mask, int32_t window,
                        const void* summary_keys, const float* summary_values,
                        int32_t n_summary, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * sd_draft_attn_noalloc -- sd_draft_attn for callers that cannot allocate.
 *
 * For code that must not call hipMalloc or any allocating routine: work
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, operation, results (bit for bit) and errors as
 * sd_draft_attn, without workspace arguments: the work list and split-K
 * partials live in a device array inside the library,
 * sd_draft_attn_noalloc_max_scratch() bytes (128 MiB) per GPU, created when
 * the library's code is loaded on that GPU and held until the process ends.
 * A call whose sd_draft_attn_workspace_size(...) exceeds that size returns
 * SD_ERR_SCRATCH before anything is launched (e.g. 16 requests of 128K
 * tokens need about 24 MiB, 64 requests of 4K about 48 MiB, 128 requests of
 * 1K-128K, 3.2M tokens in all, about 113 MiB).
 *
 * The array is shared by every call on the same GPU and keeps the last
 * call's contents (nothing in it needs to start at zero).  Calls that
 * overlap in time on one GPU (e.g. on two streams, or from two threads
 * without ordering) race on it and give undefined results; calls on
 * different GPUs do not interact.  The first call on a GPU looks up the
 * array's device address (hipGetSymbolAddress); it allocates nothing.
 * ------------------------------------------------------------------------ */
size_t sd_draft_attn_noalloc_max_scratch(void);

sd_status sd_draft_attn_noalloc(const void* q, const void* k_blk, const void* v_blk,
                                const void* k_cache, const void* v_cache,
                                const int32_t* page_table, const int32_t* ctx_len,
                                const int32_t* q_off, int32_t batch, int32_t total_q,
                                int32_t max_draft_k, int32_t num_pages,
                                int32_t max_pages, int32_t page_size,
                                int32_t num_heads_q, int32_t num_heads_kv,
                                int32_t head_dim, int64_t max_total_ctx,
                                int32_t split_tokens, float softmax_scale,
                                int32_t block_mask, int32_t window,
                                const void* summary_keys, const float* summary_values,
                                int32_t n_summary, void* out, void* stream);

/* ------------------------------------------------------------------------
 * sd_summary_update -- maintain the global context summary.
 *
 * Defined by: "LongSpark", sec. 2.2, eq. (5) (for fixed summary queries U,
 * the summary values are the attention of U over all retained target KV
 * rows) and App. A.2, eqs. (10)-(11) (per query, the summary value Z and
 * log-normaliser c of a set of rows; two disjoint sets merge as
 * c = log(e^c_a + e^c_b), Z = e^(c_a - c) Z_a + e^(c_b - c) Z_b; after
 * verification at most K + 1 new rows are folded in; an empty set leaves the
 * state unchanged).
 *
 * For every request b and KV head g, with s_it = softmax_scale * U[g, i] . k_t
 * over cache rows t of head g:
 *   accepted_len == NULL: initialise from the whole prefix, rows 0..N_b-1
 *     (N_b = ctx_len[b]); N_b = 0 gives the empty state (c = -inf, Z = 0).
 *   accepted_len != NULL: fold rows N_b .. N_b + accepted_len[b] (the
 *     committed token and the a_b accepted drafts, which the target's
 *     verification pass has already written to the cache) into the stored
 *     state; a stored c = -inf is the empty state.
 * Arithmetic is fp32 (scores and weighted sums accumulate in fp32; the
 * softmax weights enter the value sums as a bf16 pair hi + lo, ~2^-18
 * relative), then the merge.
 *
 * Arguments
 *   summary_queries bf16 [Hkv, n_summary, D]  U (fixed, shared by requests),
 *                   16-byte aligned
 *   k_cache, v_cache, page_table, num_pages, max_pages, page_size
 *                   as for sd_draft_attn (rows are read in place)
 *   ctx_len         int32 [batch]  N_b before the new rows
 *   accepted_len    int32 [batch]  a_b (e.g. from sd_verify), or NULL
 *   n_summary       1 .. 64
 *   softmax_scale   > 0, usually 1/sqrt(head_dim)
 *   summary_values  fp32 [batch, Hkv, n_summary, D]  Z, updated in place
 *   summary_lse     fp32 [batch, Hkv, n_summary]     c, updated in place
 *   workspace       initialisation (accepted_len == NULL) only: at least
 *                   sd_summary_workspace_size(...) bytes; folds ignore it
 * Work: one wavefront per (request, KV head) for a fold.  An initialisation
 * runs 1,024 wavefronts over the concatenation of every (request, KV head)'s
 * rows, each taking an equal run of max(512, ceil(Hkv * sum_b N_b / 1024))
 * rows whatever the lengths (read on the device), and merges the pieces of
 * each (request, KV head) in a second kernel.
 * Errors: SD_ERR_NULL, SD_ERR_SHAPE (as listed above, unaligned pointers),
 * SD_ERR_WORKSPACE (initialisation with a missing or short workspace),
 * SD_ERR_LAUNCH.
 * ------------------------------------------------------------------------ */
size_t sd_summary_workspace_size(int32_t batch, int32_t num_heads_kv, int32_t n_summary,
                                 int32_t head_dim, int32_t max_pages, int32_t page_size);
sd_status sd_summary_update(const void* summary_queries, const void* k_cache,
                            const void* v_cache, const int32_t* page_table,
                            const int32_t* ctx_len, const int32_t* accepted_len,
                            int32_t batch, int32_t num_pages, int32_t max_pages,
                            int32_t page_size, int32_t num_heads_kv,
                            int32_t head_dim, int32_t n_summary,
                            float softmax_scale, float* summary_values,
                            float* summary_lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * sd_schedule_draft -- pre-draft estimation and the joint draft /
 * verification schedule.
 *
 * Defined by: "ForeSpark", sec. 4.2, eqs. (2)-(3) (the pre-draft survival
 * estimator reads the context feature c_i and the anchor embedding e_i:
 * u_i = SiLU(W_c c_i + W_e e_i), z_i = W_o u_i holds K(K+1)/2
 * conditional-acceptance logits, row d = a length-d draft; survival benefits
 * S_{i,d,j} = prod_{t<=j} sigmoid(z^(d)_{i,t}); Reward_i(d, b) =
 * sum_{j<=b} S_{i,d,j}, e.g. benefits 0.9, 0.7, 0.3 give Reward(3, 3) = 1.9,
 * Fig. 5) and sec. 4.3 (R_i(d) = Reward_i(d, d), R_i(0) = 0; F_i its upper
 * concave envelope on {0..K}; survival scores g_{i,d} = F_i(d) - F_i(d-1);
 * all scores pooled and sorted; eq. (4): (D, B) = argmax
 * (n + sum_{r<=B} g_(r)) / (T_draft(D) + T_verify(N + B)) over B <= sum d_i,
 * with latencies constant within token-count buckets, searched with one
 * candidate -- the largest feasible schedule -- per pair of buckets).  The
 * per-entry calibration of sec. 4.5 (a scale and a bias per logit) and the
 * biases the page omits are optional.
 *
 * Conventions: entry (d, t) of a triangle is at index d(d-1)/2 + t - 1.  The
 * drafter processes n + sum_i d_i tokens (anchor plus masks), the verifier
 * N + B; a token count takes the latency of the first bucket whose capacity
 * holds it; counts above the last bucket are infeasible.  Within a bucket
 * pair B is the largest feasible count of positive scores.  Equal scores are
 * ordered by (request, d) and ties of eq. (4) go to the first pair in
 * (draft bucket, verify bucket) order.  Everything runs on the device (no
 * host synchronisation): the outputs feed sd_draft_attn (q_off) and
 * sd_schedule_verify (verify_budget) directly.  Arithmetic is fp32.
 *
 * Arguments
 *   ctx_feat, anchor_emb  bf16 [n, d_h]  c_i and e_i
 *   w_c, w_e   bf16 [r, d_h];  b_u fp32 [r] or NULL
 *   w_o        bf16 [K(K+1)/2, r];  b_o fp32 [K(K+1)/2] or NULL
 *   cal_scale, cal_bias  fp32 [K(K+1)/2] or NULL (z = scale * z + bias)
 *   n (1..1024), d_h and r (multiples of 16), K (1..32), n * K <= 4096
 *   draft_caps int32 [n_draft_buckets] increasing token capacities,
 *   draft_lat  fp32  [n_draft_buckets] latencies (any unit, same as verify)
 *   verify_caps, verify_lat, n_verify_buckets: the verifier's table
 *   n_nonspec  N, the verification batch's non-speculative tokens
 *   logits     fp32 [n, K(K+1)/2] out (calibrated z)
 *   scores     fp32 [n, K] out (g_{i,d}, non-increasing in d)
 *   draft_len  int32 [n] out (d_i);  q_off int32 [n+1] out or NULL
 *   verify_budget int32 [1] out (B);  objective fp32 [1] out or NULL
 *   workspace  sd_schedule_workspace_size(n, r, max_rows, m) bytes (one
 *              workspace serves both scheduling calls)
 * ------------------------------------------------------------------------ */
size_t sd_schedule_workspace_size(int32_t n, int32_t r, int32_t max_rows,
                                  int32_t m);

sd_status sd_schedule_draft(const void* ctx_feat, const void* anchor_emb,
                            const void* w_c, const void* w_e, const float* b_u,
                            const void* w_o, const float* b_o,
                            const float* cal_scale, const float* cal_bias,
                            int32_t n, int32_t d_h, int32_t r, int32_t K,
                            const int32_t* draft_caps, const float* draft_lat,
                            int32_t n_draft_buckets, const int32_t* verify_caps,
                            const float* verify_lat, int32_t n_verify_buckets,
                            int32_t n_nonspec, float* logits, float* scores,
                            int32_t* draft_len, int32_t* q_off,
                            int32_t* verify_budget, float* objective,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------
 * sd_schedule_verify -- post-draft estimation and budget distribution.
 *
 * Defined by: "ForeSpark", sec. 4.4, eq. (5) (p_{i,j} = sigmoid(w . [h_{i,j};
 * s_{i,j}]) with selector feature s_{i,j} = (W_s h_{i,j}) * E_pred(x_{i,j-1}),
 * x_{i,0} the anchor token; S^_{i,j} = prod_{t<=j} p_{i,t}; the B positions
 * with the highest S^ across the batch are verified, a prefix of every
 * draft) and sec. 4.5 (a temperature per position calibrates p).  With the
 * bias c: p = sigmoid((w . [h; s] + c) / theta_j).  Equal S^ are ordered by
 * (request, position).  B is read on the device (from sd_schedule_draft) and
 * capped at the drafted rows.  Arithmetic is fp32 (W_s h on MFMA, bf16
 * products).
 *
 * Arguments
 *   hidden   bf16 [max_rows, H]  h_{i,j}, rows packed by q_off (the LM head's
 *            input rows); rows past q_off[n] are read but unused
 *   w_s      bf16 [m, H];  e_pred bf16 [V, m];  w fp32 [H + m];  bias c
 *   temperature fp32 [K] or NULL (theta_j of position j)
 *   anchor_tokens int32 [n];  draft_tokens int32 [max_rows] (packed)
 *   q_off    int32 [n+1] device (e.g. from sd_schedule_draft)
 *   verify_budget int32 [1] device
 *   n (1..1024), max_rows (1..4096) host bound on q_off[n], H and m
 *   multiples of 16, V >= 1, K (1..32)
 *   accept_prob, survival fp32 [max_rows] out (p and S^ of every drafted row;
 *            rows from q_off[n] on are not written)
 *   verify_len int32 [n] out (b_i);  t_off int32 [n+1] out or NULL
 *            (t_off[i+1] - t_off[i] = b_i + 1 target rows, as sd_verify takes)
 * ------------------------------------------------------------------------ */
sd_status sd_schedule_verify(const void* hidden, const void* w_s,
                             const void* e_pred, const float* w, float bias,
                             const float* temperature,
                             const int32_t* anchor_tokens,
                             const int32_t* draft_tokens, const int32_t* q_off,
                             const int32_t* verify_budget, int32_t n,
                             int32_t max_rows, int32_t H, int32_t m, int32_t V,
                             int32_t K, float* accept_prob, float* survival,
                             int32_t* verify_len, int32_t* t_off,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* ------------------------------------------------------------------------
 * sd_lm_head_probs -- drafter LM head, softmax statistics, draft sampling.
 *
 * Defined by: "LongSpark", sec. 2.3 and App. A.1, Fig. 6 (the frozen target
 * normalisation and vocabulary head map the final draft states to base
 * logits for all positions in parallel) and sec. 2.1, eq. (4) (the proposal
 * of slot j is softmax of its logits; slots are sampled independently);
 * "DeLS-Spec: Decoupled long-short contexts for parallel speculative
 * drafting" (block-parallel drafting is one forward pass then one sampling
 * step).
 *
 * For every row m < M and drafter vocabulary entry v < V, with W_v the row
 * w_vocab[v] (or w_vocab[vocab_map[v]] when the drafter's vocabulary is
 * pruned):  logits[m, v] = sum_k hidden[m, k] * W_v[k] (bf16 products, fp32
 * accumulation), lse[m] = log sum_v exp(logits[m, v]), and the drawn entry
 * v* = argmax_v (logits[m, v] - log(-log u_v)) with the stream-0 uniforms of
 * (request b, position j = m - q_off[b] + 1), or v* = argmax_v logits[m, v]
 * when greedy = 1 (temperature 0; no uniforms).  draft_tokens[m] = v*, or
 * vocab_map[v*] (a target token id) when the vocabulary is pruned.  The
 * draft distribution is q_m = exp(logits[m, :] - lse[m]) over the V entries.
 *
 * Variants: a pruned drafter vocabulary restricts drafting to a subset of
 * the target's vocabulary, reading those rows of the target's head in place
 * ("H-Spec", App. B.2); greedy decoding is the temperature-0 setting the
 * pages also evaluate ("LongSpark", App. D.1).
 *
 * Arguments
 *   hidden   bf16 [M, H]  final draft states after the target's final norm
 *   w_vocab  bf16 [w_rows, H] the target's LM head (nn.Linear layout), in
 *            place; [V, H] when vocab_map is NULL
 *   M >= 1, H a multiple of 64 (<= 65536), 1 <= V < 2^31
 *   q_off    int32 [batch+1] row offsets of the requests (as for attention);
 *            rows outside [0, q_off[batch]) use position m + 1 of request 0
 *   req_id   uint32 [batch]  Philox counter word of each request
 *   vocab_map int32 [V] target token id of each drafter entry (0 <= id <
 *            w_rows), or NULL (the drafter predicts over all V rows)
 *   w_rows   rows of w_vocab when vocab_map is given (ignored otherwise)
 *   greedy   0 (sample) or 1 (argmax; the smallest index wins a tie)
 *   logits   fp32 [M, V] out;  lse fp32 [M] out;  draft_tokens int32 [M] out
 * ------------------------------------------------------------------------ */
size_t sd_lm_head_workspace_size(int32_t M, int32_t V);

sd_status sd_lm_head_probs(const void* hidden, const void* w_vocab, int32_t M,
                           int32_t H, int32_t V, const int32_t* q_off,
                           int32_t batch, const uint32_t* req_id,
                           uint64_t seed, const int32_t* vocab_map,
                           int32_t w_rows, int32_t greedy, float* logits,
                           float* lse, int32_t* draft_tokens, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * sd_markov_sample -- sequential (Markov) correction and sampling of the
 * draft distributions.
 *
 * Defined by: "LongSpark", sec. 2.3, eqs. (7)-(8) (the base logits l_j^(0) of
 * all K_b positions, computed in parallel, are refined as
 * l_j = l_j^(0) + W_c e_c(y_{j-1}) with y_0 the committed token and a
 * rank-r correction embedding e_c and output mapping W_c; q_j = softmax(l_j)
 * is sampled position by position and the same q_j are used for
 * verification; only the correction and the sampling are sequential), and
 * "DeLS-Spec" (logit fusion at inference with the Markov local head: the
 * long logits plus alpha times W_M e_M(x_{i-1}) minus beta times the log
 * unigram prior; alpha = beta = 0.3 by default).
 *
 * For every request b and j = 1..K_b (row m = q_off[b] + j - 1):
 *   logits[m, v] += alpha * sum_k W_c[v, k] e_c[y_{j-1}, k] + vocab_bias[v]
 *                   (bf16 products, fp32 accumulation and sums)
 *   lse[m] = log sum_v exp(logits[m, v])
 *   draft_tokens[m] = y_j = argmax_v (logits[m, v] - log(-log u_v)), the
 *   stream-0 uniforms of (request b, position j), as sd_lm_head_probs draws
 *   (greedy = 1: argmax_v logits[m, v], no uniforms; smallest index on ties)
 * so W_c = 0 (or alpha = 0) without a bias gives exactly the draws of
 * sd_lm_head_probs.  LongSpark: alpha = 1, vocab_bias = NULL.  DeLS-Spec:
 * vocab_bias = -beta log p~_0 from sd_log_prior_bias.  The positions run in
 * order on the stream (one launch each, plus one before and one after);
 * nothing returns to the host.
 *
 * Arguments
 *   logits   fp32 [M, V] in: base logits (e.g. from sd_lm_head_probs);
 *            out: the corrected logits l_j
 *   lse fp32 [M] out;  draft_tokens int32 [M] out
 *   anchor_tokens int32 [batch]  y_0 of every request
 *   w_c, e_c bf16 [V, r]  (r a multiple of 16, 16-byte aligned)
 *   alpha    finite scale of the correction
 *   vocab_bias fp32 [V] or NULL
 *   greedy   0 (sample) or 1 (temperature 0)
 *   q_off    int32 [batch+1]; positions beyond max_draft_k (host bound,
 *            0..4096) are left untouched
 *   req_id, seed: as for sd_lm_head_probs
 *   workspace sd_markov_workspace_size(batch, V, max_draft_k) bytes
 * Errors: NULL -> SD_ERR_NULL; sizes out of range, unaligned tables or a
 * non-finite alpha, greedy not 0 or 1 -> SD_ERR_SHAPE; M == 0 or max_draft_k == 0 -> SD_OK with
 * nothing launched; short or unaligned workspace -> SD_ERR_WORKSPACE.
 * ------------------------------------------------------------------------ */
size_t sd_markov_workspace_size(int32_t batch, int32_t V, int32_t max_draft_k);

sd_status sd_markov_sample(float* logits, float* lse, int32_t* draft_tokens,
                           const int32_t* anchor_tokens, const void* w_c,
                           const void* e_c, float alpha, const float* vocab_bias,
                           int32_t greedy, const int32_t* q_off, int32_t batch,
                           int32_t M, int32_t V, int32_t r, int32_t max_draft_k,
                           const uint32_t* req_id, uint64_t seed,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * sd_log_prior_bias -- scaled, smoothed unigram log-prior for the fusion bias.
 *
 * Defined by: "DeLS-Spec", appendix on the unigram prior (corpus counts c(v)
 * with additive smoothing, lambda = 1 by default; its log is a fixed
 * vocabulary-level bias).
 *   out[v] = scale * log((c(v) + lambda) / (sum_u c(u) + lambda V))
 * computed in fp64, stored as fp32 (scale = -beta gives the fusion bias).
 * One-time setup, one workgroup.
 *
 * Arguments
 *   counts int64 [V] device (negative counts are read as 0); out fp32 [V]
 *   lambda > 0 and finite; scale finite
 * Errors: NULL -> SD_ERR_NULL; V < 1 or a bad lambda / scale -> SD_ERR_SHAPE.
 * ------------------------------------------------------------------------ */
sd_status sd_log_prior_bias(const int64_t* counts, int32_t V, double lambda, float scale,
                            float* out, void* stream);

/* ------------------------------------------------------------------------
 * sd_verify -- lossless speculative-sampling verification.
 *
 * Defined by: "LongSpark", sec. 2.1, eq. (1) (drafts are tested in order and
 * y_j is accepted with probability min(1, p_j(y_j) / q_j(y_j))), eq. (2)
 * (at the first rejection the correction token is drawn from
 * [p_j - q_j]_+ / sum [p_j - q_j]_+) and the text after eq. (2) (if every
 * tested draft is accepted one more token is drawn from the target's next
 * distribution); "ForeSpark", sec. 4.4 (only a prefix of b_b <= K_b drafts is
 * verified; the target scores them as one packed batch).
 *
 * Request b owns target rows t_off[b] .. t_off[b+1]-1, i.e. b_b + 1 rows:
 * p_j = softmax(target_logits[t_off[b] + j - 1]) for j = 1 .. b_b + 1.  Its
 * drafts are draft_tokens[q_off[b] + j - 1] with distribution
 * q_j = exp(draft_logits[q_off[b] + j - 1] - draft_lse[...]).  For j = 1..b_b:
 * r_j = min(1, p_j(y_j) / q_j(y_j)) (1 if q_j(y_j) underflows to 0); y_j is
 * accepted iff u_j < r_j with u_j the stream-1 uniform of position j.  The
 * first rejection j gives accepted_len = j - 1 and next_token = Gumbel-max
 * draw from [p_j - q_j]_+ (from p_j if that is identically 0); if none is
 * rejected accepted_len = b_b and next_token is a Gumbel-max draw from
 * p_{b_b+1}.  Draws use the stream-2 uniforms of position j (b_b + 1 for the
 * bonus).  Probabilities are evaluated in fp32.
 *
 * Variants: with a pruned drafter vocabulary q_j is zero outside it (its
 * entry for target token v is draft_logits[.., draft_vocab_inv[v]], absent
 * when that is -1), which keeps verification lossless ("H-Spec", App. B.2).
 * With greedy = 1 both sides are at temperature 0: p_j and q_j are one-hot
 * at their argmax, so y_j is accepted iff it is the first argmax of
 * target_logits row j, and next_token is the first argmax of the first
 * rejected row, or of row b_b + 1 (the limit of the rules above; no
 * uniforms).
 *
 * Arguments
 *   target_logits fp32 [total_target_rows, V]
 *   t_off    int32 [batch+1], 0 <= b_b = t_off[b+1] - t_off[b] - 1 <= K_b
 *   draft_logits  fp32 [total_q, V], or [total_q, v_draft] with a pruned
 *                 vocabulary (as written by sd_lm_head_probs)
 *   draft_lse     fp32 [total_q] or NULL (then computed here; required with
 *                 a pruned vocabulary)
 *   draft_tokens  int32 [total_q]  target token ids
 *   q_off    int32 [batch+1]  as for sd_lm_head_probs
 *   draft_vocab_inv int32 [V] drafter entry of each target token, -1 if
 *            outside the drafter's vocabulary; NULL when it is not pruned
 *   v_draft  drafter vocabulary size (ignored when draft_vocab_inv is NULL)
 *   greedy   0 (speculative sampling) or 1 (temperature 0)
 *   req_id   uint32 [batch], seed: as for sd_lm_head_probs
 *   accepted_len int32 [batch] out;  next_token int32 [batch] out
 *   accept_ratio fp32 [total_q] out or NULL: r_j at every tested position,
 *                NaN at positions not tested
 * ------------------------------------------------------------------------ */
size_t sd_verify_workspace_size(int32_t batch, int32_t total_q,
                                int32_t total_target_rows, int32_t V);

sd_status sd_verify(const float* target_logits, const int32_t* t_off,
                    const float* draft_logits, const float* draft_lse,
                    const int32_t* draft_tokens, const int32_t* q_off,
                    int32_t batch, int32_t total_q, int32_t total_target_rows,
                    int32_t V, const int32_t* draft_vocab_inv, int32_t v_draft,
                    int32_t greedy, const uint32_t* req_id, uint64_t seed,
                    int32_t* accepted_len, int32_t* next_token,
                    float* accept_ratio, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SD_H */
