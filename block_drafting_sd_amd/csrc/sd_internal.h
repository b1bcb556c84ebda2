// Launch-argument structs and launcher entry points behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sd {

// Launch `k(args)` and return that launch's own status.  (The thread's
// last-error state is not consulted: it may hold a stale, unrelated status
// such as hipErrorNotReady left by an event or stream query of the caller.)
template <typename Arg>
hipError_t launch_kernel(void (*k)(Arg), dim3 grid, dim3 block, hipStream_t s, Arg arg) {
  void* argv[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, argv, 0, s);
}

// ----------------------------------------------------------- draft attention
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* ctx_len;
  const int32_t* q_off;
  uint16_t* out;
  int32_t batch, total_q, max_draft_k, num_pages, max_pages;
  int32_t hq, hkv, group;
  int32_t block_mask;     // 0: bidirectional inside the block; 1: causal inside the block
  int32_t window;         // 0: the whole prefix; W > 0: only its last W tokens
  const uint16_t* sum_k;  // [hkv][n_summary][D] summary keys, or null
  const float* sum_v;     // [batch][hkv][n_summary][D] summary values
  int32_t n_summary;      // 0 when there is no summary
  int32_t split_tokens;   // prefix tokens per work item (multiple of 64, <= 32768)
  int32_t max_items;      // work items the partial buffers hold
  int32_t max_units;      // bound on the work units (request, split) of the call
  int32_t rows;           // query rows per work item: 64 (two waves) or 128 (four)
  int32_t direct;         // 1: every request is at most one work item (its prefix span fits
                          // one split and there is no summary), so the item of a request
                          // writes its rows itself: no work list, no partials, no merge
  float scale_log2;       // softmax_scale * log2(e)
  int32_t* item_off;      // [batch + 1] first work item of each request
  int32_t* unit_off;      // [3][batch + 1] first unit of each request among the block
                          // (+ summary) units, the full-length and the last prefix splits;
                          // then [batch + 1]: the requests of the last splits in run order
  float* part_lse;        // [max_items][rows]       (log2 units)
  float* part_o;          // [max_items][D/4][rows][4]
};

constexpr int kAttnMaxRows = 128;    // query rows of one (request, kv head): G * K_b
// Query rows per work item for a group size and draft-budget bound.
inline int32_t attn_item_rows(int32_t group, int32_t max_draft_k) {
  return static_cast<int64_t>(group) * max_draft_k <= 64 ? 64 : 128;
}
constexpr int kAttnTile = 32;        // keys per inner tile (two 16-token pages)
constexpr int kAttnStages = 4;       // LDS ring stages of the prefix stream
constexpr int kAttnMaxSplitPages = 2048;   // split_tokens <= 2048 * 16
constexpr int kAttnMaxSummary = 64;  // summary entries per KV head
constexpr int kAttnLocalScan = 64;   // batches up to this size: each split-K workgroup
                                     // scans the requests itself (no work-list launch)
constexpr int kAttnSortMax = 1024;   // batches up to this size: last splits run longest first

int64_t attn_max_items(int32_t batch, int32_t hkv, int64_t max_total_ctx,
                       int32_t split_tokens);
int32_t attn_split_tokens(int32_t batch, int32_t hkv, int64_t max_total_ctx, int32_t requested);
hipError_t launch_draft_attn(const AttnArgs& a, int head_dim, hipStream_t s);

// ------------------------------------------------------------ context summary
struct SummaryArgs {
  const uint16_t* u;          // [hkv][n_summary][D] summary queries
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;  // [batch][max_pages]
  const int32_t* ctx_len;     // [batch]
  const int32_t* accepted;    // [batch], or null to initialise from the prefix
  float* z;                   // [batch][hkv][n_summary][D]
  float* c;                   // [batch][hkv][n_summary]
  // slices of a whole-prefix initialisation: partial states per slice slot
  // [slots][n_summary] (max in base 2, sum) and [slots][n_summary][D]
  // (unnormalised values), in the workspace
  float2* part_ml;
  float* part_o;
  int32_t batch, hkv, n_summary, num_pages, max_pages, head_dim;
  float scale;
};

constexpr int kSummaryMax = 64;            // summary entries per KV head
constexpr int kSummaryInitWaves = 1024;    // waves of an initialisation (one per SIMD)
constexpr int kSummaryMinSplit = 512;      // fewest rows per wave

// Partial slots of an initialisation: the piece of pair p that wave w covers
// goes to slot p + w, so kSummaryInitWaves + batch * hkv of them.
int64_t summary_init_slots(int64_t batch, int64_t hkv);

// Launches summary_rows (and, for an initialisation, summary_merge).
hipError_t launch_summary(const SummaryArgs& a, hipStream_t s);

// ------------------------------------------------------------- scheduling
struct SchedGemmArgs {        // c = a1 b1^T (+ a2 b2^T) (+ bias, SiLU)
  const uint16_t* a1;         // [M][K]
  const uint16_t* b1;         // [N][K]
  const uint16_t* a2;         // [M][K] or null
  const uint16_t* b2;         // [N][K]
  const float* bias;          // [N] or null
  float* c;                   // [M][N]
  float* part;                // [ksplit][M][N] partial sums (ksplit > 1)
  int32_t M, N, K, silu, ksplit;
};
constexpr int kSchedSplitK = 8;   // K splits of the pre-draft estimator GEMM (few rows)

struct SchedArgs {
  const float* u;             // [n][r] estimator hidden layer
  const uint16_t* w_o;        // [T][r]
  const float* b_o;           // [T] or null
  const float* cal_scale;     // [T] or null
  const float* cal_bias;      // [T] or null
  const int32_t* d_caps;      // [n_dbuckets] drafter token capacities (increasing)
  const float* d_lat;         // [n_dbuckets]
  const int32_t* v_caps;      // [n_vbuckets] verifier token capacities (increasing)
  const float* v_lat;         // [n_vbuckets]
  float* logits;              // [n][T]
  float* rewards;             // [n][K + 1] reward curves (workspace)
  float* scores;              // [n][K]
  int32_t* draft_len;         // [n]
  int32_t* q_off;             // [n + 1] or null
  int32_t* budget;            // [1]
  float* objective;           // [1] or null
  int32_t n, r, K, n_dbuckets, n_vbuckets, n_nonspec;
};

struct SchedPostArgs {
  const uint16_t* hidden;     // [M][H]
  const float* sh;            // [M][ms] = hidden W_s^T
  const uint16_t* e_pred;     // [V][ms]
  const float* w;             // [H + ms]
  const float* temperature;   // [K] or null
  const int32_t* anchor;      // [n]
  const int32_t* tokens;      // [M]
  const int32_t* q_off;       // [n + 1]
  const int32_t* budget;      // [1]
  float* prob;                // [M]
  float* survival;            // [M]
  int32_t* verify_len;        // [n]
  int32_t* t_off;             // [n + 1] or null
  float bias;
  int32_t n, M, H, ms, V, K;
};

constexpr int kSchedMaxEntries = 4096;   // n K (and draft rows) sorted in one workgroup
constexpr int kSchedMaxRequests = 1024;
constexpr int kSchedMaxK = 32;

hipError_t launch_sched_gemm(const SchedGemmArgs& g, hipStream_t s);
hipError_t launch_schedule_draft(const SchedGemmArgs& g, const SchedArgs& a, hipStream_t s);
hipError_t launch_schedule_verify(const SchedGemmArgs& g, const SchedPostArgs& a, hipStream_t s);

// ------------------------------------------------------------------ LM head
struct LmArgs {
  const uint16_t* hidden;   // [M, H]
  const uint16_t* w;        // [V, H]
  const int32_t* q_off;     // [batch + 1]
  const uint32_t* req_id;   // [batch]
  float* logits;            // [M, V]
  float* lse;               // [M]
  int32_t* tokens;          // [M]
  float4* part;             // [M][n_vt] (max, sumexp, best key, best index)
  const int32_t* vmap;      // [V] W row of each drafter vocab entry, or null (identity)
  int32_t w_rows;           // rows of w (bound for vmap entries)
  int32_t greedy;           // 1: tokens are argmax of the logits (no uniforms)
  int32_t M, H, V, batch, n_vt, n_mt;
  uint32_t key0, key1;
};

constexpr int kLmBV = 128;   // vocab rows per workgroup tile
constexpr int kLmBM = 256;   // draft rows per workgroup tile
constexpr int kLmHMultiple = 64;   // H must be a multiple of this

hipError_t launch_lm_head(const LmArgs& a, hipStream_t s);

// ------------------------------------------------------- Markov correction
struct MarkovArgs {
  float* logits;              // [M][V] base logits in, corrected out
  float* lse;                 // [M]
  int32_t* tokens;            // [M]
  const int32_t* anchor;      // [batch] committed tokens y_0
  const uint16_t* w_c;        // [V][r]
  const uint16_t* e_c;        // [V][r]
  const float* vbias;         // [V] added to every row, or null
  float alpha;                // scale of the correction
  int32_t greedy;             // 1: draws are the argmax of the corrected logits
  const int32_t* q_off;       // [batch + 1]
  const uint32_t* req_id;     // [batch]
  float2* part;               // [max_k][batch][n_parts] (max, sum exp) (workspace)
  unsigned long long* cell;   // [max_k][kMarkovCells][cell_stride] packed draws (workspace)
  int32_t batch, M, V, r, max_k, n_chunks, n_parts, cell_stride;
  int32_t vec4;               // logits rows 16-byte aligned (V % 4 == 0, aligned base)
  uint32_t key0, key1;
};

constexpr int kMarkovCells = 16;     // draw cells per (position, request)
inline int32_t markov_cell_stride(int32_t batch) { return (batch + 63) / 64 * 64; }  // 512-byte groups
int32_t markov_chunks(int32_t V);   // 128-row vocab chunks
int32_t markov_parts(int32_t V);    // partial statistics per (position, request)
hipError_t launch_markov(const MarkovArgs& a, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(int iters, float* sink, hipStream_t s);
hipError_t launch_log_prior_bias(const int64_t* counts, int V, double lam, float scale, float* out,
                                 hipStream_t s);

// ------------------------------------------------------------------- verify
struct VerifyArgs {
  const float* target;      // [R, V]
  const int32_t* t_off;     // [batch + 1]
  const float* draft;       // [total_q, v_draft]
  const float* draft_lse;   // [total_q] or null
  const int32_t* vinv;      // [V] drafter vocab entry of each target entry (-1: none), or null
  int32_t v_draft;          // row length of draft (V unless the drafter vocab is pruned)
  int32_t greedy;           // 1: temperature 0 on both sides
  const int32_t* tokens;    // [total_q]
  const int32_t* q_off;     // [batch + 1]
  const uint32_t* req_id;   // [batch]
  int32_t* accepted;        // [batch]
  int32_t* next_token;      // [batch]
  float* accept_ratio;      // [total_q] or null
  float4* row_part;         // [(R + total_q) * n_chunks] (max, sumexp, argmax, -)
  float4* samp_part;        // [batch * n_schunks * 2]
  float4* decision;         // [batch] (accepted as int bits or -1, lse_p, lse_q, tested as int bits)
  int32_t batch, total_q, R, V, n_chunks, n_schunks;
  uint32_t key0, key1;
};

constexpr int kVerifyChunk = 8192;   // vocab entries per row-statistics workgroup
constexpr int kSampleChunk = 2048;   // vocab entries per sampling workgroup

hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);

}  // namespace sd
