// C ABI of the draft-and-verify step (declared in include/sd.h): host-side
// validation, workspace layout and kernel launches.  No allocation, no
// synchronisation, no reads of device memory.
#include "sd.h"

#include <math.h>

#include "sd_internal.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sd_status from_hip(hipError_t e) {
  if (e == hipSuccess) return SD_OK;
  if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction ||
      e == hipErrorNoDevice || e == hipErrorInvalidDevice)
    return SD_ERR_DEVICE;
  return SD_ERR_LAUNCH;
}

// ------------------------------------------------------------ attention
struct AttnLayout {
  int32_t split;
  int64_t max_items;
  size_t off_item_off, off_lse, off_o, total;
};

AttnLayout attn_layout(int32_t batch, int32_t hkv, int32_t head_dim, int64_t max_total_ctx,
                       int32_t split_tokens) {
  AttnLayout L;
  L.split = sd::attn_split_tokens(hkv, max_total_ctx, split_tokens);
  L.max_items = sd::attn_max_items(batch, hkv, max_total_ctx, L.split);
  L.off_item_off = 0;
  L.off_lse = align_up(static_cast<size_t>(batch + 1) * sizeof(int32_t));
  L.off_o = L.off_lse + align_up(static_cast<size_t>(L.max_items) * sd::kAttnRows * sizeof(float));
  L.total = L.off_o + align_up(static_cast<size_t>(L.max_items) * sd::kAttnRows * head_dim * sizeof(float));
  return L;
}

// --------------------------------------------------------------- LM head
struct LmLayout {
  int32_t n_vt, n_mt;
  size_t total;
};

LmLayout lm_layout(int32_t M, int32_t V) {
  LmLayout L;
  L.n_vt = (V + sd::kLmBV - 1) / sd::kLmBV;
  L.n_mt = (M + sd::kLmBM - 1) / sd::kLmBM;
  L.total = align_up(static_cast<size_t>(M) * L.n_vt * sizeof(float4));
  return L;
}

// ---------------------------------------------------------------- verify
struct VerifyLayout {
  int32_t n_chunks, n_schunks;
  size_t off_row, off_samp, total;
};

VerifyLayout verify_layout(int32_t batch, int32_t total_q, int32_t R, int32_t V) {
  VerifyLayout L;
  L.n_chunks = (V + sd::kVerifyChunk - 1) / sd::kVerifyChunk;
  L.n_schunks = (V + sd::kSampleChunk - 1) / sd::kSampleChunk;
  L.off_row = 0;
  L.off_samp = align_up(static_cast<size_t>(R + total_q) * L.n_chunks * sizeof(float4));
  L.total = L.off_samp + align_up(static_cast<size_t>(batch) * L.n_schunks * 2 * sizeof(float4));
  return L;
}

}  // namespace

extern "C" {

const char* sd_status_str(sd_status s) {
  switch (s) {
    case SD_OK: return "ok";
    case SD_ERR_NULL: return "a required pointer is NULL";
    case SD_ERR_SHAPE: return "a size argument is out of the supported range (or a pointer is not 16-byte aligned)";
    case SD_ERR_WORKSPACE: return "workspace is NULL or smaller than required";
    case SD_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case SD_ERR_DEVICE: return "the current device cannot run gfx950 code";
    default: return "unknown status";
  }
}

const char* sd_version(void) { return "0.1.0"; }

size_t sd_draft_attn_workspace_size(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                    int32_t head_dim, int64_t max_total_ctx, int32_t split_tokens) {
  (void)num_heads_q;
  if (batch < 1 || num_heads_kv < 1 || head_dim < 1 || max_total_ctx < 0 || split_tokens < 0)
    return 0;
  return attn_layout(batch, num_heads_kv, head_dim, max_total_ctx, split_tokens).total;
}

sd_status sd_draft_attn(const void* q, const void* k_blk, const void* v_blk, const void* k_cache,
                        const void* v_cache, const int32_t* page_table, const int32_t* ctx_len,
                        const int32_t* q_off, int32_t batch, int32_t total_q, int32_t max_draft_k,
                        int32_t num_pages, int32_t max_pages, int32_t page_size,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        int64_t max_total_ctx, int32_t split_tokens, float softmax_scale,
                        int32_t block_mask, int32_t window, const void* summary_keys,
                        const float* summary_values, int32_t n_summary,
                        void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_blk || !v_blk || !k_cache || !v_cache || !page_table || !ctx_len || !q_off || !out)
    return SD_ERR_NULL;
  if (n_summary > 0 && (!summary_keys || !summary_values)) return SD_ERR_NULL;
  if ((block_mask != SD_MASK_NONE && block_mask != SD_MASK_CAUSAL) || window < 0 || n_summary < 0 ||
      n_summary > sd::kAttnMaxSummary || !(softmax_scale > 0.f))
    return SD_ERR_SHAPE;
  if (n_summary > 0 && !aligned16(summary_keys)) return SD_ERR_SHAPE;
  if (batch < 1 || total_q < 0 || max_draft_k < 1 || num_pages < 1 || max_pages < 1 ||
      page_size != 16 || num_heads_kv < 1 || num_heads_q < num_heads_kv ||
      num_heads_q % num_heads_kv != 0 || (head_dim != 64 && head_dim != 128) ||
      max_total_ctx < 0 || split_tokens < 0 || split_tokens % 64 != 0 ||
      split_tokens > sd::kAttnMaxSplitPages * 16 || !isfinite(softmax_scale))
    return SD_ERR_SHAPE;
  const int32_t group = num_heads_q / num_heads_kv;
  if (static_cast<int64_t>(group) * max_draft_k > sd::kAttnRows) return SD_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * page_size > (int64_t(1) << 30)) return SD_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * max_pages > (int64_t(1) << 31) - 1) return SD_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out))
    return SD_ERR_SHAPE;
  const AttnLayout L = attn_layout(batch, num_heads_kv, head_dim, max_total_ctx, split_tokens);
  if (L.max_items > (int64_t(1) << 31) - 1) return SD_ERR_SHAPE;
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SD_ERR_WORKSPACE;
  if (total_q == 0) return SD_OK;

  char* ws = static_cast<char*>(workspace);
  sd::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k_blk = static_cast<const uint16_t*>(k_blk);
  a.v_blk = static_cast<const uint16_t*>(v_blk);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.page_table = page_table;
  a.ctx_len = ctx_len;
  a.q_off = q_off;
  a.out = static_cast<uint16_t*>(out);
  a.batch = batch;
  a.total_q = total_q;
  a.max_draft_k = max_draft_k;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.hq = num_heads_q;
  a.hkv = num_heads_kv;
  a.group = group;
  a.block_mask = block_mask;
  a.window = window;
  a.sum_k = n_summary > 0 ? static_cast<const uint16_t*>(summary_keys) : nullptr;
  a.sum_v = n_summary > 0 ? summary_values : nullptr;
  a.n_summary = n_summary;
  a.split_tokens = L.split;
  a.max_items = static_cast<int32_t>(L.max_items);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.item_off = reinterpret_cast<int32_t*>(ws + L.off_item_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.off_lse);
  a.part_o = reinterpret_cast<float*>(ws + L.off_o);
  return from_hip(sd::launch_draft_attn(a, head_dim, static_cast<hipStream_t>(stream)));
}

sd_status sd_summary_update(const void* summary_queries, const void* k_cache, const void* v_cache,
                            const int32_t* page_table, const int32_t* ctx_len,
                            const int32_t* accepted_len, int32_t batch, int32_t num_pages,
                            int32_t max_pages, int32_t page_size, int32_t num_heads_kv,
                            int32_t head_dim, int32_t n_summary, float softmax_scale,
                            float* summary_values, float* summary_lse, void* stream) {
  if (!summary_queries || !k_cache || !v_cache || !page_table || !ctx_len || !summary_values ||
      !summary_lse)
    return SD_ERR_NULL;
  if (batch < 1 || num_pages < 1 || max_pages < 1 || page_size != 16 || num_heads_kv < 1 ||
      (head_dim != 64 && head_dim != 128) || n_summary < 1 || n_summary > sd::kSummaryMax ||
      !(softmax_scale > 0.f) || !isfinite(softmax_scale))
    return SD_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * page_size > (int64_t(1) << 30)) return SD_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * max_pages > (int64_t(1) << 31) - 1 ||
      static_cast<int64_t>(batch) * num_heads_kv > (int64_t(1) << 31) - 1)
    return SD_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return SD_ERR_SHAPE;
  sd::SummaryArgs a;
  a.u = static_cast<const uint16_t*>(summary_queries);
  a.k_cache = static_cast<const uint16_t*>(k_cache);
  a.v_cache = static_cast<const uint16_t*>(v_cache);
  a.page_table = page_table;
  a.ctx_len = ctx_len;
  a.accepted = accepted_len;
  a.z = summary_values;
  a.c = summary_lse;
  a.batch = batch;
  a.hkv = num_heads_kv;
  a.n_summary = n_summary;
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.scale = softmax_scale;
  return from_hip(sd::launch_summary(a, head_dim, static_cast<hipStream_t>(stream)));
}

size_t sd_lm_head_workspace_size(int32_t M, int32_t V) {
  if (M < 1 || V < 1) return 0;
  return lm_layout(M, V).total;
}

sd_status sd_lm_head_probs(const void* hidden, const void* w_vocab, int32_t M, int32_t H, int32_t V,
                           const int32_t* q_off, int32_t batch, const uint32_t* req_id,
                           uint64_t seed, const int32_t* vocab_map, int32_t w_rows,
                           int32_t greedy, float* logits, float* lse, int32_t* draft_tokens,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!hidden || !w_vocab || !q_off || !req_id || !logits || !lse || !draft_tokens)
    return SD_ERR_NULL;
  if (M < 1 || batch < 1 || V < 1 || H < sd::kLmHMultiple || H > 65536 ||
      H % sd::kLmHMultiple != 0 || (greedy != 0 && greedy != 1) || (vocab_map && w_rows < 1))
    return SD_ERR_SHAPE;
  if (!aligned16(hidden) || !aligned16(w_vocab) || !aligned16(logits)) return SD_ERR_SHAPE;
  const LmLayout L = lm_layout(M, V);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SD_ERR_WORKSPACE;
  if (static_cast<int64_t>((L.n_vt + 7) / 8) * 8 * L.n_mt > (int64_t(1) << 31) - 1 ||
      static_cast<int64_t>(M) * L.n_vt > (int64_t(1) << 31) - 1)
    return SD_ERR_SHAPE;
  sd::LmArgs a;
  a.hidden = static_cast<const uint16_t*>(hidden);
  a.w = static_cast<const uint16_t*>(w_vocab);
  a.q_off = q_off;
  a.req_id = req_id;
  a.logits = logits;
  a.lse = lse;
  a.tokens = draft_tokens;
  a.part = static_cast<float4*>(workspace);
  a.vmap = vocab_map;
  a.w_rows = vocab_map ? w_rows : V;
  a.greedy = greedy;
  a.M = M;
  a.H = H;
  a.V = V;
  a.batch = batch;
  a.n_vt = L.n_vt;
  a.n_mt = L.n_mt;
  a.key0 = static_cast<uint32_t>(seed);
  a.key1 = static_cast<uint32_t>(seed >> 32);
  return from_hip(sd::launch_lm_head(a, static_cast<hipStream_t>(stream)));
}

size_t sd_verify_workspace_size(int32_t batch, int32_t total_q, int32_t total_target_rows, int32_t V) {
  if (batch < 1 || total_q < 0 || total_target_rows < 1 || V < 1) return 0;
  return verify_layout(batch, total_q, total_target_rows, V).total;
}

sd_status sd_verify(const float* target_logits, const int32_t* t_off, const float* draft_logits,
                    const float* draft_lse, const int32_t* draft_tokens, const int32_t* q_off,
                    int32_t batch, int32_t total_q, int32_t total_target_rows, int32_t V,
                    const int32_t* draft_vocab_inv, int32_t v_draft, int32_t greedy,
                    const uint32_t* req_id, uint64_t seed, int32_t* accepted_len,
                    int32_t* next_token, float* accept_ratio, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!target_logits || !t_off || !q_off || !req_id || !accepted_len || !next_token)
    return SD_ERR_NULL;
  if (total_q > 0 && (!draft_logits || !draft_tokens)) return SD_ERR_NULL;
  if (draft_vocab_inv && total_q > 0 && !draft_lse) return SD_ERR_NULL;
  if (batch < 1 || total_q < 0 || total_target_rows < 1 || V < 1 || (greedy != 0 && greedy != 1) ||
      (draft_vocab_inv && v_draft < 1))
    return SD_ERR_SHAPE;
  const VerifyLayout L = verify_layout(batch, total_q, total_target_rows, V);
  if (static_cast<int64_t>(total_target_rows + total_q) * L.n_chunks > (int64_t(1) << 31) - 1 ||
      static_cast<int64_t>(batch) * L.n_schunks > (int64_t(1) << 31) - 1)
    return SD_ERR_SHAPE;
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return SD_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  sd::VerifyArgs a;
  a.target = target_logits;
  a.t_off = t_off;
  a.draft = draft_logits;
  a.draft_lse = draft_lse;
  a.vinv = draft_vocab_inv;
  a.v_draft = draft_vocab_inv ? v_draft : V;
  a.greedy = greedy;
  a.tokens = draft_tokens;
  a.q_off = q_off;
  a.req_id = req_id;
  a.accepted = accepted_len;
  a.next_token = next_token;
  a.accept_ratio = accept_ratio;
  a.row_part = reinterpret_cast<float4*>(ws + L.off_row);
  a.samp_part = reinterpret_cast<float4*>(ws + L.off_samp);
  a.batch = batch;
  a.total_q = total_q;
  a.R = total_target_rows;
  a.V = V;
  a.n_chunks = L.n_chunks;
  a.n_schunks = L.n_schunks;
  a.key0 = static_cast<uint32_t>(seed);
  a.key1 = static_cast<uint32_t>(seed >> 32);
  return from_hip(sd::launch_verify(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
