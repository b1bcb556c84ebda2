// C ABI of the draft-and-verify step (declared in include/sd.h, the ceiling
// probes in include/sd_probe.h): host-side
// validation, workspace layout and kernel launches.  No allocation, no
// synchronisation, no reads of device memory.
#include "sd.h"
#include "sd_probe.h"

#include <math.h>

#include <algorithm>
#include <mutex>

#include "sd_internal.h"

// Scratch of sd_draft_attn_noalloc (its work list and split-K partials): a
// file-scope device array, one copy per GPU, held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

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
  int32_t split, rows;
  int64_t max_items;
  size_t off_item_off, off_unit_off, off_lse, off_o, total;
};

AttnLayout attn_layout(int32_t batch, int32_t group, int32_t hkv, int32_t head_dim,
                       int32_t max_draft_k, int64_t max_total_ctx, int32_t split_tokens) {
  AttnLayout L;
  L.split = sd::attn_split_tokens(batch, hkv, max_total_ctx, split_tokens);
  L.rows = sd::attn_item_rows(group, max_draft_k);
  L.max_items = sd::attn_max_items(batch, hkv, max_total_ctx, L.split);
  L.off_item_off = 0;
  L.off_unit_off = align_up(static_cast<size_t>(batch + 1) * sizeof(int32_t));
  L.off_lse = L.off_unit_off + align_up(4 * static_cast<size_t>(batch + 1) * sizeof(int32_t));
  L.off_o = L.off_lse + align_up(static_cast<size_t>(L.max_items) * L.rows * sizeof(float));
  L.total = L.off_o + align_up(static_cast<size_t>(L.max_items) * L.rows * head_dim * sizeof(float));
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
  size_t off_row, off_samp, off_dec, total;
};

VerifyLayout verify_layout(int32_t batch, int32_t total_q, int32_t R, int32_t V) {
  VerifyLayout L;
  L.n_chunks = (V + sd::kVerifyChunk - 1) / sd::kVerifyChunk;
  L.n_schunks = (V + sd::kSampleChunk - 1) / sd::kSampleChunk;
  L.off_row = 0;
  L.off_samp = align_up(static_cast<size_t>(R + total_q) * L.n_chunks * sizeof(float4));
  L.off_dec = L.off_samp + align_up(static_cast<size_t>(batch) * L.n_schunks * 2 * sizeof(float4));
  L.total = L.off_dec + align_up(static_cast<size_t>(batch) * sizeof(float4));
  return L;
}

// Validation, work-list layout and launches of sd_draft_attn.  The scratch
// memory comes from `get_ws`: given the bytes the call needs it returns the
// status and, on SD_OK, a 16-byte aligned device buffer of at least that
// size (the caller's workspace, or the no-allocation variant's array).
template <typename GetWs>
sd_status draft_attn_impl(const void* q, const void* k_blk, const void* v_blk, const void* k_cache,
                          const void* v_cache, const int32_t* page_table, const int32_t* ctx_len,
                          const int32_t* q_off, int32_t batch, int32_t total_q, int32_t max_draft_k,
                          int32_t num_pages, int32_t max_pages, int32_t page_size,
                          int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                          int64_t max_total_ctx, int32_t split_tokens, float softmax_scale,
                          int32_t block_mask, int32_t window, const void* summary_keys,
                          const float* summary_values, int32_t n_summary, void* out,
                          GetWs get_ws, void* stream) {
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
  if (static_cast<int64_t>(group) * max_draft_k > sd::kAttnMaxRows) return SD_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * page_size > (int64_t(1) << 30)) return SD_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * max_pages > (int64_t(1) << 31) - 1) return SD_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_blk) || !aligned16(v_blk) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out))
    return SD_ERR_SHAPE;
  const AttnLayout L = attn_layout(batch, group, num_heads_kv, head_dim, max_draft_k, max_total_ctx,
                                   split_tokens);
  if (L.max_items > (int64_t(1) << 31) - 1) return SD_ERR_SHAPE;
  char* ws = nullptr;
  const sd_status wst = get_ws(L.total, &ws);
  if (wst != SD_OK) return wst;
  if (total_q == 0) return SD_OK;

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
  a.max_items = static_cast<int32_t>(L.max_items);
  a.rows = L.rows;
  {
    // longest prefix span one request can stream: the whole page table row,
    // or with a window its last W tokens from the page start below them
    const int64_t span = window > 0 ? std::min<int64_t>(int64_t(window) + 15, int64_t(max_pages) * 16)
                                    : int64_t(max_pages) * 16;
    // The automatic split is sized from the whole prefixes, which is what
    // the workspace size sees.  A window much shorter than them would leave
    // one item per (request, KV head) and most CUs idle, so the window is
    // cut into k pieces of at least 512 tokens, enough for two items per CU
    // slot (512 in all), when their items still fit the workspace.
    a.split_tokens = L.split;
    if (split_tokens == 0 && window > 0) {
      const int64_t pairs = static_cast<int64_t>(batch) * num_heads_kv;
      const int64_t k = std::min<int64_t>((512 + pairs - 1) / pairs, span / 512);
      if (k >= 2) {
        const int64_t s_w = ((span + k - 1) / k + 63) / 64 * 64;
        const int64_t items = pairs * ((span + s_w - 1) / s_w + (n_summary > 0 ? 1 : 0));
        if (s_w < L.split && items <= L.max_items) a.split_tokens = static_cast<int32_t>(s_w);
      }
    }
    const int64_t split = a.split_tokens;
    a.direct = span <= split && n_summary == 0 ? 1 : 0;
    // Work units per request: its prefix splits (at least one unit, the
    // block alone, for an empty prefix) and the summary unit.  The launch
    // covers the smaller of this bound and the workspace's, so that a short
    // window over long prefixes does not launch workgroups for work that
    // cannot exist.
    const int64_t per_req = std::max<int64_t>((span + split - 1) / split, 1) + (n_summary > 0 ? 1 : 0);
    a.max_units = static_cast<int32_t>(
        std::min<int64_t>(L.max_items / num_heads_kv, static_cast<int64_t>(batch) * per_req));
  }
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.item_off = reinterpret_cast<int32_t*>(ws + L.off_item_off);
  a.unit_off = reinterpret_cast<int32_t*>(ws + L.off_unit_off);
  a.part_lse = reinterpret_cast<float*>(ws + L.off_lse);
  a.part_o = reinterpret_cast<float*>(ws + L.off_o);
  return from_hip(sd::launch_draft_attn(a, head_dim, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------ no-allocation variant
// The device address of `scratch` (below the includes) is looked up once per
// device, with that device current, and only that address is ever handed to
// kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
sd_status scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SD_ERR_DEVICE;
  if (dev >= kMaxDevices) return SD_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return e == hipSuccess ? SD_ERR_DEVICE : from_hip(e);
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return SD_OK;
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
    case SD_ERR_SCRATCH: return "the call needs more scratch than the no-allocation variant's fixed device array holds";
    default: return "unknown status";
  }
}

const char* sd_version(void) { return "0.1.0"; }

sd_status sd_probe_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return SD_ERR_NULL;
  if (bytes < 16 || !aligned16(src)) return SD_ERR_SHAPE;
  return from_hip(sd::launch_probe_read(src, bytes, static_cast<uint32_t*>(sink),
                                        static_cast<hipStream_t>(stream)));
}

int64_t sd_probe_mfma_flops(int32_t iters) {
  // 512 workgroups x 4 waves x iters x 8 MFMAs x (2 x 32 x 32 x 16) flops
  return iters < 1 ? 0 : static_cast<int64_t>(512) * 4 * iters * 8 * 2 * 32 * 32 * 16;
}

sd_status sd_probe_mfma(int32_t iters, void* sink, void* stream) {
  if (!sink) return SD_ERR_NULL;
  if (iters < 1 || iters > (1 << 24)) return SD_ERR_SHAPE;
  return from_hip(sd::launch_probe_mfma(iters, static_cast<float*>(sink), static_cast<hipStream_t>(stream)));
}

size_t sd_draft_attn_workspace_size(int32_t batch, int32_t num_heads_q, int32_t num_heads_kv,
                                    int32_t head_dim, int32_t max_draft_k, int64_t max_total_ctx,
                                    int32_t split_tokens) {
  if (batch < 1 || num_heads_kv < 1 || num_heads_q < num_heads_kv || head_dim < 1 ||
      max_draft_k < 1 || max_total_ctx < 0 || split_tokens < 0)
    return 0;
  return attn_layout(batch, num_heads_q / num_heads_kv, num_heads_kv, head_dim, max_draft_k,
                     max_total_ctx, split_tokens).total;
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
  auto ws = [&](size_t need, char** p) -> sd_status {
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SD_ERR_WORKSPACE;
    *p = static_cast<char*>(workspace);
    return SD_OK;
  };
  return draft_attn_impl(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, q_off, batch,
                         total_q, max_draft_k, num_pages, max_pages, page_size, num_heads_q,
                         num_heads_kv, head_dim, max_total_ctx, split_tokens, softmax_scale,
                         block_mask, window, summary_keys, summary_values, n_summary, out, ws,
                         stream);
}

size_t sd_draft_attn_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

sd_status sd_draft_attn_noalloc(const void* q, const void* k_blk, const void* v_blk,
                                const void* k_cache, const void* v_cache,
                                const int32_t* page_table, const int32_t* ctx_len,
                                const int32_t* q_off, int32_t batch, int32_t total_q,
                                int32_t max_draft_k, int32_t num_pages, int32_t max_pages,
                                int32_t page_size, int32_t num_heads_q, int32_t num_heads_kv,
                                int32_t head_dim, int64_t max_total_ctx, int32_t split_tokens,
                                float softmax_scale, int32_t block_mask, int32_t window,
                                const void* summary_keys, const float* summary_values,
                                int32_t n_summary, void* out, void* stream) {
  auto ws = [](size_t need, char** p) -> sd_status {
    if (need > kNoAllocScratchBytes) return SD_ERR_SCRATCH;
    return scratch_of_current_device(p);
  };
  return draft_attn_impl(q, k_blk, v_blk, k_cache, v_cache, page_table, ctx_len, q_off, batch,
                         total_q, max_draft_k, num_pages, max_pages, page_size, num_heads_q,
                         num_heads_kv, head_dim, max_total_ctx, split_tokens, softmax_scale,
                         block_mask, window, summary_keys, summary_values, n_summary, out, ws,
                         stream);
}

// Workspace of a whole-prefix initialisation: the slices' partial states.
static size_t summary_ws_bytes(int64_t batch, int64_t hkv, int64_t n_summary, int64_t head_dim) {
  const size_t parts = static_cast<size_t>(sd::summary_init_slots(batch, hkv) * n_summary);
  return align_up(parts * 2 * sizeof(float)) + align_up(parts * head_dim * sizeof(float));
}

size_t sd_summary_workspace_size(int32_t batch, int32_t num_heads_kv, int32_t n_summary,
                                 int32_t head_dim, int32_t max_pages, int32_t page_size) {
  if (batch < 1 || num_heads_kv < 1 || n_summary < 1 || head_dim < 1 || max_pages < 1 ||
      page_size != 16)
    return 0;
  return summary_ws_bytes(batch, num_heads_kv, n_summary, head_dim);
}

sd_status sd_summary_update(const void* summary_queries, const void* k_cache, const void* v_cache,
                            const int32_t* page_table, const int32_t* ctx_len,
                            const int32_t* accepted_len, int32_t batch, int32_t num_pages,
                            int32_t max_pages, int32_t page_size, int32_t num_heads_kv,
                            int32_t head_dim, int32_t n_summary, float softmax_scale,
                            float* summary_values, float* summary_lse, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!summary_queries || !k_cache || !v_cache || !page_table || !ctx_len || !summary_values ||
      !summary_lse)
    return SD_ERR_NULL;
  if (batch < 1 || num_pages < 1 || max_pages < 1 || page_size != 16 || num_heads_kv < 1 ||
      (head_dim != 64 && head_dim != 128) || n_summary < 1 || n_summary > sd::kSummaryMax ||
      !(softmax_scale > 0.f) || !isfinite(softmax_scale))
    return SD_ERR_SHAPE;
  if (static_cast<int64_t>(max_pages) * page_size > (int64_t(1) << 30)) return SD_ERR_SHAPE;
  if (static_cast<int64_t>(batch) * max_pages > (int64_t(1) << 31) - 1 ||
      sd::summary_init_slots(batch, num_heads_kv) > (int64_t(1) << 31) - 1)
    return SD_ERR_SHAPE;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(summary_queries))
    return SD_ERR_SHAPE;
  sd::SummaryArgs a{};
  if (!accepted_len) {
    const size_t need = summary_ws_bytes(batch, num_heads_kv, n_summary, head_dim);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SD_ERR_WORKSPACE;
    const size_t parts = static_cast<size_t>(sd::summary_init_slots(batch, num_heads_kv) * n_summary);
    char* w = static_cast<char*>(workspace);
    a.part_ml = reinterpret_cast<float2*>(w);
    a.part_o = reinterpret_cast<float*>(w + align_up(parts * 2 * sizeof(float)));
  }
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
  a.head_dim = head_dim;
  a.scale = softmax_scale;
  return from_hip(sd::launch_summary(a, static_cast<hipStream_t>(stream)));
}

size_t sd_schedule_workspace_size(int32_t n, int32_t r, int32_t max_rows, int32_t m) {
  if (n < 1 || r < 1 || max_rows < 0 || m < 1) return 0;
  return align_up(static_cast<size_t>(n) * r * sizeof(float)) +
         align_up(static_cast<size_t>(n) * (sd::kSchedMaxK + 1) * sizeof(float)) +
         align_up(static_cast<size_t>(max_rows) * m * sizeof(float)) +
         align_up(static_cast<size_t>(sd::kSchedSplitK) * n * r * sizeof(float));
}

sd_status sd_schedule_draft(const void* ctx_feat, const void* anchor_emb, const void* w_c,
                            const void* w_e, const float* b_u, const void* w_o, const float* b_o,
                            const float* cal_scale, const float* cal_bias, int32_t n, int32_t d_h,
                            int32_t r, int32_t K, const int32_t* draft_caps, const float* draft_lat,
                            int32_t n_draft_buckets, const int32_t* verify_caps,
                            const float* verify_lat, int32_t n_verify_buckets, int32_t n_nonspec,
                            float* logits, float* scores, int32_t* draft_len, int32_t* q_off,
                            int32_t* verify_budget, float* objective, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!ctx_feat || !anchor_emb || !w_c || !w_e || !w_o || !draft_caps || !draft_lat ||
      !verify_caps || !verify_lat || !logits || !scores || !draft_len || !verify_budget)
    return SD_ERR_NULL;
  if (n < 1 || n > sd::kSchedMaxRequests || K < 1 || K > sd::kSchedMaxK ||
      n * K > sd::kSchedMaxEntries || d_h < 16 || d_h % 16 != 0 || r < 16 || r % 16 != 0 ||
      d_h > 65536 || r > 65536 || n_draft_buckets < 1 || n_verify_buckets < 1 ||
      n_draft_buckets > 4096 || n_verify_buckets > 4096 || n_nonspec < 0)
    return SD_ERR_SHAPE;
  if (!aligned16(ctx_feat) || !aligned16(anchor_emb) || !aligned16(w_c) || !aligned16(w_e))
    return SD_ERR_SHAPE;
  const size_t need = sd_schedule_workspace_size(n, r, 0, 1);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SD_ERR_WORKSPACE;
  float* u = static_cast<float*>(workspace);
  sd::SchedGemmArgs g;
  g.a1 = static_cast<const uint16_t*>(ctx_feat);
  g.b1 = static_cast<const uint16_t*>(w_c);
  g.a2 = static_cast<const uint16_t*>(anchor_emb);
  g.b2 = static_cast<const uint16_t*>(w_e);
  g.bias = b_u;
  g.c = u;
  // after u and the rewards (the post-draft slot is empty: max_rows = 0)
  g.part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                    align_up(static_cast<size_t>(n) * r * sizeof(float)) +
                                    align_up(static_cast<size_t>(n) * (sd::kSchedMaxK + 1) * sizeof(float)));
  g.ksplit = sd::kSchedSplitK;
  g.M = n;
  g.N = r;
  g.K = d_h;
  g.silu = 1;
  sd::SchedArgs a;
  a.u = u;
  a.w_o = static_cast<const uint16_t*>(w_o);
  a.b_o = b_o;
  a.cal_scale = cal_scale;
  a.cal_bias = cal_bias;
  a.d_caps = draft_caps;
  a.d_lat = draft_lat;
  a.v_caps = verify_caps;
  a.v_lat = verify_lat;
  a.logits = logits;
  a.rewards = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       align_up(static_cast<size_t>(n) * r * sizeof(float)));
  a.scores = scores;
  a.draft_len = draft_len;
  a.q_off = q_off;
  a.budget = verify_budget;
  a.objective = objective;
  a.n = n;
  a.r = r;
  a.K = K;
  a.n_dbuckets = n_draft_buckets;
  a.n_vbuckets = n_verify_buckets;
  a.n_nonspec = n_nonspec;
  return from_hip(sd::launch_schedule_draft(g, a, static_cast<hipStream_t>(stream)));
}

sd_status sd_schedule_verify(const void* hidden, const void* w_s, const void* e_pred,
                             const float* w, float bias, const float* temperature,
                             const int32_t* anchor_tokens, const int32_t* draft_tokens,
                             const int32_t* q_off, const int32_t* verify_budget, int32_t n,
                             int32_t max_rows, int32_t H, int32_t m, int32_t V, int32_t K,
                             float* accept_prob, float* survival, int32_t* verify_len,
                             int32_t* t_off, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!hidden || !w_s || !e_pred || !w || !anchor_tokens || !draft_tokens || !q_off ||
      !verify_budget || !accept_prob || !survival || !verify_len)
    return SD_ERR_NULL;
  if (n < 1 || n > sd::kSchedMaxRequests || max_rows < 1 || max_rows > sd::kSchedMaxEntries ||
      H < 16 || H % 16 != 0 || H > 65536 || m < 16 || m % 16 != 0 || m > 65536 || V < 1 ||
      K < 1 || K > sd::kSchedMaxK || !isfinite(bias))
    return SD_ERR_SHAPE;
  if (!aligned16(hidden) || !aligned16(w_s)) return SD_ERR_SHAPE;
  const size_t need = sd_schedule_workspace_size(1, 1, max_rows, m);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SD_ERR_WORKSPACE;
  float* sh = static_cast<float*>(workspace);
  sd::SchedGemmArgs g;
  g.a1 = static_cast<const uint16_t*>(hidden);
  g.b1 = static_cast<const uint16_t*>(w_s);
  g.a2 = nullptr;
  g.b2 = nullptr;
  g.bias = nullptr;
  g.c = sh;
  g.part = nullptr;   // many rows fill the GPU without splitting K (a 4-way split measured slower)
  g.ksplit = 1;
  g.M = max_rows;
  g.N = m;
  g.K = H;
  g.silu = 0;
  sd::SchedPostArgs a;
  a.hidden = static_cast<const uint16_t*>(hidden);
  a.sh = sh;
  a.e_pred = static_cast<const uint16_t*>(e_pred);
  a.w = w;
  a.temperature = temperature;
  a.anchor = anchor_tokens;
  a.tokens = draft_tokens;
  a.q_off = q_off;
  a.budget = verify_budget;
  a.prob = accept_prob;
  a.survival = survival;
  a.verify_len = verify_len;
  a.t_off = t_off;
  a.bias = bias;
  a.n = n;
  a.M = max_rows;
  a.H = H;
  a.ms = m;
  a.V = V;
  a.K = K;
  return from_hip(sd::launch_schedule_verify(g, a, static_cast<hipStream_t>(stream)));
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

size_t sd_markov_workspace_size(int32_t batch, int32_t V, int32_t max_draft_k) {
  if (batch < 1 || V < 1 || max_draft_k < 1) return 0;
  const size_t cells = static_cast<size_t>(max_draft_k) * batch;
  const size_t draw = static_cast<size_t>(max_draft_k) * sd::kMarkovCells * sd::markov_cell_stride(batch);
  return align_up(cells * sd::markov_parts(V) * sizeof(float2)) +
         align_up(draw * sizeof(unsigned long long));
}

sd_status sd_markov_sample(float* logits, float* lse, int32_t* draft_tokens,
                           const int32_t* anchor_tokens, const void* w_c, const void* e_c,
                           float alpha, const float* vocab_bias, int32_t greedy, const int32_t* q_off, int32_t batch, int32_t M, int32_t V, int32_t r,
                           int32_t max_draft_k, const uint32_t* req_id, uint64_t seed,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !lse || !draft_tokens || !anchor_tokens || !w_c || !e_c || !q_off || !req_id)
    return SD_ERR_NULL;
  if (batch < 1 || M < 0 || V < 1 || r < 16 || r % 16 != 0 || r > 65536 || max_draft_k < 0 ||
      max_draft_k > 4096)
    return SD_ERR_SHAPE;
  if (!aligned16(w_c) || !aligned16(e_c) || !isfinite(alpha) || (greedy != 0 && greedy != 1))
    return SD_ERR_SHAPE;
  if (static_cast<int64_t>(max_draft_k) * batch * sd::markov_parts(V) > (int64_t(1) << 31) - 1)
    return SD_ERR_SHAPE;
  if (M == 0 || max_draft_k == 0) return SD_OK;
  const size_t need = sd_markov_workspace_size(batch, V, max_draft_k);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SD_ERR_WORKSPACE;
  sd::MarkovArgs a;
  a.logits = logits;
  a.lse = lse;
  a.tokens = draft_tokens;
  a.anchor = anchor_tokens;
  a.w_c = static_cast<const uint16_t*>(w_c);
  a.e_c = static_cast<const uint16_t*>(e_c);
  a.vbias = vocab_bias;
  a.alpha = alpha;
  a.greedy = greedy;
  a.q_off = q_off;
  a.req_id = req_id;
  const size_t cells = static_cast<size_t>(max_draft_k) * batch;
  a.part = static_cast<float2*>(workspace);
  a.cell = reinterpret_cast<unsigned long long*>(
      static_cast<char*>(workspace) + align_up(cells * sd::markov_parts(V) * sizeof(float2)));
  a.batch = batch;
  a.M = M;
  a.V = V;
  a.r = r;
  a.max_k = max_draft_k;
  a.n_chunks = sd::markov_chunks(V);
  a.n_parts = sd::markov_parts(V);
  a.cell_stride = sd::markov_cell_stride(batch);
  a.vec4 = (V % 4 == 0 && aligned16(logits) && (!vocab_bias || aligned16(vocab_bias))) ? 1 : 0;
  a.key0 = static_cast<uint32_t>(seed);
  a.key1 = static_cast<uint32_t>(seed >> 32);
  return from_hip(sd::launch_markov(a, static_cast<hipStream_t>(stream)));
}

sd_status sd_log_prior_bias(const int64_t* counts, int32_t V, double lambda, float scale, float* out,
                            void* stream) {
  if (!counts || !out) return SD_ERR_NULL;
  if (V < 1 || !(lambda > 0.0) || !isfinite(lambda) || !isfinite(scale)) return SD_ERR_SHAPE;
  return from_hip(sd::launch_log_prior_bias(counts, V, lambda, scale, out, static_cast<hipStream_t>(stream)));
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
  a.decision = reinterpret_cast<float4*>(ws + L.off_dec);
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
