// Draft-block attention over the target's paged KV cache.
//
// The K_b draft queries of request b attend, with one softmax and no mask, to
// the N_b prefix keys of the target's cache (read in place through the page
// table) and to the K_b keys of the draft block ("ForeSpark", sec. 4.1;
// "LongSpark", App. A.1, Fig. 6; "H-Spec", sec. 3.3.2).
//
// Work decomposition (split-K, flash-decoding style):
//   item = (request b, kv head g, split s); splits 0..ns_b-1 cover the prefix
//   in chunks of `split_tokens`, and the last of them also attends the K_b
//   draft-block keys (an empty prefix gets one item for the block alone; the
//   fixed-cost context adds one item for the summary entries).  All G*K_b
//   query rows of (b, g) share one item, so every prefix KV byte is read from
//   HBM exactly once.  Each item writes fp32 partial results (normalised
//   output and log-sum-exp), which `attn_combine` merges with the log-sum-exp
//   rule of "LongSpark", App. A.2, eq. (11); a (b, g) with a single item
//   writes its bf16 output directly and the merge skips it.  The hkv items of
//   one (request, split) are given neighbouring workgroup slots on one XCD
//   (`locate_item`): they walk the same pages, whose per-head slices are
//   adjacent in the cache, so each page is fetched as one contiguous block
//   through one L2 and one set of address translations.  With a shuffled
//   page table this is worth a few per cent of HBM bandwidth.
//
// Launch shapes: when the host can see that every request is at most one item
// per kv head (its streamable span fits one split, no summary), the item of
// workgroup slot u is request u itself and only the split-K kernel runs (no
// work list, no partials, no merge).  Otherwise the items are located through
// prefix sums over the requests: computed in LDS by every split-K workgroup
// for up to kAttnLocalScan requests, by the `attn_worklist` kernel above that.
//
// Prefix items stream the cache through a ring of NS LDS stages of 32 keys
// (two 16-token pages, 128*D bytes) filled by gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4): a load writes 16 bytes per lane straight into
// LDS without passing through registers, so NS-1 stages (NS-1 x 16 KiB at
// D = 128) are in flight per workgroup while the current one is computed.
// The KV loads use the non-temporal cache policy: a call reads every KV line
// exactly once, and streaming gigabytes through the caches with the default
// policy displaces what is reused (measured: 75% -> 85% of the HBM peak at
// 128K context, batch 16).
// Wave 0 fetches the stage's keys, wave 1 its values; each 1 KiB wave load is
// laid out so that lane l of the consuming wave reads its MFMA operand at
// byte 16 l of a 1 KiB chunk (conflict-free ds_read_b128).  The waits are
// explicit: a wave waits for its own loads of the stage (vmcnt), then a
// workgroup barrier publishes the stage to both waves and frees the stage
// computed in the previous iteration for the next loads.
//
// Inner tile (per wave, 32 query rows x 32 keys):
//   S^T[32 keys x 32 queries] = K * Q^T      (MFMA 32x32x16 bf16, D/16 steps)
//   O^T[D x 32 queries]     += V^T * P^T     (MFMA 32x32x16 bf16, 2 per 32 dims)
// The key order inside a tile is permuted so that the softmax values a lane
// holds after the first product are exactly the B operand of the second one
// (no LDS round trip).  All waves compute from the same stage: wave w owns
// query rows 32w .. 32w+31 of the item's rows (two waves for up to 64 rows,
// four for up to 128: large GQA groups).
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {

int32_t attn_split_tokens(int32_t batch, int32_t hkv, int64_t max_total_ctx, int32_t requested) {
  if (requested > 0) return requested;
  // The largest power of two in [2048, 32768] tokens that still leaves at
  // least 512 prefix items (two per CU) and at most the mean prefix length
  // (a ragged mix's long requests then spread over several items).
  // Measured on MI355X (attention call, % of 8 TB/s): 16 x 32K: 4096 66%,
  // 8192 69%, 16384 61%; 16 x 128K: 16384 73.8%, 32768 74.8%; 64 x 4K:
  // 1024 55%, 2048 60%, 4096 66%; 128 ragged 1K-128K: 4096 68%, 8192 70.0%,
  // 16384 70.5% (32768 56% before the block keys rode on the last split).
  // Powers of two divide the usual prefix lengths, so no request ends in a
  // short split (6144 at 32K: 54%).
  const int64_t work = static_cast<int64_t>(hkv) * max_total_ctx;
  const int64_t mean = batch > 0 ? max_total_ctx / batch : 0;
  int64_t s = 32768;
  while (s > 2048 && (work / s < 512 || s > mean)) s >>= 1;
  static_assert(32768 <= kAttnMaxSplitPages * 16, "split pages staged in LDS");
  return static_cast<int32_t>(s);
}

int64_t attn_max_items(int32_t batch, int32_t hkv, int64_t max_total_ctx,
                       int32_t split_tokens) {
  // A request has ceil(N_b / S) prefix items (one block item instead when
  // N_b = 0) and at most one summary item: fewer than N_b / S + 2 (exactly
  // that at N_b = 0), so the integer sum is at most floor(sum_b N_b / S) +
  // 2 * batch (a window only shortens the streamed range)
  return static_cast<int64_t>(hkv) * (max_total_ctx / split_tokens + 2 * static_cast<int64_t>(batch));
}

namespace {

struct ReqInfo {
  int n;        // prefix length N_b (clamped)
  int n0;       // first prefix token attended (N_b - W with a window, else 0)
  int a0;       // n0 rounded down to a page: the streamed range is [a0, n)
  int q0;       // first query row
  int kb;       // draft rows K_b (clamped)
  int ns;       // prefix splits
  int per;      // items per KV head: ns prefix splits, the block, the summary
};

__device__ __forceinline__ ReqInfo request_info(const AttnArgs& a, int b) {
  ReqInfo r;
  r.n = clampi(a.ctx_len[b], 0, a.max_pages * 16);
  r.n0 = a.window > 0 ? max(0, r.n - a.window) : 0;
  r.a0 = r.n0 & ~15;
  r.q0 = clampi(a.q_off[b], 0, a.total_q);
  r.kb = min(clampi(a.q_off[b + 1], r.q0, a.total_q) - r.q0, a.max_draft_k);
  r.ns = (r.n - r.a0 + a.split_tokens - 1) / a.split_tokens;
  // the draft block rides on the last prefix split; only an empty prefix
  // needs a block item of its own
  r.per = r.ns + (r.ns == 0 ? 1 : 0) + (a.n_summary > 0 ? 1 : 0);
  return r;
}

// Work units of a request, by kind: its block (and summary) units, its
// full-length prefix splits and its shorter last split (0 or 1).
__device__ __forceinline__ void unit_counts(const AttnArgs& a, const ReqInfo& r, int (&v)[3]) {
  v[0] = v[1] = v[2] = 0;
  if (r.kb <= 0) return;
  v[1] = (r.n - r.a0) / a.split_tokens;
  v[2] = r.ns - v[1];
  v[0] = r.per - r.ns;
}

// Exclusive prefix sums over the requests, by one workgroup of T threads:
// of each kind of unit (unit_off[c (batch + 1) + b], the execution order) and
// of the work items (item_off[b], the partials' slots), with the totals at
// index batch.  T requests per round: a shuffle scan inside each wave, then
// the sums of the preceding waves.  Then the order of the shorter last
// splits, which run last: unit_off[3 (batch + 1) + r] is the request whose
// last split has rank r, longest first (ties by request), so that the final
// round of workgroups ends evenly (up to MaxSort requests, ranked by
// counting; above that in request order).  Every thread of the workgroup
// calls it.
template <int T, int MaxSort>
__device__ void scan_units(const AttnArgs& a, int* unit_off, int* item_off) {
  constexpr int NW = T / 64;
  __shared__ int wsum[3][NW];
  __shared__ int carry[3];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < 3) carry[tid] = 0;
  __syncthreads();
  for (int base = 0; base < a.batch; base += T) {
    const int b = base + tid;
    int v[3] = {0, 0, 0};
    if (b < a.batch) unit_counts(a, request_info(a, b), v);
    int inc[3] = {v[0], v[1], v[2]};
#pragma unroll
    for (int off = 1; off < 64; off <<= 1)
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int t = __shfl_up(inc[c], off, 64);
        if (lane >= off) inc[c] += t;
      }
    if (lane == 63)
#pragma unroll
      for (int c = 0; c < 3; ++c) wsum[c][w] = inc[c];
    __syncthreads();
    int ex[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      int acc = carry[c];
      for (int i = 0; i < w; ++i) acc += wsum[c][i];
      ex[c] = acc + inc[c] - v[c];
    }
    if (b < a.batch) {
#pragma unroll
      for (int c = 0; c < 3; ++c) unit_off[c * (a.batch + 1) + b] = ex[c];
      item_off[b] = a.hkv * (ex[0] + ex[1] + ex[2]);
    }
    __syncthreads();   // every thread has read carry and wsum
    if (tid == T - 1)
#pragma unroll
      for (int c = 0; c < 3; ++c) carry[c] = ex[c] + v[c];
    __syncthreads();
  }
  if (tid == 0) {
#pragma unroll
    for (int c = 0; c < 3; ++c) unit_off[c * (a.batch + 1) + a.batch] = carry[c];
    item_off[a.batch] = a.hkv * (carry[0] + carry[1] + carry[2]);
  }
  __syncthreads();
  int* perm = unit_off + 3 * (a.batch + 1);
  const int* po = unit_off + 2 * (a.batch + 1);
  if (a.batch <= MaxSort) {
    __shared__ int s_len[MaxSort];   // length of b's shorter last split, or -1
    for (int b = tid; b < a.batch; b += T) {
      const ReqInfo r = request_info(a, b);
      int v[3];
      unit_counts(a, r, v);
      s_len[b] = v[2] ? (r.n - r.a0) - (r.ns - 1) * a.split_tokens : -1;
    }
    __syncthreads();
    for (int b = tid; b < a.batch; b += T) {
      const int lb = s_len[b];
      if (lb < 0) continue;
      int rank = 0;
      for (int c = 0; c < a.batch; ++c) {
        const int lc = s_len[c];
        rank += lc > lb || (lc == lb && c < b);
      }
      perm[rank] = b;
    }
  } else {
    for (int b = tid; b < a.batch; b += T)
      if (po[b + 1] > po[b]) perm[po[b]] = b;
  }
  __syncthreads();
}

// The work list in global memory, for batches too large for the split-K
// workgroups to scan themselves.
__global__ __launch_bounds__(1024) void attn_worklist(AttnArgs a) {
  scan_units<1024, kAttnSortMax>(a, a.unit_off, a.item_off);
}

// Work item of a workgroup.  A unit is one (request, split) -- a prefix split,
// the draft block or the summary; its hkv items (one per kv head) read the
// same pages, whose per-head slices are adjacent in the cache
// ([page][hkv][...]).  Units run in three groups: every block and summary
// unit (short), then every full-length prefix split, then the requests'
// shorter last splits, so that with ragged prefix lengths the last
// workgroups to start are short ones and the kernel's tail stays short.
// Workgroups are dealt to the 8 XCDs round robin, so blockIdx x runs on XCD
// x % 8; the mapping below gives the hkv items of a unit consecutive slots on
// one XCD: they run side by side, share that XCD's L2 and address
// translations, and fetch each page as one contiguous hkv-slice block.  The
// item (the slot of its partials) is item_off[b] + g per + split, whatever
// the order.  Returns false past the last item.
struct ItemLoc {
  int b, g, sp, item;
  ReqInfo r;
};

__device__ __forceinline__ bool locate_item(const AttnArgs& a, int block, const int* unit_off,
                                            const int* item_off, ItemLoc& L) {
  const int x = block & 7;
  const int k = block >> 3;
  const int u = (k / a.hkv) * 8 + x;       // unit, in execution order
  L.g = k % a.hkv;
  if (a.direct) {
    // every request is one unit (a prefix within one split, with the draft
    // block on it, or the block alone): the unit is the request and its
    // single item writes its rows, so no work list or partial slot is used
    if (u >= a.batch) return false;
    L.b = u;
    L.r = request_info(a, u);
    L.sp = 0;
    L.item = -1;
    // (per is 1 whenever the host chose this shape; the test keeps an item
    // from ever writing a partial slot that does not exist)
    return L.r.kb > 0 && L.r.per == 1;
  }
  // Work items beyond the partials' capacity (the prefix lengths add up to
  // more than the host bound) make the whole call invalid: nothing is
  // computed and attn_combine marks every row
  if (item_off[a.batch] > a.max_items) return false;
  const int total = item_off[a.batch];
  const int* eo = unit_off;                     // block and summary units
  const int* fo = eo + (a.batch + 1);           // full-length prefix splits
  const int* po = fo + (a.batch + 1);           // shorter last splits
  const int ne = eo[a.batch], nf = fo[a.batch], np = po[a.batch];
  if (u >= ne + nf + np) return false;
  const int kind = u < ne ? 0 : (u < ne + nf ? 1 : 2);
  const int* off = kind == 0 ? eo : (kind == 1 ? fo : po);
  const int uu = u - (kind == 0 ? 0 : (kind == 1 ? ne : ne + nf));
  // request owning the unit: for block and full-length units the largest b
  // with off[b] <= uu (it has a unit of this kind, since off[b + 1] > uu);
  // the shorter last splits run in the order scan_units chose
  int lo = 0;
  if (kind == 2) {
    lo = clampi(unit_off[3 * (a.batch + 1) + uu], 0, a.batch - 1);
  } else {
    int hi = a.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= uu) lo = mid;
      else hi = mid;
    }
  }
  L.b = lo;
  L.r = request_info(a, lo);
  L.sp = kind == 0 ? L.r.ns + (uu - off[lo]) : (kind == 1 ? uu - off[lo] : L.r.ns - 1);
  L.item = item_off[lo] + L.g * L.r.per + L.sp;
  return L.item < total;
}

// Workgroups covering every item under locate_item's mapping.
inline int attn_grid(const AttnArgs& a) {
  const int units = a.max_units;
  return (units + 7) / 8 * 8 * a.hkv;
}

// Operand registers of one 32-key tile.
template <int D>
struct KvTile {
  bf16x8 k[D / 16];          // A operands of S^T = K Q^T, one per 16-dim step
  bf16x8 v[D / 32][2];       // A operands of O^T += V^T P^T, per 32-dim tile and page
};

// Key held by row rho of the S^T tile: page rho/16 ... permuted so that
// output element i of a lane in half h is key (page (i/8), slot 8h + i%8).
__device__ __forceinline__ void tile_row_key(int rho, int& page_sel, int& slot) {
  const int a = rho >> 3, hp = (rho >> 2) & 1, bq = rho & 3;
  page_sel = a >> 1;
  slot = 8 * hp + 4 * (a & 1) + bq;
}

// Draft-block keys/values [total_q][hkv][D], tile keys kappa = base..base+31.
template <int D>
__device__ __forceinline__ void load_block_tile(const AttnArgs& a, int g, int q0, int kb,
                                                int base, int lane, KvTile<D>& t) {
  const int h = lane >> 5;
  int sel, slot;
  tile_row_key(lane & 31, sel, slot);
  const int kap = base + 16 * sel + slot;
  const bool ok = kap < kb;
  const uint16_t* kr = a.k_blk + (static_cast<size_t>(q0 + (ok ? kap : 0)) * a.hkv + g) * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) t.k[s] = ok ? load_bf16x8(kr + 8 * (2 * s + h)) : zero_bf16x8();
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const int d = 32 * m + (lane & 31);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k2 = base + 16 * p + 8 * h + e;
        const uint16_t bits =
            k2 < kb ? a.v_blk[(static_cast<size_t>(q0 + k2) * a.hkv + g) * D + d] : uint16_t(0);
        v[e] = __builtin_bit_cast(__bf16, bits);
      }
      t.v[m][p] = v;
    }
  }
}

// Summary entries as keys and values ("LongSpark", sec. 2.2, eq. (6)): keys
// are the summary queries U [hkv][S][D] (bf16), values the request's summary
// values Z [batch][hkv][S][D] (fp32, rounded to bf16 like every other value
// row); tile keys kappa = base .. base+31.
template <int D>
__device__ __forceinline__ void load_summary_tile(const AttnArgs& a, int b, int g, int base,
                                                  int lane, KvTile<D>& t) {
  const int h = lane >> 5;
  int sel, slot;
  tile_row_key(lane & 31, sel, slot);
  const int kap = base + 16 * sel + slot;
  const bool ok = kap < a.n_summary;
  const uint16_t* kr = a.sum_k + (static_cast<size_t>(g) * a.n_summary + (ok ? kap : 0)) * D;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) t.k[s] = ok ? load_bf16x8(kr + 8 * (2 * s + h)) : zero_bf16x8();
  const float* vr = a.sum_v + (static_cast<size_t>(b) * a.hkv + g) * a.n_summary * D;
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
    const int d = 32 * m + (lane & 31);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int k2 = base + 16 * p + 8 * h + e;
        const uint16_t bits = k2 < a.n_summary ? f32_to_bf16_bits(vr[static_cast<size_t>(k2) * D + d])
                                               : uint16_t(0);
        v[e] = __builtin_bit_cast(__bf16, bits);
      }
      t.v[m][p] = v;
    }
  }
}

template <int D>
struct AttnState {
  bf16x8 q[D / 16];          // B operands Q^T of this wave's 32 query rows
  f32x16 o[D / 32];          // O^T accumulators, one per 32-dim tile
  float m, l;                // exponent reference (log2 units), partial sum
};

// Growth of the running maximum (log2 units) tolerated before the output is
// rescaled: probabilities are then at most 2^8 before normalisation, far
// from fp32 / bf16 overflow, and the rescale (a pass over every accumulator)
// runs only a handful of times per work item.
constexpr float kRescaleLog2 = 8.f;

// One 32-key tile: scores, online softmax, P V.  Keys lo .. hi-1 of the tile
// take part (per lane: a causal block mask gives every query its own hi);
// the rest are masked.  st.m is a running upper
// bound on nothing: it is the reference point of the exponentials, raised to
// the tile maximum only when that exceeds it by more than kRescaleLog2 (the
// softmax is invariant to the choice; "LongSpark", App. A.2, eq. (11)).
template <int D>
__device__ __forceinline__ void attend_tile(AttnState<D>& st, const KvTile<D>& t, int lo, int hi,
                                            float sl2, int lane) {
  const int h = lane >> 5;
  f32x16 s = {};
#pragma unroll
  for (int k = 0; k < D / 16; ++k) s = mfma_32x32x16(t.k[k], st.q[k], s);
  if (lo > 0 || hi < kAttnTile) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 16 * (i >> 3) + 8 * h + (i & 7);
      if (key < lo || key >= hi) s[i] = -INFINITY;
    }
  }
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = fmaxf(mx, xor_shuffle(mx, 32)) * sl2;        // log2 units
  const bool raise = mx > st.m + kRescaleLog2;       // always true on the first tile
  if (__any(raise)) {
    const float m_new = raise ? mx : st.m;
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) st.o[mt] *= alpha;
    st.m = m_new;
  }
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl2, -st.m));
  const bf16x8 p0 = pack_bf16x8(p);
  const bf16x8 p1 = pack_bf16x8(p + 8);
  // The normaliser sums the same bf16-rounded weights that multiply V, so the
  // rounding of a dominant weight cancels in O / l.
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ps += static_cast<float>(p0[i]) + static_cast<float>(p1[i]);
  st.l += ps;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
    st.o[mt] = mfma_32x32x16(t.v[mt][0], p0, st.o[mt]);
    st.o[mt] = mfma_32x32x16(t.v[mt][1], p1, st.o[mt]);
  }
}

// ------------------------------------------------------- LDS-staged stream
// Elements (uint16) of one stage: D/16 key chunks then D/16 value chunks of
// 512 elements (1 KiB) each.
template <int D>
constexpr int stage_elems() { return (D / 8) * 512; }

// Issue this wave's direct-to-LDS loads of one 32-key stage (pages pg0, pg1).
//  wave 0: key chunk c (c < D/16): lane l = (row rho = l % 32, half h = l / 32)
//          fetches dims 16 c + 8 h .. +8 of the key that S^T row rho holds.
//  wave 1: value chunk (page p, dims 32 m ..): lane l fetches 8 tokens
//          8 h .. 8 h + 7 of dim 32 m + l % 32.
//  other waves: nothing.
template <int D>
__device__ __forceinline__ void issue_stage(const AttnArgs& a, int g, int pg0, int pg1, int wave,
                                            int lane, uint16_t* stage) {
  const int h = lane >> 5;
  const uint32_t lds = lds_addr(stage);
  if (wave == 0) {
    int sel, slot;
    tile_row_key(lane & 31, sel, slot);
    const int pg = sel ? pg1 : pg0;
    const uint16_t* src =
        a.k_cache + (static_cast<size_t>(pg) * a.hkv + g) * (D * 16) + h * 128 + slot * 8;
    static_for<0, D / 16>([&](auto c) { dma16_stream(src + c * 256, lds + c * 1024); });
  } else if (wave == 1) {
    const size_t col = (lane & 31) * 16 + 8 * h;
    const uint16_t* src0 = a.v_cache + (static_cast<size_t>(pg0) * a.hkv + g) * (D * 16) + col;
    const uint16_t* src1 = a.v_cache + (static_cast<size_t>(pg1) * a.hkv + g) * (D * 16) + col;
    static_for<0, D / 32>([&](auto m) {
      dma16_stream(src0 + m * 512, lds + (D / 16 + m) * 1024);
      dma16_stream(src1 + m * 512, lds + (D / 16 + D / 32 + m) * 1024);
    });
  }
}

// MFMA operands of one staged tile, read back from LDS (lane l reads bytes
// 16 l .. 16 l + 15 of every 1 KiB chunk).
template <int D>
__device__ __forceinline__ void read_stage(const uint16_t* stage, int lane, KvTile<D>& t) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) t.k[c] = load_bf16x8(stage + c * 512 + lane * 8);
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int p = 0; p < 2; ++p)
      t.v[m][p] = load_bf16x8(stage + (D / 16 + p * (D / 32) + m) * 512 + lane * 8);
}

// Value rows of the keys outside [lo, hi) of a staged tile are set to zero.
// Their weights are already zero, but a cache slot past a request's last
// token (or outside its window) holds whatever the target left there, and a
// NaN or infinity times a zero weight would still reach the output.  Element
// e of v[m][p] is key 16 p + 8 h + e of the tile (h = lane / 32); each 32-bit
// word holds two consecutive keys, the lower one in its low half.
template <int D>
__device__ __forceinline__ void zero_values_outside(KvTile<D>& t, int lo, int hi, int lane) {
  const int h = lane >> 5;
  uint32_t keep[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int k = 16 * p + 8 * h + 2 * w;
      keep[p][w] = (k >= lo && k < hi ? 0x0000ffffu : 0u) | (k + 1 >= lo && k + 1 < hi ? 0xffff0000u : 0u);
    }
#pragma unroll
  for (int m = 0; m < D / 32; ++m)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      u32x4 v = __builtin_bit_cast(u32x4, t.v[m][p]);
#pragma unroll
      for (int w = 0; w < 4; ++w) v[w] &= keep[p][w];
      t.v[m][p] = __builtin_bit_cast(bf16x8, v);
    }
}

// The normalised output of one 32-row half written straight to `out` (bf16,
// nearest even) when the request's KV head has a single work item: the
// merge of one partial would reproduce exactly these values.
template <int D>
__device__ __forceinline__ void write_output(const AttnArgs& a, const AttnState<D>& st, const ReqInfo& r,
                                             int g, int half, int lane) {
  const int h = lane >> 5;
  const float l = st.l + xor_shuffle(st.l, 32);
  const float inv = 1.f / l;
  const int qi = 32 * half + (lane & 31);
  if (qi >= a.group * r.kb) return;
  const int j = qi / a.group, hh = qi % a.group;
  uint16_t* op = a.out + (static_cast<size_t>(r.q0 + j) * a.hq + g * a.group + hh) * D;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int ar = 0; ar < 4; ++ar) {
      const int d4 = 8 * mt + 2 * ar + h;
      const float v0 = st.o[mt][4 * ar] * inv, v1 = st.o[mt][4 * ar + 1] * inv;
      const float v2 = st.o[mt][4 * ar + 2] * inv, v3 = st.o[mt][4 * ar + 3] * inv;
      const uint32_t lo = f32_to_bf16_bits(v0) | (static_cast<uint32_t>(f32_to_bf16_bits(v1)) << 16);
      const uint32_t hi2 = f32_to_bf16_bits(v2) | (static_cast<uint32_t>(f32_to_bf16_bits(v3)) << 16);
      *reinterpret_cast<uint2*>(op + 4 * d4) = make_uint2(lo, hi2);
    }
  }
}

// Normalised partial output and log2-sum-exp2 of one 32-row half.
template <int D>
__device__ __forceinline__ void write_partial(const AttnArgs& a, const AttnState<D>& st, int item,
                                              int half, int lane) {
  const int h = lane >> 5;
  const int R = a.rows;
  float* po = a.part_o + static_cast<size_t>(item) * (D / 4) * R * 4;
  const float l = st.l + xor_shuffle(st.l, 32);
  const float inv = 1.f / l;
  const int qi = 32 * half + (lane & 31);
  if (h == 0) a.part_lse[static_cast<size_t>(item) * R + qi] = st.m + log2f(l);
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int ar = 0; ar < 4; ++ar) {
      const int d4 = 8 * mt + 2 * ar + h;
      f32x4 v = {st.o[mt][4 * ar] * inv, st.o[mt][4 * ar + 1] * inv, st.o[mt][4 * ar + 2] * inv,
                 st.o[mt][4 * ar + 3] * inv};
      *reinterpret_cast<f32x4*>(po + (static_cast<size_t>(d4) * R + qi) * 4) = v;
    }
  }
}

// The draft block's keys and values for this wave's query rows (attended by
// the last prefix split of the request, or by its own item when the prefix
// is empty); with the causal mask, block row j sees block keys 0..j.
template <int D>
__device__ __forceinline__ void attend_block(const AttnArgs& a, const ReqInfo& r, int g,
                                             AttnState<D>& st, int wave, int lane, float sl2) {
  const int qi = 32 * wave + (lane & 31);
  const int j = qi / a.group;
  for (int base = 0; base < r.kb; base += kAttnTile) {
    KvTile<D> t;
    load_block_tile<D>(a, g, r.q0, r.kb, base, lane, t);
    const int hi = min(kAttnTile, r.kb - base);
    attend_tile<D>(st, t, 0, a.block_mask ? min(hi, j - base + 1) : hi, sl2, lane);
  }
}

// One workgroup (W waves) per work item; wave w owns query rows
// 32w .. 32w+31 of the item's (up to) 32 W rows.  Waves 0 and 1 load the
// stages (keys, values); with W = 4 (more than 64 rows: large GQA groups)
// the two other waves only compute, from the same stages, so every KV byte
// is still read once per (request, KV head).
template <int D, int NS, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_splitk(AttnArgs a) {
  static_assert(NS >= 2, "at least two stages");
  static_assert(W == 2 || W == 4, "two or four waves");
  __shared__ __attribute__((aligned(1024))) uint16_t s_kv[NS * stage_elems<D>()];
  __shared__ int s_pages[kAttnMaxSplitPages];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  ItemLoc L;
  if (!a.direct && a.batch <= kAttnLocalScan) {
    // the workgroup scans the requests itself (no work-list launch);
    // workgroup 0 also stores the offsets for attn_combine
    __shared__ int s_unit_off[4 * (kAttnLocalScan + 1)];
    __shared__ int s_item_off[kAttnLocalScan + 1];
    scan_units<64 * W, kAttnLocalScan>(a, s_unit_off, s_item_off);
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < 4 * (a.batch + 1); i += 64 * W) a.unit_off[i] = s_unit_off[i];
      for (int i = threadIdx.x; i <= a.batch; i += 64 * W) a.item_off[i] = s_item_off[i];
    }
    if (!locate_item(a, blockIdx.x, s_unit_off, s_item_off, L)) return;
  } else if (!locate_item(a, blockIdx.x, a.unit_off, a.item_off, L)) {
    return;
  }
  const int b = L.b, g = L.g, sp = L.sp, item = L.item;
  const ReqInfo r = L.r;
  const int rows = a.group * r.kb;
  const bool active = 32 * wave < rows;   // this wave has query rows
  const float sl2 = a.scale_log2;

  AttnState<D> st;
  {
    const int h = lane >> 5;
    const int qi = 32 * wave + (lane & 31);
    const bool ok = qi < rows;
    const int j = ok ? qi / a.group : 0;
    const int hh = ok ? qi % a.group : 0;
    const uint16_t* qp = a.q + ((static_cast<size_t>(r.q0 + j) * a.hq) + g * a.group + hh) * D;
#pragma unroll
    for (int k = 0; k < D / 16; ++k) st.q[k] = ok ? load_bf16x8(qp + 16 * k + 8 * h) : zero_bf16x8();
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) st.o[mt] = f32x16{};
    st.m = -INFINITY;
    st.l = 0.f;
  }

  if (sp < r.ns) {
    // prefix split: tokens [t_begin, t_end), 32 per stage; tokens before n0
    // (outside the window) are masked
    const int t_begin = r.a0 + sp * a.split_tokens;
    const int t_end = min(r.n, t_begin + a.split_tokens);
    const int n_pages = (t_end - t_begin + 15) >> 4;
    const int* pt = a.page_table + static_cast<size_t>(b) * a.max_pages + (t_begin >> 4);
    for (int i = threadIdx.x; i < 2 * ((n_pages + 1) >> 1); i += 64 * W)
      s_pages[i] = clampi(pt[min(i, n_pages - 1)], 0, a.num_pages - 1);
    // Q operands loaded (a wait the compiler sees, so that it does not keep
    // a wait for them inside the stream loop) and page ids visible
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    constexpr int L = D / 16;              // direct-to-LDS loads per wave per stage
    const int n_tiles = (t_end - t_begin + kAttnTile - 1) / kAttnTile;
#pragma unroll
    for (int t = 0; t < NS - 1; ++t)
      if (t < n_tiles)
        issue_stage<D>(a, g, s_pages[2 * t], s_pages[2 * t + 1], wave, lane,
                       s_kv + t * stage_elems<D>());
    for (int t = 0; t < n_tiles; ++t) {
      wait_stage<L, NS - 2>(n_tiles - 1 - t);
      stage_barrier();
      const int tn = t + NS - 1;           // refill the stage computed last iteration
      if (tn < n_tiles)
        issue_stage<D>(a, g, s_pages[2 * tn], s_pages[2 * tn + 1], wave, lane,
                       s_kv + (tn % NS) * stage_elems<D>());
      if (active) {
        KvTile<D> kv;
        read_stage<D>(s_kv + (t % NS) * stage_elems<D>(), lane, kv);
        const int first = t_begin + t * kAttnTile;
        const int lo = max(0, r.n0 - first), hi = min(kAttnTile, t_end - first);
        if (lo > 0 || hi < kAttnTile) zero_values_outside<D>(kv, lo, hi, lane);
        attend_tile<D>(st, kv, lo, hi, sl2, lane);
      }
    }
    if (sp == r.ns - 1 && active) attend_block<D>(a, r, g, st, wave, lane, sl2);
  } else if (sp == r.ns && r.ns == 0) {
    // an empty prefix: the draft block alone
    if (!active) return;
    attend_block<D>(a, r, g, st, wave, lane, sl2);
  } else {
    // the summary entries
    if (!active) return;
    for (int base = 0; base < a.n_summary; base += kAttnTile) {
      KvTile<D> t;
      load_summary_tile<D>(a, b, g, base, lane, t);
      attend_tile<D>(st, t, 0, min(kAttnTile, a.n_summary - base), sl2, lane);
    }
  }
  if (!active) return;

  if (r.per == 1) write_output<D>(a, st, r, g, wave, lane);
  else write_partial<D>(a, st, item, wave, lane);
}

// Merge the partials of one (request, kv head) with the log-sum-exp rule and
// write bf16 outputs.  Block: 64 query rows (the z-th 64 of the item's rows)
// x 4 float4 columns.
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int pair = blockIdx.x;
  const int b = pair / a.hkv;
  const int g = pair % a.hkv;
  const int qi = 64 * blockIdx.z + (threadIdx.x & 63);
  const int d4 = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int R = a.rows;
  const ReqInfo r = request_info(a, b);
  if (r.kb <= 0 || qi >= a.group * r.kb) return;
  const int first = a.item_off[b] + g * r.per;
  const int j = qi / a.group, hh = qi % a.group;
  uint16_t* op = a.out + (static_cast<size_t>(r.q0 + j) * a.hq + g * a.group + hh) * D + 4 * d4;
  if (a.item_off[a.batch] > a.max_items) {
    // The work items did not fit the partials (the prefix lengths add up to
    // more than the host bound they were sized for) and nothing was
    // computed: every row is marked NaN rather than left stale.
    *reinterpret_cast<uint2*>(op) = make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
    return;
  }
  if (r.per == 1) return;   // a single item wrote its rows
  const int n = r.per;
  // Loads are issued eight partials at a time so their latencies overlap;
  // past the last partial (a uniform condition) nothing is loaded.
  constexpr int U = 8;
  const float* lse = a.part_lse + static_cast<size_t>(first) * R + qi;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < n; s0 += U) {
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) l[u] = s0 + u < n ? lse[static_cast<size_t>(s0 + u) * R] : -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) mx = fmaxf(mx, l[u]);
  }
  const float* po = a.part_o + ((static_cast<size_t>(first) * (D / 4) + d4) * R + qi) * 4;
  const size_t item_stride = static_cast<size_t>(D / 4) * R * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s0 = 0; s0 < n; s0 += U) {
    float l[U];
    f32x4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t it = static_cast<size_t>(s0 + u);
      l[u] = s0 + u < n ? lse[it * R] : -INFINITY;
      o[u] = s0 + u < n ? *reinterpret_cast<const f32x4*>(po + it * item_stride) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float w = s0 + u < n ? __builtin_amdgcn_exp2f(l[u] - mx) : 0.f;
      acc += w * o[u];
      wsum += w;
    }
  }
  acc *= 1.f / wsum;
  const uint32_t lo = f32_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
  const uint32_t hi2 = f32_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
  *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi2);
}

template <int D>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  if (a.direct) {
    // one item per (request, kv head), each writing its own rows
    const dim3 grid((a.batch + 7) / 8 * 8 * a.hkv);
    return a.rows > 64 ? launch_kernel(attn_splitk<D, kAttnStages, 4>, grid, dim3(256), s, a)
                       : launch_kernel(attn_splitk<D, kAttnStages, 2>, grid, dim3(128), s, a);
  }
  hipError_t e = a.batch > kAttnLocalScan ? launch_kernel(attn_worklist, dim3(1), dim3(1024), s, a)
                                           : hipSuccess;
  if (e == hipSuccess && a.max_items > 0)
    e = a.rows > 64 ? launch_kernel(attn_splitk<D, kAttnStages, 4>, dim3(attn_grid(a)), dim3(256), s, a)
                    : launch_kernel(attn_splitk<D, kAttnStages, 2>, dim3(attn_grid(a)), dim3(128), s, a);
  if (e == hipSuccess)
    e = launch_kernel(attn_combine<D>, dim3(a.batch * a.hkv, D / 16, a.rows / 64), dim3(256), s, a);
  return e;
}

}  // namespace

hipError_t launch_draft_attn(const AttnArgs& a, int head_dim, hipStream_t s) {
  return head_dim == 64 ? launch<64>(a, s) : launch<128>(a, s);
}

}  // namespace sd
