// Draft-block attention over the target's paged KV cache.
//
// The K_b draft queries of request b attend, with one softmax and no mask, to
// the N_b prefix keys of the target's cache (read in place through the page
// table) and to the K_b keys of the draft block ("ForeSpark", sec. 4.1;
// "LongSpark", App. A.1, Fig. 6; "H-Spec", sec. 3.3.2).
//
// Work decomposition (split-K, flash-decoding style):
//   item = (request b, kv head g, split s); splits 0..ns_b-1 cover the prefix
//   in chunks of `split_tokens`, split ns_b covers the draft block.  All G*K_b
//   query rows of (b, g) share one item, so every prefix KV byte is read from
//   HBM exactly once.  Each item writes fp32 partial results (normalised
//   output and log-sum-exp), which `attn_combine` merges with the log-sum-exp
//   rule of "LongSpark", App. A.2, eq. (11).
//
// Inner tile (one wave): 32 keys = two 16-token pages.
//   S^T[32 keys x 32 queries] = K * Q^T      (MFMA 32x32x16 bf16, D/16 steps)
//   O^T[D x 32 queries]     += V^T * P^T     (MFMA 32x32x16 bf16, 2 steps)
// The key order inside a tile is permuted so that the softmax values a lane
// holds after the first product are exactly the B operand of the second one
// (no LDS round trip), and so that every K and V operand is one coalesced
// 16-byte load from the cache layouts [page][g][D/8][16][8] and [page][g][D][16].
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {

int32_t attn_split_tokens(int32_t hkv, int64_t max_total_ctx, int32_t requested) {
  if (requested > 0) return requested;
  // aim for ~2048 prefix work items (8 per CU), at least 256 tokens each
  const int64_t target_items = 2048;
  int64_t s = (static_cast<int64_t>(hkv) * max_total_ctx + target_items - 1) / target_items;
  s = (s + 255) / 256 * 256;
  if (s < 256) s = 256;
  if (s > 65536) s = 65536;
  return static_cast<int32_t>(s);
}

int64_t attn_max_items(int32_t batch, int32_t hkv, int64_t max_total_ctx,
                       int32_t split_tokens) {
  // sum_b (ceil(N_b / S) + 1) <= sum_b N_b / S + 2 * batch
  return static_cast<int64_t>(hkv) * (max_total_ctx / split_tokens + 2 * static_cast<int64_t>(batch));
}

namespace {

struct ReqInfo {
  int n;        // prefix length N_b (clamped)
  int q0;       // first query row
  int kb;       // draft rows K_b (clamped)
  int ns;       // prefix splits
};

__device__ __forceinline__ ReqInfo request_info(const AttnArgs& a, int b) {
  ReqInfo r;
  r.n = clampi(a.ctx_len[b], 0, a.max_pages * 16);
  r.q0 = clampi(a.q_off[b], 0, a.total_q);
  r.kb = min(clampi(a.q_off[b + 1], r.q0, a.total_q) - r.q0, a.max_draft_k);
  r.ns = (r.n + a.split_tokens - 1) / a.split_tokens;
  return r;
}

// Exclusive prefix sum of the work items of every request (one workgroup).
__global__ __launch_bounds__(1024) void attn_worklist(AttnArgs a) {
  __shared__ int sh[1024];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < a.batch; base += 1024) {
    const int b = base + threadIdx.x;
    int v = 0;
    if (b < a.batch) {
      const ReqInfo r = request_info(a, b);
      v = r.kb > 0 ? a.hkv * (r.ns + 1) : 0;
    }
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int t = threadIdx.x >= off ? sh[threadIdx.x - off] : 0;
      __syncthreads();
      sh[threadIdx.x] += t;
      __syncthreads();
    }
    if (b < a.batch) a.item_off[b] = carry + sh[threadIdx.x] - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry += sh[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.item_off[a.batch] = carry;
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

template <int D>
__device__ __forceinline__ void load_cache_tile(const AttnArgs& a, int g, int pg0, int pg1,
                                                int lane, KvTile<D>& t) {
  const int h = lane >> 5;
  int sel, slot;
  tile_row_key(lane & 31, sel, slot);
  const int pk = sel ? pg1 : pg0;
  const uint16_t* kb = a.k_cache + (static_cast<size_t>(pk) * a.hkv + g) * (D / 8) * 128 + slot * 8;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) t.k[s] = load_bf16x8(kb + (2 * s + h) * 128);
#pragma unroll
  for (int m = 0; m < D / 32; ++m) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int pg = p ? pg1 : pg0;
      const uint16_t* vb = a.v_cache +
                           ((static_cast<size_t>(pg) * a.hkv + g) * D + 32 * m + (lane & 31)) * 16 + 8 * h;
      t.v[m][p] = load_bf16x8(vb);
    }
  }
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

template <int D>
struct AttnState {
  bf16x8 q[D / 16];          // B operands Q^T of this wave's 32 query rows
  f32x16 o[D / 32];          // O^T accumulators, one per 32-dim tile
  float m, l;                // running max (raw score units), partial sum
};

// One 32-key tile: scores, online softmax, P V.  `valid` = number of keys of
// the tile that exist (keys past it are masked).
template <int D>
__device__ __forceinline__ void attend_tile(AttnState<D>& st, const KvTile<D>& t, int valid,
                                            float sl2, int lane) {
  const int h = lane >> 5;
  f32x16 s = {};
#pragma unroll
  for (int k = 0; k < D / 16; ++k) s = mfma_32x32x16(t.k[k], st.q[k], s);
  if (valid < kAttnTile) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 16 * (i >> 3) + 8 * h + (i & 7);
      if (key >= valid) s[i] = -INFINITY;
    }
  }
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = fmaxf(mx, xor_shuffle(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float alpha = __builtin_amdgcn_exp2f((st.m - m_new) * sl2);
  float p[16];
  float ps = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = __builtin_amdgcn_exp2f((s[i] - m_new) * sl2);
    ps += p[i];
  }
  st.l = st.l * alpha + ps;
  st.m = m_new;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt) st.o[mt] *= alpha;
  }
  const bf16x8 p0 = pack_bf16x8(p);
  const bf16x8 p1 = pack_bf16x8(p + 8);
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
    st.o[mt] = mfma_32x32x16(t.v[mt][0], p0, st.o[mt]);
    st.o[mt] = mfma_32x32x16(t.v[mt][1], p1, st.o[mt]);
  }
}

// One workgroup per work item; wave w owns query rows 32w .. 32w+31 of the
// item's (up to) 64 rows.  Both waves stream the same keys, so the second
// wave's requests are served by the CU's L1 / the XCD's L2, not HBM.
template <int D>
__global__ __launch_bounds__(128) void attn_splitk(AttnArgs a) {
  const int item = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int total = min(a.item_off[a.batch], a.max_items);
  if (item >= total) return;
  // request owning this item: largest b with item_off[b] <= item
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.item_off[mid] <= item) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const ReqInfo r = request_info(a, b);
  const int rel = item - a.item_off[b];
  const int g = rel / (r.ns + 1);
  const int sp = rel % (r.ns + 1);
  const int rows = a.group * r.kb;
  if (32 * wave >= rows) return;          // no query rows for this wave
  const int h = lane >> 5;
  const float sl2 = a.scale_log2;

  AttnState<D> st;
  {
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
    // prefix split: tokens [t_begin, t_end), 32 per tile
    const int t_begin = sp * a.split_tokens;
    const int t_end = min(r.n, t_begin + a.split_tokens);
    const int* pt = a.page_table + static_cast<size_t>(b) * a.max_pages;
    auto pages = [&](int tt, int& p0, int& p1) {
      const int lp = tt >> 4;
      p0 = clampi(pt[lp], 0, a.num_pages - 1);
      p1 = tt + 16 < t_end ? clampi(pt[lp + 1], 0, a.num_pages - 1) : p0;
    };
    // ping-pong between two register tiles: the next tile's loads are in
    // flight while the current one is computed
    KvTile<D> ta, tb;
    int p0, p1;
    pages(t_begin, p0, p1);
    load_cache_tile<D>(a, g, p0, p1, lane, ta);
    for (int tt = t_begin;;) {
      if (tt + kAttnTile < t_end) {
        pages(tt + kAttnTile, p0, p1);
        load_cache_tile<D>(a, g, p0, p1, lane, tb);
      }
      attend_tile<D>(st, ta, min(kAttnTile, t_end - tt), sl2, lane);
      tt += kAttnTile;
      if (tt >= t_end) break;
      if (tt + kAttnTile < t_end) {
        pages(tt + kAttnTile, p0, p1);
        load_cache_tile<D>(a, g, p0, p1, lane, ta);
      }
      attend_tile<D>(st, tb, min(kAttnTile, t_end - tt), sl2, lane);
      tt += kAttnTile;
      if (tt >= t_end) break;
    }
  } else {
    for (int base = 0; base < r.kb; base += kAttnTile) {
      KvTile<D> t;
      load_block_tile<D>(a, g, r.q0, r.kb, base, lane, t);
      attend_tile<D>(st, t, min(kAttnTile, r.kb - base), sl2, lane);
    }
  }

  // normalised partial output and log2-sum-exp2 of the scaled scores
  float* po = a.part_o + static_cast<size_t>(item) * (D / 4) * kAttnRows * 4;
  const float l = st.l + xor_shuffle(st.l, 32);
  const float inv = 1.f / l;
  const int qi = 32 * wave + (lane & 31);
  if (h == 0) a.part_lse[static_cast<size_t>(item) * kAttnRows + qi] = st.m * sl2 + log2f(l);
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt) {
#pragma unroll
    for (int ar = 0; ar < 4; ++ar) {
      const int d4 = 8 * mt + 2 * ar + h;
      f32x4 v = {st.o[mt][4 * ar] * inv, st.o[mt][4 * ar + 1] * inv, st.o[mt][4 * ar + 2] * inv,
                 st.o[mt][4 * ar + 3] * inv};
      *reinterpret_cast<f32x4*>(po + (static_cast<size_t>(d4) * kAttnRows + qi) * 4) = v;
    }
  }
}

// Merge the partials of one (request, kv head) with the log-sum-exp rule and
// write bf16 outputs.  Block: 64 query rows x 4 float4 columns.
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int pair = blockIdx.x;
  const int b = pair / a.hkv;
  const int g = pair % a.hkv;
  const int qi = threadIdx.x & 63;
  const int d4 = blockIdx.y * 4 + (threadIdx.x >> 6);
  const ReqInfo r = request_info(a, b);
  if (r.kb <= 0 || qi >= a.group * r.kb) return;
  const int first = a.item_off[b] + g * (r.ns + 1);
  const int n = min(r.ns + 1, a.max_items - first);
  if (n <= 0) return;
  float mx = -INFINITY;
  for (int s = 0; s < n; ++s) mx = fmaxf(mx, a.part_lse[static_cast<size_t>(first + s) * kAttnRows + qi]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s = 0; s < n; ++s) {
    const size_t it = static_cast<size_t>(first + s);
    const float w = __builtin_amdgcn_exp2f(a.part_lse[it * kAttnRows + qi] - mx);
    const f32x4 o = *reinterpret_cast<const f32x4*>(
        a.part_o + ((it * (D / 4) + d4) * kAttnRows + qi) * 4);
    acc += w * o;
    wsum += w;
  }
  acc *= 1.f / wsum;
  const int j = qi / a.group, hh = qi % a.group;
  uint16_t* op = a.out + (static_cast<size_t>(r.q0 + j) * a.hq + g * a.group + hh) * D + 4 * d4;
  const uint32_t lo = f32_to_bf16_bits(acc[0]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[1])) << 16);
  const uint32_t hi2 = f32_to_bf16_bits(acc[2]) | (static_cast<uint32_t>(f32_to_bf16_bits(acc[3])) << 16);
  *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi2);
}

template <int D>
hipError_t launch(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_worklist, dim3(1), dim3(1024), 0, s, a);
  if (a.max_items > 0)
    hipLaunchKernelGGL((attn_splitk<D>), dim3(a.max_items), dim3(128), 0, s, a);
  hipLaunchKernelGGL((attn_combine<D>), dim3(a.batch * a.hkv, D / 16), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_draft_attn(const AttnArgs& a, int head_dim, hipStream_t s) {
  return head_dim == 64 ? launch<64>(a, s) : launch<128>(a, s);
}

}  // namespace sd
