// Global context summary of the fixed-cost drafter ("LongSpark", sec. 2.2,
// eq. (5), and App. A.2, eqs. (10)-(11)).
//
// Each KV head g of a request keeps, for S fixed summary queries u_i, the
// attention of u_i over every target KV row retained so far:
//     c_i = log sum_t exp(s_it),  Z_i = sum_t exp(s_it - c_i) v_t,
//     s_it = scale * u_i . k_t.
// After verification the a_b + 1 newly retained rows (the committed token
// and the accepted drafts, already written to the target's cache) are folded
// in: their own statistics (c', Z') over the new rows, then the merge of
// eq. (11), c'' = log(e^c + e^c'), Z'' = e^(c - c'') Z + e^(c' - c'') Z'.
// An empty set of new rows leaves the state as it is.
//
// summary_fold: one workgroup per (request, KV head).  The new rows are read
// in place through the page table in tiles of 64; scores, the running max
// and sum and the weighted values are fp32.  A step folds at most K + 1 rows
// (one tile); initialising from a whole prefix is the same loop over all of
// its tiles.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;   // rows per tile

template <int D>
__global__ __launch_bounds__(kThreads) void summary_fold(SummaryArgs a) {
  __shared__ float s_u[D * kSummaryMax];          // summary queries, [d][i] (fp32)
  __shared__ uint16_t s_k[D * kRows];             // key tile, [d][row] (bf16 bits)
  __shared__ uint16_t s_v[kRows * D];             // value tile
  __shared__ float s_p[kSummaryMax * kRows];      // scores, then weights
  __shared__ float s_m[kSummaryMax], s_l[kSummaryMax], s_alpha[kSummaryMax];

  const int b = blockIdx.x / a.hkv;
  const int g = blockIdx.x % a.hkv;
  const int tid = threadIdx.x;
  const int S = a.n_summary;
  const int n_max = a.max_pages * 16;
  const int n = clampi(a.ctx_len[b], 0, n_max);
  int r0, r1;   // rows [r0, r1) to fold
  if (a.accepted) {
    r0 = n;
    r1 = min(n_max, n + clampi(a.accepted[b], 0, n_max) + 1);
  } else {
    r0 = 0;
    r1 = n;
  }
  float* zs = a.z + (static_cast<size_t>(b) * a.hkv + g) * S * D;
  float* cs = a.c + (static_cast<size_t>(b) * a.hkv + g) * S;
  if (r1 <= r0) {
    if (!a.accepted) {   // initialising from an empty prefix: the empty state
      for (int i = tid; i < S; i += kThreads) cs[i] = -INFINITY;
      for (int i = tid; i < S * D; i += kThreads) zs[i] = 0.f;
    }
    return;
  }

  const uint16_t* uq = a.u + static_cast<size_t>(g) * S * D;
  for (int i = tid; i < S * D; i += kThreads)
    s_u[(i % D) * S + i / D] = __uint_as_float(static_cast<uint32_t>(uq[i]) << 16);
  for (int i = tid; i < S; i += kThreads) {
    s_m[i] = -INFINITY;
    s_l[i] = 0.f;
  }
  // weighted values of the new rows: thread t owns entries t, t + 256, ...
  constexpr int kOwn = kSummaryMax * D / kThreads;
  float acc[kOwn];
#pragma unroll
  for (int e = 0; e < kOwn; ++e) acc[e] = 0.f;
  const int* pt = a.page_table + static_cast<size_t>(b) * a.max_pages;

  for (int t0 = r0; t0 < r1; t0 += kRows) {
    const int rows = min(kRows, r1 - t0);
    __syncthreads();   // the previous tile's readers are done
    // keys: one 16-byte chunk (8 dims) per (row, chunk), stored transposed;
    // values: per (row, dim)
    for (int i = tid; i < kRows * (D / 8); i += kThreads) {
      const int rr = i % kRows, c = i / kRows;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (rr < rows) {
        const int tok = t0 + rr;
        const int pg = clampi(pt[tok >> 4], 0, a.num_pages - 1);
        const uint16_t* src =
            a.k_cache + ((static_cast<size_t>(pg) * a.hkv + g) * (D / 8) + c) * 128 + (tok & 15) * 8;
        v = *reinterpret_cast<const u32x4*>(src);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        s_k[(8 * c + e) * kRows + rr] = static_cast<uint16_t>(v[e / 2] >> (16 * (e & 1)));
    }
    for (int i = tid; i < kRows * D; i += kThreads) {
      const int rr = i / D, d = i % D;
      uint16_t v = 0;
      if (rr < rows) {
        const int tok = t0 + rr;
        const int pg = clampi(pt[tok >> 4], 0, a.num_pages - 1);
        v = a.v_cache[((static_cast<size_t>(pg) * a.hkv + g) * D + d) * 16 + (tok & 15)];
      }
      s_v[rr * D + d] = v;
    }
    __syncthreads();
    // scores s_ik = scale * u_i . k_k
    for (int i = tid; i < S * kRows; i += kThreads) {
      const int q = i / kRows, k = i % kRows;
      float s = -INFINITY;
      if (k < rows) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d)
          dot += s_u[d * S + q] * __uint_as_float(static_cast<uint32_t>(s_k[d * kRows + k]) << 16);
        s = dot * a.scale;
      }
      s_p[i] = s;
    }
    __syncthreads();
    // online softmax per query: new max, rescale factor, weights, sum
    for (int q = tid; q < S; q += kThreads) {
      float mx = s_m[q];
      for (int k = 0; k < rows; ++k) mx = fmaxf(mx, s_p[q * kRows + k]);
      const float alpha = expf(s_m[q] - mx);   // 0 on the first tile (s_m = -inf)
      float l = s_l[q] * alpha;
      for (int k = 0; k < kRows; ++k) {
        const float w = k < rows ? expf(s_p[q * kRows + k] - mx) : 0.f;
        s_p[q * kRows + k] = w;
        l += w;
      }
      s_m[q] = mx;
      s_l[q] = l;
      s_alpha[q] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kOwn; ++e) {
      const int idx = tid + kThreads * e;
      if (idx < S * D) {
        const int q = idx / D, d = idx % D;
        float v = acc[e] * s_alpha[q];
        for (int k = 0; k < rows; ++k)
          v += s_p[q * kRows + k] * __uint_as_float(static_cast<uint32_t>(s_v[k * D + d]) << 16);
        acc[e] = v;
      }
    }
  }
  __syncthreads();

  // merge with the stored state (eq. (11)); initialisation replaces it
#pragma unroll
  for (int e = 0; e < kOwn; ++e) {
    const int idx = tid + kThreads * e;
    if (idx < S * D) {
      const int q = idx / D;
      const float c_new = s_m[q] + logf(s_l[q]);
      const float z_new = acc[e] / s_l[q];
      const float c_old = a.accepted ? cs[q] : -INFINITY;
      if (c_old == -INFINITY) {
        zs[idx] = z_new;
      } else {
        const float mx = fmaxf(c_old, c_new);
        const float c = mx + logf(expf(c_old - mx) + expf(c_new - mx));
        zs[idx] = expf(c_old - c) * zs[idx] + expf(c_new - c) * z_new;
      }
    }
  }
  __syncthreads();   // every thread has read cs[] before it is overwritten
  for (int q = tid; q < S; q += kThreads) {
    const float c_new = s_m[q] + logf(s_l[q]);
    const float c_old = a.accepted ? cs[q] : -INFINITY;
    if (c_old == -INFINITY) {
      cs[q] = c_new;
    } else {
      const float mx = fmaxf(c_old, c_new);
      cs[q] = mx + logf(expf(c_old - mx) + expf(c_new - mx));
    }
  }
}

}  // namespace

hipError_t launch_summary(const SummaryArgs& a, int head_dim, hipStream_t s) {
  const dim3 grid(a.batch * a.hkv), block(kThreads);
  return head_dim == 64 ? launch_kernel(summary_fold<64>, grid, block, s, a)
                        : launch_kernel(summary_fold<128>, grid, block, s, a);
}

}  // namespace sd
