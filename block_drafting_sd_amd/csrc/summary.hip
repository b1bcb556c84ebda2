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
// summary_fold: one workgroup (4 waves) per (request, KV head).  The new rows
// are read in place through the page table in tiles of 64: the tile's page
// ids first, then every key chunk and every 8-token value chunk as
// independent 16-byte loads.  Lane l of every wave owns row l of the tile;
// wave w owns the summary queries w, w + 4, ...: its scores are dot products
// of the lane's key row (read once per 8 dims) with each query (a broadcast
// read), the online softmax of a query is a wave reduction, and the weighted
// values are summed per (query, dim) entry with independent accumulators.
// Everything is fp32.  A step folds at most K + 1 rows (one tile);
// initialising from a whole prefix is the same loop over all of its tiles.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 64;                         // rows per tile = lanes

// D: head dim; SMAX: the most summary entries this instance handles (16, or
// kSummaryMax), which sizes the per-wave query registers and accumulators.
template <int D, int SMAX>
__global__ __launch_bounds__(kThreads) void summary_fold(SummaryArgs a) {
  constexpr int kQPerWave = SMAX / kWaves;        // summary queries per wave (max)
  constexpr int KP = D + 8;                       // key row pitch (bf16): spreads banks
  __shared__ __attribute__((aligned(16))) float s_u[SMAX * D];          // queries [q][d]
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kRows * KP];     // keys [row][d]
  __shared__ uint16_t s_v[kRows * D];                                   // values [row][d]
  __shared__ float s_p[SMAX * kRows];                                   // weights [q][row]
  __shared__ float s_alpha[SMAX];
  __shared__ int s_pg[kRows];

  const int b = blockIdx.x / a.hkv;
  const int g = blockIdx.x % a.hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  for (int i = tid; i < S * D; i += kThreads) s_u[i] = __uint_as_float(static_cast<uint32_t>(uq[i]) << 16);
  // running max and sum of the wave's queries (wave-uniform)
  float m_run[kQPerWave], l_run[kQPerWave];
#pragma unroll
  for (int j = 0; j < kQPerWave; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
  }
  // weighted values: thread t owns entries t, t + 256, ... of [q][d]
  static_assert(kThreads % D == 0, "a thread's entries share one dim");
  constexpr int kOwn = SMAX * D / kThreads;
  float acc[kOwn];
#pragma unroll
  for (int e = 0; e < kOwn; ++e) acc[e] = 0.f;
  const int* pt = a.page_table + static_cast<size_t>(b) * a.max_pages;

  for (int t0 = r0; t0 < r1; t0 += kRows) {
    const int rows = min(kRows, r1 - t0);
    __syncthreads();   // the previous tile's readers are done
    if (tid < kRows) s_pg[tid] = tid < rows ? clampi(pt[(t0 + tid) >> 4], 0, a.num_pages - 1) : 0;
    __syncthreads();
    // keys: one 16-byte chunk (8 dims) per (row, chunk)
    constexpr int kKeyLoads = kRows * (D / 8) / kThreads;
    u32x4 kv[kKeyLoads];
#pragma unroll
    for (int j = 0; j < kKeyLoads; ++j) {
      const int i = tid + kThreads * j;
      const int rr = i % kRows, c = i / kRows;
      kv[j] = u32x4{0u, 0u, 0u, 0u};
      if (rr < rows)
        kv[j] = *reinterpret_cast<const u32x4*>(
            a.k_cache + ((static_cast<size_t>(s_pg[rr]) * a.hkv + g) * (D / 8) + c) * 128 + ((t0 + rr) & 15) * 8);
    }
    // values: one 16-byte chunk = 8 consecutive tokens (8-aligned, so inside
    // one page) of one dim; chunk ch covers tokens 8 ch .. 8 ch + 7
    const int ch0 = t0 >> 3;
    const int nch = ((t0 + rows - 1) >> 3) - ch0 + 1;           // <= kRows / 8 + 1
    constexpr int kValLoads = (kRows / 8 + 1) * D / kThreads + 1;
    u32x4 vv[kValLoads];
#pragma unroll
    for (int j = 0; j < kValLoads; ++j) {
      const int i = tid + kThreads * j;
      const int cj = i / D, d = i % D;
      vv[j] = u32x4{0u, 0u, 0u, 0u};
      if (cj < nch) {
        const int first = max((ch0 + cj) * 8, t0);                // a row of this tile in the chunk's page
        vv[j] = *reinterpret_cast<const u32x4*>(
            a.v_cache + ((static_cast<size_t>(s_pg[first - t0]) * a.hkv + g) * D + d) * 16 + ((ch0 + cj) * 8 & 15));
      }
    }
#pragma unroll
    for (int j = 0; j < kKeyLoads; ++j) {
      const int i = tid + kThreads * j;
      const int rr = i % kRows, c = i / kRows;
      *reinterpret_cast<u32x4*>(s_k + rr * KP + 8 * c) = kv[j];
    }
#pragma unroll
    for (int j = 0; j < kValLoads; ++j) {
      const int i = tid + kThreads * j;
      const int cj = i / D, d = i % D;
      if (cj < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int rr = (ch0 + cj) * 8 + e - t0;
          if (rr >= 0 && rr < rows) s_v[rr * D + d] = static_cast<uint16_t>(vv[j][e / 2] >> (16 * (e & 1)));
        }
      }
    }
    for (int i = tid; i < (kRows - rows) * D; i += kThreads) s_v[rows * D + i] = 0;
    __syncthreads();

    // scores of the wave's queries against row `lane`
    float sc[kQPerWave];
#pragma unroll
    for (int j = 0; j < kQPerWave; ++j) sc[j] = 0.f;
#pragma unroll 2
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 kc = *reinterpret_cast<const u32x4*>(s_k + lane * KP + 8 * c);
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = __uint_as_float((e & 1) ? (kc[e / 2] & 0xffff0000u) : (kc[e / 2] << 16));
#pragma unroll
      for (int j = 0; j < kQPerWave; ++j) {
        const int q = wave + kWaves * j;
        if (q < S) {                                     // wave-uniform
          const float4 u0 = *reinterpret_cast<const float4*>(s_u + q * D + 8 * c);
          const float4 u1 = *reinterpret_cast<const float4*>(s_u + q * D + 8 * c + 4);
          sc[j] += u0.x * kf[0] + u0.y * kf[1] + u0.z * kf[2] + u0.w * kf[3] + u1.x * kf[4] + u1.y * kf[5] +
                   u1.z * kf[6] + u1.w * kf[7];
        }
      }
    }
    // online softmax of each query over the tile (a wave reduction)
#pragma unroll
    for (int j = 0; j < kQPerWave; ++j) {
      const int q = wave + kWaves * j;
      if (q < S) {                                       // wave-uniform
        const float s = lane < rows ? sc[j] * a.scale : -INFINITY;
        float mx = s;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float mnew = fmaxf(m_run[j], mx);
        const float w = lane < rows ? expf(s - mnew) : 0.f;
        float sum = w;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o, 64);
        const float alpha = expf(m_run[j] - mnew);       // 0 on the first tile (m_run = -inf)
        l_run[j] = l_run[j] * alpha + sum;
        m_run[j] = mnew;
        s_p[q * kRows + lane] = w;
        if (lane == 0) s_alpha[q] = alpha;
      }
    }
    __syncthreads();
    // entry e of this thread is (query (tid + 256 e) / D, dim tid % D): one
    // value read per row serves all of them
#pragma unroll
    for (int e = 0; e < kOwn; ++e) {
      const int idx = tid + kThreads * e;
      if (idx < S * D) acc[e] *= s_alpha[idx / D];
    }
    for (int k = 0; k < rows; ++k) {
      const float vk = __uint_as_float(static_cast<uint32_t>(s_v[k * D + tid % D]) << 16);
#pragma unroll
      for (int e = 0; e < kOwn; ++e) {
        const int idx = tid + kThreads * e;
        if (idx < S * D) acc[e] += s_p[(idx / D) * kRows + k] * vk;
      }
    }
  }
  // publish each query's running max and sum (s_alpha and s_p are free)
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kQPerWave; ++j) {
    const int q = wave + kWaves * j;
    if (q < S && lane == 0) {
      s_alpha[q] = m_run[j];
      s_p[q] = l_run[j];
    }
  }
  __syncthreads();

  // merge with the stored state (eq. (11)); initialisation replaces it
#pragma unroll
  for (int e = 0; e < kOwn; ++e) {
    const int idx = tid + kThreads * e;
    if (idx < S * D) {
      const int q = idx / D;
      const float c_new = s_alpha[q] + logf(s_p[q]);
      const float z_new = acc[e] / s_p[q];
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
    const float c_new = s_alpha[q] + logf(s_p[q]);
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
  if (a.n_summary <= 16)
    return head_dim == 64 ? launch_kernel(summary_fold<64, 16>, grid, block, s, a)
                          : launch_kernel(summary_fold<128, 16>, grid, block, s, a);
  return head_dim == 64 ? launch_kernel(summary_fold<64, kSummaryMax>, grid, block, s, a)
                        : launch_kernel(summary_fold<128, kSummaryMax>, grid, block, s, a);
}

}  // namespace sd
