// Drafter LM head: logits = hidden W^T on MFMA, fused with the draft
// softmax statistics and Gumbel-max draft sampling ("LongSpark", sec. 2.1,
// eq. (4) and App. A.1, Fig. 6: the frozen target vocabulary head produces
// every slot's base logits in parallel and each slot is sampled
// independently).
//
// lm_gemm: one workgroup (4 waves) computes a 128-vocab x 128-row tile of
// logits^T = W * hidden^T with MFMA 32x32x16 bf16 (fp32 accumulation); both
// operands are H-contiguous and are staged through double-buffered LDS in
// 64-wide K slices.  Each lane ends up owning one draft row and 32 vocab
// entries, so the epilogue's row statistics are mostly in-lane: it stores the
// fp32 logits, and writes per (row, vocab tile) the max, the sum of exp
// relative to it and the best Gumbel-max candidate (Philox stream 0).
// Tiles are ordered so that all row tiles of one vocab tile, and a compact
// block of vocab tiles, run together on one XCD (blockIdx % 8 picks the XCD),
// which keeps every W and hidden slice in that XCD's L2 across row tiles.
//
// lm_row_reduce: merges the per-tile statistics of a row into lse and the
// draft token.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kThreads = 256;
constexpr int kLdk = kLmBK + 8;   // LDS row stride (elements); 144 B avoids bank conflicts

__device__ __forceinline__ void row_owner(const LmArgs& a, int m, uint32_t& rid, uint32_t& pos) {
  // request b with q_off[b] <= m < q_off[b+1]
  const int total = a.q_off[a.batch];
  if (m >= total || m < 0) {
    rid = a.req_id[0];
    pos = static_cast<uint32_t>(m + 1);
    return;
  }
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.q_off[mid] <= m) lo = mid;
    else hi = mid;
  }
  rid = a.req_id[lo];
  pos = static_cast<uint32_t>(m - a.q_off[lo] + 1);
}

__global__ __launch_bounds__(kThreads, 2) void lm_gemm(LmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (kLmBV + kLmBM) * kLdk];
  const int P = blockIdx.x;
  const int xcd = P & 7, slot = P >> 3;
  const int vt = (slot / a.n_mt) * 8 + xcd;
  const int mt = slot % a.n_mt;
  if (vt >= a.n_vt) return;
  const int v0 = vt * kLmBV, m0 = mt * kLmBM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave & 1, wm = wave >> 1, h = lane >> 5;

  // stage `buf`: W tile at smem + buf * stage, hidden tile right after it
  constexpr int kStage = (kLmBV + kLmBM) * kLdk;
  auto sA = [&](int buf) { return smem + buf * kStage; };
  auto sB = [&](int buf) { return smem + buf * kStage + kLmBV * kLdk; };

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, kc = c & 7;
      const int v = v0 + row, m = m0 + row;
      ra[i] = v < a.V ? *reinterpret_cast<const u32x4*>(a.w + static_cast<size_t>(v) * a.H + k0 + kc * 8)
                      : u32x4{0u, 0u, 0u, 0u};
      rb[i] = m < a.M ? *reinterpret_cast<const u32x4*>(a.hidden + static_cast<size_t>(m) * a.H + k0 + kc * 8)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, kc = c & 7;
      store_u32x4(sA(buf) + row * kLdk + kc * 8, ra[i]);
      store_u32x4(sB(buf) + row * kLdk + kc * 8, rb[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = a.H / kLmBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * kLmBK);
#pragma unroll
    for (int s = 0; s < kLmBK / 16; ++s) {
      bf16x8 af[2], bf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = 64 * wv + 32 * t + (lane & 31);
        af[t] = load_bf16x8(sA(buf) + r * kLdk + (2 * s + h) * 8);
        const int cidx = 64 * wm + 32 * t + (lane & 31);
        bf[t] = load_bf16x8(sB(buf) + cidx * kLdk + (2 * s + h) * 8);
      }
#pragma unroll
      for (int tv = 0; tv < 2; ++tv)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) acc[tv][tm] = mfma_32x32x16(af[tv], bf[tm], acc[tv][tm]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // acc[tv][tm][i]: vocab v0 + 64 wv + 32 tv + 8 (i/4) + 4 h + i%4,
  //                 row    m0 + 64 wm + 32 tm + lane%32
  float* red = reinterpret_cast<float*>(smem);   // [2 (tm)][32][4] per wm, reused LDS
  const bool vec_ok = (a.V & 3) == 0;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int m = m0 + 64 * wm + 32 * tm + (lane & 31);
    const bool mok = m < a.M;
    uint32_t rid = 0, pos = 0;
    if (mok) row_owner(a, m, rid, pos);
    float mx = -FLT_MAX;
#pragma unroll
    for (int tv = 0; tv < 2; ++tv)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 64 * wv + 32 * tv + 8 * (i >> 2) + 4 * h + (i & 3);
        if (v < a.V) mx = fmaxf(mx, acc[tv][tm][i]);
      }
    float se = 0.f;
    Cand best{-FLT_MAX, 0x7fffffff};
#pragma unroll
    for (int tv = 0; tv < 2; ++tv) {
#pragma unroll
      for (int ar = 0; ar < 4; ++ar) {
        const int vb = v0 + 64 * wv + 32 * tv + 8 * ar + 4 * h;   // multiple of 4
        const float z0 = acc[tv][tm][4 * ar], z1 = acc[tv][tm][4 * ar + 1];
        const float z2 = acc[tv][tm][4 * ar + 2], z3 = acc[tv][tm][4 * ar + 3];
        if (mok) {
          float* dst = a.logits + static_cast<size_t>(m) * a.V + vb;
          if (vec_ok && vb + 3 < a.V) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{z0, z1, z2, z3};
          } else {
            if (vb < a.V) dst[0] = z0;
            if (vb + 1 < a.V) dst[1] = z1;
            if (vb + 2 < a.V) dst[2] = z2;
            if (vb + 3 < a.V) dst[3] = z3;
          }
          if (vb < a.V) {
            const u32x4 w = philox4x32_10(u32x4{static_cast<uint32_t>(vb >> 2), pos, rid, kStreamDraft},
                                          a.key0, a.key1);
            const float zz[4] = {z0, z1, z2, z3};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (vb + e < a.V) {
                se += __builtin_amdgcn_exp2f((zz[e] - mx) * kLog2e);
                const float key = zz[e] + gumbel_from_bits(w[e]);
                if (better(key, vb + e, best.key, best.idx)) best = Cand{key, vb + e};
              }
            }
          }
        }
      }
    }
    // merge the two halves of the wave (same row, other vocab entries)
    {
      const float omx = xor_shuffle(mx, 32), ose = xor_shuffle(se, 32);
      const float nmx = fmaxf(mx, omx);
      se = se * __builtin_amdgcn_exp2f((mx - nmx) * kLog2e) + ose * __builtin_amdgcn_exp2f((omx - nmx) * kLog2e);
      mx = nmx;
      const float ok = xor_shuffle(best.key, 32);
      const int oi = xor_shuffle(best.idx, 32);
      if (better(ok, oi, best.key, best.idx)) best = Cand{ok, oi};
    }
    // merge the two vocab waves (wv = 0, 1) of this row block through LDS
    float* slot4 = red + ((wm * 2 + tm) * 32 + (lane & 31)) * 4;
    __syncthreads();
    if (wv == 1 && h == 0) {
      slot4[0] = mx;
      slot4[1] = se;
      slot4[2] = best.key;
      slot4[3] = __int_as_float(best.idx);
    }
    __syncthreads();
    if (wv == 0 && h == 0 && mok) {
      const float omx = slot4[0], ose = slot4[1], ok = slot4[2];
      const int oi = __float_as_int(slot4[3]);
      const float nmx = fmaxf(mx, omx);
      se = se * __builtin_amdgcn_exp2f((mx - nmx) * kLog2e) + ose * __builtin_amdgcn_exp2f((omx - nmx) * kLog2e);
      if (better(ok, oi, best.key, best.idx)) best = Cand{ok, oi};
      a.part[static_cast<size_t>(m) * a.n_vt + vt] = make_float4(nmx, se, best.key, __int_as_float(best.idx));
    }
  }
}

__global__ __launch_bounds__(kThreads) void lm_row_reduce(LmArgs a) {
  __shared__ float sh[kThreads / 64];
  __shared__ float shk[kThreads / 64];
  __shared__ int shi[kThreads / 64];
  const int m = blockIdx.x;
  const float4* p = a.part + static_cast<size_t>(m) * a.n_vt;
  float mx = -FLT_MAX;
  for (int i = threadIdx.x; i < a.n_vt; i += kThreads) mx = fmaxf(mx, p[i].x);
  mx = block_reduce_max<kThreads>(mx, sh);
  float se = 0.f;
  Cand best{-FLT_MAX, 0x7fffffff};
  for (int i = threadIdx.x; i < a.n_vt; i += kThreads) {
    const float4 q = p[i];
    se += q.y * __builtin_amdgcn_exp2f((q.x - mx) * kLog2e);
    const int idx = __float_as_int(q.w);
    if (better(q.z, idx, best.key, best.idx)) best = Cand{q.z, idx};
  }
  se = block_reduce_sum<kThreads>(se, sh);
  best = block_best<kThreads>(best, shk, shi);
  if (threadIdx.x == 0) {
    a.lse[m] = mx + logf(se);
    a.tokens[m] = best.idx;
  }
}

}  // namespace

hipError_t launch_lm_head(const LmArgs& a, hipStream_t s) {
  const int slots = (a.n_vt + 7) / 8 * a.n_mt;
  hipLaunchKernelGGL(lm_gemm, dim3(slots * 8), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(lm_row_reduce, dim3(a.M), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sd
