// Drafter LM head: logits = hidden W^T on MFMA, then the draft softmax
// statistics and Gumbel-max draft sampling ("LongSpark", sec. 2.1, eq. (4)
// and App. A.1, Fig. 6: the frozen target vocabulary head produces every
// slot's base logits in parallel and each slot is sampled independently).
//
// lm_gemm<Shape>: one workgroup computes a BV-vocab x BM-row tile of
// logits^T = W * hidden^T with MFMA 32x32x16 bf16 (fp32 accumulation); each
// wave owns a (32 TV) x (32 TM) sub-tile.  Both operands are H-contiguous.
// They stream through a ring of LDS stages of BK hidden dims (W rows, then
// hidden rows, per stage), filled by direct-to-LDS loads: each 1 KiB wave
// load covers whole BK-dim row segments (16 rows x 64 bytes at BK = 32, 8
// rows x 128 bytes at BK = 64), so global reads stay coalesced, and rows are
// stored with a 16-byte-chunk XOR swizzle so the MFMA operand reads (32 rows,
// one chunk) are conflict-free.  Six shapes:
//   Tall   (320 x 256, 8 waves of 160 x 64, 64-dim stages, 2 x 72 KiB ring,
//           one workgroup per CU): the fewest operand bytes per output that
//           the registers allow (160 accumulators per lane), and at a
//           151,936-entry vocabulary 475 vocab tiles, under two rounds over
//           the 256 CUs.  Used above 128 rows whenever it yields at
//           least one tile per CU.
//   Narrow (128 x 256, 4 waves of 64 x 128, 32-dim stages, 3 x 24 KiB ring,
//           two workgroups per CU): more, smaller tiles for launches too
//           small to fill the CUs with the tall tiles (e.g. a 32,000-entry
//           pruned vocabulary at 256 rows: 250 tiles against 100).
//   Small  (128 x 128, 4 waves of 64 x 64, 64-dim stages, 2 x 32 KiB ring):
//           twice as many tiles again, for launches whose narrow tiles
//           would still leave the CUs' second slots empty.
//   Short  (320 x 64, 4 waves of 160 x 32, 64-dim stages, 3 x 48 KiB ring,
//           one workgroup per CU): up to 64 draft rows (small decode
//           batches), where the W stream is the whole cost and the tall
//           tile's 256 rows would be mostly padding; two W stages in flight
//           per CU.  0.31-0.34 -> 0.24 ms at 16-64 rows x 151,936 x 4096.
//   Mid    (320 x 128, 4 waves of 160 x 64, 64-dim stages, 2 x 56 KiB ring,
//           one workgroup per CU): 65-128 rows on the same grounds,
//           0.33-0.34 -> 0.29-0.31 ms at that vocabulary.
//   Slim   (128 x 64, 4 waves of 64 x 32, 64-dim stages, 3 x 24 KiB ring,
//           two workgroups per CU): up to 64 rows when the short tiles would
//           not fill the CUs (small or pruned vocabularies); at 32,000 x 4096
//           0.10 -> 0.065 ms, and the small tiles at 65-128 rows
//           0.12 -> 0.08 ms.
// The per-CU rate at which the operand loads arrive, not the MFMAs (the
// LDS-to-MFMA loop alone runs at the MFMA ceiling), bounds this kernel, so
// the tile shape that moves the fewest bytes per output wins: measured at
// 151,936 x 4096, 0.48 -> 0.39 ms at 256 rows and 1.45 -> 1.38 ms at 1,024
// rows against 256 x 256 tiles of 64 x 128 per wave.  All shapes but the
// small one deal each wave's refill loads over the stage's k-steps instead
// of issuing them in one burst (about 3% faster for the tall and narrow
// tiles; the small shape, with two loads per k-step, is faster with the
// burst).
// Tiles are ordered so that all row tiles of one vocab tile, and a compact
// block of vocab tiles, run together on one XCD (blockIdx % 8 picks the XCD),
// which keeps every W and hidden slice in that XCD's L2 across row tiles.
// The epilogue stores the fp32 logits and writes per (row, vocab tile) the
// max, the sum of exp relative to it and the best Gumbel-max candidate
// (Philox stream 0).
//
// lm_row_reduce: merges the per-tile statistics of a row into lse and the
// draft token.
#include "sd_common.h"
#include "sd_internal.h"

#include <float.h>

namespace sd {
namespace {

constexpr int kThreads = 256;                       // lm_row_reduce: 4 waves
constexpr int kShortMaxRows = 64;                   // draft rows up to which the short tiles serve
constexpr int kMidMaxRows = 128;                    // and then the mid tiles

// Tile shape: TV x TM MFMA tiles (32 x 32) per wave, WVN x WMN waves (vocab x
// rows), BK hidden dims per stage, NS stages in the LDS ring.
template <int TV_, int TM_, int WVN_, int WMN_, int BK_, int NS_, bool Spread_>
struct LmShape {
  static constexpr int TV = TV_, TM = TM_, WVN = WVN_, WMN = WMN_, BK = BK_, NS = NS_;
  static constexpr bool Spread = Spread_;   // stage refill dealt over the k-steps
  static constexpr int Waves = WVN * WMN;
  static constexpr int Threads = 64 * Waves;
  static constexpr int BV = 32 * TV * WVN;                // vocab rows per tile
  static constexpr int BM = 32 * TM * WMN;                // draft rows per tile
  static constexpr int RowBytes = 2 * BK;                 // one row of a stage
  static constexpr int Chunks = BK / 8;                   // 16-byte chunks per row
  static constexpr int RowsPerLoad = 1024 / RowBytes;     // rows one wave load covers
  static constexpr int KSteps = BK / 16;                  // MFMA k-steps per stage
  static constexpr int WBytes = BV * RowBytes;            // W rows of one stage
  static constexpr int HBytes = BM * RowBytes;            // hidden rows of one stage
  static constexpr int StageBytes = WBytes + HBytes;
  static constexpr int WLoads = WBytes / 1024 / Waves;    // direct-to-LDS loads per wave per stage
  static constexpr int HLoads = HBytes / 1024 / Waves;
  static constexpr int Loads = WLoads + HLoads;
  static_assert(WLoads * 1024 * Waves == WBytes && HLoads * 1024 * Waves == HBytes,
                "a stage is a whole number of wave loads per wave");
  // 16-byte chunk c of row r of a staged tile sits at byte
  // RowBytes r + 16 (c ^ swz(r)).  A 256-byte span of LDS covers all 64
  // banks; the rows sharing one span (256 / RowBytes of them) keep their
  // chunks in place and consecutive spans rotate them, so 16 consecutive rows
  // of one chunk fall in 16 different 16-byte bank groups.
  static __device__ __forceinline__ int swz(int r) { return (r / (256 / RowBytes)) & (Chunks - 1); }
};
using TallShape = LmShape<5, 2, 2, 4, 64, 2, true>;     // 320 x 256: 8 waves of 160 x 64
using NarrowShape = LmShape<2, 4, 2, 2, 32, 3, true>;   // 128 x 256: 4 waves of 64 x 128
using SmallShape = LmShape<2, 2, 2, 2, 64, 2, false>;   // 128 x 128: 4 waves of 64 x 64
using ShortShape = LmShape<5, 1, 2, 2, 64, 3, true>;    // 320 x 64: 4 waves of 160 x 32
using MidShape = LmShape<5, 2, 2, 2, 64, 2, true>;      // 320 x 128: 4 waves of 160 x 64
using SlimShape = LmShape<2, 1, 2, 2, 64, 3, true>;     // 128 x 64: 4 waves of 64 x 32
static_assert(kLmHMultiple % 64 == 0, "H is a whole number of stages of either shape");
static_assert(NarrowShape::BV == kLmBV && SmallShape::BV == kLmBV && SlimShape::BV == kLmBV,
              "the workspace is sized for the 128-vocab tiles");
static_assert(SmallShape::NS * SmallShape::StageBytes == 64 * 1024, "two small workgroups per CU");
static_assert(ShortShape::NS * ShortShape::StageBytes == 144 * 1024, "one short workgroup per CU");
static_assert(MidShape::NS * MidShape::StageBytes == 112 * 1024, "one mid workgroup per CU");
static_assert(SlimShape::NS * SlimShape::StageBytes == 72 * 1024, "two slim workgroups per CU");
static_assert(TallShape::NS * TallShape::StageBytes == 144 * 1024 &&
              NarrowShape::NS * NarrowShape::StageBytes == 72 * 1024,
              "one tall or two narrow workgroups per CU");

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

template <typename T>
__global__ __launch_bounds__(T::Threads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void lm_gemm(LmArgs a) {
  constexpr int BK = T::BK, WV = T::WVN, TV = T::TV, TM = T::TM;
  constexpr int kNS = T::NS, kStageBytes = T::StageBytes, kWBytes = T::WBytes;
  constexpr int kRow = T::RowBytes, kChunks = T::Chunks, kRowsPerLoad = T::RowsPerLoad;
  constexpr int kWLoads = T::WLoads, kHLoads = T::HLoads, kLoadsPerWave = T::Loads;
  __shared__ __attribute__((aligned(1024))) char smem[kNS * kStageBytes];
  const int P = blockIdx.x;
  const int xcd = P & 7, slot = P >> 3;
  const int vt = (slot / a.n_mt) * 8 + xcd;
  const int mt = slot % a.n_mt;
  if (vt >= a.n_vt) return;
  const int v0 = vt * T::BV, m0 = mt * T::BM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave % WV, wm = wave / WV, h = lane >> 5;

  // ------------------------------------------------ direct-to-LDS loads
  // Wave w fetches its share of the W rows (loads q = WLoads w ..) and of
  // the hidden rows (loads q = HLoads w ..); load q covers rows
  // RowsPerLoad q .. RowsPerLoad (q + 1) - 1 of its tile, lane l fetching
  // chunk (l % Chunks) ^ swz(row) of row RowsPerLoad q + l / Chunks, so the
  // lanes of one row read its whole BK-dim segment.  Rows past V (or M) read
  // the last row instead and are never stored.
  const uint16_t* src[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const bool is_w = i < kWLoads;
    const int q = is_w ? kWLoads * wave + i : kHLoads * wave + (i - kWLoads);
    const int r = kRowsPerLoad * q + lane / kChunks;
    const int c = (lane % kChunks) ^ T::swz(r);
    const int wr = min(v0 + r, a.V - 1);   // drafter vocab entry -> row of W
    src[i] = is_w ? a.w + static_cast<size_t>(a.vmap ? clampi(a.vmap[wr], 0, a.w_rows - 1) : wr) * a.H + 8 * c
                  : a.hidden + static_cast<size_t>(min(m0 + r, a.M - 1)) * a.H + 8 * c;
  }
  const uint32_t lds_ring = lds_addr(smem);
  // Loads of stage kt; with part >= 0 only the share of k-step `part` (the
  // wave's loads dealt evenly over the stage's k-steps).
  auto issue = [&](int kt, int part) {
    const uint32_t base = lds_ring + (kt % kNS) * kStageBytes;
    static_for<0, kLoadsPerWave>([&](auto i) {
      if (part >= 0 && i * T::KSteps / kLoadsPerWave != part) return;
      constexpr bool is_w = i < kWLoads;
      const uint32_t dst = is_w ? base + (kWLoads * wave + i) * 1024
                                : base + kWBytes + (kHLoads * wave + (i - kWLoads)) * 1024;
      // W is read once per vocab tile at one row tile (and by the few row
      // tiles of one XCD otherwise): the non-temporal policy keeps it from
      // pushing the shared hidden rows out of the caches
      if constexpr (is_w) dma16_stream(src[i] + kt * BK, dst);
      else dma16(src[i] + kt * BK, dst);
    });
  };

  // ---------------------------------------------------- operand offsets
  // A operand (W row 64 wv + 32 tv + l % 32) and B operand (hidden row
  // 128 wm + 32 tm + l % 32), chunk 2 s + h of the stage's BK dims.
  const int rr = lane & 31;
  const int sw = T::swz(rr);   // swz(32 k + rr) == swz(rr)
  int offA[T::KSteps], offB[T::KSteps];
#pragma unroll
  for (int s = 0; s < T::KSteps; ++s) {
    offA[s] = (32 * TV * wv + rr) * kRow + (((2 * s + h) ^ sw) << 4);
    offB[s] = kWBytes + (32 * TM * wm + rr) * kRow + (((2 * s + h) ^ sw) << 4);
  }

  f32x16 acc[TV][TM];
#pragma unroll
  for (int i = 0; i < TV; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x16{};

  const int nk = a.H / BK;
#pragma unroll
  for (int t = 0; t < kNS - 1; ++t)
    if (t < nk) issue(t, -1);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed; issued so far: stages up to kt + kNS - 2
    wait_stage<kLoadsPerWave, kNS - 2>(nk - 1 - kt);
    stage_barrier();
    // refill the stage every wave finished reading last iteration: in one
    // burst, or (Spread) a share before each k-step's operand reads, so that
    // no wave holds its MFMAs back behind a queue of load issues
    const bool refill = kt + kNS - 1 < nk;
    if (!T::Spread && refill) issue(kt + kNS - 1, -1);
    const char* st = smem + (kt % kNS) * kStageBytes;
#pragma unroll
    for (int s = 0; s < T::KSteps; ++s) {
      if (T::Spread && refill) issue(kt + kNS - 1, s);
      bf16x8 af[TV], bfr[TM];
#pragma unroll
      for (int t = 0; t < TV; ++t)
        af[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + offA[s] + t * 32 * kRow));
#pragma unroll
      for (int t = 0; t < TM; ++t)
        bfr[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + offB[s] + t * 32 * kRow));
#pragma unroll
      for (int tv = 0; tv < TV; ++tv)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) acc[tv][tm] = mfma_32x32x16(af[tv], bfr[tm], acc[tv][tm]);
    }
  }

  // ---------------------------------------------------------------- epilogue
  // acc[tv][tm][i]: vocab v0 + 32 TV wv + 32 tv + 8 (i/4) + 4 h + i%4,
  //                 row    m0 + 32 TM wm + 32 tm + lane%32
  // Each lane holds 16 TV vocab entries of one row per row tile: it stores them
  // and folds them into the row's (max, sum of exp, best Gumbel-max
  // candidate) over this vocab tile; the WV vocab waves (wv) merge through
  // LDS (the ring is free once every wave is past the loop).
  //
  // Full tiles (every row and vocab entry in range, 16-byte aligned rows; all
  // but the last vocab tile) take a branch-free path that draws with the
  // ratio form of the Gumbel-max key: with p_v = exp(z_v - max) (the terms of
  // the sum of exp) and E_v = -ln u_v, argmax_v (z_v - ln E_v) is argmax_v
  // p_v / E_v, tracked by comparing p_v E_best > p_best E_v, so each entry
  // costs one logarithm instead of two; the lane's best key in log form is
  // max + ln(p_best / E_best).  It ranks entries as the log form does up to
  // fp32 rounding (about 1e-7 in key units).
  __syncthreads();
  float4* red = reinterpret_cast<float4*>(smem);   // [wv][wm][tm][32]
  const bool vec_ok = (a.V & 3) == 0;
  const bool full = !a.greedy && vec_ok && v0 + T::BV <= a.V && m0 + T::BM <= a.M;
  static_for<0, TM>([&](auto TMi) {
    const int m = m0 + 32 * TM * wm + 32 * TMi + rr;
    const bool mok = m < a.M;
    uint32_t rid = 0, pos = 0;
    if (mok) row_owner(a, m, rid, pos);
    float mx = -FLT_MAX;
    float se = 0.f;
    Cand best{-FLT_MAX, 0x7fffffff};
    if (full) {
      static_for<0, TV>([&](auto TVi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[TVi][TMi][i]);
      });
      float* row = a.logits + static_cast<size_t>(m) * a.V;
      float pb = -1.f, eb = 1.f;
      int ib = 0x7fffffff;
      static_for<0, TV>([&](auto TVi) {
#pragma unroll
        for (int ar = 0; ar < 4; ++ar) {
          const int vb = v0 + 32 * TV * wv + 32 * TVi + 8 * ar + 4 * h;   // multiple of 4
          const f32x4 z = {acc[TVi][TMi][4 * ar], acc[TVi][TMi][4 * ar + 1], acc[TVi][TMi][4 * ar + 2],
                           acc[TVi][TMi][4 * ar + 3]};
          *reinterpret_cast<f32x4*>(row + vb) = z;
          const u32x4 w = philox4x32_10(u32x4{static_cast<uint32_t>(vb >> 2), pos, rid, kStreamDraft},
                                        a.key0, a.key1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f((z[e] - mx) * kLog2e);
            se += pv;
            const float u = static_cast<float>((w[e] >> 9) * 2u + 1u) * 5.9604644775390625e-8f;
            const float ev = -kLn2 * __builtin_amdgcn_logf(u);              // -ln u > 0
            // entries arrive in increasing order: a tie keeps the smaller index
            if (pv * eb > pb * ev) {
              pb = pv;
              eb = ev;
              ib = vb + e;
            }
          }
        }
      });
      best = Cand{mx + kLn2 * (__builtin_amdgcn_logf(pb) - __builtin_amdgcn_logf(eb)), ib};
    } else {
    static_for<0, TV>([&](auto TVi) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 32 * TV * wv + 32 * TVi + 8 * (i >> 2) + 4 * h + (i & 3);
        if (v < a.V) mx = fmaxf(mx, acc[TVi][TMi][i]);
      }
    });
    if (mok) {
      float* row = a.logits + static_cast<size_t>(m) * a.V;
      static_for<0, TV>([&](auto TVi) {
#pragma unroll
        for (int ar = 0; ar < 4; ++ar) {
          const int vb = v0 + 32 * TV * wv + 32 * TVi + 8 * ar + 4 * h;   // multiple of 4
          const f32x4 z = {acc[TVi][TMi][4 * ar], acc[TVi][TMi][4 * ar + 1], acc[TVi][TMi][4 * ar + 2],
                           acc[TVi][TMi][4 * ar + 3]};
          if (vec_ok && vb + 3 < a.V) {
            *reinterpret_cast<f32x4*>(row + vb) = z;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (vb + e < a.V) row[vb + e] = z[e];
          }
          if (vb < a.V) {
            // Gumbel-max keys; greedy decoding ranks the logits themselves
            const u32x4 w = a.greedy ? u32x4{0u, 0u, 0u, 0u}
                                     : philox4x32_10(u32x4{static_cast<uint32_t>(vb >> 2), pos, rid,
                                                           kStreamDraft},
                                                     a.key0, a.key1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (vb + e < a.V) {
                se += __builtin_amdgcn_exp2f((z[e] - mx) * kLog2e);
                const float key = a.greedy ? z[e] : z[e] + gumbel_from_bits(w[e]);
                if (better(key, vb + e, best.key, best.idx)) best = Cand{key, vb + e};
              }
            }
          }
        }
      });
    }
    }
    // the two halves of the wave hold the same row, other vocab entries
    {
      const float omx = xor_shuffle(mx, 32), ose = xor_shuffle(se, 32);
      const float nmx = fmaxf(mx, omx);
      se = se * __builtin_amdgcn_exp2f((mx - nmx) * kLog2e) + ose * __builtin_amdgcn_exp2f((omx - nmx) * kLog2e);
      mx = nmx;
      const float ok = xor_shuffle(best.key, 32);
      const int oi = xor_shuffle(best.idx, 32);
      if (better(ok, oi, best.key, best.idx)) best = Cand{ok, oi};
    }
    if (wv != 0 && h == 0)
      red[((wv * T::WMN + wm) * TM + TMi) * 32 + rr] = make_float4(mx, se, best.key, __int_as_float(best.idx));
    __syncthreads();
    if (wv == 0 && h == 0 && mok) {
#pragma unroll
      for (int o2 = 1; o2 < WV; ++o2) {
        const float4 o = red[((o2 * T::WMN + wm) * TM + TMi) * 32 + rr];
        const int oi = __float_as_int(o.w);
        const float nmx = fmaxf(mx, o.x);
        se = se * __builtin_amdgcn_exp2f((mx - nmx) * kLog2e) + o.y * __builtin_amdgcn_exp2f((o.x - nmx) * kLog2e);
        mx = nmx;
        if (better(o.z, oi, best.key, best.idx)) best = Cand{o.z, oi};
      }
      a.part[static_cast<size_t>(m) * a.n_vt + vt] = make_float4(mx, se, best.key, __int_as_float(best.idx));
    }
  });
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
    const int t = clampi(best.idx, 0, a.V - 1);
    a.tokens[m] = a.vmap ? clampi(a.vmap[t], 0, a.w_rows - 1) : t;
  }
}

}  // namespace

template <typename T>
hipError_t launch_gemm(LmArgs& b, hipStream_t s) {
  b.n_vt = (b.V + T::BV - 1) / T::BV;
  b.n_mt = (b.M + T::BM - 1) / T::BM;
  const int slots = (b.n_vt + 7) / 8 * b.n_mt;
  return launch_kernel(lm_gemm<T>, dim3(slots * 8), dim3(T::Threads), s, b);
}

hipError_t launch_lm_head(const LmArgs& a, hipStream_t s) {
  // up to 64 rows, the 64-row short tiles when they give every CU a tile
  // (the 256-row tall tiles would compute three quarters padding) and the
  // 128-wide slim ones when they do not; up to 128 rows the 128-row mid
  // tiles on the same condition, else the 128 x 128 small ones; above, the
  // tall tiles when they give every CU at least one tile, else the narrow
  // ones (two workgroups per CU, 2.5x as many tiles); when even those leave
  // CUs' second slots empty (a pruned vocabulary at 256 rows), the 128-row
  // small tiles, twice as many again
  LmArgs b = a;
  const int64_t mt = (a.M + kLmBM - 1) / kLmBM;
  const int64_t tall_tiles = static_cast<int64_t>((a.V + TallShape::BV - 1) / TallShape::BV) * mt;
  const int64_t narrow_tiles = static_cast<int64_t>((a.V + NarrowShape::BV - 1) / NarrowShape::BV) * mt;
  const int64_t short_tiles =
      static_cast<int64_t>((a.V + ShortShape::BV - 1) / ShortShape::BV) * ((a.M + ShortShape::BM - 1) / ShortShape::BM);
  const int64_t mid_tiles =
      static_cast<int64_t>((a.V + MidShape::BV - 1) / MidShape::BV) * ((a.M + MidShape::BM - 1) / MidShape::BM);
  hipError_t e;
  if (a.M <= kShortMaxRows) e = short_tiles >= 256 ? launch_gemm<ShortShape>(b, s) : launch_gemm<SlimShape>(b, s);
  else if (a.M <= kMidMaxRows) e = mid_tiles >= 256 ? launch_gemm<MidShape>(b, s) : launch_gemm<SmallShape>(b, s);
  else if (tall_tiles >= 256) e = launch_gemm<TallShape>(b, s);
  else if (narrow_tiles < 512) e = launch_gemm<SmallShape>(b, s);
  else e = launch_gemm<NarrowShape>(b, s);
  if (e == hipSuccess) e = launch_kernel(lm_row_reduce, dim3(b.M), dim3(kThreads), s, b);
  return e;
}

}  // namespace sd
