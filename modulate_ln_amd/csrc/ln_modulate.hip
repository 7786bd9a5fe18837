// ln_modulate: out = bf16 chain of LN(x) * (1 + scale) + shift on gfx950.
//
// Operation: prhub report on sglang PR #34015 (Sana fused adaLN), 实现拆解 §1
// and 关键源码片段 (layernorm_modulate.py pass 1 / pass 2); Welford step order:
// prhub report on sglang PR #34008, 关键源码片段 (_welford_push).
//
// Design (one wavefront per row, the row held in VGPRs):
//  * lane l of the wave owns vectors l, l+64, l+128, ... of V consecutive
//    bf16 elements (16-byte loads for V = 8), so each load instruction of the
//    wave reads one contiguous 1 KiB stretch of the row;
//  * pass 1: per-lane fp32 Welford over the lane's elements in increasing
//    position, the count a compile-time constant per step so 1/n is an exact
//    correctly rounded immediate; lanes past the row's tail skip a step and
//    carry a smaller count into the merge;
//  * merge: six butterfly levels (DPP quad permutes, ds_swizzle, DPP row
//    rotate, permlane16/32 swaps) with the Chan-Golub-LeVeque update, lower
//    lane first, so every lane ends with the row's (mean, m2);
//  * pass 2 from registers: normalize, modulate and store -- a single HBM
//    read and a single HBM write of the activation.
// Rows whose storage is not vector-aligned or not contiguous take the same
// code with element-wise gathers; the order of arithmetic is identical, so
// the result depends only on the logical values.
//
// rmsnorm_scale_shift ("Fused Kernels" page, table "Normalization":
// RMSNorm + * (1 + scale) + shift; the request-gated fusion table's
// rms_norm(x) * (1 + scale) + shift) is the same kernel family with RMSNorm
// statistics: each lane accumulates fma(x, x, ss) in the same element order,
// the lanes' sums are added pairwise nearest-first, rinv = 1/sqrt(ss/D +
// eps), and x_hat = bf16(x * rinv) enters the same modulate tail.
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include <utility>

#include "device_common.hpp"
#include "host_common.hpp"
#include "ln_row.hpp"
#include "mw_row.hpp"

namespace adaln {
namespace {

struct LnArgs {
  const uint16_t* x;
  int64_t S, D, sx_b, sx_s, sx_d;
  const uint16_t* scale;
  int64_t ssc_b;
  const uint16_t* shift;
  int64_t ssh_b;
  float eps;
  void* out;  // bf16 rows, or E4M3 bytes (kTailFp8)
  float* mean_out;
  float* rstd_out;
  int64_t R;
  const float* qscale;  // kTailFp8: device pointer to the static scale
};

// start of output row r: bf16 elements, or bytes for the FP8 tail
template <int TAIL>
__device__ __forceinline__ void* out_row(const LnArgs& a, int64_t r) {
  if constexpr (TAIL == kTailFp8) return static_cast<uint8_t*>(a.out) + r * a.D;
  return static_cast<uint16_t*>(a.out) + r * a.D;
}

template <int TAIL>
__device__ __forceinline__ float qinv_of(const LnArgs& a) {
  if constexpr (TAIL == kTailFp8) return 1.0f / *a.qscale;
  return 1.0f;
}

// NV = the largest number of vectors any lane owns for the rows this
// instantiation serves (the launcher guarantees D/V <= 64*NV).
template <int V, int NV, bool GATHER, bool RMS, int TAIL>
__global__ __launch_bounds__(256) void ln_modulate_rows(LnArgs a) {
  const float qinv = qinv_of<TAIL>(a);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nvec = a.D / V;
  const float Df = (float)a.D;
  const int64_t nv_lane = nvec > lane ? (nvec - lane + kWave - 1) / kWave : 0;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < a.R;
       r += (int64_t)gridDim.x * 4) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;

    // every lane loads every step (past the tail it re-reads the row's last
    // vector): unguarded loads issue back to back instead of one at a time
    Vec<V> buf[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kWave + lane;
      const int64_t vc = v < nvec ? v : nvec - 1;
      if constexpr (GATHER)
        buf[k] = gather_vec<V>(xr + vc * V * a.sx_d, a.sx_d);
      else
        buf[k] = load_vec<V>(xr + vc * V);
    }

    float mean = 0.0f, m2 = 0.0f;
    lane_stats<V, RMS>(buf, (int)nvec, lane, kWave, mean, m2, std::make_integer_sequence<int, NV>{});
    if constexpr (RMS) {
      sum_lanes<64>(m2);
    } else {
      float n = (float)(nv_lane * V);
      merge_lanes<64>(mean, m2, n, lane);
    }
    const float rstd = finalize_rstd(m2, Df, a.eps);
    if (lane == 0) {
      if (!RMS && a.mean_out) a.mean_out[r] = mean;
      if (a.rstd_out) a.rstd_out[r] = rstd;
    }

    const uint16_t* sc = a.scale + b * a.ssc_b;
    const uint16_t* sh = a.shift + b * a.ssh_b;
    void* orow = out_row<TAIL>(a, r);
    Vec<V> sv[NV], hv[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kWave + lane;
      const int64_t vc = v < nvec ? v : nvec - 1;
      sv[k] = GATHER ? gather_vec<V>(sc + vc * V, 1) : load_vec<V>(sc + vc * V);
      hv[k] = GATHER ? gather_vec<V>(sh + vc * V, 1) : load_vec<V>(sh + vc * V);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kWave + lane;
      if (v < nvec) {
        uint32_t o[V / 2];
        modulate_vec<V, RMS, TAIL, true>(buf[k], sv[k], hv[k], mean, rstd, o);
        put_vec<V, GATHER, TAIL>(orow, v, o, qinv);
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Fast path: contiguous, vector-aligned rows with D <= 8192.
//
// A block serves one batch sample b.  It first turns that sample's adaLN
// rows into two fp32 tables in LDS -- bf16(1 + scale) and shift -- laid out
// [quarter q][vector v][4] so a lane's 16-byte LDS reads are contiguous
// across the wave.  Each of its W waves then streams rows s = j*W + wave, += W*bpb
// (with the prefetch, the next row's loads are in flight while the current
// row is reduced, normalized, modulated and stored; non-temporal: every
// byte is touched once).  The first row's loads are issued before the table is built, so
// the table's latency hides under them.  UNIF (D % (64*V) == 0): every lane
// holds the same count and the merge tree needs no division.
// ---------------------------------------------------------------------------
// Launch shape of the fast path, measured on MI355X (all variants give the
// same bits), for rows of 7-8 vectors per lane, per output stage:
//   PF    prefetch the next row into a second buffer (the wave walks rows);
//         without it a wave holds one row and the grid covers every row
//   BPC   blocks of four waves per compute unit in total
//   XF32  keep an fp32 copy of x for the normalize pass rather than
//         re-widening it from bf16 (one VALU op per element)
//   WPB   waves per block when a wave holds one row (see kWpb)
// The LayerNorm chain and RMSNorm run best with every row in flight at
// once, one row per wave and four waves per SIMD, with the fp32 copy (108
// VGPRs): their VALU work per row is what the last waves to get their data
// wait on, and a prefetched second row costs the fp32 copy (two waves per
// SIMD would remain).  The FP8 stage runs every row in flight too, with the
// fp32 copy (104 VGPRs once its table values are read at their own step):
// 12.57-12.75 us against 13.07-13.31 re-widening x, which once ran 13.23 us
// against 13.40 with the prefetch at two blocks per compute unit (15.66 at
// three).
// The fold keeps the prefetch at three blocks per compute unit.  Shorter rows keep one buffer and an fp32
// copy of x at five blocks per compute unit; longer rows (up to 16 vectors
// per lane, 64 KiB of tables) keep one buffer and re-widen.
#ifndef ADALN_TAB_WPB_LN
#define ADALN_TAB_WPB_LN 16
#endif
#ifndef ADALN_TAB_WPB_FOLD
#define ADALN_TAB_WPB_FOLD 4
#endif
#ifndef ADALN_TAB_WPB_RMS
#define ADALN_TAB_WPB_RMS 4
#endif
#ifndef ADALN_TAB_WPB_FP8
#define ADALN_TAB_WPB_FP8 16
#endif
#ifndef ADALN_TAB_PF_SHORT
#define ADALN_TAB_PF_SHORT 0
#endif
#ifndef ADALN_TAB_BPC_SHORT
#define ADALN_TAB_BPC_SHORT 5
#endif
#ifndef ADALN_TAB_PF_LN
#define ADALN_TAB_PF_LN 0
#endif
#ifndef ADALN_TAB_BPC_LN
#define ADALN_TAB_BPC_LN 4
#endif
#ifndef ADALN_TAB_XF32_LN
#define ADALN_TAB_XF32_LN 1
#endif
#ifndef ADALN_TAB_PF_FOLD
#define ADALN_TAB_PF_FOLD 1
#endif
#ifndef ADALN_TAB_BPC_FOLD
#define ADALN_TAB_BPC_FOLD 3
#endif
#ifndef ADALN_TAB_XF32_FOLD
#define ADALN_TAB_XF32_FOLD 0
#endif
#ifndef ADALN_TAB_PF_RMS
#define ADALN_TAB_PF_RMS 0
#endif
#ifndef ADALN_TAB_BPC_RMS
#define ADALN_TAB_BPC_RMS 4
#endif
#ifndef ADALN_TAB_XF32_RMS
#define ADALN_TAB_XF32_RMS 1
#endif
#ifndef ADALN_TAB_PF_FP8
#define ADALN_TAB_PF_FP8 0
#endif
#ifndef ADALN_TAB_BPC_FP8
#define ADALN_TAB_BPC_FP8 2
#endif
#ifndef ADALN_TAB_XF32_FP8
#define ADALN_TAB_XF32_FP8 1
#endif
// MANY: more rows than the 16-wave shape holds at one per wave (16 per
// compute unit); those take the fold's shape instead, a prefetched next row
// in 4-wave blocks at three per compute unit.  Measured at D = 4096, 16-wave
// blocks vs the prefetch: 4352 rows 18.06 vs 14.08 us, 5120 rows 19.58 vs
// 15.35, 8192 rows 26.28 vs 24.46; FP8 20.95 vs 15.25, 20.89 vs 16.02,
// 23.82 vs 23.23 (at 4096 rows the 16-wave blocks stay: 11.52 vs 12.46).
#ifndef ADALN_TAB_BPC_MANY
#define ADALN_TAB_BPC_MANY 3
#endif
template <int NV, bool UNIF, bool RMS, int TAIL, bool MANY = false>
struct TabShape {
  static constexpr bool kLong = NV == 7 || NV == 8;
  static constexpr int kBpcLong = MANY                ? ADALN_TAB_BPC_MANY
                                  : TAIL == kTailFp8  ? ADALN_TAB_BPC_FP8
                                  : TAIL == kTailFold ? ADALN_TAB_BPC_FOLD
                                  : RMS               ? ADALN_TAB_BPC_RMS
                                                      : ADALN_TAB_BPC_LN;
  static constexpr bool kXf32Long = MANY                ? false
                                    : TAIL == kTailFp8  ? ADALN_TAB_XF32_FP8
                                    : TAIL == kTailFold ? ADALN_TAB_XF32_FOLD
                                    : RMS               ? ADALN_TAB_XF32_RMS
                                                        : ADALN_TAB_XF32_LN;
  static constexpr bool kPfLong = MANY                ? true
                                  : TAIL == kTailFp8  ? ADALN_TAB_PF_FP8
                                  : TAIL == kTailFold ? ADALN_TAB_PF_FOLD
                                  : RMS               ? ADALN_TAB_PF_RMS
                                                      : ADALN_TAB_PF_LN;
  static constexpr bool kPrefetch = kLong ? kPfLong : (NV <= 6 && ADALN_TAB_PF_SHORT);
  static constexpr bool kXf32 = NV <= 6 || (kLong && kXf32Long);
  // waves per block: one row per wave and every row in flight lets one
  // block per compute unit hold all its waves, so the tables are built once
  // per compute unit rather than once per four rows.  Rows with a partial
  // last vector step need more than the 128 VGPRs a 16-wave block allows
  // (they would spill), so they keep 4-wave blocks.
  // Measured: the LayerNorm chain 11.57 us at 16 waves per block, 11.79 at
  // 8, 12.12 at 4 ((1,4096,4096)); RMSNorm, whose statistic is a quarter of
  // the Welford work per element, 11.04 at 4, 11.45 at 16.  The fold keeps
  // its prefetch (11.32 us; 11.66 with one row per wave in 16-wave blocks).
  static constexpr int kWpbLong = TAIL == kTailFold   ? ADALN_TAB_WPB_FOLD
                                  : TAIL == kTailFp8  ? ADALN_TAB_WPB_FP8
                                  : RMS               ? ADALN_TAB_WPB_RMS
                                                      : ADALN_TAB_WPB_LN;
  static constexpr int kWpb = (kLong && !kPrefetch && UNIF) ? kWpbLong : 4;
  static constexpr int kBlocksPerCu =
      NV <= 6 ? ADALN_TAB_BPC_SHORT : (kLong ? (kBpcLong * 4 + kWpb - 1) / kWpb : 2);
};


template <int V, int NV, bool UNIF, bool RMS, int TAIL, bool MANY = false>
__global__ __launch_bounds__((TabShape<NV, UNIF, RMS, TAIL, MANY>::kWpb * 64)) void ln_modulate_tab(LnArgs a,
                                                                                                  int bpb) {
  constexpr int kWpb = TabShape<NV, UNIF, RMS, TAIL, MANY>::kWpb;
  constexpr bool kPrefetch = TabShape<NV, UNIF, RMS, TAIL, MANY>::kPrefetch;
  constexpr bool kXf32 = TabShape<NV, UNIF, RMS, TAIL, MANY>::kXf32;
  extern __shared__ float4 tab[];  // [2][V/4][nvec] float4: bf16(1+scale), then shift
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = (int)a.D;
  const int nvec = D / V;
  const int S = (int)a.S;
  const int b = blockIdx.x / bpb;
  const int j = blockIdx.x - b * bpb;
  const int row_step = kWpb * bpb;
  int s = kWpb * j + wave;

  const uint16_t* xb = a.x + (int64_t)b * a.sx_b;
  auto load_row = [&](Vec<V>* buf, int ss) {
    const uint16_t* xr = xb + (int64_t)ss * a.sx_s;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * kWave + lane;
      const int vc = (UNIF || v < nvec) ? v : nvec - 1;
      buf[k] = load_vec_nt<V>(xr + vc * V);
    }
  };

  Vec<V> bufA[NV];
  Vec<V> bufB[kPrefetch ? NV : 1];
  if (s < S) load_row(bufA, s);
  const bool fin = build_tables<V>(tab, a.scale + (int64_t)b * a.ssc_b, a.shift + (int64_t)b * a.ssh_b, nvec,
                                   threadIdx.x, kWpb * kWave);
  bool tab_finite = true;
  if constexpr (TAIL == kTailFp8)
    tab_finite = __syncthreads_and(fin);
  else
    __syncthreads();
  if (s >= S) return;

  const float Df = (float)D;
  const float qinv = qinv_of<TAIL>(a);
  auto process = [&](const Vec<V>* buf, int ss) {
    const int64_t r = (int64_t)b * S + ss;
    normalize_row<V, NV, UNIF, kXf32, RMS, TAIL>(buf, tab, nvec, lane, Df, a.eps, out_row<TAIL>(a, r),
                                                 a.mean_out ? a.mean_out + r : nullptr,
                                                 a.rstd_out ? a.rstd_out + r : nullptr, qinv, tab_finite);
  };

  if constexpr (kPrefetch) {
    // double buffer: row s is in A (or B) while the next row loads into B (or A)
    while (true) {
      int s1 = s + row_step;
      if (s1 < S) load_row(bufB, s1);
      process(bufA, s);
      if (s1 >= S) break;
      s = s1;
      s1 = s + row_step;
      if (s1 < S) load_row(bufA, s1);
      process(bufB, s);
      if (s1 >= S) break;
      s = s1;
    }
  } else {
    while (true) {
      process(bufA, s);
      s += row_step;
      if (s >= S) break;
      load_row(bufA, s);
    }
  }
}

// ---------------------------------------------------------------------------
// Transposed input: tokens contiguous (sx_s == 1), hidden elements sx_d apart
// -- the permuted activations the Sana report describes (实现拆解 §3, the
// layout copy aten's LayerNorm pays).  A block of 8 waves takes a tile of 8
// consecutive tokens of one sample.  Thread i loads hidden positions i,
// i + 512, ..., each as one 16-byte load of the tile's 8 tokens (so every
// 128-byte line of the input is read once, by the 8 tiles that share it,
// and the lanes of a wave read consecutive hidden positions), and scatters
// the 8 values into an LDS tile [token][hidden].  Wave w then runs the same
// per-row routine as the contiguous kernel on token w, reading its row from
// LDS: identical bits, one HBM read and one HBM write, no layout copy.
// (Measured on MI355X at (2,1024,2240): 10.52 us against 10.70 us when each
// thread loaded its vector's 8 hidden positions and transposed 8x8 blocks
// in registers; 4-token tiles (twice the blocks, 8-byte loads) 13.1 us and
// 16-token tiles 14.5 us in a copy of the same layout.)
// ---------------------------------------------------------------------------
constexpr int kTrTokens = 8;

template <int NV, bool UNIF, bool RMS, int TAIL>
__global__ __launch_bounds__(512) void ln_modulate_tr(LnArgs a, int tiles_per_sample) {
  constexpr int V = 8;
  extern __shared__ float4 smem[];  // tables [2][2][nvec], then the x tile [8][nvec] (uint4)
  const int D = (int)a.D;
  const int nvec = D / V;
  const int S = (int)a.S;
  // tiles of one XCD (blockIdx mod 8) are consecutive, so the 8 tiles that
  // share each input line run on the same L2
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int tile = (nblk % 8 == 0) ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
  const int b = tile / tiles_per_sample;
  const int t0 = (tile - b * tiles_per_sample) * kTrTokens;
  float4* tab = smem;
  uint4* xt = reinterpret_cast<uint4*>(smem + 4 * nvec);

  const uint16_t* xb = a.x + (int64_t)b * a.sx_b + t0;
  uint16_t* xs = reinterpret_cast<uint16_t*>(xt);  // the tile as [token][D] bf16
  uint4 c[NV];  // c[k]: tokens t0..t0+7 of hidden position threadIdx.x + 512 k
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int h = threadIdx.x + 512 * k;
    if (h < D) {
      u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xb + (int64_t)h * a.sx_d));
      c[k] = make_uint4(t[0], t[1], t[2], t[3]);
    }
  }
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int h = threadIdx.x + 512 * k;
    if (h < D) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = (&c[k].x)[q];
        xs[(2 * q) * D + h] = (uint16_t)(w & 0xffffu);
        xs[(2 * q + 1) * D + h] = (uint16_t)(w >> 16);
      }
    }
  }
  const bool fin = build_tables<V>(tab, a.scale + (int64_t)b * a.ssc_b, a.shift + (int64_t)b * a.ssh_b, nvec,
                                   threadIdx.x, 512);
  bool tab_finite = true;
  if constexpr (TAIL == kTailFp8)
    tab_finite = __syncthreads_and(fin);
  else
    __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // token within the tile
  Vec<V> buf[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = k * kWave + lane;
    const uint4 t = xt[w * nvec + ((UNIF || v < nvec) ? v : nvec - 1)];
    buf[k].w[0] = t.x;
    buf[k].w[1] = t.y;
    buf[k].w[2] = t.z;
    buf[k].w[3] = t.w;
  }
  const int64_t r = (int64_t)b * S + t0 + w;
  normalize_row<V, NV, UNIF, true, RMS, TAIL>(buf, tab, nvec, lane, (float)D, a.eps, out_row<TAIL>(a, r),
                                              a.mean_out ? a.mean_out + r : nullptr,
                                              a.rstd_out ? a.rstd_out + r : nullptr, qinv_of<TAIL>(a), tab_finite);
}

// ---------------------------------------------------------------------------
// Rows of more than 4096 elements: W = 2 .. 16 waves per row (one row per
// block of 64 * W threads at a time), every lane holding at most 64 elements
// of the row in registers (a single HBM read and a single HBM write at any
// D), the waves' states merged through LDS in the fixed tree of mw_row.hpp.
// The per-sample adaLN rows are read through the caches (a sample's rows are
// shared by all its tokens).  NV: the most vector steps a lane takes (8 for
// V = 8, 16 for V = 4); UNIF: every lane takes all NV.
// ---------------------------------------------------------------------------
template <int V, int NV, bool UNIF, bool GATHER, bool RMS, int TAIL>
__global__ __launch_bounds__(kMaxWaves * 64) void ln_modulate_mw(LnArgs a) {
  __shared__ MwSlots slots;
  const int W = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int L = W * kWave;
  const int g = threadIdx.x;
  const int lane = g & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(g >> 6);
  const int nvec = (int)(a.D / V);
  const float Df = (float)a.D;
  const float qinv = qinv_of<TAIL>(a);
  int parity = 0;
  for (int64_t r = blockIdx.x; r < a.R; r += gridDim.x, parity ^= 1) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;
    Vec<V> buf[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (UNIF || k * L < nvec) {  // block-uniform: steps past the row are not loaded
        const int v = k * L + g;
        const int vc = v < nvec ? v : nvec - 1;
        if constexpr (GATHER)
          buf[k] = gather_vec<V>(xr + (int64_t)vc * V * a.sx_d, a.sx_d);
        else
          buf[k] = load_vec_nt<V>(xr + (uint32_t)(vc * V));  // 32-bit offset from a scalar row base
      }
    }
    float mean, m2;
    mw_stats<V, NV, UNIF, RMS>(buf, nvec, g, lane, wave, W, slots.s[parity], mean, m2);
    const float rstd = finalize_rstd(m2, Df, a.eps, pow2_inverse_f(Df));
    if (g == 0) {
      if (!RMS && a.mean_out) a.mean_out[r] = mean;
      if (a.rstd_out) a.rstd_out[r] = rstd;
    }
    const uint16_t* sc = a.scale + b * a.ssc_b;
    const uint16_t* sh = a.shift + b * a.ssh_b;
    void* orow = out_row<TAIL>(a, r);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * L + g;
      if (UNIF || v < nvec) {
        const uint32_t off = (uint32_t)(v * V);
        const Vec<V> sv = GATHER ? gather_vec<V>(sc + off, 1) : load_vec<V>(sc + off);
        const Vec<V> hv = GATHER ? gather_vec<V>(sh + off, 1) : load_vec<V>(sh + off);
        uint32_t o[V / 2];
        modulate_vec<V, RMS, TAIL, true>(buf[k], sv, hv, mean, rstd, o);
        put_vec<V, GATHER, TAIL>(orow, v, o, qinv);
      }
    }
  }
}

// Rows of 4097 .. 16384 elements with 16-byte vectors, P = 16 / W rows of one
// sample per block of 16 waves: group q (waves qW .. qW + W - 1) takes row
// s0 + q.  The sample's tables -- bf16(1 + scale) and shift as fp32, the
// tabled kernel's layout -- are built in LDS once per block, where
// ln_modulate_mw has each row's block fetch the bf16 rows through the caches
// and widen and round them per element.  Lanes, steps and merges are
// ln_modulate_mw's (the group's lanes g = 0 .. 64W - 1 in the same fixed
// tree), and the tables hold the values its tail computes, so the bits are
// the same.
template <int NV, bool UNIF, bool RMS, int TAIL, int TPB>
__global__ __launch_bounds__(TPB) void ln_modulate_mwt(LnArgs a, int bps, int W) {
  constexpr int V = 8;
  constexpr int kRuns = (2048 + TPB - 1) / TPB;  // adaLN vectors per thread: D <= 2048 * 8
  extern __shared__ float4 tab[];  // [2][V / 4][D / V]
  __shared__ MwSlots slots;
  const int L = W * kWave;
  const int P = TPB / L;  // rows per block
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = wave / W;              // the block's row group
  const int g = threadIdx.x - q * L;   // lane of the row's lane map
  const int lane = threadIdx.x & (kWave - 1);
  const int nvec = (int)(a.D / V);
  const float Df = (float)a.D;
  const float qinv = qinv_of<TAIL>(a);
  const int64_t b = blockIdx.x / bps;
  const int64_t s = (int64_t)(blockIdx.x - b * bps) * P + q;
  const bool act = s < a.S;
  const int64_t r = b * a.S + (act ? s : a.S - 1);  // a group past the sample's rows reads its last row

  // the adaLN vectors are issued first and turned into tables once the row's loads are out
  const uint16_t* sc = a.scale + b * a.ssc_b;
  const uint16_t* sh = a.shift + b * a.ssh_b;
  Vec<V> ts[kRuns], th[kRuns];
#pragma unroll
  for (int i = 0; i < kRuns; ++i) {
    const int j = i * TPB + (int)threadIdx.x;
#pragma unroll
    for (int e = 0; e < V / 2; ++e) ts[i].w[e] = th[i].w[e] = 0u;
    if (j < nvec) {
      ts[i] = load_vec<V>(sc + j * V);
      th[i] = load_vec<V>(sh + j * V);
    }
  }
  const uint16_t* xr = a.x + b * a.sx_b + (r - b * a.S) * a.sx_s;
  Vec<V> buf[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (UNIF || k * L < nvec) {  // wave-uniform: steps past the row are not loaded
      const int v = k * L + g;
      const int vc = v < nvec ? v : nvec - 1;
      buf[k] = load_vec_nt<V>(xr + (uint32_t)(vc * V));
    }
  }
#pragma unroll
  for (int i = 0; i < kRuns; ++i) {
    const int j = i * TPB + (int)threadIdx.x;
    if (j < nvec) put_tables<V>(tab, ts[i], th[i], j, nvec);
  }
  float mean, m2;
  // the group's slots; the barrier inside also publishes the tables
  mw_stats<V, NV, UNIF, RMS>(buf, nvec, g, lane, wave - q * W, W, slots.s[0] + q * W, mean, m2);
  if (!act) return;  // no barrier follows
  const float rstd = finalize_rstd(m2, Df, a.eps, pow2_inverse_f(Df));
  if (g == 0) {
    if (!RMS && a.mean_out) a.mean_out[r] = mean;
    if (a.rstd_out) a.rstd_out[r] = rstd;
  }
  void* orow = out_row<TAIL>(a, r);
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = k * L + g;
    if (UNIF || v < nvec) {
      uint32_t o[V / 2];
#pragma unroll
      for (int h = 0; h < V / 4; ++h) {
        const float4 oc = tab[h * nvec + v], hc = tab[(V / 4 + h) * nvec + v];
        const float x0 = lo_f32_again(buf[k].w[2 * h]), x1 = hi_f32_again(buf[k].w[2 * h]);
        const float x2 = lo_f32_again(buf[k].w[2 * h + 1]), x3 = hi_f32_again(buf[k].w[2 * h + 1]);
        const float n0 = RMS ? x0 * rstd : (x0 - mean) * rstd;
        const float n1 = RMS ? x1 * rstd : (x1 - mean) * rstd;
        const float n2 = RMS ? x2 * rstd : (x2 - mean) * rstd;
        const float n3 = RMS ? x3 * rstd : (x3 - mean) * rstd;
        o[2 * h] = tail_pair<TAIL>(n0, n1, oc.x, oc.y, hc.x, hc.y);
        o[2 * h + 1] = tail_pair<TAIL>(n2, n3, oc.z, oc.w, hc.z, hc.w);
      }
      put_vec<V, false, TAIL>(orow, v, o, qinv);
    }
  }
}

// ---------------------------------------------------------------------------
// Transposed storage read in whole lines, with a workspace (ln_modulate_ws).
// A 128-byte line of [B, D, S] storage holds 64 consecutive tokens of one
// hidden position, so whole-line reads need 64 tokens per block; to keep 256
// compute units busy the 64 lanes of the fixed order are split over 8
// blocks: block c of a 64-token group owns lanes 8c .. 8c + 7 of every token
// (vectors 64k + 8c + j), reads those hidden positions in whole lines, runs
// the lanes' Welford passes and merges them at offsets 1, 2, 4 -- the first
// three levels of the one-wave tree.  Every block then takes the 8 blocks'
// states of its tokens and merges them at offsets 1, 2, 4 -- the tree's
// levels 8, 16, 32.  Same order, same merges: the bits of ln_modulate.
//
// The hand-over needs no fence: each state travels as two 64-bit relaxed
// atomics (tag | mean, tag | m2; the count is known from D), so a reader
// that sees the expected tag in a word has that word's value.  The tag is
// the group's exchange number, kept in one 64-bit word per group
// (generation << 32 | arrivals): each block arrives with one atomic add,
// which returns the generation g, and tags with g + 1; the 8th arrival
// writes generation g + 1 with no arrivals.  After a call every record of
// the group carries the group's generation, so a record of an earlier call
// never carries the tag a reader waits for.  Each group's records and word
// sit in a slab of their own at a fixed place, so this holds whatever
// shapes used the workspace before, as long as it started zero-filled.
//
// The grid is at most what the device holds at once (occupancy x compute
// units), so the 8 blocks of a group run together; the 8 blocks of a slot
// take groups slot, slot + nslots, ... .  The wait is bounded all the same:
// past wait_ticks of the constant-rate clock a thread recomputes the state
// it is missing from x itself (the same arithmetic, so the same bits).
// Measured on MI355X against the one-block-per-8-token-tile kernel above,
// same bits: (2,1024,2240) 8.46 us vs 10.7 (one block per group, row and
// adaLN values in registers: 8.80 with them re-read from LDS), (1,4096,4096)
// 17.5 vs 33.3, (4,4096,3072) 57.9 vs 89.3; the hand-over costs about two
// device-scope memory latencies (~2.3 us per group).
// ---------------------------------------------------------------------------
constexpr int kCoopTokens = 64;  // tokens per group (one 128-byte line per hidden position)
constexpr int kCoopBlocks = 8;   // blocks per group (8 lanes of the 64 each)

// The workspace: one slab of kCoopSlab bytes per token group, at the same
// place whatever the shape of the call (so calls of different shapes can
// share a workspace): [64 tokens][8 blocks] words tag << 32 | mean bits,
// the same for m2, then the group's word generation << 32 | arrivals (no
// arrivals between calls).
constexpr int kCoopRecs = kCoopTokens * kCoopBlocks;  // records per group
constexpr int64_t kCoopSlab = 2 * kCoopRecs * 8 + 64;  // bytes per group (64-byte aligned slabs)
constexpr int64_t coop_ws_bytes(int64_t ntg) { return ntg * kCoopSlab; }

// bytes (lo, hi) of a and bytes (lo, hi) of b -> one word: lo halves or hi halves
__device__ __forceinline__ uint32_t join_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t join_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Lane g's Welford pass over its vectors g, g + 64, ... of one token
// (element h at xt + h * sx_d), one gathered vector at a time, as a runtime
// loop: the k-th element's 1/k is the correctly rounded reciprocal, the
// same value as the compile-time constant of the main pass.
__device__ __forceinline__ void coop_lane_state(const uint16_t* xt, int64_t sx_d, int nvec, int g, float& mean,
                                                float& m2, float& n) {
  mean = 0.0f;
  m2 = 0.0f;
  int cnt = 0;
#pragma unroll 1
  for (int v = g; v < nvec; v += kWave) {
    const Vec<8> x = gather_vec<8>(xt + (int64_t)(8 * v) * sx_d, sx_d);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xe = (e & 1) ? hi_f32(x.w[e / 2]) : lo_f32(x.w[e / 2]);
      ++cnt;
      const float r = __fdiv_rn(1.0f, (float)cnt);
      const float delta = xe - mean;
      mean = __builtin_fmaf(delta, r, mean);
      m2 = __builtin_fmaf(delta, xe - mean, m2);
    }
  }
  n = (float)cnt;
}

// The state of lanes 8c .. 8c + 7 of one token merged at offsets 1, 2, 4 --
// the recompute of another block's share when its hand-over is late.  The
// lanes are taken in turn and merged as a binary counter (after an odd lane
// its pair, after lane 3 mod 4 its quad, after lane 7 the eight), the lower
// state first: the same merges in the same order as the lanes' tree, so the
// same bits.
__device__ __forceinline__ void coop_group_state(const uint16_t* xt, int64_t sx_d, int nvec, int c, float& mean,
                                                 float& m2) {
  float m0 = 0.0f, q0 = 0.0f, n0 = 0.0f;  // pending pair (lane i - 1)
  float m1 = 0.0f, q1 = 0.0f, n1 = 0.0f;  // pending quad half (lanes i - 3 .. i - 2)
  float m4 = 0.0f, q4 = 0.0f, n4 = 0.0f;  // lanes 0 .. 3
  float m = 0.0f, q = 0.0f, n = 0.0f;
#pragma unroll 1
  for (int i = 0; i < 8; ++i) {
    coop_lane_state(xt, sx_d, nvec, 8 * c + i, m, q, n);
    if (i & 1) {
      welford_merge(m0, q0, n0, m, q, n);
      m = m0, q = q0, n = n0;
      if (i & 2) {
        welford_merge(m1, q1, n1, m, q, n);
        m = m1, q = q1, n = n1;
        if (i & 4) {
          welford_merge(m4, q4, n4, m, q, n);
          m = m4, q = q4, n = n4;
        } else {
          m4 = m, q4 = q, n4 = n;
        }
      } else {
        m1 = m, q1 = q, n1 = n;
      }
    } else {
      m0 = m, q0 = q, n0 = n;
    }
  }
  mean = m;
  m2 = q;
}

// ONE: every group has a block of its own (the grid covers the groups in one
// pass, one block per compute unit), so registers are no longer shared with a
// second block: each thread keeps its row and its own fp32 adaLN values
// (loaded while it waits for the hand-over) in registers, and the tail reads
// no LDS.  Otherwise the tail re-reads the row from the LDS tile and the
// adaLN values from per-block LDS tables (two blocks per compute unit).
template <int NV, bool ONE>
__global__ __launch_bounds__(512) void ln_modulate_trc(LnArgs a, char* ws, int groups_per_sample, int ngroups,
                                                      uint64_t wait_ticks) {
  constexpr int V = 8;
  constexpr int NT = ONE ? 1 : NV;  // steps of the LDS tables
  // [step][token][lane of the block ^ (token / 8)]: 16-byte vectors; the xor
  // spreads the 8 tokens 8 apart that one transpose writes over the banks
  __shared__ uint4 tile[NV][kCoopTokens][8];
  __shared__ float4 otab[NT][8][2];  // bf16(1 + scale) of the block's vectors
  __shared__ float4 htab[NT][8][2];  // shift of the block's vectors
  __shared__ uint32_t tag_sh;
  const int D = (int)a.D;
  const float Df = (float)D;
  // 8 consecutive blocks form a slot (one block per XCD); a slot takes token
  // groups slot, slot + nslots, ... (the grid is sized to be resident at once)
  const int slot = blockIdx.x / kCoopBlocks;
  const int c = blockIdx.x - slot * kCoopBlocks;
  const int nslots = gridDim.x / kCoopBlocks;

  for (int tg = slot; tg < ngroups; tg += nslots) {
    const int b = tg / groups_per_sample;
    const int t0 = (tg - b * groups_per_sample) * kCoopTokens;
    const uint16_t* xg = a.x + (int64_t)b * a.sx_b + t0;  // token t0 of hidden position 0
    uint64_t* mst = reinterpret_cast<uint64_t*>(ws + (int64_t)tg * kCoopSlab);  // the group's slab
    uint64_t* vst = mst + kCoopRecs;
    uint64_t* sync = vst + kCoopRecs;
    if (tg != slot) __syncthreads();  // the previous group's tile, tables and tag have been read
    // the thread index, hidden stride and vector count, opaque to the compiler
    // in each group: what derives from them (indices, LDS and memory offsets,
    // lane counts) is recomputed per group rather than held in registers
    // across the loop
    int tid = threadIdx.x;
    int64_t sx_d = a.sx_d;
    int nvec = D / V;
    __asm__ volatile("" : "+v"(tid), "+s"(sx_d), "+s"(nvec));

    // loads: wave 7 first issues the block's adaLN vectors and the arrival
    // (one atomic add returns the generation and the arrivals before it: the
    // 8th arrival writes the next generation); then thread (k, j, p) of waves
    // 0 .. NV - 1 reads the 8 hidden positions of vector 64k + 8c + j for
    // tokens 8p .. 8p + 7 (a wave's load instruction covers 8 whole lines) and
    // transposes the 8x8 block.  The arrival's result is first used after the
    // transposes, so no wait lies between the loads.
    {
      const int k = tid >> 6, j = (tid >> 3) & 7, p = tid & 7;
      const int tl = tid & (kWave - 1), tk = tl >> 3, tj = tl & 7, tv = 64 * tk + 8 * c + tj;
      const bool tab = !ONE && k == 7 && tl < NV * 8 && tv < nvec;
      Vec<V> sv, hv;
      if (tab) {
        sv = load_vec<V>(a.scale + (int64_t)b * a.ssc_b + V * tv);
        hv = load_vec<V>(a.shift + (int64_t)b * a.ssh_b + V * tv);
      }
      uint64_t old = 0;
      if (tid == 7 * kWave) {
        int z = 0;  // an index the compiler cannot see is zero: a plain one-lane atomic
        __asm__ volatile("" : "+v"(z));
        old = __hip_atomic_fetch_add(sync + z, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const int v = 64 * k + 8 * c + j;
      const bool act = k < NV && v < nvec;
      uint4 cc[V];
      if (act) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          u32x4 t = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(xg + (int64_t)(V * v + e) * sx_d + 8 * p));
          cc[e] = make_uint4(t[0], t[1], t[2], t[3]);
        }
      }
      if (act) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w0 = (&cc[0].x)[q], w1 = (&cc[1].x)[q], w2 = (&cc[2].x)[q], w3 = (&cc[3].x)[q];
          const uint32_t w4 = (&cc[4].x)[q], w5 = (&cc[5].x)[q], w6 = (&cc[6].x)[q], w7 = (&cc[7].x)[q];
          tile[k][8 * p + 2 * q][j ^ p] =
              make_uint4(join_lo(w0, w1), join_lo(w2, w3), join_lo(w4, w5), join_lo(w6, w7));
          tile[k][8 * p + 2 * q + 1][j ^ p] =
              make_uint4(join_hi(w0, w1), join_hi(w2, w3), join_hi(w4, w5), join_hi(w6, w7));
        }
      }
      if (tab) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float o0 = 1.0f + lo_f32(sv.w[2 * q]), o1 = 1.0f + hi_f32(sv.w[2 * q]);
          float o2 = 1.0f + lo_f32(sv.w[2 * q + 1]), o3 = 1.0f + hi_f32(sv.w[2 * q + 1]);
          round_pair(o0, o1);  // bf16(1 + scale)
          round_pair(o2, o3);
          otab[ONE ? 0 : tk][tj][q] = make_float4(o0, o1, o2, o3);
          htab[ONE ? 0 : tk][tj][q] = make_float4(lo_f32(hv.w[2 * q]), hi_f32(hv.w[2 * q]),
                                                  lo_f32(hv.w[2 * q + 1]), hi_f32(hv.w[2 * q + 1]));
        }
      }
      __asm__ volatile("" : "+v"(old));  // the arrival's result is first needed here
      if (tid == 7 * kWave) {
        const uint32_t g0 = (uint32_t)(old >> 32);
        if ((uint32_t)old == kCoopBlocks - 1)
          __hip_atomic_store(sync, (uint64_t)(g0 + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tag_sh = g0 + 1u;
      }
    }
    __syncthreads();

    // thread (t, j): token t, lane 8c + j of the order; the 8 lanes of a token are adjacent
    const int t = tid >> 3, j = tid & 7, lane = tid & (kWave - 1);
    const int g = 8 * c + j;
    const int col = j ^ (t >> 3);
    float mean = 0.0f, m2 = 0.0f;
    Vec<V> buf[NV];  // with ONE kept for the tail; else live for the pass only (the tail re-reads the tile)
#pragma unroll
    for (int k = 0; k < NV; ++k)
      if (64 * k + g < nvec) {
        const uint4 w = tile[k][t][col];
        buf[k].w[0] = w.x;
        buf[k].w[1] = w.y;
        buf[k].w[2] = w.z;
        buf[k].w[3] = w.w;
      }
    // ONE: this thread's adaLN vectors, issued now and turned into fp32 values while the
    // hand-over is in flight
    Vec<V> sv[ONE ? NV : 1], hv[ONE ? NV : 1];
    if constexpr (ONE) {
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (64 * k + g < nvec) {
          sv[k] = load_vec<V>(a.scale + (int64_t)b * a.ssc_b + V * (64 * k + g));
          hv[k] = load_vec<V>(a.shift + (int64_t)b * a.ssh_b + V * (64 * k + g));
        }
    }
    lane_stats<V, false>(buf, nvec, g, kWave, mean, m2, std::make_integer_sequence<int, NV>{});
    float n = (float)((nvec > g ? (nvec - g + kWave - 1) / kWave : 0) * V);
    merge_level<1>(mean, m2, n, lane);
    merge_level<2>(mean, m2, n, lane);
    merge_level<4>(mean, m2, n, lane);  // every lane of the token: the state of lanes 8c .. 8c + 7

    // hand the state over, take the 8 blocks' states of token t (block j's in lane j)
    const uint64_t tag = (uint64_t)tag_sh << 32;
    const int ri = t * kCoopBlocks;
    if (j == 0) {
      __hip_atomic_store(mst + ri + c, tag | __builtin_bit_cast(uint32_t, mean), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(vst + ri + c, tag | __builtin_bit_cast(uint32_t, m2), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    float of[ONE ? NV : 1][V], hf[ONE ? NV : 1][V];
    if constexpr (ONE) {
#pragma unroll
      for (int k = 0; k < NV; ++k)
        if (64 * k + g < nvec) {
#pragma unroll
          for (int e = 0; e < V; ++e) {
            const uint32_t sw = sv[k].w[e / 2], hw = hv[k].w[e / 2];
            of[k][e] = round_f32(1.0f + ((e & 1) ? hi_f32(sw) : lo_f32(sw)));  // bf16(1 + scale)
            hf[k][e] = (e & 1) ? hi_f32(hw) : lo_f32(hw);
          }
        }
    }
    n = 0.0f;  // elements of lanes 8j .. 8j + 7: whole numbers, exact in any order
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int gi = 8 * j + i;
      n += (float)((nvec > gi ? (nvec - gi + kWave - 1) / kWave : 0) * V);
    }
    if (j != c) {
      // poll both words (each wave's 64 pairs are 512 contiguous bytes twice)
      const uint64_t deadline = (uint64_t)wall_clock64() + wait_ticks;
      uint64_t w0, w1;
      bool ok;
      while (true) {
        w0 = __hip_atomic_load(mst + ri + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w1 = __hip_atomic_load(vst + ri + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = (w0 & ~0xffffffffull) == tag && (w1 & ~0xffffffffull) == tag;
        if (ok || (uint64_t)wall_clock64() > deadline) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (ok) {
        mean = __builtin_bit_cast(float, (uint32_t)w0);
        m2 = __builtin_bit_cast(float, (uint32_t)w1);
      } else {
        coop_group_state(xg + t, sx_d, nvec, j, mean, m2);
      }
    }
    merge_level<1>(mean, m2, n, lane);  // the tree's levels 8, 16, 32: the row's state in every lane
    merge_level<2>(mean, m2, n, lane);
    merge_level<4>(mean, m2, n, lane);
    const float rstd = finalize_rstd(m2, Df, a.eps, pow2_inverse_f(Df));
    const int64_t r = (int64_t)b * a.S + t0 + t;
    if (c == 0 && j == 0) {
      if (a.mean_out) a.mean_out[r] = mean;
      if (a.rstd_out) a.rstd_out[r] = rstd;
    }
    uint16_t* orow = static_cast<uint16_t*>(a.out) + r * D;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = 64 * k + g;
      if (v < nvec) {
        uint32_t xs[4];
        if constexpr (ONE) {
#pragma unroll
          for (int i = 0; i < 4; ++i) xs[i] = buf[k].w[i];
        } else {
          const uint4 xw = tile[k][t][col];
          xs[0] = xw.x, xs[1] = xw.y, xs[2] = xw.z, xs[3] = xw.w;
        }
        Vec<V> ov;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float4 o, h;
          if constexpr (ONE) {
            o = make_float4(of[k][4 * q], of[k][4 * q + 1], of[k][4 * q + 2], of[k][4 * q + 3]);
            h = make_float4(hf[k][4 * q], hf[k][4 * q + 1], hf[k][4 * q + 2], hf[k][4 * q + 3]);
          } else {
            o = otab[NT == 1 ? 0 : k][j][q];
            h = htab[NT == 1 ? 0 : k][j][q];
          }
          const float n0 = (lo_f32(xs[2 * q]) - mean) * rstd;
          const float n1 = (hi_f32(xs[2 * q]) - mean) * rstd;
          const float n2 = (lo_f32(xs[2 * q + 1]) - mean) * rstd;
          const float n3 = (hi_f32(xs[2 * q + 1]) - mean) * rstd;
          ov.w[2 * q] = tail_pair<kTailChain>(n0, n1, o.x, o.y, h.x, h.y);
          ov.w[2 * q + 1] = tail_pair<kTailChain>(n2, n3, o.z, o.w, h.z, h.w);
        }
        store_vec_nt<V>(orow + V * v, ov);
      }
    }
  }
}

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

inline unsigned grid_for(int64_t R) {
  int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  return (unsigned)std::min(blocks, kMaxBlocks);
}

template <int V, int NV, bool GATHER, bool RMS, int TAIL>
int launch_rows(const LnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((ln_modulate_rows<V, NV, GATHER, RMS, TAIL>), dim3(grid_for(a.R)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// one row per block of 64 * W threads at a time: the hardware dispatcher
// hands a compute unit a new row as soon as one of its blocks finishes
template <int V, int NV, bool UNIF, bool GATHER, bool RMS, int TAIL>
int launch_mw(const LnArgs& a, int W, hipStream_t st) {
  const unsigned blocks = (unsigned)std::min<int64_t>(a.R, kMaxBlocks);
  hipLaunchKernelGGL((ln_modulate_mw<V, NV, UNIF, GATHER, RMS, TAIL>), dim3(blocks), dim3(W * kWave), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// blocks of TPB threads holding TPB / (64 W) rows of one sample, the
// sample's adaLN tables in LDS
template <int NV, bool UNIF, bool RMS, int TAIL, int TPB>
int launch_mwt(const LnArgs& a, int W, hipStream_t st) {
  const int64_t P = TPB / (W * kWave);
  const int64_t B = a.R / a.S;
  const int64_t bps = (a.S + P - 1) / P;
  const size_t lds = (size_t)a.D * 2 * sizeof(float);
  hipLaunchKernelGGL((ln_modulate_mwt<NV, UNIF, RMS, TAIL, TPB>), dim3((unsigned)(B * bps)), dim3(TPB), lds, st, a,
                     (int)bps, W);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// W waves per row (W = 2 .. 16): every lane holds at most 64 elements, NV
// vector steps of V.  Vector-aligned rows of up to 16384 elements share each
// sample's adaLN tables across the rows of a block (ln_modulate_mwt) when the
// blocks fill at least three quarters of the compute units: 16-wave blocks
// if they do (and leave no nearly empty last round), else 8-wave blocks of
// half as many rows if those fill one round, else one row per block.
// Measured, 16-wave blocks vs one row per block at D = 16384: 128 blocks
// 10.66 vs 9.07 us, 192 blocks 11.38 vs 11.61, 256 13.4 vs 14.8, 320 (a
// last round of 64) 21.5 vs 18.1, 384 22.6 vs 24.3, 512 26.3 vs 30.1;
// 8-wave blocks of 2 rows at 256 blocks 8.02 vs 8.93.
template <int V, bool GATHER, bool RMS, int TAIL>
int dispatch_mw(const LnArgs& a, int W, hipStream_t st) {
  constexpr int NV = 64 / V;
  const int64_t nvec = a.D / V;
  const bool unif = V == 8 && nvec == (int64_t)NV * W * kWave;
  if constexpr (V == 8 && !GATHER) {
    const int cus = cu_count();
    const int64_t B = a.R / a.S;
    const int64_t n = cus > 0 ? cus : 256;
    // P rows per block: enough blocks for three quarters of the compute units,
    // not too many for one launch, and (one block per compute unit at a time)
    // a last round at least half full when there is more than one
    auto fills = [&](int64_t P) {
      const int64_t blocks = B * ((a.S + P - 1) / P), rem = blocks % n;
      return a.S >= P && blocks < ((int64_t)1 << 22) && 4 * blocks >= 3 * n &&
             (blocks <= n || rem == 0 || 2 * rem >= n);
    };
    if (W <= 4 && fills(kMaxWaves / W))
      return unif ? launch_mwt<NV, true, RMS, TAIL, 1024>(a, W, st) : launch_mwt<NV, false, RMS, TAIL, 1024>(a, W, st);
    if (W <= 4 && fills(kMaxWaves / 2 / W) && B * ((a.S + kMaxWaves / 2 / W - 1) / (kMaxWaves / 2 / W)) <= n)
      return unif ? launch_mwt<NV, true, RMS, TAIL, 512>(a, W, st) : launch_mwt<NV, false, RMS, TAIL, 512>(a, W, st);
  }
  if constexpr (V == 8) {
    if (unif) return launch_mw<V, NV, true, GATHER, RMS, TAIL>(a, W, st);
  } else {
    // 8-byte vectors: rows just past a multiple of 64 W vectors per lane step
    // (D % 8 == 4) take an instantiation sized to their steps, which frees
    // the registers of the unused ones
    if (nvec <= (int64_t)10 * W * kWave) return launch_mw<V, 10, false, GATHER, RMS, TAIL>(a, W, st);
  }
  return launch_mw<V, NV, false, GATHER, RMS, TAIL>(a, W, st);
}

template <int V, int NV, bool UNIF, bool RMS, int TAIL, bool MANY = false>
int launch_tab(const LnArgs& a, hipStream_t st) {
  using Shape = TabShape<NV, UNIF, RMS, TAIL, MANY>;
  constexpr int kWpb = Shape::kWpb;
  // Shape::kBlocksPerCu blocks per compute unit in total, at least one row per
  // wave, and no more than a compute unit holds at once: the instantiations
  // for rows with a partial last step take more registers (4-6 steps of 8:
  // 100-122 VGPRs, 4 waves per SIMD where the launch is sized for 5; 7-8
  // steps: 134-150 VGPRs, 3 where it is sized for 4).  Measured, sized vs
  // capped: (1,5120,2240) 12.80 vs 10.97 us, (1,5120,1800) 10.44 vs 9.26,
  // (1,4096,4000) 16.09 vs 14.73, (1,8192,4000) 29.71 vs 28.13; RMSNorm
  // (1,4096,4000) 15.49 vs 13.36; FP8 (1,5120,2240) 14.23 vs 11.54.
  static std::atomic<int> held[64];
  const int h = resident_blocks_per_cu(held, ln_modulate_tab<V, NV, UNIF, RMS, TAIL, MANY>, kWpb * kWave,
                                       (size_t)2 * NV * kWave * V * sizeof(float));
  const int64_t bpc = h > 0 ? std::min<int64_t>(Shape::kBlocksPerCu, h) : Shape::kBlocksPerCu;
  const int64_t B = a.R / a.S;
  const int cus = cu_count();
  const int64_t n = cus > 0 ? cus : 256;
  const int64_t target = bpc * n;
  int64_t bpb = (target + B - 1) / B;
  bpb = std::max<int64_t>(1, std::min<int64_t>(bpb, (a.S + kWpb - 1) / kWpb));
  const int64_t blocks = B * bpb;
  if constexpr (kWpb > 4) {
    // 16-wave blocks of few rows would leave most compute units idle: the row
    // kernel (4 rows per block, the same lanes and merges, so the same bits)
    // spreads them wider.  Measured at D = 4096, tabled vs row kernel: 128 rows
    // 7.80 vs 5.47 us, 1024 rows 8.28 vs 6.34, 2048 rows 8.57 vs 8.50, 3072
    // rows 9.36 vs 12.16.
    if (2 * blocks < n) return launch_rows<V, 8, false, RMS, TAIL>(a, st);
    // more rows than one per wave: the prefetching shape (MANY above)
    if (a.R > (int64_t)kWpb * n) return launch_tab<V, NV, UNIF, RMS, TAIL, true>(a, st);
  }
  const size_t lds = (size_t)2 * a.D * sizeof(float);
  hipLaunchKernelGGL((ln_modulate_tab<V, NV, UNIF, RMS, TAIL, MANY>), dim3((unsigned)blocks), dim3(kWpb * kWave), lds,
                     st, a, (int)bpb);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <int NV, bool UNIF, bool RMS, int TAIL>
int launch_tr(const LnArgs& a, hipStream_t st) {
  const int64_t B = a.R / a.S;
  const int64_t tiles_per_sample = a.S / kTrTokens;
  const int64_t nvec = a.D / 8;
  const size_t lds = (size_t)nvec * (4 * sizeof(float4) + kTrTokens * sizeof(uint4));
  hipLaunchKernelGGL((ln_modulate_tr<NV, UNIF, RMS, TAIL>), dim3((unsigned)(B * tiles_per_sample)), dim3(512),
                     lds, st, a, (int)tiles_per_sample);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

constexpr int kTrMaxD = 4096;  // 96 KiB of LDS (tables + tile)

// One-shot grids stay under 2^32 work-items (a dispatch counts its grid in
// 32 bits): the tabled kernels take up to 1024 threads per sample, the
// 8-token tile kernel 512 per tile; larger launches go to the row kernels,
// whose grids are capped and walk the rows.
constexpr int64_t kMaxTabSamples = ((int64_t)1 << 22) - 1;
constexpr int64_t kMaxTrTiles = (int64_t)1 << 23;

template <bool RMS, int TAIL>
int dispatch_tr(const LnArgs& a, hipStream_t st) {
  const int64_t nvec = a.D / 8;
  const int64_t nv = (nvec + kWave - 1) / kWave;
  const bool unif = nvec % kWave == 0;
#define ADALN_TR_CASE(N) \
  if (nv == N) return unif ? launch_tr<N, true, RMS, TAIL>(a, st) : launch_tr<N, false, RMS, TAIL>(a, st);
  ADALN_TR_CASE(1)
  ADALN_TR_CASE(2)
  ADALN_TR_CASE(3)
  ADALN_TR_CASE(4)
  ADALN_TR_CASE(5)
  ADALN_TR_CASE(6)
  ADALN_TR_CASE(7)
  ADALN_TR_CASE(8)
#undef ADALN_TR_CASE
  return ADALN_ERR_TOO_LARGE;  // not reached: the caller bounds D
}

template <int V, bool RMS, int TAIL>
int dispatch_tab(const LnArgs& a, hipStream_t st) {
  const int64_t nvec = a.D / V;
  const int64_t nv = (nvec + kWave - 1) / kWave;
  const bool unif = nvec % kWave == 0;
#define ADALN_TAB_CASE(N)                                                           \
  if (nv == N)                                                                     \
    return unif ? launch_tab<V, N, true, RMS, TAIL>(a, st) : launch_tab<V, N, false, RMS, TAIL>(a, st);
  ADALN_TAB_CASE(1)
  ADALN_TAB_CASE(2)
  ADALN_TAB_CASE(3)
  ADALN_TAB_CASE(4)
  ADALN_TAB_CASE(5)
  ADALN_TAB_CASE(6)
  ADALN_TAB_CASE(7)
  ADALN_TAB_CASE(8)
  if constexpr (V == 4) {  // rows of up to 4096 elements: 16 steps of 4
    ADALN_TAB_CASE(9)
    ADALN_TAB_CASE(10)
    ADALN_TAB_CASE(11)
    ADALN_TAB_CASE(12)
    ADALN_TAB_CASE(13)
    ADALN_TAB_CASE(14)
    ADALN_TAB_CASE(15)
    ADALN_TAB_CASE(16)
  }
#undef ADALN_TAB_CASE
  return ADALN_ERR_TOO_LARGE;  // not reached: the caller bounds D
}

// vectors per lane -> the register-resident instantiation that covers it
// (one wave per row: at most 64 elements per lane)
template <int V, bool GATHER, bool RMS, int TAIL>
int dispatch(const LnArgs& a, hipStream_t st) {
  const int64_t nv = (a.D / V + kWave - 1) / kWave;
#define ADALN_NV_CASE(N) \
  if (nv <= N) return launch_rows<V, N, GATHER, RMS, TAIL>(a, st);
  ADALN_NV_CASE(1)
  ADALN_NV_CASE(2)
  ADALN_NV_CASE(3)
  ADALN_NV_CASE(4)
  ADALN_NV_CASE(5)
  ADALN_NV_CASE(6)
  ADALN_NV_CASE(8)
  if constexpr (V == 4) {
    ADALN_NV_CASE(10)
    ADALN_NV_CASE(12)
    ADALN_NV_CASE(16)
  }
#undef ADALN_NV_CASE
  return ADALN_ERR_TOO_LARGE;  // not reached: W == 1 rows hold at most 64 elements per lane
}

// whole 64-token groups of transposed storage, 16-byte runs, one wave per row
// (the kernel indexes tokens within a sample and blocks in 32 bits)
inline bool coop_shape_ok(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s, int64_t sx_d) {
  return sx_s == 1 && D % 8 == 0 && D <= kTrMaxD && S % kCoopTokens == 0 && S < INT32_MAX && sx_d % 8 == 0 &&
         (B <= 1 || sx_b % 8 == 0) && B * (S / kCoopTokens) * kCoopBlocks < INT32_MAX;
}

constexpr int kMaxDevices = 64;  // device ordinals with cached launch attributes

// How long a thread waits for another block's state before recomputing it
// from x itself: ADALN_WS_WAIT_US microseconds (default 200; 0 recomputes
// every state), in ticks of the device's constant-rate clock.
inline uint64_t coop_wait_ticks(int dev) {
  static std::atomic<int> rate_khz[kMaxDevices];
  int khz = dev >= 0 && dev < kMaxDevices ? rate_khz[dev].load(std::memory_order_relaxed) : 0;
  if (khz <= 0) {
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0) khz = 100000;
    if (dev >= 0 && dev < kMaxDevices) rate_khz[dev].store(khz, std::memory_order_relaxed);
  }
  long us = 200;
  const char* e = getenv("ADALN_WS_WAIT_US");
  if (e && *e) us = std::max(0L, std::min(strtol(e, nullptr, 10), 10000000L));
  return (uint64_t)us * (uint64_t)khz / 1000u;
}

// Blocks of ln_modulate_trc<NV, ONE> resident at once on the device (cached per
// device): the grid never exceeds it, so the 8 blocks of a slot run together.
template <int NV, bool ONE>
int coop_resident_blocks(int dev) {
  static std::atomic<int> cache[kMaxDevices];
  int v = dev >= 0 && dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (v > 0) return v;
  int per_cu = 0, cus = 0, cur = 0;
  // the occupancy query reads the current device: make it the stream's for the query
  if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess)) return 0;
  const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ln_modulate_trc<NV, ONE>, 512, 0) ==
                      hipSuccess &&
                  hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  if ((cur != dev && hipSetDevice(cur) != hipSuccess) || !ok) {
    (void)hipGetLastError();  // not left for the launch check that follows
    return 0;
  }
  v = per_cu * cus;
  if (dev >= 0 && dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// the device a stream belongs to (the current device for the null stream)
inline hipError_t stream_device(hipStream_t st, int* dev) {
  return st == nullptr ? hipGetDevice(dev) : hipStreamGetDevice(st, dev);
}

template <int NV>
int launch_trc(const LnArgs& a, void* ws, hipStream_t st) {
  int dev = 0;
  if (stream_device(st, &dev) != hipSuccess) return ADALN_ERR_HIP;
  const int64_t groups_per_sample = a.S / kCoopTokens;
  const int64_t ntg = (a.R / a.S) * groups_per_sample;
  // one block per group when the groups fit one pass of the register-heavy kernel (its
  // row and adaLN values fit the registers up to 5 vector steps, D <= 2560)
  if constexpr (NV <= 5) {
    const int64_t one_slots = coop_resident_blocks<NV, true>(dev) / kCoopBlocks;
    if (ntg <= one_slots) {
      hipLaunchKernelGGL((ln_modulate_trc<NV, true>), dim3((unsigned)(ntg * kCoopBlocks)), dim3(512), 0, st, a,
                         static_cast<char*>(ws), (int)groups_per_sample, (int)ntg, coop_wait_ticks(dev));
      return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
    }
  }
  const int64_t slots = coop_resident_blocks<NV, false>(dev) / kCoopBlocks;
  if (slots < 1) return ADALN_ERR_HIP;
  const unsigned grid = (unsigned)(std::min(ntg, slots) * kCoopBlocks);
  hipLaunchKernelGGL((ln_modulate_trc<NV, false>), dim3(grid), dim3(512), 0, st, a, static_cast<char*>(ws),
                     (int)groups_per_sample, (int)ntg,
                     coop_wait_ticks(dev));
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

int dispatch_trc(const LnArgs& a, void* ws, hipStream_t st) {
  const int64_t nv = (a.D / 8 + kWave - 1) / kWave;
  switch (nv) {
    case 1: return launch_trc<1>(a, ws, st);
    case 2: return launch_trc<2>(a, ws, st);
    case 3: return launch_trc<3>(a, ws, st);
    case 4: return launch_trc<4>(a, ws, st);
    case 5: return launch_trc<5>(a, ws, st);
    case 6: return launch_trc<6>(a, ws, st);
    case 7: return launch_trc<7>(a, ws, st);
    case 8: return launch_trc<8>(a, ws, st);
    default: return ADALN_ERR_TOO_LARGE;  // not reached: coop_shape_ok bounds D
  }
}

// ---------------------------------------------------------------------------
// The workspace of ln_modulate_noalloc: a fixed array of device memory, for
// callers that cannot allocate (each device the library runs on holds its
// own copy until the process ends; device globals start zero-filled, which
// is the state the hand-over protocol starts from, and every call leaves it
// ready for the next).  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels get the address hipGetSymbolAddress
// returns for the device, looked up once per device with it current.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchGroups = 1024;  // 65536 tokens of transposed storage
constexpr int64_t kScratchBytes = kScratchGroups * kCoopSlab;
static __device__ __align__(256) char scratch[kScratchBytes];

int scratch_address(hipStream_t st, void** out) {
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex lookup;
  int dev = 0;
  if (stream_device(st, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ADALN_ERR_HIP;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> hold(lookup);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      if (hipGetDevice(&cur) != hipSuccess) return ADALN_ERR_HIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return ADALN_ERR_HIP;
      void* q = nullptr;
      const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return ADALN_ERR_HIP;
      if (e != hipSuccess || q == nullptr) return ADALN_ERR_HIP;
      addr[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return ADALN_OK;
}

}  // namespace

// Shape/stride/dtype acceptance shared by the entry point and its predicate.
static int ln_modulate_check_shape(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                   int64_t sx_d, int64_t sscale_b, int64_t sshift_b, int dtype) {
  if (dtype != ADALN_BF16) return ADALN_ERR_DTYPE;
  if (B < 0 || S < 0 || D < 4 || D % 4 != 0) return ADALN_ERR_SHAPE;
  if (D > 65536) return ADALN_ERR_TOO_LARGE;
  if (sx_b < 0 || sx_s < 0 || sx_d < 0 || sscale_b < 0 || sshift_b < 0) return ADALN_ERR_STRIDE;
  int64_t R;
  if (!mul_ok(B, S, &R)) return ADALN_ERR_TOO_LARGE;
  int64_t RD;
  if (!mul_ok(R, D, &RD)) return ADALN_ERR_TOO_LARGE;
  if (!extent_ok({{B, sx_b}, {S, sx_s}, {D, sx_d}}) || !extent_ok({{B, sscale_b}, {D, 1}}) ||
      !extent_ok({{B, sshift_b}, {D, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

// The entry point of every norm + modulate variant: validation, aliasing
// rules, then the kernel family the layout selects (RMS: RMSNorm statistics,
// no mean; TAIL: the output stage, see kTailChain / kTailFold / kTailFp8).
template <bool RMS, int TAIL>
static int norm_modulate(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                         int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                         int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                         float* rstd_out, const float* qscale, void* stream, void* ws = nullptr,
                         int64_t ws_bytes = 0, bool lib_scratch = false) {
  constexpr bool kFp8 = TAIL == kTailFp8;
  int rc = ln_modulate_check_shape(B, S, D, sx_b, sx_s, sx_d, sscale_b, sshift_b, dtype);
  if (rc != ADALN_OK) return rc;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return ADALN_ERR_ARG;  // also rejects NaN
  const int64_t R = B * S;
  if (R == 0) return ADALN_OK;
  if (!x || !scale || !shift || !out || (kFp8 && !qscale)) return ADALN_ERR_NULL;
  adaln_order ord{};
  order_of(RMS ? ADALN_OP_RMSNORM_SCALE_SHIFT : ADALN_OP_LN_MODULATE, D, &ord);
  const int V = ord.V;
  if (!aligned(x, 2) || !aligned(scale, 2) || !aligned(shift, 2) || !aligned(out, kFp8 ? V : 2) ||
      !aligned(mean_out, 4) || !aligned(rstd_out, 4) || !aligned(qscale, 4))
    return ADALN_ERR_ALIGN;

  // overlap rules: a bf16 out may be exactly a contiguous x; nothing else may overlap
  const Span so = span_of(out, {{R * D, 1}}, kFp8 ? 1 : 2);
  const Span sx = span_of(x, {{B, sx_b}, {S, sx_s}, {D, sx_d}});
  const Span ssc = span_of(scale, {{B, sscale_b}, {D, 1}});
  const Span ssh = span_of(shift, {{B, sshift_b}, {D, 1}});
  const Span sq = qscale ? Span{(uintptr_t)qscale, (uintptr_t)(qscale + 1)} : Span{};
  const bool x_contig = sx_d == 1 && (S == 1 || sx_s == D) && (B == 1 || sx_b == S * D);
  if (overlaps(so, sx) && (kFp8 || !(x == out && x_contig))) return ADALN_ERR_ALIAS;
  if (overlaps(so, ssc) || overlaps(so, ssh) || overlaps(so, sq)) return ADALN_ERR_ALIAS;
  const Span sm = mean_out ? Span{(uintptr_t)mean_out, (uintptr_t)(mean_out + R)} : Span{};
  const Span sr = rstd_out ? Span{(uintptr_t)rstd_out, (uintptr_t)(rstd_out + R)} : Span{};
  for (const Span* t : {&so, &sx, &ssc, &ssh, &sq})
    if (overlaps(sm, *t) || overlaps(sr, *t)) return ADALN_ERR_ALIAS;
  if (overlaps(sm, sr)) return ADALN_ERR_ALIAS;
  if (ws_bytes < 0) return ADALN_ERR_ARG;
  if (ws) {
    if (!aligned(ws, 16)) return ADALN_ERR_ALIGN;
    const Span sw = Span{(uintptr_t)ws, (uintptr_t)ws + (uintptr_t)ws_bytes};
    for (const Span* t : {&so, &sx, &ssc, &ssh, &sq, &sm, &sr})
      if (overlaps(sw, *t)) return ADALN_ERR_ALIAS;
  }

  LnArgs a;
  a.x = (const uint16_t*)x;
  a.S = S;
  a.D = D;
  a.sx_b = sx_b;
  a.sx_s = sx_s;
  a.sx_d = sx_d;
  a.scale = (const uint16_t*)scale;
  a.ssc_b = sscale_b;
  a.shift = (const uint16_t*)shift;
  a.ssh_b = sshift_b;
  a.eps = eps;
  a.out = out;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.R = R;
  a.qscale = qscale;

  // vector loads need every row start of x, scale, shift and out on a 2V-byte
  // boundary (V bytes for an FP8 out)
  const uintptr_t vb = (uintptr_t)(2 * V);
  const uintptr_t ob = kFp8 ? (uintptr_t)V : vb;
  auto stride_ok = [&](int64_t n, int64_t st) { return n <= 1 || ((uintptr_t)st * 2u) % vb == 0; };
  const bool vec = sx_d == 1 && aligned(x, vb) && aligned(scale, vb) && aligned(shift, vb) &&
                   aligned(out, ob) && stride_ok(B, sx_b) && stride_ok(S, sx_s) &&
                   stride_ok(B, sscale_b) && stride_ok(B, sshift_b);
  hipStream_t st = (hipStream_t)stream;
  if (ord.W > 1) {  // rows of more than 4096 elements: W waves per row
    if (V == 8) return vec ? dispatch_mw<8, false, RMS, TAIL>(a, ord.W, st) : dispatch_mw<8, true, RMS, TAIL>(a, ord.W, st);
    return vec ? dispatch_mw<4, false, RMS, TAIL>(a, ord.W, st) : dispatch_mw<4, true, RMS, TAIL>(a, ord.W, st);
  }
  // the tabled fast path indexes rows, samples and offsets in 32 bits, and
  // launches a block of up to 1024 threads per sample
  const bool tab = vec && S <= INT32_MAX / 4 && B <= kMaxTabSamples;
  if (tab) return V == 8 ? dispatch_tab<8, RMS, TAIL>(a, st) : dispatch_tab<4, RMS, TAIL>(a, st);
  // transposed storage with a workspace (the caller's, or the library's
  // scratch): whole lines, 8 blocks per 64-token group
  if constexpr (!RMS && TAIL == kTailChain) {
    if ((ws || lib_scratch) && coop_shape_ok(B, S, D, sx_b, sx_s, sx_d) && aligned(x, 16) && aligned(scale, 16) &&
        aligned(shift, 16) && aligned(out, 16) && stride_ok(B, sscale_b) && stride_ok(B, sshift_b)) {
      const int64_t need = coop_ws_bytes(B * (S / kCoopTokens));
      if (lib_scratch) {
        if (need > kScratchBytes) return ADALN_ERR_TOO_LARGE;
        void* p = nullptr;
        rc = scratch_address(st, &p);
        return rc != ADALN_OK ? rc : dispatch_trc(a, p, st);
      }
      if (ws_bytes >= need) return dispatch_trc(a, ws, st);
    }
  }
  // transposed storage: whole 8-token tiles, each tile's 16-byte token runs aligned
  const bool tr = sx_s == 1 && V == 8 && D <= kTrMaxD && S % kTrTokens == 0 && S < INT32_MAX &&
                  B * (S / kTrTokens) < kMaxTrTiles && aligned(x, 16) && sx_d % 8 == 0 &&
                  (B == 1 || sx_b % 8 == 0) && aligned(scale, 16) && aligned(shift, 16) &&
                  aligned(out, kFp8 ? 8 : 16) && stride_ok(B, sscale_b) && stride_ok(B, sshift_b);
  if (tr) return dispatch_tr<RMS, TAIL>(a, st);
  if (V == 8) return vec ? dispatch<8, false, RMS, TAIL>(a, st) : dispatch<8, true, RMS, TAIL>(a, st);
  return vec ? dispatch<4, false, RMS, TAIL>(a, st) : dispatch<4, true, RMS, TAIL>(a, st);
}

}  // namespace adaln

using namespace adaln;

extern "C" int ln_modulate_can_use(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                   int64_t sx_d, int64_t sscale_b, int64_t sshift_b, int dtype) {
  return ln_modulate_check_shape(B, S, D, sx_b, sx_s, sx_d, sscale_b, sshift_b, dtype) == ADALN_OK;
}

extern "C" int ln_modulate(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b,
                           int64_t sx_s, int64_t sx_d, const void* scale, int64_t sscale_b,
                           const void* shift, int64_t sshift_b, float eps, int dtype, void* out,
                           float* mean_out, float* rstd_out, void* stream) {
  return norm_modulate<false, kTailChain>(x, B, S, D, sx_b, sx_s, sx_d, scale, sscale_b, shift, sshift_b,
                                          eps, dtype, out, mean_out, rstd_out, nullptr, stream);
}

extern "C" int64_t ln_modulate_workspace_size(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                              int64_t sx_d) {
  if (ln_modulate_check_shape(B, S, D, sx_b, sx_s, sx_d, 0, 0, ADALN_BF16) != ADALN_OK) return 0;
  if (B * S == 0 || !coop_shape_ok(B, S, D, sx_b, sx_s, sx_d)) return 0;
  return coop_ws_bytes(B * (S / kCoopTokens));
}

extern "C" int ln_modulate_ws(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                              int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                              int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                              float* rstd_out, void* workspace, int64_t workspace_bytes, void* stream) {
  return norm_modulate<false, kTailChain>(x, B, S, D, sx_b, sx_s, sx_d, scale, sscale_b, shift, sshift_b,
                                          eps, dtype, out, mean_out, rstd_out, nullptr, stream, workspace,
                                          workspace_bytes);
}

extern "C" int ln_modulate_noalloc(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                   int64_t sx_d, const void* scale, int64_t sscale_b, const void* shift,
                                   int64_t sshift_b, float eps, int dtype, void* out, float* mean_out,
                                   float* rstd_out, void* stream) {
  return norm_modulate<false, kTailChain>(x, B, S, D, sx_b, sx_s, sx_d, scale, sscale_b, shift, sshift_b,
                                          eps, dtype, out, mean_out, rstd_out, nullptr, stream, nullptr, 0, true);
}

extern "C" int rmsnorm_scale_shift_can_use(int64_t B, int64_t S, int64_t D, int64_t sx_b,
                                           int64_t sx_s, int64_t sx_d, int64_t sscale_b,
                                           int64_t sshift_b, int dtype) {
  return ln_modulate_check_shape(B, S, D, sx_b, sx_s, sx_d, sscale_b, sshift_b, dtype) == ADALN_OK;
}

extern "C" int rmsnorm_scale_shift(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b,
                                   int64_t sx_s, int64_t sx_d, const void* scale, int64_t sscale_b,
                                   const void* shift, int64_t sshift_b, float eps, int dtype,
                                   void* out, float* rinv_out, void* stream) {
  return norm_modulate<true, kTailChain>(x, B, S, D, sx_b, sx_s, sx_d, scale, sscale_b, shift, sshift_b, eps,
                                         dtype, out, nullptr, rinv_out, nullptr, stream);
}

extern "C" int ln_modulate_fold(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b,
                                int64_t sx_s, int64_t sx_d, const void* scale, int64_t sscale_b,
                                const void* shift, int64_t sshift_b, float eps, int dtype, void* out,
                                float* mean_out, float* rstd_out, void* stream) {
  return norm_modulate<false, kTailFold>(x, B, S, D, sx_b, sx_s, sx_d, scale, sscale_b, shift, sshift_b,
                                         eps, dtype, out, mean_out, rstd_out, nullptr, stream);
}

extern "C" int ln_modulate_fp8(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b,
                               int64_t sx_s, int64_t sx_d, const void* scale, int64_t sscale_b,
                               const void* shift, int64_t sshift_b, float eps, const float* qscale,
                               int dtype, void* out, float* mean_out, float* rstd_out, void* stream) {
  return norm_modulate<false, kTailFp8>(x, B, S, D, sx_b, sx_s, sx_d, scale, sscale_b, shift, sshift_b,
                                        eps, dtype, out, mean_out, rstd_out, qscale, stream);
}
