// ln_row.hpp -- the per-row LayerNorm + adaLN-modulate routine shared by the
// tabled kernels (ln_modulate and the residual-update-fused variant).
//
// One wave holds one row as NV packed bf16 vectors per lane (lane l owns
// vectors l, l + 64, ...); the per-sample adaLN rows sit in LDS as fp32
// tables.  Operation: prhub report on sglang PR #34015 (Sana fused adaLN),
// 关键源码片段 (layernorm_modulate.py pass 2); Welford step order: prhub report
// on sglang PR #34008, 关键源码片段 (_welford_push).
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "mw_row.hpp"

namespace adaln {
namespace {

template <int V, int K, int... E>
__device__ __forceinline__ void push_f32(const float* xk, float& mean, float& m2,
                                         std::integer_sequence<int, E...>) {
  (welford_push<K * V + E + 1>(mean, m2, xk[E]), ...);
}

template <int V, int... E>
__device__ __forceinline__ void sumsq_f32(const float* xk, float& ss, std::integer_sequence<int, E...>) {
  ((ss = __builtin_fmaf(xk[E], xk[E], ss)), ...);
}

// RMSNorm's per-lane sum of squares, same element order as the Welford pass
template <int V, bool UNIF, int... K>
__device__ __forceinline__ void sumsq_lane_f32(const float (*xf)[V], int nvec, int lane, float& ss,
                                               std::integer_sequence<int, K...>) {
  (
      [&] {
        if (UNIF || K * kWave + lane < nvec) sumsq_f32<V>(xf[K], ss, std::make_integer_sequence<int, V>{});
      }(),
      ...);
}

template <int V, bool UNIF, int... K>
__device__ __forceinline__ void welford_f32(const float (*xf)[V], int nvec, int lane, float& mean,
                                            float& m2, std::integer_sequence<int, K...>) {
  (
      [&] {
        if (UNIF || K * kWave + lane < nvec)
          push_f32<V, K>(xf[K], mean, m2, std::make_integer_sequence<int, V>{});
      }(),
      ...);
}

// The per-sample tables: bf16(1 + scale) and shift as fp32, float4-packed
// [table][V/4][nvec] so a lane's reads for vector v are contiguous across
// the wave.  Built cooperatively by the nthreads threads of a block.
// Returns whether every value this thread wrote is finite.
// Vector v of the tables from the sample's scale and shift vectors; returns
// whether the values written are finite.
template <int V>
__device__ __forceinline__ bool put_tables(float4* tab, const Vec<V>& sv, const Vec<V>& hv, int v, int nvec) {
  const int shift_off = (V / 4) * nvec;
  bool finite = true;
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    float o0 = 1.0f + lo_f32(sv.w[2 * q]), o1 = 1.0f + hi_f32(sv.w[2 * q]);
    float o2 = 1.0f + lo_f32(sv.w[2 * q + 1]), o3 = 1.0f + hi_f32(sv.w[2 * q + 1]);
    round_pair(o0, o1);  // bf16(1 + scale)
    round_pair(o2, o3);
    tab[q * nvec + v] = make_float4(o0, o1, o2, o3);
    const float h0 = lo_f32(hv.w[2 * q]), h1 = hi_f32(hv.w[2 * q]);
    const float h2 = lo_f32(hv.w[2 * q + 1]), h3 = hi_f32(hv.w[2 * q + 1]);
    tab[shift_off + q * nvec + v] = make_float4(h0, h1, h2, h3);
    finite = finite && __builtin_isfinite(o0) && __builtin_isfinite(o1) && __builtin_isfinite(o2) &&
             __builtin_isfinite(o3) && __builtin_isfinite(h0) && __builtin_isfinite(h1) &&
             __builtin_isfinite(h2) && __builtin_isfinite(h3);
  }
  return finite;
}

template <int V>
__device__ __forceinline__ bool build_tables(float4* tab, const uint16_t* sc, const uint16_t* sh,
                                             int nvec, int tid, int nthreads) {
  bool finite = true;
  for (int v = tid; v < nvec; v += nthreads) {
    const Vec<V> sv = load_vec<V>(sc + v * V);
    const Vec<V> hv = load_vec<V>(sh + v * V);
    finite = put_tables<V>(tab, sv, hv, v, nvec) && finite;
  }
  return finite;
}

// Third table of the residual-update-fused kernel: the per-sample gate as
// fp32, same [V/4][nvec] float4 layout, after the two tables above.
template <int V>
__device__ __forceinline__ void build_gate_table(float4* tab, const uint16_t* gt, int nvec, int tid,
                                                 int nthreads) {
  const int gate_off = 2 * (V / 4) * nvec;
  for (int v = tid; v < nvec; v += nthreads) {
    const Vec<V> gv = load_vec<V>(gt + v * V);
#pragma unroll
    for (int q = 0; q < V / 4; ++q)
      tab[gate_off + q * nvec + v] = make_float4(lo_f32(gv.w[2 * q]), hi_f32(gv.w[2 * q]),
                                                 lo_f32(gv.w[2 * q + 1]), hi_f32(gv.w[2 * q + 1]));
  }
}

// One row, held by one wave as NV packed vectors per lane (lane l owns
// vectors l, l + 64, ...): statistics (Welford for LayerNorm, the sum of
// squares for RMSNorm), merge tree, then normalize, modulate with the LDS
// tables and store (non-temporal).  LayerNorm normalizes (x - mean) * rstd,
// RMSNorm x * rinv with rinv = 1/sqrt(mean(x^2) + eps) (written to
// rstd_out; mean_out is unused).
// kXf32: widen the row once and keep it in fp32 for both passes; otherwise
// widen it for the reduction and again (opaque to the compiler, so no fp32
// copy stays live) when normalizing.  TAIL selects the output stage
// (kTailChain, kTailFold: bf16 row at orow; kTailFp8: E4M3 bytes at orow,
// scaled by qinv).
template <int V, int NV, bool UNIF, bool kXf32, bool RMS = false, int TAIL = kTailChain>
__device__ __forceinline__ void normalize_row(const Vec<V>* buf, const float4* tab, int nvec, int lane,
                                              float Df, float eps, void* orow, float* mean_out,
                                              float* rstd_out, float qinv = 1.0f, bool tab_finite = false) {
  const int shift_off = (V / 4) * nvec;
  float xf[NV][V];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int i = 0; i < V / 2; ++i) {
      xf[k][2 * i] = lo_f32(buf[k].w[i]);
      xf[k][2 * i + 1] = hi_f32(buf[k].w[i]);
    }
  auto xval = [&](int k, int e) -> float {
    if constexpr (kXf32) return xf[k][e];
    return (e & 1) ? hi_f32_again(buf[k].w[e / 2]) : lo_f32_again(buf[k].w[e / 2]);
  };
  float mean = 0.0f, m2 = 0.0f;
  if constexpr (RMS) {
    sumsq_lane_f32<V, UNIF>(xf, nvec, lane, m2, std::make_integer_sequence<int, NV>{});
    sum_down<1>(m2);
    sum_down<2>(m2);
    sum_down<4>(m2);
    sum_down<8>(m2);
    sum_down<16>(m2);
    sum_down<32>(m2);
  } else if constexpr (UNIF) {
    welford_f32<V, UNIF>(xf, nvec, lane, mean, m2, std::make_integer_sequence<int, NV>{});
    const float c = (float)(NV * V);
    merge_down_equal<1>(mean, m2, c);
    merge_down_equal<2>(mean, m2, c);
    merge_down_equal<4>(mean, m2, c);
    merge_down_equal<8>(mean, m2, c);
    merge_down_equal<16>(mean, m2, c);
    merge_down_equal<32>(mean, m2, c);
  } else {
    welford_f32<V, UNIF>(xf, nvec, lane, mean, m2, std::make_integer_sequence<int, NV>{});
    float n = (float)((nvec / kWave + (lane < nvec % kWave ? 1 : 0)) * V);
    merge_down<1>(mean, m2, n);
    merge_down<2>(mean, m2, n);
    merge_down<4>(mean, m2, n);
    merge_down<8>(mean, m2, n);
    merge_down<16>(mean, m2, n);
    merge_down<32>(mean, m2, n);
  }
  if constexpr (!RMS) mean = bcast_lane0(mean);
  m2 = bcast_lane0(m2);
  const float rstd = finalize_rstd(m2, Df, eps, pow2_inverse_f(Df));
  if (lane == 0) {
    if (!RMS && mean_out) *mean_out = mean;
    if (rstd_out) *rstd_out = rstd;
  }
  __builtin_amdgcn_sched_barrier(0);
  // table values for step k are read one step ahead of their use
  float4 ot[V / 4], ht[V / 4];
  auto read_tab = [&](int k) {
    const int v = k * kWave + lane;
    const int vc = (UNIF || v < nvec) ? v : nvec - 1;
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      ot[q] = tab[q * nvec + vc];
      ht[q] = tab[shift_off + q * nvec + vc];
    }
  };
  // NO_NAN (FP8 only) is decided once per row, so the vector loop has no
  // branch that would split its schedule
  auto steps = [&](auto no_nan_c) {
    constexpr bool NO_NAN = decltype(no_nan_c)::value;
    // Table values are read one step ahead, except where the registers that
    // takes cost waves: the FP8 stage over rows of 7-8 steps with an fp32
    // copy of x (the look-ahead would push it past the 128 VGPRs of a
    // 16-wave block, 44 bytes of spill); rows of 7-8 steps with a partial
    // last step (102-112 VGPRs instead of 138-150: 4 waves per SIMD, as the
    // launch asks, instead of 3; (1,4096,3840) 14.24 vs 13.38 us, RMSNorm
    // 12.85 vs 11.01); RMSNorm over rows of 4-6 steps with a partial last
    // step (78-88 VGPRs instead of 96-118, 5 waves per SIMD: (1,5120,2240)
    // 9.55 vs 8.51 us; the LayerNorm chain there gains too but loses 2.3 %
    // at (2,1024,2240), and keeps the look-ahead).
    constexpr bool kAhead = !(TAIL == kTailFp8 && kXf32 && NV >= 7) && !(RMS && !UNIF && NV >= 4 && NV <= 6) &&
                            !(TAIL == kTailChain && !UNIF && NV >= 7);
    if constexpr (kAhead) read_tab(0);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if constexpr (!kAhead) read_tab(k);
      float4 oc[V / 4], hc[V / 4];
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        oc[q] = ot[q];
        hc[q] = ht[q];
      }
      if constexpr (kAhead)
        if (k + 1 < NV) read_tab(k + 1);
      const int v = k * kWave + lane;
      if (UNIF || v < nvec) {
        uint32_t o[V / 2];  // bf16 pairs
        float y8[TAIL == kTailFp8 ? V : 1];  // FP8: the chain's output as fp32 values
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
          float n0, n1, n2, n3;
          if constexpr (RMS) {
            n0 = xval(k, 4 * q) * rstd;
            n1 = xval(k, 4 * q + 1) * rstd;
            n2 = xval(k, 4 * q + 2) * rstd;
            n3 = xval(k, 4 * q + 3) * rstd;
          } else {
            n0 = (xval(k, 4 * q) - mean) * rstd;
            n1 = (xval(k, 4 * q + 1) - mean) * rstd;
            n2 = (xval(k, 4 * q + 2) - mean) * rstd;
            n3 = (xval(k, 4 * q + 3) - mean) * rstd;
          }
          // n = rstd * (x - mean), or x * rinv; then the output stage
          if constexpr (TAIL == kTailFp8) {
            y8[4 * q] = chain_f32(n0, oc[q].x, hc[q].x);
            y8[4 * q + 1] = chain_f32(n1, oc[q].y, hc[q].y);
            y8[4 * q + 2] = chain_f32(n2, oc[q].z, hc[q].z);
            y8[4 * q + 3] = chain_f32(n3, oc[q].w, hc[q].w);
          } else {
            o[2 * q] = tail_pair<TAIL>(n0, n1, oc[q].x, oc[q].y, hc[q].x, hc[q].y);
            o[2 * q + 1] = tail_pair<TAIL>(n2, n3, oc[q].z, oc[q].w, hc[q].z, hc[q].w);
          }
        }
        if constexpr (TAIL == kTailFp8) {
          uint32_t q8[V / 4];
          fp8_stage_f32<V>(y8, qinv, NO_NAN, q8);
          store_fp8_nt<V>(static_cast<uint8_t*>(orow) + v * V, q8);
        } else {
          Vec<V> ov;
#pragma unroll
          for (int i = 0; i < V / 2; ++i) ov.w[i] = o[i];
          store_vec_nt<V>(static_cast<uint16_t*>(orow) + v * V, ov);
        }
      }
      // keep two steps' table values live at a time (the scheduler would
      // otherwise hoist every LDS read and halve the occupancy)
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if constexpr (TAIL == kTailFp8) {
    // FP8: with a finite mean, a finite non-zero rstd (so m2 is finite and
    // no x - mean overflows), finite adaLN rows and a finite 1/qscale no
    // output can be NaN (an overflow to infinity still clamps to +-448).  A
    // row whose m2 overflows has rstd = 0 while x - mean may be infinite:
    // inf * 0 is NaN, which the NaN-preserving clamp keeps.
    const bool no_nan = tab_finite && __builtin_isfinite(mean) && __builtin_isfinite(rstd) && rstd > 0.0f &&
                        __builtin_isfinite(qinv);
    if (no_nan)
      steps(std::true_type{});
    else
      steps(std::false_type{});
  } else {
    steps(std::false_type{});
  }
}

}  // namespace
}  // namespace adaln
