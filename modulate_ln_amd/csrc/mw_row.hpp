// mw_row.hpp -- rows held by the W waves of one block (W = 1, 2, 4, 8, 16).
//
// A row of D elements is cut into vectors of V consecutive elements; with
// L = 64 * W lanes, lane g (lane l of wave w: g = 64 w + l) owns vectors
// g, g + L, g + 2L, ... -- at most 64 elements, so the whole row stays in
// registers and is read from memory once, whatever D up to 65536.
//
// Statistics, in the fixed order the library reports (adaln_order_for):
//  * each lane pushes its elements into its own fp32 Welford state in
//    increasing position (prhub report on sglang PR #34008, 关键源码片段,
//    _welford_push: delta = x - mean; mean += delta * (1/n); m2 += delta *
//    (x - mean)), 1/n the correctly rounded reciprocal of a compile-time
//    count; RMSNorm accumulates fma(x, x, ss) instead;
//  * lane states are merged pairwise at offsets 1, 2, ..., 32 toward lane 0
//    of each wave (DPP / permlane exchanges, lower lane first), then across
//    the waves at wave offsets 1, 2, 4, 8 -- lane offsets 64 .. 512 of the
//    same tree -- through LDS: lane 0 of wave w stores its state in slot w,
//    and after the barrier lane w of every wave takes slot w and runs the
//    same tree over lanes 0..15 (lanes >= W hold the empty state, which the
//    guarded merge leaves out, so every wave computes the row's state with
//    identical bits);
//  * var = m2 / D, rstd = 1 / sqrt(var + eps), IEEE division and square root.
// The tail (normalize, modulate, round at every eager op boundary, store)
// follows the prhub report on sglang PR #34015, 关键源码片段
// (layernorm_modulate.py pass 2).
#pragma once

#include <utility>

#include "device_common.hpp"

namespace adaln {
namespace {

template <int V, int E>
__device__ __forceinline__ float elem(const Vec<V>& v) {
  return (E & 1) ? hi_f32(v.w[E / 2]) : lo_f32(v.w[E / 2]);
}

// push the V elements of the lane's K-th vector; counts K*V+1 .. K*V+V
template <int V, int K, int... E>
__device__ __forceinline__ void push_vec(const Vec<V>& v, float& mean, float& m2,
                                         std::integer_sequence<int, E...>) {
  (welford_push<K * V + E + 1>(mean, m2, elem<V, E>(v)), ...);
}

// RMSNorm: the lane's sum of squares, same element order as push_vec
template <int V, int... E>
__device__ __forceinline__ void sumsq_vec(const Vec<V>& v, float& ss, std::integer_sequence<int, E...>) {
  ((ss = __builtin_fmaf(elem<V, E>(v), elem<V, E>(v), ss)), ...);
}

// The lane's statistic over its vectors g, g + L, ... (those below nvec).
template <int V, bool RMS, int... K>
__device__ __forceinline__ void lane_stats(const Vec<V>* buf, int nvec, int g, int L, float& mean, float& m2,
                                           std::integer_sequence<int, K...>) {
  (
      [&] {
        if (K * L + g < nvec) {
          if constexpr (RMS)
            sumsq_vec<V>(buf[K], m2, std::make_integer_sequence<int, V>{});
          else
            push_vec<V, K>(buf[K], mean, m2, std::make_integer_sequence<int, V>{});
        }
      }(),
      ...);
}

// bf16 -> fp32 widening the compiler may not merge with an earlier one of
// the same word: widening a row again from its packed form costs one VALU
// op per element but spares the VGPRs an fp32 copy of the row would hold.
__device__ __forceinline__ float lo_f32_again(uint32_t w) {
  uint32_t r;
  asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(w));
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ float hi_f32_again(uint32_t w) {
  uint32_t r;
  asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(r) : "v"(w));
  return __builtin_bit_cast(float, r);
}

// the per-element tail for one vector (RMS: x * rinv, no mean): V/2 bf16
// pairs (the chain's output also for the FP8 tail, quantized by put_vec).
// AGAIN: widen x again rather than reuse the statistics pass's fp32 values.
template <int V, bool RMS, int TAIL, bool AGAIN = false>
__device__ __forceinline__ void modulate_vec(const Vec<V>& xv, const Vec<V>& sv, const Vec<V>& hv, float mean,
                                             float rstd, uint32_t* o) {
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    const float x0 = AGAIN ? lo_f32_again(xv.w[i]) : lo_f32(xv.w[i]);
    const float x1 = AGAIN ? hi_f32_again(xv.w[i]) : hi_f32(xv.w[i]);
    const float n0 = RMS ? x0 * rstd : (x0 - mean) * rstd;
    const float n1 = RMS ? x1 * rstd : (x1 - mean) * rstd;
    float p0 = 1.0f + lo_f32(sv.w[i]);
    float p1 = 1.0f + hi_f32(sv.w[i]);
    round_pair(p0, p1);  // bf16(1 + scale)
    o[i] = tail_pair<TAIL>(n0, n1, p0, p1, lo_f32(hv.w[i]), hi_f32(hv.w[i]));
  }
}

// store one vector's output at element v*V of row orow (bf16 rows may be
// misaligned under GATHER; FP8 rows are V-byte aligned)
template <int V, bool GATHER, int TAIL>
__device__ __forceinline__ void put_vec(void* orow, int64_t v, const uint32_t* o, float qinv) {
  if constexpr (TAIL == kTailFp8) {
    uint32_t q8[V / 4];
    fp8_stage<V>(o, qinv, false, q8);
    store_fp8_nt<V>(static_cast<uint8_t*>(orow) + v * V, q8);
  } else {
    Vec<V> ov;
#pragma unroll
    for (int i = 0; i < V / 2; ++i) ov.w[i] = o[i];
    if constexpr (GATHER)
      scatter_vec<V>(static_cast<uint16_t*>(orow) + v * V, ov);
    else
      store_vec_nt<V>(static_cast<uint16_t*>(orow) + v * V, ov);
  }
}

// Largest number of waves per row (rows of up to 64 * 16 * 64 = 65536
// elements), and the LDS the cross-wave exchange uses: two sets of slots,
// alternating from row to row, so one barrier per row suffices (a slot set
// is rewritten two rows later, after every wave has passed the barrier of
// the row in between, which follows its reads of that set).
constexpr int kMaxWaves = 16;
struct MwSlots {
  float4 s[2][kMaxWaves];
};

// The row's (mean, m2) -- or RMSNorm's sum of squares in m2 -- in every lane
// of every wave of the block, for the row held in buf (NV vector steps per
// lane, vectors g + k*L).  UNIF: every lane holds NV full vectors (nvec ==
// NV * L), so the in-wave merges have equal halves and need no division.
// Must be reached by every thread of the block (it contains a barrier).
template <int V, int NV, bool UNIF, bool RMS>
__device__ __forceinline__ void mw_stats(const Vec<V>* buf, int nvec, int g, int lane, int wave, int W,
                                         float4* slots, float& mean, float& m2) {
  const int L = W * kWave;
  mean = 0.0f;
  m2 = 0.0f;
  lane_stats<V, RMS>(buf, nvec, g, L, mean, m2, std::make_integer_sequence<int, NV>{});
  float n = 0.0f;
  if constexpr (RMS) {
    sum_down<1>(m2);
    sum_down<2>(m2);
    sum_down<4>(m2);
    sum_down<8>(m2);
    sum_down<16>(m2);
    sum_down<32>(m2);
  } else if constexpr (UNIF) {
    const float c = (float)(NV * V);
    merge_down_equal<1>(mean, m2, c);
    merge_down_equal<2>(mean, m2, c);
    merge_down_equal<4>(mean, m2, c);
    merge_down_equal<8>(mean, m2, c);
    merge_down_equal<16>(mean, m2, c);
    merge_down_equal<32>(mean, m2, c);
    n = c * (float)kWave;
  } else {
    const int steps = (nvec > g) ? (nvec - g + L - 1) / L : 0;
    n = (float)(steps * V);
    merge_down<1>(mean, m2, n);
    merge_down<2>(mean, m2, n);
    merge_down<4>(mean, m2, n);
    merge_down<8>(mean, m2, n);
    merge_down<16>(mean, m2, n);
    merge_down<32>(mean, m2, n);
  }
  if (W > 1) {
    if (lane == 0) slots[wave] = make_float4(mean, m2, n, 0.0f);
    __syncthreads();
    const float4 t = lane < W ? slots[lane] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    mean = t.x;
    m2 = t.y;
    n = t.z;
    if constexpr (RMS) {
      sum_down<1>(m2);
      sum_down<2>(m2);
      sum_down<4>(m2);
      sum_down<8>(m2);
    } else {
      merge_down<1>(mean, m2, n);
      merge_down<2>(mean, m2, n);
      merge_down<4>(mean, m2, n);
      merge_down<8>(mean, m2, n);
    }
  }
  if constexpr (!RMS) mean = bcast_lane0(mean);
  m2 = bcast_lane0(m2);
}

}  // namespace
}  // namespace adaln
