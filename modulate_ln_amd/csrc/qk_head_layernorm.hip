// qk_head_layernorm: per-head affine LayerNorm of q and k in one launch.
//
// Operation: "Fused Kernels" page, table "Normalization" (qk_head_layernorm:
// per-head LayerNorm on q/k, bit-exact); prhub report on sglang PR #34008,
// 实现拆解 §1 (fused_qk_head_layernorm) and §3 (called when attention has
// both q and k).  The affine LayerNorm is one eager op, so the output is
// rounded to bf16 once: out = bf16(fma(w, (x - mean) * rstd, b)).
//
// qk_rmsnorm ("Fused Kernels" page, table "Normalization": qk_rmsnorm_native,
// per-head QK RMSNorm, bit-exact) is the same kernel family with RMSNorm
// statistics: out = bf16((x * rinv) * w), each product rounded to fp32 --
// torch's rms_norm is one op, computed in fp32 and rounded once.
//
// Design: a head row (Dh <= 256) is small, so 16 lanes -- one DPP row --
// own a head and a wave normalizes four heads at once.  Lane l of the group
// owns vectors l, l+16, ... (16-byte loads for V = 8); the merge tree is the
// four in-row levels 1, 2, 4, 8 (DPP quad permutes, ds_swizzle, row rotate),
// so no LDS and no cross-row traffic.  Vector-aligned inputs take qk_heads:
// grid row 0 normalizes q, grid row 1 k; each lane keeps its slice of that
// side's weight and bias in fp32 VGPRs for the whole launch, and each
// 16-lane group loads HP heads (non-temporal, unguarded) before reducing
// them, so several heads per lane are in flight.
#include <utility>

#include "device_common.hpp"
#include "host_common.hpp"

namespace adaln {
namespace {

constexpr int kGroup = 16;                  // lanes per head
constexpr int kGroupsPerBlock = 256 / kGroup;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

struct QkSide {
  const uint16_t* x;
  int64_t s_b, s_s, s_h;
  const uint16_t* w;
  const uint16_t* bias;
  uint16_t* out;
};

struct QkArgs {
  QkSide side[2];  // q, k
  int64_t S, H, Dh;
  int64_t Rq;  // head rows per side (B*S*H)
  float eps;
};

template <int V, int E>
__device__ __forceinline__ float elem(const Vec<V>& v) {
  return (E & 1) ? hi_f32(v.w[E / 2]) : lo_f32(v.w[E / 2]);
}

template <int V, int K, int... E>
__device__ __forceinline__ void push_vec(const Vec<V>& v, float& mean, float& m2,
                                         std::integer_sequence<int, E...>) {
  (welford_push<K * V + E + 1>(mean, m2, elem<V, E>(v)), ...);
}

template <int V, int... K>
__device__ __forceinline__ void welford_lane(const Vec<V>* buf, int64_t nvec, int l16, float& mean,
                                             float& m2, std::integer_sequence<int, K...>) {
  (
      [&] {
        if ((int64_t)K * kGroup + l16 < nvec)
          push_vec<V, K>(buf[K], mean, m2, std::make_integer_sequence<int, V>{});
      }(),
      ...);
}

// RMSNorm: the lane's sum of squares, same element order as welford_lane
template <int V, int K, int... E>
__device__ __forceinline__ void sumsq_vec(const Vec<V>& v, float& ss, std::integer_sequence<int, E...>) {
  ((ss = __builtin_fmaf(elem<V, E>(v), elem<V, E>(v), ss)), ...);
}

template <int V, int... K>
__device__ __forceinline__ void sumsq_lane(const Vec<V>* buf, int64_t nvec, int l16, float& ss,
                                           std::integer_sequence<int, K...>) {
  (
      [&] {
        if ((int64_t)K * kGroup + l16 < nvec) sumsq_vec<V, K>(buf[K], ss, std::make_integer_sequence<int, V>{});
      }(),
      ...);
}

// UNIFORM: head rows of a side sit at a constant stride s_h (q viewed as
// [B*S*H, Dh]); otherwise the row index is decomposed into (b, s, h).
// RMS: RMSNorm statistics (sum of squares), x * rinv, weight only.
template <bool RMS, int V, int NV, bool UNIFORM, bool AFFINE, bool GATHER>
__global__ __launch_bounds__(256) void qk_rows(QkArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int l16 = lane & (kGroup - 1);
  const int64_t nvec = a.Dh / V;
  const float Df = (float)a.Dh;
  const float invD = pow2_inverse(a.Dh);
  const int64_t nv_lane = nvec > l16 ? (nvec - l16 + kGroup - 1) / kGroup : 0;
  const int64_t total = 2 * a.Rq;
  for (int64_t h = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4); h < total;
       h += (int64_t)gridDim.x * kGroupsPerBlock) {
    const int which = h >= a.Rq ? 1 : 0;
    const int64_t rr = h - which * a.Rq;
    const QkSide& sd = a.side[which];
    const uint16_t* xr;
    if constexpr (UNIFORM) {
      xr = sd.x + rr * sd.s_h;
    } else {
      const int64_t hh = rr % a.H;
      const int64_t t = rr / a.H;
      const int64_t s = t % a.S;
      const int64_t b = t / a.S;
      xr = sd.x + b * sd.s_b + s * sd.s_s + hh * sd.s_h;
    }

    Vec<V> buf[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kGroup + l16;
      if (v < nvec) buf[k] = GATHER ? gather_vec<V>(xr + v * V, 1) : load_vec<V>(xr + v * V);
    }

    float mean = 0.0f, m2 = 0.0f;
    if constexpr (RMS) {
      sumsq_lane<V>(buf, nvec, l16, m2, std::make_integer_sequence<int, NV>{});
      sum_lanes<kGroup>(m2);
    } else {
      welford_lane<V>(buf, nvec, l16, mean, m2, std::make_integer_sequence<int, NV>{});
      float n = (float)(nv_lane * V);
      merge_lanes<kGroup>(mean, m2, n, lane);
    }
    const float rstd = finalize_rstd(m2, Df, a.eps, invD);

    uint16_t* orow = sd.out + rr * a.Dh;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kGroup + l16;
      if (v < nvec) {
        Vec<V> o;
        Vec<V> wv, bv;
        if constexpr (AFFINE) {
          wv = GATHER ? gather_vec<V>(sd.w + v * V, 1) : load_vec<V>(sd.w + v * V);
          if constexpr (!RMS)
            bv = GATHER ? gather_vec<V>(sd.bias + v * V, 1) : load_vec<V>(sd.bias + v * V);
        }
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
          float y0 = RMS ? lo_f32(buf[k].w[i]) * rstd : (lo_f32(buf[k].w[i]) - mean) * rstd;
          float y1 = RMS ? hi_f32(buf[k].w[i]) * rstd : (hi_f32(buf[k].w[i]) - mean) * rstd;
          if constexpr (AFFINE && RMS) {
            y0 = y0 * lo_f32(wv.w[i]);
            y1 = y1 * hi_f32(wv.w[i]);
          } else if constexpr (AFFINE) {
            y0 = __builtin_fmaf(lo_f32(wv.w[i]), y0, lo_f32(bv.w[i]));
            y1 = __builtin_fmaf(hi_f32(wv.w[i]), y1, hi_f32(bv.w[i]));
          }
          o.w[i] = pack_bf16(y0, y1);
        }
        if constexpr (GATHER)
          scatter_vec<V>(orow + v * V, o);
        else
          store_vec<V>(orow + v * V, o);
      }
    }
  }
}

// Fast path: vector-aligned q/k.  HP heads per group per iteration.
template <bool RMS, int V, int NV, int HP, bool UNIFORM, bool AFFINE, bool EQ>
__global__ __launch_bounds__(256) void qk_heads(QkArgs a) {
  const QkSide& sd = a.side[blockIdx.y];
  const int lane = threadIdx.x & (kWave - 1);
  const int l16 = lane & (kGroup - 1);
  const int group = threadIdx.x >> 4;
  const int nvec = (int)(a.Dh / V);
  const float Df = (float)a.Dh;
  const float invD = pow2_inverse(a.Dh);
  const int nv_lane = nvec / kGroup + (l16 < nvec % kGroup ? 1 : 0);
  int off[NV];  // element offset of the lane's k-th vector within a head (clamped)
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = k * kGroup + l16;
    off[k] = (EQ || v < nvec ? v : nvec - 1) * V;
  }
  float wf[NV][V], bf[NV][V];
  if constexpr (AFFINE) {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const Vec<V> wv = load_vec<V>(sd.w + off[k]);
#pragma unroll
      for (int i = 0; i < V / 2; ++i) {
        wf[k][2 * i] = lo_f32(wv.w[i]);
        wf[k][2 * i + 1] = hi_f32(wv.w[i]);
      }
      if constexpr (!RMS) {
        const Vec<V> bv = load_vec<V>(sd.bias + off[k]);
#pragma unroll
        for (int i = 0; i < V / 2; ++i) {
          bf[k][2 * i] = lo_f32(bv.w[i]);
          bf[k][2 * i + 1] = hi_f32(bv.w[i]);
        }
      }
    }
  }
  const int64_t step = (int64_t)gridDim.x * kGroupsPerBlock * HP;
  auto load = [&](Vec<V> (*buf)[NV], int64_t h0) {
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      const int64_t rr = h0 + i < a.Rq ? h0 + i : a.Rq - 1;
      const uint16_t* xr;
      if constexpr (UNIFORM) {
        xr = sd.x + rr * sd.s_h;
      } else {
        const int64_t hh = rr % a.H;
        const int64_t t = rr / a.H;
        xr = sd.x + (t / a.S) * sd.s_b + (t % a.S) * sd.s_s + hh * sd.s_h;
      }
#pragma unroll
      for (int k = 0; k < NV; ++k) buf[i][k] = load_vec_nt<V>(xr + off[k]);
    }
  };
  auto process = [&](const Vec<V> (*buf)[NV], int64_t h0) {
    // statistics of the HP heads: after the tree toward lane 0, lane 0 of
    // each 16-lane group holds its head's (mean, m2)
    float mean[HP], m2[HP];
#pragma unroll
    for (int i = 0; i < HP; ++i) {
      mean[i] = 0.0f;
      m2[i] = 0.0f;
      if constexpr (RMS) {
        sumsq_lane<V>(buf[i], EQ ? (int64_t)NV * kGroup : (int64_t)nvec, l16, m2[i],
                      std::make_integer_sequence<int, NV>{});
        sum_down<1>(m2[i]);
        sum_down<2>(m2[i]);
        sum_down<4>(m2[i]);
        sum_down<8>(m2[i]);
      } else if constexpr (EQ) {
        welford_lane<V>(buf[i], (int64_t)NV * kGroup, l16, mean[i], m2[i], std::make_integer_sequence<int, NV>{});
        const float c = (float)(NV * V);
        merge_down_equal<1>(mean[i], m2[i], c);
        merge_down_equal<2>(mean[i], m2[i], c);
        merge_down_equal<4>(mean[i], m2[i], c);
        merge_down_equal<8>(mean[i], m2[i], c);
      } else {
        welford_lane<V>(buf[i], (int64_t)nvec, l16, mean[i], m2[i], std::make_integer_sequence<int, NV>{});
        float n = (float)(nv_lane * V);
        merge_down<1>(mean[i], m2[i], n);
        merge_down<2>(mean[i], m2[i], n);
        merge_down<4>(mean[i], m2[i], n);
        merge_down<8>(mean[i], m2[i], n);
      }
    }
    // one finalize for all HP heads: head i's m2 moves to lane 4i of the
    // group (DPP row shift written to bank i only), every lane finalizes,
    // and head i's rstd is broadcast back from lane 4i
    float g = m2[0];
    static_for<HP>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i > 0) g = row_shr_bank<4 * i, 1 << i>(g, m2[i]);
    });
    const float rstd_all = finalize_rstd(g, Df, a.eps, invD);
    static_for<HP>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const float rstd = row_bcast<4 * i>(rstd_all);
      const float mu = RMS ? 0.0f : row_bcast<0>(mean[i]);
      if (h0 + i < a.Rq) {
        uint16_t* orow = sd.out + (h0 + i) * a.Dh;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
          if (EQ || k * kGroup + l16 < nvec) {
            Vec<V> o;
#pragma unroll
            for (int j = 0; j < V / 2; ++j) {
              float y0 = RMS ? lo_f32(buf[i][k].w[j]) * rstd : (lo_f32(buf[i][k].w[j]) - mu) * rstd;
              float y1 = RMS ? hi_f32(buf[i][k].w[j]) * rstd : (hi_f32(buf[i][k].w[j]) - mu) * rstd;
              if constexpr (AFFINE && RMS) {
                y0 = y0 * wf[k][2 * j];
                y1 = y1 * wf[k][2 * j + 1];
              } else if constexpr (AFFINE) {
                y0 = __builtin_fmaf(wf[k][2 * j], y0, bf[k][2 * j]);
                y1 = __builtin_fmaf(wf[k][2 * j + 1], y1, bf[k][2 * j + 1]);
              }
              o.w[j] = pack_bf16(y0, y1);
            }
            store_vec_nt<V>(orow + off[k], o);
          }
        }
      }
    });
  };
  int64_t h0 = ((int64_t)blockIdx.x * kGroupsPerBlock + group) * HP;
  if (h0 >= a.Rq) return;
  // the next iteration's loads are issued as soon as this one's stores are
  Vec<V> buf[HP][NV];
  load(buf, h0);
  while (true) {
    process(buf, h0);
    h0 += step;
    if (h0 >= a.Rq) break;
    load(buf, h0);
  }
}

// One-shot grid: each 16-lane group takes HP heads (per side), normalizes
// them and exits; the hardware dispatcher keeps the compute units full.
// Measured on MI355X at (1,4360,32,128) q+k: 24.2 us with HP = 2, 24.4 with
// 4, against 25.3 for a persistent grid of 4 blocks per compute unit whose
// groups walk the heads.  (The kernel keeps its grid-stride loop for grids
// beyond kMaxHeadBlocks.)
#ifndef ADALN_QK_HP1
#define ADALN_QK_HP1 2
#endif
// at most 2^31 work-items (a dispatch counts its grid in 32 bits); the
// groups of a smaller grid walk the remaining heads
constexpr int64_t kMaxHeadBlocks = (int64_t)1 << 23;

template <bool RMS, int V, int NV, bool UNIFORM, bool AFFINE, bool EQ>
int launch_heads(const QkArgs& a, hipStream_t st) {
  constexpr int HP = NV == 1 ? ADALN_QK_HP1 : (NV == 2 ? 2 : 1);
  const int64_t need = (a.Rq + (int64_t)kGroupsPerBlock * HP - 1) / ((int64_t)kGroupsPerBlock * HP);
  const int64_t gx = std::max<int64_t>(1, std::min(need, kMaxHeadBlocks));
  hipLaunchKernelGGL((qk_heads<RMS, V, NV, HP, UNIFORM, AFFINE, EQ>), dim3((unsigned)gx, 2), dim3(256), 0,
                     st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <bool RMS, int V, int NV, bool UNIFORM, bool AFFINE>
int pick_eq(const QkArgs& a, hipStream_t st) {
  const bool eq = (a.Dh / V) == (int64_t)NV * kGroup;
  return eq ? launch_heads<RMS, V, NV, UNIFORM, AFFINE, true>(a, st)
            : launch_heads<RMS, V, NV, UNIFORM, AFFINE, false>(a, st);
}

template <bool RMS, int V, int NV>
int dispatch_heads(const QkArgs& a, bool uniform, bool affine, hipStream_t st) {
  if (uniform)
    return affine ? pick_eq<RMS, V, NV, true, true>(a, st) : pick_eq<RMS, V, NV, true, false>(a, st);
  return affine ? pick_eq<RMS, V, NV, false, true>(a, st) : pick_eq<RMS, V, NV, false, false>(a, st);
}

inline unsigned grid_for(int64_t heads) {
  int64_t blocks = (heads + kGroupsPerBlock - 1) / kGroupsPerBlock;
  return (unsigned)std::min(blocks, kMaxBlocks);
}

template <bool RMS, int V, int NV, bool UNIFORM, bool AFFINE, bool GATHER>
int launch(const QkArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((qk_rows<RMS, V, NV, UNIFORM, AFFINE, GATHER>), dim3(grid_for(2 * a.Rq)), dim3(256),
                     0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <bool RMS, int V, int NV, bool UNIFORM, bool AFFINE>
int pick_gather(const QkArgs& a, bool gather, hipStream_t st) {
  return gather ? launch<RMS, V, NV, UNIFORM, AFFINE, true>(a, st)
                : launch<RMS, V, NV, UNIFORM, AFFINE, false>(a, st);
}

template <bool RMS, int V, int NV, bool UNIFORM>
int pick_affine(const QkArgs& a, bool affine, bool gather, hipStream_t st) {
  return affine ? pick_gather<RMS, V, NV, UNIFORM, true>(a, gather, st)
                : pick_gather<RMS, V, NV, UNIFORM, false>(a, gather, st);
}

template <bool RMS, int V, int NV>
int pick_uniform(const QkArgs& a, bool uniform, bool affine, bool gather, hipStream_t st) {
  return uniform ? pick_affine<RMS, V, NV, true>(a, affine, gather, st)
                 : pick_affine<RMS, V, NV, false>(a, affine, gather, st);
}

}  // namespace

static int qk_check_shape(int64_t B, int64_t S, int64_t H, int64_t Dh, int64_t sq_b, int64_t sq_s,
                          int64_t sq_h, int64_t sk_b, int64_t sk_s, int64_t sk_h, int dtype) {
  if (dtype != ADALN_BF16) return ADALN_ERR_DTYPE;
  if (B < 0 || S < 0 || H < 0 || Dh < 4 || Dh % 4 != 0) return ADALN_ERR_SHAPE;
  if (Dh > 256) return ADALN_ERR_TOO_LARGE;
  if (sq_b < 0 || sq_s < 0 || sq_h < 0 || sk_b < 0 || sk_s < 0 || sk_h < 0) return ADALN_ERR_STRIDE;
  int64_t BS, R, RD;
  if (!mul_ok(B, S, &BS) || !mul_ok(BS, H, &R) || !mul_ok(R, Dh, &RD) || !mul_ok(R, 2, &BS))
    return ADALN_ERR_TOO_LARGE;
  if (!extent_ok({{B, sq_b}, {S, sq_s}, {H, sq_h}, {Dh, 1}}) ||
      !extent_ok({{B, sk_b}, {S, sk_s}, {H, sk_h}, {Dh, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

// The entry point of both per-head norms (RMS: RMSNorm with an optional
// weight and no bias; bq and bk are then NULL).
template <bool RMS>
static int qk_norm(const void* q, int64_t sq_b, int64_t sq_s, int64_t sq_h, const void* k,
                   int64_t sk_b, int64_t sk_s, int64_t sk_h, int64_t B, int64_t S, int64_t H,
                   int64_t Dh, const void* wq, const void* bq, const void* wk, const void* bk,
                   float eps, int dtype, void* q_out, void* k_out, void* stream) {
  int rc = qk_check_shape(B, S, H, Dh, sq_b, sq_s, sq_h, sk_b, sk_s, sk_h, dtype);
  if (rc != ADALN_OK) return rc;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return ADALN_ERR_ARG;
  const int64_t R = B * S * H;
  if (R == 0) return ADALN_OK;
  if (!q || !k || !q_out || !k_out) return ADALN_ERR_NULL;
  if (!RMS && ((wq == nullptr) != (bq == nullptr) || (wk == nullptr) != (bk == nullptr)))
    return ADALN_ERR_NULL;
  if ((wq == nullptr) != (wk == nullptr)) return ADALN_ERR_NULL;  // affine on both sides or neither
  const bool affine = wq != nullptr;
  for (const void* p : {q, k, (const void*)q_out, (const void*)k_out, wq, bq, wk, bk})
    if (!aligned(p, 2)) return ADALN_ERR_ALIGN;

  const Span sqo = span_of(q_out, {{R * Dh, 1}});
  const Span sko = span_of(k_out, {{R * Dh, 1}});
  const Span sq = span_of(q, {{B, sq_b}, {S, sq_s}, {H, sq_h}, {Dh, 1}});
  const Span sk = span_of(k, {{B, sk_b}, {S, sk_s}, {H, sk_h}, {Dh, 1}});
  auto contig = [&](int64_t sb, int64_t ss, int64_t sh) {
    return (H == 1 || sh == Dh) && (S == 1 || ss == H * Dh) && (B == 1 || sb == S * H * Dh);
  };
  if (overlaps(sqo, sko)) return ADALN_ERR_ALIAS;
  if (overlaps(sqo, sq) && !(q_out == q && contig(sq_b, sq_s, sq_h))) return ADALN_ERR_ALIAS;
  if (overlaps(sko, sk) && !(k_out == k && contig(sk_b, sk_s, sk_h))) return ADALN_ERR_ALIAS;
  if (overlaps(sqo, sk) || overlaps(sko, sq)) return ADALN_ERR_ALIAS;
  if (affine) {
    for (const void* p : {wq, bq, wk, bk}) {
      if (!p) continue;
      const Span sw = span_of(p, {{Dh, 1}});
      if (overlaps(sw, sqo) || overlaps(sw, sko)) return ADALN_ERR_ALIAS;
    }
  }

  QkArgs a;
  a.side[0] = QkSide{(const uint16_t*)q, sq_b, sq_s, sq_h, (const uint16_t*)wq, (const uint16_t*)bq,
                     (uint16_t*)q_out};
  a.side[1] = QkSide{(const uint16_t*)k, sk_b, sk_s, sk_h, (const uint16_t*)wk, (const uint16_t*)bk,
                     (uint16_t*)k_out};
  a.S = S;
  a.H = H;
  a.Dh = Dh;
  a.Rq = R;
  a.eps = eps;

  const int V = vec_of(RMS ? ADALN_OP_QK_RMSNORM : ADALN_OP_QK_HEAD_LAYERNORM, Dh);
  const uintptr_t vb = (uintptr_t)(2 * V);
  auto st_ok = [&](int64_t n, int64_t s) { return n <= 1 || ((uintptr_t)s * 2u) % vb == 0; };
  bool vec = true;
  for (const void* p : {q, k, (const void*)q_out, (const void*)k_out, wq, bq, wk, bk})
    if (p && !aligned(p, vb)) vec = false;
  vec = vec && st_ok(B, sq_b) && st_ok(S, sq_s) && st_ok(H, sq_h) && st_ok(B, sk_b) &&
        st_ok(S, sk_s) && st_ok(H, sk_h);
  // one row stride per side: head rows of q (and of k) evenly spaced, so
  // row rr of the [B*S*H, Dh] view starts at rr * stride
  auto row_stride = [&](int64_t sb, int64_t ss, int64_t sh, int64_t* r) {
    *r = H > 1 ? sh : (S > 1 ? ss : sb);
    return (S == 1 || ss == H * *r) && (B == 1 || sb == S * H * *r);
  };
  int64_t rq = 0, rk = 0;
  const bool uniform = row_stride(sq_b, sq_s, sq_h, &rq) && row_stride(sk_b, sk_s, sk_h, &rk);
  if (uniform) {
    a.side[0].s_h = rq;
    a.side[1].s_h = rk;
  }
  hipStream_t st = (hipStream_t)stream;
  const bool gather = !vec;
  const int64_t nv = (Dh / V + kGroup - 1) / kGroup;
  if (vec) {
    if (V == 8) return nv <= 1 ? dispatch_heads<RMS, 8, 1>(a, uniform, affine, st)
                               : dispatch_heads<RMS, 8, 2>(a, uniform, affine, st);
    if (nv <= 1) return dispatch_heads<RMS, 4, 1>(a, uniform, affine, st);
    if (nv <= 2) return dispatch_heads<RMS, 4, 2>(a, uniform, affine, st);
    return dispatch_heads<RMS, 4, 4>(a, uniform, affine, st);
  }
  if (V == 8) {
    if (nv <= 1) return pick_uniform<RMS, 8, 1>(a, uniform, affine, gather, st);
    return pick_uniform<RMS, 8, 2>(a, uniform, affine, gather, st);
  }
  if (nv <= 1) return pick_uniform<RMS, 4, 1>(a, uniform, affine, gather, st);
  if (nv <= 2) return pick_uniform<RMS, 4, 2>(a, uniform, affine, gather, st);
  return pick_uniform<RMS, 4, 4>(a, uniform, affine, gather, st);
}

}  // namespace adaln

using namespace adaln;

extern "C" int qk_head_layernorm_can_use(int64_t B, int64_t S, int64_t H, int64_t Dh, int64_t sq_b,
                                         int64_t sq_s, int64_t sq_h, int64_t sk_b, int64_t sk_s,
                                         int64_t sk_h, int dtype) {
  return qk_check_shape(B, S, H, Dh, sq_b, sq_s, sq_h, sk_b, sk_s, sk_h, dtype) == ADALN_OK;
}

extern "C" int qk_head_layernorm(const void* q, int64_t sq_b, int64_t sq_s, int64_t sq_h,
                                 const void* k, int64_t sk_b, int64_t sk_s, int64_t sk_h, int64_t B,
                                 int64_t S, int64_t H, int64_t Dh, const void* wq, const void* bq,
                                 const void* wk, const void* bk, float eps, int dtype, void* q_out,
                                 void* k_out, void* stream) {
  return qk_norm<false>(q, sq_b, sq_s, sq_h, k, sk_b, sk_s, sk_h, B, S, H, Dh, wq, bq, wk, bk, eps,
                        dtype, q_out, k_out, stream);
}

extern "C" int qk_rmsnorm_can_use(int64_t B, int64_t S, int64_t H, int64_t Dh, int64_t sq_b,
                                  int64_t sq_s, int64_t sq_h, int64_t sk_b, int64_t sk_s,
                                  int64_t sk_h, int dtype) {
  return qk_check_shape(B, S, H, Dh, sq_b, sq_s, sq_h, sk_b, sk_s, sk_h, dtype) == ADALN_OK;
}

extern "C" int qk_rmsnorm(const void* q, int64_t sq_b, int64_t sq_s, int64_t sq_h, const void* k,
                          int64_t sk_b, int64_t sk_s, int64_t sk_h, int64_t B, int64_t S, int64_t H,
                          int64_t Dh, const void* wq, const void* wk, float eps, int dtype,
                          void* q_out, void* k_out, void* stream) {
  return qk_norm<true>(q, sq_b, sq_s, sq_h, k, sk_b, sk_s, sk_h, B, S, H, Dh, wq, nullptr, wk,
                       nullptr, eps, dtype, q_out, k_out, stream);
}
