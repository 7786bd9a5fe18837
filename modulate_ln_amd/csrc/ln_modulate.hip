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
#include <utility>

#include "device_common.hpp"
#include "host_common.hpp"

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
  uint16_t* out;
  float* mean_out;
  float* rstd_out;
  int64_t R;
};

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

template <int V, int... K>
__device__ __forceinline__ void welford_lane(const Vec<V>* buf, int64_t nvec, int lane, float& mean,
                                             float& m2, std::integer_sequence<int, K...>) {
  (
      [&] {
        if ((int64_t)K * kWave + lane < nvec)
          push_vec<V, K>(buf[K], mean, m2, std::make_integer_sequence<int, V>{});
      }(),
      ...);
}

// the per-element tail of the chain for one vector
template <int V>
__device__ __forceinline__ Vec<V> modulate_vec(const Vec<V>& xv, const Vec<V>& sv, const Vec<V>& hv,
                                               float mean, float rstd) {
  Vec<V> o;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    float n0 = (lo_f32(xv.w[i]) - mean) * rstd;
    float n1 = (hi_f32(xv.w[i]) - mean) * rstd;
    round_pair(n0, n1);  // x_hat = bf16(rstd * (x - mean))
    float p0 = 1.0f + lo_f32(sv.w[i]);
    float p1 = 1.0f + hi_f32(sv.w[i]);
    round_pair(p0, p1);  // bf16(1 + scale)
    float y0 = n0 * p0;
    float y1 = n1 * p1;
    round_pair(y0, y1);  // bf16(x_hat * (1 + scale))
    o.w[i] = pack_bf16(y0 + lo_f32(hv.w[i]), y1 + hi_f32(hv.w[i]));  // bf16(y + shift)
  }
  return o;
}

// NV = the largest number of vectors any lane owns for the rows this
// instantiation serves (the launcher guarantees D/V <= 64*NV).
template <int V, int NV, bool GATHER>
__global__ __launch_bounds__(256) void ln_modulate_rows(LnArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nvec = a.D / V;
  const float Df = (float)a.D;
  const int64_t nv_lane = nvec > lane ? (nvec - lane + kWave - 1) / kWave : 0;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < a.R;
       r += (int64_t)gridDim.x * 4) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;

    Vec<V> buf[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kWave + lane;
      if (v < nvec) {
        if constexpr (GATHER)
          buf[k] = gather_vec<V>(xr + v * V * a.sx_d, a.sx_d);
        else
          buf[k] = load_vec<V>(xr + v * V);
      }
    }

    float mean = 0.0f, m2 = 0.0f;
    welford_lane<V>(buf, nvec, lane, mean, m2, std::make_integer_sequence<int, NV>{});
    float n = (float)(nv_lane * V);
    merge_lanes<64>(mean, m2, n, lane);
    const float rstd = finalize_rstd(m2, Df, a.eps);
    if (lane == 0) {
      if (a.mean_out) a.mean_out[r] = mean;
      if (a.rstd_out) a.rstd_out[r] = rstd;
    }

    const uint16_t* sc = a.scale + b * a.ssc_b;
    const uint16_t* sh = a.shift + b * a.ssh_b;
    uint16_t* orow = a.out + r * a.D;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t v = (int64_t)k * kWave + lane;
      if (v < nvec) {
        if constexpr (GATHER) {
          Vec<V> sv = gather_vec<V>(sc + v * V, 1);
          Vec<V> hv = gather_vec<V>(sh + v * V, 1);
          scatter_vec<V>(orow + v * V, modulate_vec<V>(buf[k], sv, hv, mean, rstd));
        } else {
          Vec<V> sv = load_vec<V>(sc + v * V);
          Vec<V> hv = load_vec<V>(sh + v * V);
          store_vec<V>(orow + v * V, modulate_vec<V>(buf[k], sv, hv, mean, rstd));
        }
      }
    }
  }
}

// Rows too long to hold in registers: the same order, pass 2 re-reads the
// row (from L2 when it is still resident).  1/n comes from a table of
// correctly rounded reciprocals built at compile time.
constexpr int kMaxStreamSteps = 65536 / kWave;  // counts per lane at D = 65536
struct RcpTable {
  float v[kMaxStreamSteps + 1];
};
constexpr RcpTable make_rcp_table() {
  RcpTable t{};
  t.v[0] = 0.0f;
  for (int i = 1; i <= kMaxStreamSteps; ++i) t.v[i] = 1.0f / (float)i;
  return t;
}
__constant__ RcpTable kRcp = make_rcp_table();

template <int V, bool GATHER>
__global__ __launch_bounds__(256) void ln_modulate_stream(LnArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nvec = a.D / V;
  const float Df = (float)a.D;
  const int64_t nv_lane = nvec > lane ? (nvec - lane + kWave - 1) / kWave : 0;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < a.R;
       r += (int64_t)gridDim.x * 4) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;
    float mean = 0.0f, m2 = 0.0f;
    for (int64_t k = 0; k < nv_lane; ++k) {
      const int64_t v = k * kWave + lane;
      Vec<V> xv = GATHER ? gather_vec<V>(xr + v * V * a.sx_d, a.sx_d) : load_vec<V>(xr + v * V);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float x = (e & 1) ? hi_f32(xv.w[e / 2]) : lo_f32(xv.w[e / 2]);
        const float rc = kRcp.v[k * V + e + 1];
        float delta = x - mean;
        mean = __builtin_fmaf(delta, rc, mean);
        m2 = __builtin_fmaf(delta, x - mean, m2);
      }
    }
    float n = (float)(nv_lane * V);
    merge_lanes<64>(mean, m2, n, lane);
    const float rstd = finalize_rstd(m2, Df, a.eps);
    if (lane == 0) {
      if (a.mean_out) a.mean_out[r] = mean;
      if (a.rstd_out) a.rstd_out[r] = rstd;
    }
    const uint16_t* sc = a.scale + b * a.ssc_b;
    const uint16_t* sh = a.shift + b * a.ssh_b;
    uint16_t* orow = a.out + r * a.D;
    for (int64_t k = 0; k < nv_lane; ++k) {
      const int64_t v = k * kWave + lane;
      if constexpr (GATHER) {
        Vec<V> xv = gather_vec<V>(xr + v * V * a.sx_d, a.sx_d);
        Vec<V> sv = gather_vec<V>(sc + v * V, 1);
        Vec<V> hv = gather_vec<V>(sh + v * V, 1);
        scatter_vec<V>(orow + v * V, modulate_vec<V>(xv, sv, hv, mean, rstd));
      } else {
        Vec<V> xv = load_vec<V>(xr + v * V);
        Vec<V> sv = load_vec<V>(sc + v * V);
        Vec<V> hv = load_vec<V>(sh + v * V);
        store_vec<V>(orow + v * V, modulate_vec<V>(xv, sv, hv, mean, rstd));
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

template <int V, int NV, bool GATHER>
int launch_rows(const LnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((ln_modulate_rows<V, NV, GATHER>), dim3(grid_for(a.R)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <int V, bool GATHER>
int launch_stream(const LnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((ln_modulate_stream<V, GATHER>), dim3(grid_for(a.R)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// vectors per lane -> the register-resident instantiation that covers it
template <int V, bool GATHER>
int dispatch(const LnArgs& a, hipStream_t st) {
  const int64_t nv = (a.D / V + kWave - 1) / kWave;
#define ADALN_NV_CASE(N) \
  if (nv <= N) return launch_rows<V, N, GATHER>(a, st);
  ADALN_NV_CASE(1)
  ADALN_NV_CASE(2)
  ADALN_NV_CASE(3)
  ADALN_NV_CASE(4)
  ADALN_NV_CASE(5)
  ADALN_NV_CASE(6)
  ADALN_NV_CASE(8)
  ADALN_NV_CASE(10)
  ADALN_NV_CASE(12)
  ADALN_NV_CASE(16)
  ADALN_NV_CASE(24)
  ADALN_NV_CASE(32)
#undef ADALN_NV_CASE
  return launch_stream<V, GATHER>(a, st);
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
  int rc = ln_modulate_check_shape(B, S, D, sx_b, sx_s, sx_d, sscale_b, sshift_b, dtype);
  if (rc != ADALN_OK) return rc;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return ADALN_ERR_ARG;  // also rejects NaN
  const int64_t R = B * S;
  if (R == 0) return ADALN_OK;
  if (!x || !scale || !shift || !out) return ADALN_ERR_NULL;
  if (!aligned(x, 2) || !aligned(scale, 2) || !aligned(shift, 2) || !aligned(out, 2) ||
      !aligned(mean_out, 4) || !aligned(rstd_out, 4))
    return ADALN_ERR_ALIGN;

  // overlap rules: out may be exactly a contiguous x; nothing else may overlap
  const Span so = span_of(out, {{R * D, 1}});
  const Span sx = span_of(x, {{B, sx_b}, {S, sx_s}, {D, sx_d}});
  const Span ssc = span_of(scale, {{B, sscale_b}, {D, 1}});
  const Span ssh = span_of(shift, {{B, sshift_b}, {D, 1}});
  const bool x_contig = sx_d == 1 && (S == 1 || sx_s == D) && (B == 1 || sx_b == S * D);
  if (overlaps(so, sx) && !(x == out && x_contig)) return ADALN_ERR_ALIAS;
  if (overlaps(so, ssc) || overlaps(so, ssh)) return ADALN_ERR_ALIAS;
  const Span sm = mean_out ? Span{(uintptr_t)mean_out, (uintptr_t)(mean_out + R)} : Span{};
  const Span sr = rstd_out ? Span{(uintptr_t)rstd_out, (uintptr_t)(rstd_out + R)} : Span{};
  for (const Span* t : {&so, &sx, &ssc, &ssh})
    if (overlaps(sm, *t) || overlaps(sr, *t)) return ADALN_ERR_ALIAS;
  if (overlaps(sm, sr)) return ADALN_ERR_ALIAS;

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
  a.out = (uint16_t*)out;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.R = R;

  int V = 0;
  order_for(ADALN_OP_LN_MODULATE, D, &V, nullptr);
  // vector loads need every row start of x, scale, shift and out on a 2V-byte boundary
  const uintptr_t vb = (uintptr_t)(2 * V);
  auto stride_ok = [&](int64_t n, int64_t st) { return n <= 1 || ((uintptr_t)st * 2u) % vb == 0; };
  const bool vec = sx_d == 1 && aligned(x, vb) && aligned(scale, vb) && aligned(shift, vb) &&
                   aligned(out, vb) && stride_ok(B, sx_b) && stride_ok(S, sx_s) &&
                   stride_ok(B, sscale_b) && stride_ok(B, sshift_b);
  hipStream_t st = (hipStream_t)stream;
  if (V == 8) return vec ? dispatch<8, false>(a, st) : dispatch<8, true>(a, st);
  return vec ? dispatch<4, false>(a, st) : dispatch<4, true>(a, st);
}
