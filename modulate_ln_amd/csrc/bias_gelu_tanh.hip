// bias_gelu_tanh: z = bf16(x + bias); out = bf16(gelu_tanh(z)) on gfx950.
//
// Operation: PR #37075 report (Wan2.2 NVFP4 bias + GELU), 实现拆解 §1 and
// 关键源码片段 (bias_gelu.cuh): the bias is added in fp32, the sum is rounded
// back to bf16 (the eager rounding boundary between the add and the GELU),
// then tanh-GELU is evaluated in fp32 and rounded.
//
// GELU: gelu_tanh(z) = 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3)
// (Hendrycks & Gimpel).  Using 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)) it is
// z * sigmoid(2u); the exponential is taken of -|2u| only (never overflows),
// through the hardware base-2 exponential, and the sigmoid of a negative
// argument is e/(1+e).  Result within one bf16 ulp of the correctly rounded
// value.
//
// Design: streaming, one wavefront per row, U independent 16-byte loads per
// lane in flight; the bias row stays in cache.
#include "device_common.hpp"
#include "host_common.hpp"

namespace adaln {
namespace {

struct GeluArgs {
  const uint16_t* x;
  int64_t sx_row;
  const uint16_t* bias;
  uint16_t* out;
  int64_t rows, width;
};

__device__ __forceinline__ float gelu_tanh_f32(float z) {
  const float k0 = 0.797884560802865355f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float log2e = 1.44269504088896341f;
  float z3 = (z * z) * z;
  float u = k0 * (z + k1 * z3);
  float t = 2.0f * u;
  float e = __builtin_exp2f(-__builtin_fabsf(t) * log2e);  // e^(-|t|) in [0, 1]
  float num = (t >= 0.0f) ? z : z * e;
  return num * __builtin_amdgcn_rcpf(1.0f + e);  // 1 + e in [1, 2]
}

template <int V>
__device__ __forceinline__ Vec<V> bias_gelu_vec(const Vec<V>& xv, const Vec<V>& bv) {
  Vec<V> o;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    float z0 = lo_f32(xv.w[i]) + lo_f32(bv.w[i]);
    float z1 = hi_f32(xv.w[i]) + hi_f32(bv.w[i]);
    round_pair(z0, z1);  // bf16(x + bias)
    o.w[i] = pack_bf16(gelu_tanh_f32(z0), gelu_tanh_f32(z1));
  }
  return o;
}

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

template <int V, int U>
__global__ __launch_bounds__(256) void gelu_rows_vec(GeluArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nvec = a.width / V;
  for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < a.rows;
       r += (int64_t)gridDim.x * kRowsPerBlock) {
    const uint16_t* xr = a.x + r * a.sx_row;
    uint16_t* orow = a.out + r * a.width;
    for (int64_t base = lane; base < nvec; base += (int64_t)U * kWave) {
      Vec<V> xv[U], bv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = base + (int64_t)u * kWave;
        if (v < nvec) {
          xv[u] = load_vec<V>(xr + v * V);
          bv[u] = load_vec<V>(a.bias + v * V);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t v = base + (int64_t)u * kWave;
        if (v < nvec) store_vec<V>(orow + v * V, bias_gelu_vec<V>(xv[u], bv[u]));
      }
    }
  }
}

__global__ __launch_bounds__(256) void gelu_rows_scalar(GeluArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < a.rows;
       r += (int64_t)gridDim.x * kRowsPerBlock) {
    const uint16_t* xr = a.x + r * a.sx_row;
    uint16_t* orow = a.out + r * a.width;
    for (int64_t j = lane; j < a.width; j += kWave) {
      float z = u16_f32(to_bf16(u16_f32(xr[j]) + u16_f32(a.bias[j])));
      orow[j] = to_bf16(gelu_tanh_f32(z));
    }
  }
}

inline unsigned grid_for(int64_t R) {
  int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  return (unsigned)std::min(blocks, kMaxBlocks);
}

}  // namespace

static int gelu_check_shape(int64_t rows, int64_t width, int64_t sx_row, int dtype) {
  if (dtype != ADALN_BF16) return ADALN_ERR_DTYPE;
  if (rows < 0 || width < 0) return ADALN_ERR_SHAPE;
  if (sx_row < 0) return ADALN_ERR_STRIDE;
  int64_t n;
  if (!mul_ok(rows, width, &n) || !extent_ok({{rows, sx_row}, {width, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

}  // namespace adaln

using namespace adaln;

extern "C" int bias_gelu_tanh_can_use(int64_t rows, int64_t width, int64_t sx_row, int dtype) {
  return gelu_check_shape(rows, width, sx_row, dtype) == ADALN_OK;
}

extern "C" int bias_gelu_tanh(const void* x, int64_t rows, int64_t width, int64_t sx_row,
                              const void* bias, int dtype, void* out, void* stream) {
  int rc = gelu_check_shape(rows, width, sx_row, dtype);
  if (rc != ADALN_OK) return rc;
  if (rows == 0 || width == 0) return ADALN_OK;
  if (!x || !bias || !out) return ADALN_ERR_NULL;
  if (!aligned(x, 2) || !aligned(bias, 2) || !aligned(out, 2)) return ADALN_ERR_ALIGN;
  const Span so = span_of(out, {{rows * width, 1}});
  const Span sx = span_of(x, {{rows, sx_row}, {width, 1}});
  const Span sb = span_of(bias, {{width, 1}});
  const bool x_contig = rows == 1 || sx_row == width;
  if (overlaps(so, sx) && !(x == out && x_contig)) return ADALN_ERR_ALIAS;
  if (overlaps(so, sb)) return ADALN_ERR_ALIAS;

  GeluArgs a{(const uint16_t*)x, sx_row, (const uint16_t*)bias, (uint16_t*)out, rows, width};
  auto vec_ok = [&](uintptr_t vb) {
    return width % (int64_t)(vb / 2) == 0 && aligned(x, vb) && aligned(bias, vb) &&
           aligned(out, vb) && (rows <= 1 || ((uintptr_t)sx_row * 2u) % vb == 0);
  };
  hipStream_t st = (hipStream_t)stream;
  if (vec_ok(16))
    hipLaunchKernelGGL((gelu_rows_vec<8, 8>), dim3(grid_for(rows)), dim3(256), 0, st, a);
  else if (vec_ok(8))
    hipLaunchKernelGGL((gelu_rows_vec<4, 8>), dim3(grid_for(rows)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(gelu_rows_scalar, dim3(grid_for(rows)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}
