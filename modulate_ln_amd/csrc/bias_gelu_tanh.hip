// bias_gelu_tanh: z = bf16(x + bias); out = bf16(gelu_tanh(z)) on gfx950.
//
// Operation: PR #37075 report (Wan2.2 NVFP4 bias + GELU), 实现拆解 §1 and
// 关键源码片段 (bias_gelu.cuh): the bias is added in fp32, the sum is rounded
// back to bf16 (the eager rounding boundary between the add and the GELU),
// then tanh-GELU is evaluated in fp32 and rounded.
//
// GELU: gelu_tanh(z) = 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3)
// (Hendrycks & Gimpel).  Using 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)) it is
// z * sigmoid(2u), evaluated with one base-2 exponential and one hardware
// reciprocal (see gelu_tanh_f32).  Result within one bf16 ulp of the
// correctly rounded value.
//
// Design: streaming.  Vector-aligned rows take a one-shot grid: each thread
// loads two 16-byte vectors of x (non-temporal) and the matching bias
// vectors (cached: every row reads the same bias), computes and stores, and
// the wave exits; the hardware dispatcher keeps the compute units full.
// Grids too large for one launch take the column-chunk kernel: wave w of
// chunk c owns vectors c*64*U + lane + 64*u (u < U) of every row it visits,
// keeps that chunk of the bias in VGPRs for the whole launch and loads the
// next row it visits while it computes the current one.

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

// t = 2u log2(e) = z (c0 + c1 z^2) with c0 = 2 sqrt(2/pi) log2(e) and
// c1 = 0.044715 c0; t has the sign of z.  sigmoid(2u) = 1 / (1 + 2^-t) for
// t >= 0 and 2^t / (1 + 2^t) otherwise, so the exponential is only ever
// taken of -|t|.  The hardware exp2 returns normal numbers only, so it is
// evaluated at 64 - |t| (normal down to |t| = 190) and scaled back by the
// exact factor 2^-64, which keeps denormal e; beyond |t| = 190 the result is
// below every bf16 subnormal anyway.
__device__ __forceinline__ float gelu_tanh_f32(float z) {
  const float c0 = 2.302208198144324889f;  // 2 * sqrt(2/pi) * log2(e)
  const float c1 = 0.102943239580023487f;  // 0.044715 * c0
  const float t = z * __builtin_fmaf(z * z, c1, c0);
  const float e = __builtin_amdgcn_exp2f(64.0f - __builtin_fabsf(t)) * 0x1p-64f;  // 2^-|t|
  const float num = (t >= 0.0f) ? z : z * e;
  return num * __builtin_amdgcn_rcpf(1.0f + e);  // 1 + e in [1, 2]
}

// The same function in fewer operations, for t >= kFastMinT: sigmoid(2u) =
// 1 / (1 + 2^-t) directly.  There 2^-t is a normal number (or underflows
// where the result is z itself) and 1 / (1 + 2^-t) >= 2^-120 stays normal,
// so no rescaling and no select are needed: one exponential, one add, one
// reciprocal, one product.  Below kFastMinT (z < -9.4, and -inf) the
// reciprocal would leave the normal range: gelu_tanh_f32 takes those.
constexpr float kGeluC0 = 2.302208198144324889f;  // 2 * sqrt(2/pi) * log2(e)
constexpr float kGeluC1 = 0.102943239580023487f;  // 0.044715 * c0
constexpr float kFastMinT = -120.0f;

__device__ __forceinline__ float gelu_fast(float z, float t) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-t));
}

// gelu of z given its t: the fast form, or gelu_tanh_f32 below kFastMinT
__device__ __forceinline__ float gelu_eval(float z, float t) {
  return t < kFastMinT ? gelu_tanh_f32(z) : gelu_fast(z, t);
}

template <int V>
__device__ __forceinline__ Vec<V> bias_gelu_vec(const Vec<V>& xv, const Vec<V>& bv) {
  float z[V], t[V];
  bool tail = false;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    z[2 * i] = lo_f32(xv.w[i]) + lo_f32(bv.w[i]);
    z[2 * i + 1] = hi_f32(xv.w[i]) + hi_f32(bv.w[i]);
    round_pair(z[2 * i], z[2 * i + 1]);  // bf16(x + bias)
  }
#pragma unroll
  for (int e = 0; e < V; ++e) {
    t[e] = z[e] * __builtin_fmaf(z[e] * z[e], kGeluC1, kGeluC0);
    tail = tail || t[e] < kFastMinT;
  }
  float g[V];
  if (__builtin_amdgcn_ballot_w64(tail) != 0) {  // wave-uniform: a far negative z somewhere
#pragma unroll
    for (int e = 0; e < V; ++e) g[e] = gelu_eval(z[e], t[e]);
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) g[e] = gelu_fast(z[e], t[e]);
  }
  Vec<V> o;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) o.w[i] = pack_bf16(g[2 * i], g[2 * i + 1]);
  return o;
}

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

template <int V, int U>
__global__ __launch_bounds__(256) void gelu_chunks(GeluArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nvec = a.width / V;
  const int64_t step = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (r >= a.rows) return;
  bool ok[U];
  uint32_t off[U];  // element offset of the lane's u-th vector (clamped in-bounds; width < 2^31)
  Vec<V> bv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)blockIdx.y * kWave * U + (int64_t)u * kWave + lane;
    ok[u] = v < nvec;
    off[u] = (uint32_t)((ok[u] ? v : nvec - 1) * V);
    bv[u] = load_vec<V>(a.bias + off[u]);
  }
  auto load_row = [&](Vec<V>* xv, int64_t rr) {
    const uint16_t* xr = a.x + rr * a.sx_row;
#pragma unroll
    for (int u = 0; u < U; ++u) xv[u] = load_vec_nt<V>(xr + off[u]);
  };
  auto store_row = [&](const Vec<V>* xv, int64_t rr) {
    uint16_t* orow = a.out + rr * a.width;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) store_vec_nt<V>(orow + off[u], bias_gelu_vec<V>(xv[u], bv[u]));
      __builtin_amdgcn_sched_barrier(0);  // one vector's temporaries live at a time
    }
  };
  Vec<V> xa[U], xb[U];
  load_row(xa, r);
  while (true) {  // double buffer: row r in xa (or xb), row r + step loading into the other
    int64_t r1 = r + step;
    if (r1 < a.rows) load_row(xb, r1);
    store_row(xa, r);
    if (r1 >= a.rows) break;
    r = r1;
    r1 = r + step;
    if (r1 < a.rows) load_row(xa, r1);
    store_row(xb, r);
    if (r1 >= a.rows) break;
    r = r1;
  }
}

// One-shot grid: block b covers vectors [c*256*U, (c+1)*256*U) of row
// b / bpr (c = b % bpr); thread t takes vectors c*256*U + u*256 + t.  Every
// wave reads and writes whole 1 KiB runs and exits.
template <int V, int U>
__global__ __launch_bounds__(256) void gelu_flat(GeluArgs a, int bpr) {
  const int64_t row = blockIdx.x / bpr;
  const int c = blockIdx.x - (int)row * bpr;
  const int nvec = (int)(a.width / V);
  const uint16_t* xr = a.x + row * a.sx_row;
  uint16_t* orow = a.out + row * a.width;
  Vec<V> xv[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int v = c * 256 * U + u * 256 + (int)threadIdx.x;
    ok[u] = v < nvec;
    if (ok[u]) xv[u] = load_vec_nt<V>(xr + v * V);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int v = c * 256 * U + u * 256 + (int)threadIdx.x;
    if (ok[u]) {
      const Vec<V> bv = load_vec<V>(a.bias + v * V);
      store_vec_nt<V>(orow + v * V, bias_gelu_vec<V>(xv[u], bv));
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
      orow[j] = to_bf16(gelu_eval(z, z * __builtin_fmaf(z * z, kGeluC1, kGeluC0)));
    }
  }
}

inline unsigned grid_for(int64_t R) {
  int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  return (unsigned)std::min(blocks, kMaxBlocks);
}

// grid size of the column-chunk kernel (blocks per compute unit in total),
// measured on MI355X; overridable at build time
#ifndef ADALN_CHUNK_BLOCKS_PER_CU
#define ADALN_CHUNK_BLOCKS_PER_CU 16
#endif
constexpr int kChunkBlocksPerCu = ADALN_CHUNK_BLOCKS_PER_CU;

template <int V, int U>
int launch_chunks(const GeluArgs& a, hipStream_t st) {
  const int64_t nvec = a.width / V;
  const int64_t nchunks = (nvec + kWave * U - 1) / (kWave * U);
  if (nchunks > 65535) {  // grid.y limit: very long rows go element-wise
    hipLaunchKernelGGL(gelu_rows_scalar, dim3(grid_for(a.rows)), dim3(256), 0, st, a);
    return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
  }
  const int cus = cu_count();
  const int64_t target = (int64_t)kChunkBlocksPerCu * (cus > 0 ? cus : 256);
  int64_t gx = (target + nchunks - 1) / nchunks;
  gx = std::max<int64_t>(1, std::min<int64_t>(gx, (a.rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((gelu_chunks<V, U>), dim3((unsigned)gx, (unsigned)nchunks), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// most vectors per lane in one chunk (VGPRs: two row buffers and the bias)
#ifndef ADALN_GELU_MAX_U
#define ADALN_GELU_MAX_U 4
#endif

// Vectors per thread of the one-shot grid (0: column chunks only).  The
// one-shot grid, whose waves each read and write two 1 KiB runs and exit,
// measured 5 % faster on MI355X than the column chunks at (16384, 12288).
#ifndef ADALN_GELU_FLAT_U
#define ADALN_GELU_FLAT_U 2
#endif

template <int V>
int dispatch_chunks(const GeluArgs& a, hipStream_t st) {
  if constexpr (ADALN_GELU_FLAT_U > 0) {
    constexpr int U = ADALN_GELU_FLAT_U;
    const int64_t nvec = a.width / V;
    const int64_t bpr = (nvec + 256 * U - 1) / (256 * U);
    if (a.rows * bpr < ((int64_t)1 << 24)) {
      hipLaunchKernelGGL((gelu_flat<V, U>), dim3((unsigned)(a.rows * bpr)), dim3(256), 0, st, a, (int)bpr);
      return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
    }
  }
  const int64_t per_lane = (a.width / V + kWave - 1) / kWave;
  switch (std::min<int64_t>(per_lane, ADALN_GELU_MAX_U)) {
    case 1: return launch_chunks<V, 1>(a, st);
    case 2: return launch_chunks<V, 2>(a, st);
    case 3: return launch_chunks<V, 3>(a, st);
    case 4: return launch_chunks<V, 4>(a, st);
    case 5: return launch_chunks<V, 5>(a, st);
    case 6: return launch_chunks<V, 6>(a, st);
    case 7: return launch_chunks<V, 7>(a, st);
    default: return launch_chunks<V, 8>(a, st);
  }
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
  if (width >= ((int64_t)1 << 31)) return ADALN_ERR_TOO_LARGE;
  if (overlaps(so, sx) && !(x == out && x_contig)) return ADALN_ERR_ALIAS;
  if (overlaps(so, sb)) return ADALN_ERR_ALIAS;

  GeluArgs a{(const uint16_t*)x, sx_row, (const uint16_t*)bias, (uint16_t*)out, rows, width};
  auto vec_ok = [&](uintptr_t vb) {
    return width % (int64_t)(vb / 2) == 0 && aligned(x, vb) && aligned(bias, vb) &&
           aligned(out, vb) && (rows <= 1 || ((uintptr_t)sx_row * 2u) % vb == 0);
  };
  hipStream_t st = (hipStream_t)stream;
  if (vec_ok(16)) return dispatch_chunks<8>(a, st);
  if (vec_ok(8)) return dispatch_chunks<4>(a, st);
  hipLaunchKernelGGL(gelu_rows_scalar, dim3(grid_for(rows)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}
