// temb_table_slices: the nmod adaLN slices of (table + temb) in one pass, on
// gfx950.
//
// Operation: "Fused Kernels" page, table "adaLN modulation and gating"
// (temb_table_slices, bit-exact) and the note under it: the eager
// (scale_shift_table + temb.float()).chunk(6, dim=2) materializes the fp32 sum
// and hands out strided slices whose .contiguous() copies each one again.
// Here slice m of the sum is written straight into its own contiguous block:
//   out[m][b, l, d] = table[m, d] + float(temb[b, l, m, d])   (one fp32 add)
// so each slice is ready for the modulate that reads it.
//
// Design: streaming.  A one-shot grid whose blocks are ordered (slice, row,
// column block), so the output -- two thirds of the traffic -- is written in
// address order by short-lived waves (measured 12 % faster on MI355X than
// column-chunk waves that walk the rows, which remain for grids too large
// for one launch).  Each lane handles runs of 4 elements (8 bytes of bf16 or
// 16 of fp32 in, 16 bytes of fp32 out), so every store instruction of a wave
// writes one contiguous 1 KiB -- measured 1.28x faster than 8-element runs,
// whose 32-byte lane stores leave every instruction's lines half written.
// temb is read and the output written non-temporally; the table, which every
// row reads, through the caches.
#include "device_common.hpp"
#include "host_common.hpp"

namespace adaln {
namespace {

struct TembArgs {
  const float* table;
  int64_t st_m;  // table row stride (elements)
  const void* temb;
  int64_t se_b, se_l, se_m;  // temb strides (elements)
  int64_t L, nmod, D, R;     // R = B * L
  float* out;                // [nmod][R][D]
};

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// V consecutive elements of temb widened to fp32 (V = 4: one 8-byte load of
// bf16 or 16 of fp32; V = 8: 16 bytes of bf16 or 32 of fp32)
template <int V>
__device__ __forceinline__ void loadv(const uint16_t* p, float* f) {
  const Vec<V> v = load_vec_nt<V>(p);
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    f[2 * i] = lo_f32(v.w[i]);
    f[2 * i + 1] = hi_f32(v.w[i]);
  }
}

template <int V>
__device__ __forceinline__ void loadv(const float* p, float* f) {
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + q);
#pragma unroll
    for (int i = 0; i < 4; ++i) f[4 * q + i] = a[i];
  }
}

template <int V>
__device__ __forceinline__ void storev(float* p, const float* f) {
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    f32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = f[4 * q + i];
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p) + q);
  }
}

template <typename T, int V, int U>
__global__ __launch_bounds__(256) void temb_chunks(TembArgs a, int nchunks) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t m = blockIdx.y / nchunks;
  const int64_t c = blockIdx.y - m * nchunks;
  const int64_t nvec = a.D / V;
  const int64_t step = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (r >= a.R) return;
  int64_t b = r / a.L;
  int64_t l = r - b * a.L;
  const int64_t db = step / a.L;
  const int64_t dl = step - db * a.L;

  bool ok[U];
  int64_t off[U];
  float tv[U][V];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = c * kWave * U + (int64_t)u * kWave + lane;
    ok[u] = v < nvec;
    off[u] = (ok[u] ? v : nvec - 1) * V;
    const float* tr = a.table + m * a.st_m + off[u];
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const f32x4 t = *(reinterpret_cast<const f32x4*>(tr) + q);
#pragma unroll
      for (int i = 0; i < 4; ++i) tv[u][4 * q + i] = t[i];
    }
  }
  const T* temb = static_cast<const T*>(a.temb);
  float* out_m = a.out + m * a.R * a.D;
  while (true) {
    const T* er = temb + b * a.se_b + l * a.se_l + m * a.se_m;
    float e[U][V];
#pragma unroll
    for (int u = 0; u < U; ++u) loadv<V>(er + off[u], e[u]);
    float* orow = out_m + r * a.D;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) {
        float s[V];
#pragma unroll
        for (int i = 0; i < V; ++i) s[i] = tv[u][i] + e[u][i];  // table + float(temb)
        storev<V>(orow + off[u], s);
      }
    }
    r += step;
    if (r >= a.R) break;
    l += dl;
    b += db;
    if (l >= a.L) {
      l -= a.L;
      ++b;
    }
  }
}

// One-shot grid: block b covers vectors [c*256*U, (c+1)*256*U) of row r of
// slice m, with b = (m * R + r) * bpr + c, so blocks write each slice in
// address order; thread t takes vectors c*256*U + u*256 + t.
template <typename T, int V, int U>
__global__ __launch_bounds__(256) void temb_flat(TembArgs a, int bpr) {
  const uint32_t rc = blockIdx.x;
  const uint32_t q = rc / (uint32_t)bpr;  // m * R + r
  const int c = (int)(rc - q * (uint32_t)bpr);
  const int64_t m = q / (uint32_t)a.R;
  const int64_t r = q - m * a.R;
  const int64_t b = r / a.L;
  const int64_t l = r - b * a.L;
  const int64_t nvec = a.D / V;  // 64-bit: rows may exceed 2^31 elements
  const T* er = static_cast<const T*>(a.temb) + b * a.se_b + l * a.se_l + m * a.se_m;
  const float* tr = a.table + m * a.st_m;
  float* orow = a.out + (m * a.R + r) * a.D;
  float e[U][V];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)c * 256 * U + u * 256 + (int)threadIdx.x;
    ok[u] = v < nvec;
    if (ok[u]) loadv<V>(er + v * V, e[u]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)c * 256 * U + u * 256 + (int)threadIdx.x;
    if (ok[u]) {
      float s[V];
#pragma unroll
      for (int q4 = 0; q4 < V / 4; ++q4) {
        const f32x4 t = *(reinterpret_cast<const f32x4*>(tr + v * V) + q4);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[4 * q4 + i] = t[i] + e[u][4 * q4 + i];  // table + float(temb)
      }
      storev<V>(orow + v * V, s);
    }
  }
}

// any D, any alignment: one element per lane step
template <typename T>
__global__ __launch_bounds__(256) void temb_scalar(TembArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const T* temb = static_cast<const T*>(a.temb);
  const int64_t rows = a.R * a.nmod;
  for (int64_t q = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); q < rows;
       q += (int64_t)gridDim.x * kRowsPerBlock) {
    const int64_t m = q / a.R;
    const int64_t r = q - m * a.R;
    const int64_t b = r / a.L;
    const int64_t l = r - b * a.L;
    const T* er = temb + b * a.se_b + l * a.se_l + m * a.se_m;
    const float* tr = a.table + m * a.st_m;
    float* orow = a.out + (m * a.R + r) * a.D;
    for (int64_t j = lane; j < a.D; j += kWave) {
      float e;
      if constexpr (sizeof(T) == 2)
        e = u16_f32(er[j]);
      else
        e = er[j];
      orow[j] = tr[j] + e;
    }
  }
}

// grid size (blocks per compute unit in total) and vectors per lane in a
// chunk, measured on MI355X; overridable at build time
#ifndef ADALN_TEMB_BLOCKS_PER_CU
#define ADALN_TEMB_BLOCKS_PER_CU 16
#endif
#ifndef ADALN_TEMB_MAX_U
#define ADALN_TEMB_MAX_U 4
#endif
#ifndef ADALN_TEMB_V
#define ADALN_TEMB_V 4
#endif
constexpr int kTembBlocksPerCu = ADALN_TEMB_BLOCKS_PER_CU;

template <typename T, int U>
int launch_temb(const TembArgs& a, hipStream_t st) {
  constexpr int V = ADALN_TEMB_V;
  const int64_t nvec = a.D / V;
  const int64_t nchunks = (nvec + kWave * U - 1) / (kWave * U);
  const int64_t gy = nchunks * a.nmod;
  const int cus = cu_count();
  const int64_t target = (int64_t)kTembBlocksPerCu * (cus > 0 ? cus : 256);
  int64_t gx = (target + gy - 1) / gy;
  gx = std::max<int64_t>(1, std::min<int64_t>(gx, (a.R + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((temb_chunks<T, V, U>), dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st, a,
                     (int)nchunks);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <typename T, int U>
int launch_temb_flat(const TembArgs& a, hipStream_t st) {
  constexpr int V = ADALN_TEMB_V;
  const int64_t bpr = (a.D / V + 256 * U - 1) / (256 * U);
  hipLaunchKernelGGL((temb_flat<T, V, U>), dim3((unsigned)(a.nmod * a.R * bpr)), dim3(256), 0, st, a, (int)bpr);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <typename T>
int dispatch_temb(const TembArgs& a, hipStream_t st) {
  // one-shot grid (measured 12 % faster than the column chunks at (1,109120,6,3072)): a
  // block takes a whole row of up to 1024 vectors, longer rows go in 256-vector blocks
  const int64_t nvec = a.D / ADALN_TEMB_V;
  const int64_t per_thread = nvec <= 1024 ? (nvec + 255) / 256 : 1;
  const int64_t bpr = (nvec + 256 * per_thread - 1) / (256 * per_thread);
  if (a.nmod * a.R * bpr < ((int64_t)1 << 24)) {
    switch (per_thread) {
      case 1: return launch_temb_flat<T, 1>(a, st);
      case 2: return launch_temb_flat<T, 2>(a, st);
      case 3: return launch_temb_flat<T, 3>(a, st);
      default: return launch_temb_flat<T, 4>(a, st);
    }
  }
  const int64_t per_lane = (a.D / ADALN_TEMB_V + kWave - 1) / kWave;
  switch (std::min<int64_t>(per_lane, ADALN_TEMB_MAX_U)) {
    case 1: return launch_temb<T, 1>(a, st);
#if ADALN_TEMB_MAX_U >= 2
    case 2: return launch_temb<T, 2>(a, st);
#endif
#if ADALN_TEMB_MAX_U >= 3
    case 3: return launch_temb<T, 3>(a, st);
#endif
#if ADALN_TEMB_MAX_U > 4
    case 4: return launch_temb<T, 4>(a, st);
    case 5: return launch_temb<T, 5>(a, st);
    case 6: return launch_temb<T, 6>(a, st);
    case 7: return launch_temb<T, 7>(a, st);
    default: return launch_temb<T, 8>(a, st);
#elif ADALN_TEMB_MAX_U == 4
    default: return launch_temb<T, 4>(a, st);
#elif ADALN_TEMB_MAX_U == 3
    default: return launch_temb<T, 3>(a, st);
#elif ADALN_TEMB_MAX_U == 2
    default: return launch_temb<T, 2>(a, st);
#else
    default: return launch_temb<T, 1>(a, st);
#endif
  }
}

}  // namespace

static int temb_check_shape(int64_t B, int64_t L, int64_t nmod, int64_t D, int64_t st_m, int64_t se_b,
                            int64_t se_l, int64_t se_m, int dtype) {
  if (dtype != ADALN_BF16 && dtype != ADALN_F32) return ADALN_ERR_DTYPE;
  if (B < 0 || L < 0 || nmod < 0 || D < 0) return ADALN_ERR_SHAPE;
  if (st_m < 0 || se_b < 0 || se_l < 0 || se_m < 0) return ADALN_ERR_STRIDE;
  int64_t R, RM, RMD;
  if (!mul_ok(B, L, &R) || !mul_ok(R, nmod, &RM) || !mul_ok(RM, D, &RMD) || RMD > kMaxElems)
    return ADALN_ERR_TOO_LARGE;
  if (!extent_ok({{nmod, st_m}, {D, 1}}) || !extent_ok({{B, se_b}, {L, se_l}, {nmod, se_m}, {D, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

}  // namespace adaln

using namespace adaln;

extern "C" int temb_table_slices_can_use(int64_t B, int64_t L, int64_t nmod, int64_t D, int64_t st_m,
                                         int64_t se_b, int64_t se_l, int64_t se_m, int dtype) {
  return temb_check_shape(B, L, nmod, D, st_m, se_b, se_l, se_m, dtype) == ADALN_OK;
}

extern "C" int temb_table_slices(const float* table, int64_t st_m, const void* temb, int64_t se_b,
                                 int64_t se_l, int64_t se_m, int64_t B, int64_t L, int64_t nmod, int64_t D,
                                 int dtype, float* out, void* stream) {
  int rc = temb_check_shape(B, L, nmod, D, st_m, se_b, se_l, se_m, dtype);
  if (rc != ADALN_OK) return rc;
  const int64_t R = B * L;
  if (R == 0 || nmod == 0 || D == 0) return ADALN_OK;
  if (!table || !temb || !out) return ADALN_ERR_NULL;
  const size_t esz = dtype == ADALN_F32 ? 4 : 2;
  if (!aligned(table, 4) || !aligned(temb, esz) || !aligned(out, 4)) return ADALN_ERR_ALIGN;

  const Span so = span_of(out, {{nmod * R * D, 1}}, 4);
  const Span st = span_of(table, {{nmod, st_m}, {D, 1}}, 4);
  const Span se = span_of(temb, {{B, se_b}, {L, se_l}, {nmod, se_m}, {D, 1}}, esz);
  if (overlaps(so, st) || overlaps(so, se)) return ADALN_ERR_ALIAS;

  TembArgs a;
  a.table = table;
  a.st_m = st_m;
  a.temb = temb;
  a.se_b = se_b;
  a.se_l = se_l;
  a.se_m = se_m;
  a.L = L;
  a.nmod = nmod;
  a.D = D;
  a.R = R;
  a.out = out;
  hipStream_t s = (hipStream_t)stream;
  // vector path: runs of V elements; temb rows aligned to a run of temb
  // (V * esz bytes), table and out rows to 16 bytes; grid.y = nmod * chunks
  // within limits
  constexpr int64_t V = ADALN_TEMB_V;
  const uintptr_t tb = (uintptr_t)(V * esz) < 16 ? (uintptr_t)(V * esz) : 16;
  auto ok_stride = [&](int64_t n, int64_t stv, size_t sz, uintptr_t al) {
    return n <= 1 || ((uintptr_t)stv * sz) % al == 0;
  };
  const int64_t nchunks_max = (D / V + kWave - 1) / kWave;
  const bool vec = D % V == 0 && aligned(table, 16) && aligned(temb, tb) && aligned(out, 16) &&
                   ok_stride(nmod, st_m, 4, 16) && ok_stride(B, se_b, esz, tb) && ok_stride(L, se_l, esz, tb) &&
                   ok_stride(nmod, se_m, esz, tb) && nchunks_max * nmod <= 65535 && nmod <= INT32_MAX;
  if (vec) return dtype == ADALN_F32 ? dispatch_temb<float>(a, s) : dispatch_temb<uint16_t>(a, s);
  const int64_t blocks = std::min<int64_t>((R * nmod + kRowsPerBlock - 1) / kRowsPerBlock, kMaxBlocks);
  if (dtype == ADALN_F32)
    hipLaunchKernelGGL(temb_scalar<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(temb_scalar<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}
