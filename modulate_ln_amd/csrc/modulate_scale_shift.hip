// modulate_scale_shift: out = bf16 chain of x * (1 + scale) + shift on gfx950.
//
// Operation: "Fused Kernels" page, table "adaLN modulation and gating"
// (modulate_scale_shift replaces x * (1 + scale) + shift, bit-exact; LingBot
// World's camera conditioning uses it with one affine row per token).  Three
// eager bf16 ops, so three roundings: one_plus = bf16(1 + scale),
// y = bf16(x * one_plus), out = bf16(y + shift) -- the tail of ln_modulate
// with x in place of the normalized row.
//
// Design: pure streaming.  Per-sample rows of up to 4096 elements take the
// row-per-wave layout of ln_modulate: a block serves one sample, turns its
// bf16(1 + scale) and shift into fp32 tables in LDS behind its waves' first
// row loads, and each wave holds one whole row (every row of the launch in
// flight at once when the grid covers them).  Per-token rows (3 reads + 1
// write per element) and other large per-sample problems take a one-shot
// grid: each thread loads two
// vectors of x (and of the per-token scale and shift rows), computes, stores
// and exits, so the output is written in address order.  Smaller per-sample
// problems take the column-chunk layout of residual_gate_add: wave w of chunk
// c owns vectors c*64*U + lane + 64*u (u < U) of every row it visits, the
// next row's loads in flight while the current row is computed, and keeps
// bf16(1 + scale) and shift of its chunk in fp32 VGPRs while it stays in a
// sample (1 read + 1 write per element).  Streams are non-temporal; the
// per-sample rows come through the caches.
#include "device_common.hpp"
#include "host_common.hpp"
#include "ln_row.hpp"  // build_tables: the per-sample fp32 tables of the norm kernels

namespace adaln {
namespace {

struct ModArgs {
  const uint16_t* x;
  int64_t sx_b, sx_s;
  const uint16_t* scale;
  int64_t ssc_b, ssc_s;
  const uint16_t* shift;
  int64_t ssh_b, ssh_s;
  int64_t S, D, R;
  uint16_t* out;
};

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

// x * o + h with the two roundings, o = bf16(1 + scale) and h = shift in fp32
template <int V>
__device__ __forceinline__ Vec<V> mod_vec(const Vec<V>& xv, const float* o, const float* h) {
  Vec<V> r;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    float y0 = lo_f32(xv.w[i]) * o[2 * i];
    float y1 = hi_f32(xv.w[i]) * o[2 * i + 1];
    round_pair(y0, y1);  // bf16(x * one_plus)
    r.w[i] = pack_bf16(y0 + h[2 * i], y1 + h[2 * i + 1]);  // bf16(y + shift)
  }
  return r;
}

// bf16(1 + scale) and shift of one vector, widened to fp32
template <int V>
__device__ __forceinline__ void mod_rows(const Vec<V>& sv, const Vec<V>& hv, float* o, float* h) {
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    o[2 * i] = 1.0f + lo_f32(sv.w[i]);
    o[2 * i + 1] = 1.0f + hi_f32(sv.w[i]);
    round_pair(o[2 * i], o[2 * i + 1]);  // bf16(1 + scale)
    h[2 * i] = lo_f32(hv.w[i]);
    h[2 * i + 1] = hi_f32(hv.w[i]);
  }
}

// One row step of a wave: the row's x (and, per token, scale and shift)
// vectors of the lane's chunk.
template <int V, int U, bool PER_TOKEN>
struct ModRow {
  Vec<V> x[U];
  Vec<V> sc[PER_TOKEN ? U : 1];
  Vec<V> sh[PER_TOKEN ? U : 1];
};

// Rows r = first, first + step, ... of the chunk; the next row's loads are in
// flight while the current row is computed and stored (two row buffers).
template <int V, int U, bool PER_TOKEN>
__global__ __launch_bounds__(256) void mod_chunks(ModArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nvec = a.D / V;
  const int64_t step = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (r >= a.R) return;

  bool ok[U];
  int64_t off[U];  // element offset of the lane's u-th vector (clamped in-bounds)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)blockIdx.y * kWave * U + (int64_t)u * kWave + lane;
    ok[u] = v < nvec;
    off[u] = (ok[u] ? v : nvec - 1) * V;
  }
  auto load_row = [&](ModRow<V, U, PER_TOKEN>& row, int64_t rr) {
    const int64_t b = rr / a.S;
    const int64_t s = rr - b * a.S;
    const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;
#pragma unroll
    for (int u = 0; u < U; ++u) row.x[u] = load_vec_nt<V>(xr + off[u]);
    if constexpr (PER_TOKEN) {
      const uint16_t* sr = a.scale + b * a.ssc_b + s * a.ssc_s;
      const uint16_t* hr = a.shift + b * a.ssh_b + s * a.ssh_s;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        row.sc[u] = load_vec_nt<V>(sr + off[u]);
        row.sh[u] = load_vec_nt<V>(hr + off[u]);
      }
    }
  };
  int64_t cached_b = -1;
  float o[U][V], h[U][V];
  auto process = [&](const ModRow<V, U, PER_TOKEN>& row, int64_t rr) {
    if constexpr (PER_TOKEN) {
#pragma unroll
      for (int u = 0; u < U; ++u) mod_rows<V>(row.sc[u], row.sh[u], o[u], h[u]);
    } else {
      const int64_t b = rr / a.S;
      if (b != cached_b) {
        const uint16_t* sr = a.scale + b * a.ssc_b;
        const uint16_t* hr = a.shift + b * a.ssh_b;
#pragma unroll
        for (int u = 0; u < U; ++u) mod_rows<V>(load_vec<V>(sr + off[u]), load_vec<V>(hr + off[u]), o[u], h[u]);
        cached_b = b;
      }
    }
    uint16_t* orow = a.out + rr * a.D;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) store_vec_nt<V>(orow + off[u], mod_vec<V>(row.x[u], o[u], h[u]));
  };

  ModRow<V, U, PER_TOKEN> bufA, bufB;
  load_row(bufA, r);
  while (true) {
    int64_t r1 = r + step;
    if (r1 < a.R) load_row(bufB, r1);
    process(bufA, r);
    if (r1 >= a.R) break;
    r = r1;
    r1 = r + step;
    if (r1 < a.R) load_row(bufA, r1);
    process(bufB, r);
    if (r1 >= a.R) break;
    r = r1;
  }
}

// any D, any 2-byte alignment: one element per lane step
// One-shot grid: block b covers vectors [c*256*U, (c+1)*256*U) of row
// b / bpr (c = b % bpr); thread t takes vectors c*256*U + u*256 + t.  The
// per-sample adaLN rows come through the caches; per-token rows stream.
template <int V, int U, bool PER_TOKEN>
__global__ __launch_bounds__(256) void mod_flat(ModArgs a, int bpr) {
  const int64_t r = blockIdx.x / bpr;
  const int c = blockIdx.x - (int)r * bpr;
  const int64_t b = r / a.S;
  const int64_t s = r - b * a.S;
  const int64_t nvec = a.D / V;  // 64-bit: rows may exceed 2^31 elements
  const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;
  const uint16_t* scr = a.scale + b * a.ssc_b + (PER_TOKEN ? s * a.ssc_s : 0);
  const uint16_t* shr = a.shift + b * a.ssh_b + (PER_TOKEN ? s * a.ssh_s : 0);
  uint16_t* orow = a.out + r * a.D;
  Vec<V> xv[U], sv[U], hv[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)c * 256 * U + u * 256 + (int)threadIdx.x;
    ok[u] = v < nvec;
    if (ok[u]) {
      xv[u] = load_vec_nt<V>(xr + v * V);
      if constexpr (PER_TOKEN) {
        sv[u] = load_vec_nt<V>(scr + v * V);
        hv[u] = load_vec_nt<V>(shr + v * V);
      } else {
        sv[u] = load_vec<V>(scr + v * V);
        hv[u] = load_vec<V>(shr + v * V);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)c * 256 * U + u * 256 + (int)threadIdx.x;
    if (ok[u]) {
      float o[V], h[V];
      mod_rows<V>(sv[u], hv[u], o, h);
      store_vec_nt<V>(orow + v * V, mod_vec<V>(xv[u], o, h));
    }
  }
}

// Per-sample rows, one row per wave: block j of sample b builds the tables
// (bf16(1 + scale), shift; [quarter][vector] float4 in LDS) and its wave w
// takes rows s = 4j + w, += 4*bpb, NV 16-byte vectors per lane (lane l owns
// vectors l, l + 64, ...).  UNIF: nvec % 64 == 0.
template <int NV, bool UNIF>
__global__ __launch_bounds__(256) void mod_tab(ModArgs a, int bpb) {
  constexpr int V = 8;
  extern __shared__ float4 tab[];  // [2][V/4][nvec] float4: bf16(1+scale), then shift
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nvec = (int)(a.D / V);
  const int S = (int)a.S;
  const int b = blockIdx.x / bpb;
  const int j = blockIdx.x - b * bpb;
  const int row_step = 4 * bpb;
  const int shift_off = (V / 4) * nvec;
  int s = 4 * j + wave;
  const uint16_t* xb = a.x + (int64_t)b * a.sx_b;
  Vec<V> xv[NV];
  auto load_row = [&](int ss) {
    const uint16_t* xr = xb + (int64_t)ss * a.sx_s;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * kWave + lane;
      xv[k] = load_vec_nt<V>(xr + ((UNIF || v < nvec) ? v : nvec - 1) * V);
    }
  };
  if (s < S) load_row(s);
  build_tables<V>(tab, a.scale + (int64_t)b * a.ssc_b, a.shift + (int64_t)b * a.ssh_b, nvec, threadIdx.x, 256);
  __syncthreads();
  if (s >= S) return;
  while (true) {
    uint16_t* orow = a.out + ((int64_t)b * S + s) * a.D;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * kWave + lane;
      if (UNIF || v < nvec) {
        Vec<V> ov;
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
          const float4 o = tab[q * nvec + v];
          const float4 h = tab[shift_off + q * nvec + v];
          const uint32_t w0 = xv[k].w[2 * q], w1 = xv[k].w[2 * q + 1];
          float y0 = lo_f32(w0) * o.x, y1 = hi_f32(w0) * o.y;
          float y2 = lo_f32(w1) * o.z, y3 = hi_f32(w1) * o.w;
          round_pair(y0, y1);  // bf16(x * one_plus)
          round_pair(y2, y3);
          ov.w[2 * q] = pack_bf16(y0 + h.x, y1 + h.y);  // bf16(y + shift)
          ov.w[2 * q + 1] = pack_bf16(y2 + h.z, y3 + h.w);
        }
        store_vec_nt<V>(orow + v * V, ov);
      }
      // one step's table values live at a time: hoisting every step's LDS
      // reads took 167 VGPRs at 8 steps (3 waves per SIMD), 60 with this
      __builtin_amdgcn_sched_barrier(0);
    }
    s += row_step;
    if (s >= S) break;
    load_row(s);
  }
}

__global__ __launch_bounds__(256) void mod_rows_scalar(ModArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < a.R;
       r += (int64_t)gridDim.x * kRowsPerBlock) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* xr = a.x + b * a.sx_b + s * a.sx_s;
    const uint16_t* sr = a.scale + b * a.ssc_b + s * a.ssc_s;
    const uint16_t* hr = a.shift + b * a.ssh_b + s * a.ssh_s;
    uint16_t* orow = a.out + r * a.D;
    for (int64_t j = lane; j < a.D; j += kWave) {
      const float o = u16_f32(to_bf16(1.0f + u16_f32(sr[j])));
      const float y = u16_f32(to_bf16(u16_f32(xr[j]) * o));
      orow[j] = to_bf16(y + u16_f32(hr[j]));
    }
  }
}

inline unsigned grid_for(int64_t R) {
  int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  return (unsigned)std::min(blocks, kMaxBlocks);
}

// grid size (blocks per compute unit in total: 4 with per-sample rows, 8
// with per-token rows) and vectors per lane in a chunk, measured on MI355X
// at (1,4096,4096); overridable at build time
#ifndef ADALN_MOD_BLOCKS_PER_CU
#define ADALN_MOD_BLOCKS_PER_CU 4
#endif
#ifndef ADALN_MOD_TOKEN_BLOCKS_PER_CU
#define ADALN_MOD_TOKEN_BLOCKS_PER_CU 8
#endif
#ifndef ADALN_MOD_MAX_U
#define ADALN_MOD_MAX_U 4
#endif

template <int V, int U, bool PER_TOKEN>
int launch_mod(const ModArgs& a, hipStream_t st) {
  const int64_t nvec = a.D / V;
  const int64_t nchunks = (nvec + kWave * U - 1) / (kWave * U);
  if (nchunks > 65535) {  // grid.y limit: rows of more than 2^24 vectors go element-wise
    hipLaunchKernelGGL(mod_rows_scalar, dim3(grid_for(a.R)), dim3(256), 0, st, a);
    return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
  }
  const int cus = cu_count();
  const int64_t per_cu = PER_TOKEN ? ADALN_MOD_TOKEN_BLOCKS_PER_CU : ADALN_MOD_BLOCKS_PER_CU;
  const int64_t target = per_cu * (cus > 0 ? cus : 256);
  int64_t gx = (target + nchunks - 1) / nchunks;
  gx = std::max<int64_t>(1, std::min<int64_t>(gx, (a.R + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((mod_chunks<V, U, PER_TOKEN>), dim3((unsigned)gx, (unsigned)nchunks), dim3(256), 0,
                     st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// vectors per lane in one chunk: as many as a row needs, at most
// ADALN_MOD_MAX_U (the per-sample rows stay in VGPRs as fp32: 2*U*V registers)
// The one-shot grid (two vectors per thread) measured faster on MI355X
// with per-token rows -- (1,4096,4096) 25.0 -> 23.4 us -- and with per-sample
// rows from 2^25 elements on -- (4,4096,3072) 38.4 -> 36.3 us -- but slower
// for smaller per-sample problems ((1,4096,4096) 12.7 -> 14.8 us), where the
// column chunks stay.  Per-sample rows of up to 4096 elements take the
// row-per-wave kernel ahead of both; the others stay here.
#ifndef ADALN_MOD_FLAT_U
#define ADALN_MOD_FLAT_U 2
#endif
#ifndef ADALN_MOD_FLAT_MIN_ELEMS
#define ADALN_MOD_FLAT_MIN_ELEMS ((int64_t)1 << 25)
#endif

// Row-per-wave layout for per-sample rows of up to kModTabMaxNv vectors per
// lane (all sizes: ALL), blocks per compute unit in total, measured on
// MI355X against the chunk and one-shot kernels: (1,4096,4096) 11.5 us
// (12.2 when the kernel held 3 waves per SIMD and took 3 blocks per CU) vs
// 12.55; (4,4096,3072) 35.0 vs 36.2; (4,4096,4096) 45.7 vs 49.5;
// (2,1024,2240) 4.9 vs 6.6.  6 blocks per CU: (1,8192,4096) 25.7 against
// 24.1 at 4.
#ifndef ADALN_MOD_TAB
#define ADALN_MOD_TAB 1
#endif
#ifndef ADALN_MOD_TAB_BPC
#define ADALN_MOD_TAB_BPC 4
#endif
#ifndef ADALN_MOD_TAB_ALL
#define ADALN_MOD_TAB_ALL 1
#endif
constexpr int kModTabMaxNv = 8;  // D <= 4096: 32 KiB of LDS tables per block

template <int NV, bool UNIF>
int launch_mod_tab(const ModArgs& a, hipStream_t st) {
  const int64_t B = a.R / a.S;
  const int cus = cu_count();
  const int64_t ncu = cus > 0 ? cus : 256;
  const int64_t target = (int64_t)ADALN_MOD_TAB_BPC * ncu;
  int64_t bpb = (target + B - 1) / B;
  bpb = std::max<int64_t>(1, std::min<int64_t>(bpb, (a.S + 3) / 4));
  const size_t lds = (size_t)2 * a.D * sizeof(float);
  hipLaunchKernelGGL((mod_tab<NV, UNIF>), dim3((unsigned)(B * bpb)), dim3(256), lds, st, a, (int)bpb);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <bool UNIF>
int dispatch_mod_tab(const ModArgs& a, int nv, hipStream_t st) {
  switch (nv) {
    case 1: return launch_mod_tab<1, UNIF>(a, st);
    case 2: return launch_mod_tab<2, UNIF>(a, st);
    case 3: return launch_mod_tab<3, UNIF>(a, st);
    case 4: return launch_mod_tab<4, UNIF>(a, st);
    case 5: return launch_mod_tab<5, UNIF>(a, st);
    case 6: return launch_mod_tab<6, UNIF>(a, st);
    case 7: return launch_mod_tab<7, UNIF>(a, st);
    default: return launch_mod_tab<8, UNIF>(a, st);
  }
}

template <int V, bool PER_TOKEN>
int dispatch_mod(const ModArgs& a, hipStream_t st) {
  if constexpr (V == 8 && !PER_TOKEN && ADALN_MOD_TAB) {
    const int64_t nvec = a.D / V;
    const int64_t nv = (nvec + kWave - 1) / kWave;
    // the grid is B * bpb blocks with bpb <= S/4: sizes that fit an int index
    if (nv <= kModTabMaxNv && a.S < ((int64_t)1 << 30) && a.R / a.S < ((int64_t)1 << 20) &&
        (ADALN_MOD_TAB_ALL || a.R * a.D < ADALN_MOD_FLAT_MIN_ELEMS))
      return nvec % kWave == 0 ? dispatch_mod_tab<true>(a, (int)nv, st) : dispatch_mod_tab<false>(a, (int)nv, st);
  }
  if constexpr (ADALN_MOD_FLAT_U > 0) {
    constexpr int U = ADALN_MOD_FLAT_U;
    const int64_t bpr = (a.D / V + 256 * U - 1) / (256 * U);
    if ((PER_TOKEN || a.R * a.D >= ADALN_MOD_FLAT_MIN_ELEMS) && a.R * bpr < ((int64_t)1 << 24)) {
      hipLaunchKernelGGL((mod_flat<V, U, PER_TOKEN>), dim3((unsigned)(a.R * bpr)), dim3(256), 0, st, a, (int)bpr);
      return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
    }
  }
  const int64_t per_lane = (a.D / V + kWave - 1) / kWave;
  switch (std::min<int64_t>(per_lane, ADALN_MOD_MAX_U)) {
    case 1: return launch_mod<V, 1, PER_TOKEN>(a, st);
    case 2: return launch_mod<V, 2, PER_TOKEN>(a, st);
    case 3: return launch_mod<V, 3, PER_TOKEN>(a, st);
#if ADALN_MOD_MAX_U > 4
    case 4: return launch_mod<V, 4, PER_TOKEN>(a, st);
    case 5: return launch_mod<V, 5, PER_TOKEN>(a, st);
    case 6: return launch_mod<V, 6, PER_TOKEN>(a, st);
    case 7: return launch_mod<V, 7, PER_TOKEN>(a, st);
    default: return launch_mod<V, 8, PER_TOKEN>(a, st);
#else
    default: return launch_mod<V, 4, PER_TOKEN>(a, st);
#endif
  }
}

}  // namespace

static int mod_check_shape(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s, int64_t ssc_b,
                           int64_t ssc_s, int64_t ssh_b, int64_t ssh_s, int dtype) {
  if (dtype != ADALN_BF16) return ADALN_ERR_DTYPE;
  if (B < 0 || S < 0 || D < 0) return ADALN_ERR_SHAPE;
  if (sx_b < 0 || sx_s < 0 || ssc_b < 0 || ssc_s < 0 || ssh_b < 0 || ssh_s < 0) return ADALN_ERR_STRIDE;
  int64_t R, RD;
  if (!mul_ok(B, S, &R) || !mul_ok(R, D, &RD)) return ADALN_ERR_TOO_LARGE;
  if (!extent_ok({{B, sx_b}, {S, sx_s}, {D, 1}}) || !extent_ok({{B, ssc_b}, {S, ssc_s}, {D, 1}}) ||
      !extent_ok({{B, ssh_b}, {S, ssh_s}, {D, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

}  // namespace adaln

using namespace adaln;

extern "C" int modulate_scale_shift_can_use(int64_t B, int64_t S, int64_t D, int64_t sx_b, int64_t sx_s,
                                            int64_t ssc_b, int64_t ssc_s, int64_t ssh_b, int64_t ssh_s,
                                            int dtype) {
  return mod_check_shape(B, S, D, sx_b, sx_s, ssc_b, ssc_s, ssh_b, ssh_s, dtype) == ADALN_OK;
}

extern "C" int modulate_scale_shift(const void* x, int64_t sx_b, int64_t sx_s, const void* scale,
                                    int64_t ssc_b, int64_t ssc_s, const void* shift, int64_t ssh_b,
                                    int64_t ssh_s, int64_t B, int64_t S, int64_t D, int dtype, void* out,
                                    void* stream) {
  int rc = mod_check_shape(B, S, D, sx_b, sx_s, ssc_b, ssc_s, ssh_b, ssh_s, dtype);
  if (rc != ADALN_OK) return rc;
  const int64_t R = B * S;
  if (R == 0 || D == 0) return ADALN_OK;
  if (!x || !scale || !shift || !out) return ADALN_ERR_NULL;
  if (!aligned(x, 2) || !aligned(scale, 2) || !aligned(shift, 2) || !aligned(out, 2)) return ADALN_ERR_ALIGN;

  const Span so = span_of(out, {{R * D, 1}});
  const Span sx = span_of(x, {{B, sx_b}, {S, sx_s}, {D, 1}});
  const Span ssc = span_of(scale, {{B, ssc_b}, {S, ssc_s}, {D, 1}});
  const Span ssh = span_of(shift, {{B, ssh_b}, {S, ssh_s}, {D, 1}});
  const bool x_contig = (S == 1 || sx_s == D) && (B == 1 || sx_b == S * D);
  if (overlaps(so, sx) && !(x == out && x_contig)) return ADALN_ERR_ALIAS;
  if (overlaps(so, ssc) || overlaps(so, ssh)) return ADALN_ERR_ALIAS;

  ModArgs a;
  a.x = (const uint16_t*)x;
  a.sx_b = sx_b;
  a.sx_s = sx_s;
  a.scale = (const uint16_t*)scale;
  a.ssc_b = ssc_b;
  a.ssc_s = ssc_s;
  a.shift = (const uint16_t*)shift;
  a.ssh_b = ssh_b;
  a.ssh_s = ssh_s;
  a.S = S;
  a.D = D;
  a.R = R;
  a.out = (uint16_t*)out;
  const bool per_token = S > 1 && (ssc_s != 0 || ssh_s != 0);

  hipStream_t st = (hipStream_t)stream;
  auto vec_ok = [&](uintptr_t vb) {
    auto so_ = [&](int64_t n, int64_t s) { return n <= 1 || ((uintptr_t)s * 2u) % vb == 0; };
    return D % (int64_t)(vb / 2) == 0 && aligned(x, vb) && aligned(scale, vb) && aligned(shift, vb) &&
           aligned(out, vb) && so_(B, sx_b) && so_(S, sx_s) && so_(B, ssc_b) && so_(S, ssc_s) &&
           so_(B, ssh_b) && so_(S, ssh_s);
  };
  if (vec_ok(16)) return per_token ? dispatch_mod<8, true>(a, st) : dispatch_mod<8, false>(a, st);
  if (vec_ok(8)) return per_token ? dispatch_mod<4, true>(a, st) : dispatch_mod<4, false>(a, st);
  hipLaunchKernelGGL(mod_rows_scalar, dim3(grid_for(R)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}
