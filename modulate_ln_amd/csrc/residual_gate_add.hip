// residual_gate_add: out = bf16(residual + bf16(gate * update)) on gfx950.
//
// Operation: "Fused Kernels" page, table "adaLN modulation and gating"
// (residual_gate_add replaces residual + gate * update, bit-exact); prhub
// report on sglang PR #34008, 实现拆解 §2-3 (GLM-Image ff-gate sites).  The
// eager chain is two bf16 ops (a multiply, then an add), so the product is
// rounded to bf16 before the add.
//
// Design: pure streaming (2 reads + 1 write per element).  Large
// vector-aligned problems take a one-shot grid (each thread two vectors,
// output written in address order); smaller ones the column-chunk kernel: wave w of chunk c owns vectors
// c*64*U + lane + 64*u (u < U) of every row it visits (rows w, w + W, ...),
// keeps that chunk of the current sample's gate in VGPRs, and issues all
// 2*U residual/update loads of a row (non-temporal, unguarded) before it
// computes; when each wave visits only a few rows, the next row's loads are
// in flight while the current row is computed.  Other layouts take an
// element-wise kernel.

#include "device_common.hpp"
#include "host_common.hpp"

namespace adaln {
namespace {

struct RgaArgs {
  const uint16_t* res;
  int64_t sr_b, sr_s;
  const uint16_t* gate;
  int64_t sg_b;
  const uint16_t* upd;
  int64_t su_b, su_s;
  int64_t S, D, R;
  uint16_t* out;
};

template <int V>
__device__ __forceinline__ Vec<V> gate_add_vec(const Vec<V>& rv, const Vec<V>& gv, const Vec<V>& uv) {
  Vec<V> o;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    float t0 = lo_f32(gv.w[i]) * lo_f32(uv.w[i]);
    float t1 = hi_f32(gv.w[i]) * hi_f32(uv.w[i]);
    round_pair(t0, t1);  // bf16(gate * update)
    o.w[i] = pack_bf16(lo_f32(rv.w[i]) + t0, hi_f32(rv.w[i]) + t1);  // bf16(residual + t)
  }
  return o;
}

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxBlocks = (int64_t)1 << 20;

// Whether the new residual is stored non-temporally (measured faster on
// MI355X, also when the next LayerNorm of the chain reads it right away).
#ifndef ADALN_RGA_NT_STORE
#define ADALN_RGA_NT_STORE 1
#endif

// Column-chunk streaming kernel (vector-aligned rows, unit element stride).
template <int V, int U>
__global__ __launch_bounds__(256) void rga_chunks(RgaArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nvec = a.D / V;
  const int64_t step = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + wave;
  if (r >= a.R) return;
  int64_t b = r / a.S;
  int64_t s = r - b * a.S;
  const int64_t db = step / a.S;
  const int64_t ds = step - db * a.S;

  bool ok[U];
  int64_t off[U];  // element offset of the lane's u-th vector (clamped in-bounds)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)blockIdx.y * kWave * U + (int64_t)u * kWave + lane;
    ok[u] = v < nvec;
    off[u] = (ok[u] ? v : nvec - 1) * V;
  }
  int64_t cached_b = -1;
  Vec<V> gv[U];
  while (true) {
    if (b != cached_b) {
      const uint16_t* gr = a.gate + b * a.sg_b;
#pragma unroll
      for (int u = 0; u < U; ++u) gv[u] = load_vec<V>(gr + off[u]);
      cached_b = b;
    }
    const uint16_t* rr = a.res + b * a.sr_b + s * a.sr_s;
    const uint16_t* ur = a.upd + b * a.su_b + s * a.su_s;
    Vec<V> rv[U], uv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      rv[u] = load_vec_nt<V>(rr + off[u]);
      uv[u] = load_vec_nt<V>(ur + off[u]);
    }
    uint16_t* orow = a.out + r * a.D;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) {
        if constexpr (ADALN_RGA_NT_STORE)
          store_vec_nt<V>(orow + off[u], gate_add_vec<V>(rv[u], gv[u], uv[u]));
        else
          store_vec<V>(orow + off[u], gate_add_vec<V>(rv[u], gv[u], uv[u]));
      }
    r += step;
    if (r >= a.R) break;
    s += ds;
    b += db;
    if (s >= a.S) {
      s -= a.S;
      ++b;
    }
  }
}

// The column-chunk kernel with the next row's residual and update loads in
// flight while the current row is computed and stored (two row buffers).
template <int V, int U>
struct RgaRow {
  Vec<V> r[U], u[U];
};

template <int V, int U>
__global__ __launch_bounds__(256) void rga_chunks_pf(RgaArgs a) {
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
  auto load_row = [&](RgaRow<V, U>& row, int64_t rr) {
    const int64_t b = rr / a.S;
    const int64_t s = rr - b * a.S;
    const uint16_t* res = a.res + b * a.sr_b + s * a.sr_s;
    const uint16_t* upd = a.upd + b * a.su_b + s * a.su_s;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      row.r[u] = load_vec_nt<V>(res + off[u]);
      row.u[u] = load_vec_nt<V>(upd + off[u]);
    }
  };
  int64_t cached_b = -1;
  Vec<V> gv[U];
  auto process = [&](const RgaRow<V, U>& row, int64_t rr) {
    const int64_t b = rr / a.S;
    if (b != cached_b) {
      const uint16_t* gr = a.gate + b * a.sg_b;
#pragma unroll
      for (int u = 0; u < U; ++u) gv[u] = load_vec<V>(gr + off[u]);
      cached_b = b;
    }
    uint16_t* orow = a.out + rr * a.D;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) {
        if constexpr (ADALN_RGA_NT_STORE)
          store_vec_nt<V>(orow + off[u], gate_add_vec<V>(row.r[u], gv[u], row.u[u]));
        else
          store_vec<V>(orow + off[u], gate_add_vec<V>(row.r[u], gv[u], row.u[u]));
      }
  };
  RgaRow<V, U> bufA, bufB;
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
// r = b / bpr (c = b % bpr); thread t takes vectors c*256*U + u*256 + t,
// loads residual and update (non-temporal) and the gate (cached), stores
// and exits, so the output is written in address order.
template <int V, int U>
__global__ __launch_bounds__(256) void rga_flat(RgaArgs a, int bpr) {
  const int64_t r = blockIdx.x / bpr;
  const int c = blockIdx.x - (int)r * bpr;
  const int64_t b = r / a.S;
  const int64_t s = r - b * a.S;
  const int64_t nvec = a.D / V;  // 64-bit: rows may exceed 2^31 elements
  const uint16_t* rr = a.res + b * a.sr_b + s * a.sr_s;
  const uint16_t* ur = a.upd + b * a.su_b + s * a.su_s;
  const uint16_t* gr = a.gate + b * a.sg_b;
  uint16_t* orow = a.out + r * a.D;
  Vec<V> rv[U], uv[U], gv[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)c * 256 * U + u * 256 + (int)threadIdx.x;
    ok[u] = v < nvec;
    if (ok[u]) {
      rv[u] = load_vec_nt<V>(rr + v * V);
      uv[u] = load_vec_nt<V>(ur + v * V);
      gv[u] = load_vec<V>(gr + v * V);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t v = (int64_t)c * 256 * U + u * 256 + (int)threadIdx.x;
    if (ok[u]) {
      const Vec<V> o = gate_add_vec<V>(rv[u], gv[u], uv[u]);
      if constexpr (ADALN_RGA_NT_STORE)
        store_vec_nt<V>(orow + v * V, o);
      else
        store_vec<V>(orow + v * V, o);
    }
  }
}

__global__ __launch_bounds__(256) void rga_rows_scalar(RgaArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < a.R;
       r += (int64_t)gridDim.x * kRowsPerBlock) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* rr = a.res + b * a.sr_b + s * a.sr_s;
    const uint16_t* ur = a.upd + b * a.su_b + s * a.su_s;
    const uint16_t* gr = a.gate + b * a.sg_b;
    uint16_t* orow = a.out + r * a.D;
    for (int64_t j = lane; j < a.D; j += kWave) {
      float t = u16_f32(gr[j]) * u16_f32(ur[j]);
      float tr = u16_f32(to_bf16(t));
      orow[j] = to_bf16(u16_f32(rr[j]) + tr);
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
#define ADALN_CHUNK_BLOCKS_PER_CU 2
#endif
// the prefetching kernel for grids whose waves visit at most this many rows
// (measured on MI355X: (1,4096,4096) 19.6 -> 17.5 us, (2,1024,2240) 7.4 ->
// 6.4 us; (4,4096,3072), 8 rows per wave, is 4 % faster without)
#ifndef ADALN_RGA_PREFETCH_MAX_ROWS
#define ADALN_RGA_PREFETCH_MAX_ROWS 4
#endif
#ifndef ADALN_RGA_MAX_U
#define ADALN_RGA_MAX_U 8
#endif
constexpr int kChunkBlocksPerCu = ADALN_CHUNK_BLOCKS_PER_CU;

template <int V, int U>
int launch_chunks(const RgaArgs& a, hipStream_t st) {
  const int64_t nvec = a.D / V;
  const int64_t nchunks = (nvec + kWave * U - 1) / (kWave * U);
  if (nchunks > 65535) {  // grid.y limit: rows of more than 2^25 vectors go element-wise
    hipLaunchKernelGGL(rga_rows_scalar, dim3(grid_for(a.R)), dim3(256), 0, st, a);
    return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
  }
  const int cus = cu_count();
  const int64_t target = (int64_t)kChunkBlocksPerCu * (cus > 0 ? cus : 256);
  int64_t gx = (target + nchunks - 1) / nchunks;
  gx = std::max<int64_t>(1, std::min<int64_t>(gx, (a.R + kRowsPerBlock - 1) / kRowsPerBlock));
  const int64_t rows_per_wave = (a.R + gx * kRowsPerBlock - 1) / (gx * kRowsPerBlock);
  if (rows_per_wave <= ADALN_RGA_PREFETCH_MAX_ROWS)
    hipLaunchKernelGGL((rga_chunks_pf<V, U>), dim3((unsigned)gx, (unsigned)nchunks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((rga_chunks<V, U>), dim3((unsigned)gx, (unsigned)nchunks), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

// The one-shot grid (two vectors per thread) for problems from 2^25
// elements on, measured on MI355X: (4,4096,3072) 50.5 -> 48.2 us; smaller
// ones keep the column chunks ((1,4096,4096) 17.8 us vs 17.9-18.1 flat).
#ifndef ADALN_RGA_FLAT_U
#define ADALN_RGA_FLAT_U 2
#endif
#ifndef ADALN_RGA_FLAT_MIN_ELEMS
#define ADALN_RGA_FLAT_MIN_ELEMS ((int64_t)1 << 25)
#endif

// vectors per lane in one chunk: as many as a row needs, at most 8
template <int V>
int dispatch_chunks(const RgaArgs& a, hipStream_t st) {
  if constexpr (ADALN_RGA_FLAT_U > 0) {
    constexpr int U = ADALN_RGA_FLAT_U;
    const int64_t bpr = (a.D / V + 256 * U - 1) / (256 * U);
    if (a.R * a.D >= ADALN_RGA_FLAT_MIN_ELEMS && a.R * bpr < ((int64_t)1 << 24)) {
      hipLaunchKernelGGL((rga_flat<V, U>), dim3((unsigned)(a.R * bpr)), dim3(256), 0, st, a, (int)bpr);
      return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
    }
  }
  const int64_t per_lane = (a.D / V + kWave - 1) / kWave;
  switch (std::min<int64_t>(per_lane, ADALN_RGA_MAX_U)) {
    case 1: return launch_chunks<V, 1>(a, st);
    case 2: return launch_chunks<V, 2>(a, st);
    case 3: return launch_chunks<V, 3>(a, st);
#if ADALN_RGA_MAX_U > 4
    case 4: return launch_chunks<V, 4>(a, st);
    case 5: return launch_chunks<V, 5>(a, st);
    case 6: return launch_chunks<V, 6>(a, st);
    case 7: return launch_chunks<V, 7>(a, st);
    default: return launch_chunks<V, 8>(a, st);
#else
    default: return launch_chunks<V, 4>(a, st);
#endif
  }
}

}  // namespace

static int rga_check_shape(int64_t B, int64_t S, int64_t D, int64_t sr_b, int64_t sr_s,
                           int64_t sg_b, int64_t su_b, int64_t su_s, int dtype) {
  if (dtype != ADALN_BF16) return ADALN_ERR_DTYPE;
  if (B < 0 || S < 0 || D < 0) return ADALN_ERR_SHAPE;
  if (sr_b < 0 || sr_s < 0 || sg_b < 0 || su_b < 0 || su_s < 0) return ADALN_ERR_STRIDE;
  int64_t R, RD;
  if (!mul_ok(B, S, &R) || !mul_ok(R, D, &RD)) return ADALN_ERR_TOO_LARGE;
  if (!extent_ok({{B, sr_b}, {S, sr_s}, {D, 1}}) || !extent_ok({{B, su_b}, {S, su_s}, {D, 1}}) ||
      !extent_ok({{B, sg_b}, {D, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

}  // namespace adaln

using namespace adaln;

extern "C" int residual_gate_add_can_use(int64_t B, int64_t S, int64_t D, int64_t sr_b,
                                         int64_t sr_s, int64_t sg_b, int64_t su_b, int64_t su_s,
                                         int dtype) {
  return rga_check_shape(B, S, D, sr_b, sr_s, sg_b, su_b, su_s, dtype) == ADALN_OK;
}

extern "C" int residual_gate_add(const void* residual, int64_t sr_b, int64_t sr_s, const void* gate,
                                 int64_t sg_b, const void* update, int64_t su_b, int64_t su_s,
                                 int64_t B, int64_t S, int64_t D, int dtype, void* out,
                                 void* stream) {
  int rc = rga_check_shape(B, S, D, sr_b, sr_s, sg_b, su_b, su_s, dtype);
  if (rc != ADALN_OK) return rc;
  const int64_t R = B * S;
  if (R == 0 || D == 0) return ADALN_OK;
  if (!residual || !gate || !update || !out) return ADALN_ERR_NULL;
  if (!aligned(residual, 2) || !aligned(gate, 2) || !aligned(update, 2) || !aligned(out, 2))
    return ADALN_ERR_ALIGN;

  const Span so = span_of(out, {{R * D, 1}});
  const Span sres = span_of(residual, {{B, sr_b}, {S, sr_s}, {D, 1}});
  const Span supd = span_of(update, {{B, su_b}, {S, su_s}, {D, 1}});
  const Span sg = span_of(gate, {{B, sg_b}, {D, 1}});
  auto contig = [&](int64_t sb, int64_t ss) {
    return (S == 1 || ss == D) && (B == 1 || sb == S * D);
  };
  if (overlaps(so, sres) && !(residual == out && contig(sr_b, sr_s))) return ADALN_ERR_ALIAS;
  if (overlaps(so, supd) && !(update == out && contig(su_b, su_s))) return ADALN_ERR_ALIAS;
  if (overlaps(so, sg)) return ADALN_ERR_ALIAS;

  RgaArgs a;
  a.res = (const uint16_t*)residual;
  a.sr_b = sr_b;
  a.sr_s = sr_s;
  a.gate = (const uint16_t*)gate;
  a.sg_b = sg_b;
  a.upd = (const uint16_t*)update;
  a.su_b = su_b;
  a.su_s = su_s;
  a.S = S;
  a.D = D;
  a.R = R;
  a.out = (uint16_t*)out;

  hipStream_t st = (hipStream_t)stream;
  auto vec_ok = [&](uintptr_t vb) {
    auto so_ = [&](int64_t n, int64_t s) { return n <= 1 || ((uintptr_t)s * 2u) % vb == 0; };
    return D % (int64_t)(vb / 2) == 0 && aligned(residual, vb) && aligned(update, vb) &&
           aligned(gate, vb) && aligned(out, vb) && so_(B, sr_b) && so_(S, sr_s) && so_(B, su_b) &&
           so_(S, su_s) && so_(B, sg_b);
  };
  if (vec_ok(16)) return dispatch_chunks<8>(a, st);
  if (vec_ok(8)) return dispatch_chunks<4>(a, st);
  hipLaunchKernelGGL(rga_rows_scalar, dim3(grid_for(R)), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}
