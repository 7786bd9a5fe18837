// residual_gate_add_ln_modulate: the gated residual update followed by
// ln_modulate of the updated residual, in one pass, on gfx950.
//
// Operation: "Fused Kernels" page, table "Normalization"
// (scale_residual_norm_scale_shift: the norm + scale/shift with the
// preceding residual + gate * update folded in).  Both results are written:
//   res_out = bf16(residual + bf16(gate * update))      (two eager ops)
//   out     = bf16 chain of LN(res_out) * (1 + scale) + shift
// with exactly the roundings and the Welford order of the two unfused ops,
// so the results are bit-identical to residual_gate_add then ln_modulate.
//
// Design: the tabled ln_modulate kernel with a gate-add prologue.  A block
// serves one batch sample and holds three fp32 tables in LDS: bf16(1 +
// scale), shift and gate.  Each wave streams rows: it loads the row of
// residual and of update (non-temporal 16-byte loads, issued before the
// tables are built for the first row), forms the new residual in packed
// bf16, stores it, and hands the packed row to the same per-row routine as
// ln_modulate.  Per element: 2 reads + 2 writes of bf16 (8 bytes), against
// 6 + 4 for the two unfused ops, one launch instead of two.
// Rows of more than 4096 elements take W waves per row (rga_ln_modulate_mw)
// when D % 8 == 0.  Rows that are not vector-aligned, and rows of more than
// 4096 elements with D % 8 != 0, run the two unfused entry points back to
// back: same bits, two launches.

#include "device_common.hpp"
#include "host_common.hpp"
#include "ln_row.hpp"
#include "mw_row.hpp"

// the unfused entry points, for the layouts the fused kernel does not take
extern "C" int residual_gate_add(const void* residual, int64_t sr_b, int64_t sr_s, const void* gate,
                                 int64_t sg_b, const void* update, int64_t su_b, int64_t su_s,
                                 int64_t B, int64_t S, int64_t D, int dtype, void* out, void* stream);
extern "C" int ln_modulate(const void* x, int64_t B, int64_t S, int64_t D, int64_t sx_b,
                           int64_t sx_s, int64_t sx_d, const void* scale, int64_t sscale_b,
                           const void* shift, int64_t sshift_b, float eps, int dtype, void* out,
                           float* mean_out, float* rstd_out, void* stream);

namespace adaln {
namespace {

struct FusedArgs {
  const uint16_t* res;
  int64_t sr_b, sr_s;
  const uint16_t* gate;
  int64_t sg_b;
  const uint16_t* upd;
  int64_t su_b, su_s;
  const uint16_t* scale;
  int64_t ssc_b;
  const uint16_t* shift;
  int64_t ssh_b;
  float eps;
  uint16_t* res_out;
  uint16_t* out;
  float* mean_out;
  float* rstd_out;
  int64_t S, D, R;
};

// Launch shape, measured on MI355X (every choice gives the same bits).
// Rows of up to 6 vectors per lane prefetch the next row's residual and
// update into a second pair of buffers; longer rows do not (the VGPRs would
// cut the waves per SIMD).  Rows of up to 8 vectors per lane keep an fp32
// copy of the updated residual for the normalize pass instead of
// re-widening it (24.7 vs 25.0 us at (1,4096,4096); even at (4,4096,3072));
// longer rows re-widen.  Blocks per compute unit: 4, or as many as the
// three tables (12*D bytes of LDS per block) allow.
#ifndef ADALN_FUSED_XF32_MAX
#define ADALN_FUSED_XF32_MAX 8
#endif
#ifndef ADALN_FUSED_PF_MAX
#define ADALN_FUSED_PF_MAX 6
#endif
#ifndef ADALN_FUSED_WPB
#define ADALN_FUSED_WPB 16
#endif
// MANY: more rows than 16-wave blocks hold at one per wave (16 per compute
// unit) keep 4-wave blocks; a second round of 16-wave blocks starts only as
// whole blocks drain.  At D = 4096, 16- vs 4-wave blocks: 4160 rows 33.1 vs
// 27.5 us, 5120 rows 37.7 vs 32.5, 16384 rows 103.5 vs 100.0 (prefetching
// the next row instead: 29.3, 33.6, 99.1).
template <int NV, bool UNIF, bool MANY = false>
struct FusedShape {
  static constexpr bool kPrefetch = NV <= ADALN_FUSED_PF_MAX;
  static constexpr bool kXf32 = NV <= ADALN_FUSED_XF32_MAX;
  static constexpr int kBlocksPerCu = 4;
  // waves per block (one row each): 16 holds every row of a compute unit's
  // share in one block, so the three tables are built once per compute
  // unit ((1,4096,4096): 23.6 us, against 24.7 with 4-wave blocks and 30.6
  // with 12); rows with a partial last vector step or more than 8 vectors
  // per lane keep 4 (their VGPRs would not fit a larger block's budget)
  static constexpr int kWpb = (!MANY && !kPrefetch && UNIF && NV <= 8) ? ADALN_FUSED_WPB : 4;
};

template <int V, int NV, bool UNIF, bool MANY = false>
__global__ __launch_bounds__((FusedShape<NV, UNIF, MANY>::kWpb * 64)) void rga_ln_modulate_tab(FusedArgs a, int bpb) {
  constexpr int kWpb = FusedShape<NV, UNIF, MANY>::kWpb;
  constexpr bool kPrefetch = FusedShape<NV, UNIF, MANY>::kPrefetch;
  constexpr bool kXf32 = FusedShape<NV, UNIF, MANY>::kXf32;
  extern __shared__ float4 tab[];  // [3][V/4][nvec] float4: bf16(1+scale), shift, gate
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int D = (int)a.D;
  const int nvec = D / V;
  const int S = (int)a.S;
  const int b = blockIdx.x / bpb;
  const int j = blockIdx.x - b * bpb;
  const int row_step = kWpb * bpb;
  const int gate_off = 2 * (V / 4) * nvec;
  int s = kWpb * j + wave;

  const uint16_t* rb = a.res + (int64_t)b * a.sr_b;
  const uint16_t* ub = a.upd + (int64_t)b * a.su_b;
  auto load_rows = [&](Vec<V>* rbuf, Vec<V>* ubuf, int ss) {
    const uint16_t* rr = rb + (int64_t)ss * a.sr_s;
    const uint16_t* ur = ub + (int64_t)ss * a.su_s;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * kWave + lane;
      const int vc = (UNIF || v < nvec) ? v : nvec - 1;
      rbuf[k] = load_vec_nt<V>(rr + vc * V);
      ubuf[k] = load_vec_nt<V>(ur + vc * V);
    }
  };

  Vec<V> rA[NV], uA[NV];
  Vec<V> rB[kPrefetch ? NV : 1], uB[kPrefetch ? NV : 1];
  if (s < S) load_rows(rA, uA, s);
  build_tables<V>(tab, a.scale + (int64_t)b * a.ssc_b, a.shift + (int64_t)b * a.ssh_b, nvec,
                  threadIdx.x, kWpb * kWave);
  build_gate_table<V>(tab, a.gate + (int64_t)b * a.sg_b, nvec, threadIdx.x, kWpb * kWave);
  __syncthreads();
  if (s >= S) return;

  const float Df = (float)D;
  auto process = [&](const Vec<V>* rbuf, const Vec<V>* ubuf, int ss) {
    const int64_t r = (int64_t)b * S + ss;
    uint16_t* xrow = a.res_out + r * D;
    Vec<V> xn[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * kWave + lane;
      const int vc = (UNIF || v < nvec) ? v : nvec - 1;
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        const float4 g = tab[gate_off + q * nvec + vc];
        const uint32_t u0 = ubuf[k].w[2 * q], u1 = ubuf[k].w[2 * q + 1];
        const uint32_t r0 = rbuf[k].w[2 * q], r1 = rbuf[k].w[2 * q + 1];
        float t0 = g.x * lo_f32(u0), t1 = g.y * hi_f32(u0);
        float t2 = g.z * lo_f32(u1), t3 = g.w * hi_f32(u1);
        round_pair(t0, t1);  // bf16(gate * update)
        round_pair(t2, t3);
        xn[k].w[2 * q] = pack_bf16(lo_f32(r0) + t0, hi_f32(r0) + t1);  // bf16(residual + t)
        xn[k].w[2 * q + 1] = pack_bf16(lo_f32(r1) + t2, hi_f32(r1) + t3);
      }
      if (UNIF || v < nvec) store_vec_nt<V>(xrow + v * V, xn[k]);
    }
    __builtin_amdgcn_sched_barrier(0);
    normalize_row<V, NV, UNIF, kXf32>(xn, tab, nvec, lane, Df, a.eps, a.out + r * D,
                                      a.mean_out ? a.mean_out + r : nullptr,
                                      a.rstd_out ? a.rstd_out + r : nullptr);
  };

  if constexpr (kPrefetch) {
    while (true) {
      int s1 = s + row_step;
      if (s1 < S) load_rows(rB, uB, s1);
      process(rA, uA, s);
      if (s1 >= S) break;
      s = s1;
      s1 = s + row_step;
      if (s1 < S) load_rows(rA, uA, s1);
      process(rB, uB, s);
      if (s1 >= S) break;
      s = s1;
    }
  } else {
    while (true) {
      process(rA, uA, s);
      s += row_step;
      if (s >= S) break;
      load_rows(rA, uA, s);
    }
  }
}

// bf16(residual + bf16(gate * update)) for one vector, packed
template <int V>
__device__ __forceinline__ Vec<V> gate_add_vec(const Vec<V>& r, const Vec<V>& u, const Vec<V>& g) {
  Vec<V> x;
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    float t0 = lo_f32(g.w[i]) * lo_f32(u.w[i]), t1 = hi_f32(g.w[i]) * hi_f32(u.w[i]);
    round_pair(t0, t1);  // bf16(gate * update)
    x.w[i] = pack_bf16(lo_f32(r.w[i]) + t0, hi_f32(r.w[i]) + t1);  // bf16(residual + t)
  }
  return x;
}

// Rows of more than 4096 elements: W = 2 .. 16 waves per row, one row per
// block of 64 * W threads at a time (the layout of ln_modulate's long rows):
// each lane forms the new residual of its vectors (at most 64 elements),
// stores it, and the block reduces it in the fixed tree of mw_row.hpp.  The
// per-sample gate, scale and shift rows are read through the caches.
template <int V, int NV, bool UNIF>
__global__ __launch_bounds__(kMaxWaves * 64) void rga_ln_modulate_mw(FusedArgs a) {
  __shared__ MwSlots slots;
  const int W = __builtin_amdgcn_readfirstlane(blockDim.x >> 6);
  const int L = W * kWave;
  const int g = threadIdx.x;
  const int lane = g & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(g >> 6);
  const int nvec = (int)(a.D / V);
  const float Df = (float)a.D;
  int parity = 0;
  for (int64_t r = blockIdx.x; r < a.R; r += gridDim.x, parity ^= 1) {
    const int64_t b = r / a.S;
    const int64_t s = r - b * a.S;
    const uint16_t* rr = a.res + b * a.sr_b + s * a.sr_s;
    const uint16_t* ur = a.upd + b * a.su_b + s * a.su_s;
    const uint16_t* gt = a.gate + b * a.sg_b;
    uint16_t* xrow = a.res_out + r * a.D;
    Vec<V> xn[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (UNIF || k * L < nvec) {  // block-uniform: steps past the row are not loaded
        const int v = k * L + g;
        const int vc = v < nvec ? v : nvec - 1;
        const uint32_t off = (uint32_t)(vc * V);  // 32-bit offsets from scalar row bases
        const Vec<V> rv = load_vec_nt<V>(rr + off);
        const Vec<V> uv = load_vec_nt<V>(ur + off);
        const Vec<V> gv = load_vec<V>(gt + off);
        xn[k] = gate_add_vec<V>(rv, uv, gv);
        if (UNIF || v < nvec) store_vec_nt<V>(xrow + (uint32_t)(v * V), xn[k]);
      }
    }
    float mean, m2;
    mw_stats<V, NV, UNIF, false>(xn, nvec, g, lane, wave, W, slots.s[parity], mean, m2);
    const float rstd = finalize_rstd(m2, Df, a.eps, pow2_inverse_f(Df));
    if (g == 0) {
      if (a.mean_out) a.mean_out[r] = mean;
      if (a.rstd_out) a.rstd_out[r] = rstd;
    }
    const uint16_t* sc = a.scale + b * a.ssc_b;
    const uint16_t* sh = a.shift + b * a.ssh_b;
    uint16_t* orow = a.out + r * a.D;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int v = k * L + g;
      if (UNIF || v < nvec) {
        const Vec<V> sv = load_vec<V>(sc + v * V);
        const Vec<V> hv = load_vec<V>(sh + v * V);
        uint32_t o[V / 2];
        modulate_vec<V, false, kTailChain, true>(xn[k], sv, hv, mean, rstd, o);
        put_vec<V, false, kTailChain>(orow, v, o, 1.0f);
      }
    }
  }
}

// Rows of 4097 .. 16384 elements, P = 16 / W rows of one sample per block of
// 16 waves (group q of W waves takes row s0 + q), the layout of
// ln_modulate_mwt: the sample's tables bf16(1 + scale) and shift are built
// in LDS as fp32 once per block, where rga_ln_modulate_mw fetches the bf16
// rows through the caches and widens and rounds them per element.  The gate
// is needed before the statistics, so it comes through the caches as there.
// Same lanes, merges and values, so the same bits.
template <int NV, bool UNIF, int TPB>
__global__ __launch_bounds__(TPB) void rga_ln_modulate_mwt(FusedArgs a, int bps, int W) {
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
  const int64_t b = blockIdx.x / bps;
  const int64_t s = (int64_t)(blockIdx.x - b * bps) * P + q;
  const bool act = s < a.S;
  const int64_t sr = act ? s : a.S - 1;  // a group past the sample's rows reads its last row
  const int64_t r = b * a.S + sr;

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
  const uint16_t* rr = a.res + b * a.sr_b + sr * a.sr_s;
  const uint16_t* ur = a.upd + b * a.su_b + sr * a.su_s;
  const uint16_t* gt = a.gate + b * a.sg_b;
  uint16_t* xrow = a.res_out + r * a.D;
  Vec<V> xn[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (UNIF || k * L < nvec) {  // wave-uniform: steps past the row are not loaded
      const int v = k * L + g;
      const uint32_t off = (uint32_t)((v < nvec ? v : nvec - 1) * V);  // 32-bit offsets from scalar row bases
      const Vec<V> rv = load_vec_nt<V>(rr + off);
      const Vec<V> uv = load_vec_nt<V>(ur + off);
      const Vec<V> gv = load_vec<V>(gt + off);
      xn[k] = gate_add_vec<V>(rv, uv, gv);
      if (act && (UNIF || v < nvec)) store_vec_nt<V>(xrow + (uint32_t)(v * V), xn[k]);
    }
  }
#pragma unroll
  for (int i = 0; i < kRuns; ++i) {
    const int j = i * TPB + (int)threadIdx.x;
    if (j < nvec) put_tables<V>(tab, ts[i], th[i], j, nvec);
  }
  float mean, m2;
  // the group's slots; the barrier inside also publishes the tables
  mw_stats<V, NV, UNIF, false>(xn, nvec, g, lane, wave - q * W, W, slots.s[0] + q * W, mean, m2);
  if (!act) return;  // no barrier follows
  const float rstd = finalize_rstd(m2, Df, a.eps, pow2_inverse_f(Df));
  if (g == 0) {
    if (a.mean_out) a.mean_out[r] = mean;
    if (a.rstd_out) a.rstd_out[r] = rstd;
  }
  uint16_t* orow = a.out + r * a.D;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = k * L + g;
    if (UNIF || v < nvec) {
      uint32_t o[V / 2];
#pragma unroll
      for (int h = 0; h < V / 4; ++h) {
        const float4 oc = tab[h * nvec + v], hc = tab[(V / 4 + h) * nvec + v];
        const float n0 = (lo_f32_again(xn[k].w[2 * h]) - mean) * rstd;
        const float n1 = (hi_f32_again(xn[k].w[2 * h]) - mean) * rstd;
        const float n2 = (lo_f32_again(xn[k].w[2 * h + 1]) - mean) * rstd;
        const float n3 = (hi_f32_again(xn[k].w[2 * h + 1]) - mean) * rstd;
        o[2 * h] = tail_pair<kTailChain>(n0, n1, oc.x, oc.y, hc.x, hc.y);
        o[2 * h + 1] = tail_pair<kTailChain>(n2, n3, oc.z, oc.w, hc.z, hc.w);
      }
      put_vec<V, false, kTailChain>(orow, v, o, 1.0f);
    }
  }
}

constexpr int64_t kLdsPerCu = 160 * 1024;

template <int V, int NV, bool UNIF, bool MANY = false>
int launch_fused(const FusedArgs& a, hipStream_t st) {
  using Shape = FusedShape<NV, UNIF, MANY>;
  const int64_t B = a.R / a.S;
  const size_t lds = (size_t)3 * a.D * sizeof(float);
  constexpr int kWpb = Shape::kWpb;
  // waves per compute unit: 4 per block of the 4-wave layout, as many blocks as LDS allows
  const int64_t waves_per_cu = 4 * std::max<int64_t>(1, std::min<int64_t>(Shape::kBlocksPerCu,
                                                                           kLdsPerCu / (int64_t)lds));
  int64_t per_cu = std::max<int64_t>(1, waves_per_cu / kWpb);
  const int cus = cu_count();
  // When that gives each wave at most one row, no more blocks than a compute
  // unit holds at once (registers: 2-3 blocks of 4 waves for rows of 3-6
  // steps of 8), else the last blocks wait for a second round; with more rows
  // the extra blocks balance the tail.  Measured, sized as above vs capped:
  // (1,4096,2048) 14.93 vs 12.22 us, (1,4096,2240) 17.69 vs 16.30,
  // (1,4096,3072) 19.71 vs 19.07; (4,4096,3072) 71.6 vs 75.0 (4 rows per wave).
  static std::atomic<int> held[64];
  if (a.R <= per_cu * kWpb * (cus > 0 ? cus : 256)) {
    const int h = resident_blocks_per_cu(held, rga_ln_modulate_tab<V, NV, UNIF, MANY>, kWpb * kWave,
                                         (size_t)3 * NV * kWave * V * sizeof(float));
    if (h > 0) per_cu = std::min<int64_t>(per_cu, h);
  }
  const int64_t target = per_cu * (cus > 0 ? cus : 256);
  int64_t bpb = (target + B - 1) / B;
  bpb = std::max<int64_t>(1, std::min<int64_t>(bpb, (a.S + kWpb - 1) / kWpb));
  if constexpr (V == 8 && kWpb > 4) {
    // 16-wave blocks of few rows would leave most compute units idle: one
    // wave per row in blocks of their own (the long-row kernel at W = 1: the
    // same lanes and merges, so the same bits) spreads them wider
    if (2 * B * bpb < (cus > 0 ? cus : 256)) {
      // that kernel's UNIF: all 8 of its steps full (D = 4096), not this one's NV
      const dim3 grid((unsigned)std::min<int64_t>(a.R, (int64_t)1 << 20));
      if (a.D == (int64_t)8 * V * kWave)
        hipLaunchKernelGGL((rga_ln_modulate_mw<V, 8, true>), grid, dim3(kWave), 0, st, a);
      else
        hipLaunchKernelGGL((rga_ln_modulate_mw<V, 8, false>), grid, dim3(kWave), 0, st, a);
      return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
    }
    // more rows than one per wave: 4-wave blocks (MANY above)
    if (a.R > (int64_t)kWpb * (cus > 0 ? cus : 256)) return launch_fused<V, NV, UNIF, true>(a, st);
  }
  hipLaunchKernelGGL((rga_ln_modulate_tab<V, NV, UNIF, MANY>), dim3((unsigned)(B * bpb)), dim3(kWpb * kWave), lds,
                     st, a, (int)bpb);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

template <int V>
int dispatch_fused(const FusedArgs& a, hipStream_t st) {
  const int64_t nvec = a.D / V;
  const int64_t nv = (nvec + kWave - 1) / kWave;
  const bool unif = nvec % kWave == 0;
#define ADALN_FUSED_CASE(N) \
  if (nv == N) return unif ? launch_fused<V, N, true>(a, st) : launch_fused<V, N, false>(a, st);
  ADALN_FUSED_CASE(1)
  ADALN_FUSED_CASE(2)
  ADALN_FUSED_CASE(3)
  ADALN_FUSED_CASE(4)
  ADALN_FUSED_CASE(5)
  ADALN_FUSED_CASE(6)
  ADALN_FUSED_CASE(7)
  ADALN_FUSED_CASE(8)
  if constexpr (V == 4) {  // rows of up to 4096 elements: 16 steps of 4
    ADALN_FUSED_CASE(9)
    ADALN_FUSED_CASE(10)
    ADALN_FUSED_CASE(11)
    ADALN_FUSED_CASE(12)
    ADALN_FUSED_CASE(13)
    ADALN_FUSED_CASE(14)
    ADALN_FUSED_CASE(15)
    ADALN_FUSED_CASE(16)
  }
#undef ADALN_FUSED_CASE
  return ADALN_ERR_TOO_LARGE;  // not reached: the caller bounds D
}

// W waves per row (W = 2 .. 16), every lane holding at most 64 elements in
// 8 vectors of 8.  (Rows with D % 8 != 0 would need 16 steps of 4 with three
// inputs each, more than the VGPRs of a 1024-thread block: they take the two
// unfused kernels.)
int dispatch_fused_mw(const FusedArgs& a, int W, hipStream_t st) {
  constexpr int V = 8, NV = 8;
  const bool unif = a.D / V == (int64_t)NV * W * kWave;
  // rows of up to 16384 elements: blocks holding several rows of one sample
  // and sharing its tables when the blocks fill at least three quarters of the
  // compute units (16 waves, else 8 in one round), else one row per block.
  // Measured, 16-wave blocks vs one row per block at D = 16384: 128 blocks
  // 20.37 vs 15.59 us, 256 blocks 25.6 vs 28.2, 320 (a last round of 64)
  // 42.6 vs 36.7, 512 50.2 vs 54.0.
  const int64_t B = a.R / a.S;
  const int cus = cu_count();
  const size_t lds = (size_t)a.D * 2 * sizeof(float);
  const int64_t n = cus > 0 ? cus : 256;
  auto fills = [&](int64_t P) {  // as for ln_modulate's long rows
    const int64_t blocks = B * ((a.S + P - 1) / P), rem = blocks % n;
    return W <= 4 && a.S >= P && blocks < ((int64_t)1 << 22) && 4 * blocks >= 3 * n &&
           (blocks <= n || rem == 0 || 2 * rem >= n);
  };
  if (fills(kMaxWaves / W)) {
    const int64_t P = kMaxWaves / W, bps = (a.S + P - 1) / P;
    if (unif)
      hipLaunchKernelGGL((rga_ln_modulate_mwt<NV, true, 1024>), dim3((unsigned)(B * bps)), dim3(1024), lds, st, a,
                         (int)bps, W);
    else
      hipLaunchKernelGGL((rga_ln_modulate_mwt<NV, false, 1024>), dim3((unsigned)(B * bps)), dim3(1024), lds, st, a,
                         (int)bps, W);
    return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
  }
  if (fills(kMaxWaves / 2 / W) && B * ((a.S + kMaxWaves / 2 / W - 1) / (kMaxWaves / 2 / W)) <= n) {
    const int64_t P = kMaxWaves / 2 / W, bps = (a.S + P - 1) / P;
    if (unif)
      hipLaunchKernelGGL((rga_ln_modulate_mwt<NV, true, 512>), dim3((unsigned)(B * bps)), dim3(512), lds, st, a,
                         (int)bps, W);
    else
      hipLaunchKernelGGL((rga_ln_modulate_mwt<NV, false, 512>), dim3((unsigned)(B * bps)), dim3(512), lds, st, a,
                         (int)bps, W);
    return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
  }
  const unsigned blocks = (unsigned)std::min<int64_t>(a.R, (int64_t)1 << 20);
  if (unif)
    hipLaunchKernelGGL((rga_ln_modulate_mw<V, NV, true>), dim3(blocks), dim3(W * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((rga_ln_modulate_mw<V, NV, false>), dim3(blocks), dim3(W * kWave), 0, st, a);
  return hipGetLastError() == hipSuccess ? ADALN_OK : ADALN_ERR_HIP;
}

}  // namespace

static int fused_check_shape(int64_t B, int64_t S, int64_t D, int64_t sr_b, int64_t sr_s,
                             int64_t sg_b, int64_t su_b, int64_t su_s, int64_t sscale_b,
                             int64_t sshift_b, int dtype) {
  if (dtype != ADALN_BF16) return ADALN_ERR_DTYPE;
  if (B < 0 || S < 0 || D < 4 || D % 4 != 0) return ADALN_ERR_SHAPE;
  if (D > 65536) return ADALN_ERR_TOO_LARGE;
  if (sr_b < 0 || sr_s < 0 || sg_b < 0 || su_b < 0 || su_s < 0 || sscale_b < 0 || sshift_b < 0)
    return ADALN_ERR_STRIDE;
  int64_t R, RD;
  if (!mul_ok(B, S, &R) || !mul_ok(R, D, &RD)) return ADALN_ERR_TOO_LARGE;
  if (!extent_ok({{B, sr_b}, {S, sr_s}, {D, 1}}) || !extent_ok({{B, su_b}, {S, su_s}, {D, 1}}) ||
      !extent_ok({{B, sg_b}, {D, 1}}) || !extent_ok({{B, sscale_b}, {D, 1}}) ||
      !extent_ok({{B, sshift_b}, {D, 1}}))
    return ADALN_ERR_TOO_LARGE;
  return ADALN_OK;
}

}  // namespace adaln

using namespace adaln;

extern "C" int residual_gate_add_ln_modulate_can_use(int64_t B, int64_t S, int64_t D, int64_t sr_b,
                                                     int64_t sr_s, int64_t sg_b, int64_t su_b,
                                                     int64_t su_s, int64_t sscale_b,
                                                     int64_t sshift_b, int dtype) {
  return fused_check_shape(B, S, D, sr_b, sr_s, sg_b, su_b, su_s, sscale_b, sshift_b, dtype) ==
         ADALN_OK;
}

extern "C" int residual_gate_add_ln_modulate(const void* residual, int64_t sr_b, int64_t sr_s,
                                             const void* gate, int64_t sg_b, const void* update,
                                             int64_t su_b, int64_t su_s, int64_t B, int64_t S,
                                             int64_t D, const void* scale, int64_t sscale_b,
                                             const void* shift, int64_t sshift_b, float eps,
                                             int dtype, void* residual_out, void* out,
                                             float* mean_out, float* rstd_out, void* stream) {
  int rc = fused_check_shape(B, S, D, sr_b, sr_s, sg_b, su_b, su_s, sscale_b, sshift_b, dtype);
  if (rc != ADALN_OK) return rc;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return ADALN_ERR_ARG;  // also rejects NaN
  const int64_t R = B * S;
  if (R == 0) return ADALN_OK;
  if (!residual || !gate || !update || !scale || !shift || !residual_out || !out)
    return ADALN_ERR_NULL;
  if (!aligned(residual, 2) || !aligned(gate, 2) || !aligned(update, 2) || !aligned(scale, 2) ||
      !aligned(shift, 2) || !aligned(residual_out, 2) || !aligned(out, 2) ||
      !aligned(mean_out, 4) || !aligned(rstd_out, 4))
    return ADALN_ERR_ALIGN;

  // overlap rules: residual_out may be exactly a contiguous residual, out
  // exactly a contiguous update; nothing else may overlap an output
  const Span sro = span_of(residual_out, {{R * D, 1}});
  const Span so = span_of(out, {{R * D, 1}});
  const Span sres = span_of(residual, {{B, sr_b}, {S, sr_s}, {D, 1}});
  const Span supd = span_of(update, {{B, su_b}, {S, su_s}, {D, 1}});
  const Span sg = span_of(gate, {{B, sg_b}, {D, 1}});
  const Span ssc = span_of(scale, {{B, sscale_b}, {D, 1}});
  const Span ssh = span_of(shift, {{B, sshift_b}, {D, 1}});
  const Span sm = mean_out ? Span{(uintptr_t)mean_out, (uintptr_t)(mean_out + R)} : Span{};
  const Span sr = rstd_out ? Span{(uintptr_t)rstd_out, (uintptr_t)(rstd_out + R)} : Span{};
  auto contig = [&](int64_t sb, int64_t ss) {
    return (S == 1 || ss == D) && (B == 1 || sb == S * D);
  };
  if (overlaps(sro, sres) && !(residual_out == residual && contig(sr_b, sr_s))) return ADALN_ERR_ALIAS;
  if (overlaps(so, supd) && !(out == update && contig(su_b, su_s))) return ADALN_ERR_ALIAS;
  for (const Span* t : {&supd, &sg, &ssc, &ssh, &so, &sm, &sr})
    if (overlaps(sro, *t)) return ADALN_ERR_ALIAS;
  for (const Span* t : {&sres, &sg, &ssc, &ssh, &sm, &sr})
    if (overlaps(so, *t)) return ADALN_ERR_ALIAS;
  for (const Span* t : {&sres, &supd, &sg, &ssc, &ssh})
    if (overlaps(sm, *t) || overlaps(sr, *t)) return ADALN_ERR_ALIAS;
  if (overlaps(sm, sr)) return ADALN_ERR_ALIAS;

  adaln_order ord{};
  order_of(ADALN_OP_RESIDUAL_GATE_ADD_LN_MODULATE, D, &ord);
  const int V = ord.V;
  const uintptr_t vb = (uintptr_t)(2 * V);
  auto stride_ok = [&](int64_t n, int64_t st) { return n <= 1 || ((uintptr_t)st * 2u) % vb == 0; };
  // one launch for vector-aligned rows (the tabled kernel indexes rows,
  // samples and offsets in 32 bits and launches a block of up to 1024
  // threads per sample: under 2^32 work-items)
  const bool fused = (ord.W > 1 ? V == 8 : (S <= INT32_MAX / 4 && B < ((int64_t)1 << 22))) && aligned(residual, vb) &&
                     aligned(update, vb) &&
                     aligned(gate, vb) && aligned(scale, vb) && aligned(shift, vb) &&
                     aligned(residual_out, vb) && aligned(out, vb) && stride_ok(B, sr_b) &&
                     stride_ok(S, sr_s) && stride_ok(B, su_b) && stride_ok(S, su_s) &&
                     stride_ok(B, sg_b) && stride_ok(B, sscale_b) && stride_ok(B, sshift_b);
  hipStream_t st = (hipStream_t)stream;
  if (!fused) {
    rc = ::residual_gate_add(residual, sr_b, sr_s, gate, sg_b, update, su_b, su_s, B, S, D, dtype,
                             residual_out, stream);
    if (rc != ADALN_OK) return rc;
    return ::ln_modulate(residual_out, B, S, D, S * D, D, 1, scale, sscale_b, shift, sshift_b, eps,
                         dtype, out, mean_out, rstd_out, stream);
  }

  FusedArgs a;
  a.res = (const uint16_t*)residual;
  a.sr_b = sr_b;
  a.sr_s = sr_s;
  a.gate = (const uint16_t*)gate;
  a.sg_b = sg_b;
  a.upd = (const uint16_t*)update;
  a.su_b = su_b;
  a.su_s = su_s;
  a.scale = (const uint16_t*)scale;
  a.ssc_b = sscale_b;
  a.shift = (const uint16_t*)shift;
  a.ssh_b = sshift_b;
  a.eps = eps;
  a.res_out = (uint16_t*)residual_out;
  a.out = (uint16_t*)out;
  a.mean_out = mean_out;
  a.rstd_out = rstd_out;
  a.S = S;
  a.D = D;
  a.R = R;
  if (ord.W > 1) return dispatch_fused_mw(a, ord.W, st);
  return V == 8 ? dispatch_fused<8>(a, st) : dispatch_fused<4>(a, st);
}
