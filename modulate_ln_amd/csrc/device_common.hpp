// Device helpers shared by the adaLN kernels (gfx950, wave64).
//
// Numerics: this file is compiled with -ffp-contract=off, so every fp32
// operation rounds on its own; the only fused multiply-adds are the explicit
// __builtin_fmaf calls the reduction order names.  fp32 denormals are kept
// (the gfx950 default), division and square root are the IEEE-correct
// sequences hipcc emits by default.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>
#include <utility>

namespace adaln {

constexpr int kWave = 64;

// Compute units of the current device (cached; 0 if the query fails).
inline int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();  // not left for the launch check that follows
      return 0;
    }
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Blocks of one kernel that a compute unit of the current device holds at
// once (its registers, LDS and waves; lds: the most dynamic LDS a block of it
// asks for), cached per device in the caller's array; 0 when the query fails.
// A launch sized for more blocks per compute unit than this runs its last
// blocks in a second round.
template <typename F>
inline int resident_blocks_per_cu(std::atomic<int>* cache, F kernel, int threads, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n <= 0) {
      (void)hipGetLastError();  // not left for the launch check that follows
      return 0;
    }
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  A 32-bit word holds two consecutive bf16 elements: the
// lower-addressed one in bits 0..15.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lo_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}
__device__ __forceinline__ float u16_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Round two fp32 values to bf16 (round-to-nearest-even; one v_cvt_pk_bf16_f32)
// and pack them, lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t to_bf16(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Round one fp32 value to bf16 and keep it in fp32 format: converting the
// pair (0, v) puts bf16(v) in the high half-word over a zero low half-word,
// which is the widened value itself (one v_cvt_pk_bf16_f32 with an inline
// zero, where packing two values and splitting them again takes three ops).
__device__ __forceinline__ float round_f32(float v) {
  f32x2 f = {0.0f, v};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(float, h);
}

// Round a pair to bf16 and widen back: the values the eager chain stores.
__device__ __forceinline__ void round_pair(float& a, float& b) {
  a = round_f32(a);
  b = round_f32(b);
}

// ---------------------------------------------------------------------------
// Welford push with a compile-time count: N is the count after this element,
// 1/N is folded by the compiler to the correctly rounded fp32 reciprocal.
// Order (the pages' _welford_push): delta = x - mean; mean += delta/N as one
// fma with the reciprocal; m2 += delta * (x - mean_new) as one fma.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void welford_push(float& mean, float& m2, float x) {
  constexpr float r = 1.0f / (float)N;
  float delta = x - mean;
  mean = __builtin_fmaf(delta, r, mean);
  m2 = __builtin_fmaf(delta, x - mean, m2);
}

// Chan-Golub-LeVeque merge of two partial states; (ma, m2a, na) is the state
// of the LOWER lane.  An empty side leaves the other unchanged.
__device__ __forceinline__ void welford_merge(float& ma, float& m2a, float& na, float mb, float m2b,
                                              float nb) {
  float n = na + nb;
  float f = nb / n;
  float delta = mb - ma;
  float m = __builtin_fmaf(delta, f, ma);
  float m2 = (m2a + m2b) + (delta * delta) * (na * f);
  bool a_empty = (na == 0.0f);
  bool b_empty = (nb == 0.0f);
  float rm = b_empty ? ma : (a_empty ? mb : m);
  float rm2 = b_empty ? m2a : (a_empty ? m2b : m2);
  float rn = b_empty ? na : (a_empty ? nb : n);
  ma = rm;
  m2a = rm2;
  na = rn;
}

// ---------------------------------------------------------------------------
// Cross-lane exchange: value held by lane (lane ^ OFF) of the same wave.
// OFF 1, 2: DPP quad permutes; 4: ds_swizzle xor mode; 8: DPP row rotate
// by 8 (within 16 lanes that is xor 8); 16, 32: gfx950 permlane swaps.
// ---------------------------------------------------------------------------
template <int OFF>
__device__ __forceinline__ float lane_xor(float v) {
  int i = __builtin_bit_cast(int, v);
  if constexpr (OFF == 1) {
    i = __builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (OFF == 2) {
    i = __builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (OFF == 4) {
    i = __builtin_amdgcn_ds_swizzle(i, (4 << 10) | 0x1F);  // and 0x1f, or 0, xor 4
  } else if constexpr (OFF == 8) {
    i = __builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (OFF == 16) {
    // odd rows of the first operand swap with even rows of the second
    auto p = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    i = (lane & 16) ? (int)p[0] : (int)p[1];
  } else {
    static_assert(OFF == 32, "lane_xor: offset must be 1, 2, 4, 8, 16 or 32");
    // upper half of the first operand swaps with lower half of the second
    auto p = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    i = (lane & 32) ? (int)p[0] : (int)p[1];
  }
  return __builtin_bit_cast(float, i);
}

// One level of the pairwise merge tree at distance OFF: lanes l and l^OFF
// both compute merge(lower, upper), so after the levels 1..OFF every lane
// of an aligned group of 2*OFF lanes holds the group's state.
template <int OFF>
__device__ __forceinline__ void merge_level(float& m, float& m2, float& n, int lane) {
  float pm = lane_xor<OFF>(m);
  float pm2 = lane_xor<OFF>(m2);
  float pn = lane_xor<OFF>(n);
  const bool upper = (lane & OFF) != 0;
  float am = upper ? pm : m, am2 = upper ? pm2 : m2, an = upper ? pn : n;
  float bm = upper ? m : pm, bm2 = upper ? m2 : pm2, bn = upper ? n : pn;
  welford_merge(am, am2, an, bm, bm2, bn);
  m = am;
  m2 = am2;
  n = an;
}

// Butterfly level when both halves hold `cnt_half` elements: nb/n = 0.5
// exactly, so no division (bit-identical to merge_level with those counts).
template <int OFF>
__device__ __forceinline__ void merge_level_equal(float& m, float& m2, float cnt_half, int lane) {
  const float pm = lane_xor<OFF>(m);
  const float pm2 = lane_xor<OFF>(m2);
  const bool upper = (lane & OFF) != 0;
  const float am = upper ? pm : m, bm = upper ? m : pm;  // lower lane's mean, upper lane's mean
  const float delta = bm - am;
  const float mm = __builtin_fmaf(delta, 0.5f, am);
  m2 = (m2 + pm2) + (delta * delta) * (cnt_half * 0.5f);
  m = mm;
}

// Merge groups of 16 lanes that each hold `cnt` elements.
__device__ __forceinline__ void merge_lanes16_equal(float& m, float& m2, float cnt, int lane) {
  merge_level_equal<1>(m, m2, cnt, lane);
  merge_level_equal<2>(m, m2, 2.0f * cnt, lane);
  merge_level_equal<4>(m, m2, 4.0f * cnt, lane);
  merge_level_equal<8>(m, m2, 8.0f * cnt, lane);
}

// Merge the per-lane states of groups of L lanes (L = 16 or 64).
template <int L>
__device__ __forceinline__ void merge_lanes(float& m, float& m2, float& n, int lane) {
  merge_level<1>(m, m2, n, lane);
  merge_level<2>(m, m2, n, lane);
  merge_level<4>(m, m2, n, lane);
  merge_level<8>(m, m2, n, lane);
  if constexpr (L == 64) {
    merge_level<16>(m, m2, n, lane);
    merge_level<32>(m, m2, n, lane);
  } else {
    static_assert(L == 16, "merge_lanes: L must be 16 or 64");
  }
}

// Value held by lane (lane + OFF) of the same wave, for the merge tree that
// collects the row's state in lane 0.  Lanes whose partner falls outside
// their DPP row (OFF <= 8) or outside the wave receive unspecified values;
// the tree never reads them for a lane it keeps.
template <int OFF>
__device__ __forceinline__ float lane_down(float v) {
  int i = __builtin_bit_cast(int, v);
  if constexpr (OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8) {
    i = __builtin_amdgcn_update_dpp(0, i, 0x100 + OFF, 0xF, 0xF, false);  // row_shl:OFF
  } else if constexpr (OFF == 16) {
    auto p = __builtin_amdgcn_permlane16_swap((unsigned)i, (unsigned)i, false, false);
    i = (int)p[1];  // even rows receive the odd row above them
  } else {
    static_assert(OFF == 32, "lane_down: offset must be 1, 2, 4, 8, 16 or 32");
    auto p = __builtin_amdgcn_permlane32_swap((unsigned)i, (unsigned)i, false, false);
    i = (int)p[1];  // the lower half receives the upper half
  }
  return __builtin_bit_cast(float, i);
}

// Within each DPP row of 16 lanes: the value of lane (l - K), written only
// into the lanes of the 4-lane banks set in BANKS (the others keep `old`).
template <int K, int BANKS>
__device__ __forceinline__ float row_shr_bank(float old, float v) {
  static_assert(K >= 1 && K <= 15 && BANKS >= 1 && BANKS <= 15, "row_shr_bank: K in 1..15");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), 0x110 + K, 0xF,
                                                               BANKS, false));
}

// Lane N of each DPP row of 16 lanes, broadcast to the whole row (gfx950
// row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  static_assert(N >= 0 && N <= 15, "row_bcast: N in 0..15");
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xF, 0xF, false));
}

// f(std::integral_constant<int, I>) for I = 0 .. N-1, in order.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One level of the merge tree toward lane 0: lane l merges lane l + OFF into
// its own state (lower lane first).  After levels 1, 2, ..., 32 lane 0 holds
// the state of the whole wave -- the same pairwise tree as merge_lanes.
template <int OFF>
__device__ __forceinline__ void merge_down(float& m, float& m2, float& n) {
  const float mb = lane_down<OFF>(m);
  const float m2b = lane_down<OFF>(m2);
  const float nb = lane_down<OFF>(n);
  welford_merge(m, m2, n, mb, m2b, nb);
}

// The same level when every lane of the wave holds `cnt` elements: the
// merged halves are equal, so nb/n = 0.5 exactly and the update needs no
// division (bit-identical to welford_merge with those counts).
template <int OFF>
__device__ __forceinline__ void merge_down_equal(float& m, float& m2, float cnt) {
  const float mb = lane_down<OFF>(m);
  const float m2b = lane_down<OFF>(m2);
  const float na = cnt * (float)OFF;  // lower half's count (exact)
  const float delta = mb - m;
  const float mm = __builtin_fmaf(delta, 0.5f, m);
  m2 = (m2 + m2b) + (delta * delta) * (na * 0.5f);
  m = mm;
}

// ---------------------------------------------------------------------------
// RMSNorm statistics: per-lane sums of squares (ss = fma(x, x, ss) in
// increasing position) summed pairwise, nearest first.  fp32 addition is
// commutative bit for bit, so the butterfly (every lane of a 2*OFF group
// computes lower + upper) and the tree toward lane 0 give the same sums as
// lane l taking ss[l] + ss[l + OFF].  Lanes without elements hold +0.
// ---------------------------------------------------------------------------
template <int OFF>
__device__ __forceinline__ void sum_level(float& s) {
  s = s + lane_xor<OFF>(s);
}

template <int L>
__device__ __forceinline__ void sum_lanes(float& s) {
  sum_level<1>(s);
  sum_level<2>(s);
  sum_level<4>(s);
  sum_level<8>(s);
  if constexpr (L == 64) {
    sum_level<16>(s);
    sum_level<32>(s);
  } else {
    static_assert(L == 16, "sum_lanes: L must be 16 or 64");
  }
}

template <int OFF>
__device__ __forceinline__ void sum_down(float& s) {
  s = s + lane_down<OFF>(s);
}

// ---------------------------------------------------------------------------
// The output stage of the norm + modulate kernels.
//   kTailChain  the eager chain: x_hat, x_hat * (1 + scale) and + shift each
//               rounded to bf16
//   kTailFold   one affine op: bf16(fma(1 + scale, n, shift)) on the unrounded
//               normalized value n
//   kTailFp8    the chain's bf16 output times 1/qscale, clamped to +-448 and
//               converted to OCP FP8 E4M3 (round to nearest even): one byte
// ---------------------------------------------------------------------------
constexpr int kTailChain = 0;
constexpr int kTailFold = 1;
constexpr int kTailFp8 = 2;

// clamp to the largest finite E4M3 magnitude; NaN passes (the compares are false)
__device__ __forceinline__ float clamp448(float v) {
  v = v > 448.0f ? 448.0f : v;
  return v < -448.0f ? -448.0f : v;
}

// The same clamp for values known not to be NaN: one v_med3_f32 (which would
// turn a NaN into -448).
__device__ __forceinline__ float clamp448_finite(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}

// four fp32 values -> four E4M3 bytes (gfx950's conversion is OCP E4M3 with
// round-to-nearest-even; it gives NaN, not 448, past 464, hence the clamp)
// (The first conversion fills the low half-word and keeps the high one, which
// the second overwrites: seeding it with a's bits spares a register clear.)
__device__ __forceinline__ uint32_t fp8_quad(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// The tail of one element pair: n0, n1 are the normalized values before any
// rounding, o = bf16(1 + scale) and h = shift as fp32.  Returns two bf16
// (the chain or the fold).
template <int TAIL>
__device__ __forceinline__ uint32_t tail_pair(float n0, float n1, float o0, float o1, float h0, float h1) {
  if constexpr (TAIL == kTailFold) {
    return pack_bf16(__builtin_fmaf(o0, n0, h0), __builtin_fmaf(o1, n1, h1));
  } else {
    round_pair(n0, n1);  // x_hat = bf16(n)
    float y0 = n0 * o0, y1 = n1 * o1;
    round_pair(y0, y1);  // bf16(x_hat * (1 + scale))
    return pack_bf16(y0 + h0, y1 + h1);  // bf16(y + shift)
  }
}

// The chain's output for one element as the fp32 value of its bf16 (the
// rounding of x_hat, of x_hat * (1 + scale) and of + shift), for a stage
// that consumes it in fp32 rather than as packed bf16.
__device__ __forceinline__ float chain_f32(float n, float o, float h) {
  return round_f32(round_f32(round_f32(n) * o) + h);
}

// The FP8 stage for V values y (the chain's output as fp32): q = e4m3(clamp(
// y * qinv)), packed four bytes per word into q[0 .. V/4); no_nan as below.
template <int V>
__device__ __forceinline__ void fp8_stage_f32(const float* y, float qinv, bool no_nan, uint32_t* q) {
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) v[i] = y[i] * qinv;
  if (no_nan) {
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = clamp448_finite(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = clamp448(v[i]);
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) q[i] = fp8_quad(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// The FP8 stage for V/2 bf16 pairs w (the chain's output): q = e4m3(clamp(y *
// qinv)), packed four bytes per word into q[0 .. V/4).  no_nan: the caller
// knows no value can be NaN (finite row statistics and finite adaLN rows),
// so the clamp is one v_med3 per element; otherwise NaN-preserving compares.
template <int V>
__device__ __forceinline__ void fp8_stage(const uint32_t* w, float qinv, bool no_nan, uint32_t* q) {
  float v[V];
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    v[2 * i] = lo_f32(w[i]) * qinv;
    v[2 * i + 1] = hi_f32(w[i]) * qinv;
  }
  if (no_nan) {
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = clamp448_finite(v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = clamp448(v[i]);
  }
#pragma unroll
  for (int i = 0; i < V / 4; ++i) q[i] = fp8_quad(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

__device__ __forceinline__ float bcast_lane0(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// 2^-k when D = 2^k, else 0.  For such D, m2 * 2^-k is exactly m2 / D (both
// are the correctly rounded value of the same real number), without the
// division sequence.
__device__ __forceinline__ float pow2_inverse(int64_t D) {
  return (D > 0 && (D & (D - 1)) == 0) ? __builtin_ldexpf(1.0f, -__builtin_ctzll((uint64_t)D)) : 0.0f;
}

// The same for a row length given as a float (an integer below 2^24): 1/D
// when D is a power of two, else 0.
__device__ __forceinline__ float pow2_inverse_f(float D) {
  const uint32_t b = __builtin_bit_cast(uint32_t, D);
  return (D >= 1.0f && (b & 0x7fffffu) == 0) ? __builtin_bit_cast(float, (254u - (b >> 23)) << 23) : 0.0f;
}

// var = m2/D, rstd = 1/sqrt(var + eps): IEEE division and square root.
// (With m2 the sum of squares this is RMSNorm's 1/sqrt(mean(x^2) + eps).)
// invD: pow2_inverse(D), a wave-uniform value; non-zero selects the exact
// multiplication in place of the division.
__device__ __forceinline__ float finalize_rstd(float m2, float D, float eps, float invD = 0.0f) {
  float var;
  if (invD != 0.0f)
    var = m2 * invD;
  else
    var = m2 / D;
  float t = var + eps;
  float s = __builtin_sqrtf(t);
  return 1.0f / s;
}

// ---------------------------------------------------------------------------
// Vectors of V bf16 elements as V/2 packed words.
// ---------------------------------------------------------------------------
template <int V>
struct Vec {
  uint32_t w[V / 2];
};

template <int V>
__device__ __forceinline__ Vec<V> load_vec(const uint16_t* p) {
  Vec<V> r;
  if constexpr (V == 8) {
    uint4 t = *reinterpret_cast<const uint4*>(p);
    r.w[0] = t.x;
    r.w[1] = t.y;
    r.w[2] = t.z;
    r.w[3] = t.w;
  } else {
    static_assert(V == 4, "V must be 4 or 8");
    uint2 t = *reinterpret_cast<const uint2*>(p);
    r.w[0] = t.x;
    r.w[1] = t.y;
  }
  return r;
}

template <int V>
__device__ __forceinline__ void store_vec(uint16_t* p, const Vec<V>& v) {
  if constexpr (V == 8) {
    *reinterpret_cast<uint4*>(p) = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(v.w[0], v.w[1]);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) vector load/store: data touched once per call.
template <int V>
__device__ __forceinline__ Vec<V> load_vec_nt(const uint16_t* p) {
  Vec<V> r;
  if constexpr (V == 8) {
    u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    r.w[0] = t[0];
    r.w[1] = t[1];
    r.w[2] = t[2];
    r.w[3] = t[3];
  } else {
    u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r.w[0] = t[0];
    r.w[1] = t[1];
  }
  return r;
}

template <int V>
__device__ __forceinline__ void store_vec_nt(uint16_t* p, const Vec<V>& v) {
  if constexpr (V == 8) {
    u32x4 t = {v.w[0], v.w[1], v.w[2], v.w[3]};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
  } else {
    u32x2 t = {v.w[0], v.w[1]};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
  }
}

// V E4M3 bytes (four per word of q); p is V-byte aligned
template <int V>
__device__ __forceinline__ void store_fp8_nt(uint8_t* p, const uint32_t* q) {
  if constexpr (V == 8) {
    u32x2 t = {q[0], q[1]};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
  } else {
    __builtin_nontemporal_store(q[0], reinterpret_cast<uint32_t*>(p));
  }
}

// element-wise gather of V elements at stride s (any alignment)
template <int V>
__device__ __forceinline__ Vec<V> gather_vec(const uint16_t* p, int64_t s) {
  Vec<V> r;
#pragma unroll
  for (int i = 0; i < V / 2; ++i)
    r.w[i] = (uint32_t)p[(2 * i) * s] | ((uint32_t)p[(2 * i + 1) * s] << 16);
  return r;
}

template <int V>
__device__ __forceinline__ void scatter_vec(uint16_t* p, const Vec<V>& v) {
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    p[2 * i] = (uint16_t)(v.w[i] & 0xffffu);
    p[2 * i + 1] = (uint16_t)(v.w[i] >> 16);
  }
}

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

}  // namespace adaln
