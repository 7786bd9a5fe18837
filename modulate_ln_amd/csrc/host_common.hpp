// Host-side argument checks shared by the entry points.  Pure C++: nothing
// here touches the HIP runtime, so every check runs before any launch and
// on machines without a GPU.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <initializer_list>

#include "../../include/adaln.h"

namespace adaln {

// Largest element count the kernels index (signed 64-bit byte offsets with
// ample headroom).
constexpr int64_t kMaxElems = (int64_t)1 << 46;

struct Dim {
  int64_t size;
  int64_t stride;  // elements
};

// Byte range [lo, hi) touched by a tensor of elem-byte elements (bf16 by
// default) with the given dims.  Empty tensors touch nothing (lo == hi).
struct Span {
  uintptr_t lo = 0, hi = 0;
};

inline bool dims_ok(std::initializer_list<Dim> dims) {
  for (const Dim& d : dims)
    if (d.size < 0 || d.stride < 0) return false;
  return true;
}

inline Span span_of(const void* p, std::initializer_list<Dim> dims, size_t elem = 2) {
  Span s;
  int64_t last = 0;
  for (const Dim& d : dims) {
    if (d.size == 0) return s;
    last += (d.size - 1) * d.stride;
  }
  s.lo = (uintptr_t)p;
  s.hi = s.lo + (uintptr_t)(last + 1) * (uintptr_t)elem;
  return s;
}

inline bool overlaps(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

inline bool aligned(const void* p, uintptr_t bytes) { return ((uintptr_t)p % bytes) == 0; }

// product with overflow guard against kMaxElems
inline bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxElems / a) return false;
  *out = a * b;
  return *out <= kMaxElems;
}

// every stride and offset the kernels form stays below kMaxElems
inline bool extent_ok(std::initializer_list<Dim> dims) {
  int64_t last = 0;
  for (const Dim& d : dims) {
    if (d.size == 0) return true;
    int64_t t;
    if (!mul_ok(d.size - 1, d.stride, &t)) return false;
    last += t;
    if (last > kMaxElems) return false;
  }
  return true;
}

// Lanes of one wave per q/k head: a DPP row.
constexpr int kHeadLanes = 16;
constexpr int kWaveLanes = 64;
constexpr int64_t kLaneElems = 64;  // most elements of a row one lane holds
constexpr int64_t kMaxRowD = 65536;  // longest row of the row ops
constexpr int64_t kMaxHeadD = 256;   // longest q/k head

// The fixed reduction order of op for rows of D elements (the descriptor
// adaln_order_for reports; the kernels follow it, whatever the storage).
inline int order_of(int op, int64_t D, adaln_order* o) {
  const bool row_op = op == ADALN_OP_LN_MODULATE || op == ADALN_OP_RESIDUAL_GATE_ADD_LN_MODULATE ||
                      op == ADALN_OP_RMSNORM_SCALE_SHIFT;
  const bool head_op = op == ADALN_OP_QK_HEAD_LAYERNORM || op == ADALN_OP_QK_RMSNORM;
  if (!row_op && !head_op) return ADALN_ERR_ARG;
  if (D <= 0 || D % 4 != 0) return ADALN_ERR_SHAPE;
  if (head_op && D > kMaxHeadD) return ADALN_ERR_SHAPE;
  if (row_op && D > kMaxRowD) return ADALN_ERR_TOO_LARGE;
  o->V = (D % 8 == 0) ? 8 : 4;
  // row ops: the fewest waves (a power of two) that leave at most 64
  // elements per lane; a q/k head is 16 lanes of one wave
  int w = 1;
  while (row_op && (int64_t)w * kWaveLanes * kLaneElems < D) w *= 2;
  o->W = w;
  o->L = head_op ? kHeadLanes : 64 * o->W;
  o->map = ADALN_MAP_INTERLEAVED;
  o->fold = ADALN_FOLD_PAIRWISE;
  return ADALN_OK;
}

// Elements per vector of op's order (D already validated by the caller).
inline int vec_of(int op, int64_t D) {
  adaln_order o{};
  return order_of(op, D, &o) == ADALN_OK ? o.V : 0;
}

}  // namespace adaln
