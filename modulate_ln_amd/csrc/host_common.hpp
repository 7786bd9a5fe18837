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

inline int order_for(int op, int64_t D, int* V, int* L) {
  if (D <= 0 || D % 4 != 0) return ADALN_ERR_SHAPE;
  int v = (D % 8 == 0) ? 8 : 4;
  int l;
  if (op == ADALN_OP_LN_MODULATE || op == ADALN_OP_RESIDUAL_GATE_ADD_LN_MODULATE ||
      op == ADALN_OP_RMSNORM_SCALE_SHIFT)
    l = 64;
  else if (op == ADALN_OP_QK_HEAD_LAYERNORM || op == ADALN_OP_QK_RMSNORM)
    l = 16;
  else
    return ADALN_ERR_ARG;
  if (V) *V = v;
  if (L) *L = l;
  return ADALN_OK;
}

}  // namespace adaln
