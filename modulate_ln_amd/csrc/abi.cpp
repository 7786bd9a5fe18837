// Library-level entry points: status names, ABI version, reduction order.
// Pure host code (no HIP runtime calls).
#include "../../include/adaln.h"
#include "host_common.hpp"

extern "C" const char* adaln_status_str(int status) {
  switch (status) {
    case ADALN_OK:
      return "ok";
    case ADALN_ERR_NULL:
      return "a required pointer is NULL";
    case ADALN_ERR_SHAPE:
      return "invalid shape (negative size, hidden % 4 != 0 or head size out of range)";
    case ADALN_ERR_DTYPE:
      return "unsupported dtype (only bf16)";
    case ADALN_ERR_ALIGN:
      return "a tensor pointer is misaligned";
    case ADALN_ERR_ALIAS:
      return "an output overlaps an input in a way the op does not allow";
    case ADALN_ERR_TOO_LARGE:
      return "a size exceeds what the kernels support";
    case ADALN_ERR_STRIDE:
      return "a stride is negative or unsupported";
    case ADALN_ERR_HIP:
      return "the HIP runtime reported a launch error";
    case ADALN_ERR_ARG:
      return "invalid argument";
    default:
      return "unknown status";
  }
}

extern "C" int adaln_abi_version(void) { return ADALN_ABI_VERSION; }

extern "C" int adaln_order_for(int op, int64_t D, int64_t sx_d, int align_bytes, adaln_order* out) {
  adaln_order o{};
  const int rc = adaln::order_of(op, D, &o);
  if (rc != ADALN_OK) return rc;
  if (sx_d < 0) return ADALN_ERR_STRIDE;
  if (align_bytes < 2 || (align_bytes & (align_bytes - 1)) != 0) return ADALN_ERR_ALIGN;
  if (!out) return ADALN_ERR_NULL;
  *out = o;
  return ADALN_OK;
}
