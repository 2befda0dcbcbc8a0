// The four-wave kernel instances without GEMV bodies (see mk_instances.h).
#include <hip/hip_runtime.h>

#include "mk_instances.h"
#include "mk_kernels.h"

namespace mk {
const void* instances_gemm(bool persistent, unsigned ops, int nt) {
  using namespace mkd;
  if (nt != 256) return nullptr;
  if (persistent) {
    if (ops == kOpGemm) return reinterpret_cast<const void*>(mk_persistent<kOpGemm>);
    if (ops == (kOpGemm | kOpOther)) return reinterpret_cast<const void*>(mk_persistent<kOpGemm | kOpOther>);
    return nullptr;
  }
  if (ops == kOpGemm) return reinterpret_cast<const void*>(mk_node_kernel<kOpGemm>);
  if (ops == (kOpGemm | kOpOther)) return reinterpret_cast<const void*>(mk_node_kernel<kOpGemm | kOpOther>);
  return nullptr;
}
}  // namespace mk
