// The eight-wave kernel instances (see mk_instances.h).
#include <hip/hip_runtime.h>

#include "mk_instances.h"
#include "mk_kernels.h"

namespace mk {
const void* instances_wide(bool persistent, unsigned ops, int nt) {
  using namespace mkd;
  if (nt != 512) return nullptr;
  if (persistent) {
    if (ops == kOpGemm) return reinterpret_cast<const void*>(mk_persistent<kOpGemm, 512>);
    if (ops == (kOpGemm | kOpOther)) return reinterpret_cast<const void*>(mk_persistent<kOpGemm | kOpOther, 512>);
    return nullptr;
  }
  if (ops == kOpGemm) return reinterpret_cast<const void*>(mk_node_kernel<kOpGemm, 512>);
  if (ops == kOpOther) return reinterpret_cast<const void*>(mk_node_kernel<kOpOther, 512>);
  if (ops == (kOpGemm | kOpOther)) return reinterpret_cast<const void*>(mk_node_kernel<kOpGemm | kOpOther, 512>);
  return nullptr;
}
}  // namespace mk
