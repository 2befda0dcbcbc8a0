// The four-wave GEMV and GEMV + other kernel instances (see mk_instances.h).
#include <hip/hip_runtime.h>

#include "mk_instances.h"
#include "mk_kernels.h"

namespace mk {
const void* instances_gemv(bool persistent, unsigned ops, int nt) {
  using namespace mkd;
  if (nt != 256) return nullptr;
  if (persistent) {
    if (ops == kOpGemv) return reinterpret_cast<const void*>(mk_persistent<kOpGemv>);
    if (ops == (kOpGemv | kOpOther)) return reinterpret_cast<const void*>(mk_persistent<kOpGemv | kOpOther>);
    return nullptr;
  }
  if (ops == kOpGemv) return reinterpret_cast<const void*>(mk_node_kernel<kOpGemv>);
  if (ops == (kOpGemv | kOpOther)) return reinterpret_cast<const void*>(mk_node_kernel<kOpGemv | kOpOther>);
  return nullptr;
}
}  // namespace mk
