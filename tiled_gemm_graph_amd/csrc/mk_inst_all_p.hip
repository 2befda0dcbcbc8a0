// The four-wave kernel instance with every body, persistent loop (see
// mk_instances.h).
#include <hip/hip_runtime.h>

#include "mk_instances.h"
#include "mk_kernels.h"

namespace mk {
const void* instances_all_p(bool persistent, unsigned ops, int nt) {
  if (nt != 256 || !persistent || ops != mkd::kOpAll) return nullptr;
  return reinterpret_cast<const void*>(mk_persistent<mkd::kOpAll>);
}
}  // namespace mk
