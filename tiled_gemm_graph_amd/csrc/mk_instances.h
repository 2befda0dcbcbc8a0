// Kernel instances of the persistent loop and of the per-op baseline, each
// compiled in one of five translation units so that the library builds
// in parallel.  A unit returns the entry point of the instance (persistent
// loop or per-op kernel, op families `ops`, `nt` threads per workgroup) if
// it holds it, and nullptr otherwise.
#pragma once

namespace mk {
// mk_inst_wide.hip: the eight-wave instances (packed GEMM, REDUCE, RMSNORM,
// ATTENTION, elementwise bodies)
const void* instances_wide(bool persistent, unsigned ops, int nt);
// mk_inst_gemv.hip: the four-wave GEMV and GEMV + other instances
const void* instances_gemv(bool persistent, unsigned ops, int nt);
// mk_inst_all_p.hip, mk_inst_all_n.hip: the four-wave instances with every
// body, persistent loop and per-op kernel
const void* instances_all_p(bool persistent, unsigned ops, int nt);
const void* instances_all_n(bool persistent, unsigned ops, int nt);
// mk_inst_gemm.hip: the four-wave instances without GEMV bodies
const void* instances_gemm(bool persistent, unsigned ops, int nt);
}  // namespace mk
