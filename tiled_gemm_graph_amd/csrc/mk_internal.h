// Internal structures of the host compiler and runtime (not part of the ABI).
#pragma once
#include <array>
#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "mk.h"

namespace mk {

using I64 = int64_t;
using Shape4 = std::array<I64, 4>;

struct Tensor {
  mk_dtype dt = MK_F16;
  mk_role role = MK_INTERMEDIATE;
  int ndim = 0;
  Shape4 shape{1, 1, 1, 1};   // left-padded
  bool is_view = false;
  int root = -1;              // views: root tensor id (never a view)
  Shape4 lo{0, 0, 0, 0}, hi{0, 0, 0, 0};  // views: range on the root
  // internal tensors created by the compiler
  bool internal = false;
  int const_kind = 0;         // 1 = rotary cos/sin table
  int rope_half = 0;
  float rope_theta = 0.f;
};

struct OpRec {
  mk_op_kind kind;
  std::vector<int> in;
  int out = -1;
  mk_op_attrs attrs{};
};

// A step-1 range on a root tensor (views resolved).
struct Edge {
  int tensor = -1;
  Shape4 lo{0, 0, 0, 0}, hi{0, 0, 0, 0};
  I64 rows() const { return hi[2] - lo[2]; }
  I64 cols() const { return hi[3] - lo[3]; }
};

struct Box {
  Shape4 lo, hi;
  bool operator<(const Box& o) const {
    if (lo != o.lo) return lo < o.lo;
    return hi < o.hi;
  }
  bool operator==(const Box& o) const { return lo == o.lo && hi == o.hi; }
};

struct Access {
  int tensor;
  Box box;
};

struct Instr {
  int32_t coord[4] = {0, 0, 0, 0};
  int32_t r0 = 0, r1 = 0, c0 = 0, c1 = 0, k0 = 0, k1 = 0, s = 0;
  std::vector<Access> reads, writes;
};

struct Node {
  int op = -1;
  int opcode = MK_I_NOOP;
  int flags = 0;
  int out = -1;                 // root tensor written
  std::vector<Edge> edges;      // every input edge (for readers / slots)
  std::vector<Instr> ins;
  int start = 0, end = 0;       // [start, end) in the flat list, incl. pads
  mk_node desc{};
};

// A weight tensor that a GEMV reads as packed column tiles.
struct PackInfo {
  int kind = 1;      // 1: GEMV column tiles [T][K][wc]; 2: GEMM tiles [T][K/64][bn][64]
  int tensor = -1;
  I64 K = 0, N = 0;
  int bn = 0;        // GEMV: output positions per tile; GEMM: weight columns per tile
  int wc = 0;        // GEMV: packed row width (bn, or 2 * bn under SILU_MUL); GEMM: bn
  I64 tiles = 0;
  bool silu = false;
  int head_dim = 0;  // > 0: positions [0, rope_cols) interleave rotation pairs
  I64 rope_cols = 0;
  mk_dtype dt = MK_F16;
  I64 bytes = 0;
};

}  // namespace mk

struct mk_graph {
  std::vector<mk::Tensor> t;
  std::vector<mk::OpRec> ops;
};

struct mk_plan_device;  // runtime-owned device state (mk_runtime.hip)

struct mk_plan {
  mk_build_options opts{};
  std::vector<mk::Tensor> tensors;   // graph tensors + internal tensors
  int n_graph_tensors = 0;
  std::vector<mk::OpRec> ops;
  std::vector<mk_tile> op_tiles;
  std::vector<mk::Node> nodes;
  std::vector<mk_instr> records;     // n_iters * num_cus (zero-filled tail)
  std::vector<mk_node> node_descs;
  std::vector<int32_t> targets;
  std::vector<int32_t> slot_of_tensor;   // by tensor id (graph + internal)
  std::vector<int32_t> slot_owner;       // slot -> representative tensor id
  std::vector<mk::I64> slot_bytes;
  std::vector<mk::PackInfo> packs;   // weights read in the packed layout
  mk_plan_stats stats{};
  int64_t n_instr = 0;
  int64_t epoch = 0;
  std::string unsupported;          // why the GPU path cannot run it ("" = runnable)
  std::vector<std::vector<float>> const_data;  // by slot: contents of constant tables
  mk_plan_device* dev = nullptr;
  int noalloc_device = -1;          // device of the last megakernel_run_noalloc call
};

namespace mk {
void set_error(const std::string& msg);
int dtype_bytes(mk_dtype d);
}  // namespace mk
