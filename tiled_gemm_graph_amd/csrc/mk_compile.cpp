// Host compiler: graph -> flat list of tile instructions with per-tile
// dependency counters.
//
// Phases follow "MegaKittens Internals", section 04 (count and place, tensor
// slots with a reuse pool, fine-grained barriers from unit cells, emit) and
// section 05 (instruction i on CU i % num_cus, iteration i / num_cus).  The
// lowering of a GEMM into split-K partial + reduce nodes, and epilogues as
// instruction flags, follow "Implementing a Mega Kernel for B300", section 2.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <numeric>
#include <set>
#include <string>
#include <unordered_map>

#include "mk_internal.h"

namespace mk {

static thread_local std::string g_err;
void set_error(const std::string& m) { g_err = m; }
int dtype_bytes(mk_dtype d) { return d == MK_F32 || d == MK_I32 ? 4 : 2; }

namespace {

struct Fail {
  mk_status st;
  std::string msg;
};
[[noreturn]] void fail(mk_status st, const std::string& msg) { throw Fail{st, msg}; }
I64 cdiv(I64 a, I64 b) { return (a + b - 1) / b; }
I64 numel(const Shape4& s) { return s[0] * s[1] * s[2] * s[3]; }

Edge edge_of(const std::vector<Tensor>& t, int id) {
  const Tensor& x = t[id];
  Edge e;
  if (x.is_view) {
    e.tensor = x.root;
    e.lo = x.lo;
    e.hi = x.hi;
  } else {
    e.tensor = id;
    e.lo = {0, 0, 0, 0};
    e.hi = x.shape;
  }
  return e;
}

bool is2d(const Edge& e) { return e.hi[0] - e.lo[0] == 1 && e.hi[1] - e.lo[1] == 1; }

Box box2(const Edge& e, I64 r0, I64 r1, I64 c0, I64 c1) {
  if (!(0 <= r0 && r0 <= r1 && r1 <= e.rows() && 0 <= c0 && c0 <= c1 && c1 <= e.cols()))
    fail(MK_E_INVALID, "internal: box outside its view");
  Box b;
  b.lo = {e.lo[0], e.lo[1], e.lo[2] + r0, e.lo[3] + c0};
  b.hi = {e.hi[0], e.hi[1], e.lo[2] + r1, e.lo[3] + c1};
  return b;
}

Box full_box(const Tensor& t) { return Box{{0, 0, 0, 0}, t.shape}; }

// K cut into `S` chunks of roundup(ceil(K/S), 64) rows, none empty.
std::vector<std::pair<I64, I64>> k_chunks(I64 K, I64 S) {
  I64 kc = cdiv(cdiv(K, S), 64) * 64;
  std::vector<std::pair<I64, I64>> ch;
  for (I64 s = 0; s < S; ++s) {
    I64 k0 = s * kc, k1 = std::min(K, (s + 1) * kc);
    if (k0 >= k1) fail(MK_E_INVALID, "split leaves an empty K chunk");
    ch.push_back({k0, k1});
  }
  return ch;
}

bool chunks_ok(I64 K, I64 S) {
  I64 kc = cdiv(cdiv(K, S), 64) * 64;
  return (S - 1) * kc < K;
}

// Largest activation chunk (rows x K elements) a GEMV instruction stages in
// LDS as fp32: one row may take up to 16384 elements, more rows 8192 in all.
I64 gemv_x_limit(I64 rows) { return rows <= 1 ? 16384 : 8192; }

// Output columns of packed-tile positions [c0, c1) as contiguous runs.
// With hd > 0, positions [0, rope_cols) interleave each head's rotation
// pairs: position p of head h = p / hd, i = (p % hd) / 2, is column
// h * hd + i + (p % 2) * hd / 2.  c0 and every head boundary are even.
std::vector<std::pair<I64, I64>> pos_runs(I64 c0, I64 c1, I64 hd, I64 rope_cols) {
  std::vector<std::pair<I64, I64>> r;
  I64 p = c0;
  if (hd > 0) {
    while (p < c1 && p < rope_cols) {
      const I64 h = p / hd, pe = std::min(std::min(c1, (h + 1) * hd), rope_cols);
      const I64 i0 = (p - h * hd) / 2, i1 = (pe - h * hd + 1) / 2;
      r.push_back({h * hd + i0, h * hd + i1});
      r.push_back({h * hd + hd / 2 + i0, h * hd + hd / 2 + i1});
      p = pe;
    }
  }
  if (p < c1) r.push_back({p, c1});
  return r;
}

struct Compiler {
  const mk_graph& g;
  mk_plan& p;
  int ncu;
  std::string unsupported;  // first reason the GPU path cannot run this plan

  Compiler(const mk_graph& g_, mk_plan& p_) : g(g_), p(p_) { ncu = p.opts.num_cus; }

  int add_internal(mk_dtype dt, Shape4 shape) {
    Tensor t;
    t.dt = dt;
    t.role = MK_INTERMEDIATE;
    t.ndim = 4;
    t.shape = shape;
    t.internal = true;
    p.tensors.push_back(t);
    return (int)p.tensors.size() - 1;
  }

  void unsup(const std::string& why) {
    if (unsupported.empty()) unsupported = why;
  }

  // ---------------------------------------------------------------- tiles
  // b_produced: B is written by an earlier op.  The GEMV body streams B
  // before the instruction's counters clear (only weights may be read that
  // early, MegaKittens Internals, section 09), so such a GEMM takes the
  // GEMM body, whose loads all follow the wait.
  mk_tile choose_gemm_tile(const OpRec& op, I64 M, I64 N, I64 K, bool silu, int dt,
                           bool packable, bool b_produced) {
    mk_tile t = op.attrs.tile;
    if (t.dup <= 0) t.dup = 1;
    if (t.gemv < 0 || t.gemv > 1) fail(MK_E_INVALID, "tile.gemv must be 0 or 1");
    if (t.layout < 0 || t.layout > 2) fail(MK_E_INVALID, "tile.layout must be 0, 1 or 2");
    if (t.layout == 2 && !packable)
      fail(MK_E_INVALID, "a packed weight must be a whole 2-D weight tensor read by no other op");
    const bool explicit_gemv = op.attrs.tile.gemv != 0 || op.attrs.tile.bm != 0;
    if (!explicit_gemv && M <= p.opts.gemv_max_m && !b_produced) t.gemv = 1;
    const bool rope = op.attrs.epilogue & MK_EP_ROPE;
    const I64 hd = op.attrs.head_dim > 0 ? op.attrs.head_dim : 1;
    if (t.gemv) {
      if (t.layout == 0) {
        // Packed column tiles need no K split and no REDUCE node; they pay
        // when there are enough 8-column tiles to give every CU one.
        const bool wide = cdiv(N, 8) >= ncu;
        t.layout = (packable && t.split <= 1 && (p.opts.pack == 2 || (p.opts.pack == 0 && wide))) ? 2 : 1;
      }
      if (t.layout == 2) {
        if (t.split > 1) fail(MK_E_INVALID, "packed GEMV tiles take no K split");
        if (t.bm <= 0) t.bm = (int)std::max<I64>(M, 1);
        if (t.bn <= 0) t.bn = (int)std::max<I64>(8, cdiv(cdiv(N, ncu), 8) * 8);
        t.split = 1;
        if (t.rbm <= 0) t.rbm = t.bm;
        if (t.rbn <= 0) t.rbn = t.bn;
        return t;
      }
      if (t.bm <= 0) t.bm = (int)std::max<I64>(M, 1);
      const I64 rows = std::min<I64>(std::max<I64>(M, 1), t.bm);
      // Streaming GEMV: pick the weight-tile width and the K split that
      // minimise a makespan estimate: waves of CUs times (per-instruction
      // overhead + bytes loaded / per-CU bandwidth), with 32-512 KB of
      // weights per instruction and the activation chunk small enough for
      // LDS.  192 threads stream the tile, 8 columns each, so the per-CU
      // bandwidth scales with the fraction of them a width keeps busy, and
      // the bytes loaded include the rounding of each thread's rows up to
      // whole 4-row batches.
      const double bw_cu = 22e3;   // bytes per microsecond per CU
      const double ovh = 2.5;      // microseconds per instruction
      const int eb = dtype_bytes((mk_dtype)dt);
      double best = 1e300;
      int best_bn = t.bn > 0 ? t.bn : (silu ? 128 : 256), best_s = t.split > 0 ? t.split : 1;
      const int bns[] = {768, 512, 448, 384, 320, 256, 224, 192, 128, 96, 64};  // wide first on ties
      for (int bn : bns) {
        if (t.bn > 0 && bn != t.bn) continue;
        const I64 wc = (I64)bn * (silu ? 2 : 1);
        if (wc > 1536 || bn > std::max<I64>(N, 8)) continue;
        const I64 tiles = cdiv(std::max<I64>(M, 1), t.bm) * cdiv(N, bn);
        for (I64 s = 1; s <= 128; ++s) {
          if (t.split > 0 && s != t.split) continue;
          if (!chunks_ok(K, s)) continue;
          const I64 kc = std::min<I64>(K, cdiv(cdiv(K, s), 64) * 64);
          if (kc * rows > gemv_x_limit(rows)) continue;
          const double bytes = (double)kc * wc * eb;
          if (bytes > 512 * 1024.0 || (bytes < 32 * 1024.0 && s > 1)) continue;
          const I64 ncg = wc / 8, kpar = 192 / ncg;
          const I64 loaded_rows = kpar * cdiv(cdiv(kc, kpar), 4) * 4;   // 4-row batches
          const double active = (double)(kpar * ncg) / 192.0;
          const double loaded = (double)loaded_rows * wc * eb;
          const double cost = (double)cdiv(tiles * s, ncu) * (ovh + loaded / (bw_cu * active));
          if (cost < best * (1 - 1e-9)) {
            best = cost;
            best_bn = bn;
            best_s = (int)s;
          }
        }
      }
      if (t.bn <= 0) t.bn = best_bn;
      if (t.split <= 0) t.split = best_s;
      if (t.rbm <= 0) t.rbm = t.bm;
      if (t.rbn <= 0) t.rbn = 256;
      return t;
    }
    // GEMM body.  Packed weights take the LDS-streamed body with 128/256
    // tiles; the row-major body keeps 64/128 tiles.
    if (t.layout == 0) {
      const int wbn = t.bn * (silu ? 2 : 1);
      const bool shape_ok = (t.bm == 0 || t.bm == 128 || t.bm == 256) && (t.bn == 0 || wbn == 128 || wbn == 256);
      t.layout = (packable && p.opts.pack != 1 && shape_ok && K % 64 == 0 && (!rope || hd == 64 || hd == 128))
                     ? 2 : 1;
    }
    if (t.layout == 2) {
      // Makespan estimate over tile shapes and K splits: waves of CUs times
      // the tile's MFMA time at an efficiency that grows with the tile (its
      // flops per byte staged), plus a per-instruction overhead, plus the
      // fp32 partial traffic and the REDUCE hop of a split.
      struct Cand { int bm, bn; double eff; };
      // (256 x 256 would need all 256 accumulator registers of a wave, more
      // than the persistent kernel can spare beside its other bodies.)  The
      // efficiencies are measured ones: a 128 x 128 tile reaches about 0.6
      // of peak on the M = 256, K = 8192 chains, where it avoids a split-K
      // reduction that 256 x 128 would need to fill the CUs.
      const Cand cands[] = {{256, 128, 0.62}, {128, 256, 0.62}, {128, 128, 0.60}};
      const double peak_cu = 2.5e15 / 256.0 / 1e6;   // flops per microsecond per CU
      double best = 1e300;
      int bbm = 0, bbn = 0, bs = 1;
      for (const Cand& c : cands) {
        if (t.bm > 0 && c.bm != t.bm) continue;
        if (t.bn > 0 && c.bn != t.bn * (silu ? 2 : 1)) continue;
        if (rope && c.bn % hd) continue;
        const I64 bn_out = silu ? c.bn / 2 : c.bn;
        const I64 tiles = cdiv(std::max<I64>(M, 1), c.bm) * cdiv(N, bn_out);
        for (I64 sp = 1; sp <= 16; ++sp) {
          if (t.split > 0 && sp != t.split) continue;
          if (!chunks_ok(K, sp)) continue;
          const I64 kc = std::min<I64>(K, cdiv(cdiv(K, sp), 64) * 64);
          const double t_inst = 2.0 * c.bm * c.bn * kc / (peak_cu * c.eff) + 2.0;
          double cost = (double)cdiv(tiles * sp, ncu) * t_inst;
          if (sp > 1) cost += 8.0 * sp * M * (silu ? 2 * N : N) / 5e6 + 6.0;
          if (cost < best * (1 - 1e-9)) {
            best = cost;
            bbm = c.bm;
            bbn = c.bn;
            bs = (int)sp;
          }
        }
      }
      if (bbm == 0) fail(MK_E_INVALID, "no packed GEMM tile fits these tile parameters");
      t.bm = bbm;
      t.bn = silu ? bbn / 2 : bbn;   // tile.bn counts output columns
      t.split = bs;
      // REDUCE tiles of at most 16384 fp32 sums (64 KB of LDS), so that
      // the eight-wave REDUCE body fits beside its per-thread partials; and
      // rows halved (down to 32) while that leaves CUs without a REDUCE
      // instruction: the node is latency-bound, so more, smaller tiles
      // finish sooner
      const bool auto_rows = t.rbm <= 0;
      if (t.rbm <= 0) t.rbm = std::min(t.bm, 128);
      if (t.rbn <= 0) {
        const int cap = 16384 / (t.rbm * (silu ? 2 : 1));
        t.rbn = std::max(8, std::min(t.bn, cap / 8 * 8));
      }
      if (t.split > 1 && auto_rows)
        while (t.rbm > 32 && cdiv(std::max<I64>(M, 1), t.rbm) * cdiv(N, t.rbn) < ncu) t.rbm /= 2;
      return t;
    }
    if (t.bm <= 0 || t.bn <= 0) {
      // Largest kernel tile that still fills one wave of CUs.
      // Rotary tiles must hold whole heads.
      const int cand[3][2] = {{128, 128}, {64, 128}, {64, 64}};
      int pick = rope ? 1 : 2;
      for (int c = 0; c < 3; ++c) {
        int bnk = cand[c][1];
        int bn = silu ? bnk / 2 : bnk;
        if (rope && bn % hd) continue;
        if (cdiv(M, cand[c][0]) * cdiv(N, bn) >= ncu) {
          pick = c;
          break;
        }
      }
      if (t.bm <= 0) t.bm = cand[pick][0];
      if (t.bn <= 0) t.bn = silu ? cand[pick][1] / 2 : cand[pick][1];
    }
    if (t.split <= 0) t.split = 1;
    if (t.rbm <= 0) t.rbm = t.bm;
    if (t.rbn <= 0) t.rbn = t.bn;
    return t;
  }

  // ------------------------------------------------------------- lowering
  std::vector<int> uses;  // op inputs naming each root tensor

  void lower() {
    uses.assign(p.tensors.size(), 0);
    for (const OpRec& op : g.ops)
      for (int i : op.in) uses[edge_of(p.tensors, i).tensor]++;
    for (size_t oi = 0; oi < g.ops.size(); ++oi) {
      const OpRec& op = g.ops[oi];
      mk_tile tile{};
      switch (op.kind) {
        case MK_OP_GEMM: tile = lower_gemm((int)oi, op); break;
        case MK_OP_RMSNORM: tile = lower_rmsnorm((int)oi, op); break;
        case MK_OP_ATTENTION: tile = lower_attention((int)oi, op); break;
        case MK_OP_ADD:
        case MK_OP_RELU: tile = lower_elementwise((int)oi, op); break;
        case MK_OP_DECODE_ATTENTION: tile = lower_decode_attention((int)oi, op); break;
        default: fail(MK_E_INVALID, "unknown op kind");
      }
      p.op_tiles.push_back(tile);
    }
  }

  mk_tile lower_gemm(int oi, const OpRec& op) {
    const auto& T = p.tensors;
    const uint32_t fl = op.attrs.epilogue;
    Edge A = edge_of(T, op.in[0]), B = edge_of(T, op.in[1]);
    int ai = 2;
    Edge bias, res, gamma;
    if (fl & MK_EP_BIAS) bias = edge_of(T, op.in[ai++]);
    if (fl & MK_EP_RESIDUAL) res = edge_of(T, op.in[ai++]);
    if (fl & MK_EP_RMSNORM_INPUT) gamma = edge_of(T, op.in[ai++]);
    const Tensor& O = T[op.out];
    if (!is2d(A) || !is2d(B)) fail(MK_E_INVALID, "GEMM operands must be 2-D views");
    if (O.shape[0] != 1 || O.shape[1] != 1) fail(MK_E_INVALID, "GEMM output must be 2-D");
    I64 M = A.rows(), K = A.cols(), N = O.shape[3];
    bool silu = fl & MK_EP_SILU_MUL;
    I64 Nb = silu ? 2 * N : N;
    if (O.shape[2] != M) fail(MK_E_INVALID, "GEMM output rows != A rows");
    if (B.rows() != K || B.cols() != Nb)
      fail(MK_E_INVALID, "GEMM B must be [K, N] (or [K, 2N] with SILU_MUL)");
    for (const Edge* e : {&bias, &res}) {
      if (e->tensor < 0) continue;
      if (!is2d(*e) || e->rows() != M || e->cols() != N)
        fail(MK_E_INVALID, "GEMM bias/residual must be [M, N]");
    }
    if (gamma.tensor >= 0 && (gamma.rows() != 1 || gamma.cols() != K || !is2d(gamma)))
      fail(MK_E_INVALID, "GEMM gamma must have K elements");
    if (fl & MK_EP_PARTIAL) fail(MK_E_INVALID, "PARTIAL is set by the compiler only");
    mk_dtype dt = T[A.tensor].dt;
    if (T[B.tensor].dt != dt || O.dt != dt) fail(MK_E_INVALID, "GEMM dtypes differ");
    if (K < 1) fail(MK_E_INVALID, "GEMM needs K >= 1");
    // A weight may be packed when the op reads it whole and alone.
    bool packable = !T[op.in[1]].is_view && T[B.tensor].role == MK_WEIGHT && uses[B.tensor] == 1 &&
                    (dt == MK_F16 || dt == MK_BF16) && K % 8 == 0 && N % 8 == 0;
    const bool b_produced = T[B.tensor].role == MK_OUTPUT || T[B.tensor].role == MK_INTERMEDIATE;
    mk_tile t = choose_gemm_tile(op, M, N, K, silu, dt, packable, b_produced);
    if (t.bm <= 0 || t.bn <= 0 || t.split <= 0 || t.dup <= 0)
      fail(MK_E_INVALID, "bad GEMM tile");
    int S = t.split;
    auto chunks = k_chunks(std::max<I64>(K, 1), S);
    bool gemv = t.gemv != 0;
    const bool packed = gemv && t.layout == 2;       // GEMV column tiles
    const bool packed_gemm = !gemv && t.layout == 2;  // GEMM K tiles
    int opcode = gemv ? MK_I_GEMV : MK_I_GEMM;
    // kernel support
    if (dt != MK_F16 && dt != MK_BF16) unsup("GEMM dtype must be fp16 or bf16");
    if (N % 8) unsup("GEMM N must be a multiple of 8");
    if (gemv) {
      int wc = t.bn * (silu ? 2 : 1);
      if (b_produced) unsup("the GEMV body reads B before its counters clear: B must be a weight or input");
      if (t.bm > 8) unsup("GEMV body handles at most 8 rows per tile");
      if (wc > 1536 || wc % 8) unsup("GEMV weight tile must be <= 1536 columns, multiple of 8");
      if (K % 8) unsup("GEMV K must be a multiple of 8");
      {
        const I64 kc = std::min<I64>(K, cdiv(cdiv(K, S), 64) * 64);
        const I64 rows = std::min<I64>(std::max<I64>(M, 1), t.bm);
        if (kc * rows > gemv_x_limit(rows))
          unsup("GEMV activation chunk exceeds 16384 elements (one row) or 8192 (more rows)");
      }
      if (packed && (t.bn % 8 || t.dup != 1)) unsup("packed GEMV tiles are multiples of 8 columns");
    } else if (packed_gemm) {
      int bnk = t.bn * (silu ? 2 : 1);
      if (!((t.bm == 128 || t.bm == 256) && (bnk == 128 || bnk == 256)) || (t.bm == 256 && bnk == 256))
        unsup("packed GEMM tiles are 256 x 128, 128 x 256 or 128 x 128 (rows x weight columns)");
      if (K % 64) unsup("GEMM K must be a multiple of 64");
      if (A.lo[3] % 8 || T[A.tensor].shape[3] % 8) unsup("packed GEMM A rows must be 16-byte aligned");
      if (fl & MK_EP_RMSNORM_INPUT) unsup("RMSNORM_INPUT needs the GEMV body");
      if (t.dup != 1) unsup("duplicated tiles are a host profile only");
      if ((fl & MK_EP_ROPE) && S == 1) {
        const int hd = op.attrs.head_dim;
        // the epilogue reads a rotary partner (half a head away) from the
        // tile's fp32 LDS strip, so a tile must hold whole heads
        if ((hd != 64 && hd != 128) || bnk % hd)
          unsup("ROPE on a packed GEMM tile needs head_dim 64 or 128 and whole heads in a tile");
      }
    } else {
      int bnk = t.bn * (silu ? 2 : 1);
      if (!((t.bm == 64 || t.bm == 128) && (bnk == 64 || bnk == 128)))
        unsup("GEMM kernel tiles are 64 or 128 rows x 64 or 128 weight columns");
      if (K % 64) unsup("GEMM K must be a multiple of 64");
      if (fl & MK_EP_RMSNORM_INPUT) unsup("RMSNORM_INPUT needs the GEMV body");
      if (t.dup != 1) unsup("duplicated tiles are a host profile only");
    }
    if (fl & MK_EP_ROPE) {
      int hd = op.attrs.head_dim;
      int rc = op.attrs.rope_cols ? op.attrs.rope_cols : (int)N;
      if (hd <= 0 || hd % 2 || hd > 256) fail(MK_E_INVALID, "ROPE needs an even head_dim <= 256");
      if (rc % hd || rc > N) fail(MK_E_INVALID, "rope_cols must be a multiple of head_dim <= N");
      int tbn = S > 1 ? t.rbn : t.bn;
      if (!packed && !(packed_gemm && S == 1) && tbn % hd) unsup("ROPE tiles must hold whole heads");
      if (hd % 16) unsup("ROPE head_dim must be a multiple of 16");
      if (silu) fail(MK_E_INVALID, "ROPE and SILU_MUL cannot be combined");
    }
    if (gemv && !packed && S == 1 && (fl & MK_EP_ROPE)) unsup("ROPE on the row-major GEMV body needs a split");
    // The REDUCE body keeps its tile's fp32 sums in the 144 KB LDS arena
    // beside 320 floats of row scales and 8 floats per thread (256 threads).
    // (and a row scale for each of at most 256 rows)
    if (S > 1 && ((320 + 256 * 8 + (I64)t.rbm * t.rbn * (silu ? 2 : 1)) * 4 > 144 * 1024 || t.rbm > 256))
      unsup("REDUCE tile (rbm x rbn, twice the columns under SILU_MUL) exceeds the LDS arena");
    int pt = -1;
    if (S > 1) pt = add_internal(MK_F32, {1, S, M, Nb});
    int rope_t = -1;
    if (fl & MK_EP_ROPE) {
      rope_t = add_internal(MK_F32, {1, 1, std::max<I64>(M, 1), op.attrs.head_dim});
      p.tensors[rope_t].const_kind = 1;
      p.tensors[rope_t].rope_half = op.attrs.head_dim / 2;
      p.tensors[rope_t].rope_theta = op.attrs.rope_theta > 0 ? op.attrs.rope_theta : 10000.f;
    }
    Edge out = edge_of(T, op.out);
    Node n;
    n.op = oi;
    n.opcode = opcode;
    n.flags = S == 1 ? (int)fl : (MK_EP_PARTIAL | (int)(fl & (MK_EP_SILU_MUL | MK_EP_RMSNORM_INPUT)));
    n.out = S == 1 ? op.out : pt;
    n.edges = {A, B};
    if (gamma.tensor >= 0) n.edges.push_back(gamma);
    if (S == 1) {
      if (bias.tensor >= 0) n.edges.push_back(bias);
      if (res.tensor >= 0) n.edges.push_back(res);
    }
    Edge P;
    if (S > 1) P = edge_of(p.tensors, pt);
    const I64 rope_cols = (fl & MK_EP_ROPE) ? (op.attrs.rope_cols ? op.attrs.rope_cols : N) : 0;
    for (const auto& tile_rc : tile_order(cdiv(M, t.bm), cdiv(N, t.bn), S, !gemv)) {
      {
        const I64 tm = tile_rc.first, tn = tile_rc.second;
        I64 r0 = tm * t.bm, r1 = std::min(M, r0 + t.bm);
        I64 c0 = tn * t.bn, c1 = std::min(N, c0 + t.bn);
        for (int s = 0; s < S; ++s) {
          I64 k0 = chunks[s].first, k1 = std::min(K, chunks[s].second);
          Instr in;
          in.coord[0] = (int32_t)tm;
          in.coord[1] = (int32_t)tn;
          in.coord[2] = s;
          in.r0 = (int32_t)r0; in.r1 = (int32_t)r1; in.c0 = (int32_t)c0; in.c1 = (int32_t)c1;
          in.k0 = (int32_t)k0; in.k1 = (int32_t)k1; in.s = s;
          in.reads.push_back({A.tensor, box2(A, r0, r1, k0, k1)});
          if (packed) {
            // positions [c0, c1) cover the columns of pos_runs
            const auto runs = pos_runs(c0, c1, (fl & MK_EP_ROPE) ? op.attrs.head_dim : 0, rope_cols);
            for (const auto& rc : runs) in.reads.push_back({B.tensor, box2(B, 0, K, rc.first, rc.second)});
            if (silu)
              for (const auto& rc : runs)
                in.reads.push_back({B.tensor, box2(B, 0, K, N + rc.first, N + rc.second)});
            if (fl & MK_EP_RMSNORM_INPUT) in.reads.push_back({gamma.tensor, box2(gamma, 0, 1, 0, K)});
            for (const auto& rc : runs) {
              if (fl & MK_EP_BIAS) in.reads.push_back({bias.tensor, box2(bias, r0, r1, rc.first, rc.second)});
              if (fl & MK_EP_RESIDUAL) in.reads.push_back({res.tensor, box2(res, r0, r1, rc.first, rc.second)});
            }
            for (const auto& rc : runs) in.writes.push_back({op.out, box2(out, r0, r1, rc.first, rc.second)});
            n.ins.push_back(in);
            continue;
          }
          in.reads.push_back({B.tensor, box2(B, k0, k1, c0, c1)});
          if (silu) in.reads.push_back({B.tensor, box2(B, k0, k1, N + c0, N + c1)});
          if (fl & MK_EP_RMSNORM_INPUT) in.reads.push_back({gamma.tensor, box2(gamma, 0, 1, k0, k1)});
          if (S == 1) {
            if (fl & MK_EP_BIAS) in.reads.push_back({bias.tensor, box2(bias, r0, r1, c0, c1)});
            if (fl & MK_EP_RESIDUAL) in.reads.push_back({res.tensor, box2(res, r0, r1, c0, c1)});
            in.writes.push_back({op.out, box2(out, r0, r1, c0, c1)});
          } else {
            Box b{{0, s, r0, c0}, {1, s + 1, r1, c1}};
            in.writes.push_back({pt, b});
            if (silu) in.writes.push_back({pt, Box{{0, s, r0, N + c0}, {1, s + 1, r1, N + c1}}});
          }
          for (int r = 0; r < t.dup; ++r) {
            Instr c = in;
            c.coord[3] = r;
            n.ins.push_back(c);
          }
        }
      }
    }
    // node descriptor (slots filled later)
    mk_node& d = n.desc;
    d.opcode = opcode;
    d.flags = n.flags;
    d.dtype = dt;
    d.M = (int32_t)M; d.N = (int32_t)N; d.K = (int32_t)K; d.Nb = (int32_t)Nb;
    d.split = S;
    d.eps = op.attrs.eps > 0 ? op.attrs.eps : 1e-6f;
    d.head_dim = op.attrs.head_dim;
    d.rope_cols = (fl & MK_EP_ROPE) ? (op.attrs.rope_cols ? op.attrs.rope_cols : (int)N) : 0;
    d.part_plane = M * Nb;
    d.tile_m = t.bm;
    d.tile_n = t.bn * (silu ? 2 : 1);
    d.layout = packed ? 1 : packed_gemm ? 2 : 0;
    if (packed_gemm) {
      PackInfo pk;
      pk.kind = 2;
      pk.tensor = B.tensor;
      pk.K = K;
      pk.N = N;
      pk.bn = d.tile_n;
      pk.wc = d.tile_n;
      pk.tiles = cdiv(N, t.bn);
      pk.silu = silu;
      pk.dt = dt;
      pk.bytes = pk.tiles * K * pk.wc * dtype_bytes(dt);
      p.packs.push_back(pk);
    }
    if (packed) {
      PackInfo pk;
      pk.tensor = B.tensor;
      pk.K = K;
      pk.N = N;
      pk.bn = t.bn;
      pk.wc = d.tile_n;
      pk.tiles = cdiv(N, t.bn);
      pk.silu = silu;
      pk.head_dim = (fl & MK_EP_ROPE) ? op.attrs.head_dim : 0;
      pk.rope_cols = rope_cols;
      pk.dt = dt;
      pk.bytes = pk.tiles * K * pk.wc * dtype_bytes(dt);
      p.packs.push_back(pk);
    }
    p.nodes.push_back(n);
    node_edges.push_back({{"a", A}, {"b", B}, {"gamma", gamma},
                          {"bias", S == 1 ? bias : Edge{}}, {"res", S == 1 ? res : Edge{}},
                          {"out", S == 1 ? out : Edge{}}, {"part", S > 1 ? P : Edge{}},
                          {"aux", rope_t >= 0 && S == 1 ? edge_of(p.tensors, rope_t) : Edge{}}});
    if (S > 1) {
      Node r;
      r.op = oi;
      r.opcode = MK_I_REDUCE;
      r.flags = (int)fl;
      r.out = op.out;
      r.edges = {P};
      if (bias.tensor >= 0) r.edges.push_back(bias);
      if (res.tensor >= 0) r.edges.push_back(res);
      if (fl & MK_EP_RMSNORM_INPUT) r.edges.push_back(A);
      for (I64 tm = 0; tm < cdiv(M, t.rbm); ++tm)
        for (I64 tn = 0; tn < cdiv(N, t.rbn); ++tn) {
          I64 r0 = tm * t.rbm, r1 = std::min(M, r0 + t.rbm);
          I64 c0 = tn * t.rbn, c1 = std::min(N, c0 + t.rbn);
          Instr in;
          in.coord[0] = (int32_t)tm;
          in.coord[1] = (int32_t)tn;
          in.r0 = (int32_t)r0; in.r1 = (int32_t)r1; in.c0 = (int32_t)c0; in.c1 = (int32_t)c1;
          in.k0 = 0; in.k1 = (int32_t)K;
          in.reads.push_back({pt, Box{{0, 0, r0, c0}, {1, S, r1, c1}}});
          if (silu) in.reads.push_back({pt, Box{{0, 0, r0, N + c0}, {1, S, r1, N + c1}}});
          if (fl & MK_EP_BIAS) in.reads.push_back({bias.tensor, box2(bias, r0, r1, c0, c1)});
          if (fl & MK_EP_RESIDUAL) in.reads.push_back({res.tensor, box2(res, r0, r1, c0, c1)});
          if (fl & MK_EP_RMSNORM_INPUT) in.reads.push_back({A.tensor, box2(A, r0, r1, 0, K)});
          in.writes.push_back({op.out, box2(out, r0, r1, c0, c1)});
          r.ins.push_back(in);
        }
      mk_node& rd = r.desc;
      rd = d;
      rd.opcode = MK_I_REDUCE;
      rd.flags = (int)fl;
      p.nodes.push_back(r);
      node_edges.push_back({{"a", A}, {"out", out}, {"part", P},
                            {"bias", bias}, {"res", res},
                            {"aux", rope_t >= 0 ? edge_of(p.tensors, rope_t) : Edge{}}});
    }
    return t;
  }

  // Tile order of a GEMM node: groups of gm x gn tiles (gm = min(TM, 32),
  // gn = min(TN, max(1, B / (gm * S))), B = num_cus / 8 when num_cus is a
  // multiple of 8, else 32), groups row-major over the group grid, tiles
  // row-major inside a group.  A wave of num_cus consecutive instructions
  // then covers up to 32 row panels of A and few column panels of B, so
  // the weight panels a wave reads are reused by every row panel while
  // they are still in the memory-side cache (a 256-row panel at K = 8192
  // is 4 MB, the size of one XCD's L2).  Against groups of 4 row panels,
  // prefill measured 3.1 % and mlp3 2.4 % faster, the others the same.
  // Other nodes (grouped = false) run row-major.
  std::vector<std::pair<I64, I64>> tile_order(I64 TM, I64 TN, I64 S, bool grouped) const {
    std::vector<std::pair<I64, I64>> v;
    if (TM <= 0 || TN <= 0) return v;
    v.reserve(TM * TN);
    if (!grouped) {
      for (I64 tm = 0; tm < TM; ++tm)
        for (I64 tn = 0; tn < TN; ++tn) v.push_back({tm, tn});
      return v;
    }
    const I64 B = ncu % 8 == 0 ? ncu / 8 : 32;
    const I64 gm = std::min<I64>(TM, 32);
    const I64 gn = std::min<I64>(TN, std::max<I64>(1, B / (gm * S)));
    for (I64 g0 = 0; g0 < TM; g0 += gm)
      for (I64 h0 = 0; h0 < TN; h0 += gn)
        for (I64 tm = g0; tm < std::min(TM, g0 + gm); ++tm)
          for (I64 tn = h0; tn < std::min(TN, h0 + gn); ++tn) v.push_back({tm, tn});
    return v;
  }

  mk_tile lower_rmsnorm(int oi, const OpRec& op) {
    const auto& T = p.tensors;
    Edge x = edge_of(T, op.in[0]), gm = edge_of(T, op.in[1]), out = edge_of(T, op.out);
    if (!is2d(x) || !is2d(gm) || !is2d(out)) fail(MK_E_INVALID, "RMSNORM operands must be 2-D");
    I64 M = x.rows(), H = x.cols();
    if (gm.rows() != 1 || gm.cols() != H || out.rows() != M || out.cols() != H)
      fail(MK_E_INVALID, "RMSNORM shapes: x [M,H], gamma [H], out [M,H]");
    mk_dtype dt = T[x.tensor].dt;
    if (T[gm.tensor].dt != dt || T[out.tensor].dt != dt) fail(MK_E_INVALID, "RMSNORM dtypes differ");
    if (H % 8) unsup("RMSNORM H must be a multiple of 8");
    mk_tile t = op.attrs.tile;
    if (t.rows <= 0) t.rows = (int)std::max<I64>(1, M / ncu);
    Node n;
    n.op = oi;
    n.opcode = MK_I_RMSNORM;
    n.out = op.out;
    n.edges = {x, gm};
    for (I64 rb = 0; rb < cdiv(M, t.rows); ++rb) {
      I64 r0 = rb * t.rows, r1 = std::min(M, r0 + t.rows);
      Instr in;
      in.coord[0] = (int32_t)rb;
      in.r0 = (int32_t)r0; in.r1 = (int32_t)r1; in.c0 = 0; in.c1 = (int32_t)H;
      in.reads.push_back({x.tensor, box2(x, r0, r1, 0, H)});
      in.reads.push_back({gm.tensor, box2(gm, 0, 1, 0, H)});
      in.writes.push_back({op.out, box2(out, r0, r1, 0, H)});
      n.ins.push_back(in);
    }
    mk_node& d = n.desc;
    d.opcode = MK_I_RMSNORM;
    d.dtype = dt;
    d.M = (int32_t)M; d.N = (int32_t)H; d.K = (int32_t)H;
    d.eps = op.attrs.eps > 0 ? op.attrs.eps : 1e-6f;
    p.nodes.push_back(n);
    node_edges.push_back({{"a", x}, {"gamma", gm}, {"out", out}});
    return t;
  }

  mk_tile lower_attention(int oi, const OpRec& op) {
    const auto& T = p.tensors;
    Edge q = edge_of(T, op.in[0]), k = edge_of(T, op.in[1]), v = edge_of(T, op.in[2]);
    Edge o = edge_of(T, op.out);
    int Hq = op.attrs.n_heads, Hkv = op.attrs.n_kv_heads, d = op.attrs.head_dim;
    if (Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) fail(MK_E_INVALID, "ATTENTION heads");
    if (!is2d(q) || !is2d(k) || !is2d(v) || !is2d(o)) fail(MK_E_INVALID, "ATTENTION operands must be 2-D");
    I64 S = q.rows();
    if (q.cols() != (I64)Hq * d || k.cols() != (I64)Hkv * d || v.cols() != (I64)Hkv * d ||
        k.rows() != S || v.rows() != S || o.rows() != S || o.cols() != (I64)Hq * d)
      fail(MK_E_INVALID, "ATTENTION shapes: q [S, Hq*d], k/v [S, Hkv*d], o [S, Hq*d]");
    mk_dtype dt = T[q.tensor].dt;
    if (T[k.tensor].dt != dt || T[v.tensor].dt != dt || T[o.tensor].dt != dt)
      fail(MK_E_INVALID, "ATTENTION dtypes differ");
    if (d != 128) unsup("ATTENTION body needs head_dim 128");
    mk_tile t = op.attrs.tile;
    if (t.bq <= 0) t.bq = 128;
    if (t.bq != 128) unsup("ATTENTION body handles 128 query rows per instruction");
    bool causal = op.attrs.causal != 0;
    Node n;
    n.op = oi;
    n.opcode = MK_I_ATTENTION;
    n.out = op.out;
    n.edges = {q, k, v};
    I64 nqb = cdiv(S, t.bq);
    for (I64 qb = nqb - 1; qb >= 0; --qb) {
      I64 q0 = qb * t.bq, q1 = std::min(S, q0 + t.bq);
      I64 kend = causal ? q1 : S;  // keys the body visits; the boxes cover all S rows
                                   // so q blocks of one kv head share a dependency set
      for (int h = 0; h < Hq; ++h) {
        int kh = h / (Hq / Hkv);
        Instr in;
        in.coord[0] = (int32_t)qb;
        in.coord[1] = h;
        in.r0 = (int32_t)q0; in.r1 = (int32_t)q1; in.c0 = h; in.c1 = kh;
        in.k0 = 0; in.k1 = (int32_t)kend;
        in.reads.push_back({q.tensor, box2(q, q0, q1, (I64)h * d, (I64)h * d + d)});
        in.reads.push_back({k.tensor, box2(k, 0, S, (I64)kh * d, (I64)kh * d + d)});
        in.reads.push_back({v.tensor, box2(v, 0, S, (I64)kh * d, (I64)kh * d + d)});
        in.writes.push_back({op.out, box2(o, q0, q1, (I64)h * d, (I64)h * d + d)});
        n.ins.push_back(in);
      }
    }
    // Instruction j runs on the same CU as j + num_cus.  The list runs from
    // the most keys (last query block) to the fewest, and every other run of
    // num_cus instructions is reversed, so each CU's blocks add up to about
    // the same work under the causal mask (a static form of longest-first
    // scheduling).
    for (size_t c0 = ncu; c0 < n.ins.size(); c0 += 2 * (size_t)ncu)
      std::reverse(n.ins.begin() + c0, n.ins.begin() + std::min(n.ins.size(), c0 + (size_t)ncu));
    mk_node& dd = n.desc;
    dd.opcode = MK_I_ATTENTION;
    dd.dtype = dt;
    dd.M = (int32_t)S; dd.N = Hq * d;
    dd.heads = Hq; dd.kv_heads = Hkv; dd.head_dim = d; dd.causal = causal; dd.seq = (int32_t)S;
    dd.scale = 1.0f / std::sqrt((float)d);
    p.nodes.push_back(n);
    node_edges.push_back({{"a", q}, {"b", k}, {"aux", v}, {"out", o}});
    return t;
  }

  mk_tile lower_elementwise(int oi, const OpRec& op) {
    const auto& T = p.tensors;
    bool add = op.kind == MK_OP_ADD;
    Edge a = edge_of(T, op.in[0]), o = edge_of(T, op.out);
    Edge b;
    if (add) b = edge_of(T, op.in[1]);
    if (!is2d(a) || !is2d(o) || (add && !is2d(b))) fail(MK_E_INVALID, "elementwise operands must be 2-D");
    I64 M = a.rows(), N = a.cols();
    if (o.rows() != M || o.cols() != N || (add && (b.rows() != M || b.cols() != N)))
      fail(MK_E_INVALID, "elementwise shapes differ (no broadcasting)");
    mk_dtype dt = T[a.tensor].dt;
    if (T[o.tensor].dt != dt || (add && T[b.tensor].dt != dt)) fail(MK_E_INVALID, "elementwise dtypes differ");
    if (N % 8) unsup("elementwise N must be a multiple of 8");
    mk_tile t = op.attrs.tile;
    if (t.er <= 0) t.er = 64;
    if (t.ec <= 0) t.ec = 256;
    Node n;
    n.op = oi;
    n.opcode = add ? MK_I_EW_ADD : MK_I_EW_RELU;
    n.out = op.out;
    n.edges = {a};
    if (add) n.edges.push_back(b);
    for (I64 tr = 0; tr < cdiv(M, t.er); ++tr)
      for (I64 tc = 0; tc < cdiv(N, t.ec); ++tc) {
        I64 r0 = tr * t.er, r1 = std::min(M, r0 + t.er);
        I64 c0 = tc * t.ec, c1 = std::min(N, c0 + t.ec);
        Instr in;
        in.coord[0] = (int32_t)tr;
        in.coord[1] = (int32_t)tc;
        in.r0 = (int32_t)r0; in.r1 = (int32_t)r1; in.c0 = (int32_t)c0; in.c1 = (int32_t)c1;
        in.reads.push_back({a.tensor, box2(a, r0, r1, c0, c1)});
        if (add) in.reads.push_back({b.tensor, box2(b, r0, r1, c0, c1)});
        in.writes.push_back({op.out, box2(o, r0, r1, c0, c1)});
        n.ins.push_back(in);
      }
    mk_node& d = n.desc;
    d.opcode = n.opcode;
    d.dtype = dt;
    d.M = (int32_t)M; d.N = (int32_t)N;
    p.nodes.push_back(n);
    node_edges.push_back({{"a", a}, {"b", add ? b : Edge{}}, {"out", o}});
    return t;
  }

  // Split-KV decode attention ("Implementing a Mega Kernel for B300",
  // section 2, flash-decoding): a partial node of one instruction per (key
  // chunk c, kv head g), which rotates q and k_new at the run-time position
  // p, appends the rotated k_new and v_new to row p of the caches (the
  // instruction whose chunk holds p), and writes, for each query head of
  // the group, the chunk's running max m, sum of exp2 l and unnormalised
  // output (fp32) to P [chunks, Hq, d + 4]; then a combine node of one
  // instruction per kv head that merges the chunks j0 <= p by log-sum-exp
  // and writes o.  Operand slots of the partial node's descriptor: a = q,
  // b = k_new, res = v_new, bias = k_cache, gamma = v_cache, out = P,
  // aux = rotary table [S_max, d], part = pos; combine: a = P, out = o,
  // part = pos.
  mk_tile lower_decode_attention(int oi, const OpRec& op) {
    const auto& T = p.tensors;
    Edge q = edge_of(T, op.in[0]), kn = edge_of(T, op.in[1]), vn = edge_of(T, op.in[2]);
    Edge kc = edge_of(T, op.in[3]), vc = edge_of(T, op.in[4]), ps = edge_of(T, op.in[5]);
    Edge o = edge_of(T, op.out);
    const int Hq = op.attrs.n_heads, Hkv = op.attrs.n_kv_heads, d = op.attrs.head_dim;
    if (Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) fail(MK_E_INVALID, "DECODE_ATTENTION heads");
    for (const Edge* e : {&q, &kn, &vn, &kc, &vc, &o})
      if (!is2d(*e)) fail(MK_E_INVALID, "DECODE_ATTENTION operands must be 2-D");
    if (q.rows() != 1 || kn.rows() != 1 || vn.rows() != 1 || o.rows() != 1)
      fail(MK_E_INVALID, "DECODE_ATTENTION decodes one token: q, k_new, v_new and o have one row");
    if (q.cols() != (I64)Hq * d || o.cols() != (I64)Hq * d || kn.cols() != (I64)Hkv * d ||
        vn.cols() != (I64)Hkv * d)
      fail(MK_E_INVALID, "DECODE_ATTENTION shapes: q, o [1, Hq*d]; k_new, v_new [1, Hkv*d]");
    const I64 S = kc.rows();
    if (S < 1 || vc.rows() != S || kc.cols() != (I64)Hkv * d || vc.cols() != (I64)Hkv * d)
      fail(MK_E_INVALID, "DECODE_ATTENTION caches must be [S_max, Hkv*d]");
    for (const Edge* e : {&kc, &vc}) {
      const Tensor& t = T[e->tensor];
      if (T[op.in[e == &kc ? 3 : 4]].is_view || t.role != MK_INPUT)
        fail(MK_E_INVALID, "DECODE_ATTENTION caches must be whole caller-owned INPUT tensors");
    }
    {
      const Tensor& t = T[ps.tensor];
      if (t.dt != MK_I32 || t.role != MK_INPUT || numel(t.shape) != 1 || T[op.in[5]].is_view)
        fail(MK_E_INVALID, "DECODE_ATTENTION pos must be a one-element MK_I32 INPUT tensor");
    }
    const mk_dtype dt = T[q.tensor].dt;
    for (const Edge* e : {&kn, &vn, &kc, &vc, &o})
      if (T[e->tensor].dt != dt) fail(MK_E_INVALID, "DECODE_ATTENTION dtypes differ");
    if (dt != MK_F16 && dt != MK_BF16) unsup("DECODE_ATTENTION dtype must be fp16 or bf16");
    if (d != 128) unsup("DECODE_ATTENTION body needs head_dim 128");
    const int G = Hq / Hkv;
    if (G > 8) unsup("DECODE_ATTENTION body handles at most 8 query heads per kv head");
    mk_tile t = op.attrs.tile;
    if (t.bq <= 0) {
      const I64 per = cdiv(S * Hkv, ncu);
      t.bq = (int)std::min<I64>(256, std::max<I64>(64, cdiv(per, 64) * 64));
    }
    if (t.bq % 64 || t.bq > 256) unsup("DECODE_ATTENTION chunks are 64, 128, 192 or 256 keys");
    const I64 C = t.bq, NC = cdiv(S, C), W = d + 4;
    const int pt = add_internal(MK_F32, {1, NC, Hq, W});
    const int rope_t = add_internal(MK_F32, {1, 1, S, d});
    p.tensors[rope_t].const_kind = 1;
    p.tensors[rope_t].rope_half = d / 2;
    p.tensors[rope_t].rope_theta = op.attrs.rope_theta > 0 ? op.attrs.rope_theta : 10000.f;
    Edge P = edge_of(p.tensors, pt);
    Node n;
    n.op = oi;
    n.opcode = MK_I_ATTN_PARTIAL;
    n.out = pt;
    n.edges = {q, kn, vn, kc, vc, ps};
    for (I64 c = 0; c < NC; ++c)
      for (int g = 0; g < Hkv; ++g) {
        Instr in;
        in.coord[0] = (int32_t)c;
        in.coord[1] = g;
        in.r0 = (int32_t)(c * C);
        in.r1 = (int32_t)std::min(S, (c + 1) * C);
        in.c0 = g;
        in.c1 = G;
        in.reads.push_back({q.tensor, box2(q, 0, 1, (I64)g * G * d, (I64)(g + 1) * G * d)});
        in.reads.push_back({kn.tensor, box2(kn, 0, 1, (I64)g * d, (I64)(g + 1) * d)});
        in.reads.push_back({vn.tensor, box2(vn, 0, 1, (I64)g * d, (I64)(g + 1) * d)});
        in.reads.push_back({kc.tensor, box2(kc, in.r0, in.r1, (I64)g * d, (I64)(g + 1) * d)});
        in.reads.push_back({vc.tensor, box2(vc, in.r0, in.r1, (I64)g * d, (I64)(g + 1) * d)});
        in.reads.push_back({ps.tensor, full_box(T[ps.tensor])});
        in.writes.push_back({pt, Box{{0, c, (I64)g * G, 0}, {1, c + 1, (I64)(g + 1) * G, W}}});
        n.ins.push_back(in);
      }
    mk_node& dd = n.desc;
    dd.opcode = MK_I_ATTN_PARTIAL;
    dd.dtype = dt;
    dd.M = 1;
    dd.N = (int32_t)NC;
    dd.K = (int32_t)C;
    dd.heads = Hq;
    dd.kv_heads = Hkv;
    dd.head_dim = d;
    dd.seq = (int32_t)S;
    dd.scale = 1.0f / std::sqrt((float)d);
    p.nodes.push_back(n);
    node_edges.push_back({{"a", q}, {"b", kn}, {"res", vn}, {"bias", kc}, {"gamma", vc}, {"out", P},
                          {"aux", edge_of(p.tensors, rope_t)}, {"part", ps}});
    Node m;
    m.op = oi;
    m.opcode = MK_I_ATTN_COMBINE;
    m.out = op.out;
    m.edges = {P, ps};
    for (int g = 0; g < Hkv; ++g) {
      Instr in;
      in.coord[0] = g;
      in.r0 = 0;
      in.r1 = 1;
      in.c0 = g;
      in.c1 = G;
      in.reads.push_back({pt, Box{{0, 0, (I64)g * G, 0}, {1, NC, (I64)(g + 1) * G, W}}});
      in.reads.push_back({ps.tensor, full_box(T[ps.tensor])});
      in.writes.push_back({op.out, box2(o, 0, 1, (I64)g * G * d, (I64)(g + 1) * G * d)});
      m.ins.push_back(in);
    }
    mk_node& md = m.desc;
    md = dd;
    md.opcode = MK_I_ATTN_COMBINE;
    p.nodes.push_back(m);
    node_edges.push_back({{"a", P}, {"out", o}, {"part", ps}});
    return t;
  }

  std::vector<std::map<std::string, Edge>> node_edges;

  // -------------------------------------------------------------- placing
  void place() {
    int cs = p.opts.cluster_size;
    I64 pos = 0;
    for (auto& n : p.nodes) {
      // a GEMM node of at least num_cus instructions starts on an XCD block
      // boundary (num_cus / 8 instructions), so its tile groups line up with
      // the XCDs; the gap is Noops
      if (n.opcode == MK_I_GEMM && ncu % 8 == 0 && (I64)n.ins.size() >= ncu)
        pos = cdiv(pos, ncu / 8) * (ncu / 8);
      n.start = (int)pos;
      pos += cdiv((I64)n.ins.size(), cs) * cs;
      n.end = (int)pos;
    }
    p.n_instr = pos;
  }

  // ---------------------------------------------------------------- slots
  struct PoolEntry {
    int slot;
    mk_dtype dt;
    Shape4 shape;
    int end;
    int old_tensor;
  };
  std::vector<std::pair<int, std::pair<int, int>>> reuse_events;  // node, (slot, old tensor)
  int n_data_slots = 0;  // slots of graph and node tensors (constant tables excluded)
  std::map<int, std::vector<int>> readers;  // root tensor -> reader nodes (ascending)
  std::map<int, int> producer;              // root tensor -> node

  void assign_slots() {
    const int nt = (int)p.tensors.size();
    p.slot_of_tensor.assign(nt, -1);
    for (size_t ni = 0; ni < p.nodes.size(); ++ni) {
      producer[p.nodes[ni].out] = (int)ni;
      for (const Edge& e : p.nodes[ni].edges) {
        auto& v = readers[e.tensor];
        if (v.empty() || v.back() != (int)ni) v.push_back((int)ni);
      }
    }
    int nslots = 0;
    auto new_slot = [&](int tid) {
      p.slot_owner.push_back(tid);
      p.slot_bytes.push_back(numel(p.tensors[tid].shape) * dtype_bytes(p.tensors[tid].dt));
      return nslots++;
    };
    for (int ti = 0; ti < p.n_graph_tensors; ++ti) {
      const Tensor& t = p.tensors[ti];
      if (t.is_view) continue;
      if ((t.role == MK_INPUT || t.role == MK_WEIGHT) && (readers.count(ti) || producer.count(ti)))
        p.slot_of_tensor[ti] = new_slot(ti);
    }
    std::vector<PoolEntry> pool;
    const int reuse = p.opts.reuse;
    for (size_t ni = 0; ni < p.nodes.size(); ++ni) {
      const Node& n = p.nodes[ni];
      const Tensor& t = p.tensors[n.out];
      int take = -1;
      if (reuse && (t.role == MK_INTERMEDIATE || (reuse == 2 && t.role == MK_OUTPUT))) {
        for (size_t k = 0; k < pool.size(); ++k) {
          const PoolEntry& e = pool[k];
          if (e.dt == t.dt && e.shape == t.shape && n.start - e.end >= ncu &&
              (take < 0 || e.slot < pool[take].slot))
            take = (int)k;
        }
      }
      if (take >= 0) {
        p.slot_of_tensor[n.out] = pool[take].slot;
        reuse_events.push_back({(int)ni, {pool[take].slot, pool[take].old_tensor}});
        pool.erase(pool.begin() + take);
      } else {
        p.slot_of_tensor[n.out] = new_slot(n.out);
      }
      if (!reuse) continue;
      std::set<int> seen;
      for (const Edge& e : n.edges) {
        int tt = e.tensor;
        if (!seen.insert(tt).second) continue;
        if (!producer.count(tt) || readers[tt].back() != (int)ni) continue;
        if (p.tensors[tt].role != MK_INTERMEDIATE) continue;
        int end = 0;
        for (int r : readers[tt]) end = std::max(end, p.nodes[r].end);
        pool.push_back({p.slot_of_tensor[tt], p.tensors[tt].dt, p.tensors[tt].shape, end, tt});
      }
    }
    n_data_slots = nslots;
    // tensors no node reads or writes (e.g. constant tables) go last
    for (int ti = 0; ti < nt; ++ti) {
      const Tensor& t = p.tensors[ti];
      if (t.is_view || p.slot_of_tensor[ti] >= 0) continue;
      if (t.internal) p.slot_of_tensor[ti] = new_slot(ti);
    }
    if (nslots > MK_MAX_TENSORS) fail(MK_E_LIMIT, "more than MK_MAX_TENSORS buffer slots");
  }

  // ------------------------------------------------------------- barriers
  struct Bar {
    int first;
    int kind;  // 0 input, 1 reuse
    int node;
    std::vector<int> arrive;
    std::vector<int> wait;
  };
  std::vector<Bar> bars;

  static I64 gcd64(I64 a, I64 b) { return std::gcd(a, b); }

  void derive_barriers() {
    // Unit-cell method ("MegaKittens Internals", section 04, phase 3): for
    // each producer -> consumer edge, cells whose per-dimension size is the
    // GCD of every box boundary on both sides; cell -> producers; a
    // consumer's dependency set is the union over the cells it reads.
    std::map<std::pair<int, std::vector<int>>, int> key2bar;
    for (size_t ci = 0; ci < p.nodes.size(); ++ci) {
      const Node& c = p.nodes[ci];
      // producer nodes this consumer reads from
      std::set<int> prods;
      for (const auto& in : c.ins)
        for (const auto& a : in.reads)
          if (producer.count(a.tensor)) prods.insert(producer[a.tensor]);
      for (int pi : prods) {
        const Node& pn = p.nodes[pi];
        const int tt = pn.out;
        Shape4 gc{0, 0, 0, 0};
        auto fold = [&](const Box& b) {
          for (int d = 0; d < 4; ++d) {
            gc[d] = gcd64(gc[d], b.lo[d]);
            gc[d] = gcd64(gc[d], b.hi[d]);
          }
        };
        for (const auto& in : pn.ins)
          for (const auto& w : in.writes) fold(w.box);
        for (const auto& in : c.ins)
          for (const auto& r : in.reads)
            if (r.tensor == tt) fold(r.box);
        for (int d = 0; d < 4; ++d)
          if (gc[d] == 0) gc[d] = 1;
        const Shape4& sh = p.tensors[tt].shape;
        Shape4 ncell;
        for (int d = 0; d < 4; ++d) ncell[d] = cdiv(sh[d], gc[d]);
        auto cell_id = [&](I64 a, I64 b, I64 c_, I64 d_) {
          return ((a * ncell[1] + b) * ncell[2] + c_) * ncell[3] + d_;
        };
        std::unordered_map<I64, std::vector<int>> writers;
        for (size_t j = 0; j < pn.ins.size(); ++j)
          for (const auto& w : pn.ins[j].writes)
            for (I64 a = w.box.lo[0] / gc[0]; a < w.box.hi[0] / gc[0]; ++a)
              for (I64 b = w.box.lo[1] / gc[1]; b < w.box.hi[1] / gc[1]; ++b)
                for (I64 c_ = w.box.lo[2] / gc[2]; c_ < w.box.hi[2] / gc[2]; ++c_)
                  for (I64 d_ = w.box.lo[3] / gc[3]; d_ < w.box.hi[3] / gc[3]; ++d_)
                    writers[cell_id(a, b, c_, d_)].push_back(pn.start + (int)j);
        std::map<std::vector<Box>, std::vector<int>> cache;
        for (size_t j = 0; j < c.ins.size(); ++j) {
          std::vector<Box> boxes;
          for (const auto& r : c.ins[j].reads)
            if (r.tensor == tt) boxes.push_back(r.box);
          if (boxes.empty()) continue;
          auto it = cache.find(boxes);
          if (it == cache.end()) {
            std::vector<int> dep;
            for (const Box& bx : boxes)
              for (I64 a = bx.lo[0] / gc[0]; a < bx.hi[0] / gc[0]; ++a)
                for (I64 b = bx.lo[1] / gc[1]; b < bx.hi[1] / gc[1]; ++b)
                  for (I64 c_ = bx.lo[2] / gc[2]; c_ < bx.hi[2] / gc[2]; ++c_)
                    for (I64 d_ = bx.lo[3] / gc[3]; d_ < bx.hi[3] / gc[3]; ++d_) {
                      auto w = writers.find(cell_id(a, b, c_, d_));
                      if (w != writers.end()) dep.insert(dep.end(), w->second.begin(), w->second.end());
                    }
            std::sort(dep.begin(), dep.end());
            dep.erase(std::unique(dep.begin(), dep.end()), dep.end());
            it = cache.emplace(boxes, dep).first;
          }
          if (it->second.empty()) continue;
          int gi = c.start + (int)j;
          auto key = std::make_pair(pi, it->second);
          auto kb = key2bar.find(key);
          if (kb == key2bar.end()) {
            bars.push_back(Bar{gi, 0, pi, it->second, {}});
            kb = key2bar.emplace(key, (int)bars.size() - 1).first;
          }
          Bar& B = bars[kb->second];
          B.wait.push_back(gi);
          B.first = std::min(B.first, gi);
        }
      }
    }
    for (const auto& ev : reuse_events) {
      int ni = ev.first, old = ev.second.second;
      const Node& n = p.nodes[ni];
      Bar B;
      B.kind = 1;
      B.node = ni;
      for (int r : readers[old])
        for (size_t j = 0; j < p.nodes[r].ins.size(); ++j) B.arrive.push_back(p.nodes[r].start + (int)j);
      std::sort(B.arrive.begin(), B.arrive.end());
      for (size_t j = 0; j < n.ins.size(); ++j) B.wait.push_back(n.start + (int)j);
      if (B.wait.empty()) continue;
      B.first = B.wait.front();
      bars.push_back(B);
    }
    if (p.opts.sync == 1) level_barriers();
    std::stable_sort(bars.begin(), bars.end(), [](const Bar& a, const Bar& b) {
      if (a.first != b.first) return a.first < b.first;
      if (a.kind != b.kind) return a.kind < b.kind;
      return a.node < b.node;
    });
  }

  // Level-synchronous mode ("Implementing a Mega Kernel for B300", section 7,
  // computing the levels): an instruction's level is one more than the
  // highest level among the producer instructions it reads from (0 without
  // any), and the tile counters give way to one counter per level boundary:
  // every instruction of level L waits for all instructions of level L - 1,
  // as a grid barrier between levels would.  Instructions run in list order
  // on their CUs, so a level is raised to the previous instruction's level
  // where it is lower: the levels then cover contiguous runs of the list and
  // no instruction waits on a later one.
  void level_barriers() {
    std::vector<int> node_of((size_t)p.n_instr, -1);
    for (size_t ni = 0; ni < p.nodes.size(); ++ni)
      for (size_t j = 0; j < p.nodes[ni].ins.size(); ++j) node_of[(size_t)p.nodes[ni].start + j] = (int)ni;
    std::vector<std::vector<int>> parents((size_t)p.n_instr);
    for (const Bar& B : bars)
      if (B.kind == 0)
        for (int i : B.wait) parents[(size_t)i].insert(parents[(size_t)i].end(), B.arrive.begin(), B.arrive.end());
    std::vector<int> level((size_t)p.n_instr, 0);
    int prev = 0;
    for (I64 i = 0; i < p.n_instr; ++i) {
      int lv = prev;
      for (int a : parents[(size_t)i]) lv = std::max(lv, level[(size_t)a] + 1);
      level[(size_t)i] = lv;
      prev = lv;
    }
    // real instructions of each level, in list order
    std::vector<std::vector<int>> members;
    for (I64 i = 0; i < p.n_instr; ++i) {
      if (node_of[(size_t)i] < 0) continue;
      const int lv = level[(size_t)i];
      if ((int)members.size() <= lv) members.resize((size_t)lv + 1);
      members[(size_t)lv].push_back((int)i);
    }
    std::vector<Bar> kept;
    for (Bar& B : bars)
      if (B.kind != 0) kept.push_back(std::move(B));
    for (size_t lv = 1; lv < members.size(); ++lv) {
      if (members[lv].empty() || members[lv - 1].empty()) fail(MK_E_INVALID, "internal: empty level");
      Bar B;
      B.kind = 0;
      B.node = node_of[(size_t)members[lv - 1].front()];
      B.arrive = members[lv - 1];
      B.wait = members[lv];
      B.first = B.wait.front();
      kept.push_back(std::move(B));
    }
    bars = std::move(kept);
  }

  // ----------------------------------------------------------------- emit
  mk_operand operand(const Edge& e) {
    mk_operand o{};
    o.slot = -1;
    if (e.tensor < 0) return o;
    const Shape4& s = p.tensors[e.tensor].shape;
    o.slot = p.slot_of_tensor[e.tensor];
    o.ld = (int32_t)s[3];
    o.off = ((e.lo[0] * s[1] + e.lo[1]) * s[2] + e.lo[2]) * s[3] + e.lo[3];
    return o;
  }

  // The persistent kernel keeps at most 48 node descriptors in LDS.  A plan
  // of more nodes runs with a window of 48 consecutive node ids per
  // workgroup, which must hold the nodes of every three consecutive records
  // of a CU (the running one and the two fetched ahead); the work queue
  // hands out records in an order this cannot bound.
  void check_node_window() {
    constexpr I64 kWindow = 48;
    if ((I64)p.nodes.size() <= kWindow) return;
    if (p.opts.queue) {
      unsup("plans of more than 48 lowered nodes run in static placement only");
      return;
    }
    const I64 n_iters = cdiv(p.n_instr, ncu);
    for (I64 c = 0; c < ncu; ++c)
      for (I64 it = 0; it < n_iters; ++it) {
        int lo = -1, hi = -1;
        for (I64 k = it; k < std::min(n_iters, it + 3); ++k) {
          const mk_instr& r = p.records[(size_t)(k * ncu + c)];
          if (r.opcode == MK_I_NOOP) continue;
          lo = lo < 0 ? r.node : std::min(lo, r.node);
          hi = std::max(hi, r.node);
        }
        if (lo >= 0 && hi - lo >= kWindow) {
          unsup("three consecutive records of a CU span 48 or more lowered nodes (the LDS node window)");
          return;
        }
      }
  }

  void emit() {
    const I64 n_iters = cdiv(p.n_instr, ncu);
    p.records.assign((size_t)(n_iters * ncu), mk_instr{});
    std::vector<std::vector<std::pair<int, int>>> src(p.n_instr);
    std::vector<std::vector<std::pair<int, int>>> dst(p.n_instr);   // (counter, arrival rank or -1)
    p.targets.clear();
    I64 n_in = 0, n_re = 0;
    for (size_t b = 0; b < bars.size(); ++b) {
      const Bar& B = bars[b];
      int tgt = (int)B.arrive.size();
      p.targets.push_back(tgt);
      (B.kind ? n_re : n_in)++;
      for (int i : B.wait) src[i].push_back({(int)b, tgt});
      std::vector<int> arrive = B.arrive;
      std::sort(arrive.begin(), arrive.end());
      const bool sliced = tgt <= MK_SLICE_MAX;
      for (size_t r = 0; r < arrive.size(); ++r) {
        const int i = arrive[r];
        if (i >= B.first) fail(MK_E_INVALID, "internal: dependency on a later instruction");
        dst[i].push_back({(int)b, sliced ? (int)r : -1});
      }
    }
    for (size_t ni = 0; ni < p.nodes.size(); ++ni) {
      Node& n = p.nodes[ni];
      // node descriptor operands
      mk_node& d = n.desc;
      d.node_start = n.start;
      d.n_instr = (int32_t)n.ins.size();
      auto& ed = node_edges[ni];
      auto get = [&](const char* k) { auto it = ed.find(k); return it == ed.end() ? Edge{} : it->second; };
      d.a = operand(get("a"));
      d.b = operand(get("b"));
      d.out = operand(get("out"));
      d.bias = operand(get("bias"));
      d.res = operand(get("res"));
      d.gamma = operand(get("gamma"));
      d.part = operand(get("part"));
      d.aux = operand(get("aux"));
      p.node_descs.push_back(d);
      for (int j = 0; j < n.end - n.start; ++j) {
        int i = n.start + j;
        mk_instr& r = p.records[i];
        std::memset(&r, 0, sizeof(r));
        r.node = (int32_t)ni;
        if (j >= (int)n.ins.size()) continue;  // Noop pad
        const Instr& in = n.ins[j];
        r.opcode = n.opcode;
        r.flags = n.flags;
        for (int c = 0; c < 4; ++c) r.coord[c] = in.coord[c];
        r.r0 = in.r0; r.r1 = in.r1; r.c0 = in.c0; r.c1 = in.c1; r.k0 = in.k0; r.k1 = in.k1;
        r.split_idx = in.s;
        auto& s = src[i];
        std::sort(s.begin(), s.end());
        auto& t = dst[i];
        std::sort(t.begin(), t.end());
        if (s.size() > MK_MAX_SRC || t.size() > MK_MAX_DST)
          fail(MK_E_LIMIT, "instruction " + std::to_string(i) + " exceeds the counter limits (16 src, 8 dst)");
        r.n_src = (int32_t)s.size();
        r.n_dst = (int32_t)t.size();
        for (size_t k = 0; k < s.size(); ++k) {
          r.src_id[k] = s[k].first;
          r.src_target[k] = s[k].second;
        }
        for (size_t k = 0; k < t.size(); ++k) {
          r.dst_id[k] = t[k].first;
          r.dst_rank[k] = t[k].second;
        }
      }
    }
    mk_plan_stats& st = p.stats;
    st.n_instr = p.n_instr;
    st.n_iters = n_iters;
    st.n_nodes = (I64)p.nodes.size();
    st.n_barriers = (I64)bars.size();
    st.n_input_barriers = n_in;
    st.n_reuse_barriers = n_re;
    st.n_slots = n_data_slots;
    st.num_cus = ncu;
    I64 ib = 0;
    for (size_t s = 0; s < p.slot_owner.size(); ++s) {
      const Tensor& t = p.tensors[p.slot_owner[s]];
      if (t.role == MK_INTERMEDIATE) ib += p.slot_bytes[s];
    }
    st.intermediate_bytes = ib;
  }

  void algorithmic_counts() {
    double flops = 0, bytes = 0;
    std::set<int> read_once;
    for (const OpRec& op : g.ops) {
      if (op.kind == MK_OP_GEMM) {
        Edge A = edge_of(p.tensors, op.in[0]), B = edge_of(p.tensors, op.in[1]);
        flops += 2.0 * (double)A.rows() * (double)B.cols() * (double)A.cols();
      } else if (op.kind == MK_OP_ATTENTION) {
        Edge q = edge_of(p.tensors, op.in[0]);
        double S = (double)q.rows(), hd = op.attrs.head_dim, H = op.attrs.n_heads;
        flops += op.attrs.causal ? 4.0 * H * hd * S * (S + 1) / 2 : 4.0 * H * hd * S * S;
      } else if (op.kind == MK_OP_DECODE_ATTENTION) {
        // counted over the whole cache (the position is known only at run time)
        Edge kc = edge_of(p.tensors, op.in[3]);
        flops += 4.0 * op.attrs.n_heads * op.attrs.head_dim * (double)kc.rows();
      }
      for (int id : op.in) {
        Edge e = edge_of(p.tensors, id);
        const Tensor& t = p.tensors[e.tensor];
        if (t.role == MK_INPUT || t.role == MK_WEIGHT) {
          if (read_once.insert(e.tensor).second)
            bytes += (double)numel(t.shape) * dtype_bytes(t.dt);
        } else {
          Shape4 ext;
          for (int d = 0; d < 4; ++d) ext[d] = e.hi[d] - e.lo[d];
          bytes += (double)numel(ext) * dtype_bytes(t.dt);
        }
      }
      const Tensor& o = p.tensors[op.out];
      bytes += (double)numel(o.shape) * dtype_bytes(o.dt);
    }
    p.stats.flops = flops;
    p.stats.bytes = bytes;
  }

  // Contents of the compiler's constant tables, by slot.  Rotary table
  // (const_kind 1): row p = [cos(p th_i) for i < half | sin(p th_i) for
  // i < half], th_i = theta^(-2i / head_dim), evaluated in double.
  void const_tables() {
    p.const_data.assign(p.slot_owner.size(), {});
    for (size_t s = 0; s < p.slot_owner.size(); ++s) {
      const Tensor& t = p.tensors[p.slot_owner[s]];
      if (t.const_kind != 1) continue;
      const int half = t.rope_half;
      const I64 rows = t.shape[2];
      std::vector<float>& tab = p.const_data[s];
      tab.resize((size_t)rows * 2 * half);
      for (I64 pos = 0; pos < rows; ++pos)
        for (int i = 0; i < half; ++i) {
          const double th = std::pow((double)t.rope_theta, -2.0 * i / (2.0 * half));
          tab[(size_t)pos * 2 * half + i] = (float)std::cos((double)pos * th);
          tab[(size_t)pos * 2 * half + half + i] = (float)std::sin((double)pos * th);
        }
    }
  }

  // Row-major GEMM nodes whose counter waits may skip the cache
  // invalidation (mk_node.lines_own).  Every tensor such a node reads that
  // the run writes must be written in whole 128-byte lines (row length and
  // every write box's column range multiples of 128 bytes) and hold its
  // slot alone (no reuse).  A reader of any byte of such a line then waits
  // on every writer of that line, so no cache of the device can have taken
  // the line before it was complete (caches start each launch clean).  The
  // KV caches, which decode attention appends to, count as written.
  void mark_lines_own() {
    std::map<int, std::vector<Box>> writes;
    for (const Node& n : p.nodes)
      for (const Instr& in : n.ins)
        for (const Access& w : in.writes) writes[w.tensor].push_back(w.box);
    std::set<int> appended, shared;
    for (const OpRec& op : p.ops)
      if (op.kind == MK_OP_DECODE_ATTENTION && op.in.size() > 4) {
        appended.insert(edge_of(p.tensors, op.in[3]).tensor);
        appended.insert(edge_of(p.tensors, op.in[4]).tensor);
      }
    for (const auto& ev : reuse_events) {
      shared.insert(ev.second.second);
      shared.insert(p.nodes[ev.first].out);
    }
    std::map<int, bool> own;   // tensor -> lines written whole, slot alone
    auto lines_ok = [&](int t) {
      auto it = own.find(t);
      if (it != own.end()) return it->second;
      bool ok = !appended.count(t) && !shared.count(t);
      const I64 es = dtype_bytes(p.tensors[t].dt);
      if (ok && (p.tensors[t].shape[3] * es) % 128) ok = false;
      for (const Box& b : writes[t])
        if ((b.lo[3] * es) % 128 || (b.hi[3] * es) % 128) ok = false;
      own[t] = ok;
      return ok;
    };
    for (Node& n : p.nodes) {
      n.desc.lines_own = 0;
      if (n.opcode != MK_I_GEMM || n.desc.layout != 0) continue;
      bool ok = true;
      for (const Instr& in : n.ins) {
        for (const Access& r : in.reads)
          if ((writes.count(r.tensor) || appended.count(r.tensor)) && !lines_ok(r.tensor)) ok = false;
        if (!ok) break;
      }
      n.desc.lines_own = ok ? 1 : 0;
    }
    for (size_t ni = 0; ni < p.nodes.size(); ++ni) p.node_descs[ni].lines_own = p.nodes[ni].desc.lines_own;
  }

  void run() {
    p.tensors = g.t;
    p.n_graph_tensors = (int)g.t.size();
    p.ops = g.ops;
    lower();
    place();
    assign_slots();
    derive_barriers();
    emit();
    mark_lines_own();
    check_node_window();
    algorithmic_counts();
    const_tables();
    p.stats.reserved = unsupported.empty() ? 0 : 1;
    unsupported_reason = unsupported;
  }
  std::string unsupported_reason;
};

}  // namespace
}  // namespace mk

using namespace mk;

const char* mk_plan_unsupported_reason(const mk_plan* p) { return p->unsupported.c_str(); }

extern "C" {

const char* mk_last_error(void) { return mk::g_err.c_str(); }
int32_t mk_abi_version(void) { return MK_ABI_VERSION; }

mk_status mk_graph_create(mk_graph** g) {
  if (!g) { set_error("null graph pointer"); return MK_E_INVALID; }
  *g = new mk_graph();
  return MK_OK;
}

void mk_graph_destroy(mk_graph* g) { delete g; }

mk_status mk_graph_tensor(mk_graph* g, mk_dtype dt, int ndim, const int64_t* shape,
                          mk_role role, int32_t* id) {
  if (!g || !shape || !id) { set_error("null argument"); return MK_E_INVALID; }
  if (dt != MK_F16 && dt != MK_BF16 && dt != MK_F32 && dt != MK_I32) { set_error("bad dtype"); return MK_E_INVALID; }
  if (ndim < 1 || ndim > 4) { set_error("tensors have 1..4 dims"); return MK_E_INVALID; }
  if (role < MK_INPUT || role > MK_INTERMEDIATE) { set_error("bad role"); return MK_E_INVALID; }
  if ((int)g->t.size() >= MK_MAX_TENSORS) { set_error("more than MK_MAX_TENSORS tensors"); return MK_E_LIMIT; }
  Tensor t;
  t.dt = dt;
  t.role = role;
  t.ndim = ndim;
  for (int d = 0; d < ndim; ++d) {
    if (shape[d] < 0 || shape[d] > (int64_t)1 << 31) { set_error("bad shape"); return MK_E_INVALID; }
    t.shape[4 - ndim + d] = shape[d];
  }
  g->t.push_back(t);
  *id = (int32_t)g->t.size() - 1;
  return MK_OK;
}

mk_status mk_graph_view(mk_graph* g, int32_t src, const int64_t lo[4], const int64_t hi[4],
                        int32_t* id) {
  if (!g || !lo || !hi || !id) { set_error("null argument"); return MK_E_INVALID; }
  if (src < 0 || src >= (int)g->t.size()) { set_error("bad view source"); return MK_E_INVALID; }
  if ((int)g->t.size() >= MK_MAX_TENSORS) { set_error("more than MK_MAX_TENSORS tensors"); return MK_E_LIMIT; }
  const Tensor& s = g->t[src];
  Shape4 sh = s.is_view ? Shape4{s.hi[0] - s.lo[0], s.hi[1] - s.lo[1], s.hi[2] - s.lo[2], s.hi[3] - s.lo[3]}
                        : s.shape;
  Tensor v;
  v.dt = s.dt;
  v.role = s.role;
  v.ndim = 4;
  v.is_view = true;
  v.root = s.is_view ? s.root : src;
  for (int d = 0; d < 4; ++d) {
    if (lo[d] < 0 || lo[d] > hi[d] || hi[d] > sh[d]) {
      set_error("view range outside its source (step-1 ranges only)");
      return MK_E_INVALID;
    }
    Shape4 base = s.is_view ? s.lo : Shape4{0, 0, 0, 0};
    v.lo[d] = base[d] + lo[d];
    v.hi[d] = base[d] + hi[d];
    v.shape[d] = hi[d] - lo[d];
  }
  g->t.push_back(v);
  *id = (int32_t)g->t.size() - 1;
  return MK_OK;
}

mk_status mk_graph_op(mk_graph* g, mk_op_kind kind, const int32_t* in, int n_in, int32_t out,
                      const mk_op_attrs* attrs) {
  if (!g || (n_in > 0 && !in)) { set_error("null argument"); return MK_E_INVALID; }
  mk_op_attrs a{};
  if (attrs) a = *attrs;
  int want = 0;
  switch (kind) {
    case MK_OP_GEMM:
      want = 2 + !!(a.epilogue & MK_EP_BIAS) + !!(a.epilogue & MK_EP_RESIDUAL) +
             !!(a.epilogue & MK_EP_RMSNORM_INPUT);
      if (a.epilogue & ~0x3Fu) { set_error("unknown epilogue flag"); return MK_E_INVALID; }
      break;
    case MK_OP_RMSNORM: want = 2; break;
    case MK_OP_ATTENTION: want = 3; break;
    case MK_OP_ADD: want = 2; break;
    case MK_OP_RELU: want = 1; break;
    case MK_OP_DECODE_ATTENTION: want = 6; break;
    default: set_error("unknown op kind"); return MK_E_INVALID;
  }
  if (kind != MK_OP_GEMM && a.epilogue) { set_error("epilogue flags apply to GEMM only"); return MK_E_INVALID; }
  if (n_in != want) {
    set_error("op expects " + std::to_string(want) + " inputs, got " + std::to_string(n_in));
    return MK_E_INVALID;
  }
  const int nt = (int)g->t.size();
  if (out < 0 || out >= nt) { set_error("bad output id"); return MK_E_INVALID; }
  const Tensor& o = g->t[out];
  if (o.is_view) { set_error("op outputs must be whole tensors, not views"); return MK_E_INVALID; }
  if (o.role != MK_OUTPUT && o.role != MK_INTERMEDIATE) {
    set_error("op output must have role OUTPUT or INTERMEDIATE");
    return MK_E_INVALID;
  }
  auto root = [&](int id) { return g->t[id].is_view ? g->t[id].root : id; };
  for (const OpRec& prev : g->ops) {
    if (prev.out == out) { set_error("tensor written by two ops"); return MK_E_INVALID; }
    for (int i : prev.in)
      if (root(i) == out) { set_error("op output already read by an earlier op (not topological)"); return MK_E_INVALID; }
  }
  for (int k = 0; k < n_in; ++k) {
    if (in[k] < 0 || in[k] >= nt) { set_error("bad input id"); return MK_E_INVALID; }
    int r = root(in[k]);
    if (r == out) { set_error("op reads its own output"); return MK_E_INVALID; }
    const Tensor& t = g->t[r];
    if (t.role == MK_OUTPUT || t.role == MK_INTERMEDIATE) {
      bool written = false;
      for (const OpRec& prev : g->ops) written |= prev.out == r;
      if (!written) { set_error("op reads a tensor no earlier op writes (not topological)"); return MK_E_INVALID; }
    }
  }
  OpRec op;
  op.kind = kind;
  op.in.assign(in, in + n_in);
  op.out = out;
  op.attrs = a;
  g->ops.push_back(op);
  return MK_OK;
}

mk_status megakernel_build(const mk_graph* g, const mk_build_options* opts, mk_plan** plan) {
  if (!g || !plan) { set_error("null argument"); return MK_E_INVALID; }
  *plan = nullptr;
  mk_plan* p = new mk_plan();
  if (opts) p->opts = *opts;
  if (p->opts.num_cus <= 0) p->opts.num_cus = 256;
  if (p->opts.cluster_size <= 0) p->opts.cluster_size = 1;
  if (p->opts.gemv_max_m <= 0) p->opts.gemv_max_m = 8;
  if (p->opts.spin_limit_us <= 0) p->opts.spin_limit_us = 2000000;
  if (p->opts.reuse < 0 || p->opts.reuse > 2) { delete p; set_error("reuse must be 0, 1 or 2"); return MK_E_INVALID; }
  if (p->opts.pack < 0 || p->opts.pack > 2) { delete p; set_error("pack must be 0, 1 or 2"); return MK_E_INVALID; }
  if (p->opts.sync < 0 || p->opts.sync > 1) { delete p; set_error("sync must be 0 or 1"); return MK_E_INVALID; }
  if (p->opts.queue < 0 || p->opts.queue > 2) { delete p; set_error("queue must be 0, 1 or 2"); return MK_E_INVALID; }
  if (p->opts.queue == 2 && p->opts.num_cus % 8) {
    delete p;
    set_error("queue = 2 (one queue per XCD) needs num_cus to be a multiple of 8");
    return MK_E_INVALID;
  }
  if (p->opts.debug_poison < 0 || p->opts.debug_poison > 1) {
    delete p;
    set_error("debug_poison must be 0 or 1");
    return MK_E_INVALID;
  }
  bool has_out = false;
  for (const OpRec& op : g->ops) has_out |= g->t[op.out].role == MK_OUTPUT;
  if (!g->ops.empty() && !has_out) { delete p; set_error("graph has no OUTPUT tensor"); return MK_E_INVALID; }
  try {
    Compiler c(*g, *p);
    c.run();
    p->unsupported = c.unsupported_reason;
  } catch (const Fail& f) {
    delete p;
    set_error(f.msg);
    return f.st;
  } catch (const std::exception& e) {
    delete p;
    set_error(std::string("internal error: ") + e.what());
    return MK_E_INVALID;
  }
  *plan = p;
  return MK_OK;
}

mk_status mk_plan_stats_get(const mk_plan* p, mk_plan_stats* out) {
  if (!p || !out) { set_error("null argument"); return MK_E_INVALID; }
  *out = p->stats;
  return MK_OK;
}

mk_status mk_plan_instructions(const mk_plan* p, const int32_t** words, int64_t* n_instr,
                               int32_t* wpi) {
  if (!p || !words || !n_instr || !wpi) { set_error("null argument"); return MK_E_INVALID; }
  *words = reinterpret_cast<const int32_t*>(p->records.data());
  *n_instr = p->n_instr;
  *wpi = MK_INSTR_WORDS;
  return MK_OK;
}

mk_status mk_plan_nodes(const mk_plan* p, const int32_t** words, int64_t* n, int32_t* wpn) {
  if (!p || !words || !n || !wpn) { set_error("null argument"); return MK_E_INVALID; }
  *words = reinterpret_cast<const int32_t*>(p->node_descs.data());
  *n = (int64_t)p->node_descs.size();
  *wpn = MK_NODE_WORDS;
  return MK_OK;
}

mk_status mk_plan_barriers(const mk_plan* p, const int32_t** targets, int64_t* n) {
  if (!p || !targets || !n) { set_error("null argument"); return MK_E_INVALID; }
  *targets = p->targets.data();
  *n = (int64_t)p->targets.size();
  return MK_OK;
}

mk_status mk_plan_slots(const mk_plan* p, const int32_t** slot_of_tensor, int64_t* n) {
  if (!p || !slot_of_tensor || !n) { set_error("null argument"); return MK_E_INVALID; }
  *slot_of_tensor = p->slot_of_tensor.data();
  *n = p->n_graph_tensors;
  return MK_OK;
}

mk_status mk_plan_op_tile(const mk_plan* p, int32_t op, mk_tile* out) {
  if (!p || !out) { set_error("null argument"); return MK_E_INVALID; }
  if (op < 0 || op >= (int)p->op_tiles.size()) { set_error("bad op index"); return MK_E_INVALID; }
  *out = p->op_tiles[op];
  return MK_OK;
}

mk_status mk_plan_weight_layout(const mk_plan* p, int32_t tensor, int32_t* packed, int64_t* bytes) {
  if (!p || !packed || !bytes) { set_error("null argument"); return MK_E_INVALID; }
  if (tensor < 0 || tensor >= p->n_graph_tensors) { set_error("bad tensor id"); return MK_E_INVALID; }
  *packed = 0;
  *bytes = 0;
  for (const PackInfo& pk : p->packs)
    if (pk.tensor == tensor) {
      *packed = 1;
      *bytes = pk.bytes;
    }
  return MK_OK;
}

mk_status mk_plan_epoch(const mk_plan* p, int64_t* epoch) {
  if (!p || !epoch) { set_error("null argument"); return MK_E_INVALID; }
  *epoch = p->epoch;
  return MK_OK;
}

}  // extern "C"
