/*
 * mk.h — C ABI of the MI355X persistent tile-graph megakernel.
 *
 * A static graph of GEMMs (with bias / ReLU / residual / SiLU-mul /
 * RMSNorm-input / rotary epilogues), RMSNorms, causal attention and
 * elementwise ops is compiled on the host into a flat list of tile-sized
 * instructions with per-tile int32 dependency counters, then executed by one
 * persistent HIP kernel (one workgroup per compute unit) per forward.
 *
 * Design sources (web pages):
 *   "MegaKittens Internals" — sections 02 (graph, views as ranges), 04
 *     (scheduler: placement, tensor slots, fine-grained barriers), 05
 *     (per-SM placement), 06 (256-byte instruction), 07 (dispatcher), 11
 *     (global barriers, deadlock argument), 12-14 (instruction types).
 *   "Implementing a Mega Kernel for B300" — sections 1-2 (graph builder,
 *     epilogues as GEMV flags, 64-byte POD descriptors with buffer indices
 *     instead of pointers, ABI size guards), 5-6 (buffer table, upload).
 *   "Beating torch.compile with Megakernels in CuTe DSL" — "Cooperative
 *     Kernel", "Dependency Management and Scheduling" (round-robin
 *     placement, counter spin-wait with acquire loads).
 *
 * Conventions
 *   - Every call returns an mk_status; mk_last_error() gives a message for
 *     the calling thread's last non-OK status.  No C++ exception crosses
 *     this boundary.
 *   - Tensors are row-major and contiguous, of at most 4 dimensions,
 *     left-padded to 4-D for ranges.  A GEMM computes out = A @ B with
 *     A [M, K] and B [K, N] (weights stored K-major).
 *   - Pointers passed to megakernel_run* are device pointers; every other
 *     pointer argument is a host pointer.
 *   - The graph and every input / weight / output device buffer belong to
 *     the caller.  A plan owns its device copy of the instruction records,
 *     its counters, its intermediate buffers and its error record; they are
 *     allocated on the plan's first run and freed by mk_plan_destroy.
 *   - A plan runs on one stream at a time: its counters and intermediates
 *     are shared by every run of that plan.
 */
#ifndef MK_H
#define MK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 5
#define MK_MAX_TENSORS 256      /* graph tensors incl. views and internals */
#define MK_MAX_SRC 16           /* counters one instruction waits on       */
#define MK_MAX_DST 8            /* counters one instruction arrives on     */
#define MK_INSTR_WORDS 64       /* int32 words per instruction record      */
#define MK_SLICE_MAX 256        /* counters with at most this target are
                                   kept as one slot per arrival (below)    */
#define MK_NODE_WORDS 64        /* int32 words per node descriptor         */

typedef enum {
  MK_OK = 0,
  MK_E_INVALID = 1,     /* bad argument, shape mismatch, non-topological */
  MK_E_UNSUPPORTED = 2, /* valid graph the kernels do not implement      */
  MK_E_LIMIT = 3,       /* a fixed limit (tensors, counters per instr)   */
  MK_E_HIP = 4,         /* a HIP runtime call failed                     */
  MK_E_DEADLOCK = 5     /* a counter wait exceeded the spin limit        */
} mk_status;

typedef enum { MK_F16 = 1, MK_BF16 = 2, MK_F32 = 3,
               MK_I32 = 4   /* runtime scalars only (the decode position) */
} mk_dtype;

typedef enum {
  MK_INPUT = 0,        /* caller-owned activation input                  */
  MK_WEIGHT = 1,       /* caller-owned constant input                    */
  MK_OUTPUT = 2,       /* caller-owned output buffer                     */
  MK_INTERMEDIATE = 3  /* plan-owned                                     */
} mk_role;

typedef enum {
  MK_OP_GEMM = 1,      /* in: A, B [, bias][, residual][, gamma]         */
  MK_OP_RMSNORM = 2,   /* in: x, gamma                                   */
  MK_OP_ATTENTION = 3, /* in: q, k, v (column ranges of a QKV tensor)    */
  MK_OP_ADD = 4,       /* in: a, b  (same shape, no broadcasting)        */
  MK_OP_RELU = 5,      /* in: a                                          */
  MK_OP_DECODE_ATTENTION = 6
                       /* in: q [1, Hq*d], k_new [1, Hkv*d], v_new [1,
                          Hkv*d] (column ranges of the QKV output),
                          k_cache [S_max, Hkv*d], v_cache [S_max, Hkv*d]
                          (caller-owned INPUT tensors), pos (INPUT, MK_I32,
                          one element: the position p of the new token,
                          read at run time, 0 <= p < S_max); out o [1,
                          Hq*d].  With rotary embedding at position p
                          (rotate-half pairs, base rope_theta) applied to q
                          and k_new: o[h] = sum over keys j <= p of
                          softmax_j(q'_h . K_j / sqrt(d)) V_j for kv head
                          h / (Hq / Hkv), where K_j, V_j are cache row j for
                          j < p and the rotated k_new (rounded to the cache
                          dtype) and v_new for j = p.  The op also writes
                          those two values into row p of k_cache and
                          v_cache (the append), which no other op of the
                          graph may read.  Split over the cache in chunks of
                          tile.bq keys ("Implementing a Mega Kernel for
                          B300", section 2: flash-decoding partials and a
                          log-sum-exp combine)                             */
} mk_op_kind;

/* GEMM epilogue flags ("Implementing a Mega Kernel for B300", section 2:
 * fusions are flags on the GEMV; MegaKittens Internals section 02: bias then
 * ReLU).  Order of application: RMSNORM_INPUT scales the A rows, then the
 * fp32 product, then SILU_MUL, BIAS, RESIDUAL, ROPE, RELU, then one
 * round-to-nearest-even cast to the output dtype. */
enum {
  MK_EP_BIAS = 1,          /* + bias, a full [M, N] tensor                 */
  MK_EP_RELU = 2,          /* max(., 0)                                    */
  MK_EP_RESIDUAL = 4,      /* + residual [M, N]                            */
  MK_EP_SILU_MUL = 8,      /* B has 2N columns [gate | up]; out = silu(g)*u */
  MK_EP_RMSNORM_INPUT = 16,/* A rows normalised: A*gamma/sqrt(mean(A^2)+eps) */
  MK_EP_ROPE = 32,         /* rotate-half rotary embedding on the leading
                              rope_cols columns, position = row index      */
  MK_EP_PARTIAL = 64       /* internal: instruction writes fp32 split-K partial
                              sums (set by the compiler, never by callers) */
};

/* Instruction opcodes (the record's first word). */
enum {
  MK_I_NOOP = 0, MK_I_GEMM = 1, MK_I_GEMV = 2, MK_I_REDUCE = 3,
  MK_I_RMSNORM = 4, MK_I_ATTENTION = 5, MK_I_EW_ADD = 6, MK_I_EW_RELU = 7,
  MK_I_ATTN_PARTIAL = 8, MK_I_ATTN_COMBINE = 9
};

/* Tile parameters of one op; 0 in any field = the compiler's choice.
 * GEMM: bm x bn output tile (bn counts output columns, so a SILU_MUL tile
 * reads 2*bn weight columns), split = K chunks (> 1 adds a REDUCE node over
 * rbm x rbn tiles), dup = copies of each tile (cluster duplicate, host
 * profile only).  gemv = 1 selects the small-M streaming body.  layout
 * selects how the weight is read: 0 = the compiler's choice, 1 = the
 * row-major [K, N] tensor, 2 = the packed layout of mk_plan_weight_layout
 * (GEMV: column tiles of bn outputs over the whole K, no split, no REDUCE
 * node; GEMM: bm x w tiles of 256 x 128, 128 x 256 or 128 x 128, w = the
 * tile's weight columns, bn or 2 * bn under SILU_MUL; a K split is
 * allowed).
 * RMSNORM: rows per instruction.  ATTENTION: bq query rows per instruction.
 * DECODE_ATTENTION: bq cache keys per partial instruction (a multiple of
 * 64; 0: about Hkv * ceil(S_max / bq) = num_cus instructions).
 * ADD / RELU: er x ec tiles. */
typedef struct {
  int32_t bm, bn, split, dup, gemv;
  int32_t rbm, rbn;
  int32_t rows;
  int32_t bq;
  int32_t er, ec;
  int32_t layout;
} mk_tile;

typedef struct {
  uint32_t epilogue;    /* MK_EP_* (GEMM only)                            */
  float eps;            /* RMSNorm epsilon; 0 -> 1e-6                      */
  float rope_theta;     /* 0 -> 10000                                      */
  int32_t n_heads;      /* ATTENTION / ROPE: query heads                   */
  int32_t n_kv_heads;   /* ATTENTION: kv heads (query head h reads h / (n_heads/n_kv_heads)) */
  int32_t head_dim;     /* ATTENTION / ROPE                                */
  int32_t causal;       /* ATTENTION: key j visible to query i iff j <= i  */
  int32_t rope_cols;    /* ROPE: leading output columns rotated; 0 -> all  */
  mk_tile tile;
} mk_op_attrs;

typedef struct {
  int32_t num_cus;      /* 0 -> 256 (MI355X); placement modulus            */
  int32_t cluster_size; /* 0 -> 1; node ranges padded to a multiple        */
  int32_t reuse;        /* 0: no buffer pooling; 1: pool intermediates;
                           2: also let outputs take pooled slots (host
                           profile of dispatcher-owned outputs only)       */
  int32_t gemv_max_m;   /* 0 -> 8: GEMMs with M <= this use the GEMV body  */
  int64_t spin_limit_us;/* 0 -> 2000000: a counter wait longer than this
                           aborts the run with MK_E_DEADLOCK               */
  int32_t cooperative;  /* 1: hipLaunchCooperativeKernel (residency of all
                           num_cus workgroups guaranteed by the runtime);
                           0: ordinary launch of num_cus workgroups, which
                           the kernel's LDS use pins to one per CU.  An
                           ordinary launch avoids a ~20 us gap between
                           consecutive cooperative launches; should a
                           workgroup not become resident, the bounded waits
                           end the run with MK_E_DEADLOCK instead of a hang */
  int32_t pack;         /* weights read in the packed layout (tile.layout
                           0 = compiler's choice): a weight qualifies when
                           it is a whole 2-D weight tensor read by no other
                           op.  0: GEMMs whenever it qualifies, GEMVs when
                           it also has at least num_cus 8-column tiles;
                           1: never; 2: whenever it qualifies               */
  int32_t sync;         /* 0: per-tile counters (a consumer waits on the
                           producer tiles it reads); 1: level-synchronous
                           ("Implementing a Mega Kernel for B300", section
                           on task levels): a node's level is one more than
                           its producers' highest level, raised to keep
                           levels non-decreasing in node order, and every
                           instruction of level L waits on one counter that
                           all instructions of level L - 1 arrive on, as a
                           grid barrier per level would.  Reuse barriers
                           are kept as they are.  For A/B comparison.       */
  int32_t queue;        /* 0: static placement, instruction i on workgroup
                           i mod num_cus in iteration i / num_cus
                           (MegaKittens Internals, section 05); 1: a work
                           queue ("MegaKittens Internals", section 07,
                           global-work-queue mode): each workgroup takes the
                           next instruction index from a device counter
                           with an atomic add, two ahead of the one it runs.
                           Indices are taken in list order and every
                           dependency points to a lower index, so the
                           lowest unfinished index is always running and
                           any number of resident workgroups completes the
                           run.  2: one such queue per XCD: workgroup w
                           takes, in list order, the instructions i with
                           i mod 8 = w mod 8 (those static placement puts
                           on its XCD), so tiles keep their L2 neighbours;
                           the run completes while every residue class mod
                           8 has a resident workgroup (num_cus a multiple
                           of 8).  The records and counters are the same in
                           every mode.                                      */
  int32_t debug_poison; /* 1: before every run fill each plan-owned
                           intermediate (and split-K partial buffer) with
                           all-ones bytes, a NaN in fp16, bf16 and fp32, so
                           a read of a value no instruction of this run has
                           written shows up in the output.  Debug aid; one
                           extra fill launch per buffer per run.            */
} mk_build_options;

typedef struct {
  int64_t n_instr;        /* list length incl. Noop pads                   */
  int64_t n_iters;        /* waves: ceil(n_instr / num_cus)                */
  int64_t n_nodes;
  int64_t n_barriers;
  int64_t n_input_barriers;
  int64_t n_reuse_barriers;
  int64_t n_slots;        /* buffer slots of graph and node tensors        */
  int64_t intermediate_bytes; /* plan-owned device bytes                   */
  double flops;           /* algorithmic: 2MNK per GEMM + causal attention */
  double bytes;           /* algorithmic HBM bytes: inputs/weights read once,
                             every intermediate written once and read once
                             per consuming node, outputs written once      */
  int32_t num_cus;
  int32_t reserved;
} mk_plan_stats;

/* Instruction record: exactly 256 bytes (MegaKittens Internals section 06:
 * a fixed 256-byte POD loaded with coalesced per-lane words).  Packed
 * [n_iters][num_cus] so record i sits at index i. */
typedef struct {
  int32_t opcode;      /* MK_I_*                                           */
  int32_t flags;       /* MK_EP_* of this node                             */
  int32_t node;        /* index into the node table                        */
  int32_t n_src, n_dst;
  int32_t coord[4];    /* tile coordinates (see mk_plan_instructions)      */
  int32_t r0, r1;      /* output rows [r0, r1) (attention: query rows)     */
  int32_t c0, c1;      /* output columns [c0, c1) (attention: head h in c0)*/
  int32_t k0, k1;      /* K range of a GEMM / GEMV instruction             */
  int32_t split_idx;   /* K chunk index (partials plane)                   */
  int32_t src_id[MK_MAX_SRC];     /* counters waited on, ascending        */
  int32_t src_target[MK_MAX_SRC]; /* their targets (arrivals per run)     */
  int32_t dst_id[MK_MAX_DST];     /* counters arrived on, ascending       */
  int32_t dst_rank[MK_MAX_DST];   /* position of this instruction among the
                                     arrivals of dst_id[k], ordered by
                                     instruction index, when that counter's
                                     target is <= MK_SLICE_MAX; else -1   */
} mk_instr;

/* Counters in device memory.  Counter b takes `stride` int32 slots at
 * b * stride, stride being the largest target up to MK_SLICE_MAX rounded up
 * to 32 (so every counter starts a 128-byte line of its own).  A counter
 * with target T <= MK_SLICE_MAX is sliced: arrival r (dst_rank) stores the
 * epoch into slot r and a waiter needs every one of its T slots at the
 * epoch.  A counter with a larger target lives in its first slot: each
 * arrival adds 1 (agent-scope atomic) and a waiter needs epoch * T there.
 * Either way the counter's value, the sum of its slots, is epoch * T after
 * a run.  A sliced counter's arrivals meet no contended read-modify-write:
 * hundreds of producers adding to one word serialise at the memory side,
 * which made up most of a whole-grid counter wait, and even a handful of
 * producers adding to one word wait on each other's round trips. */

/* Operand of a node: buffer-table slot, element offset and row stride. */
typedef struct {
  int32_t slot;        /* -1 = absent                                      */
  int32_t ld;          /* row stride in elements                           */
  int64_t off;         /* element offset of logical element (0, 0)         */
} mk_operand;

/* Node descriptor: exactly 256 bytes, shared by a node's instructions. */
typedef struct {
  int32_t opcode, flags, dtype, node_start;
  int32_t M, N, K, Nb;       /* GEMM: out [M,N], B [K,Nb]; others: rows, cols */
  int32_t split, n_instr, heads, kv_heads;
  int32_t head_dim, causal, rope_cols, seq;
  float eps, scale, reserved_f0, reserved_f1;
  mk_operand a, b, out, bias, res, gamma, part, aux;
  int64_t part_plane;        /* elements between split-K planes of part     */
  int32_t tile_m, tile_n;    /* GEMM kernel tile: rows x weight columns     */
  int32_t layout;            /* weight: 0 row-major [K, Nb]; 1 packed GEMV
                                column tiles [tiles][K][tile_n]; 2 packed
                                GEMM tiles [tiles][K/64][tile_n][64]       */
  int32_t lines_own;         /* 1: every tensor this node reads that the run
                                writes is written in whole 128-byte lines,
                                each by instructions its readers wait on, in
                                a slot of its own (row-major GEMM nodes
                                only); their counter waits then skip the
                                cache invalidation when all buffers are
                                128-byte aligned                           */
  int32_t reserved[MK_NODE_WORDS - 20 - 8 * 4 - 2 - 2 - 1 - 1];
} mk_node;

typedef struct mk_graph mk_graph;
typedef struct mk_plan mk_plan;

/* Error record of a failed run (filled when a wait times out). */
typedef struct {
  int32_t code;        /* MK_OK or MK_E_DEADLOCK                           */
  int32_t cu;          /* virtual CU that gave up                          */
  int32_t instr;       /* instruction index it was waiting in              */
  int32_t barrier;     /* counter id                                       */
  int32_t value;       /* counter value seen                               */
  int32_t need;        /* value waited for (epoch * target)                */
} mk_run_error;

/* ---- graph building (host only; "Implementing a Mega Kernel for B300",
 *      section 1) --------------------------------------------------------- */
mk_status mk_graph_create(mk_graph **g);
void mk_graph_destroy(mk_graph *g);
/* New tensor; shape has ndim (1..4) entries.  Ids are dense from 0. */
mk_status mk_graph_tensor(mk_graph *g, mk_dtype dt, int ndim, const int64_t *shape,
                          mk_role role, int32_t *id);
/* Step-1 range view [lo, hi) of tensor src in its left-padded 4-D
 * coordinates (MegaKittens Internals section 02, step 4).  A view gets its
 * own id and may be used wherever a tensor id is accepted. */
mk_status mk_graph_view(mk_graph *g, int32_t src, const int64_t lo[4],
                        const int64_t hi[4], int32_t *id);
/* Append an op; ops must be added in topological order. */
mk_status mk_graph_op(mk_graph *g, mk_op_kind kind, const int32_t *in, int n_in,
                      int32_t out, const mk_op_attrs *attrs);

/* ---- compile (host only, no GPU needed) -------------------------------- */
/* Compile graph g into a plan: lower every op into tile instructions with
 * read and write boxes, place instruction i on CU i mod num_cus in
 * iteration i / num_cus, give tensors buffer slots (pooled under `reuse`),
 * derive one counter per (producer node, dependency set) with target = the
 * set's size, and pack the 256-byte records (MegaKittens Internals, section
 * 04, the scheduler's four phases, and section 05, placement; the split-K
 * GEMV tasks and epilogue flags of "Implementing a Mega Kernel for B300",
 * section 2).  opts may be NULL (all defaults).  On MK_OK *plan is a new
 * plan owned by the caller (mk_plan_destroy); the graph may be destroyed
 * afterwards.  Errors: MK_E_INVALID (shapes, dtypes, non-topological
 * order), MK_E_LIMIT (more than MK_MAX_SRC / MK_MAX_DST counters on one
 * instruction, more than MK_MAX_TENSORS slots); *plan is NULL then.  A
 * valid graph the GPU kernels do not implement still builds (for host
 * profiles) and its runs fail with MK_E_UNSUPPORTED. */
mk_status megakernel_build(const mk_graph *g, const mk_build_options *opts,
                           mk_plan **plan);
/* Free a plan and its device state (records, counters, intermediates).
 * The caller must have synchronised every stream the plan ran on. */
void mk_plan_destroy(mk_plan *p);

/* ---- run --------------------------------------------------------------- */
/* One forward as one persistent launch of num_cus workgroups on `stream`
 * (a hipStream_t; 0 = the null stream): each workgroup walks its column of
 * the instruction list, waits until every source counter of an
 * instruction reaches epoch * target, runs the tile body and arrives on the
 * destination counters (MegaKittens Internals, section 07, one launch per
 * call, and sections 08-09, the interpreter loop; "Beating torch.compile
 * with Megakernels in CuTe DSL", "Cooperative Kernel" and "Dependency
 * Management and Scheduling").  buffers[i] is the device pointer of tensor
 * id i for every caller-owned tensor (inputs, weights, outputs), 16-byte
 * aligned; entries of views and intermediates are ignored; n_buffers is at
 * least the number of graph tensors.  A weight the plan packs
 * (mk_plan_weight_layout) is passed as its packed buffer.  When every
 * buffer is 128-byte aligned (torch allocations are), nodes marked
 * lines_own skip the cache invalidation after their counter waits; with
 * any buffer less aligned they keep it, and the results are the same.
 *
 * Residency: with opts.cooperative = 0 the launch is an ordinary one, and
 * the kernel's LDS use allows one workgroup per CU, so all num_cus
 * workgroups are resident together only when no other work holds a CU.
 * Under the static placement a workgroup that never becomes resident
 * leaves its instructions unrun: the other workgroups' waits then give up
 * after spin_limit_us and the run ends with the error record set.  With
 * opts.queue = 1 instructions are taken from a work queue in list order
 * and any number of resident workgroups completes the run.
 * opts.cooperative = 1 has the runtime guarantee residency.
 *
 * Asynchronous: returns once the launch is queued; call mk_plan_check to
 * learn whether a counter wait gave up.  Errors: MK_E_UNSUPPORTED (plan
 * the kernels do not implement, or built for another CU count),
 * MK_E_INVALID (missing or misaligned buffer, plan uploaded to another
 * device), MK_E_HIP (runtime call failed), MK_E_DEADLOCK (an earlier run
 * of this plan is known, from the host-visible copy of its error record,
 * to have given up and mk_plan_check has not been called since; nothing
 * is launched). */
mk_status megakernel_run(mk_plan *p, void *const *buffers, int n_buffers, void *stream);
/* megakernel_run that also writes four wall-clock stamps per executed
 * instruction (fetched, counters satisfied, body done, released) to the
 * caller-owned device array trace[4 * n_iters * num_cus + 4 * num_cus]
 * (uint64; instruction i at 4 * i, Noop slots left untouched).  The stamps
 * come from the GPU's constant-rate wall clock; a debugging aid after the
 * intra-kernel timing of "Beating torch.compile with Megakernels in CuTe
 * DSL", "Intrakernel Profiling".  The last 4 * num_cus words hold, for
 * workgroup b at 4 * (n_iters * num_cus + b): the wall clock and the
 * shader-clock counter when it starts, then both again when it finishes
 * (left untouched if it exits early), so that the core clock during the
 * run is (d shader clock) / (d wall clock) * mk_wall_clock_khz. */
mk_status megakernel_run_traced(mk_plan *p, void *const *buffers, int n_buffers, void *stream,
                                uint64_t *trace);
/* The per-op baseline: the same records and tile bodies, one ordinary
 * launch per node (grid = the node's instruction count) with stream order
 * in place of counters; the comparison that "Beating torch.compile with
 * Megakernels in CuTe DSL", "Takeaways", makes against one launch per op.
 * Arguments, ownership and errors as megakernel_run. */
mk_status megakernel_run_per_op(mk_plan *p, void *const *buffers, int n_buffers,
                                void *stream);
/* megakernel_run for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It calls no hipMalloc, hipFree or other allocating routine:
 * the plan's error record, counters, records, node table and plan-owned
 * intermediates live in a file-scope device array of 64 MiB per GPU,
 * held from the library's load until the process ends.  Every call
 * clears the error record and counters with a fill kernel, uploads the
 * plan's records, node table and constant tables (asynchronous copies
 * from host memory the plan owns; keep the plan alive until the stream has
 * passed them), then launches as megakernel_run.  The array keeps the last
 * call's contents and is shared by every call on that GPU, whatever the
 * plan: calls that overlap on one GPU (other streams, other threads) race
 * and give wrong results.  Errors: MK_E_LIMIT when the plan needs more
 * than 64 MiB (the message gives the size; nothing is launched), and those
 * of megakernel_run, except that no earlier abort is refused (each call
 * starts from a cleared record).  mk_plan_check afterwards reads the error
 * record of the last allocation-free call on the plan's device. */
mk_status megakernel_run_noalloc(mk_plan *p, void *const *buffers, int n_buffers, void *stream);
/* Synchronise `stream` and read the plan's error record. */
mk_status mk_plan_check(mk_plan *p, void *stream, mk_run_error *err);

/* ---- introspection ----------------------------------------------------- */
/* Plan statistics: instruction and wave counts, counters, slots (the
 * scheduler figures MegaKittens Internals, section 04, reports for its
 * worked example) and the algorithmic flops and HBM bytes of the graph,
 * computed from the graph that was compiled ("Implementing a Mega Kernel
 * for B300", the section on measuring: count from the graph that runs,
 * not from hand-typed shapes).  MK_E_INVALID on a null argument. */
mk_status mk_plan_stats_get(const mk_plan *p, mk_plan_stats *out);
/* The flat instruction list (MegaKittens Internals, section 04, phase 4,
 * emit, and section 06, the fixed 256-byte record): n_instr records of
 * MK_INSTR_WORDS int32 each, laid out as mk_instr, record i for CU
 * i mod num_cus.  *words points into the plan and stays valid until
 * mk_plan_destroy.  coord: GEMM/GEMV (tm, tn, s, dup copy); REDUCE
 * (tm, tn, 0, 0); RMSNORM (row block, 0, 0, 0); ATTENTION (q block, head,
 * 0, 0); EW_* (tile row, tile col, 0, 0); ATTN_PARTIAL (key chunk, kv
 * head, 0, 0); ATTN_COMBINE (kv head, 0, 0, 0).  MK_E_INVALID on a null
 * argument. */
mk_status mk_plan_instructions(const mk_plan *p, const int32_t **words,
                               int64_t *n_instr, int32_t *words_per_instr);
mk_status mk_plan_nodes(const mk_plan *p, const int32_t **words, int64_t *n_nodes,
                        int32_t *words_per_node);
/* Target of every counter (MegaKittens Internals, section 04, phase 3:
 * one barrier per (producer node, dependency set), target = the number of
 * producer instructions in the set; reuse barriers count every reader of a
 * pooled slot's previous tensor).  Counter ids are canonical: ordered by
 * the first instruction that waits on them, input barriers before reuse
 * barriers, then by producer node.  *targets points into the plan. */
mk_status mk_plan_barriers(const mk_plan *p, const int32_t **targets, int64_t *n);
/* slot of each tensor id (-1 for views and unused tensors). */
mk_status mk_plan_slots(const mk_plan *p, const int32_t **slot_of_tensor, int64_t *n);
/* Tile parameters the compiler chose for graph op `op`. */
mk_status mk_plan_op_tile(const mk_plan *p, int32_t op, mk_tile *out);
/* Layout in which the plan reads weight tensor `tensor`.  *packed = 0: the
 * caller's row-major tensor as declared.  *packed = 1: a GEMV reads it as
 * packed column tiles and every run takes, in buffers[tensor], a device
 * buffer of *bytes bytes filled by mk_plan_pack_weight.
 *
 * GEMV packed layout (bn = the op's tile.bn output columns per tile, T =
 * ceil(N / bn) tiles, w = bn, or 2 * bn under SILU_MUL): element
 * [t][k][j] of a [T][K][w] array holds W[k][col(t * bn + j)] for j < bn
 * and, under SILU_MUL, W[k][N + col(t * bn + j - bn)] for j >= bn; entries
 * whose position t * bn + j (mod bn under SILU_MUL) reaches N are zero.
 * col() is the identity except under ROPE, where output positions
 * [0, rope_cols) are interleaved in rotation pairs: position p of head
 * h = p / head_dim, i = (p % head_dim) / 2 maps to column
 * h * head_dim + i + (p % 2) * head_dim / 2, so each tile holds both
 * columns of every rotation pair it touches.
 *
 * GEMM packed layout (w = weight columns per tile = tile.bn, or 2 * tile.bn
 * under SILU_MUL; T = ceil(N / tile.bn) tiles): element [t][kt][j][kk] of
 * a [T][K/64][w][64] array holds W[64 kt + kk][col], col = t * w + j;
 * under SILU_MUL each half of a tile (h = j / (w/2), q = j % (w/2)) holds
 * the gate columns, then the up columns, of the same w/4 outputs
 * o = t * w/2 + h * w/4 + q % (w/4): col = o for q < w/4, else N + o.
 * Columns whose output reaches N are zero.
 *
 * Both layouts are this library's own: they make each instruction's
 * weight tile (per K step for GEMM) one contiguous stream with every
 * weight column's K values together. */
mk_status mk_plan_weight_layout(const mk_plan *p, int32_t tensor, int32_t *packed,
                                int64_t *bytes);
/* Fill the packed buffer dst (device, mk_plan_weight_layout bytes) from the
 * row-major weight src (device) on `stream`.  Call once per weight value;
 * runs read dst, not src.  Fails with MK_E_INVALID for a tensor the plan
 * does not pack. */
mk_status mk_plan_pack_weight(mk_plan *p, int32_t tensor, const void *src, void *dst,
                              void *stream);
/* Copy the counters (each the sum of its slots) to host memory after a run
 * (synchronises `stream`); host has room for n >= the number of counters.
 * After e completed runs every counter equals e * its target, the
 * post-run check of MegaKittens Internals, section 07 (counters return to
 * a known state between calls; here by epochs instead of zeroing).
 * MK_E_INVALID if host is null or too small, MK_E_HIP on a runtime error. */
mk_status mk_plan_read_counters(mk_plan *p, int32_t *host, int64_t n, void *stream);
/* Runs so far (the epoch the next run waits against is this + 1). */
mk_status mk_plan_epoch(const mk_plan *p, int64_t *epoch);

/* Rate of the GPU wall clock that megakernel_run_traced stamps, in kHz, for
 * the current device. */
mk_status mk_wall_clock_khz(int32_t *khz);

/* Calibration, not part of the path: the MFMA rate this part sustains
 * when nothing but v_mfma_f32_32x32x16_{f16,bf16} runs, as a measured
 * ceiling beside the nominal peak (the measurement discipline of
 * "Hand-writing a Blackwell GEMM", "How I measured": rates against what
 * the hardware delivers, on realistic data).  `blocks` workgroups of 512
 * threads (one per CU); thread t of workgroup b reads 16 sixteen-byte
 * operand fragments at ops[(b * 512 + t) * 16 ..] (caller-owned device
 * memory of blocks * 131072 bytes, fp16 or bf16 values per `dtype`) into
 * registers, then issues iters * 8 MFMAs that cycle through 8 A and 8 B
 * fragments into 4 independent accumulators, and writes one float per
 * thread to out[b * 512 + t] (device, blocks * 2048 bytes).  One launch is
 * blocks * iters * 2097152 flops.  Asynchronous on `stream`; the caller
 * times it.  MK_E_INVALID for null pointers, blocks outside 1..65535,
 * iters < 1 or a dtype other than MK_F16 / MK_BF16; MK_E_HIP on a launch
 * error. */
mk_status mk_probe_mfma(const void *ops, float *out, int32_t blocks, int32_t iters, int32_t dtype,
                        void *stream);

const char *mk_last_error(void);
int32_t mk_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
