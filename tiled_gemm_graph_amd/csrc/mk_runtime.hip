// Runtime: device state of a plan, one-launch forward, per-op baseline.
//
// The plan's records, node table and counters are uploaded once on the first
// run ("Implementing a Mega Kernel for B300", section 6: upload the
// descriptors once; only addresses change per call).  Counters are never
// reset between runs: run e waits for epoch * target, so after e runs every
// counter equals e * target.  (MegaKittens Internals section 07 instead
// zeroes them with a kernel before every launch.)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mk_instances.h"
#include "mk_internal.h"
#include "mk_kernels.h"

const char* mk_plan_unsupported_reason(const mk_plan* p);

struct mk_plan_device {
  int device = -1;
  mk_instr* d_instrs = nullptr;
  mk_node* d_nodes = nullptr;
  int* d_counters = nullptr;
  int* d_err = nullptr;
  int* h_abort = nullptr;     // pinned host copy of the abort flag
  std::vector<void*> owned;   // by slot (plan-owned buffers), else nullptr
  std::vector<size_t> owned_bytes;
  std::vector<char> poison;   // by slot: filled with NaN bytes before a run
  long long spin_ticks = 0;
  int max_target = 1;
  int ctr_stride = 1;         // int32 slots per counter (counter layout of mk.h)
  size_t ctr_slots = 1;       // counter slots; the two work-queue ticket
                              // words follow on a 128-byte line of their own
  unsigned ops = 0;           // op families of the plan's instructions
};
constexpr size_t kTicketPad = 32;   // int32 words after the counter slots

// The array behind megakernel_run_noalloc (64 MiB per GPU, see below).
static __device__ __align__(256) unsigned char scratch[(size_t)64 << 20];

// MFMA issue-rate probe (mk_probe_mfma): operands in registers, changing
// every instruction, four independent accumulators per wave, two waves per
// SIMD; 96 KB of LDS keeps it to one workgroup per CU.
template <int DT>
__global__ void __launch_bounds__(512, 1) mk_probe_mfma_kernel(const mkd::u32x4* __restrict__ ops, float* __restrict__ out,
                                                              int iters) {
  __shared__ int pin[24 * 1024];
  const int t = threadIdx.x;
  if (t == 0) pin[0] = 0;
  __syncthreads();
  const mkd::u32x4* p = ops + ((size_t)blockIdx.x * 512 + t) * 16;
  mkd::u32x4 A[8], B[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    A[j] = p[j];
    B[j] = p[8 + j];
  }
  mkd::f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      c0 = mkd::mfma32<DT>(A[j], B[j], c0);
      c1 = mkd::mfma32<DT>(A[j + 1], B[(j + 3) & 7], c1);
      c2 = mkd::mfma32<DT>(A[j + 2], B[(j + 6) & 7], c2);
      c3 = mkd::mfma32<DT>(A[j + 3], B[(j + 1) & 7], c3);
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) sum += c0[e] + c1[e] + c2[e] + c3[e];
  out[(size_t)blockIdx.x * 512 + t] = sum + (float)pin[0];
}

// Fill n 32-bit words with v (the NaN poison of debug_poison runs).
__global__ void mk_fill_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Packed column tiles of a row-major weight src [K][ld] (the layout of
// mk_plan_weight_layout): element e of dst [tiles][K][wc] takes src at row k
// and the column of tile position t * bn + j (gate) or N + that column (up,
// j >= bn under SILU_MUL); positions at or past N are zero.
__global__ void mk_pack_kernel(const unsigned short* __restrict__ src, unsigned short* __restrict__ dst,
                               long K, long N, long ld, int bn, int wc, long tiles, int silu, int hd,
                               long rope_cols) {
  const long total = tiles * K * wc;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const int j = (int)(e % wc);
    const long k = (e / wc) % K;
    const long t = e / ((long)wc * K);
    int pj = j;
    long up = 0;
    if (silu && j >= bn) {
      pj = j - bn;
      up = N;
    }
    const long pos = t * bn + pj;
    unsigned short v = 0;
    if (pos < N) {
      long col = pos;
      if (hd > 0 && pos < rope_cols) {
        const long h = pos / hd, w = pos - h * hd;
        col = h * hd + (w >> 1) + (w & 1) * (hd >> 1);
      }
      v = src[k * ld + up + col];
    }
    dst[e] = v;
  }
}

// GEMM tiles of a row-major weight src [K][ld] (mk_plan_weight_layout):
// element e of dst [tiles][K/64][bn][64] is src[kt * 64 + kk][col] for
// weight column j of tile t.  Plain: col = t * bn + j.  SILU_MUL: each half
// of the tile (wn = bn / 2 columns) holds gate columns then up columns of
// the same wn / 2 outputs o = t * bn / 2 + (j / wn) * wn / 2 + (j % wn) % (wn / 2),
// col = o (gate) or N + o (up).  Outputs at or past N are zero.
__global__ void mk_pack_gemm_kernel(const unsigned short* __restrict__ src, unsigned short* __restrict__ dst,
                                    long K, long N, long ld, int bn, long tiles, int silu) {
  const long nkt = K / 64;
  const long total = tiles * K * bn;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (long)gridDim.x * blockDim.x) {
    const long kk = e % 64;
    const long j = (e / 64) % bn;
    const long kt = (e / (64L * bn)) % nkt;
    const long t = e / (64L * bn * nkt);
    long o, col;
    if (silu) {
      const long wn = bn / 2, q = j % wn;
      o = t * (bn / 2) + (j / wn) * (wn / 2) + q % (wn / 2);
      col = q < wn / 2 ? o : N + o;
    } else {
      o = t * bn + j;
      col = o;
    }
    dst[e] = o < N ? src[(kt * 64 + kk) * ld + col] : (unsigned short)0;
  }
}

namespace {

// The kernel instance a plan (or node) runs on and its workgroup size: an
// eight-wave instance when every instruction is a packed GEMM tile or a
// REDUCE, RMSNORM, ATTENTION or elementwise instruction (at least one packed
// GEMM among them) and every REDUCE tile fits the eight-wave body's LDS;
// otherwise the smallest four-wave instance whose op families cover `ops`.
struct Launch {
  const void* fn;
  int threads;
};
bool wide_ok(const mk_plan* p) {
  bool any = false;
  for (const mk::Node& n : p->nodes) {
    if (n.ins.empty()) continue;
    switch (n.opcode) {
      case MK_I_GEMM:
        if (n.desc.layout != 2) return false;
        any = true;
        break;
      case MK_I_REDUCE:
        for (const mk::Instr& in : n.ins) {
          const long wc = (long)(in.c1 - in.c0) * ((n.flags & MK_EP_SILU_MUL) ? 2 : 1);
          if ((320 + 512 * 8 + (long)(in.r1 - in.r0) * wc) * 4 > mkd::kSmemBytes) return false;
        }
        break;
      case MK_I_RMSNORM:
      case MK_I_ATTENTION:
      case MK_I_EW_ADD:
      case MK_I_EW_RELU:
        break;
      default:
        return false;
    }
  }
  return any;
}
// Entry point of a kernel instance; the instances live in three units of
// their own (mk_instances.h).  Every (persistent, ops, nt) the selection
// below asks for is held by one of them.
const void* instance(bool persistent, unsigned ops, int nt) {
  const void* f = mk::instances_wide(persistent, ops, nt);
  if (!f) f = mk::instances_gemv(persistent, ops, nt);
  if (!f) f = mk::instances_gemm(persistent, ops, nt);
  if (!f) f = mk::instances_all_p(persistent, ops, nt);
  if (!f) f = mk::instances_all_n(persistent, ops, nt);
  return f;
}
Launch persistent_for(unsigned ops, bool wide) {
  using namespace mkd;
  if (wide && (ops & ~(kOpGemm | kOpOther)) == 0) {
    if (ops == kOpGemm) return {instance(true, kOpGemm, 512), 512};
    return {instance(true, kOpGemm | kOpOther, 512), 512};
  }
  if ((ops & ~kOpGemv) == 0) return {instance(true, kOpGemv, 256), 256};
  if ((ops & ~kOpGemm) == 0) return {instance(true, kOpGemm, 256), 256};
  if ((ops & kOpGemv) == 0) return {instance(true, kOpGemm | kOpOther, 256), 256};
  if ((ops & kOpGemm) == 0) return {instance(true, kOpGemv | kOpOther, 256), 256};
  return {instance(true, kOpAll, 256), 256};
}
Launch node_kernel_for(unsigned ops, bool wide) {
  using namespace mkd;
  if (wide && (ops & kOpGemv) == 0) {
    if (ops == kOpGemm) return {instance(false, kOpGemm, 512), 512};
    if (ops == kOpOther) return {instance(false, kOpOther, 512), 512};
    return {instance(false, kOpGemm | kOpOther, 512), 512};
  }
  if ((ops & ~kOpGemv) == 0) return {instance(false, kOpGemv, 256), 256};
  if ((ops & ~kOpGemm) == 0) return {instance(false, kOpGemm, 256), 256};
  if ((ops & kOpGemv) == 0) return {instance(false, kOpGemm | kOpOther, 256), 256};
  if ((ops & kOpGemm) == 0) return {instance(false, kOpGemv | kOpOther, 256), 256};
  return {instance(false, kOpAll, 256), 256};
}

using mk::set_error;

mk_status hip_fail(hipError_t e, const char* what) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return MK_E_HIP;
}
#define HIPCHK(x)                                        \
  do {                                                   \
    hipError_t e_ = (x);                                 \
    if (e_ != hipSuccess) return hip_fail(e_, #x);       \
  } while (0)

void free_device(mk_plan_device* d) {
  if (!d) return;
  if (d->d_instrs) (void)hipFree(d->d_instrs);
  if (d->d_nodes) (void)hipFree(d->d_nodes);
  if (d->d_counters) (void)hipFree(d->d_counters);
  if (d->d_err) (void)hipFree(d->d_err);
  if (d->h_abort) (void)hipHostFree(d->h_abort);
  for (void* q : d->owned)
    if (q) (void)hipFree(q);
  delete d;
}

mk_status ensure_device(mk_plan* p) {
  const char* why = mk_plan_unsupported_reason(p);
  if (why && *why) {
    set_error(std::string("plan cannot run on the GPU: ") + why);
    return MK_E_UNSUPPORTED;
  }
  if (p->opts.reuse == 2) {
    set_error("reuse mode 2 (outputs in pooled slots) is a host-only profile");
    return MK_E_UNSUPPORTED;
  }
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  if (p->dev) {
    if (p->dev->device != dev) {
      set_error("plan was uploaded to another device");
      return MK_E_INVALID;
    }
    return MK_OK;
  }
  int ncu = 0;
  HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  if (ncu != p->opts.num_cus) {
    set_error("plan was built for " + std::to_string(p->opts.num_cus) + " CUs, device has " +
              std::to_string(ncu));
    return MK_E_UNSUPPORTED;
  }
  int coop = 0;
  HIPCHK(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
  if (!coop) {
    set_error("device does not support cooperative launch");
    return MK_E_UNSUPPORTED;
  }
  for (const Launch& k : {persistent_for(mkd::kOpAll, false), persistent_for(mkd::kOpGemv, false),
                          persistent_for(mkd::kOpGemm, false), persistent_for(mkd::kOpGemm | mkd::kOpOther, false),
                          persistent_for(mkd::kOpGemm, true), persistent_for(mkd::kOpGemm | mkd::kOpOther, true),
                          persistent_for(mkd::kOpGemv | mkd::kOpOther, false)}) {
    int blocks = 0;
    HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k.fn, k.threads, 0));
    if (blocks < 1) {
      set_error("persistent kernel does not fit one workgroup per CU");
      return MK_E_UNSUPPORTED;
    }
  }
  auto* d = new mk_plan_device();
  d->device = dev;
  auto bail = [&](hipError_t e, const char* w) {
    free_device(d);
    return hip_fail(e, w);
  };
  hipError_t e;
  const size_t rec_bytes = p->records.size() * sizeof(mk_instr);
  if ((e = hipMalloc(&d->d_instrs, std::max<size_t>(rec_bytes, 256))) != hipSuccess) return bail(e, "hipMalloc records");
  if (rec_bytes && (e = hipMemcpy(d->d_instrs, p->records.data(), rec_bytes, hipMemcpyHostToDevice)) != hipSuccess)
    return bail(e, "hipMemcpy records");
  const size_t nd_bytes = p->node_descs.size() * sizeof(mk_node);
  if ((e = hipMalloc(&d->d_nodes, std::max<size_t>(nd_bytes, 256))) != hipSuccess) return bail(e, "hipMalloc nodes");
  if (nd_bytes && (e = hipMemcpy(d->d_nodes, p->node_descs.data(), nd_bytes, hipMemcpyHostToDevice)) != hipSuccess)
    return bail(e, "hipMemcpy nodes");
  for (int32_t t : p->targets)
    if (t <= MK_SLICE_MAX) d->ctr_stride = std::max(d->ctr_stride, (int)((t + 31) / 32 * 32));
  d->ctr_slots = std::max<size_t>(p->targets.size(), 1) * (size_t)d->ctr_stride;
  const size_t ctr_bytes = (d->ctr_slots + kTicketPad) * sizeof(int);
  if ((e = hipMalloc(&d->d_counters, ctr_bytes)) != hipSuccess) return bail(e, "hipMalloc counters");
  if ((e = hipMemset(d->d_counters, 0, ctr_bytes)) != hipSuccess) return bail(e, "hipMemset counters");
  if ((e = hipMalloc(&d->d_err, 8 * sizeof(int))) != hipSuccess) return bail(e, "hipMalloc error record");
  if ((e = hipMemset(d->d_err, 0, 8 * sizeof(int))) != hipSuccess) return bail(e, "hipMemset error record");
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&d->h_abort), sizeof(int), hipHostMallocMapped)) != hipSuccess)
    return bail(e, "hipHostMalloc abort flag");
  *reinterpret_cast<volatile int*>(d->h_abort) = 0;
  for (int32_t t : p->targets) d->max_target = std::max(d->max_target, (int)t);
  for (const mk_instr& r : p->records) d->ops |= mkd::op_family(r.opcode);
  // plan-owned buffers: intermediates, split-K partials, constant tables
  d->owned.assign(p->slot_owner.size(), nullptr);
  d->owned_bytes.assign(p->slot_owner.size(), 0);
  d->poison.assign(p->slot_owner.size(), 0);
  for (size_t s = 0; s < p->slot_owner.size(); ++s) {
    const mk::Tensor& t = p->tensors[p->slot_owner[s]];
    if (t.role != MK_INTERMEDIATE) continue;
    const size_t bytes = ((size_t)std::max<mk::I64>(p->slot_bytes[s], 16) + 15) / 16 * 16;
    if ((e = hipMalloc(&d->owned[s], bytes)) != hipSuccess) return bail(e, "hipMalloc intermediate");
    d->owned_bytes[s] = bytes;
    d->poison[s] = t.const_kind == 0 && p->opts.debug_poison;
    const std::vector<float>& tab = p->const_data[s];
    if (!tab.empty() &&
        (e = hipMemcpy(d->owned[s], tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice)) != hipSuccess)
      return bail(e, "hipMemcpy constant table");
  }
  int rate_khz = 0;
  if ((e = hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess)
    return bail(e, "wall clock rate");
  if (rate_khz <= 0) rate_khz = 100000;
  d->spin_ticks = (long long)(p->opts.spin_limit_us * (double)rate_khz / 1000.0);
  p->dev = d;
  return MK_OK;
}

unsigned ops_of(const mk_plan* p) {
  unsigned ops = 0;
  for (const mk_instr& r : p->records) ops |= mkd::op_family(r.opcode);
  return ops;
}

// 1 when every buffer slot starts a 128-byte line: the condition under
// which nodes marked lines_own skip the cache invalidation of their waits.
int lines_aligned(const mk_plan* p, const mkd::KArgs& a) {
  for (size_t s = 0; s < p->slot_owner.size(); ++s)
    if (reinterpret_cast<uintptr_t>(a.bufs[s]) % 128) return 0;
  return 1;
}

mk_status fill_args(mk_plan* p, void* const* buffers, int n_buffers, mkd::KArgs& a) {
  std::memset(&a, 0, sizeof(a));
  if (n_buffers < p->n_graph_tensors) {
    set_error("buffers must have one entry per graph tensor id");
    return MK_E_INVALID;
  }
  for (size_t s = 0; s < p->slot_owner.size(); ++s) {
    const int tid = p->slot_owner[s];
    const mk::Tensor& t = p->tensors[tid];
    if (t.role == MK_INTERMEDIATE) {
      a.bufs[s] = p->dev->owned[s];
    } else {
      if (!buffers || !buffers[tid]) {
        set_error("missing device buffer for tensor id " + std::to_string(tid));
        return MK_E_INVALID;
      }
      if (reinterpret_cast<uintptr_t>(buffers[tid]) % 16) {
        set_error("device buffer of tensor id " + std::to_string(tid) + " is not 16-byte aligned");
        return MK_E_INVALID;
      }
      a.bufs[s] = buffers[tid];
    }
  }
  a.lines_ok = lines_aligned(p, a);
  a.instrs = p->dev->d_instrs;
  a.nodes = p->dev->d_nodes;
  a.counters = p->dev->d_counters;
  a.ticket = p->dev->d_counters + p->dev->ctr_slots;
  a.queue = p->opts.queue;
  a.n_instr = (int)p->n_instr;
  a.abort_host = p->dev->h_abort;
  a.ctr_stride = p->dev->ctr_stride;
  a.err = p->dev->d_err;
  a.spin_ticks = p->dev->spin_ticks;
  a.n_iters = (int)p->stats.n_iters;
  a.ncu = p->opts.num_cus;
  a.n_nodes = (int)p->node_descs.size();
  return MK_OK;
}

// ------------------------------------------------- allocation-free runs
// Device memory of megakernel_run_noalloc: one array per GPU, held until the
// process ends and shared by every such call on that GPU.  In host code the
// array's name only stands in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t kScratchBytes = sizeof(scratch);
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Counter layout of a plan (mk.h): slots per counter and in all.
void counter_layout(const mk_plan* p, int& stride, size_t& slots, int& max_target) {
  stride = 1;
  max_target = 1;
  for (int32_t t : p->targets) {
    if (t <= MK_SLICE_MAX) stride = std::max(stride, (int)((t + 31) / 32 * 32));
    max_target = std::max(max_target, (int)t);
  }
  slots = std::max<size_t>(p->targets.size(), 1) * (size_t)stride;
}

// Where a plan's device state sits in the array: the error record, the
// counters and ticket words (cleared by every call), the records, the node
// table, then one region per plan-owned buffer.
struct NoallocLayout {
  size_t err = 0, ctr = 0, rec = 0, nodes = 0, total = 0;
  int ctr_stride = 1, max_target = 1;
  size_t ctr_slots = 1;
  std::vector<size_t> slot_off;   // by slot, for plan-owned buffers
};
NoallocLayout noalloc_layout(const mk_plan* p) {
  NoallocLayout L;
  counter_layout(p, L.ctr_stride, L.ctr_slots, L.max_target);
  L.err = 0;
  L.ctr = 256;
  L.rec = align256(L.ctr + (L.ctr_slots + kTicketPad) * sizeof(int));
  L.nodes = align256(L.rec + p->records.size() * sizeof(mk_instr));
  size_t off = align256(L.nodes + p->node_descs.size() * sizeof(mk_node));
  L.slot_off.assign(p->slot_owner.size(), 0);
  for (size_t s = 0; s < p->slot_owner.size(); ++s) {
    if (p->tensors[p->slot_owner[s]].role != MK_INTERMEDIATE) continue;
    L.slot_off[s] = off;
    off = align256(off + (size_t)std::max<mk::I64>(p->slot_bytes[s], 16));
  }
  L.total = off;
  return L;
}

// Device address of this device's array (looked up on the first call).
mk_status scratch_for(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device index beyond the allocation-free path's table");
    return MK_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    HIPCHK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) {
      set_error("hipGetSymbolAddress gave a null address for the scratch array");
      return MK_E_HIP;
    }
    g_scratch[dev] = ptr;
  }
  *out = static_cast<unsigned char*>(g_scratch[dev]);
  return MK_OK;
}

}  // namespace

extern "C" {

mk_status megakernel_run_traced(mk_plan* p, void* const* buffers, int n_buffers, void* stream,
                                uint64_t* trace) {
  if (!p) { set_error("null plan"); return MK_E_INVALID; }
  mk_status st = ensure_device(p);
  if (st != MK_OK) return st;
  mkd::KArgs a;
  if ((st = fill_args(p, buffers, n_buffers, a)) != MK_OK) return st;
  a.trace = reinterpret_cast<unsigned long long*>(trace);
  if (*reinterpret_cast<volatile int*>(p->dev->h_abort)) {
    set_error("an earlier run of this plan gave up a counter wait; call mk_plan_check first");
    return MK_E_DEADLOCK;
  }
  if (p->n_instr == 0) return MK_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // counters hold epoch * target; restart from zero well before int32 overflow
  if ((p->epoch + 1) * (int64_t)p->dev->max_target > (1LL << 30)) {
    HIPCHK(hipMemsetAsync(p->dev->d_counters, 0, (p->dev->ctr_slots + kTicketPad) * sizeof(int), s));
    p->epoch = 0;
  }
  for (size_t k = 0; k < p->dev->owned.size(); ++k) {
    if (!p->dev->poison[k]) continue;
    const size_t n = p->dev->owned_bytes[k] / 4;
    const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(mk_fill_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p->dev->owned[k]), n,
                       0xffffffffu);
    HIPCHK(hipGetLastError());
  }
  a.epoch = (int)(p->epoch + 1);
  const Launch k = persistent_for(p->dev->ops, wide_ok(p));
  void* args[] = {&a};
  if (p->opts.cooperative) {
    HIPCHK(hipLaunchCooperativeKernel(k.fn, dim3(p->opts.num_cus), dim3(k.threads), args, 0, s));
  } else {
    HIPCHK(hipLaunchKernel(k.fn, dim3(p->opts.num_cus), dim3(k.threads), args, 0, s));
  }
  p->epoch += 1;
  return MK_OK;
}

mk_status megakernel_run(mk_plan* p, void* const* buffers, int n_buffers, void* stream) {
  return megakernel_run_traced(p, buffers, n_buffers, stream, nullptr);
}

mk_status megakernel_run_per_op(mk_plan* p, void* const* buffers, int n_buffers, void* stream) {
  if (!p) { set_error("null plan"); return MK_E_INVALID; }
  mk_status st = ensure_device(p);
  if (st != MK_OK) return st;
  mkd::KArgs a;
  if ((st = fill_args(p, buffers, n_buffers, a)) != MK_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool plan_wide = wide_ok(p);
  for (const mk::Node& n : p->nodes) {
    if (n.ins.empty()) continue;
    a.first = n.start;
    a.count = (int)n.ins.size();
    unsigned ops = 0;
    for (int i = 0; i < a.count; ++i) ops |= mkd::op_family(p->records[n.start + i].opcode);
    void* args[] = {&a};
    // the bodies of the megakernel's instance: eight waves for every node
    // of a plan that runs on an eight-wave instance, and for packed GEMM
    // nodes in any plan
    const bool wide = plan_wide || (n.opcode == MK_I_GEMM && n.desc.layout == 2);
    const Launch k = node_kernel_for(ops, wide);
    HIPCHK(hipLaunchKernel(k.fn, dim3(a.count), dim3(k.threads), args, 0, s));
  }
  return MK_OK;
}

mk_status megakernel_run_noalloc(mk_plan* p, void* const* buffers, int n_buffers, void* stream) {
  if (!p) { set_error("null plan"); return MK_E_INVALID; }
  const char* why = mk_plan_unsupported_reason(p);
  if (why && *why) {
    set_error(std::string("plan cannot run on the GPU: ") + why);
    return MK_E_UNSUPPORTED;
  }
  if (p->opts.reuse == 2) {
    set_error("reuse mode 2 (outputs in pooled slots) is a host-only profile");
    return MK_E_UNSUPPORTED;
  }
  const NoallocLayout lay = noalloc_layout(p);
  if (lay.total > kScratchBytes) {
    set_error("plan needs " + std::to_string(lay.total) + " bytes of device state (records, counters, " +
              "intermediates); the allocation-free path holds at most " + std::to_string(kScratchBytes));
    return MK_E_LIMIT;
  }
  if (n_buffers < p->n_graph_tensors) {
    set_error("buffers must have one entry per graph tensor id");
    return MK_E_INVALID;
  }
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  int ncu = 0;
  HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  if (ncu != p->opts.num_cus) {
    set_error("plan was built for " + std::to_string(p->opts.num_cus) + " CUs, device has " + std::to_string(ncu));
    return MK_E_UNSUPPORTED;
  }
  unsigned char* base = nullptr;
  mk_status st = scratch_for(dev, &base);
  if (st != MK_OK) return st;
  mkd::KArgs a;
  std::memset(&a, 0, sizeof(a));
  for (size_t k = 0; k < p->slot_owner.size(); ++k) {
    const int tid = p->slot_owner[k];
    if (p->tensors[tid].role == MK_INTERMEDIATE) {
      a.bufs[k] = base + lay.slot_off[k];
      continue;
    }
    if (!buffers || !buffers[tid]) {
      set_error("missing device buffer for tensor id " + std::to_string(tid));
      return MK_E_INVALID;
    }
    if (reinterpret_cast<uintptr_t>(buffers[tid]) % 16) {
      set_error("device buffer of tensor id " + std::to_string(tid) + " is not 16-byte aligned");
      return MK_E_INVALID;
    }
    a.bufs[k] = buffers[tid];
  }
  a.lines_ok = lines_aligned(p, a);
  int rate_khz = 0;
  HIPCHK(hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev));
  if (rate_khz <= 0) rate_khz = 100000;
  a.instrs = reinterpret_cast<const mk_instr*>(base + lay.rec);
  a.nodes = reinterpret_cast<const mk_node*>(base + lay.nodes);
  a.counters = reinterpret_cast<int*>(base + lay.ctr);
  a.ticket = a.counters + lay.ctr_slots;
  a.err = reinterpret_cast<int*>(base + lay.err);
  a.abort_host = nullptr;
  a.queue = p->opts.queue;
  a.n_instr = (int)p->n_instr;
  a.ctr_stride = lay.ctr_stride;
  a.spin_ticks = (long long)(p->opts.spin_limit_us * (double)rate_khz / 1000.0);
  a.n_iters = (int)p->stats.n_iters;
  a.ncu = p->opts.num_cus;
  a.n_nodes = (int)p->node_descs.size();
  a.epoch = 1;   // counters start from zero on every call
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // the array keeps the previous call's contents: clear the error record,
  // counters and ticket words (a fill kernel, not a memset), upload this
  // plan's records, node table and constant tables
  {
    const size_t words = lay.rec / 4;
    hipLaunchKernelGGL(mk_fill_kernel, dim3((unsigned)std::min<size_t>((words + 255) / 256, 1024)), dim3(256), 0, s,
                       reinterpret_cast<uint32_t*>(base), words, 0u);
    HIPCHK(hipGetLastError());
  }
  if (!p->records.empty())
    HIPCHK(hipMemcpyAsync(base + lay.rec, p->records.data(), p->records.size() * sizeof(mk_instr),
                          hipMemcpyHostToDevice, s));
  if (!p->node_descs.empty())
    HIPCHK(hipMemcpyAsync(base + lay.nodes, p->node_descs.data(), p->node_descs.size() * sizeof(mk_node),
                          hipMemcpyHostToDevice, s));
  for (size_t k = 0; k < p->slot_owner.size(); ++k) {
    if (p->tensors[p->slot_owner[k]].role != MK_INTERMEDIATE) continue;
    const std::vector<float>& tab = p->const_data[k];
    if (!tab.empty()) {
      HIPCHK(hipMemcpyAsync(base + lay.slot_off[k], tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice, s));
    } else if (p->opts.debug_poison) {
      const size_t words = align256((size_t)std::max<mk::I64>(p->slot_bytes[k], 16)) / 4;
      hipLaunchKernelGGL(mk_fill_kernel, dim3((unsigned)std::min<size_t>((words + 255) / 256, 4096)), dim3(256), 0,
                         s, reinterpret_cast<uint32_t*>(base + lay.slot_off[k]), words, 0xffffffffu);
      HIPCHK(hipGetLastError());
    }
  }
  p->noalloc_device = dev;
  if (p->n_instr == 0) return MK_OK;
  const Launch k = persistent_for(ops_of(p), wide_ok(p));
  void* args[] = {&a};
  if (p->opts.cooperative) {
    HIPCHK(hipLaunchCooperativeKernel(k.fn, dim3(p->opts.num_cus), dim3(k.threads), args, 0, s));
  } else {
    HIPCHK(hipLaunchKernel(k.fn, dim3(p->opts.num_cus), dim3(k.threads), args, 0, s));
  }
  return MK_OK;
}

mk_status mk_plan_check(mk_plan* p, void* stream, mk_run_error* err) {
  if (!p) { set_error("null plan"); return MK_E_INVALID; }
  mk_run_error r{};
  if (p->noalloc_device >= 0) {
    // the allocation-free path's error record (the last such call on that device)
    int cur = 0;
    HIPCHK(hipGetDevice(&cur));
    unsigned char* base = nullptr;
    HIPCHK(hipSetDevice(p->noalloc_device));
    mk_status st = scratch_for(p->noalloc_device, &base);
    if (st == MK_OK) {
      int h[8];
      hipError_t e1 = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
      hipError_t e2 = e1 == hipSuccess ? hipMemcpy(h, base, sizeof(h), hipMemcpyDeviceToHost) : e1;
      (void)hipSetDevice(cur);
      if (e2 != hipSuccess) return hip_fail(e2, "reading the allocation-free error record");
      p->noalloc_device = -1;   // reported once; the next call clears the record
      if (h[0] != 0 || h[6] != 0) {
        r.code = h[0]; r.cu = h[1]; r.instr = h[2]; r.barrier = h[3]; r.value = h[4]; r.need = h[5];
        if (err) *err = r;
        set_error("counter wait gave up (allocation-free run): cu " + std::to_string(r.cu) + " instr " +
                  std::to_string(r.instr) + " counter " + std::to_string(r.barrier) + " value " +
                  std::to_string(r.value) + " need " + std::to_string(r.need));
        return MK_E_DEADLOCK;
      }
    } else {
      (void)hipSetDevice(cur);
      return st;
    }
  }
  if (p->dev) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    HIPCHK(hipStreamSynchronize(s));
    int h[8];
    HIPCHK(hipMemcpy(h, p->dev->d_err, sizeof(h), hipMemcpyDeviceToHost));
    r.code = h[0]; r.cu = h[1]; r.instr = h[2]; r.barrier = h[3]; r.value = h[4]; r.need = h[5];
    if (h[0] != 0 || h[6] != 0) {
      // the aborted run left counters mid-epoch: start over from zero
      HIPCHK(hipMemset(p->dev->d_err, 0, 8 * sizeof(int)));
      HIPCHK(hipMemset(p->dev->d_counters, 0, (p->dev->ctr_slots + kTicketPad) * sizeof(int)));
      *reinterpret_cast<volatile int*>(p->dev->h_abort) = 0;
      p->epoch = 0;
      if (err) *err = r;
      set_error("counter wait gave up: cu " + std::to_string(r.cu) + " instr " + std::to_string(r.instr) +
                " counter " + std::to_string(r.barrier) + " value " + std::to_string(r.value) + " need " +
                std::to_string(r.need));
      return MK_E_DEADLOCK;
    }
  }
  if (err) *err = r;
  return MK_OK;
}

mk_status mk_plan_read_counters(mk_plan* p, int32_t* host, int64_t n, void* stream) {
  if (!p || !host) { set_error("null argument"); return MK_E_INVALID; }
  if (n < (int64_t)p->targets.size()) { set_error("host buffer too small"); return MK_E_INVALID; }
  if (!p->dev) {
    std::memset(host, 0, p->targets.size() * sizeof(int32_t));
    return MK_OK;
  }
  HIPCHK(hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)));
  if (!p->targets.empty())
  {
    // each counter is the sum of its slots
    std::vector<int32_t> slots(p->dev->ctr_slots);
    HIPCHK(hipMemcpy(slots.data(), p->dev->d_counters, slots.size() * sizeof(int32_t), hipMemcpyDeviceToHost));
    const int st = p->dev->ctr_stride;
    for (size_t b = 0; b < p->targets.size(); ++b) {
      const int w = p->targets[b] <= MK_SLICE_MAX ? p->targets[b] : 1;
      int64_t v = 0;
      for (int k = 0; k < w; ++k) v += slots[b * st + k];
      host[b] = (int32_t)v;
    }
  }
  return MK_OK;
}

mk_status mk_plan_pack_weight(mk_plan* p, int32_t tensor, const void* src, void* dst, void* stream) {
  if (!p || !src || !dst) { set_error("null argument"); return MK_E_INVALID; }
  const mk::PackInfo* pk = nullptr;
  for (const mk::PackInfo& q : p->packs)
    if (q.tensor == tensor) pk = &q;
  if (!pk) { set_error("tensor " + std::to_string(tensor) + " is not packed by this plan"); return MK_E_INVALID; }
  const long total = pk->tiles * pk->K * pk->wc;
  if (total == 0) return MK_OK;
  const long ld = p->tensors[tensor].shape[3];
  const int blocks = (int)std::min<long>((total + 255) / 256, 8192);
  if (pk->kind == 2) {
    hipLaunchKernelGGL(mk_pack_gemm_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const unsigned short*>(src), static_cast<unsigned short*>(dst), (long)pk->K,
                       (long)pk->N, ld, pk->bn, (long)pk->tiles, pk->silu ? 1 : 0);
    HIPCHK(hipGetLastError());
    return MK_OK;
  }
  hipLaunchKernelGGL(mk_pack_kernel, dim3(blocks), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const unsigned short*>(src), static_cast<unsigned short*>(dst), (long)pk->K,
                     (long)pk->N, ld, pk->bn, pk->wc, (long)pk->tiles, pk->silu ? 1 : 0, pk->head_dim,
                     (long)pk->rope_cols);
  HIPCHK(hipGetLastError());
  return MK_OK;
}

mk_status mk_probe_mfma(const void* ops, float* out, int32_t blocks, int32_t iters, int32_t dtype, void* stream) {
  if (!ops || !out) { set_error("null argument"); return MK_E_INVALID; }
  if (blocks < 1 || blocks > 65535 || iters < 1) { set_error("blocks must be 1..65535 and iters >= 1"); return MK_E_INVALID; }
  if (dtype != MK_F16 && dtype != MK_BF16) { set_error("dtype must be MK_F16 or MK_BF16"); return MK_E_INVALID; }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const mkd::u32x4* o = static_cast<const mkd::u32x4*>(ops);
  if (dtype == MK_BF16)
    hipLaunchKernelGGL(mk_probe_mfma_kernel<MK_BF16>, dim3(blocks), dim3(512), 0, s, o, out, iters);
  else
    hipLaunchKernelGGL(mk_probe_mfma_kernel<MK_F16>, dim3(blocks), dim3(512), 0, s, o, out, iters);
  HIPCHK(hipGetLastError());
  return MK_OK;
}

mk_status mk_wall_clock_khz(int32_t* khz) {
  if (!khz) { set_error("null argument"); return MK_E_INVALID; }
  int dev = 0, rate = 0;
  HIPCHK(hipGetDevice(&dev));
  HIPCHK(hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev));
  *khz = rate;
  return MK_OK;
}

void mk_plan_destroy(mk_plan* p) {
  if (!p) return;
  free_device(p->dev);
  delete p;
}

}  // extern "C"
