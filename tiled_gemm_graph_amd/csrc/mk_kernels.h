// Device side of the tile-graph megakernel for gfx950 (CDNA4).
//
// One persistent workgroup of 256 threads (4 wave64s), or 512 (8 wave64s)
// for plans of packed GEMM tiles, per compute unit walks its share of the
// host-compiled instruction list ("MegaKittens Internals", sections 05 and
// 08-11; "Beating torch.compile with Megakernels in CuTe DSL", "Cooperative
// Kernel"): fetch the 256-byte record, wait until every source counter
// reaches its target for this run (acquire, agent scope; its cache
// invalidation is skipped where skip_invalidate shows it unneeded), run the
// tile body, make the tile's stores visible (release, agent scope) and
// arrive on every destination counter.  Every wait is bounded in time: on expiry the
// workgroup records the failure, raises a shared abort flag that every other
// wait polls, and the whole grid drains.
//
// Tile bodies (all fp32 accumulate, one round-to-nearest-even cast):
//   GEMM      C = A @ B on v_mfma_f32_32x32x16_{f16,bf16}, BM x BNK tile
//             (64/128), K step 64, A and B staged through two LDS buffers;
//             B (K-major weights) is transposed in registers on the way in;
//             epilogue through an fp32 LDS tile.
//   GEMV      M <= 8 rows: each thread streams 16-byte weight chunks of one
//             K row, the activation chunk is staged in LDS, partial sums are
//             reduced across the workgroup.
//   REDUCE    sums split-K partials in a fixed order, then the epilogue.
//   RMSNORM   rows of x * gamma / sqrt(mean(x^2) + eps).
//   ATTENTION causal grouped-query flash attention, 128 queries x one head
//             per instruction, 64-key steps, online softmax in exp2.
//   EW_ADD / EW_RELU  elementwise tiles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mk.h"

namespace mkd {

constexpr int kThreads = 256;
constexpr int kBK = 64;                 // GEMM K step
constexpr int kLdsPad = 8;              // 16-bit elements of row padding
constexpr int kSmemBytes = 144 * 1024;   // dynamic tile arena (LDS); 160 KB per CU in all
constexpr int kMaxNodes = 48;           // node descriptors cached in LDS
constexpr int kGemvBatch = 4;           // 16-byte weight chunks per thread per batch
constexpr int kGemvBufs = 3;            // weight batches in flight per thread
// GEMV body LDS: activations (and later the finished sums), then the
// partial sums of one row: wc * kpad <= 2016 floats for every tile width.
constexpr int kGemvXsFloats = 16384;
constexpr int kGemvRedFloats = 2016;
static_assert((kGemvXsFloats + 8 * kGemvRedFloats + 4 * 8) * 4 <= kSmemBytes, "GEMV body LDS");

struct KArgs {
  const mk_instr* instrs;   // [n_iters][ncu]
  const mk_node* nodes;
  int* counters;
  int* err;                 // code, cu, instr, barrier, value, need, abort
  long long spin_ticks;     // wall-clock ticks a wait may take
  int n_iters, ncu, epoch;
  int first, count;         // per-op mode: records [first, first + count)
  int n_nodes;
  int ctr_stride;           // int32 slots per counter (see mk.h)
  unsigned long long* trace; // optional: 4 wall-clock stamps per instruction
  int* abort_host;          // host-visible copy of the abort flag (pinned memory)
  int* ticket;              // work-queue mode: two ticket words, run e uses e & 1
  int queue;                // 1: instructions taken from the work queue
  int n_instr;              // list length (work-queue mode)
  int lines_ok;             // every buffer 128-byte aligned (mk_node.lines_own applies)
  void* bufs[MK_MAX_TENSORS];
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The thread index, read afresh at each use: the empty volatile asm keeps
// the compiler from hoisting values derived from it out of the persistent
// loop, where every body's per-thread offsets would otherwise stay live (and
// spill) across all the other bodies of the kernel.
__device__ __forceinline__ int tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_to_f(u16 h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float f16_to_f(u16 h) { return (float)__builtin_bit_cast(_Float16, h); }
template <int DT>
__device__ __forceinline__ float to_f(u16 h) { return DT == MK_BF16 ? bf16_to_f(h) : f16_to_f(h); }

__device__ __forceinline__ u16 f_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);                      // round to nearest even
  return (u16)(u >> 16);
}
__device__ __forceinline__ u16 f_to_f16(float f) { return __builtin_bit_cast(u16, (_Float16)f); }
template <int DT>
__device__ __forceinline__ u16 from_f(float f) { return DT == MK_BF16 ? f_to_bf16(f) : f_to_f16(f); }

__device__ __forceinline__ uint32_t word(const u32x4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}
// 16-bit columns 2q+h of rows r0, r1 packed as (row r0, row r1)
__device__ __forceinline__ uint32_t pick2(const u32x4& r0, const u32x4& r1, int n) {
  const uint32_t sel = (n & 1) ? 0x07060302u : 0x05040100u;
  return __builtin_amdgcn_perm(word(r1, n >> 1), word(r0, n >> 1), sel);
}

template <int DT>
__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = word(v, i);
    f[2 * i] = to_f<DT>((u16)(w & 0xffff));
    f[2 * i + 1] = to_f<DT>((u16)(w >> 16));
  }
}
template <int DT>
__device__ __forceinline__ u32x4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (uint32_t)from_f<DT>(f[2 * i]) | ((uint32_t)from_f<DT>(f[2 * i + 1]) << 16);
  return u32x4{w[0], w[1], w[2], w[3]};
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, f32x16 c) {
  if constexpr (DT == MK_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Lane-permuted copy of v (DPP control CTRL, within rows of 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over a workgroup of NT threads; `red` holds at least NT / 64 floats
// of LDS.  The wave sums are added in wave order.
template <int NT = kThreads>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = tid() >> 6;
  __syncthreads();
  if ((tid() & 63) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) s += red[i];
  return s;
}

// Barrier that orders LDS traffic only (global loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wave index as a scalar: branches on it are taken per wave (no exec
// masking), so waits inside a branch are executed only by the waves that
// take it.  Each wave's vector-memory counter is its own; a wait emitted in
// code that every wave runs would also drain the other waves' streams.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(tid() >> 6); }

// A value every lane holds the same (record and node fields read from LDS),
// moved to a scalar register: loop bounds and branches on it become scalar
// branches instead of exec-masked ones.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const char* uni_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

// Base of operand o.  The slot is the same in every lane; saying so keeps
// the table read a scalar load instead of a vector-memory load that would
// have to complete behind every load a wave has in flight.
template <typename T>
__device__ __forceinline__ T* buf(const KArgs& a, const mk_operand& o) {
  return reinterpret_cast<T*>(a.bufs[__builtin_amdgcn_readfirstlane(o.slot)]) + o.off;
}

// ------------------------------------------------------------- epilogue
// Applies the non-partial epilogue to 8 consecutive output columns of one
// row and stores them.  raw(w) returns the 8 fp32 product values at
// weight-tile column w (w = output column for plain tiles; gate at w and up
// at w + half for SILU_MUL).  gr, gc: global row / output column.  ROPE
// rotates the values after BIAS and RESIDUAL, so the partner columns (half
// a head away) take the same steps first.
// 16-byte store that writes through to the device-coherent level (agent
// scope, as the agent-scope atomic stores of the packed GEMV do): a release
// after it needs only its completion, not an L2 write-back.
__device__ __forceinline__ void store16_wt(void* p, const u32x4& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_f32x8_wt(float* p, const float* s) {
  u32x4 lo, hi;
  lo.x = __float_as_uint(s[0]); lo.y = __float_as_uint(s[1]); lo.z = __float_as_uint(s[2]); lo.w = __float_as_uint(s[3]);
  hi.x = __float_as_uint(s[4]); hi.y = __float_as_uint(s[5]); hi.z = __float_as_uint(s[6]); hi.w = __float_as_uint(s[7]);
  store16_wt(p, lo);
  store16_wt(p + 4, hi);
}
__device__ __forceinline__ void store_u16_wt(u16* p, u16 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_u32_wt(void* p, uint32_t v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_f32x2_wt(float* p, float x, float y) {
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads that read from the device-coherent level (agent scope, like the
// counter polls): they never return a line another XCD has since
// rewritten.  A body that reads every value produced in the run through
// them needs no cache invalidation after its counter wait (see
// skip_invalidate).
__device__ __forceinline__ u32x4 ld16_coh(const void* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}
__device__ __forceinline__ u16 ld_u16_coh(const u16* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_f32x2_coh(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return float2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
}

// WT: store through to the device-coherent level (GEMM and GEMV outputs,
// released without an L2 write-back).
template <int DT, bool WT = false, typename Raw>
__device__ __forceinline__ void epilogue8(const KArgs& a, const mk_node& nd, int flags, int gr,
                                          int gc, int w, int half, Raw raw) {
  auto pre = [&](int ww, int cc, float* v) __attribute__((always_inline)) {
    if (flags & MK_EP_SILU_MUL) {
      float g[8], u[8];
      raw(ww, g);
      raw(ww + half, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = silu(g[e]) * u[e];
    } else {
      raw(ww, v);
    }
    if (flags & MK_EP_BIAS) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(buf<u16>(a, nd.bias) + (long)gr * nd.bias.ld + cc);
      float f[8];
      unpack8<DT>(b, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += f[e];
    }
    if (flags & MK_EP_RESIDUAL) {
      const u32x4 b = *reinterpret_cast<const u32x4*>(buf<u16>(a, nd.res) + (long)gr * nd.res.ld + cc);
      float f[8];
      unpack8<DT>(b, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] += f[e];
    }
  };
  float v[8];
  pre(w, gc, v);
  if ((flags & MK_EP_ROPE) && gc < nd.rope_cols) {
    const int hd = nd.head_dim, hh = hd >> 1;
    const int i0 = gc % hd;  // 8 columns never straddle the half (hd % 16 == 0)
    const bool lo = i0 < hh;
    float p[8];
    pre(lo ? w + hh : w - hh, lo ? gc + hh : gc - hh, p);
    const float* tab = buf<float>(a, nd.aux) + (long)gr * hd;  // [cos(half) | sin(half)]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = (i0 + e) % hh;
      const float c = tab[i], s = tab[hh + i];
      v[e] = lo ? v[e] * c - p[e] * s : v[e] * c + p[e] * s;
    }
  }
  if (flags & MK_EP_RELU) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = fmaxf(v[e], 0.0f);
  }
  u16* dst = buf<u16>(a, nd.out) + (long)gr * nd.out.ld + gc;
  if constexpr (WT) store16_wt(dst, pack8<DT>(v));
  else *reinterpret_cast<u32x4*>(dst) = pack8<DT>(v);
}

// ------------------------------------------------------------------ GEMM
// C[BM x BNK] = A[r0:r0+BM, k0:k1] @ B[k0:k1, cols], cols = c0.. (plain) or
// gate c0.. and up N+c0.. (SILU_MUL, BNK/2 each).
template <int BM, int BNK, int DT>
__device__ __forceinline__ void gemm_tile(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem) {
  constexpr int LDS_ROW = kBK + kLdsPad;           // 72 elements = 144 B
  constexpr int A_STAGE = BM * LDS_ROW;            // elements
  constexpr int B_STAGE = BNK * LDS_ROW;
  constexpr int WM = BM / 2, WN = BNK / 2, FM = WM / 32, FN = WN / 32;
  constexpr int A_CHUNKS = BM * kBK / 8 / kThreads;  // 16-byte chunks per thread
  constexpr int RB = BNK / 32;                       // B rows (k) per thread
  constexpr int NCG = BNK / 8;                       // B column groups

  u16* As = reinterpret_cast<u16*>(smem);
  u16* Bs = As + 2 * A_STAGE;
  const int t = tid(), lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int flags = uni(in.flags);
  const bool silu = flags & MK_EP_SILU_MUL;
  const int half = silu ? BNK / 2 : BNK;
  const int M = uni(nd.M), N = uni(nd.N);
  const int r0 = uni(in.r0), c0 = uni(in.c0), k0 = uni(in.k0), k1 = uni(in.k1);
  const u16* A = buf<const u16>(a, nd.a);
  const u16* B = buf<const u16>(a, nd.b);
  const long lda = uni(nd.a.ld), ldb = uni(nd.b.ld);

  // per-thread global addresses
  const u16* a_src[A_CHUNKS];
  int a_dst[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = t + kThreads * i, row = c >> 3, kc = c & 7;
    const int gr = min(r0 + row, M - 1);
    a_src[i] = A + (long)gr * lda + k0 + kc * 8;
    a_dst[i] = row * LDS_ROW + kc * 8;
  }
  const int ncg = t % NCG, kq = t / NCG;
  int wcol = ncg * 8;  // weight-tile column of this thread's 8-column group
  int gcol;
  if (silu) {
    const int j = wcol < half ? wcol : wcol - half;
    const int cl = min(c0 + j, N - 8);
    gcol = wcol < half ? cl : N + cl;
  } else {
    gcol = min(c0 + wcol, N - 8);
  }
  const u16* b_src = B + (long)(k0 + kq * RB) * ldb + gcol;
  // Bt row r keeps its 16-byte k chunk c at c ^ ((r >> 3) & 7): the eight
  // rows a thread writes share r >> 3 = wcol / 8, and without the swizzle
  // the threads of one k group (same kq, wcol 8 apart) would all write the
  // same bank.  MFMA operand reads apply the same swizzle.
  const int b_kswz = ((((kq * RB) >> 3) ^ (ncg & 7)) << 3) + ((kq * RB) & 7);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Global loads run D K steps ahead in a register ring (slot kt % D holds
  // step kt), about 128 registers whatever the tile: with one K step's MFMA
  // work as small as a 64 x 64 tile's, a single step of look-ahead leaves
  // every step waiting out a full memory round trip.  Steps past the end
  // re-read the last one, so every step issues the same loads and each wait
  // leaves the younger steps in flight.
  constexpr int SREGS = 4 * (A_CHUNKS + RB);   // registers per K step
  constexpr int D = (128 / SREGS) < 2 ? 2 : (128 / SREGS) > 8 ? 8 : (128 / SREGS);
  u32x4 ra[D][A_CHUNKS], rb[D][RB];
  auto gload = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) ra[slot][i] = *reinterpret_cast<const u32x4*>(a_src[i] + kt * kBK);
#pragma unroll
    for (int r = 0; r < RB; ++r) rb[slot][r] = *reinterpret_cast<const u32x4*>(b_src + (long)(kt * kBK + r) * ldb);
  };
  auto swrite = [&](int st, int slot) __attribute__((always_inline)) {
    u16* as = As + st * A_STAGE;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<u32x4*>(as + a_dst[i]) = ra[slot][i];
    // transpose RB (k) x 8 (n) into 8 rows of Bt[n][k], RB k-values each
    u16* bs = Bs + st * B_STAGE + wcol * LDS_ROW + b_kswz;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if constexpr (RB == 4) {
        *reinterpret_cast<u32x2*>(bs + n * LDS_ROW) =
            u32x2{pick2(rb[slot][0], rb[slot][1], n), pick2(rb[slot][2], rb[slot][3], n)};
      } else {
        *reinterpret_cast<uint32_t*>(bs + n * LDS_ROW) = pick2(rb[slot][0], rb[slot][1], n);
      }
    }
  };

  const int nk = (k1 - k0) / kBK;
  if (nk > 0) {
#pragma unroll
    for (int s = 0; s < D - 1; ++s) gload(min(s, nk - 1), s);
    swrite(0, 0);
  }
  __syncthreads();
  for (int kt0 = 0; kt0 < nk; kt0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int kt = kt0 + u;
      if (kt >= nk) break;
      gload(min(kt + D - 1, nk - 1), (u + D - 1) % D);
      const u16* as = As + (kt & 1) * A_STAGE;
      const u16* bs = Bs + (kt & 1) * B_STAGE;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        u32x4 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const u32x4*>(as + (wm * WM + i * 32 + (lane & 31)) * LDS_ROW + kk * 16 +
                                                  (lane >> 5) * 8);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * WN + j * 32 + (lane & 31);
          bf[j] = *reinterpret_cast<const u32x4*>(bs + row * LDS_ROW + (((kk * 2 + (lane >> 5)) ^ ((row >> 3) & 7)) << 3));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<DT>(af[i], bf[j], acc[i][j]);
      }
      if (kt + 1 < nk) swrite((kt + 1) & 1, (u + 1) % D);
      __syncthreads();
    }
  }

  // accumulators -> fp32 LDS tile Cs[BM][BNK + 4]
  constexpr int CS = BNK + 4;
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * WM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        const int col = wn * WN + j * 32 + (lane & 31);
        Cs[row * CS + col] = acc[i][j][e];
      }
  __syncthreads();

  const int r1 = in.r1, c1 = in.c1;
  if (flags & MK_EP_PARTIAL) {
    // fp32 partial sums of every weight column: P[s][row][weight col]
    float* P = buf<float>(a, nd.part) + (long)in.split_idx * nd.part_plane;
    constexpr int UNITS = BM * BNK / 8;
    for (int u = t; u < UNITS; u += kThreads) {
      const int row = u / (BNK / 8), w = (u % (BNK / 8)) * 8;
      const int gr = r0 + row;
      const int j = w < half ? w : w - half;
      if (gr >= r1 || c0 + j >= c1) continue;
      const int gc = (silu && w >= half) ? N + c0 + j : c0 + j;
      store_f32x8_wt(P + (long)gr * nd.part.ld + gc, Cs + row * CS + w);
    }
    return;
  }
  constexpr int OUNITS_MAX = BM * BNK / 8;
  const int ounits = BM * (half / 8);
  for (int u = t; u < ounits && u < OUNITS_MAX; u += kThreads) {
    const int row = u / (half / 8), w = (u % (half / 8)) * 8;
    const int gr = r0 + row, gc = c0 + w;
    if (gr >= r1 || gc >= c1) continue;
    epilogue8<DT, true>(a, nd, flags, gr, gc, w, half, [&](int ww, float* o) {
      const float* s = Cs + row * CS + ww;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = s[e];
    });
  }
}

// ----------------------------------------------------- GEMM, packed weight
// C[BM x BN] = A[r0:r0+BM, k0:k1] @ B-tile, with B read from the packed
// layout [T][K/64][BN][64]: for every 64-deep K step, each of the tile's BN
// weight columns holds its 64 k values contiguously, so A rows and B
// columns load the same way.  Both stream into LDS with direct
// global-to-LDS 16-byte loads (no registers), in a ring of ST stages of
// 64-deep K slices (as many as the arena holds, at most 4), so the loads of
// a K step are issued ST - 1 steps before it is used.  An LDS row is 128 bytes (8 chunks of 8 k values); chunk c of row
// r sits at c ^ ((r >> 1) & 7), so the 32 rows an MFMA operand read touches
// spread over all banks.  The swizzle is applied on the global side: lane L
// of a load fills LDS byte L * 16 of its 1 KB block and fetches the chunk
// that belongs there.
//
// Waves hold WM x WN blocks of v_mfma_f32_32x32x16 tiles (the layouts are
// below).  The epilogue goes through an fp32 LDS strip of the whole tile
// width: the packing puts the gate and up columns of one output (SILU_MUL)
// WN/2 columns apart inside a wave column's half, and a rotary partner is
// head_dim/2 columns away in the same tile (tiles hold whole heads).
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ void g2lds16(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)src, (lds_void_t*)lds, 16, 0, 0);
}

// The same load written out, for the GEMM K loop: the compiler cannot tell
// that the loop's LDS operand reads never touch a stage still being filled,
// and before every such read it would wait for all loads in flight.  Here
// the caller orders the loads itself (wait_vmcnt before the barrier that
// precedes a stage's use).  dst is the wave-uniform LDS byte address of the
// 1 KB block (lane L writes byte L * 16 of it); it travels in M0, which is
// restored, so the compiler's own use of M0 is undisturbed.  (readfirstlane:
// the compiler cannot always prove dst uniform, and M0 takes a scalar.)
__device__ __forceinline__ void g2lds16_asm(const void* src, unsigned dst) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src)
      : "memory");
}

// The same load with a scalar base address and a 32-bit per-lane byte
// offset (the SADDR form): the per-stage address step is a scalar add, and
// the per-lane part never changes, so a load costs no vector instruction.
__device__ __forceinline__ void g2lds16_sb(const void* sbase, unsigned voff, unsigned dst) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(sbase)
      : "memory");
}

// s_waitcnt with vmcnt(N) and lgkmcnt(0) (expcnt left alone): this wave's
// LDS reads have completed and at most N of its vector-memory loads are
// still in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// wait_vmcnt_lgkm0 with a wave-uniform count n (0 .. 63) known only at run
// time: a chain of scalar compares, for the few waits of a tile's prologue.
template <int K = 0>
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  if constexpr (K > 63) {
    wait_vmcnt_lgkm0<0>();
  } else {
    if (n <= K) {
      wait_vmcnt_lgkm0<K>();
      return;
    }
    wait_vmcnt_rt<K + 1>(n);
  }
}

// Workgroup barrier with no memory fence: the caller has already waited
// for the operations the barrier publishes (LDS is coherent within the CU);
// the signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Four waves: a 2 x 2 grid, each wave WM x WN = BM / 2 x BN / 2 over the
// whole K range.  Eight waves (two per SIMD, so one wave's MFMAs run while
// the other issues loads or waits at a barrier), with MK_GEMM_KSPLIT
// (default): the same 2 x 2 grid of WM x WN blocks, each held by a pair of
// waves w and w + 4 that take the first and the second half of every
// 64-deep K stage (sub-steps 0-1 and 2-3) and add their sums in the
// epilogue.  A wave's block is then twice as large as in a 4 x 2 grid of
// eight waves, so each MFMA needs a quarter fewer LDS operand bytes.
// Without it: a 4 x 2 grid of eight whole-K waves.
#ifndef MK_GEMM_KSPLIT
#define MK_GEMM_KSPLIT 1
#endif
template <int BM, int BN, int DT, int NW = 4>
__device__ __forceinline__ void gemm_packed_tile(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                                 char* smem, bool bpre = false) {
  constexpr int NT = NW * 64;
  constexpr int ROWB = 128;                         // bytes per LDS row: 64 k values
  constexpr int A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr bool KS = NW == 8 && MK_GEMM_KSPLIT;    // wave pairs split each K stage
  constexpr int NB = KS ? NW / 2 : NW;              // waves (or pairs) with distinct blocks
  constexpr int WGM = NB / 2;                       // wave rows (two wave columns)
  constexpr int SUB = KS ? 2 : 4;                   // 16-deep sub-steps per stage per wave
  constexpr int WM = BM / WGM, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  static_assert(FM >= 1 && FN >= 1, "every wave holds whole 32 x 32 blocks");
  constexpr int A_LOADS = BM / (8 * NW), B_LOADS = BN / (8 * NW);  // 16-byte loads per thread per stage
  static_assert(A_LOADS * 8 * NW == BM && B_LOADS * 8 * NW == BN, "loads cover the tile");
  constexpr int ST = (kSmemBytes / STAGE) < 4 ? (kSmemBytes / STAGE) : 4;
  static_assert(ST >= 2, "two stages must fit in LDS");
  constexpr int L = A_LOADS + B_LOADS;                 // loads per thread per stage
  const int t = tid(), lane = t & 63, wave = t >> 6;
  const int blk = KS ? (wave & 3) : wave;           // output block of this wave
  const int kh = KS ? (wave >> 2) : 0;              // K half of the stage (pairs)
  const int wm = blk >> 1, wn = blk & 1;
  const int flags = uni(in.flags);
  const int M = uni(nd.M), N = uni(nd.N), K = uni(nd.K);
  const int r0 = uni(in.r0), c0 = uni(in.c0), k0 = uni(in.k0), k1 = uni(in.k1);
  const u16* A = buf<const u16>(a, nd.a);
  const long lda = uni(nd.a.ld);

  // Load instruction i of this wave fills rows 8 * (wave + NW * i) .. + 8 of
  // its operand: lane -> row (lane >> 3), physical chunk (lane & 7).  The
  // rows of one lane are 8 NW apart, so they share the swizzle chunk.  Each
  // load is a scalar base (the operand at this K stage) plus a fixed 32-bit
  // byte offset per lane (A has fewer than 2^31 elements).
  const int row0 = 8 * wave + (lane >> 3);
  const unsigned a_chunk = ((lane & 7) ^ ((row0 >> 1) & 7)) << 4;   // bytes
  unsigned a_vo[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) a_vo[i] = (unsigned)(min(r0 + row0 + 8 * NW * i, M - 1) * (int)lda) * 2u + a_chunk;
  const long nkt = K / 64;
  const char* a_sb = uni_ptr(A + k0);
  const char* b_sb = uni_ptr(buf<const u16>(a, nd.b) + ((long)uni(in.coord[1]) * nkt + k0 / 64) * (long)BN * 64);
  unsigned b_vo[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int row = 8 * (wave + NW * i) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    b_vo[i] = (unsigned)(row * 64 + c * 8) * 2u;
  }
  // LDS byte address of the arena (a generic pointer to LDS keeps the LDS
  // offset in its low 32 bits) and the wave index, both as scalars
  const unsigned smem_lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)smem);
  const int wave_s = wave_id();
  // load q (< L) of K stage kt into stage buffer b
  auto load_one = [&](int kt, int b, int q) __attribute__((always_inline)) {
    const unsigned dst = smem_lds + b * STAGE;
    if (q < A_LOADS) {
      g2lds16_sb(a_sb + kt * 128, a_vo[q], dst + (8 * (wave_s + NW * q)) * ROWB);
    } else {
      const int i = q - A_LOADS;
      g2lds16_sb(b_sb + (long)kt * (BN * 128), b_vo[i], dst + A_BYTES + (8 * (wave_s + NW * i)) * ROWB);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // No load the compiler issued may still be in flight when the K loop
  // starts: one that was (a record fetched ahead, another body's prefetch
  // whose register the loop reuses) would make it wait for every
  // outstanding load, the stages in flight included, on each pass.
  wait_vmcnt_lgkm0<0>();

  // Operand fragments of a wave's 16-deep sub-steps of a stage (four, or
  // two in a K-split pair), double-buffered: the LDS reads of the next
  // sub-step are in flight during this one's MFMAs, and those of the next
  // stage's first sub-step during this stage's last one, so no sub-step
  // waits out a whole LDS round trip.
  u32x4 af[2][FM], bf[2][FN];
  auto frags = [&](const char* __restrict__ st, int kk, int b) __attribute__((always_inline)) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = wm * WM + i * 32 + (lane & 31);
      af[b][i] = *reinterpret_cast<const u32x4*>(st + row * ROWB + ((c ^ ((row >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * WN + j * 32 + (lane & 31);
      bf[b][j] = *reinterpret_cast<const u32x4*>(st + A_BYTES + row * ROWB + ((c ^ ((row >> 1) & 7)) << 4));
    }
  };
  // MFMA q of the sub-step whose fragments are in buffer b
  auto mma = [&](int b, int q) __attribute__((always_inline)) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mfma32<DT>(af[b][i], bf[b][j], acc[i][j]);
  };
  // Wait until stage s has landed in this wave, leaving the `younger`
  // stages issued after it in flight (each stage is L loads per thread),
  // and until this wave's LDS reads are done.
  // (younger <= ST - 1: at most 3 stages, 3 L <= 24 loads)
  auto land = [&](int younger) __attribute__((always_inline)) {
    if (younger >= 3) wait_vmcnt_lgkm0<(ST >= 4 ? 3 * L : 0)>();
    else if (younger == 2) wait_vmcnt_lgkm0<(ST >= 3 ? 2 * L : 0)>();
    else if (younger == 1) wait_vmcnt_lgkm0<L>();
    else wait_vmcnt_lgkm0<0>();
  };

  // Stages 0 .. ST-1 fill every buffer first; stage kt + ST is issued once
  // every wave has finished reading stage kt (its buffer), right after the
  // barrier that also publishes stage kt + 1.  That barrier sits before
  // stage kt's last sub-step, whose MFMAs then cover the first LDS reads of
  // stage kt + 1 and the issue of stage kt + ST's loads, one or two loads
  // after each MFMA.  So while stage kt is read, stages kt + 1 .. kt + ST - 1
  // are in flight, and waiting for stage kt + 1 leaves ST - 2 younger ones.
  constexpr int NQ = FM * FN;   // MFMAs per sub-step
  const int nk = (k1 - k0) / 64;
  // With bpre the weight slices of stages 0 .. ST - 1 are already in LDS
  // (issued before the counter wait, complete after the wait above), and
  // these stages load A only: waiting for stage s then leaves A_LOADS per
  // younger prologue stage and L per younger loop stage in flight.
  const int pl = bpre ? A_LOADS : L;   // loads per prologue stage
#pragma unroll
  for (int s = 0; s < ST; ++s)
    if (s < nk)
#pragma unroll
      for (int q = 0; q < L; ++q)
        if (q < A_LOADS || !bpre) load_one(s, s, q);
  // sub-steps of this wave: kb, kb + 1, ... kb + SUB - 1 (wave-uniform)
  const int kb = uni(kh * 2);
  if (nk > 0) {
    if (bpre) wait_vmcnt_rt(pl * min(ST - 1, nk - 1));
    else land(min(ST - 1, nk - 1));
    bare_barrier();
    frags(smem, kb, 0);
  }
  // Stage kt in buffer U = kt % ST (a compile-time index in each copy).  One
  // straight path for every stage (the last one waits for nothing and reads
  // a stale buffer it does not use): only the issue of the next stage's loads
  // is conditional, so the accumulators are never merged from two paths.
  auto stage = [&](auto U, int kt) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;
    const char* __restrict__ cur = smem + u * STAGE;
#pragma unroll
    for (int kk = 0; kk < SUB - 1; ++kk) {
      frags(cur, kb + kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int q = 0; q < NQ; ++q) mma(kk & 1, q);
    }
    if (bpre && kt + 1 < ST) {
      // stage kt + 1 is a prologue stage: younger are the prologue stages
      // after it (A only) and the loop stages issued so far (one per stage
      // before kt)
      wait_vmcnt_rt(pl * max(0, min(ST - 2 - kt, nk - 2 - kt)) + L * max(0, min(kt, nk - ST)));
    } else {
      land(min(ST - 2, nk - 2 - kt));
    }
    bare_barrier();
    frags(smem + ((u + 1) % ST) * STAGE, kb, 0);
    const bool more = kt + ST < nk;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      mma((SUB - 1) & 1, q);
      if (more) {
#pragma unroll
        for (int l = q * L / NQ; l < (q + 1) * L / NQ; ++l) load_one(kt + ST, u, l);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int kt0 = 0; kt0 < nk; kt0 += ST) {
    stage(std::integral_constant<int, 0>{}, kt0);
    if (kt0 + 1 < nk) stage(std::integral_constant<int, 1>{}, kt0 + 1);
    if constexpr (ST > 2) {
      if (kt0 + 2 < nk) stage(std::integral_constant<int, 2>{}, kt0 + 2);
    }
    if constexpr (ST > 3) {
      if (kt0 + 3 < nk) stage(std::integral_constant<int, (ST > 3 ? 3 : 0)>{}, kt0 + 3);
    }
  }

  // ---- epilogue, one 32-row strip of each wave row at a time: the
  // accumulators go to an fp32 LDS strip Cs[32 WGM][BN + 4] (LDS row sr
  // holds tile row (sr / 32) * WM + i * 32 + sr % 32), then 8-column units
  // run the epilogue.  acc[i][j][e] is tile row wm*WM + i*32 + 8*(e>>2) +
  // 4*(lane>>5) + (e&3), weight column wn*WN + j*32 + (lane&31).
  constexpr int CS = BN + 4;
  static_assert(32 * WGM * CS * 4 <= kSmemBytes, "epilogue strip fits the arena");
  float* Cs = reinterpret_cast<float*>(smem);
  const int r1 = in.r1, c1 = in.c1;
  const bool silu_mul = flags & MK_EP_SILU_MUL;
  constexpr int UNITS = 32 * WGM * BN / 8;   // 8-column units of a strip (weight columns)
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    __syncthreads();   // the previous strip (or the last K stage) is consumed
    // a K-split pair: the first half's sums are stored, then the second
    // half adds its own (same lane, same element)
#pragma unroll
    for (int h = 0; h < (KS ? 2 : 1); ++h) {
      if (h == 1) __syncthreads();
      if (kh == h) {
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            float* c = &Cs[(wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * CS + wn * WN + jj * 32 + (lane & 31)];
            *c = h ? *c + acc[i][jj][e] : acc[i][jj][e];
          }
      }
    }
    __syncthreads();
    for (int u = t; u < UNITS; u += NT) {
      const int sr = u / (BN / 8), w = (u % (BN / 8)) * 8;   // strip row, weight column
      const int gr = r0 + (sr >> 5) * WM + i * 32 + (sr & 31);
      if (gr >= r1) continue;
      const float* src = Cs + sr * CS;
      if (flags & MK_EP_PARTIAL) {
        // weight column w -> partial column (gate o, up N + o) or output column
        int pc;
        if (silu_mul) {
          const int h = w / WN, q = w % WN;
          const int o = c0 + h * (WN / 2) + q % (WN / 2);
          if (o >= c1) continue;
          pc = q < WN / 2 ? o : N + o;
        } else {
          pc = c0 + w;
          if (pc >= c1) continue;
        }
        store_f32x8_wt(buf<float>(a, nd.part) + (long)in.split_idx * nd.part_plane + (long)gr * nd.part.ld + pc,
                       src + w);
        continue;
      }
      int gc, ww, half;
      if (silu_mul) {
        // one unit per 8 gate columns: up is WN / 2 columns further
        const int h = w / WN, q = w % WN;
        if (q >= WN / 2) continue;
        gc = c0 + h * (WN / 2) + q;
        ww = w;
        half = WN / 2;
      } else {
        gc = c0 + w;
        ww = w;
        half = BN;
      }
      if (gc >= c1) continue;
      epilogue8<DT, true>(a, nd, flags, gr, gc, ww, half, [&](int x, float* o) {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = src[x + e];
      });
    }
  }
}

// The weight slices of a packed GEMM tile's first K stages, issued into
// their LDS stage buffers before the tile's counters clear (a packed
// weight is a caller input no instruction writes).  Waves 1 .. NW - 1
// issue them, so that wave 0's counter polls do not queue behind the
// loads; the same rows, chunks and LDS addresses as the tile body's own B
// loads.  The tile body then loads A only for these stages.
template <int BM, int BN, int NW>
__device__ __forceinline__ void gemm_packed_prefetch_b(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                                       char* smem) {
  constexpr int ROWB = 128, A_BYTES = BM * ROWB, STAGE = (BM + BN) * ROWB;
  constexpr int ST = (kSmemBytes / STAGE) < 4 ? (kSmemBytes / STAGE) : 4;
  constexpr int NB = BN / 8;   // 1 KB loads (8 weight rows) per stage
  const int w = wave_id();
  if (w == 0) return;
  const int lane = tid() & 63;
  const int K = uni(nd.K), k0 = uni(in.k0), k1 = uni(in.k1);
  const int nk = (k1 - k0) / 64;
  const long nkt = K / 64;
  const char* b_sb = uni_ptr(buf<const u16>(a, nd.b) + ((long)uni(in.coord[1]) * nkt + k0 / 64) * (long)BN * 64);
  const unsigned smem_lds = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)smem);
  for (int j = w - 1; j < NB; j += NW - 1) {
    const int row = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const unsigned vo = (unsigned)(row * 64 + c * 8) * 2u;
#pragma unroll
    for (int st = 0; st < ST; ++st)
      if (st < nk) g2lds16_sb(b_sb + (long)st * (BN * 128), vo, smem_lds + st * STAGE + A_BYTES + (8 * j) * ROWB);
  }
}

// ------------------------------------------------------------------ GEMV
// Small-M GEMM (M <= 8 rows) that streams its weight tile from HBM, with two
// wave roles.  Wave 0 is the controller: it waits on the counters, stages
// the activation chunk in LDS, sums the partial products and stores and
// releases the result.  Waves 1-3 stream the weights: thread tw owns 16-byte
// column group tw % ncg of the weight tile and K rows kr, kr + kpar, ...
// (kpar = 192 / ncg), and keeps a ring of kGemvBufs batches of kGemvBatch
// chunks in flight in registers.  Their stream runs on across consecutive
// GEMV instructions: the loads that follow the last batches of instruction i
// are the first batches of instruction i + 1, issued before that
// instruction's counters clear.
// The vector-memory counter is per wave and retires in order, so the
// controller's small dependent loads and its release never wait behind the
// weight stream.  Weight loads are unconditional (rows past the chunk
// re-read a valid row) so each wait can leave the younger batch in flight.
constexpr int kWThreads = kThreads - 64;   // weight-streaming threads

struct GemvShape {
  int bw, wc, ncg, kpar, cg, kr, kn, nb, ldb;
  long wbase;   // element offset of this thread's first weight column
  bool active;
};
__device__ __forceinline__ GemvShape gemv_shape(const mk_instr& in, const mk_node& nd) {
  GemvShape g;
  const bool silu = in.flags & MK_EP_SILU_MUL;
  const int tw = tid() - 64;
  g.bw = in.c1 - in.c0;
  g.wc = silu ? 2 * g.bw : g.bw;
  g.ncg = g.wc / 8;
  g.kpar = kWThreads / g.ncg;
  g.cg = tw >= 0 ? tw % g.ncg : 0;
  g.kr = tw >= 0 ? tw / g.ncg : g.kpar;
  g.active = tw >= 0 && g.kr < g.kpar;
  const int w = g.cg * 8;
  if (nd.layout) {
    // packed tile coord[1]: [K][tile_n] rows of (gate | up) positions
    const int pc = (silu && w >= g.bw) ? (nd.tile_n >> 1) + (w - g.bw) : w;
    g.ldb = nd.tile_n;
    g.wbase = (long)in.coord[1] * nd.K * nd.tile_n + pc;
  } else {
    g.ldb = nd.b.ld;
    g.wbase = (silu && w >= g.bw) ? nd.N + in.c0 + (w - g.bw) : in.c0 + w;
  }
  g.kn = in.k1 - in.k0;
  const int rows_per_thread = (g.kn + g.kpar - 1) / g.kpar;
  g.nb = (rows_per_thread + kGemvBatch - 1) / kGemvBatch;
  return g;
}

// A weight thread's rows of one GEMV instruction, resolved once: row r of
// the thread (chunk row kr + r * kpar) sits at p + r * step.  rv rows are
// valid; loads clamp to row nrows - 1 (nrows >= 1, a valid row even for an
// idle thread), so every load is issued and each wait can leave the younger
// batches in flight.
struct GemvStream {
  const u16* p;
  long step;
  int nrows, rv, nb;
};
__device__ __forceinline__ GemvStream gemv_stream(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                                  const GemvShape& g) {
  GemvStream st;
  const bool has = g.active && g.kr < g.kn;
  const int kr = has ? g.kr : 0;
  st.p = buf<const u16>(a, nd.b) + g.wbase + (long)(in.k0 + kr) * g.ldb;
  st.step = (long)g.kpar * g.ldb;
  st.rv = has ? (g.kn - g.kr + g.kpar - 1) / g.kpar : 0;
  st.nrows = st.rv > 0 ? st.rv : 1;
  st.nb = g.nb;
  return st;
}

// Batch b (clamped to the last one) of a stream.
__device__ __forceinline__ void gemv_load(const GemvStream& st, int b, u32x4* dst) {
  b = min(b, st.nb - 1);
#pragma unroll
  for (int j = 0; j < kGemvBatch; ++j) {
    const int r = min(b * kGemvBatch + j, st.nrows - 1);
    dst[j] = *reinterpret_cast<const u32x4*>(st.p + (long)r * st.step);
  }
}

// Weight waves: batches 0 .. kGemvBufs-1 of `in` into B.
__device__ __forceinline__ void gemv_prologue(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                              u32x4 (&B)[kGemvBufs][kGemvBatch]) {
  if (wave_id() == 0) return;
  const GemvStream st = gemv_stream(a, in, nd, gemv_shape(in, nd));
#pragma unroll
  for (int k = 0; k < kGemvBufs; ++k) gemv_load(st, k, B[k]);
}

// xk = this thread's first activation (xs + kr); rows r < rv of batch b.
template <int DT, int MAXR>
__device__ __forceinline__ void gemv_fma_batch(const u32x4* wb, int b, const float* xk, int kpar, int rv,
                                               int xstride, int rows, float (&acc)[MAXR][8]) {
#pragma unroll
  for (int j = 0; j < kGemvBatch; ++j) {
    const int r = b * kGemvBatch + j;
    if (r < rv) {
      float f[8];
      unpack8<DT>(wb[j], f);
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        if (m < rows) {
          const float x = xk[m * xstride + r * kpar];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[m][e] = fmaf(x, f[e], acc[m][e]);
        }
      }
    }
  }
}

// Epilogue of a packed column tile (controller wave).  Positions
// [c0, c0 + bw) map to output columns; under ROPE, positions below
// rope_cols come in rotation pairs (column d and d + head_dim / 2 of one
// head), so both partners of a pair are in this tile.  Order: SILU_MUL
// (of the rms-scaled gate and up), BIAS, RESIDUAL, ROPE, RELU, cast.
// Output column of packed-tile position pos (rotation pairs interleaved
// below rope_cols under ROPE).
__device__ __forceinline__ int packed_col(const mk_node& nd, bool rot, int pos) {
  if (!rot) return pos;
  const int hd = nd.head_dim, h = pos / hd, w = pos - h * hd;
  return h * hd + (w >> 1) + (w & 1) * (hd >> 1);
}

// Everything the store of a controller lane's first pair (unit u = lane)
// needs except the sums: prepared while the weight waves stream.
struct PackedEp {
  long off[2];   // output element offsets
  float add[2];  // bias + residual
  float cs, sn;  // rotation of the pair (ROPE)
  float sc;      // 1 / rms of the row (RMSNORM_INPUT), else 1
  int s0;        // sum index of the first column (m * wc + q)
  bool rot;
  bool pair;     // the two outputs are adjacent and 4-byte aligned
};

template <int DT, int MAXR>
__device__ __forceinline__ void gemv_packed_prepare(const KArgs& a, const mk_node& nd, int flags, int r0,
                                                    int c0, int rows, int bw, int wc, const float* sq,
                                                    PackedEp& ep) {
  const int npair = bw >> 1, u = tid() & 63;
  if (u >= rows * npair) return;
  const int m = u / npair, q = (u - m * npair) * 2, gr = r0 + m;
  const bool rot = (flags & MK_EP_ROPE) && c0 + q < nd.rope_cols;
  ep.rot = rot;
  ep.s0 = m * wc + q;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = packed_col(nd, rot, c0 + q + e);
    ep.off[e] = (long)gr * nd.out.ld + c;
    float x = 0.f;
    if (flags & MK_EP_BIAS) x += to_f<DT>(ld_u16_coh(buf<const u16>(a, nd.bias) + (long)gr * nd.bias.ld + c));
    if (flags & MK_EP_RESIDUAL) x += to_f<DT>(ld_u16_coh(buf<const u16>(a, nd.res) + (long)gr * nd.res.ld + c));
    ep.add[e] = x;
  }
  ep.pair = !rot && ep.off[1] == ep.off[0] + 1 && (ep.off[0] & 1) == 0;
  if (rot) {
    const int hd = nd.head_dim;
    const int c = packed_col(nd, true, c0 + q);
    const float* tab = buf<float>(a, nd.aux) + (long)gr * hd;  // [cos(half) | sin(half)]
    const int i = c - (c / hd) * hd;
    ep.cs = tab[i];
    ep.sn = tab[(hd >> 1) + i];
  }
  ep.sc = 1.0f;
  if (flags & MK_EP_RMSNORM_INPUT) {
    const float s2 = sq[m] + sq[MAXR + m] + sq[2 * MAXR + m] + sq[3 * MAXR + m];
    ep.sc = 1.0f / sqrtf(s2 / (float)nd.K + nd.eps);
  }
}

template <int DT, int MAXR>
__device__ __forceinline__ void gemv_store_packed(const KArgs& a, const mk_node& nd, int flags, int r0,
                                                  int c0, int rows, int bw, int wc, const float* sum,
                                                  const float (&rinv)[MAXR], const PackedEp& ep) {
  const bool silu_mul = flags & MK_EP_SILU_MUL, rope = flags & MK_EP_ROPE;
  const int hd = nd.head_dim, hh = hd >> 1;
  const int npair = bw >> 1;
  u16* O = buf<u16>(a, nd.out);
  for (int u = tid(); u < rows * npair; u += 64) {
    const bool first = u == tid();
    float v[2], cs = 0.f, sn = 0.f;
    long off[2];
    bool rot;
    if (first) {
      // prepared during the weight stream
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float x = sum[ep.s0 + e] * ep.sc;
        if (silu_mul) x = silu(x) * (sum[ep.s0 + bw + e] * ep.sc);
        v[e] = x + ep.add[e];
        off[e] = ep.off[e];
      }
      if (ep.pair) {
        // one 4-byte store for both outputs
        float y[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) y[e] = (flags & MK_EP_RELU) ? fmaxf(v[e], 0.0f) : v[e];
        const uint32_t w2 = (uint32_t)from_f<DT>(y[0]) | ((uint32_t)from_f<DT>(y[1]) << 16);
        __hip_atomic_store(reinterpret_cast<uint32_t*>(O + off[0]), w2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        continue;
      }
      rot = ep.rot;
      cs = ep.cs;
      sn = ep.sn;
    } else {
      const int m = u / npair, q = (u - m * npair) * 2;
      const int gr = r0 + m;
      float sc = 1.0f;
#pragma unroll
      for (int mm = 0; mm < MAXR; ++mm)
        if (mm == m) sc = rinv[mm];
      rot = rope && c0 + q < nd.rope_cols;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = packed_col(nd, rot, c0 + q + e);
        off[e] = (long)gr * nd.out.ld + c;
        float x = sum[m * wc + q + e] * sc;
        if (silu_mul) x = silu(x) * (sum[m * wc + bw + q + e] * sc);
        if (flags & MK_EP_BIAS) x += to_f<DT>(ld_u16_coh(buf<const u16>(a, nd.bias) + (long)gr * nd.bias.ld + c));
        if (flags & MK_EP_RESIDUAL) x += to_f<DT>(ld_u16_coh(buf<const u16>(a, nd.res) + (long)gr * nd.res.ld + c));
        v[e] = x;
      }
      if (rot) {
        const float* tab = buf<float>(a, nd.aux) + (long)gr * hd;  // [cos(half) | sin(half)]
        const int c = packed_col(nd, true, c0 + q);
        const int i = c - (c / hd) * hd;
        cs = tab[i];
        sn = tab[hh + i];
      }
    }
    if (rot) {
      const float x1 = v[0], x2 = v[1];
      v[0] = x1 * cs - x2 * sn;
      v[1] = x2 * cs + x1 * sn;
    }
    // Agent-scope stores write through to the device-coherent level, so the
    // release needs no L2 write-back (release_gemv).
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float y = (flags & MK_EP_RELU) ? fmaxf(v[e], 0.0f) : v[e];
      __hip_atomic_store(O + off[e], from_f<DT>(y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Body after the counter wait.  In the weight waves B[k] holds (in flight)
// batch k of `in`; on return B[k] holds batch k of `nx` (or redundant
// re-reads of `in` when nx is null).  The stream of an instruction takes a
// whole number of ring turns, so every instruction starts at buffer 0 and
// all of them run one copy of this code: with the start buffer as a template
// parameter, consecutive instructions ran different copies and each paid its
// own instruction-cache misses.
template <int DT, int MAXR>
__device__ __forceinline__ void gemv_body(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem,
                                          u32x4 (&B)[kGemvBufs][kGemvBatch], const mk_instr* nx,
                                          const mk_node* nxd) {
  const int t = tid();
  const int flags = in.flags;
  const bool silu = flags & MK_EP_SILU_MUL, rms = flags & MK_EP_RMSNORM_INPUT;
  const int N = nd.N, r0 = in.r0, rows = in.r1 - in.r0, c0 = in.c0, k0 = in.k0;
  const GemvShape g = gemv_shape(in, nd);
  const int bw = g.bw, wc = g.wc, kn = g.kn;
  const int xstride = (kn + 3) & ~3;
  float* xs = reinterpret_cast<float*>(smem);   // [rows][xstride], rows * kn <= 16384 (8192 if rows > 1)
  // red holds the kpar partial sums of each output contiguously, kpad
  // apart; sum (the finished outputs) reuses the activation area, which no
  // wave reads once every wave has passed the barrier after its stream.
  const int kpad = g.kpar >= 8 ? (g.kpar + 3) & ~3 : g.kpar;
  float* red = xs + kGemvXsFloats;              // [rows][wc][kpad]
  float* sum = xs;                              // [rows][wc]
  float* sq = red + kGemvRedFloats * MAXR;      // [4 waves][MAXR] sums of squares
  {
    // All four waves stage the activation chunk (gamma-scaled under
    // RMSNORM_INPUT) with every load of a thread in flight at once (at most
    // 8: rows * kn / 8 <= 2048 chunks; a thread past the end loads nothing,
    // where clamped re-reads of the last chunk had cost about 1.5 us per
    // decode forward); each wave adds up its squares.
    const u16* A = buf<const u16>(a, nd.a) + (long)r0 * nd.a.ld + k0;
    const int kc8 = kn / 8, nch = rows * kc8;
    u32x4 xv[8], gv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t + j * kThreads;
      if (i < nch) {
        const int m = i / kc8, kc = (i - m * kc8) * 8;
        xv[j] = ld16_coh(A + (long)m * nd.a.ld + kc);
        if (rms) gv[j] = *reinterpret_cast<const u32x4*>(buf<const u16>(a, nd.gamma) + k0 + kc);
      }
    }
    float sqt[MAXR];
#pragma unroll
    for (int m = 0; m < MAXR; ++m) sqt[m] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = t + j * kThreads;
      if (i < nch) {
        const int m = i / kc8, kc = (i - m * kc8) * 8;
        float f[8];
        unpack8<DT>(xv[j], f);
        if (rms) {
          float gm[8];
          unpack8<DT>(gv[j], gm);
          float q = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            q += f[e] * f[e];
            f[e] *= gm[e];
          }
#pragma unroll
          for (int mm = 0; mm < MAXR; ++mm)
            if (mm == m) sqt[mm] += q;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[m * xstride + kc + e] = f[e];
      }
    }
    if (rms) {
#pragma unroll
      for (int m = 0; m < MAXR; ++m) {
        const float v = wave_sum(sqt[m]);
        if ((t & 63) == 0) sq[wave_id() * MAXR + m] = v;
      }
    }
  }
  lds_barrier();
  PackedEp ep;
  if (nd.layout == 1 && wave_id() == 0 && !(flags & MK_EP_PARTIAL))
    gemv_packed_prepare<DT, MAXR>(a, nd, flags, r0, c0, rows, bw, wc, sq, ep);
  if (wave_id() != 0) {
    float acc[MAXR][8];
#pragma unroll
    for (int m = 0; m < MAXR; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[m][e] = 0.f;
    // Loads target "virtual" batches: v < nb is batch v of this
    // instruction, v >= nr (nb rounded up to whole ring turns) batch v - nr
    // of the next one (clamped to its last batch); the virtual batches in
    // between, and all past nb when there is no next GEMV, re-read this
    // tile's last batch (cache hits that keep the loads per step fixed).
    const int nr = (g.nb + kGemvBufs - 1) / kGemvBufs * kGemvBufs;
    const GemvStream sc = gemv_stream(a, in, nd, g);
    const GemvStream sn = nx ? gemv_stream(a, *nx, *nxd, gemv_shape(*nx, *nxd)) : sc;
    const int nshift = nx ? nr : 0;
    const float* xk = xs + (g.active && g.kr < g.kn ? g.kr : 0);
    auto load_v = [&](int v, u32x4* dst) __attribute__((always_inline)) {
      const bool nxt = v >= nr;
      GemvStream st;
      st.p = nxt ? sn.p : sc.p;
      st.step = nxt ? sn.step : sc.step;
      st.nrows = nxt ? sn.nrows : sc.nrows;
      st.nb = nxt ? sn.nb : sc.nb;
      gemv_load(st, nxt ? v - nshift : v, dst);
    };
    // Virtual batch v lives in B[v % kGemvBufs].  Batch v is consumed (if
    // v < nb), then its buffer receives virtual batch v + kGemvBufs, so the
    // number of loads per step is fixed and each wait leaves the younger
    // batches in flight.
    for (int v0 = 0; v0 < nr; v0 += kGemvBufs) {
#pragma unroll
      for (int k = 0; k < kGemvBufs; ++k) {
        const int v = v0 + k;
        if (v < g.nb) gemv_fma_batch<DT, MAXR>(B[k], v, xk, g.kpar, sc.rv, xstride, rows, acc);
        load_v(v + kGemvBufs, B[k]);
      }
    }
    if (g.active) {
      // partial kr of output (m, cg * 8 + e); threads kr < kpad - kpar also
      // zero the padding slots kpar + kr
      float* rp = red + (g.cg * 8) * kpad + g.kr;
      const bool pad = g.kr < kpad - g.kpar;
#pragma unroll
      for (int m = 0; m < MAXR; ++m)
        if (m < rows)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            rp[(m * wc + e) * kpad] = acc[m][e];
            if (pad) rp[(m * wc + e) * kpad + g.kpar] = 0.f;
          }
    }
  }
  lds_barrier();
  {
    // All waves finish the sums: tpu consecutive lanes per output, each
    // adding 16-byte groups of its partials, then a fixed DPP pattern over
    // the tpu lanes (every run gives the same bits).
    const int nout = rows * wc;
    int tpu = 1;
    while (tpu < 16 && tpu * 2 * nout <= kThreads) tpu *= 2;
    const int sub = t & (tpu - 1);
    const bool vec = kpad != g.kpar || (g.kpar & 3) == 0;
    for (int o0 = 0; o0 < nout; o0 += kThreads / tpu) {
      const int o = o0 + t / tpu;
      float v = 0.f;
      if (o < nout) {
        if (vec) {
          const f32x4* r4 = reinterpret_cast<const f32x4*>(red + o * kpad);
          const int nq = kpad >> 2;
          f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = {0.f, 0.f, 0.f, 0.f};
          int j = sub;
          for (; j + tpu < nq; j += 2 * tpu) {
            p0 += r4[j];
            p1 += r4[j + tpu];
          }
          if (j < nq) p0 += r4[j];
          v = ((p0[0] + p1[0]) + (p0[1] + p1[1])) + ((p0[2] + p1[2]) + (p0[3] + p1[3]));
        } else {
          for (int q = sub; q < g.kpar; q += tpu) v += red[o * kpad + q];
        }
      }
      if (tpu >= 16) v += dpp_f<0x140>(v);   // row mirror
      if (tpu >= 8) v += dpp_f<0x141>(v);    // half-row mirror
      if (tpu >= 4) v += dpp_f<0x4E>(v);     // lanes ^ 2
      if (tpu >= 2) v += dpp_f<0xB1>(v);     // lanes ^ 1
      if (sub == 0 && o < nout) sum[o] = v;
    }
  }
  lds_barrier();
  if (wave_id() != 0) return;
  if (flags & MK_EP_PARTIAL) {
    float* P = buf<float>(a, nd.part) + (long)in.split_idx * nd.part_plane;
    for (int i = t; i < rows * wc; i += 64) {
      const int m = i / wc, w = i % wc;
      const int gc = (silu && w >= bw) ? N + c0 + (w - bw) : c0 + w;
      __hip_atomic_store(P + (long)(r0 + m) * nd.part.ld + gc, sum[m * wc + w], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  float rinv[MAXR];
#pragma unroll
  for (int m = 0; m < MAXR; ++m)
    rinv[m] = rms ? 1.0f / sqrtf((sq[m] + sq[MAXR + m] + sq[2 * MAXR + m] + sq[3 * MAXR + m]) / (float)nd.K + nd.eps)
                  : 1.0f;
  if (nd.layout) {
    gemv_store_packed<DT, MAXR>(a, nd, flags, r0, c0, rows, bw, wc, sum, rinv, ep);
    return;
  }
  const int units = rows * (bw / 8);
  for (int u = t; u < units; u += 64) {
    const int m = u / (bw / 8), w = (u % (bw / 8)) * 8;
    float sc = 1.0f;
#pragma unroll
    for (int mm = 0; mm < MAXR; ++mm)
      if (mm == m) sc = rinv[mm];
    epilogue8<DT, true>(a, nd, flags, r0 + m, c0 + w, w, bw, [&](int ww, float* o) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = sum[m * wc + ww + e] * sc;
    });
  }
}

template <int DT>
__device__ __forceinline__ void gemv_body_rows(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem,
                                               u32x4 (&B)[kGemvBufs][kGemvBatch], const mk_instr* nx,
                                               const mk_node* nxd) {
  if (in.r1 - in.r0 == 1) gemv_body<DT, 1>(a, in, nd, smem, B, nx, nxd);
  else gemv_body<DT, 8>(a, in, nd, smem, B, nx, nxd);
}

// ---------------------------------------------------------------- REDUCE
template <int DT, int NT = kThreads>
__device__ __forceinline__ void reduce_tile(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem) {
  const int t = tid();
  const int flags = in.flags;
  const bool silu = flags & MK_EP_SILU_MUL, rms = flags & MK_EP_RMSNORM_INPUT;
  const int N = nd.N, S = nd.split, K = nd.K;
  const int r0 = in.r0, rows = in.r1 - in.r0, c0 = in.c0, bw = in.c1 - in.c0;
  const int wc = silu ? 2 * bw : bw;     // partial columns per row (gate | up)
  const int ncg = wc / 8;
  const int units = rows * ncg;          // 8-column partial units of the tile
  float* rinv = reinterpret_cast<float*>(smem);   // [rows]
  float* scratch = rinv + 256;
  float* psum = scratch + 64;                       // [threads][8]
  float* sum = psum + NT * 8;                 // [rows][wc]
  if (rms) {
    const u16* X = buf<const u16>(a, nd.a);
    for (int m = 0; m < rows; ++m) {
      float s = 0.f;
      for (int k = t * 8; k < K; k += NT * 8) {
        float f[8];
        unpack8<DT>(*reinterpret_cast<const u32x4*>(X + (long)(r0 + m) * nd.a.ld + k), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += f[e] * f[e];
      }
      s = block_sum<NT>(s, scratch);
      if (t == 0) rinv[m] = 1.0f / sqrtf(s / (float)K + nd.eps);
    }
  }
  const float* P = buf<const float>(a, nd.part);
  const long plane = nd.part_plane, ldp = nd.part.ld;
  // Each unit's S partial planes are split over tpu threads, each summing
  // planes sub, sub + tpu, ... in order; the tpu sums are then added in
  // thread order, so the result is the same on every run.
  int tpu = 1;
  while (tpu * 2 * units <= NT && tpu * 2 <= S) tpu *= 2;
  if (tpu == 1) {
    // One thread per unit, planes in order.  A thread takes up to UB units
    // at once and loads plane p of all of them together, unconditionally
    // (a unit past the tile re-reads unit 0), so a plane costs one memory
    // round trip for UB units.
    constexpr int UB = 4;
    for (int u0 = t; u0 < units; u0 += NT * UB) {
      const float* src[UB];
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const int u = u0 + b * NT < units ? u0 + b * NT : 0;
        const int m = u / ncg, w = (u % ncg) * 8;
        const int gc = (silu && w >= bw) ? N + c0 + (w - bw) : c0 + w;
        src[b] = P + (long)(r0 + m) * ldp + gc;
      }
      float acc[UB][8];
#pragma unroll
      for (int b = 0; b < UB; ++b)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
      for (int p = 0; p < S; ++p) {
        float4 x[UB][2];
#pragma unroll
        for (int b = 0; b < UB; ++b) {
          x[b][0] = *reinterpret_cast<const float4*>(src[b] + p * plane);
          x[b][1] = *reinterpret_cast<const float4*>(src[b] + p * plane + 4);
        }
#pragma unroll
        for (int b = 0; b < UB; ++b) {
          acc[b][0] += x[b][0].x; acc[b][1] += x[b][0].y; acc[b][2] += x[b][0].z; acc[b][3] += x[b][0].w;
          acc[b][4] += x[b][1].x; acc[b][5] += x[b][1].y; acc[b][6] += x[b][1].z; acc[b][7] += x[b][1].w;
        }
      }
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const int u = u0 + b * NT;
        if (u < units) {
          const int m = u / ncg, w = (u % ncg) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[m * wc + w + e] = acc[b][e];
        }
      }
    }
    __syncthreads();
  }
  for (int u0 = 0; tpu > 1 && u0 < units; u0 += NT / tpu) {
    const int u = u0 + t / tpu, sub = t % tpu;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (u < units) {
      const int m = u / ncg, w = (u % ncg) * 8;
      const int gc = (silu && w >= bw) ? N + c0 + (w - bw) : c0 + w;
      const float* src = P + (long)(r0 + m) * ldp + gc;
      int p = sub;
      for (; p + 3 * tpu < S; p += 4 * tpu) {
        float4 x[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          x[2 * q] = *reinterpret_cast<const float4*>(src + (p + q * tpu) * plane);
          x[2 * q + 1] = *reinterpret_cast<const float4*>(src + (p + q * tpu) * plane + 4);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[0] += x[2 * q].x; acc[1] += x[2 * q].y; acc[2] += x[2 * q].z; acc[3] += x[2 * q].w;
          acc[4] += x[2 * q + 1].x; acc[5] += x[2 * q + 1].y; acc[6] += x[2 * q + 1].z; acc[7] += x[2 * q + 1].w;
        }
      }
      for (; p < S; p += tpu) {
        const float4 x0 = *reinterpret_cast<const float4*>(src + p * plane);
        const float4 x1 = *reinterpret_cast<const float4*>(src + p * plane + 4);
        acc[0] += x0.x; acc[1] += x0.y; acc[2] += x0.z; acc[3] += x0.w;
        acc[4] += x1.x; acc[5] += x1.y; acc[6] += x1.z; acc[7] += x1.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) psum[t * 8 + e] = acc[e];
    __syncthreads();
    if (sub == 0 && u < units) {
      float tot[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int q = 0; q < tpu; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) tot[e] += psum[(t + q) * 8 + e];
      const int m = u / ncg, w = (u % ncg) * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[m * wc + w + e] = tot[e];
    }
    __syncthreads();
  }
  const int ounits = rows * (bw / 8);
  for (int u = t; u < ounits; u += NT) {
    const int m = u / (bw / 8), w = (u % (bw / 8)) * 8;
    const float sc = rms ? rinv[m] : 1.0f;
    epilogue8<DT>(a, nd, flags, r0 + m, c0 + w, w, bw, [&](int ww, float* o) {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = sum[m * wc + ww + e] * sc;
    });
  }
}

// --------------------------------------------------------------- RMSNORM
// Rows [r0, r1) of y = x * rsqrt(mean(x^2) + eps) * gamma, RMAX rows of
// CPT 16-byte chunks per thread in registers: the loads of a whole group of
// rows are in flight together, each wave adds up the squares of every row,
// and one barrier exchanges the wave sums, so a group costs one memory
// round trip instead of two per row.  The loads are unconditional (a row
// past the tile re-reads its last row, a chunk past the row end its last
// chunk): a load under a branch would make the compiler wait for the one
// before it, one memory round trip per row.
template <int DT, int CPT, int NT = kThreads, int RMAX = 16 / CPT>
__device__ __forceinline__ void rmsnorm_rows(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem) {
  const int t = tid(), H = nd.N, w = wave_id();
  constexpr int NW = NT / 64;
  float* part = reinterpret_cast<float*>(smem);  // [NW waves][RMAX] sums of squares
  const u16* X = buf<const u16>(a, nd.a);
  const u16* G = buf<const u16>(a, nd.gamma);
  u16* O = buf<u16>(a, nd.out);
  u32x4 gv[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int k = min((t + c * NT) * 8, H - 8);
    gv[c] = *reinterpret_cast<const u32x4*>(G + k);
  }
  for (int g0 = in.r0; g0 < in.r1; g0 += RMAX) {
    const int nr = min(RMAX, in.r1 - g0);
    u32x4 xv[RMAX][CPT];
#pragma unroll
    for (int rr = 0; rr < RMAX; ++rr)
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int k = min((t + c * NT) * 8, H - 8);
        xv[rr][c] = *reinterpret_cast<const u32x4*>(X + (long)(g0 + min(rr, nr - 1)) * nd.a.ld + k);
      }
#pragma unroll
    for (int rr = 0; rr < RMAX; ++rr) {
      float sq = 0.f;
      if (rr < nr) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int k = (t + c * NT) * 8;
          if (k < H) {
            float f[8];
            unpack8<DT>(xv[rr][c], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) sq += f[e] * f[e];
          }
        }
      }
      sq = wave_sum(sq);
      if ((t & 63) == 0) part[w * RMAX + rr] = sq;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RMAX; ++rr) {
      if (rr >= nr) continue;
      float tot;
      if constexpr (NW == 4) {
        tot = (part[rr] + part[RMAX + rr]) + (part[2 * RMAX + rr] + part[3 * RMAX + rr]);
      } else {
        tot = part[rr];
#pragma unroll
        for (int i = 1; i < NW; ++i) tot += part[i * RMAX + rr];
      }
      const float rinv = 1.0f / sqrtf(tot / (float)H + nd.eps);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int k = (t + c * NT) * 8;
        if (k < H) {
          float f[8], gm[8];
          unpack8<DT>(xv[rr][c], f);
          unpack8<DT>(gv[c], gm);
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = f[e] * rinv * gm[e];
          *reinterpret_cast<u32x4*>(O + (long)(g0 + rr) * nd.out.ld + k) = pack8<DT>(f);
        }
      }
    }
    __syncthreads();   // part is rewritten by the next group
  }
}

template <int DT, int NT = kThreads>
__device__ __forceinline__ void rmsnorm_tile(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem) {
  const int t = tid();
  const int H = nd.N;
  const int cpt = (H / 8 + NT - 1) / NT;   // 16-byte chunks per thread and row
  // groups of up to 16 chunks per thread, halved for tiles of few rows (a
  // group's rows past the tile are loaded too)
  const bool few = in.r1 - in.r0 <= 8 / cpt;
  if (cpt <= 1) return few ? rmsnorm_rows<DT, 1, NT, 8>(a, in, nd, smem) : rmsnorm_rows<DT, 1, NT>(a, in, nd, smem);
  if (cpt <= 2) return few ? rmsnorm_rows<DT, 2, NT, 4>(a, in, nd, smem) : rmsnorm_rows<DT, 2, NT>(a, in, nd, smem);
  if (cpt <= 4) return few ? rmsnorm_rows<DT, 4, NT, 2>(a, in, nd, smem) : rmsnorm_rows<DT, 4, NT>(a, in, nd, smem);
  // wider rows: one row at a time, streamed
  float* scratch = reinterpret_cast<float*>(smem);
  const u16* X = buf<const u16>(a, nd.a);
  const u16* G = buf<const u16>(a, nd.gamma);
  u16* O = buf<u16>(a, nd.out);
  for (int r = in.r0; r < in.r1; ++r) {
    float s = 0.f;
    for (int k = t * 8; k < H; k += NT * 8) {
      float f[8];
      unpack8<DT>(*reinterpret_cast<const u32x4*>(X + (long)r * nd.a.ld + k), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += f[e] * f[e];
    }
    s = block_sum<NT>(s, scratch);
    const float rinv = 1.0f / sqrtf(s / (float)H + nd.eps);
    for (int k = t * 8; k < H; k += NT * 8) {
      float f[8], g[8];
      unpack8<DT>(*reinterpret_cast<const u32x4*>(X + (long)r * nd.a.ld + k), f);
      unpack8<DT>(*reinterpret_cast<const u32x4*>(G + k), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * rinv * g[e];
      *reinterpret_cast<u32x4*>(O + (long)r * nd.out.ld + k) = pack8<DT>(f);
    }
  }
}

// ------------------------------------------------------------- ATTENTION
// Causal grouped-query attention for query rows [r0, r1) (at most 128) of
// query head h = c0 (kv head c1), keys [0, k1).  Each wave owns 32 queries.
// S^T = K Q^T is computed so that each lane holds one query's scores, which
// then feed the P V product as the B operand straight from registers.
// With NT = 512 the two halves of the workgroup (waves 0-3 and 4-7, two
// waves per SIMD) take alternate 64-key blocks, each half with its own
// staging area and running max and sum, and merge their (o, m, l) through
// LDS at the end (the log-sum-exp merge of two key ranges).
template <int DT, int NT = kThreads>
__device__ __forceinline__ void attention_tile(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem) {
  constexpr int D = 128, KBLK = 64, NH = NT / 256;
  constexpr int KS = D + kLdsPad;      // K tile row: 136 elements
  constexpr int VS = KBLK + kLdsPad;   // V^T tile row: 72 elements
  constexpr int HALF_ELEMS = KBLK * KS + D * VS;  // a half's K / V^T staging (elements)
  static_assert(NH * HALF_ELEMS * 2 <= kSmemBytes && (4 * 64 * 64 + 2 * 4 * 64) * 4 <= kSmemBytes,
                "attention LDS");
  const int t = tid(), lane = t & 63, wave = (t >> 6) & 3, hh = t >> 8, g = lane >> 5, l32 = lane & 31;
  const int t4 = t & 255;
  u16* Ks = reinterpret_cast<u16*>(smem) + hh * HALF_ELEMS;   // [64][136]
  u16* Vt = Ks + KBLK * KS;                                    // [128][72]
  const int S = nd.seq, h = in.c0, kh = in.c1;
  const int q0 = in.r0, q1 = in.r1, kend = in.k1;
  const bool causal = nd.causal;
  const u16* Q = buf<const u16>(a, nd.a) + h * D;
  const u16* Kp = buf<const u16>(a, nd.b) + kh * D;
  const u16* Vp = buf<const u16>(a, nd.aux) + kh * D;
  const long ldq = nd.a.ld, ldk = nd.b.ld, ldv = nd.aux.ld;
  const float c = nd.scale * 1.4426950408889634f;  // scale * log2(e)

  const int qrow = q0 + wave * 32 + l32;             // this lane's query
  const int qr = min(qrow, S - 1);
  u32x4 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const u32x4*>(Q + (long)qr * ldq + s * 16 + g * 8);

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float mrun = -INFINITY, lsum = 0.f;

  // K and V rows of a key block, one block ahead: the loads of block j + 1
  // are issued once block j is in LDS, so they are in flight during block
  // j's MFMAs and softmax.  Thread: 4 K chunks (key cidx >> 4, 8 dims at
  // (cidx & 15) * 8 for cidx = t4 + 256 i) and 8 dims of 4 keys of V.
  const int dblk = t4 & 15, kq = t4 >> 4;
  u32x4 kpre[4], vpre[4];
  auto load_kv = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = t4 + 256 * i, key = cidx >> 4, dc = (cidx & 15) * 8;
      kpre[i] = *reinterpret_cast<const u32x4*>(Kp + (long)min(kb + key, S - 1) * ldk + dc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vpre[r] = *reinterpret_cast<const u32x4*>(Vp + (long)min(kb + kq * 4 + r, S - 1) * ldv + dblk * 8);
  };
  if (hh * KBLK < kend) load_kv(hh * KBLK);

  for (int kbp = 0; kbp < kend; kbp += NH * KBLK) {
    const int kb0 = kbp + hh * KBLK;   // this half's key block
    const bool live = kb0 < kend;      // uniform per wave
    __syncthreads();
    if (live) {
      // stage K [64][128] and V^T [128][64] from the registers, then
      // request the half's next block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cidx = t4 + 256 * i, key = cidx >> 4, dc = (cidx & 15) * 8;
        *reinterpret_cast<u32x4*>(Ks + key * KS + dc) = kpre[i];
      }
#pragma unroll
      for (int n = 0; n < 8; ++n)
        *reinterpret_cast<u32x2*>(Vt + (dblk * 8 + n) * VS + kq * 4) =
            u32x2{pick2(vpre[0], vpre[1], n), pick2(vpre[2], vpre[3], n)};
      if (kb0 + NH * KBLK < kend) load_kv(kb0 + NH * KBLK);
    }
    __syncthreads();
    if (live) {
      const u16* ksb = Ks;
      const u16* vtb = Vt;
      // S^T for 64 keys x 32 queries: two 32-key blocks
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(ksb + (kb * 32 + l32) * KS + s * 16 + g * 8);
          sacc[kb] = mfma32<DT>(kf, qf[s], sacc[kb]);
        }
      }
      // mask (only blocks that reach past the end or the wave's first
      // query), running max of the raw scores, then the scale folded into
      // the exponent: p = 2^(s c - m), m in scaled units (c > 0)
      const bool edge = kb0 + KBLK > kend || (causal && kb0 + KBLK - 1 > q0 + wave * 32);
      float mloc = -INFINITY;
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kb0 + kb * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
            if (key >= kend || (causal && key > qrow)) sacc[kb][e] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[kb][e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float mnew = fmaxf(mrun, mloc * c);
      const float muse = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(mrun - muse);
      mrun = mnew;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = exp2f(fmaf(sacc[kb][e], c, -muse));
          sacc[kb][e] = p;
          psum += p;
        }
      lsum = lsum * alpha + psum;
      if (__any(alpha != 1.f)) {   // the running max moved for some lane of the wave
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      }
      // O^T += V^T P^T over four 16-key substeps
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, hf = st & 1;
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sacc[kb][hf * 8 + e];
        const u32x4 pf = pack8<DT>(pv);
        const int kbase = kb * 32 + hf * 16 + 4 * g;  // keys kbase..+3 and kbase+8..+3
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const u16* vrow = vtb + (db * 32 + l32) * VS;
          const u32x2 v0 = *reinterpret_cast<const u32x2*>(vrow + kbase);
          const u32x2 v1 = *reinterpret_cast<const u32x2*>(vrow + kbase + 8);
          o[db] = mfma32<DT>(u32x4{v0.x, v0.y, v1.x, v1.y}, pf, o[db]);
        }
      }
    }
  }
  // (no K/V prefetch is left in flight: the last block issues none)
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0); expcnt, lgkmcnt not waited
  lsum += __shfl_xor(lsum, 32, 64);
  if constexpr (NH == 2) {
    // the second half hands its (o, m, l) to the first: o' = o0 2^(m0 - M)
    // + o1 2^(m1 - M), l' likewise, M = max(m0, m1)
    __syncthreads();
    float* xo = reinterpret_cast<float*>(smem);   // [4 waves][64 values][64 lanes]
    float* xm = xo + 4 * 64 * 64;                 // [4 waves][64 lanes]
    float* xl = xm + 4 * 64;
    if (hh == 1) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) xo[(wave * 64 + db * 16 + e) * 64 + lane] = o[db][e];
      xm[wave * 64 + lane] = mrun;
      xl[wave * 64 + lane] = lsum;
    }
    __syncthreads();
    if (hh == 0) {
      const float m1 = xm[wave * 64 + lane], l1 = xl[wave * 64 + lane];
      const float mm = fmaxf(mrun, m1);
      const float mu = mm == -INFINITY ? 0.f : mm;
      const float a0 = exp2f(mrun - mu), a1 = exp2f(m1 - mu);
      lsum = lsum * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[db][e] = o[db][e] * a0 + xo[(wave * 64 + db * 16 + e) * 64 + lane] * a1;
    }
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  // O^T (d rows x 32 queries per wave) -> LDS [128 q][136] -> coalesced stores
  __syncthreads();
  u16* Os = reinterpret_cast<u16*>(smem);
  if (hh == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * g;
        const uint32_t w0 = (uint32_t)from_f<DT>(o[db][4 * j] * inv) | ((uint32_t)from_f<DT>(o[db][4 * j + 1] * inv) << 16);
        const uint32_t w1 = (uint32_t)from_f<DT>(o[db][4 * j + 2] * inv) | ((uint32_t)from_f<DT>(o[db][4 * j + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(Os + (wave * 32 + l32) * KS + d) = u32x2{w0, w1};
      }
  }
  __syncthreads();
  u16* O = buf<u16>(a, nd.out) + h * D;
  for (int i = t; i < 128 * 16; i += NT) {
    const int r = i >> 4, dc = (i & 15) * 8;
    if (q0 + r >= q1) continue;
    *reinterpret_cast<u32x4*>(O + (long)(q0 + r) * nd.out.ld + dc) = *reinterpret_cast<const u32x4*>(Os + r * KS + dc);
  }
}

// ----------------------------------------------- split-KV decode attention
// Partial: keys [r0, min(r1, p + 1)) of kv head g = c0 for its G = c1 query
// heads, p the run-time position (the pos tensor, operand `part`).  Every
// K and V row of the chunk's first 128 keys is requested at once: a pass
// holds 32 keys per wave, four keys per load (16 lanes x 16 bytes cover one
// 256-byte row).  The caches and the position are caller inputs that no
// instruction of the plan writes before this one (row p is written by this
// instruction and never read back), so the persistent loop issues these
// loads before the instruction's counters clear, as it does with weights.
// Scores reduce over the 16 lanes of a row with DPP moves; V rows go to
// LDS.  Then the max per head (running maxima of the lanes, two cross-row
// shuffles, LDS across waves), exp2 weights and their sum (thread per key),
// and P V out of LDS with lanes over head dimensions, eight keys per step.
// Writes, per query head, the unnormalised output, the running max m (log2
// units) and the sum of exp2 l to P[chunk][head][d + 4].  The instruction
// whose chunk holds p rotates k_new, rounds it to the cache dtype, and
// appends it and v_new to row p of the caches; key p is scored with that
// rounded value.
constexpr int kAttnD = 128, kAttnPass = 128, kAttnGroups = 8;
struct AttnPrefetch {
  u32x4 kr[kAttnGroups], vr[kAttnGroups];   // this lane's K and V pieces of the first pass
  int p;                                     // the position
  float cs, sn;                              // cos and sin of position p, pair t % 64
};

// K and V pieces of pass ps: rows j0 + kl, kl = 128 ps + 32 w + 4 i + sub,
// for kl < nr (the chunk's rows); zero beyond.
__device__ __forceinline__ void attn_issue_kv(const KArgs& a, const mk_node& nd, int g, int j0, int nr, int ps,
                                              u32x4* kr, u32x4* vr) {
  const int lane = tid() & 63, w = wave_id();
  const int sub = lane >> 4, part = lane & 15;
  const u16* Kc = buf<const u16>(a, nd.bias) + (long)g * kAttnD + part * 8;
  const u16* Vc = buf<const u16>(a, nd.gamma) + (long)g * kAttnD + part * 8;
#pragma unroll
  for (int i = 0; i < kAttnGroups; ++i) {
    const int kl = ps * kAttnPass + w * 32 + i * 4 + sub;
    if (kl < nr) {
      kr[i] = *reinterpret_cast<const u32x4*>(Kc + (long)(j0 + kl) * nd.bias.ld);
      vr[i] = *reinterpret_cast<const u32x4*>(Vc + (long)(j0 + kl) * nd.gamma.ld);
    } else {
      kr[i] = u32x4{0u, 0u, 0u, 0u};
      vr[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void attn_partial_prefetch(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                                      AttnPrefetch& f) {
  const int j0 = uni(in.r0), S = uni(nd.seq);
  f.p = uni(*buf<const int>(a, nd.part));
  const int pc = min(max(f.p, 0), S - 1);     // the table row stays in bounds for any p
  const float* tab = buf<const float>(a, nd.aux) + (long)pc * kAttnD;   // [cos | sin] of position p
  f.cs = tab[tid() & 63];
  f.sn = tab[64 + (tid() & 63)];
  attn_issue_kv(a, nd, uni(in.c0), j0, uni(in.r1) - j0, 0, f.kr, f.vr);
}

template <int DT, int G8>
__device__ __forceinline__ void attn_partial_run(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem,
                                                 AttnPrefetch& f) {
  constexpr int D = kAttnD, HALF = 64, KPASS = kAttnPass, GR = kAttnGroups;
  static_assert((8 * D + D + 8 * 256 + 32) * 4 + 256 * D * 2 <= kSmemBytes, "decode attention LDS");
  const int t = tid(), lane = t & 63, w = wave_id();
  const int sub = lane >> 4, part = lane & 15;   // key within a group of four; dimensions 8 part .. 8 part + 7
  const int g = uni(in.c0), G = uni(in.c1), S = uni(nd.seq), Hq = uni(nd.heads);
  const int p = f.p;
  const int j0 = uni(in.r0), r1 = uni(in.r1);
  if (p < 0 || p >= S || j0 > p) return;   // empty chunk: the combine skips it
  const int j1 = min(r1, p + 1), nk = j1 - j0;
  const bool own = p < r1;                  // this chunk holds key p, at local index nk - 1
  float* qs = reinterpret_cast<float*>(smem);        // [G8][D] rotated q * scale * log2(e)
  u16* knb = reinterpret_cast<u16*>(qs + 8 * D);     // [D] rotated k_new, rounded; then [D] v_new
  u16* vnb = knb + D;
  float* sc = qs + 9 * D;                            // [G8][256] scores, then exp2 weights
  float* red = sc + 8 * 256;                         // [4 waves][8] per-wave max / sum
  u16* vs = reinterpret_cast<u16*>(red + 32);        // [256][D] V rows of the chunk
  u32x4* kr = f.kr;
  u32x4* vr = f.vr;
  const float c = nd.scale * 1.4426950408889634f;
  const float cs = f.cs, sn = f.sn;         // pair i = t % 64 (kThreads is a multiple of 64)
  {
    const u16* Q = buf<const u16>(a, nd.a) + (long)g * G * D;
    for (int u = t; u < G8 * HALF; u += kThreads) {
      const int h = u / HALF, i = u - h * HALF;
      float y1 = 0.f, y2 = 0.f;               // heads G .. G8 - 1 score zero
      if (h < G) {
        const float x1 = to_f<DT>(ld_u16_coh(Q + h * D + i)), x2 = to_f<DT>(ld_u16_coh(Q + h * D + i + HALF));
        y1 = (x1 * cs - x2 * sn) * c;
        y2 = (x2 * cs + x1 * sn) * c;
      }
      qs[h * D + i] = y1;
      qs[h * D + i + HALF] = y2;
    }
    if (own && t < HALF) {
      const u16* Kn = buf<const u16>(a, nd.b) + (long)g * D;
      const u16* Vn = buf<const u16>(a, nd.res) + (long)g * D;
      u16* Kw = buf<u16>(a, nd.bias) + (long)p * nd.bias.ld + (long)g * D;
      u16* Vw = buf<u16>(a, nd.gamma) + (long)p * nd.gamma.ld + (long)g * D;
      const float x1 = to_f<DT>(ld_u16_coh(Kn + t)), x2 = to_f<DT>(ld_u16_coh(Kn + t + HALF));
      const u16 y1 = from_f<DT>(x1 * cs - x2 * sn), y2 = from_f<DT>(x2 * cs + x1 * sn);
      store_u16_wt(Kw + t, y1);
      store_u16_wt(Kw + t + HALF, y2);
      knb[t] = y1;
      knb[t + HALF] = y2;
      const u16 v1 = ld_u16_coh(Vn + t), v2 = ld_u16_coh(Vn + t + HALF);
      store_u16_wt(Vw + t, v1);
      store_u16_wt(Vw + t + HALF, v2);
      vnb[t] = v1;
      vnb[t + HALF] = v2;
    }
  }
  __syncthreads();
  float qr[G8][8];
#pragma unroll
  for (int h = 0; h < G8; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) qr[h][e] = qs[h * D + part * 8 + e];
  // scores: the 16 lanes of a row sum their partial dot products with DPP
  // (every lane of the row ends with the key's score and writes it: same
  // address, same value).  Keys past the chunk's end score -inf and get a
  // zero V row, so the softmax and P V below run without guards.  Key p
  // takes the rotated k_new and v_new in place of the cache row loaded for
  // it before the append.
  const int npass = (nk + KPASS - 1) / KPASS, nk8 = (nk + 7) & ~7;
  const int kp = nk - 1;
  float mloc[G8];
#pragma unroll
  for (int h = 0; h < G8; ++h) mloc[h] = -INFINITY;
  for (int ps = 0; ps < npass; ++ps) {
    if (ps > 0) attn_issue_kv(a, nd, g, j0, r1 - j0, ps, kr, vr);
    if (own && kp / KPASS == ps && w == (kp % KPASS) / 32) {
      const int ip = (kp % 32) / 4;
      const bool mine = sub == kp % 4;
      const u32x4 k4 = *reinterpret_cast<const u32x4*>(knb + part * 8);
      const u32x4 v4 = *reinterpret_cast<const u32x4*>(vnb + part * 8);
#pragma unroll
      for (int i = 0; i < GR; ++i)
        if (i == ip && mine) {
          kr[i] = k4;
          vr[i] = v4;
        }
    }
#pragma unroll
    for (int i = 0; i < GR; ++i) {
      const int kl = ps * KPASS + w * 32 + i * 4 + sub;   // < 2 KPASS = 256
      const bool valid = kl < nk;
      float kf[8];
      unpack8<DT>(kr[i], kf);
#pragma unroll
      for (int h = 0; h < G8; ++h) {
        float v = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v = fmaf(qr[h][e], kf[e], v);
        v += dpp_f<0x140>(v);   // row mirror
        v += dpp_f<0x141>(v);   // half-row mirror
        v += dpp_f<0x4E>(v);    // lanes ^ 2
        v += dpp_f<0xB1>(v);    // lanes ^ 1
        v = valid ? v : -INFINITY;
        mloc[h] = fmaxf(mloc[h], v);
        sc[h * 256 + kl] = v;
      }
      const u32x4 zero{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(vs + (long)kl * D + part * 8) = valid ? vr[i] : zero;
    }
  }
  // per head: max over the chunk (rows of a wave, then the four waves),
  // then exp2 weights (zero past the chunk's keys) and their sum
  float mx[G8], ls[G8];
#pragma unroll
  for (int h = 0; h < G8; ++h) {
    float v = mloc[h];
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    v = fmaxf(v, __shfl_xor(v, 32, 64));
    if (lane == 0) red[w * 8 + h] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G8; ++h) mx[h] = fmaxf(fmaxf(red[h], red[8 + h]), fmaxf(red[16 + h], red[24 + h]));
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G8; ++h) {
    const float e = t < nk ? exp2f(sc[h * 256 + t] - mx[h]) : 0.f;
    sc[h * 256 + t] = e;
    float v = e;
    v += dpp_f<0x140>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0xB1>(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    if (lane == 0) red[w * 8 + h] = v;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < G8; ++h) ls[h] = (red[h] + red[8 + h]) + (red[16 + h] + red[24 + h]);
  // P V: item u = (head u / 64, dimensions 2 (u % 64), +1); eight keys per
  // step, every LDS read of a step issued before its multiplies
  float* P = buf<float>(a, nd.out) + (long)in.coord[0] * Hq * (D + 4);
  for (int u = t; u < G * 64; u += kThreads) {
    const int h = u >> 6, dp = u & 63;
    const float* eh = sc + h * 256;
    const u16* vcol = vs + 2 * dp;
    float o0 = 0.f, o1 = 0.f;
    for (int k = 0; k < nk8; k += 8) {
      const float4 ea = *reinterpret_cast<const float4*>(eh + k);
      const float4 eb = *reinterpret_cast<const float4*>(eh + k + 4);
      uint32_t v2[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v2[q] = *reinterpret_cast<const uint32_t*>(vcol + (long)(k + q) * D);
      const float ev[8] = {ea.x, ea.y, ea.z, ea.w, eb.x, eb.y, eb.z, eb.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        o0 = fmaf(ev[q], to_f<DT>((u16)(v2[q] & 0xffff)), o0);
        o1 = fmaf(ev[q], to_f<DT>((u16)(v2[q] >> 16)), o1);
      }
    }
    float hm = 0.f, hl = 0.f;
#pragma unroll
    for (int hh = 0; hh < G8; ++hh)
      if (hh == h) { hm = mx[hh]; hl = ls[hh]; }
    // stores through to the device-coherent level (8-byte aligned: rows
    // of D + 4 floats), so the release needs no L2 write-back
    float* dst = P + (long)(g * G + h) * (D + 4);
    store_f32x2_wt(dst + 2 * dp, o0, o1);
    if (dp == 0) store_f32x2_wt(dst + D, hm, hl);
  }
}

// Query heads per kv head: up to 4, or up to 8 (heads past G score zero).
template <int DT>
__device__ __forceinline__ void attn_partial_dispatch(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                                      char* smem, AttnPrefetch& f) {
  if (uni(in.c1) <= 4) attn_partial_run<DT, 4>(a, in, nd, smem, f);
  else attn_partial_run<DT, 8>(a, in, nd, smem, f);
}

template <int DT>
__device__ __forceinline__ void attn_partial_tile(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem) {
  AttnPrefetch f;
  attn_partial_prefetch(a, in, nd, f);
  attn_partial_dispatch<DT>(a, in, nd, smem, f);
}

// Combine: for each query head of kv head g = c0, merge the chunks c <=
// p / chunk (each holds at least key c * chunk <= p) by log-sum-exp:
// M = max m_c, o = sum 2^(m_c - M) o_c / sum 2^(m_c - M) l_c.  A thread
// holds two output elements of one head and requests the (o, m, l) of 32
// chunks at once; more chunks are merged 32 at a time with a running max.
// p is the position (a graph input, read before the counters clear).
// Outputs are stored through to the device-coherent level.
template <int DT>
__device__ __forceinline__ void attn_combine_tile(const KArgs& a, const mk_instr& in, const mk_node& nd, int p) {
  constexpr int D = 128, W = D + 4, B = 32;
  const int t = tid();
  const int g = uni(in.c0), G = uni(in.c1), S = uni(nd.seq), Hq = uni(nd.heads), C = uni(nd.K);
  u16* O = buf<u16>(a, nd.out) + (long)g * G * D;
  if (p < 0 || p >= S) {
    for (int u = t; u < G * D; u += kThreads) store_u16_wt(O + u, 0);
    return;
  }
  const int nc = p / C + 1;
  const long cst = (long)Hq * W;                                   // floats from one chunk to the next
  for (int u = t; u < G * (D / 2); u += kThreads) {
    const int h = u / (D / 2), dp = u - h * (D / 2);
    const float* ph = buf<const float>(a, nd.a) + (long)(g * G + h) * W;
    float M = -INFINITY, den = 0.f, n0 = 0.f, n1 = 0.f;
    for (int c0 = 0; c0 < nc; c0 += B) {
      float2 o[B], ml[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const long off = (long)min(c0 + q, nc - 1) * cst;         // past nc: a repeat, weighted zero
        o[q] = ld_f32x2_coh(ph + off + 2 * dp);
        ml[q] = ld_f32x2_coh(ph + off + D);
      }
      float Mb = M;
#pragma unroll
      for (int q = 0; q < B; ++q) {
        if (c0 + q >= nc) ml[q].x = -INFINITY;
        Mb = fmaxf(Mb, ml[q].x);
      }
      const float r = exp2f(M - Mb);       // 0 for the first batch
      den *= r;
      n0 *= r;
      n1 *= r;
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const float e = exp2f(ml[q].x - Mb);
        den = fmaf(e, ml[q].y, den);
        n0 = fmaf(e, o[q].x, n0);
        n1 = fmaf(e, o[q].y, n1);
      }
      M = Mb;
    }
    const float inv = 1.f / den;
    store_u32_wt(O + h * D + 2 * dp,
                 (uint32_t)from_f<DT>(n0 * inv) | ((uint32_t)from_f<DT>(n1 * inv) << 16));
  }
}

// ----------------------------------------------------------- elementwise
template <int DT, int NT = kThreads>
__device__ __forceinline__ void elementwise_tile(const KArgs& a, const mk_instr& in, const mk_node& nd) {
  const int t = tid();
  const bool add = in.opcode == MK_I_EW_ADD;
  const int wcols = in.c1 - in.c0, units = (in.r1 - in.r0) * (wcols / 8);
  const u16* A = buf<const u16>(a, nd.a);
  const u16* B = add ? buf<const u16>(a, nd.b) : nullptr;
  u16* O = buf<u16>(a, nd.out);
  for (int u = t; u < units; u += NT) {
    const int r = in.r0 + u / (wcols / 8), c = in.c0 + (u % (wcols / 8)) * 8;
    float x[8];
    unpack8<DT>(*reinterpret_cast<const u32x4*>(A + (long)r * nd.a.ld + c), x);
    if (add) {
      float y[8];
      unpack8<DT>(*reinterpret_cast<const u32x4*>(B + (long)r * nd.b.ld + c), y);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += y[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = fmaxf(x[e], 0.f);
    }
    *reinterpret_cast<u32x4*>(O + (long)r * nd.out.ld + c) = pack8<DT>(x);
  }
}

// -------------------------------------------------------------- dispatch
// A GEMM tile as a function of its own.  Inlined into the persistent loop,
// the loop's live state constrained the tile's register allocation and
// instruction schedule (more conservative LDS waits in the K loop): the
// same tile ran 8-16 % slower than in a one-tile kernel.  The pointers keep
// their address spaces (kernel arguments, LDS), so every access in the body
// stays a scalar or an LDS access.
// Op families compiled into a kernel instance.  A plan runs on the smallest
// instance whose families cover its instructions: leaving the other bodies
// out keeps their registers and code away from the loop that runs.
constexpr unsigned kOpGemm = 1, kOpGemv = 2, kOpOther = 4, kOpAll = 7;
__host__ __device__ constexpr unsigned op_family(int opcode) {
  return opcode == MK_I_NOOP ? 0u : opcode == MK_I_GEMM ? kOpGemm : opcode == MK_I_GEMV ? kOpGemv : kOpOther;
}

// NT threads per workgroup: 256 (four waves) for every instance, or 512
// (eight waves, two per SIMD) for the instances that run plans made of
// packed GEMM tiles and the REDUCE, RMSNORM, ATTENTION and elementwise
// bodies, each of which then runs on all eight waves (the GEMV bodies, the
// row-major GEMM tile and decode attention exist with four waves only).
template <unsigned OPS, int DT, int NT>
__device__ __forceinline__ void run_body(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem,
                                         bool bpre = false) {
  if (!(op_family(in.opcode) & OPS)) return;
  switch (in.opcode) {
    case MK_I_GEMM:
      // The tile bodies are inlined: a call would save and restore the
      // callee-saved registers a body uses (300-550 bytes per lane) through
      // scratch memory on every tile.
      if constexpr (!(OPS & kOpGemm)) break;
      else if constexpr (NT == 512) {
        if (nd.tile_m == 256 && nd.tile_n == 128) gemm_packed_tile<256, 128, DT, 8>(a, in, nd, smem, bpre);
        else if (nd.tile_m == 128 && nd.tile_n == 256) gemm_packed_tile<128, 256, DT, 8>(a, in, nd, smem, bpre);
        else gemm_packed_tile<128, 128, DT, 8>(a, in, nd, smem, bpre);
      } else {
        if (nd.layout == 2) {
          if (nd.tile_m == 256 && nd.tile_n == 128) gemm_packed_tile<256, 128, DT>(a, in, nd, smem, bpre);
          else if (nd.tile_m == 128 && nd.tile_n == 256) gemm_packed_tile<128, 256, DT>(a, in, nd, smem, bpre);
          else gemm_packed_tile<128, 128, DT>(a, in, nd, smem, bpre);
        } else if (nd.tile_m == 128 && nd.tile_n == 128) gemm_tile<128, 128, DT>(a, in, nd, smem);
        else if (nd.tile_m == 64 && nd.tile_n == 128) gemm_tile<64, 128, DT>(a, in, nd, smem);
        else if (nd.tile_m == 128 && nd.tile_n == 64) gemm_tile<128, 64, DT>(a, in, nd, smem);
        else gemm_tile<64, 64, DT>(a, in, nd, smem);
      }
      break;
    case MK_I_GEMV:
      if constexpr (OPS & kOpGemv) {
        u32x4 B[kGemvBufs][kGemvBatch];
        gemv_prologue(a, in, nd, B);
        gemv_body_rows<DT>(a, in, nd, smem, B, nullptr, nullptr);
      }
      break;
    default:
      if constexpr (OPS & kOpOther) {
        switch (in.opcode) {
          case MK_I_REDUCE: reduce_tile<DT, NT>(a, in, nd, smem); break;
          case MK_I_RMSNORM: rmsnorm_tile<DT, NT>(a, in, nd, smem); break;
          case MK_I_ATTENTION: attention_tile<DT, NT>(a, in, nd, smem); break;
          case MK_I_ATTN_PARTIAL:
            if constexpr (NT == kThreads) attn_partial_tile<DT>(a, in, nd, smem);
            break;
          case MK_I_ATTN_COMBINE:
            if constexpr (NT == kThreads) attn_combine_tile<DT>(a, in, nd, uni(*buf<const int>(a, nd.part)));
            break;
          case MK_I_EW_ADD:
          case MK_I_EW_RELU: elementwise_tile<DT, NT>(a, in, nd); break;
          default: break;
        }
      }
      break;
  }
}

template <unsigned OPS, int NT>
__device__ __forceinline__ void run_instr(const KArgs& a, const mk_instr& in, const mk_node& nd, char* smem,
                                          bool bpre = false) {
  if (nd.dtype == MK_BF16) run_body<OPS, MK_BF16, NT>(a, in, nd, smem, bpre);
  else run_body<OPS, MK_F16, NT>(a, in, nd, smem, bpre);
}

// Before a packed GEMM tile's counter wait: its first weight stages
// (gemm_packed_prefetch_b), in the tile shape and wave count it runs with.
template <int NT>
__device__ __forceinline__ void prefetch_gemm_weights(const KArgs& a, const mk_instr& in, const mk_node& nd,
                                                      char* smem) {
  constexpr int NW = NT / 64;
  if (nd.tile_m == 256 && nd.tile_n == 128) gemm_packed_prefetch_b<256, 128, NW>(a, in, nd, smem);
  else if (nd.tile_m == 128 && nd.tile_n == 256) gemm_packed_prefetch_b<128, 256, NW>(a, in, nd, smem);
  else gemm_packed_prefetch_b<128, 128, NW>(a, in, nd, smem);
}

// ----------------------------------------------------- counters and waits
__device__ __forceinline__ void copy_words(int* dst, const int* src) {
  if (tid() < 64) dst[tid()] = src[tid()];
}

// Arrival on the destination counters, lane k of the controller wave
// taking dst k: a sliced counter's slot dst_rank receives the epoch, others
// get an agent-scope add (the counter layout of mk.h).  Callers have made
// the instruction's results visible at agent scope first.
__device__ __forceinline__ void arrive(const KArgs& a, const mk_instr& in) {
  const int lane = tid() & 63;
  if (lane < in.n_dst) {
    int* c = a.counters + (long)in.dst_id[lane] * a.ctr_stride;
    const int rank = in.dst_rank[lane];
    if (rank >= 0) __hip_atomic_store(c + rank, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void release_dests(const KArgs& a, const mk_instr& in) {
  // every wave: its stores have completed; then one lane makes them visible
  // at agent scope and arrives on each destination counter
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (wave_id() == 0 && in.n_dst) {
    // GEMM tiles and decode attention stored through to the coherent level:
    // completion suffices
    const bool wt = in.opcode == MK_I_GEMM || in.opcode == MK_I_ATTN_PARTIAL || in.opcode == MK_I_ATTN_COMBINE;
    if (tid() == 0 && !wt) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    arrive(a, in);
  }
}

}  // namespace mkd

// One workgroup per CU; instruction `it * ncu + vcu` in iteration `it`
// (workgroup b runs column vcu = b of the placement).
// Records sit in three LDS slots and are loaded two iterations ahead, so
// iteration it always sees its own record and the next one (the two-slot
// instruction pipeline of MegaKittens Internals, section 09, one deeper);
// node descriptors are cached in LDS.
namespace mkd {

struct Loop {
  const KArgs& a;
  mk_instr* slots;      // [3]
  const mk_node* nodes;
  int* flag;
  char* smem;
  int vcu;
  int* idx;             // work-queue mode: record index of each slot, -1 = none
  int* seen;            // [kSeenSlots] counters this workgroup saw complete in this run
  int* node_tag;        // [kMaxNodes] node id held by each descriptor slot (plans of more nodes)
};

// Node descriptors.  A plan of at most kMaxNodes nodes has all of them in
// LDS (copied at launch).  A larger plan keeps a window: descriptor id in
// slot id % kMaxNodes, its id in node_tag.  A workgroup's in-flight records
// (the current one and the two fetched ahead) then need nodes that lie
// within kMaxNodes of each other, which the compiler checks for every CU
// (and it runs such plans in static placement only).
__device__ __forceinline__ const mk_node& node_of(const Loop& L, int id) { return L.nodes[id % kMaxNodes]; }

// Wave 0: make node ids lo..hi present (hi - lo < kMaxNodes).  On a miss,
// every missing id of [lo, lo + kMaxNodes) is loaded, sixteen descriptors
// per memory round trip.
__device__ __forceinline__ void ensure_nodes(const Loop& L, int lo, int hi) {
  if (L.a.n_nodes <= kMaxNodes || lo < 0) return;
  bool miss = false;
  for (int id = lo; id <= hi; ++id) miss |= L.node_tag[id % kMaxNodes] != id;
  if (!miss) return;
  const int lane = tid() & 63;
  const int end = min(lo + kMaxNodes, L.a.n_nodes);
  mk_node* slots = const_cast<mk_node*>(L.nodes);
  for (int id0 = lo; id0 < end; id0 += 16) {
    int v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int id = id0 + k;
      v[k] = id < end && L.node_tag[id % kMaxNodes] != id ? reinterpret_cast<const int*>(L.a.nodes + id)[lane] : 0;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int id = id0 + k;
      if (id < end && L.node_tag[id % kMaxNodes] != id)
        reinterpret_cast<int*>(&slots[id % kMaxNodes])[lane] = v[k];
    }
  }
  // tags after every lane's words are in place (one wave: LDS operations in order)
  for (int id = lo + lane; id < end; id += 64) L.node_tag[id % kMaxNodes] = id;
}

// Node id of a record word set (lane 2 holds `node`, lane 0 `opcode`); -1
// for a Noop.
__device__ __forceinline__ int rec_node(int w) {
  const int op = __builtin_amdgcn_readlane(w, 0), nd = __builtin_amdgcn_readlane(w, 2);
  return op == MK_I_NOOP ? -1 : nd;
}

// Record index of local iteration it (the slot it % 3 holds it), and
// whether there is one.  Static placement: column vcu of the list.  Work
// queue: the index taken from the queue for that iteration.
__device__ __forceinline__ int rec_index(const Loop& L, int it) {
  return L.a.queue ? L.idx[it % 3] : it * L.a.ncu + L.vcu;
}
__device__ __forceinline__ bool has_rec(const Loop& L, int it) {
  return L.a.queue ? L.idx[it % 3] >= 0 : it < L.a.n_iters;
}

// Work-queue mode, controller wave: the next instruction index, or -1 when
// the list is exhausted (lane 0 takes it with one agent-scope atomic add;
// every lane gets the value).  queue = 1: one queue, indices in list order
// across the grid.  queue = 2: one queue per XCD, workgroup vcu taking from
// queue q = vcu mod 8 the indices i with i mod 8 = q in list order (the
// instructions static placement gives that XCD), so a tile keeps the L2 its
// neighbours use.  Each queue has two ticket words that alternate between
// runs: run e counts on word e & 1 and clears word (e + 1) & 1, which the
// previous run (finished, by stream order) used and the next run counts on.
__device__ __forceinline__ int take_ticket(const KArgs& a, int vcu) {
  const int q = a.queue == 2 ? (vcu & 7) : 0;
  int tk = 0;
  if ((tid() & 63) == 0)
    tk = __hip_atomic_fetch_add(a.ticket + 2 * q + (a.epoch & 1), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  tk = __shfl(tk, 0, 64);
  const long idx = a.queue == 2 ? (long)tk * 8 + q : (long)tk;
  return idx < a.n_instr ? (int)idx : -1;
}

__device__ __forceinline__ void stamp(const KArgs& a, int gidx, int k, unsigned long long v) {
  a.trace[4 * (long)gidx + k] = v;
}

// Wave 0: this lane's word of record it + 2 (clamped to the last iteration so
// the load is unconditional).
__device__ __forceinline__ int fetch_ahead(const Loop& L, int it) {
  const long r = min(it + 2, L.a.n_iters - 1);
  return reinterpret_cast<const int*>(L.a.instrs + r * L.a.ncu + L.vcu)[tid() & 63];
}
// Wave 0, work-queue mode: this lane's word of record tk (0 when tk < 0).
__device__ __forceinline__ int fetch_record(const Loop& L, int tk) {
  return tk >= 0 ? reinterpret_cast<const int*>(L.a.instrs + tk)[tid() & 63] : 0;
}

// Start of iteration it.  Wave 0 issues the load of record it + 2 (used at
// the end of the iteration) while its lanes wait on the source counters,
// one counter per lane (relaxed agent-scope polls, then one acquire); all
// waves then meet at an LDS-only barrier, so the weight waves keep their
// loads in flight.
// Returns false (uniformly) if the run was aborted.
// Controller wave: wait until every source counter holds its target for
// this run.  The counters' slots are polled in groups of up to four (a
// counter above MK_SLICE_MAX is one group of one slot), each lane taking up
// to kPollGroups groups at a time, so all waits overlap.  Returns whether
// every source cleared (false: the run was aborted).  No barrier.
constexpr int kPollGroups = 2;
constexpr int kSeenSlots = 64;   // direct-mapped record of counters seen complete (by id)
constexpr int kPollNapMax = 8;   // longest pause between polls, in units of 64 cycles
// Instructions whose counter wait needs no cache invalidation:
// * bodies that read every value produced in the run through coherent loads
//   (ld16_coh and the like): packed-tile GEMVs (activation, bias, residual)
//   and decode attention (q, k_new, v_new; the partials).  Their other
//   reads are weights, graph inputs and constant tables, which no
//   instruction of the run writes (the compiler rejects a produced GEMV
//   weight and requires the KV caches and the position to be inputs);
// * row-major GEMM tiles of nodes whose produced inputs are written in
//   whole 128-byte lines that they wait on (mk_node.lines_own), when every
//   buffer is 128-byte aligned: no cache can hold such a line from before
//   its last write.
__device__ __forceinline__ bool skip_invalidate(const Loop& L, const mk_instr& in) {
  if (in.opcode == MK_I_ATTN_PARTIAL || in.opcode == MK_I_ATTN_COMBINE) return true;
  const mk_node& nd = node_of(L, in.node);
  if (in.opcode == MK_I_GEMV) return nd.layout != 0 || (in.flags & MK_EP_PARTIAL);
  return in.opcode == MK_I_GEMM && nd.lines_own && L.a.lines_ok;
}

__device__ __forceinline__ bool poll_sources(const Loop& L, const mk_instr& in, int gidx) {
  const KArgs& a = L.a;
  const int lane = tid() & 63;
  const int ns = in.n_src;
  // A counter only grows during a run, so one this workgroup has already
  // seen complete (and acquired) is not polled again: later instructions on
  // the same producers skip the memory round trip of the poll.
  unsigned todo = 0;
  for (int k = 0; k < ns; ++k)
    if (L.seen[in.src_id[k] & (kSeenSlots - 1)] != in.src_id[k]) todo |= 1u << k;
  if (!todo) return true;
  int groups = 0;
  for (int k = 0; k < ns; ++k) {
    if (!((todo >> k) & 1)) continue;
    const int T = in.src_target[k];
    groups += T <= MK_SLICE_MAX ? (T + 3) >> 2 : 1;
  }
  int ok = 1;
  for (int g0 = 0; g0 < groups; g0 += 64 * kPollGroups) {
    // this lane's groups: first slot, slot count, value needed per slot
    const int* p[kPollGroups];
    int cnt[kPollGroups], need[kPollGroups], cid[kPollGroups];
#pragma unroll
    for (int j = 0; j < kPollGroups; ++j) {
      cnt[j] = 0;
      p[j] = a.counters;
      need[j] = 0;
      cid[j] = 0;
      int g = g0 + lane + 64 * j;
      if (g >= groups) continue;
      for (int k = 0; k < ns; ++k) {
        if (!((todo >> k) & 1)) continue;
        const int T = in.src_target[k];
        const bool sl = T <= MK_SLICE_MAX;
        const int w = sl ? (T + 3) >> 2 : 1;
        if (g < w) {
          p[j] = a.counters + (long)in.src_id[k] * a.ctr_stride + (sl ? 4 * g : 0);
          cnt[j] = sl ? min(4, T - 4 * g) : 1;
          need[j] = sl ? a.epoch : a.epoch * T;
          cid[j] = in.src_id[k];
          break;
        }
        g -= w;
      }
    }
    const long long t0 = wall_clock64();
    int nap = 1;
    for (;;) {
      // the abort flag is read with the counters, in the same round trip
      // (read only after a poll that found a counter short, it doubled the
      // time each unsuccessful poll takes)
      const int abort = __hip_atomic_load(a.err + 6, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int ready = 1, seen = 0, want = 0, who = 0;
#pragma unroll
      for (int j = 0; j < kPollGroups; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < cnt[j]) {
            const int v = __hip_atomic_load(p[j] + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (v < need[j] && ready) {
              ready = 0;
              seen = v;
              want = need[j];
              who = cid[j];
            }
          }
      if (ready) break;
      if (abort) { ok = 0; break; }
      if (wall_clock64() - t0 > a.spin_ticks) {
        if (atomicCAS(a.err, 0, (int)MK_E_DEADLOCK) == 0) {
          a.err[1] = L.vcu; a.err[2] = gidx; a.err[3] = who; a.err[4] = seen; a.err[5] = want;
          if (a.abort_host) __hip_atomic_store(a.abort_host, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        __hip_atomic_store(a.err + 6, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      // back off while the wait goes on (64, 128, ... kPollNapMax x 64
      // cycles): spinning workgroups keep re-reading the same few counter
      // lines, traffic the producers they wait for would otherwise share
      for (int k = 0; k < nap; ++k) __builtin_amdgcn_s_sleep(1);
      nap = nap < kPollNapMax ? 2 * nap : kPollNapMax;
    }
    if (!__all(ok)) return false;
  }
  // The acquire's cache invalidation (about 1 us at every wait) is skipped
  // where skip_invalidate allows; those counters are then not marked seen,
  // so a later instruction of another kind polls them again and takes the
  // acquire itself.
  if (!skip_invalidate(L, in)) {
    if (lane == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (lane < ns && ((todo >> lane) & 1)) L.seen[in.src_id[lane] & (kSeenSlots - 1)] = in.src_id[lane];
  }
  return true;
}
// Work-queue mode: the ticket for iteration it + 2 is taken before the poll
// (its round trip overlaps the wait) and the record is loaded after it; tk
// carries the index to store_ahead.  Once the queue has run dry (iteration
// it + 1 got no index) no further ticket is taken.
__device__ __forceinline__ bool wait_sources(const Loop& L, const mk_instr& in, int it, int gidx, int& w,
                                             int& tk) {
  if (wave_id() == 0) {
    bool ok;
    if (L.a.queue) {
      tk = L.idx[(it + 1) % 3] >= 0 ? take_ticket(L.a, L.vcu) : -1;
      ok = poll_sources(L, in, gidx);
      w = fetch_record(L, tk);
    } else {
      if (it > 0) w = fetch_ahead(L, it);
      ok = poll_sources(L, in, gidx);
    }
    if (tid() == 0) *L.flag = ok;
  }
  lds_barrier();
  return *L.flag != 0;
}

// End of iteration it (wave 0): park record it + 2 in slot (it + 2) % 3.
// Every wave has passed this iteration's barriers, so none still reads the
// record of iteration it - 1 that the slot held; the next iteration's
// barrier publishes it.
// (records 0, 1 and 2 are copied in at the start, so iteration 0 has
// nothing to fetch or store)
// Work-queue mode: slot (it + 2) % 3 takes record tk and idx its index
// (-1 ends the loop there); records of iterations 0 and 1 are fetched at
// the start.
__device__ __forceinline__ void store_ahead(const Loop& L, int it, int w, int tk) {
  if (wave_id() != 0) return;
  if (L.a.queue) {
    if (tk >= 0) reinterpret_cast<int*>(&L.slots[(it + 2) % 3])[tid() & 63] = w;
    if (tid() == 0) L.idx[(it + 2) % 3] = tk;
  } else if (it > 0 && it + 2 < L.a.n_iters) {
    reinterpret_cast<int*>(&L.slots[(it + 2) % 3])[tid() & 63] = w;
    if (L.a.n_nodes > kMaxNodes) {
      // the window holds the nodes of records it .. it + 2 (record it may
      // still be running: the GEMV streak stores ahead before its body)
      int lo = -1, hi = -1;
      for (int k = 0; k < 3; ++k) {
        const mk_instr& c = L.slots[(it + k) % 3];
        const int nd = k == 2 ? rec_node(w) : (c.opcode == MK_I_NOOP ? -1 : c.node);
        if (nd < 0) continue;
        lo = lo < 0 ? nd : min(lo, nd);
        hi = max(hi, nd);
      }
      ensure_nodes(L, lo, hi);
    }
  }
}

// One generic iteration.  Returns false if the run was aborted.
template <unsigned OPS, int NT>
__device__ __forceinline__ bool generic_iter(const Loop& L, int it, int& w) {
  const KArgs& a = L.a;
  const int gidx = rec_index(L, it);
  const mk_instr& in = L.slots[it % 3];
  const bool tr = a.trace && tid() == 0 && in.opcode != MK_I_NOOP;
  if (tr) stamp(a, gidx, 0, wall_clock64());
  int tk = -1;
  if constexpr ((OPS & kOpOther) != 0 && NT == kThreads) {
    if (in.opcode == MK_I_ATTN_PARTIAL) {
      // The position, its rotary row and the KV cache rows are requested
      // before the counters clear, except by the controller wave: its
      // counter polls would retire behind them (the vector-memory counter
      // retires in order), and the rotary row's address waits on the
      // position.  Wave 1 hands the controller the position and the rotary
      // pair of each lane through LDS (lane i of every wave uses pair i);
      // the controller requests its KV rows after the wait, beside the q
      // loads that need a round trip then anyway.
      __shared__ float s_rot[2 * 64 + 1];
      const mk_node& nd = node_of(L, in.node);
      AttnPrefetch f;
      if (wave_id() != 0) {
        attn_partial_prefetch(a, in, nd, f);
        if (wave_id() == 1) {
          const int lane = tid() & 63;
          s_rot[lane] = f.cs;
          s_rot[64 + lane] = f.sn;
          if (lane == 0) s_rot[128] = __int_as_float(f.p);
        }
      }
      if (!wait_sources(L, in, it, gidx, w, tk)) return false;   // its barrier publishes s_rot
      if (wave_id() == 0) {
        const int lane = tid() & 63, j0 = uni(in.r0);
        f.cs = s_rot[lane];
        f.sn = s_rot[64 + lane];
        f.p = uni(__float_as_int(s_rot[128]));
        attn_issue_kv(a, nd, uni(in.c0), j0, uni(in.r1) - j0, 0, f.kr, f.vr);
      }
      if (tr) stamp(a, gidx, 1, wall_clock64());
      if (nd.dtype == MK_BF16) attn_partial_dispatch<MK_BF16>(a, in, nd, L.smem, f);
      else attn_partial_dispatch<MK_F16>(a, in, nd, L.smem, f);
      if (tr) stamp(a, gidx, 2, wall_clock64());
      release_dests(a, in);
      if (tr) stamp(a, gidx, 3, wall_clock64());
      store_ahead(L, it, w, tk);
      return true;
    }
    if (in.opcode == MK_I_ATTN_COMBINE) {
      // the position is a graph input: read before the counters clear
      const mk_node& nd = node_of(L, in.node);
      const int p = uni(*buf<const int>(a, nd.part));
      if (!wait_sources(L, in, it, gidx, w, tk)) return false;
      if (tr) stamp(a, gidx, 1, wall_clock64());
      if (nd.dtype == MK_BF16) attn_combine_tile<MK_BF16>(a, in, nd, p);
      else attn_combine_tile<MK_F16>(a, in, nd, p);
      if (tr) stamp(a, gidx, 2, wall_clock64());
      release_dests(a, in);
      if (tr) stamp(a, gidx, 3, wall_clock64());
      store_ahead(L, it, w, tk);
      return true;
    }
  }
  // A packed GEMM tile's first weight stages go out before its counters
  // clear: every body has left the LDS arena by its release barrier.  Not
  // in instances with GEMV bodies: there the controller wave may still read
  // the GEMV's sums from LDS, without a barrier, when the other waves reach
  // the next instruction.
  bool bpre = false;
  if constexpr ((OPS & kOpGemm) != 0 && (OPS & kOpGemv) == 0) {
    if (in.opcode == MK_I_GEMM) {
      const mk_node& nd = node_of(L, in.node);
      if (nd.layout == 2) {
        prefetch_gemm_weights<NT>(a, in, nd, L.smem);
        bpre = true;
      }
    }
  }
  if (!wait_sources(L, in, it, gidx, w, tk)) return false;
  if (in.opcode != MK_I_NOOP) {
    const mk_node& nd = node_of(L, in.node);
    if (tr) stamp(a, gidx, 1, wall_clock64());
    run_instr<OPS, NT>(a, in, nd, L.smem, bpre);
    if (tr) stamp(a, gidx, 2, wall_clock64());
    release_dests(a, in);
    if (tr) stamp(a, gidx, 3, wall_clock64());
  }
  store_ahead(L, it, w, tk);
  return true;
}

// Release of a GEMV instruction: only the controller wave stored results,
// all of them with stores that write through to the device-coherent level
// (agent-scope atomic stores, or store16_wt), so their completion is enough
// and the L2 write-back of an agent-scope release fence (about 1.7 us) is
// skipped.
__device__ __forceinline__ void release_gemv(const KArgs& a, const mk_instr& in, const mk_node& nd) {
  if (wave_id() != 0) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // wave 0's stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (in.n_dst) arrive(a, in);
}

// A run of GEMV instructions with the weight stream carried across them.
// Returns -1 if the run was aborted.
template <int DT>
__device__ __forceinline__ int gemv_streak(const Loop& L, int& it, int& w) {
  const KArgs& a = L.a;
  u32x4 B[kGemvBufs][kGemvBatch];
  {
    const mk_instr& in = L.slots[it % 3];
    gemv_prologue(a, in, node_of(L, in.node), B);
  }
  for (;;) {
    const int gidx = rec_index(L, it);
    const mk_instr& in = L.slots[it % 3];
    const mk_node& nd = node_of(L, in.node);
    const bool tr = a.trace && tid() == 0;
    if (tr) stamp(a, gidx, 0, wall_clock64());
    int tk = -1;
    if (!wait_sources(L, in, it, gidx, w, tk)) return -1;
    if (tr) stamp(a, gidx, 1, wall_clock64());
    // Record it + 2 goes to its slot now, while its load is surely complete:
    // after the release it would wait behind the release's own atomic (the
    // vector-memory counter retires in order).  Nothing reads that slot
    // before the next counter wait's barrier.  (In work-queue mode the
    // record load was issued after the poll, so it is parked after the body.)
    if (!a.queue) store_ahead(L, it, w, tk);
    // the next record became visible with the barrier in wait_sources
    const mk_instr* nx = nullptr;
    const mk_node* nxd = nullptr;
    if (has_rec(L, it + 1)) {
      const mk_instr& c = L.slots[(it + 1) % 3];
      if (c.opcode == MK_I_GEMV && node_of(L, c.node).dtype == nd.dtype) {
        nx = &c;
        nxd = &node_of(L, c.node);
      }
    }
    gemv_body_rows<DT>(a, in, nd, L.smem, B, nx, nxd);
    if (a.queue) store_ahead(L, it, w, tk);
    if (tr) stamp(a, gidx, 2, wall_clock64());
    release_gemv(a, in, nd);
    if (tr) stamp(a, gidx, 3, wall_clock64());
    ++it;
    if (!nx) return 0;
  }
}

}  // namespace mkd

template <unsigned OPS, int NT = 256>
__global__ void __launch_bounds__(NT, 1) mk_persistent(mkd::KArgs args) {
  // Read the arguments in place (kernarg segment, constant memory): the
  // buffer table is indexed with runtime slots, which would otherwise force
  // a private copy of the whole struct.
  const mkd::KArgs& a = *(const mkd::KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)args;
  __shared__ mk_instr s_in[3];
  __shared__ mk_node s_nodes[mkd::kMaxNodes];
  __shared__ int s_flag;
  __shared__ int s_idx[3];
  __shared__ int s_seen[mkd::kSeenSlots];
  __shared__ int s_node_tag[mkd::kMaxNodes];
  __shared__ __attribute__((aligned(16))) char smem[mkd::kSmemBytes];
  const int t = mkd::tid();
  const int b = blockIdx.x;
  if (t < mkd::kSeenSlots) s_seen[t] = -1;
  if (t < mkd::kMaxNodes) s_node_tag[t] = -1;
  // Workgroup b runs column b of the placement, so consecutive instructions
  // land on different XCDs (b % 8), as a grid launch would place them.
  // Keeping 32 consecutive instructions on one XCD instead (for L2 sharing)
  // measured 0-3 % slower on every workload.
  const int vcu = b;
  if (a.n_nodes <= mkd::kMaxNodes)
    for (int i = t; i < a.n_nodes * 64; i += NT)
      reinterpret_cast<int*>(s_nodes)[i] = reinterpret_cast<const int*>(a.nodes)[i];
  if (a.queue) {
    // clear the other ticket word for the next run; take iterations 0 and 1
    if (b == 0 && t < 8)
      __hip_atomic_store(a.ticket + 2 * t + ((a.epoch + 1) & 1), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t < 64) {
      const int t0 = mkd::take_ticket(a, vcu);
      const int t1 = t0 >= 0 ? mkd::take_ticket(a, vcu) : -1;
      if (t0 >= 0) mkd::copy_words(reinterpret_cast<int*>(&s_in[0]), reinterpret_cast<const int*>(a.instrs + t0));
      if (t1 >= 0) mkd::copy_words(reinterpret_cast<int*>(&s_in[1]), reinterpret_cast<const int*>(a.instrs + t1));
      if (t == 0) {
        s_idx[0] = t0;
        s_idx[1] = t1;
        s_idx[2] = -1;
      }
    }
  } else {
    for (int r = 0; r < 3 && r < a.n_iters; ++r)
      mkd::copy_words(reinterpret_cast<int*>(&s_in[r]), reinterpret_cast<const int*>(a.instrs + (long)r * a.ncu + vcu));
  }
  __syncthreads();
  // traced runs: the constant-rate wall clock and the shader clock at the
  // start and end of each workgroup (their ratio is the core clock)
  unsigned long long* clk = a.trace ? a.trace + 4 * ((long)a.n_iters * a.ncu + b) : nullptr;
  if (clk && t == 0) {
    clk[0] = wall_clock64();
    clk[1] = __builtin_amdgcn_s_memtime();
  }
  const mkd::Loop L{a, s_in, s_nodes, &s_flag, smem, vcu, s_idx, s_seen, s_node_tag};
  if (a.n_nodes > mkd::kMaxNodes) {
    // a windowed plan (static placement): the nodes of records 0 .. 2
    if (t < 64) {
      int lo = -1, hi = -1;
      for (int r = 0; r < 3 && r < a.n_iters; ++r) {
        if (s_in[r].opcode == MK_I_NOOP) continue;
        const int nd = s_in[r].node;
        lo = lo < 0 ? nd : min(lo, nd);
        hi = max(hi, nd);
      }
      mkd::ensure_nodes(L, lo, hi);
    }
    __syncthreads();
  }
  int it = 0, w = 0;
  while (mkd::has_rec(L, it)) {
    const mk_instr& in = s_in[it % 3];
    if constexpr ((OPS & mkd::kOpGemv) != 0) {
      if (in.opcode == MK_I_GEMV) {
        const int st = mkd::node_of(L, in.node).dtype == MK_BF16 ? mkd::gemv_streak<MK_BF16>(L, it, w)
                                                        : mkd::gemv_streak<MK_F16>(L, it, w);
        if (st < 0) return;
        continue;
      }
    }
    if (!mkd::generic_iter<OPS, NT>(L, it, w)) return;
    ++it;
  }
  if (clk && t == 0) {
    clk[2] = wall_clock64();
    clk[3] = __builtin_amdgcn_s_memtime();
  }
}

// Per-op baseline: one launch per node, one workgroup per instruction, no
// counters (stream order carries the dependencies).
template <unsigned OPS, int NT = 256>
__global__ void __launch_bounds__(NT, 1) mk_node_kernel(mkd::KArgs args) {
  const mkd::KArgs& a = *(const mkd::KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  (void)args;
  __shared__ mk_instr s_in;
  __shared__ mk_node s_nd;
  __shared__ __attribute__((aligned(16))) char smem[mkd::kSmemBytes];
  const int gidx = a.first + blockIdx.x;
  mkd::copy_words(reinterpret_cast<int*>(&s_in), reinterpret_cast<const int*>(a.instrs + gidx));
  __syncthreads();
  if (s_in.opcode == MK_I_NOOP) return;
  mkd::copy_words(reinterpret_cast<int*>(&s_nd), reinterpret_cast<const int*>(a.nodes + s_in.node));
  __syncthreads();
  mkd::run_instr<OPS, NT>(a, s_in, s_nd, smem);
}
