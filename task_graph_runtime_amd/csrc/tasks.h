// Task bodies of the decode step (HIP, gfx950).  Each body is executed by one
// whole 512-thread workgroup; the persistent mega-kernel and the
// kernel-per-operator baseline run the same functions.
//
// Operations (MPK summary page, section 3 "Target operation, shapes &
// precision contract"): projection tiles read bf16 weights and accumulate in
// fp32.  Activations passed between tasks stay fp32 (the page's bf16 task
// outputs, compounded over 28-64 layers, drift past the 2e-2 logit bound
// against the fp32 forward); only weights and the KV cache are bf16.
// Attention is paged decode attention of one new query per request against
// its KV pages.  The decoder layer around them is the Qwen3 layer (RMSNorm,
// per-head q/k RMSNorm, rotate-half RoPE, GQA, SwiGLU).
//
// Fused bodies (fewer dependency levels per layer): an attention split also
// applies q/k RMSNorm + RoPE to its heads, the last split of (b, g) appends
// the new key/value to the cache, and the last split of (b, g) to finish
// merges the splits' partials; at batch 1 a QKV / GATEUP / LM-head tile
// computes the residual add + RMSNorm of its input itself.
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <type_traits>

#include "mpk.h"
#include "rt.h"

namespace mpk {

template <typename T>
using gptr = MPK_GLOBAL T*;

// ------------------------------------------------------------------ helpers
// The calling thread's index in the workgroup, re-derived at each use.  The
// persistent kernel runs the task bodies inside its worker loop; an index
// the compiler can see is loop-invariant gets every per-thread address built
// from it hoisted out of the loop and held in registers across all tasks,
// which starves the bodies of registers and serialises their loads.
__device__ __forceinline__ int tidx() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Vector load of type T through a global pointer of element type P.
template <typename T, typename P>
__device__ __forceinline__ T ldg(MPK_GLOBAL const P* p) {
  return *reinterpret_cast<MPK_GLOBAL const T*>(p);
}

// ------------------------------------------------------------------ task-to-task data
// Activations pass between tasks, and so between compute units on different
// XCDs, whose L2 caches are not coherent with each other.  Instead of
// release/acquire fences -- a write-back or invalidation of the whole L2 of
// the XCD, which the 32 compute units of an XCD serialise on -- every access
// to task-to-task data is agent-coherent by itself (scope bit sc1): stores go
// through to the device's point of coherence, loads read it.  A producer
// waits for its stores to complete (s_waitcnt) before it advances an event
// counter, and a consumer loads the data only after it has seen the counter,
// so the data it reads is the producer's.  Weights, constant graph records
// and the KV cache written in earlier steps are read with ordinary cached
// loads.
constexpr int kCohAux = 16;   // cache-policy operand of a direct global -> LDS load: sc1
__device__ __forceinline__ void st_coh(MPK_GLOBAL float* p, float v) {
  __hip_atomic_store(reinterpret_cast<MPK_GLOBAL uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(MPK_GLOBAL const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<MPK_GLOBAL uint32_t*>(const_cast<MPK_GLOBAL float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// 16-byte buffer load at byte offset `off` of base[0, bytes) (base is
// wavefront-uniform; a load past `bytes` returns 0 and touches no memory);
// Coh: agent-coherent (sc1).
template <bool Coh>
__device__ __forceinline__ uint4 ld16(MPK_GLOBAL const void* base, int off, int bytes) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(reinterpret_cast<const void*>(base)), 0, bytes, 0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, Coh ? kCohAux : 0));
}
// Agent-coherent load of p[i..i+4) of the n-element array p.
__device__ __forceinline__ float4 ld4_coh(MPK_GLOBAL const float* base, int i, int n) {
  return __builtin_bit_cast(float4, ld16<true>(base, i * 4, n * 4));
}

// Wait until at most N vector-memory operations of this wavefront are
// outstanding (loads complete in issue order).  Through the builtin, so the
// compiler's own wait insertion sees it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes of a batch-1 tile's weight stream, loaded non-temporally: every
// weight byte is read exactly once per step, and a stream that does not
// displace other lines of the L2 leaves it to the data tasks share (the
// activation vectors every tile stages, the attention's pages).  On one
// MI355X the 8B batch-1 step went from 4.03 to 3.86 ms.  (The matrix-core
// tiles of batch > 1 read each 128-byte line of row-major weights as two
// 64-byte halves in consecutive contraction steps, so those loads keep the
// line in the L2: non-temporal loads there measured 7.68 against 7.41 ms.
// Prepared weights, whose wavefront loads are whole contiguous 1 KB blocks,
// are read non-temporally: 6.53-6.55 against 6.64-6.71 ms at 8B batch 16.)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldw(MPK_GLOBAL const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<MPK_GLOBAL const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Element i of p[0..n) or `dflt` when i >= n (n >= 1).  The load itself is
// unconditional (from a clamped index): a load under a branch makes the
// compiler wait for it before the join, serialising round trips.
template <typename T>
__device__ __forceinline__ T ld_or(MPK_GLOBAL const T* p, int64_t i, int64_t n, T dflt) {
  const T v = p[i < n ? i : n - 1];
  return i < n ? v : dflt;
}

// 8 bf16 weights (one 16-byte load) times 8 fp32 activations, fp32 accumulate.
__device__ __forceinline__ float dot8(uint4 w, float4 x0, float4 x1, float acc) {
  acc = fmaf(bflo(w.x), x0.x, acc); acc = fmaf(bfhi(w.x), x0.y, acc);
  acc = fmaf(bflo(w.y), x0.z, acc); acc = fmaf(bfhi(w.y), x0.w, acc);
  acc = fmaf(bflo(w.z), x1.x, acc); acc = fmaf(bfhi(w.z), x1.y, acc);
  acc = fmaf(bflo(w.w), x1.z, acc); acc = fmaf(bfhi(w.w), x1.w, acc);
  return acc;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over each 16-lane row (every lane of the row gets the row total):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}
// Sum over the wavefront, as a wavefront-uniform value (row sums by DPP, then
// the four row totals read out of lanes 0, 16, 32, 48).
__device__ __forceinline__ float wave_total(float v) {
  v = row_sum(v);
  const int iv = __float_as_int(v);
  return (__int_as_float(__builtin_amdgcn_readlane(iv, 0)) + __int_as_float(__builtin_amdgcn_readlane(iv, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(iv, 32)) + __int_as_float(__builtin_amdgcn_readlane(iv, 48)));
}
// Lanes MSK = 16 or 32 apart, through gfx950's row-swap permutes (VALU, not
// the LDS permute network): with both operands v, `ev` gets in every lane
// the value of the lane of its pair that lies in the even half (rows 0 and 2
// for 16, lanes 0-31 for 32) and `od` that of the odd one, so a pairwise sum
// or merge taken in (ev, od) order is bitwise the same in both lanes.
template <int MSK>
__device__ __forceinline__ void lane_pair(float v, float& ev, float& od) {
  static_assert(MSK == 16 || MSK == 32, "rows of 16 or halves of 32");
  const uint32_t u = __float_as_uint(v);
  if constexpr (MSK == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    ev = __uint_as_float(r[0]);
    od = __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    ev = __uint_as_float(r[0]);
    od = __uint_as_float(r[1]);
  }
}
template <int MSK>
__device__ __forceinline__ float pair_sum(float v) {
  float ev, od;
  lane_pair<MSK>(v, ev, od);
  return ev + od;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  v = pair_sum<16>(v);
  return pair_sum<32>(v);
}

// Workgroup barrier for LDS data only: the wavefront's LDS operations are
// complete, its vector-memory loads may stay in flight.  (__syncthreads also
// orders global memory at workgroup scope, and after direct global -> LDS
// loads the compiler makes it wait for every outstanding load, which would
// drain the weight buffers in flight.)  The empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void bar_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum over the workgroup; `red` is kWaves floats of LDS.  All threads call it.
template <bool LdsOnly = false>
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int tid0 = tidx();
  v = wave_sum(v);
  const int w = tid0 >> 6;
  if ((tid0 & 63) == 0) red[w] = v;
  if (LdsOnly) bar_lds(); else __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  if (LdsOnly) bar_lds(); else __syncthreads();
  return t;
}

// First in-kernel error wins; later ones are dropped.
__device__ __forceinline__ void report(const KArgs& a, int32_t code, int32_t task, int32_t event, uint32_t counter,
                                       uint32_t target) {
  int32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(&a.status->code, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    a.status->wg = (int32_t)blockIdx.x;
    a.status->task = task;
    a.status->event = event;
    a.status->counter = counter;
    a.status->target = target;
    __threadfence();
  }
}

// LDS of a workgroup (one per compute unit): [0, kLdsCtl) is laid out per
// graph by the host (KArgs::lds_*); the top kLdsTop bytes hold the runtime's
// control words, the trace marks and 64 words of reduction scratch.
constexpr int kLdsCtl = kLdsBytes - kLdsTop;   // runtime control words
constexpr int kLdsRed = kLdsBytes - 256;       // 64 words of reduction scratch
constexpr int kMaxSplitPages = 4096;           // page ids staged per attention split

// The workgroup's LDS, shared by the runtime loop and every task body.
__shared__ __attribute__((aligned(16))) char g_lds[kLdsBytes];

// Trace marks: when tracing, thread 0 stamps two points inside a task body
// into the control area (the worker copies them into the task's record).
constexpr int kLdsMarks = kLdsCtl + 16;
__device__ __forceinline__ void mark(const KArgs& a, int k) {
  const int tid0 = tidx();
  if (a.trace && tid0 == 0) reinterpret_cast<unsigned long long*>(g_lds + kLdsMarks)[k] = wall_clock64();
}

// ------------------------------------------------------------------ staging into LDS
// Direct global -> LDS loads: every load of a staged vector is issued back to
// back and none of the data passes through registers, so the copy costs one
// memory round trip whatever the surrounding register pressure.  Wavefront
// w copies chunks w, w + 8, ... of 64 lanes x U bytes (U = 16 or 4); units
// past n re-read the last unit into the tail of the last chunk, so dst needs
// room for n rounded up to whole chunks.  src and dst are U-byte aligned.
// The copy is complete after lds_stage_wait().
using lds_void = __attribute__((address_space(3))) void*;
// Coh: the source is task-to-task data (agent-coherent loads).
template <int U, bool Coh = false>
__device__ __forceinline__ void lds_stage(gptr<const void> src, char* dst, int n, int tid) {
  static_assert(U == 16 || U == 4, "16- or 4-byte units");
  using unit = typename std::conditional<U == 16, uint4, uint32_t>::type;
  const int w = tid >> 6, lane = tid & 63;
  gptr<const unit> su = reinterpret_cast<gptr<const unit>>(src);
  for (int c = w; c * 64 < n; c += kWaves) {
    const int u = min(c * 64 + lane, n - 1);
    __builtin_amdgcn_global_load_lds(su + u, (lds_void)(dst + c * 64 * U), U, 0, Coh ? kCohAux : 0);
  }
}
__device__ __forceinline__ void lds_stage_wait() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}
// bytes of LDS a staged copy of `bytes` occupies (whole 1 KB chunks)
__device__ __forceinline__ int lds_chunks(int bytes) { return (bytes + 1023) & ~1023; }

// ------------------------------------------------------------------ embedding
// Row b of the embedding table for request b's token (batch > 1; at batch 1
// the layer-0 QKV tiles gather it themselves).
__device__ __forceinline__ void embed_task(const KArgs& a, int b) {
  const int tid0 = tidx();
  int id = a.token_ids[b];
  if (id < 0 || id >= a.V) {
    if (tid0 == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)id, (uint32_t)a.V);
    id = 0;
  }
  gptr<const uint16_t> row = a.embed + (int64_t)id * a.H;
  for (int i = tid0; i < a.H; i += kThreads) st_coh(a.e + (int64_t)b * a.H + i, bf2f(row[i]));
}

// ------------------------------------------------------------------ residual add + RMSNorm
// Row b: res = x + y, with y the sum of ny planes [ny][B][H] (ny = 0: no y),
// stored when `res` is given; out = RMSNorm(res) * gamma.  gamma and the
// input rows are staged in LDS with direct loads.
__device__ __forceinline__ void norm_task(const KArgs& a, int b, gptr<const float> __restrict__ x,
                                          gptr<const float> __restrict__ y, int ny, gptr<float> __restrict__ res,
                                          gptr<const uint16_t> __restrict__ gamma, gptr<float> __restrict__ out,
                                          char* lds, float* red) {
  const int tid0 = tidx();
  const int H = a.H;
  const int hb = lds_chunks(H * 4), gb = lds_chunks(H * 2);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(lds);
  const float* xr = reinterpret_cast<const float*>(lds + gb);
  const int64_t off = (int64_t)b * H;
  lds_stage<16>(gamma, lds, H / 8, tid0);
  lds_stage<16, true>(x + off, lds + gb, H / 4, tid0);
  for (int p = 0; p < ny; ++p) lds_stage<16, true>(y + p * a.st_bh + off, lds + gb + hb * (1 + p), H / 4, tid0);
  lds_stage_wait();
  mark(a, 0);
  // the row in place: xr = x + sum of the planes, each element by the thread that reads it again
  float* xw = reinterpret_cast<float*>(lds + gb);
  float ss = 0.f;
  for (int i = tid0; i < H; i += kThreads) {
    float v = xr[i];
    for (int p = 0; p < ny; ++p) v += xr[i + (1 + p) * (hb / 4)];
    xw[i] = v;
    ss = fmaf(v, v, ss);
  }
  ss = block_sum(ss, red);
  mark(a, 1);
  const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
  for (int i = tid0; i < H; i += kThreads) {
    const float v = xr[i];
    if (res) st_coh(res + off + i, v);
    st_coh(out + off + i, v * inv * bf2f(gs[i]));
  }
}

// ------------------------------------------------------------------ weight pointers
// The weight base pointers of task t (see TaskPtrs), read from the per-layer
// pointer table; all loads are issued together.
__device__ __forceinline__ TaskPtrs task_ptrs(const KArgs& a, const DevTask& t) {
  TaskPtrs r{};
  gptr<const gptr<const uint16_t>> W = a.wl + (int64_t)(t.layer < 0 ? 0 : t.layer) * LAYER_PTRS;
  switch (t.type) {
    case MPK_TASK_QKV: r.p0 = W[W_Q]; r.p1 = W[W_K]; r.p2 = W[W_V]; r.p3 = W[W_IN_NORM]; break;
    case MPK_TASK_OPROJ: r.p0 = W[W_O]; break;
    case MPK_TASK_GATEUP: r.p0 = W[W_GATE]; r.p1 = W[W_UP]; r.p3 = W[W_POST_NORM]; break;
    case MPK_TASK_DOWN: r.p0 = W[W_DOWN]; break;
    case MPK_TASK_LMHEAD: r.p0 = a.lm_head ? a.lm_head : a.embed; r.p3 = a.final_norm; break;
    case MPK_TASK_ATTN_NORM: r.p0 = W[W_IN_NORM]; break;
    case MPK_TASK_MLP_NORM: r.p0 = W[W_POST_NORM]; break;
    case MPK_TASK_FINAL_NORM: r.p0 = a.final_norm; break;
    case MPK_TASK_ATTN: r.p0 = W[W_Q_NORM]; r.p1 = W[W_K_NORM]; break;
    case MPK_TASK_ROUTER: r.p0 = W[W_ROUTER]; r.p3 = W[W_POST_NORM]; break;
    case MPK_TASK_EXPERT_GU: r.p0 = W[W_GATE]; r.p1 = W[W_UP]; break;   // (expert 0: offset by the route)
    case MPK_TASK_EXPERT_DOWN: r.p0 = W[W_DOWN]; break;
    default: break;
  }
  return r;
}

// ------------------------------------------------------------------ projection tiles
// Row r of the tile's weight rows (output columns [lo, hi); gate/up tiles
// interleave gate row and up row of each column), from the task's weight
// base pointers: pure arithmetic, no memory access.
__device__ __forceinline__ gptr<const uint16_t> gemv_row(const KArgs& a, int type, const TaskPtrs& P, int lo,
                                                         int r) {
  switch (type) {
    case MPK_TASK_QKV: {
      const int col = lo + r, g = col / a.Sg, Gd = a.G * a.d;
      int off = col - g * a.Sg;
      if (off < Gd) return P.p0 + (int64_t)(g * Gd + off) * a.H;
      off -= Gd;
      if (off < a.d) return P.p1 + (int64_t)(g * a.d + off) * a.H;
      off -= a.d;
      return P.p2 + (int64_t)(g * a.d + off) * a.H;
    }
    case MPK_TASK_OPROJ:
      return P.p0 + (int64_t)(lo + r) * (a.hq * a.d);
    case MPK_TASK_GATEUP: {
      // (select between the two pointer values, not between the fields:
      // a conditional of two lvalues selects an address and keeps P in memory)
      gptr<const uint16_t> gate = P.p0, up = P.p1;
      return ((r & 1) ? up : gate) + (int64_t)(lo + (r >> 1)) * a.H;
    }
    case MPK_TASK_DOWN:
      return P.p0 + (int64_t)(lo + r) * a.F;
    case MPK_TASK_EXPERT_GU: {   // (P: the slot's expert's gate and up matrices, as for GATEUP)
      gptr<const uint16_t> gate = P.p0, up = P.p1;
      return ((r & 1) ? up : gate) + (int64_t)(lo + (r >> 1)) * a.H;
    }
    case MPK_TASK_EXPERT_DOWN:   // (P: the slot's expert's down matrix)
      return P.p0 + (int64_t)(lo + r) * a.Fe;
    default:   // LM head, router
      return P.p0 + (int64_t)(lo + r) * a.H;
  }
}

// The input of a matrix-core tile: contraction length K, weight rows per
// output column, the fp32 rows x [B][K], and which rows the tile's nx
// columns (requests) take: row j for column j, or xrow[j] (an expert
// tile's gather of its tokens' rows, LDS) when xrow is set.
struct GemvOp {
  int K, rpc;
  gptr<const float> x;
  const int* xrow;
  int nx;
};
__device__ __forceinline__ GemvOp gemv_op(const KArgs& a, const DevTask& t) {
  const int l = t.layer;
  switch (t.type) {
    case MPK_TASK_QKV: return {a.H, 1, a.h + (int64_t)l * a.st_bh, nullptr, a.B};
    case MPK_TASK_OPROJ: return {a.hq * a.d, 1, a.attn + (int64_t)l * a.st_q, nullptr, a.B};
    case MPK_TASK_GATEUP: return {a.H, 2, a.h2 + (int64_t)l * a.st_bh, nullptr, a.B};
    case MPK_TASK_DOWN: return {a.F, 1, a.a + (int64_t)l * a.st_a, nullptr, a.B};
    case MPK_TASK_ROUTER: return {a.H, 1, a.h2 + (int64_t)l * a.st_bh, nullptr, a.B};
    default: return {a.H, 1, a.hf, nullptr, a.B};
  }
}

// Position in a tile's weight rows, advanced one 1 KB segment (64 lanes x 8
// bf16) at a time without a division per segment.
struct SegWalk {
  gptr<const uint16_t> row;
  int r, ks;
};
__device__ __forceinline__ SegWalk seg_start(const KArgs& a, const DevTask& t, const TaskPtrs& P, int nseg, int s) {
  SegWalk w;
  w.r = s / nseg;
  w.ks = s - w.r * nseg;
  w.row = gemv_row(a, t.type, P, t.a0, w.r);
  return w;
}
__device__ __forceinline__ void seg_next(const KArgs& a, const DevTask& t, const TaskPtrs& P, int nseg, SegWalk& w) {
  if (++w.ks == nseg) {
    w.ks = 0;
    ++w.r;
    w.row = gemv_row(a, t.type, P, t.a0, w.r);
  }
}

__device__ __forceinline__ MoeLds* moe_lds(const KArgs& a, char* lds) {
  return reinterpret_cast<MoeLds*>(lds + a.lds_moe);
}

// k range of projection tile n under a split of its contraction into K
// ranges: n % K (the plane its partial sums go to); K = 1: 0.
__device__ __forceinline__ int ksplit_part(int K, int n) { return K == 1 ? 0 : n % K; }

// Epilogue of a projection tile from the LDS accumulators acc[row][B]; the
// q/k/v, O and down tiles write k-split plane `plane` (0 at batch 1).
__device__ __forceinline__ void gemv_epilogue(const KArgs& a, const DevTask& t, const float* acc, float* red,
                                              int plane) {
  const int tid0 = tidx();
  const int type = t.type, l = t.layer, lo = t.a0, ncol = t.a1 - t.a0, B = a.B;
  const int w = tid0 >> 6, lane = tid0 & 63;
  switch (type) {
    case MPK_TASK_QKV: {
      const int ld = a.hkv * a.Sg;
      gptr<float> out = a.qkv + (int64_t)l * a.st_qkv + (int64_t)plane * B * ld;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        st_coh(out + (int64_t)b * ld + lo + c, acc[c * B + b]);
      }
      break;
    }
    case MPK_TASK_OPROJ: {
      gptr<float> out = a.o + (int64_t)l * a.st_o + (int64_t)plane * a.st_bh;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        st_coh(out + (int64_t)b * a.H + lo + c, acc[c * B + b]);
      }
      break;
    }
    case MPK_TASK_DOWN: {
      gptr<float> out = a.dn + (int64_t)l * a.st_dn + (int64_t)plane * a.st_bh;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        st_coh(out + (int64_t)b * a.H + lo + c, acc[c * B + b]);
      }
      break;
    }
    case MPK_TASK_GATEUP: {  // SwiGLU: silu(gate) * up
      gptr<float> out = a.a + (int64_t)l * a.st_a;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        float g = acc[(2 * c) * B + b], u = acc[(2 * c + 1) * B + b];
        st_coh(out + (int64_t)b * a.F + lo + c, g / (1.0f + expf(-g)) * u);
      }
      break;
    }
    case MPK_TASK_ROUTER: {   // router logits; at batch 1 tile 0 also zeroes d_l for the down tiles to add to
      gptr<float> out = a.rlog + (int64_t)l * a.st_rlog;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        st_coh(out + (int64_t)b * a.E + lo + c, acc[c * B + b]);
      }
      if (B == 1 && t.a2 == 0) {
        gptr<float> d = a.dn + (int64_t)l * a.st_dn;
        for (int i = tid0; i < a.H; i += kThreads) st_coh(d + i, 0.f);
      }
      break;
    }
    case MPK_TASK_EXPERT_GU: {   // SwiGLU of the slot's tokens: row j of the slot holds token j (rows past them: 0)
      const MoeLds* m = moe_lds(a, g_lds);
      const int n = m->n;
      gptr<float> out = a.a + (int64_t)l * a.st_a + (int64_t)t.a2 * B * a.Fe;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int j = i / ncol, c = i - j * ncol;
        float g = acc[(2 * c) * B + j], u = acc[(2 * c + 1) * B + j];
        st_coh(out + (int64_t)j * a.Fe + lo + c, j < n ? g / (1.0f + expf(-g)) * u : 0.f);
      }
      break;
    }
    case MPK_TASK_EXPERT_DOWN: {   // each token's output, times its weight, added into d_l
      const MoeLds* m = moe_lds(a, g_lds);
      const int n = m->n;
      gptr<float> d = a.dn + (int64_t)l * a.st_dn;
      for (int i = tid0; i < ncol * n; i += kThreads) {
        int j = i / ncol, c = i - j * ncol;
        __hip_atomic_fetch_add(d + (int64_t)m->tok[j] * a.H + lo + c, m->w[j] * acc[c * B + j], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
    default: {  // LM head: fp32 logits and the tile's (max, argmax) per request
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        a.logits[(int64_t)b * a.V + lo + c] = acc[c * B + b];
      }
      int* redi = reinterpret_cast<int*>(red + kWaves);
      for (int b = 0; b < B; ++b) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int c = tid0; c < ncol; c += kThreads) {
          float v = acc[c * B + b];
          if (v > bv) { bv = v; bi = lo + c; }   // increasing c: first max kept
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          float ov = __shfl_xor(bv, m);
          int oi = __shfl_xor(bi, m);
          if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
        }
        if (lane == 0) { red[w] = bv; redi[w] = bi; }
        __syncthreads();
        if (tid0 == 0) {
          for (int i = 1; i < kWaves; ++i)
            if (red[i] > bv || (red[i] == bv && redi[i] < bi)) { bv = red[i]; bi = redi[i]; }
          __hip_atomic_store(reinterpret_cast<MPK_GLOBAL unsigned long long*>(a.pmax + b * a.T_lm + t.a2),
                             ((unsigned long long)(uint32_t)bi << 32) | __float_as_uint(bv), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
      }
      break;
    }
  }
}

// Segments of a batch-1 projection tile: its rows x ceil(K / 512) weight
// segments of 1 KB (64 lanes x 8 bf16), numbered row by row.  With pre-load
// (pre), the first P0 = min(S, 7 pf_segs) segments are the pre-loaded prefix:
// wavefront w >= 1 holds [pb, pe) = [P0 (w-1) / 7, P0 w / 7) in its LDS
// pre-load area, filled before the tile's event fired (wavefront 0 polls for
// events and pre-loads nothing: its poll would wait behind the loads).  The
// other segments [P0, S) are streamed from HBM in chunks of D segments,
// handed out dynamically (gemv_b1).
struct GemvTile {
  int K, nrows, nseg, S, P0, pb, pe;
};
__device__ __forceinline__ GemvTile gemv_tile(const KArgs& a, const DevTask& t, int w, bool pre) {
  GemvTile r;
  r.K = t.type == MPK_TASK_OPROJ ? a.hq * a.d : t.type == MPK_TASK_DOWN ? a.F : t.type == MPK_TASK_EXPERT_DOWN ? a.Fe : a.H;
  r.nrows = (t.a1 - t.a0) * ((t.type == MPK_TASK_GATEUP || t.type == MPK_TASK_EXPERT_GU) ? 2 : 1);
  r.nseg = (r.K + 511) >> 9;
  r.S = r.nrows * r.nseg;
  r.P0 = (pre && a.pf_segs > 0) ? min(r.S, kPfWaves * min(a.pf_segs, kMaxPfSegs)) : 0;
  r.pb = w ? (int)((int64_t)r.P0 * (w - 1) / kPfWaves) : 0;
  r.pe = w ? (int)((int64_t)r.P0 * w / kPfWaves) : 0;
  return r;
}
__device__ __forceinline__ char* pf_slot(const KArgs& a, char* lds, int w, int j) {
  return lds + a.lds_pf + ((w - 1) * min(a.pf_segs, kMaxPfSegs) + j) * 1024;
}
// Projection tiles whose weights are known before their event fires (so
// they can be pre-loaded); expert tiles learn their expert from the routing.
__device__ __forceinline__ bool is_gemv(int type) {
  return type == MPK_TASK_QKV || type == MPK_TASK_OPROJ || type == MPK_TASK_GATEUP || type == MPK_TASK_DOWN ||
         type == MPK_TASK_LMHEAD || type == MPK_TASK_ROUTER;
}

// Weight pre-load of a batch-1 projection tile (MPK summary section 5,
// techniques inventory: cross-task pipelining): each pre-loading wavefront
// loads its segments [pb, pe) of the tile and writes them to its LDS
// pre-load area, before the tile's event has fired (the worker calls it
// right after its previous task).  Wavefront 0 returns at once.  (Through
// registers, not direct global -> LDS loads: a direct load still counted as
// outstanding makes the compiler drain every load in flight before each
// later LDS access, which would serialise the weight streams.)
__device__ __forceinline__ void gemv_preload(const KArgs& a, const DevTask& t, const TaskPtrs& P, char* lds) {
  const int tid0 = tidx();
  const int w = tid0 >> 6, lane = tid0 & 63;
  const GemvTile r = gemv_tile(a, t, w, true);
  const int n = r.pe - r.pb;
  if (n <= 0) return;
  SegWalk sw = seg_start(a, t, P, r.nseg, r.pb);
  uint4 v[kMaxPfSegs];
#pragma unroll
  for (int j = 0; j < kMaxPfSegs; ++j) {
    const int k = min(sw.ks * 512 + lane * 8, r.K - 8);
    v[j] = ldw(sw.row + k);
    if (r.pb + j + 1 < r.pe) seg_next(a, t, P, r.nseg, sw);
  }
#pragma unroll
  for (int j = 0; j < kMaxPfSegs; ++j)
    if (j < n) *reinterpret_cast<uint4*>(pf_slot(a, lds, w, j) + lane * 16) = v[j];
}

// Input vector of a batch-1 projection tile, staged in LDS as fp32 at offset
// 0.  OPROJ and DOWN take theirs as is (attention output, SwiGLU output);
// QKV, GATEUP and the LM head apply the residual add + RMSNorm of the layer
// first:  v = E[token] (QKV of layer 0), s_{l-1} + d_{l-1} (QKV of layer l),
// r_l + o_l (GATEUP), s_{L-1} + d_{L-1} (LM head);
// x = v / sqrt(mean(v^2) + eps) * gamma.  Tile 0 of QKV / GATEUP also
// stores v: the residual r_l / s_l that later layers add to.
// xs_issue stages the inputs: the residual summands and the gain of a
// norm tile past layer 0 into registers (thread i holds elements
// [8 (i + 512 j), +8), 16-byte loads all in flight at once: direct-to-LDS
// loads keep few requests in flight per compute unit), everything else into
// LDS with direct global -> LDS loads (agent-coherent for task-to-task
// data); xs_finish, once they have landed, computes x into LDS.
struct XSrc {
  gptr<const float> v1, v2;     // fp32 summands (v2 null only with emb or without norm)
  gptr<const uint16_t> emb;     // bf16 embedding row instead of v1 (layer-0 QKV)
  gptr<float> res;              // where to store v, or null
  gptr<float> hout;             // where to store x as well, or null (router tile 0)
  bool norm;
};
__device__ __forceinline__ XSrc gemv_xsrc(const KArgs& a, const DevTask& t, const TaskPtrs& P) {
  const int l = t.layer;
  XSrc x{nullptr, nullptr, nullptr, nullptr, nullptr, true};
  switch (t.type) {
    case MPK_TASK_QKV:
      if (l == 0) {
        int id = a.token_ids[0];
        if (id < 0 || id >= a.V) {
          if (tidx() == 0) report(a, MPK_ERR_INVALID_ARG, t.id, -1, (uint32_t)id, (uint32_t)a.V);
          id = 0;
        }
        x.emb = a.embed + (int64_t)id * a.H;
      } else {
        x.v1 = a.s + (int64_t)(l - 1) * a.st_bh;
        x.v2 = a.dn + (int64_t)(l - 1) * a.st_dn;
      }
      if (t.a2 == 0) x.res = a.r + (int64_t)l * a.st_bh;
      break;
    case MPK_TASK_GATEUP:
      x.v1 = a.r + (int64_t)l * a.st_bh;
      x.v2 = a.o + (int64_t)l * a.st_o;
      if (t.a2 == 0) x.res = a.s + (int64_t)l * a.st_bh;
      break;
    case MPK_TASK_ROUTER:   // as GATEUP; tile 0 also stores h2_l, the experts' input
      x.v1 = a.r + (int64_t)l * a.st_bh;
      x.v2 = a.o + (int64_t)l * a.st_o;
      if (t.a2 == 0) {
        x.res = a.s + (int64_t)l * a.st_bh;
        x.hout = a.h2 + (int64_t)l * a.st_bh;
      }
      break;
    case MPK_TASK_EXPERT_GU:
      x.v1 = a.h2 + (int64_t)l * a.st_bh;
      x.norm = false;
      break;
    case MPK_TASK_EXPERT_DOWN:   // (row 0 of the slot: its one token at batch 1)
      x.v1 = a.a + (int64_t)l * a.st_a + (int64_t)t.a2 * a.B * a.Fe;
      x.norm = false;
      break;
    case MPK_TASK_LMHEAD:
      x.v1 = a.s + (int64_t)(a.L - 1) * a.st_bh;
      x.v2 = a.dn + (int64_t)(a.L - 1) * a.st_dn;
      break;
    case MPK_TASK_OPROJ:
      x.v1 = a.attn + (int64_t)l * a.st_q;
      x.norm = false;
      break;
    default:  // DOWN
      x.v1 = a.a + (int64_t)l * a.st_a;
      x.norm = false;
      break;
  }
  return x;
}
constexpr int kXsIt = kMaxHidden / (8 * kThreads);
struct XRegs {
  float4 v1[2 * kXsIt], v2[2 * kXsIt];
  uint4 g[kXsIt];
};
__device__ __forceinline__ void xs_issue(const KArgs& a, const XSrc& x, int K, const TaskPtrs& P, char* lds,
                                         XRegs& xr) {
  const int tid0 = tidx();
  if (!x.norm) {
    lds_stage<16, true>(x.v1, lds, K / 4, tid0);
    return;
  }
  const int H = a.H, hb = lds_chunks(H * 4);
  if (x.emb) {
    lds_stage<16>(x.emb, lds + hb, H / 8, tid0);
    lds_stage<16>(P.p3, lds + 2 * hb, H / 8, tid0);
    return;
  }
  // (past H the buffer loads return 0)
#pragma unroll
  for (int j = 0; j < kXsIt; ++j) {
    const int e = (tid0 + j * kThreads) * 8;
    xr.v1[2 * j] = ld4_coh(x.v1, e, H);
    xr.v1[2 * j + 1] = ld4_coh(x.v1, e + 4, H);
    xr.v2[2 * j] = ld4_coh(x.v2, e, H);
    xr.v2[2 * j + 1] = ld4_coh(x.v2, e + 4, H);
    xr.g[j] = ld16<false>(P.p3, e * 2, H * 2);
  }
}
__device__ __forceinline__ void xs_finish(const KArgs& a, const XSrc& x, char* lds, float* red, const XRegs& xr) {
  if (!x.norm) return;
  const int tid0 = tidx();
  const int H = a.H, hb = lds_chunks(H * 4);
  float* xs = reinterpret_cast<float*>(lds);
  if (!x.emb) {
    float v[8 * kXsIt];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 2 * kXsIt; ++j) {
      v[4 * j] = xr.v1[j].x + xr.v2[j].x;
      v[4 * j + 1] = xr.v1[j].y + xr.v2[j].y;
      v[4 * j + 2] = xr.v1[j].z + xr.v2[j].z;
      v[4 * j + 3] = xr.v1[j].w + xr.v2[j].w;
#pragma unroll
      for (int u = 0; u < 4; ++u) ss = fmaf(v[4 * j + u], v[4 * j + u], ss);
    }
    ss = block_sum<true>(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
#pragma unroll
    for (int j = 0; j < kXsIt; ++j) {
      const int e = (tid0 + j * kThreads) * 8;
      if (e < H) {
        const uint32_t gw[4] = {xr.g[j].x, xr.g[j].y, xr.g[j].z, xr.g[j].w};
        float o[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          o[2 * u] = v[8 * j + 2 * u] * inv * bflo(gw[u]);
          o[2 * u + 1] = v[8 * j + 2 * u + 1] * inv * bfhi(gw[u]);
        }
        *reinterpret_cast<float4*>(xs + e) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(xs + e + 4) = make_float4(o[4], o[5], o[6], o[7]);
        if (x.res) {
#pragma unroll
          for (int u = 0; u < 8; ++u) st_coh(x.res + e + u, v[8 * j + u]);
        }
        if (x.hout) {
#pragma unroll
          for (int u = 0; u < 8; ++u) st_coh(x.hout + e + u, o[u]);
        }
      }
    }
    bar_lds();
    return;
  }
  // layer 0: the embedding row and the gain, staged in LDS
  const uint16_t* e16 = reinterpret_cast<const uint16_t*>(lds + hb);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(lds + 2 * hb);
  constexpr int NV = kMaxHidden / kThreads;
  float v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = bf2f(e16[min(tid0 + j * kThreads, H - 1)]);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j)
    if (tid0 + j * kThreads < H) ss = fmaf(v[j], v[j], ss);
  ss = block_sum<true>(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = tid0 + j * kThreads;
    if (i < H) {
      xs[i] = v[j] * inv * bf2f(gs[i]);
      if (x.res) st_coh(x.res + i, v[j]);
    }
  }
  bar_lds();
}

// Batch-1 projection tile: y[n] = sum_k x[k] W[n, k] for the tile's columns.
// Each wavefront first consumes its pre-loaded segments (gemv_tile), then
// streams chunks of D segments through two register buffers (the loads of
// one chunk are in flight while the other is consumed).  The streamed part
// [P0, S) is cut into nch chunks: the first 8 n_st are static -- wavefront w
// takes the contiguous run [w n_st, (w+1) n_st) -- and the rest, the tail, is
// claimed chunk by chunk from an LDS counter, so that wavefronts served
// faster by the memory system take more of it and all finish together.  A
// lane takes 8 weights per segment (one 16-byte load) against x staged in LDS
// (fp32) and keeps one fp32 partial, reduced across the wavefront into the
// row's LDS accumulator when the row changes.  The staging loads of x go out
// first and the first chunk's loads right behind them, so both round trips
// overlap; the wait for x leaves that chunk in flight.  Loads past the tile's
// last segment repeat it, so the wait counts stay static.
#ifndef MPK_LA
#define MPK_LA 0   // 1: the paged lookahead's kernel (megakernel_la.hip)
#endif
#ifndef MPK_BN
#define MPK_BN 0   // 1: the batch > 1 kernels (megakernel_bn.hip)
#endif
#ifndef MPK_B1_CHUNK
#define MPK_B1_CHUNK 4
#endif
constexpr int kB1Chunk = MPK_B1_CHUNK;   // weight segments per chunk of a batch-1 tile (two chunks in flight)
template <int D>
__device__ __forceinline__ void gemv_b1(const KArgs& a, const DevTask& t, const TaskPtrs& P, char* lds, bool pre,
                                        bool xready = false) {
  const int tid0 = tidx();
  const int lane = tid0 & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);   // (wavefront-uniform: scalar control flow)
  const GemvTile r = gemv_tile(a, t, w, pre);
  const int K = r.K, nrows = r.nrows, nseg = r.nseg, S = r.S, P0 = r.P0;
  const int nch = (S - P0 + D - 1) / D;            // streamed chunks
  // static chunks per wavefront (a run of at least 2, or none)
  const int n_st = nch / kWaves - 2 >= 2 ? nch / kWaves - 2 : 0;
  const float inv_nseg = 1.0f / (float)nseg;
  float* xs = reinterpret_cast<float*>(lds);
  float* acc = reinterpret_cast<float*>(lds + a.lds_acc);
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  int* ctr = reinterpret_cast<int*>(lds + kLdsCtl) + 3;   // tail chunks claimed so far
  const int kl = lane * 8;
  const XSrc xsrc = gemv_xsrc(a, t, P);
  XRegs xr;
  if (!xready) xs_issue(a, xsrc, K, P, lds, xr);   // (xready: the caller staged x, an unnormalised row, and waited)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);   // the staging loads stay ahead of the weight loads (counted waits)
  // segment s -> (row, segment within the row) without an integer division
  auto split = [&](int s0, int& row, int& ks) {
    row = (int)(((float)s0 + 0.5f) * inv_nseg);
    ks = s0 - row * nseg;
  };
  uint4 b0[D], b1[D];
  // (a chunk past the last one re-reads the last: issues and consumes stay
  // unconditional, so the compiler can tell which buffer's loads are the
  // older ones and places exact waits)
  auto issue = [&](uint4 (&b)[D], int c) {
    const int s0 = P0 + min(c, nch - 1) * D;
    SegWalk ld;
    split(s0, ld.r, ld.ks);
    ld.row = gemv_row(a, t.type, P, t.a0, ld.r);
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int k = min(ld.ks * 512 + kl, K - 8);
      b[u] = ldw(ld.row + k);
      if (s0 + u + 1 < S) seg_next(a, t, P, nseg, ld);
    }
  };
  // fp32 partial of the current row, reduced into its accumulator on a change
  int cur = -1;
  float accv = 0.f;
  auto flush = [&]() {
    const float v = wave_total(accv);
    if (lane == 0 && cur >= 0) atomicAdd(&acc[cur], v);
    accv = 0.f;
  };
  // segment (row, ks) of weights wv; a segment past the tile (valid false)
  // adds nothing
  auto eat = [&](const uint4& wv, int row, int ks, bool valid) {
    if (valid && row != cur) {
      flush();
      cur = row;
    }
    const int k = min(ks * 512 + kl, K - 8);
    const float4* xp = reinterpret_cast<const float4*>(xs + k);
    const float d = dot8(wv, xp[0], xp[1], 0.f);
    accv += (valid && ks * 512 + kl < K) ? d : 0.f;
  };
  auto consume = [&](const uint4 (&b)[D], int c) {
    const int s0 = P0 + c * D;
    int row, ks;
    split(min(s0, S - 1), row, ks);
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const bool valid = s0 + u < S;
      eat(b[u], row, ks, valid);
      if (valid && ++ks == nseg) { ks = 0; ++row; }
    }
  };
  // the wavefront's chunk sequence: its static run, then claimed tail chunks.
  // Its first two chunks are fixed -- the start of its static run, or tail
  // chunks w and w + 8 when there is none -- so both buffers are in flight
  // before the counter is set up; claims continue after those.
  int st_i = 2;
  auto next_chunk = [&]() {
    if (st_i < n_st) return w * n_st + st_i++;
    int c = 0;
    if (lane == 0) c = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return kWaves * n_st + (n_st > 0 ? 0 : 2 * kWaves) + __builtin_amdgcn_readfirstlane(c);
  };
  int c0 = n_st > 0 ? w * n_st : w;
  int c1 = n_st > 0 ? w * n_st + 1 : w + kWaves;
  if (nch > 0) {   // behind the loads of x: the round trips overlap
    issue(b0, c0);
    issue(b1, c1);
  }
  for (int i = tid0; i < nrows; i += kThreads) acc[i] = 0.f;
  if (tid0 == 0) *ctr = 0;
  if (nch > 0) wait_vm<2 * D>();   // the staging landed; both chunks may still be in flight
  else wait_vm<0>();
  bar_lds();
  xs_finish(a, xsrc, lds, red, xr);
  if (!xready) mark(a, 0);
  if (r.pe > r.pb) {   // the pre-loaded prefix
    int row, ks;
    split(r.pb, row, ks);
    for (int j = 0; j < r.pe - r.pb; ++j) {
      eat(*reinterpret_cast<const uint4*>(pf_slot(a, lds, w, j) + lane * 16), row, ks, true);
      if (++ks == nseg) { ks = 0; ++row; }
    }
  }
  // both buffers stay in flight: consume the older chunk, then refill its
  // buffer; chunk numbers only grow, so once the older pending chunk is past
  // the end, so is the other
  if (nch > 0) {
    while (c0 < nch) {
      consume(b0, c0);
      c0 = next_chunk();
      issue(b0, c0);
      if (c1 >= nch) break;
      consume(b1, c1);
      c1 = next_chunk();
      issue(b1, c1);
    }
  }
  flush();
  mark(a, 1);
  __syncthreads();
  gemv_epilogue(a, t, acc, red, 0);
}

// ------------------------------------------------------------------ projection tile, batch 2..16 (MFMA)
// With B requests the tile is a dense contraction Y[b][n] = sum_k W[n][k]
// X[b][k] (K2 MatMul task of the MPK summary page, batch 16 sits in its
// memory-bound regime), computed with v_mfma_f32_16x16x32_bf16:
//   A = 16 weight rows x 32 k, lane l holding row l % 16 at k 8 (l / 16) .. +7
//       (one 16-byte load straight from the weight row);
//   B = X^T, lane l holding request l % 16 at the same 8 k;
//   D = 16 rows x 16 requests, lane l holding rows 4 (l / 16) + r, request l % 16.
// The fp32 activations enter as two bf16 operands, hi = bf16(x) and
// lo = bf16(x - hi); the weights are exact bf16, so every product is exact
// in fp32 and x keeps about 16 significant bits (activations between tasks
// are fp32: bf16 rounding at every task drifts past the logit bound).
// Wavefront w takes k-steps [w nks / 8, (w + 1) nks / 8) (32 k per step) of
// every 16-row block, in passes over NRB row blocks with NRB accumulators in
// registers.  A pass walks the wavefront's k range in groups of KG steps:
// the group's x slice is converted once for all NRB blocks, and while the
// group multiplies, the next group's weights (NRB x KG x 1 KB) and x are in
// flight; the last group is peeled so that every load in the loop is
// unconditional and the compiler's waits count exactly.  At the end of a
// pass the partials go to the LDS accumulators acc[row][B] (ds_add).  Rows
// past the tile and requests past B are computed on clamped rows and dropped;
// k-steps past the wavefront's range see x = 0.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// (a, b) -> packed bf16 hi = (bf16(a), bf16(b)) and lo = bf16 of the remainders.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  const float ra = a - __uint_as_float(hi << 16), rb = b - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){ra, rb}, bf16x2));
}
struct XOp {
  bf16x8 hi, lo;
};
__device__ __forceinline__ XOp x_operand(float4 x0, float4 x1) {
  uint4 h, l;
  split_bf16(x0.x, x0.y, h.x, l.x);
  split_bf16(x0.z, x0.w, h.y, l.y);
  split_bf16(x1.x, x1.y, h.z, l.z);
  split_bf16(x1.z, x1.w, h.w, l.w);
  return {__builtin_bit_cast(bf16x8, h), __builtin_bit_cast(bf16x8, l)};
}

// Prepared weights (mpk_prepare_weights): every projection matrix [N][K] is
// stored as blocks of 16 rows x 32 k, [ceil(N/16)][K/32][64 lanes][8 bf16],
// lane l of a block holding row l % 16 at k 8 (l / 16) .. +7 -- the A operand
// of v_mfma_f32_16x16x32_bf16 as this tile loads it, so a wavefront's 16-byte
// loads of one k-step cover one contiguous 1 KB instead of sixteen 64-byte
// halves of lines.  Gate and up are one matrix of 2F interleaved rows (gate
// row c at 2c, up row c at 2c + 1, the gate/up tile's row order).  The base
// of the block holding tile row r0 (a multiple of 16) of a tile whose
// columns start at lo:
__device__ __forceinline__ gptr<const uint16_t> packed_block(const KArgs& a, int type, const TaskPtrs& P, int lo,
                                                             int r0) {
  switch (type) {
    case MPK_TASK_QKV: {
      const int col = lo + r0, g = col / a.Sg, Gd = a.G * a.d, ksn = a.H >> 5;
      int off = col - g * a.Sg;
      if (off < Gd) return P.p0 + (int64_t)((g * Gd + off) >> 4) * ksn * 512;
      off -= Gd;
      if (off < a.d) return P.p1 + (int64_t)((g * a.d + off) >> 4) * ksn * 512;
      off -= a.d;
      return P.p2 + (int64_t)((g * a.d + off) >> 4) * ksn * 512;
    }
    case MPK_TASK_OPROJ:
      return P.p0 + (int64_t)((lo + r0) >> 4) * ((a.hq * a.d) >> 5) * 512;
    case MPK_TASK_GATEUP:
      return P.p0 + (int64_t)((2 * lo + r0) >> 4) * (a.H >> 5) * 512;
    case MPK_TASK_DOWN:
      return P.p0 + (int64_t)((lo + r0) >> 4) * (a.F >> 5) * 512;
    default:
      return P.p0 + (int64_t)((lo + r0) >> 4) * (a.H >> 5) * 512;
  }
}

// One pass: row blocks [rb0, min(rb0 + NRB, rb1)) over the wavefront's
// k-steps [ks0, ks1) (blocks from rb1 on belong to other wavefronts: their
// loads repeat block rb1 - 1 and their sums are dropped).
template <int NRB, int KG, bool NT = false>
__device__ __forceinline__ void mfma_pass(const KArgs& a, const DevTask& t, const TaskPtrs& P, const GemvOp& op,
                                          float* acc, int nrows, int rb0, int rb1, int ks0, int ks1
#if MPK_BN
                                          , bool own   // acc is this wavefront's own slice: store, no atomics
#endif
                                          ) {
  const int lane = tidx() & 63, li = lane & 15, lg = lane >> 4;
  const int K = op.K, B = a.B;
  const int nkg = (ks1 - ks0 + KG - 1) / KG;
  const int klast = min((ks1 - 1) * 32 + lg * 8, K - 8);   // the lane's last k in range
  // x row of the lane's request (columns past nx repeat the last one)
  const int xoff = (op.xrow ? op.xrow[min(li, op.nx - 1)] : min(li, op.nx - 1)) * K;
  // prepared weights: the lane's 16 bytes of each 1 KB block (rows past the tile read its last block)
  gptr<const uint16_t> rows[NRB];
#pragma unroll
  for (int r = 0; r < NRB; ++r)
    rows[r] = a.wpacked ? packed_block(a, t.type, P, t.a0, min(min(rb0 + r, rb1 - 1), (nrows - 1) >> 4) * 16) + lane * 8
                        : gemv_row(a, t.type, P, t.a0, min(min(rb0 + r, rb1 - 1) * 16 + li, nrows - 1));
  uint4 wv[NRB][KG];
  float4 xr[2 * KG];
  XOp xo[KG];
  f32x4 c[NRB];
#pragma unroll
  for (int r = 0; r < NRB; ++r) c[r] = (f32x4){0.f, 0.f, 0.f, 0.f};
  auto kof = [&](int kg, int j) { return min((ks0 + kg * KG + j) * 32 + lg * 8, klast); };
  // (prepared weights: k-step ks of a block is the 1 KB at ks * 512 elements)
  auto wload = [&](int kg, int r) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
#if MPK_BN
      // (NT: prepared weights, each 1 KB block read once, non-temporally)
      if constexpr (NT) wv[r][j] = ldw(rows[r] + min(ks0 + kg * KG + j, ks1 - 1) * 512);
      else
#endif
      wv[r][j] = ldg<uint4>(rows[r] + (a.wpacked ? min(ks0 + kg * KG + j, ks1 - 1) * 512 : kof(kg, j)));
    }
  };
  auto xload = [&](int kg) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      xr[2 * j] = __builtin_bit_cast(float4, ld16<false>(op.x, (xoff + kof(kg, j)) * 4, B * K * 4));
      xr[2 * j + 1] = __builtin_bit_cast(float4, ld16<false>(op.x, (xoff + kof(kg, j) + 4) * 4, B * K * 4));
    }
  };
  auto xconvert = [&](int kg) {
    const float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const bool in = ks0 + kg * KG + j < ks1;
      xo[j] = x_operand(in ? xr[2 * j] : z, in ? xr[2 * j + 1] : z);
    }
  };
  auto mul = [&](int r) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const bf16x8 w = __builtin_bit_cast(bf16x8, wv[r][j]);
      c[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xo[j].hi, c[r], 0, 0, 0);
      c[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, xo[j].lo, c[r], 0, 0, 0);
    }
  };
  xload(0);
#pragma unroll
  for (int r = 0; r < NRB; ++r) wload(0, r);
  for (int kg = 0; kg + 1 < nkg; ++kg) {
    xconvert(kg);
    xload(kg + 1);
    // (block by block: the next group's weights of block r go out as soon as
    // block r's products are issued, so they are in flight during the other
    // blocks' products; the compiler would otherwise sink every load below
    // the last product and expose a full round trip per group)
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      mul(r);
      wload(kg + 1, r);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  xconvert(nkg - 1);
#pragma unroll
  for (int r = 0; r < NRB; ++r) mul(r);
#pragma unroll
  for (int r = 0; r < NRB; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (rb0 + r) * 16 + lg * 4 + i;
#if MPK_BN
      if (li < B && row < nrows && rb0 + r < rb1) {
        if (own) acc[row * B + li] = c[r][i];
        else atomicAdd(&acc[row * B + li], c[r][i]);
      }
#else
      if (li < B && row < nrows && rb0 + r < rb1) atomicAdd(&acc[row * B + li], c[r][i]);
#endif
    }
}

#if MPK_BN
template <int NRB, int KG>
__device__ __forceinline__ void mfma_passes(const KArgs& a, const DevTask& t, const TaskPtrs& P, const GemvOp& op,
                                            float* acc, int nrows, int rb_lo, int rb_hi, int ks0, int ks1, bool own) {
  if (a.wpacked) {
    for (int rb0 = rb_lo; rb0 < rb_hi; rb0 += NRB)
      mfma_pass<NRB, KG, true>(a, t, P, op, acc, nrows, rb0, rb_hi, ks0, ks1, own);
  } else {
    for (int rb0 = rb_lo; rb0 < rb_hi; rb0 += NRB)
      mfma_pass<NRB, KG>(a, t, P, op, acc, nrows, rb0, rb_hi, ks0, ks1, own);
  }
}
#else
template <int NRB, int KG>
__device__ __forceinline__ void mfma_passes(const KArgs& a, const DevTask& t, const TaskPtrs& P, const GemvOp& op,
                                            float* acc, int nrows, int rb_lo, int rb_hi, int ks0, int ks1) {
  for (int rb0 = rb_lo; rb0 < rb_hi; rb0 += NRB) mfma_pass<NRB, KG>(a, t, P, op, acc, nrows, rb0, rb_hi, ks0, ks1);
}
#endif

__device__ __forceinline__ void gemv_mfma(const KArgs& a, const DevTask& t, const TaskPtrs& P, char* lds,
                                          const GemvOp& op) {
  const int tid0 = tidx();
  const int K = op.K, nrows = (t.a1 - t.a0) * op.rpc, B = a.B;
  float* acc = reinterpret_cast<float*>(lds + a.lds_acc);
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  for (int i = tid0; i < nrows * B; i += kThreads) acc[i] = 0.f;
  __syncthreads();
  const int w = tid0 >> 6;
  const int nrb = (nrows + 15) >> 4;
  // the tile's k range (a split of the contraction into ks ranges, on a
  // quantum of one 32-k step) and the wavefront's share of it
  const int ks = t.type == MPK_TASK_QKV ? a.Kq : t.type == MPK_TASK_OPROJ ? a.Ko : t.type == MPK_TASK_DOWN ? a.Kd : 1;
  const int U = (K + 31) >> 5, kr = ksplit_part(ks, t.a2);
  const int kb = kr * U / ks, nks = (kr + 1) * U / ks - kb;
  // A contraction of fewer than 8 k-steps per wavefront (an expert's down
  // projection, K = 768: 3) leaves each wavefront too short a stream per row
  // block; with enough row blocks the wavefronts split the rows instead and
  // each walks the whole k range.
  const bool by_rows = nks < 8 * kWaves && nrb >= kWaves;
  const int ks0 = by_rows ? kb : kb + nks * w / kWaves, ks1 = by_rows ? kb + nks : kb + nks * (w + 1) / kWaves;
  const int rb_lo = by_rows ? nrb * w / kWaves : 0, rb_hi = by_rows ? nrb * (w + 1) / kWaves : nrb;
  const int nb = rb_hi - rb_lo;
  // The input rows are task-to-task data, read here with ordinary (L2-
  // cached) loads rather than agent-coherent ones, so that the tiles on one
  // XCD share one fetch per line instead of one each.  No L2 can hold a
  // stale copy: each input is written once per step, by agent-coherent
  // stores that are complete before this tile's event fires, and nothing
  // reads it earlier in the step, so no L2 fetched it before the event
  // (copies from earlier steps are gone: a kernel launch starts with no
  // stale cached lines, as stream order across launches requires).  A line
  // that gate/up tiles on two XCDs share (the down projection's input) holds
  // in the writer's L2 only the bytes that XCD wrote -- a write does not
  // fill the line -- so the read fetches the line, whose other bytes the
  // other tile's write-through stores have reached.
#if MPK_BN
  // (the wavefronts' partial sums: when the wavefronts split the
  // contraction and their slices fit in the staging area, which a
  // matrix-core tile does not use, each wavefront stores its own slice and
  // they are summed below in wavefront order; else they are added into acc
  // with LDS atomics.  Eight atomics on every accumulator, one per
  // wavefront, cost a tile alone 4-10 us.)
  const bool own = !by_rows && kWaves * nrows * B * 4 <= a.lds_acc;
  float* part = reinterpret_cast<float*>(lds);
  float* dst = own ? part + (int64_t)w * nrows * B : acc;
  if (ks1 > ks0 && nb > 0) {
    // weights in flight per wavefront: NRB x KG KB
    if (nb <= 2) mfma_passes<2, 4>(a, t, P, op, dst, nrows, rb_lo, rb_hi, ks0, ks1, own);
    else if (nb <= 4) mfma_passes<4, 4>(a, t, P, op, dst, nrows, rb_lo, rb_hi, ks0, ks1, own);
    else mfma_passes<8, 2>(a, t, P, op, dst, nrows, rb_lo, rb_hi, ks0, ks1, own);
  }
  __syncthreads();
  if (own) {   // (a wavefront with an empty k range stored nothing)
    for (int i = tid0; i < nrows * B; i += kThreads) {
      float v = 0.f;
      for (int u = 0; u < kWaves; ++u)
        if (nks * (u + 1) / kWaves > nks * u / kWaves) v += part[(int64_t)u * nrows * B + i];
      acc[i] = v;
    }
    __syncthreads();
  }
#else
  if (ks1 > ks0 && nb > 0) {
    // weights in flight per wavefront: NRB x KG KB
    if (nb <= 2) mfma_passes<2, 4>(a, t, P, op, acc, nrows, rb_lo, rb_hi, ks0, ks1);
    else if (nb <= 4) mfma_passes<4, 4>(a, t, P, op, acc, nrows, rb_lo, rb_hi, ks0, ks1);
    else mfma_passes<8, 2>(a, t, P, op, acc, nrows, rb_lo, rb_hi, ks0, ks1);
  }
  __syncthreads();
#endif
  mark(a, 1);
  gemv_epilogue(a, t, acc, red, kr);
}

// ------------------------------------------------------------------ paged attention, one split
// Attention slots.  Kv group g has M = S_attn attention tasks; task (j, g)
// is slot j (M >= B).  When the step runs, request b gets
// n_b = max(1, ceil(pages_b / T)) consecutive slots, in request order, with
// T the smallest split size (in pages) for which sum_b n_b <= M
// (pages_b = ceil((L_b + 1) / P); a request with an invalid length counts 0
// pages); slots past the last request's are idle.  T is at least Tmin =
// attn_min_pages: a split shorter than that costs more in its fixed latency
// (q/k/v row, norm and rotation, partial record, merge) than it saves in key
// and value streaming.  At batch 1 that makes the request's split count
// n = min(M, max(1, ceil(pages / Tmin))), so the split count follows the
// cached length at run time (a graph is built for the longest).  Every task
// computes the same allocation from the B sequence lengths, so no split is
// longer than T pages however the lengths differ.
struct AttnSlot {
  int b, s, n, start;   // request (-1: idle slot), its split, its split count, its first slot
};
__device__ __forceinline__ int attn_pages(const KArgs& a, int L) {
  return (L >= 0 && L < a.max_seq && L / a.P < a.max_pages) ? (L + a.P) / a.P : 0;
}
// (one request per lane of the first 16: one vector load of the lengths, a
// butterfly sum, a scan of the split counts and a ballot; the result is
// wavefront-uniform)
// one: batch 1, return {0, j, 0, 0} without loading anything (the caller
// sizes the splits once it has read the length).
__device__ __forceinline__ AttnSlot attn_slot(const KArgs& a, int j, bool one) {
  const int lane = tidx() & 63, B = a.B, M = a.S_attn;
  if (one) return AttnSlot{0, j, 0, 0};
  const int L = a.seq_lens[min(lane, B - 1)];
  const int pg = lane < B ? attn_pages(a, L) : 0;
  // T: binary search over [1, max pages] (T = max pages always fits: B <= M)
  int mx = pg;
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) mx = max(mx, __shfl_xor(mx, m, 16));
  auto splits = [&](int T) {   // sum_b max(1, ceil(pages_b / T)), wavefront-uniform (lanes 0..15)
    int c = lane < B ? max(1, (pg + T - 1) / T) : 0;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) c += __shfl_xor(c, m, 16);
    return __builtin_amdgcn_readfirstlane(c);
  };
  int lo = a.attn_min_pages, hi = max(__builtin_amdgcn_readfirstlane(mx), lo);
  while (lo < hi) {
    const int mid = (lo + hi) / 2;
    if (splits(mid) <= M) hi = mid;
    else lo = mid + 1;
  }
  const int n = lane < B ? max(1, (pg + lo - 1) / lo) : 0;
  int incl = n;
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    const int v = __shfl_up(incl, d, 16);
    if ((lane & 15) >= d) incl += v;
  }
  const int start = incl - n;
  const unsigned long long mine = __ballot(lane < B && j >= start && j < incl);
  if (mine == 0ull) return AttnSlot{-1, 0, 0, 0};
  const int src = __ffsll((long long)mine) - 1;
  const int st = __builtin_amdgcn_readfirstlane(__shfl(start, src));
  return AttnSlot{src, j - st, __builtin_amdgcn_readfirstlane(__shfl(n, src)), st};
}

// The most splits of one request whose partial records the combine stages
// in LDS (staging area [0, lds_acc), records padded as attn_combine does).
__device__ __forceinline__ int attn_stage_cap(const KArgs& a) {
  return max(1, (a.lds_acc / 4 - 63) / (a.G * (a.d + 2)));
}

// Merge of the n partial records (m, l, o[D]) of a request, in slots
// [start, start + n) of kv group g, into its attention output (row b):
// o = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}, M = max_s m_s (empty
// splits carry m = -inf, l = 0).  Run by the split that finishes last.  The
// records are staged in LDS first when they fit.
__device__ __forceinline__ void attn_combine(const KArgs& a, int l, int b, int g, int start, int n_split,
                                             char* lds) {
  const int tid0 = tidx();
  const int G = a.G, D = a.d, S = n_split;
  const int rec = G * (D + 2);
  gptr<const float> part =
      a.part + (int64_t)l * a.st_part + ((int64_t)g * a.S_attn + start) * (int64_t)rec;
  gptr<float> out = a.attn + (int64_t)l * a.st_q + (int64_t)b * a.hq * D + (int64_t)g * G * D;
  float* st = reinterpret_cast<float*>(lds);
  const int n = S * rec;   // (a multiple of 4: rec = G (D + 2) with D even)
  const bool staged = ((n + 63) & ~63) * 4 <= a.lds_acc;
  if (staged) {   // staged through registers: up to 16K floats in flight at once
    for (int i0 = 0; i0 < n; i0 += 8 * kThreads * 4) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld4_coh(part, i0 + (tid0 + u * kThreads) * 4, n);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + (tid0 + u * kThreads) * 4;
        if (i < n) *reinterpret_cast<float4*>(st + i) = v[u];
      }
    }
    __syncthreads();
  }
  // (the splits in groups of four whose loads go out together, one wait per
  // group instead of one per split; the sums still run in split order)
  auto merge = [&](auto at) {
    for (int e = tid0; e < G * D; e += kThreads) {
      const int h = e / D, dd = e - h * D, hb = h * (D + 2);
      float M = -INFINITY;
      for (int s0 = 0; s0 < S; s0 += 8) {
        float mm[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) mm[u] = at(min(s0 + u, S - 1) * rec + hb);
#pragma unroll
        for (int u = 0; u < 8; ++u) M = fmaxf(M, mm[u]);
      }
      float L = 0.f, O = 0.f;
      for (int s0 = 0; s0 < S; s0 += 4) {
        float ms[4], ls[4], os[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r0 = min(s0 + u, S - 1) * rec + hb;
          ms[u] = at(r0);
          ls[u] = at(r0 + 1);
          os[u] = at(r0 + 2 + dd);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (s0 + u < S && ms[u] != -INFINITY) {
            const float f = __expf(ms[u] - M);
            L = fmaf(ls[u], f, L);
            O = fmaf(os[u], f, O);
          }
        }
      }
      st_coh(out + h * D + dd, L > 0.f ? O / L : 0.f);
    }
  };
  if (staged) merge([&](int i) { return st[i]; });
  else merge([&](int i) { return ld_coh(part + i); });
}

#if MPK_LA
// (compiled into the paged lookahead's kernel only, megakernel_la.hip)
// The split of slot s at batch 1 from the one request's cached length Lb
// (the allocation attn_task makes): S = min(S_attn, staging capacity,
// ceil(pages / Tmin)) splits, at least 1 (a slot s >= S is idle); split s
// covers pages [j0, j1) and cached tokens [t0, tc1) (the new token at Lb is
// not cached yet).
struct AttnSplit {
  int S, j0, j1, t0, tc1;
  bool ok;
};
__device__ __forceinline__ AttnSplit attn_split_b1(const KArgs& a, int s, int Lb) {
  AttnSplit r;
  const int P = a.P;
  r.ok = Lb >= 0 && Lb < a.max_seq && (Lb / P) < a.max_pages;
  const int ntok = r.ok ? Lb + 1 : 0;
  const int nb = (ntok + P - 1) / P;
  r.S = max(1, min(min(a.S_attn, attn_stage_cap(a)), (nb + a.attn_min_pages - 1) / a.attn_min_pages));
  r.j0 = (int)((int64_t)s * nb / r.S);
  r.j1 = (int)((int64_t)(s + 1) * nb / r.S);
  r.t0 = r.j0 * P;
  r.tc1 = min(min(r.j1 * P, ntok), ntok - 1);
  return r;
}

// Attention staging of the paged lookahead (batch 1, attention AOT): while
// the worker waits, wavefronts 1..7 copy the cached keys and values of its
// next attention split into that task's pre-load page (a.lds_pf, a.pf_segs:
// the page) -- the cached keys and values are the caller's cache, constant
// during the step; only the new token comes from the q/k/v projection.
// Page layout: the header (valid, staged tokens n, the length Lb it was
// computed for), then the K rows [n][D] and the V rows [n][D], bf16.  n is
// every cached token of the split when they fit, else the largest multiple
// of 32 that fits (the split streams the rest).  Direct global -> LDS loads,
// 64 consecutive 16-byte units each (the rows gathered from their pages); a
// token on a bad page is staged from page 0 and skipped by the split, which
// reports the page.
struct AttnPre {
  int32_t valid, n, lb, pad;
};
constexpr int kPreUnits = kMaxPfSegs;   // direct loads per pre-staging lane, at most
__device__ __forceinline__ int attn_pre_cap(const KArgs& a, int D) {
  // (a load writes a whole 1 KB chunk: the last may pass the rows by up to 1 KB)
  const int area = kPfWaves * min(a.pf_segs, kMaxPfSegs) * 1024 - (int)sizeof(AttnPre) - 1024;
  return max(0, area / (4 * D));   // tokens whose K and V rows fit
}
template <int D>
__device__ __forceinline__ void attn_prestage(const KArgs& a, const DevTask& t, char* lds) {
  const int tid0 = tidx();
  const int w = tid0 >> 6, lane = tid0 & 63;   // wavefronts 1..7
  constexpr int UPR = D / 8;                    // 16-byte units of one row
  const int Lb = a.seq_lens[0];
  const AttnSplit sp = attn_split_b1(a, t.a0, Lb);
  const int ncached = (t.a0 < sp.S && sp.ok) ? max(0, sp.tc1 - sp.t0) : 0;
  const int cap = attn_pre_cap(a, D);
  const int n = ncached <= cap ? ncached : (cap & ~31);
  const int nunits = 2 * n * UPR;
  char* kv = lds + a.lds_pf + sizeof(AttnPre);
  const int64_t page_stride = (int64_t)a.hkv * a.P * D;
  gptr<const uint16_t> kb = a.k_pool + ((int64_t)t.layer * a.n_pages * a.hkv + t.a1) * a.P * D;
  gptr<const uint16_t> vb = a.v_pool + ((int64_t)t.layer * a.n_pages * a.hkv + t.a1) * a.P * D;
  int pid[kPreUnits];
#pragma unroll
  for (int k = 0; k < kPreUnits; ++k) {
    const int un = min(((w - 1) + k * kPfWaves) * 64 + lane, max(nunits - 1, 0));
    const int row = un / UPR, tok = sp.t0 + (row < n ? row : row - n);
    pid[k] = a.page_table[min(tok / a.P, a.max_pages - 1)];
  }
#pragma unroll
  for (int k = 0; k < kPreUnits; ++k) {
    const int c = (w - 1) + k * kPfWaves;
    if (c * 64 < nunits) {
      const int un = min(c * 64 + lane, nunits - 1);
      const int row = un / UPR, part = un - row * UPR;
      const bool isk = row < n;
      const int tok = sp.t0 + (isk ? row : row - n);
      const int pg = (pid[k] >= 0 && pid[k] < a.n_pages) ? pid[k] : 0;
      const int64_t off = (int64_t)pg * page_stride + (int64_t)(tok % a.P) * D + part * 8;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<gptr<const uint4>>((isk ? kb : vb) + off),
                                       (lds_void)(kv + c * 64 * 16), 16, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (tid0 == 64) *reinterpret_cast<AttnPre*>(lds + a.lds_pf) = AttnPre{1, n, Lb, 0};
}
#endif

// Task of slot j of kv group g, serving split s of the S splits of request b
// (attn_slot): decode attention of request b's new query against pages
// [floor(s n_b / S), floor((s+1) n_b / S)) of its n_b = ceil((L_b + 1) / P)
// pages, for all G query heads of kv group g.  An idle slot does nothing.
//  1. The group's raw q/k/v projection row (fp32) is staged in LDS; each of
//     its G query heads and its key head gets per-head RMSNorm (qk_norm) and
//     rotate-half RoPE at position L_b (angle L_b theta^(-2i/d), product and
//     reduction to [-pi, pi] in fp64, cos/sin in fp32).  The last split
//     (s = S-1, the one holding position L_b) writes the new key and value to
//     cache slot L_b in bf16 and attends to them in fp32 as they are.
//  2. Cached tokens: each row of R lanes of a wavefront owns every
//     (8 * 64 / R)-th token of the split (lane i of the row holds dims
//     [i D/R, (i+1) D/R): one coalesced key row and value row per token) and
//     keeps an online-softmax state (max m, sum l, o[d]) per head; key/value
//     rows are double-buffered in registers (loads past the split's end
//     repeat its last token so the wait counts stay static).  R = 16 when
//     G <= 4, 32 for G <= 8.  Row, wavefront and workgroup states merge with
//     the log-sum-exp rule into the split's partial (m, l, o[d]) per head.
//  3. The split writes its partial to slot j, then adds itself to the
//     (layer, b, g) arrival counter; the one that completes it (S arrivals)
//     merges the request's S partials into the attention output
//     (attn_combine) and resets the counter.
// (the paged lookahead's kernel: the split may find its first cached keys
// and values staged in its pre-load page, attn_prestage, when pre is set)
template <int D, int R, int GM>
__device__ __forceinline__ void attn_task(const KArgs& a, const DevTask& t, const TaskPtrs& Pw, char* lds
#if MPK_LA
                                          , bool pre
#endif
                                          ) {
  const int tid0 = tidx();
  constexpr int DPL = D / R;            // dims per lane
  constexpr int RPW = 64 / R;           // rows per wavefront
  constexpr int TPI = kWaves * RPW;     // tokens per iteration of the workgroup
  constexpr int HALF = D / 2;
  using KV = typename std::conditional<DPL == 8, uint4, typename std::conditional<DPL == 4, uint2, uint32_t>::type>::type;
  const int slot = t.a0, g = t.a1, l = t.layer, G = a.G, P = a.P;
  // at batch 1 the request is known (b = 0, s = slot), so the q/k/v row loads
  // go out before the split count, which needs the length, is known
  AttnSlot sl = attn_slot(a, slot, a.B == 1);
  if (sl.b < 0) return;
  const int b = sl.b, s = sl.s;
  const int w = tid0 >> 6, lane = tid0 & 63, row = lane / R, lr = lane % R;
  // LDS: wavefront merge states [kWaves][G][D + 2] at 0, the raw q/k/v row at
  // o_raw, the processed heads [G + 2][D] (G query heads scaled by 1/sqrt(D),
  // the new key, the new value) at o_qk
  const int o_raw = lds_chunks(kWaves * G * (D + 2) * 4);
  const int o_qk = o_raw + lds_chunks((G + 2) * D * 4);
  float* raw = reinterpret_cast<float*>(lds + o_raw);
  float* qk = reinterpret_cast<float*>(lds + o_qk);
  gptr<const float> src = a.qkv + (int64_t)l * a.st_qkv + (int64_t)b * a.hkv * a.Sg + (int64_t)g * a.Sg;
  // (through registers: see gemv_preload; the row is the sum of the
  // projection's t.a2 k-split planes)
  const int nraw = (G + 2) * D;
  float4 rv[(10 * 128 + 4 * kThreads - 1) / (4 * kThreads)];
#pragma unroll
  for (int j = 0; j < (int)(sizeof(rv) / sizeof(rv[0])); ++j) rv[j] = ld4_coh(src, (tid0 + j * kThreads) * 4, nraw);
  for (int p = 1; p < t.a2; ++p) {
    gptr<const float> sp = src + (int64_t)p * a.B * a.hkv * a.Sg;
#pragma unroll
    for (int j = 0; j < (int)(sizeof(rv) / sizeof(rv[0])); ++j) {
      const float4 v = ld4_coh(sp, (tid0 + j * kThreads) * 4, nraw);
      rv[j].x += v.x; rv[j].y += v.y; rv[j].z += v.z; rv[j].w += v.w;
    }
  }

#if MPK_LA
  const AttnPre hp = *reinterpret_cast<const AttnPre*>(lds + a.lds_pf);
  const bool staged = pre && a.B == 1 && hp.valid;
  const int npre = staged ? hp.n : 0;
  const int Lb = staged ? hp.lb : a.seq_lens[b];   // (the length the staging read, the same value)
#else
  const int Lb = a.seq_lens[b];
#endif
  const bool ok = Lb >= 0 && Lb < a.max_seq && (Lb / P) < a.max_pages;
  const int ntok = ok ? Lb + 1 : 0;
  const int nb = (ntok + P - 1) / P;
  // at batch 1, attn_slot's allocation for one request: min(S_attn, ceil(pages / Tmin)) splits,
  // at least 1, and no more than the split combine can stage in LDS; a slot past them is idle
  const int S = a.B == 1 ? max(1, min(min(a.S_attn, attn_stage_cap(a)), (nb + a.attn_min_pages - 1) / a.attn_min_pages))
                         : sl.n;
  if (s >= S) return;
  const bool last_split = s == S - 1;
  if (!ok && tid0 == 0) report(a, MPK_ERR_INVALID_ARG, t.id, -1, (uint32_t)Lb, 0u);
  const int j0 = (int)((int64_t)s * nb / S), j1 = (int)((int64_t)(s + 1) * nb / S);
  const int t0 = j0 * P, t1 = min(j1 * P, ntok);
  const int tc1 = min(t1, ntok - 1);    // cached tokens of the split: [t0, tc1)
  int* pids = reinterpret_cast<int*>(lds + a.lds_pid);   // page ids of pages j0..j1-1
  for (int j = j0 + tid0; j < j1; j += kThreads) {
    int pid = a.page_table[(int64_t)b * a.max_pages + j];
    if (pid < 0 || pid >= a.n_pages) {
      report(a, MPK_ERR_INVALID_ARG, t.id, -1, (uint32_t)pid, (uint32_t)a.n_pages);
      pid = -1;
    }
    pids[j - j0] = pid;
  }
  const bool act = lane < HALF;
  const int lc = min(lane, HALF - 1);
  float cs = 1.f, sn = 0.f;
  if (act) {
    const double ang = (double)(ok ? Lb : 0) * a.inv_freq[lc];
    const double two_pi = 6.283185307179586476925286766559;
    const float red_ang = (float)(ang - two_pi * rint(ang / two_pi));
    sincosf(red_ang, &sn, &cs);
  }
  float g0q = 1.f, g1q = 1.f, g0k = 1.f, g1k = 1.f;
  if (a.qk_norm) {
    gptr<const uint16_t> gq = Pw.p0, gk = Pw.p1;
    g0q = bf2f(gq[lc]); g1q = bf2f(gq[lc + HALF]);
    g0k = bf2f(gk[lc]); g1k = bf2f(gk[lc + HALF]);
  }
#pragma unroll
  for (int j = 0; j < (int)(sizeof(rv) / sizeof(rv[0])); ++j) {
    const int i = (tid0 + j * kThreads) * 4;
    if (i < nraw) *reinterpret_cast<float4*>(raw + i) = rv[j];
  }
  __syncthreads();   // raw row staged, page ids written
  const float scale = 1.0f / sqrtf((float)D);
  for (int hh = w; hh < G + 2; hh += kWaves) {
    float x0 = act ? raw[hh * D + lc] : 0.f, x1 = act ? raw[hh * D + lc + HALF] : 0.f;
    if (hh <= G) {   // query heads and the key head: q/k RMSNorm, RoPE
      if (a.qk_norm) {
        const float ss = wave_sum(x0 * x0 + x1 * x1);
        const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
        x0 = x0 * inv * (hh < G ? g0q : g0k);
        x1 = x1 * inv * (hh < G ? g1q : g1k);
      }
      const float y0 = x0 * cs - x1 * sn;
      const float y1 = x1 * cs + x0 * sn;
      const float f = hh < G ? scale : 1.f;
      x0 = y0 * f;
      x1 = y1 * f;
    }
    if (act) {
      qk[hh * D + lane] = x0;
      qk[hh * D + lane + HALF] = x1;
    }
    if (hh >= G && last_split && ok && act) {   // append the new key / value to the cache
      const int pid = pids[Lb / P - j0];
      if (pid >= 0) {
        gptr<uint16_t> pool = hh == G ? a.k_pool : a.v_pool;
        const int64_t slot = ((((int64_t)l * a.n_pages + pid) * a.hkv + g) * P + (Lb % P)) * D;
        pool[slot + lane] = f2bf(x0);
        pool[slot + lane + HALF] = f2bf(x1);
      }
    }
  }
  __syncthreads();
  float qv[GM][DPL], ov[GM][DPL], m[GM], lsum[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const float qx = qk[min(h, G - 1) * D + lr * DPL + i];
      qv[h][i] = h < G ? qx : 0.f;
      ov[h][i] = 0.f;
    }
  }
  mark(a, 0);
  gptr<const uint16_t> kbase = a.k_pool + ((int64_t)l * a.n_pages * a.hkv + g) * P * D + lr * DPL;
  gptr<const uint16_t> vbase = a.v_pool + ((int64_t)l * a.n_pages * a.hkv + g) * P * D + lr * DPL;
  const int64_t page_stride = (int64_t)a.hkv * P * D;
  // offset of cached token `tok`, clamped into the split (a bad page reads page 0 and is not used)
  auto offs = [&](int tok) -> int64_t {
    tok = min(tok, tc1 - 1);
    const int pid = pids[tok / P - j0];
    return (int64_t)(pid >= 0 ? pid : 0) * page_stride + (int64_t)(tok % P) * D;
  };
  auto good = [&](int tok) { return tok < tc1 && pids[tok / P - j0] >= 0; };
#if MPK_BN
  // (batch > 1: the splits are long and the loop is bound by its VALU work.
  // The running state (m, lsum, ov) is exact for any reference m, since
  // lsum = sum exp(p - m) and ov = sum exp(p - m) v; m is raised only when a
  // score exceeds it by more than kLazy, so exp(p - m) stays below e^8 and
  // the per-key rescale of ov is skipped in all but the few steps that raise
  // it -- a wavefront-uniform branch, taken when any of its rows needs it.)
  constexpr float kLazy = 8.f;
  auto process = [&](const float (&kf)[DPL], const float (&vf)[DPL]) {
    float pr[GM];
    bool raise = false;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      pr[h] = 0.f;
      if (h < G) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) p = fmaf(qv[h][i], kf[i], p);
        p = row_sum(p);
        if (R == 32) p = pair_sum<16>(p);
        pr[h] = p;
        raise |= p > m[h] + kLazy;
      }
    }
    if (__ballot(raise)) {
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G && pr[h] > m[h] + kLazy) {
          const float al = __expf(m[h] - pr[h]);
          lsum[h] *= al;
#pragma unroll
          for (int i = 0; i < DPL; ++i) ov[h][i] *= al;
          m[h] = pr[h];
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float e = __expf(pr[h] - m[h]);
        lsum[h] += e;
#pragma unroll
        for (int i = 0; i < DPL; ++i) ov[h][i] = fmaf(e, vf[i], ov[h][i]);
      }
    }
  };
#else
  auto process = [&](const float (&kf)[DPL], const float (&vf)[DPL]) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) p = fmaf(qv[h][i], kf[i], p);
        p = row_sum(p);
        if (R == 32) p = pair_sum<16>(p);
        const float mn = fmaxf(m[h], p);
        const float al = __expf(m[h] - mn);
        const float e = __expf(p - mn);
        lsum[h] = fmaf(lsum[h], al, e);
#pragma unroll
        for (int i = 0; i < DPL; ++i) ov[h][i] = fmaf(ov[h][i], al, e * vf[i]);
        m[h] = mn;
      }
    }
  };
#endif
  auto process_bf = [&](const KV& kc, const KV& vc) {
    float kf[DPL], vf[DPL];
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kc);
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vc);
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i) {
      kf[2 * i] = bflo(kw[i]); kf[2 * i + 1] = bfhi(kw[i]);
      vf[2 * i] = bflo(vw[i]); vf[2 * i + 1] = bfhi(vw[i]);
    }
    process(kf, vf);
  };
#if MPK_LA
  if (npre > 0) {   // the staged tokens [t0, t0 + npre), from the page
    const uint16_t* kl = reinterpret_cast<const uint16_t*>(lds + a.lds_pf + sizeof(AttnPre));
    const uint16_t* vl = kl + (int64_t)npre * D;
    for (int it = t0 + w * RPW; it < t0 + npre; it += TPI) {
      const int tok = it + row;
      if (tok < t0 + npre && good(tok))
        process_bf(*reinterpret_cast<const KV*>(kl + (tok - t0) * D + lr * DPL),
                   *reinterpret_cast<const KV*>(vl + (tok - t0) * D + lr * DPL));
    }
  }
  if (tc1 > t0 + npre) {
    const int base = t0 + npre + w * RPW;   // the wavefront's first token of each iteration (uniform)
#else
  if (tc1 > t0) {
    const int base = t0 + w * RPW;   // the wavefront's first token of each iteration (uniform)
#endif
    int tok = base + row;
    KV k0, v0, k1, v1;
    int64_t o = offs(tok);
    k0 = ldg<KV>(kbase + o);
    v0 = ldg<KV>(vbase + o);
    for (int it = base; it < tc1; it += 2 * TPI, tok += 2 * TPI) {
      o = offs(tok + TPI);
      k1 = ldg<KV>(kbase + o);
      v1 = ldg<KV>(vbase + o);
      if (good(tok)) process_bf(k0, v0);
      if (it + TPI >= tc1) break;
      o = offs(tok + 2 * TPI);
      k0 = ldg<KV>(kbase + o);
      v0 = ldg<KV>(vbase + o);
      if (good(tok + TPI)) process_bf(k1, v1);
    }
  }
  if (last_split && ok && w == 0 && row == 0) {   // the new token, in fp32
    float kf[DPL], vf[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      kf[i] = qk[G * D + lr * DPL + i];
      vf[i] = qk[(G + 1) * D + lr * DPL + i];
    }
    process(kf, vf);
  }
  mark(a, 1);
  // merge the row states of the wavefront (lanes lr, lr+R, ...), each pair
  // in (even, odd) order so that both of its lanes hold the same state
  auto merge_rows = [&](auto msk_c) {
    constexpr int MSK = decltype(msk_c)::value;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float m1, m2, l1, l2;
        lane_pair<MSK>(m[h], m1, m2);
        lane_pair<MSK>(lsum[h], l1, l2);
        const float mn = fmaxf(m1, m2);
        const float a1 = (m1 == -INFINITY) ? 0.f : __expf(m1 - mn);
        const float a2 = (m2 == -INFINITY) ? 0.f : __expf(m2 - mn);
        lsum[h] = l1 * a1 + l2 * a2;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          float o1, o2;
          lane_pair<MSK>(ov[h][i], o1, o2);
          ov[h][i] = o1 * a1 + o2 * a2;
        }
        m[h] = mn;
      }
    }
  };
  static_assert(R == 16 || R == 32, "16 or 32 lanes per row");
  if constexpr (R == 16) merge_rows(std::integral_constant<int, 16>{});
  merge_rows(std::integral_constant<int, 32>{});
  // merge the wavefronts through LDS: per wave, per head: m, l, o[D]
  float* st = reinterpret_cast<float*>(lds);  // [kWaves][G][D + 2]
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float* p = st + ((int64_t)w * G + h) * (D + 2);
        if (lr == 0) { p[0] = m[h]; p[1] = lsum[h]; }
#pragma unroll
        for (int i = 0; i < DPL; ++i) p[2 + lr * DPL + i] = ov[h][i];
      }
    }
  }
  __syncthreads();
  gptr<float> out = a.part + (int64_t)l * a.st_part + ((int64_t)g * a.S_attn + slot) * (int64_t)(G * (D + 2));
  for (int e = tid0; e < G * D; e += kThreads) {
    const int h = e / D, dd = e - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, st[(ww * G + h) * (D + 2)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float* p = st + (ww * G + h) * (D + 2);
        if (p[0] != -INFINITY) {
          const float f = __expf(p[0] - M);
          L = fmaf(p[1], f, L);
          O = fmaf(p[2 + dd], f, O);
        }
      }
    }
    st_coh(out + h * (D + 2) + 2 + dd, O);
    if (dd == 0) {
      st_coh(out + h * (D + 2), M);
      st_coh(out + h * (D + 2) + 1, L);
    }
  }
  // arrival: every wavefront's partial stores are complete before the
  // barrier, so the split that completes the count reads all S partials
  wait_vm<0>();
  __syncthreads();
  int* flag = reinterpret_cast<int*>(lds + kLdsCtl) + 2;
  if (tid0 == 0) {
    gptr<uint32_t> ctr = a.arrive + ((int64_t)l * a.B + b) * a.hkv + g;
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old + 1u == (uint32_t)S;
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(*flag)) attn_combine(a, l, b, g, sl.start, S, lds);
  __syncthreads();
}

// ------------------------------------------------------------------ final argmax
// next_ids[b] = argmax over the LM-head tile partials; ties -> lowest index.
// Wavefront w reduces requests w, w + 8, ...: each lane loads its tiles'
// partials for all of its requests at once, then the wavefront reduces each
// request by shuffles (no workgroup barrier per request).
__device__ __forceinline__ void argmax_task(const KArgs& a, char* lds) {
  (void)lds;
  const int tid0 = tidx();
  const int w = tid0 >> 6, lane = tid0 & 63;
  for (int b = w; b < a.B; b += kWaves) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int n0 = 0; n0 < a.T_lm; n0 += 64 * 8) {
      unsigned long long pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int n = min(n0 + u * 64 + lane, a.T_lm - 1);
        pv[u] = __hip_atomic_load(reinterpret_cast<MPK_GLOBAL unsigned long long*>(a.pmax + b * a.T_lm + n),
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const PMax p{__uint_as_float((uint32_t)pv[u]), (int32_t)(pv[u] >> 32)};
        if (n0 + u * 64 + lane < a.T_lm && (p.v > bv || (p.v == bv && p.i < bi))) { bv = p.v; bi = p.i; }
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) a.next_ids[b] = (bi == INT_MAX) ? 0 : bi;
  }
}

// ------------------------------------------------------------------ mixture of experts
// Routing of layer l for expert slot s (Qwen3-MoE reading of the MoE layer
// in the MPK summary's workload list): per request, the softmax of its E
// router logits, its top_k experts by probability (ties: the lower index)
// and their probabilities, renormalised to sum 1 when norm_topk.  Slot s
// serves the s-th smallest expert that any request chose (none: the slot is
// idle, e = -1) for the requests that chose it, in ascending order, each
// with its weight for that expert.  Result in MoeLds.
// moe_route_issue stages the B x E logits into LDS (direct loads, left in
// flight so that the caller can put its own staging beside them);
// moe_route_finish waits for them and routes, wavefront w taking requests
// w, w + 8, ...: lane i holds logits i, i + 64, ... as order-preserving
// integer keys; the k-th largest key is found bit by bit (32 steps of a
// wavefront count by ballots), the chosen experts are the keys above it and
// the lowest-index keys equal to it, stored in ascending expert order with
// their weights; wavefront 0 then resolves the slot.
__device__ __forceinline__ float* moe_logits(const KArgs& a, char* lds) {
  return reinterpret_cast<float*>(lds + a.lds_moe + sizeof(MoeLds));
}
__device__ __forceinline__ void moe_route_issue(const KArgs& a, int l, char* lds) {
  const int tid0 = tidx();
  MoeLds* m = moe_lds(a, lds);
  if (tid0 < kMaxExperts / 32) m->mask[tid0] = 0u;
  lds_stage<4, true>(a.rlog + (int64_t)l * a.st_rlog, reinterpret_cast<char*>(moe_logits(a, lds)), a.B * a.E, tid0);
}
// fp32 -> uint32 with the same order (-0 and +0 equal; a NaN above +inf)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = f == 0.f ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ void moe_route_finish(const KArgs& a, int s, char* lds) {
  const int tid0 = tidx();
  const int w = tid0 >> 6, lane = tid0 & 63;
  MoeLds* m = moe_lds(a, lds);
  const float* lg = moe_logits(a, lds);
  const int E = a.E, K = a.topk, B = a.B;
  constexpr int NJ = kMaxExperts / 64;
  const unsigned long long below = (1ull << lane) - 1ull;
  lds_stage_wait();
  for (int b = w; b < B; b += kWaves) {
    float v[NJ];
    uint32_t key[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = lane + 64 * j;
      v[j] = lg[b * E + min(e, E - 1)];
      key[j] = e < E ? order_key(v[j]) : 0u;   // (every real key is above 0: -inf maps to 0x007fffff)
      if (e >= E) v[j] = -INFINITY;
    }
    // the k-th largest key
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < NJ; ++j) cnt += __builtin_popcountll(__ballot(key[j] >= c));
      if (cnt >= K) T = c;
    }
    int gt = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) gt += __builtin_popcountll(__ballot(key[j] > T));
    const int need = K - gt;   // keys equal to T that are chosen, lowest index first
    bool ch[NJ];
    int taken = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const unsigned long long eq = __ballot(key[j] == T);
      ch[j] = key[j] > T || (key[j] == T && taken + __builtin_popcountll(eq & below) < need);
      taken += __builtin_popcountll(eq);
    }
    float mx = v[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) mx = fmaxf(mx, v[j]);
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) mx = fmaxf(mx, __shfl_xor(mx, k));
    float p[NJ], pc = 0.f, pa = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      p[j] = lane + 64 * j < E ? expf(v[j] - mx) : 0.f;
      pa += p[j];
      pc += ch[j] ? p[j] : 0.f;
    }
    const float den = wave_sum(a.norm_topk ? pc : pa);
    int pos = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const unsigned long long cm = __ballot(ch[j]);
      const int at = pos + __builtin_popcountll(cm & below);
      if (ch[j] && at < kMaxTopK) {
        const int e = lane + 64 * j;
        m->cid[b][at] = e;
        m->cw[b][at] = p[j] / den;
        atomicOr(&m->mask[e >> 5], 1u << (e & 31));
      }
      pos += __builtin_popcountll(cm);
    }
  }
  __syncthreads();
  if (w == 0) {
    // the s-th set bit of the chosen set
    int e = -1, r = s;
    for (int i = 0; i < kMaxExperts / 32 && e < 0; ++i) {
      uint32_t bits = m->mask[i];
      const int c = __builtin_popcount(bits);
      if (r >= c) { r -= c; continue; }
      for (; r > 0; --r) bits &= bits - 1;
      e = 32 * i + __builtin_ctz(bits);
    }
    int hit = -1;
    if (lane < B && e >= 0)
      for (int i = 0; i < K; ++i)
        if (m->cid[lane][i] == e) hit = i;
    const unsigned long long bal = __ballot(hit >= 0);
    const int pos = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (hit >= 0) {
      m->tok[pos] = lane;
      m->w[pos] = m->cw[lane][hit];
    }
    if (lane == 0) {
      m->e = e;
      m->n = __builtin_popcountll(bal);
    }
  }
  __syncthreads();
}

// An expert tile of slot s = t.a2: gate/up tiles route (moe_route_*), and
// tile 0 of the slot stores the route record [expert, count, tokens[B],
// weights[B]] that the slot's down tiles read instead of routing again.  An
// idle slot's gate/up tiles write zeros; its down tiles do nothing.
// Otherwise the slot's expert's matrices are a projection over the slot's
// tokens: batch 1, the one token's row, staged in LDS while the routing's
// loads are in flight; batch > 1, the tokens' rows gathered into the
// matrix-core tile's columns.
__device__ __forceinline__ void expert_task(const KArgs& a, const DevTask& t, const TaskPtrs& P0, char* lds) {
  const int tid0 = tidx();
  const int l = t.layer, s = t.a2, B = a.B, rw = 2 + 2 * B;
  const bool gu = t.type == MPK_TASK_EXPERT_GU;
  MoeLds* m = moe_lds(a, lds);
  gptr<int32_t> rec = a.route + (int64_t)l * a.st_route + (int64_t)s * rw;
  // batch 1: the input row (h2_l, or the slot's gate/up output) goes to LDS now
  if (B == 1) {
    const XSrc x = gemv_xsrc(a, t, P0);
    lds_stage<16, true>(x.v1, lds, (gu ? a.H : a.Fe) / 4, tid0);
  }
  if (gu) {
    moe_route_issue(a, l, lds);
    moe_route_finish(a, s, lds);
    mark(a, 0);
    if (t.a0 == 0 && tid0 < rw) {
      const int n = m->n, j = tid0 - 2, k = tid0 - 2 - B;
      const int32_t v = tid0 == 0 ? m->e
                      : tid0 == 1 ? n
                      : j < B     ? (j < n ? m->tok[j] : 0)
                                  : (k < n ? __float_as_int(m->w[k]) : 0);
      __hip_atomic_store(rec + tid0, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else {
    // (a record holding a token outside the batch is not used: no add lands outside d_l)
    int* bad = reinterpret_cast<int*>(lds + kLdsRed);
    if (tid0 == 0) *bad = 0;
    __syncthreads();
    if (tid0 < rw) {
      const int32_t v = __hip_atomic_load(rec + tid0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int j = tid0 - 2, k = tid0 - 2 - B;
      if (tid0 == 0) m->e = v;
      else if (tid0 == 1) m->n = v;
      else if (j < B) {
        m->tok[j] = v;
        if (v < 0 || v >= B) atomicOr(bad, 1);
      } else {
        m->w[k] = __int_as_float(v);
      }
    }
    if (B == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // (the staged row, too)
    __syncthreads();
    mark(a, 0);
    if (__builtin_amdgcn_readfirstlane(*bad)) return;
  }
  const int e = __builtin_amdgcn_readfirstlane(m->e), n = __builtin_amdgcn_readfirstlane(m->n);
  if (e < 0 || e >= a.E || n < 1 || n > B) {
    if (gu) {
      const int ncol = t.a1 - t.a0;
      gptr<float> out = a.a + (int64_t)l * a.st_a + (int64_t)s * B * a.Fe;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        const int j = i / ncol, c = i - j * ncol;
        st_coh(out + (int64_t)j * a.Fe + t.a0 + c, 0.f);
      }
    }
    return;
  }
  TaskPtrs P = P0;
  const int64_t ew = (int64_t)e * a.Fe * a.H;   // elements per expert matrix
  P.p0 = P0.p0 + ew;
  if (gu) P.p1 = P0.p1 + ew;
  if (B > 1) {
    const GemvOp op = gu ? GemvOp{a.H, 2, a.h2 + (int64_t)l * a.st_bh, m->tok, n}
                         : GemvOp{a.Fe, 1, a.a + (int64_t)l * a.st_a + (int64_t)s * B * a.Fe, nullptr, n};
    gemv_mfma(a, t, P, lds, op);
  } else {
    gemv_b1<kB1Chunk>(a, t, P, lds, false, true);
  }
}

// ------------------------------------------------------------------ dispatch
// Runs task t, with its resolved weight pointers P (task_ptrs), with the
// whole workgroup; pre: its weight pre-load (gemv_preload) was issued.
__device__ __forceinline__ void run_task(const KArgs& a, const DevTask& t, const TaskPtrs& P, bool pre = false) {
  char* lds = g_lds;
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  const int l = t.layer;
  switch (t.type) {
    case MPK_TASK_EMBED:
      embed_task(a, t.a0);
      break;
    case MPK_TASK_ATTN_NORM:
      if (l == 0) norm_task(a, t.a0, a.e, nullptr, 0, a.r, P.p0, a.h, lds, red);
      else
        norm_task(a, t.a0, a.s + (int64_t)(l - 1) * a.st_bh, a.dn + (int64_t)(l - 1) * a.st_dn, a.Kd,
                  a.r + (int64_t)l * a.st_bh, P.p0, a.h + (int64_t)l * a.st_bh, lds, red);
      break;
    case MPK_TASK_MLP_NORM:
      norm_task(a, t.a0, a.r + (int64_t)l * a.st_bh, a.o + (int64_t)l * a.st_o, a.Ko, a.s + (int64_t)l * a.st_bh,
                P.p0, a.h2 + (int64_t)l * a.st_bh, lds, red);
      if (a.E > 0) {   // (mixture of experts: row b of d_l starts at zero, the down tiles add to it)
        gptr<float> d = a.dn + (int64_t)l * a.st_dn + (int64_t)t.a0 * a.H;
        for (int i = tidx(); i < a.H; i += kThreads) st_coh(d + i, 0.f);
      }
      break;
    case MPK_TASK_FINAL_NORM:
      norm_task(a, t.a0, a.s + (int64_t)(a.L - 1) * a.st_bh, a.dn + (int64_t)(a.L - 1) * a.st_dn, a.Kd, nullptr,
                P.p0, a.hf, lds, red);
      break;
    case MPK_TASK_QKV:
    case MPK_TASK_OPROJ:
    case MPK_TASK_GATEUP:
    case MPK_TASK_DOWN:
    case MPK_TASK_LMHEAD:
    case MPK_TASK_ROUTER:
      if (a.B > 1) gemv_mfma(a, t, P, lds, gemv_op(a, t));
      else gemv_b1<kB1Chunk>(a, t, P, lds, pre);
      break;
    case MPK_TASK_EXPERT_GU:
    case MPK_TASK_EXPERT_DOWN:
      expert_task(a, t, P, lds);
      break;
    case MPK_TASK_ATTN:
      if (a.d == 128) {
#if MPK_LA
        if (a.G <= 4) attn_task<128, 16, 4>(a, t, P, lds, pre);
        else attn_task<128, 32, 8>(a, t, P, lds, pre);
      } else {
        attn_task<64, 16, 8>(a, t, P, lds, pre);
      }
#else
        if (a.G <= 4) attn_task<128, 16, 4>(a, t, P, lds);
        else attn_task<128, 32, 8>(a, t, P, lds);
      } else {
        attn_task<64, 16, 8>(a, t, P, lds);
      }
#endif
      break;
    case MPK_TASK_ARGMAX:
      argmax_task(a, lds);
      break;
    default:
      break;
  }
}

}  // namespace mpk
