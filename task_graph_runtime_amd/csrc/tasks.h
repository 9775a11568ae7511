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
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Sum over the workgroup; `red` is kWaves floats of LDS.  All threads call it.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int tid0 = tidx();
  v = wave_sum(v);
  const int w = tid0 >> 6;
  if ((tid0 & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  __syncthreads();
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

// LDS layout of a workgroup (one per compute unit).
constexpr int kLdsBytes = 160 * 1024;
constexpr int kLdsX = 0;                       // staged activation vector (fp32), batch 1
constexpr int kLdsXFloats = 26624;             // 104 KB: the widest K of the supported shapes
constexpr int kLdsAcc = kLdsXFloats * 4;       // projection accumulators
constexpr int kLdsAccFloats = 8192;            // 32 KB
constexpr int kLdsMisc = kLdsAcc + kLdsAccFloats * 4;   // 24 KB: page ids, control, reduction scratch
constexpr int kLdsCtl = kLdsMisc + 16384;      // runtime control words
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
template <int U>
__device__ __forceinline__ void lds_stage(gptr<const void> src, char* dst, int n, int tid) {
  static_assert(U == 16 || U == 4, "16- or 4-byte units");
  using unit = typename std::conditional<U == 16, uint4, uint32_t>::type;
  const int w = tid >> 6, lane = tid & 63;
  gptr<const unit> su = reinterpret_cast<gptr<const unit>>(src);
  for (int c = w; c * 64 < n; c += kWaves) {
    const int u = min(c * 64 + lane, n - 1);
    __builtin_amdgcn_global_load_lds(su + u, (lds_void)(dst + c * 64 * U), U, 0, 0);
  }
}
__device__ __forceinline__ void lds_stage_wait() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}
// bytes of LDS a staged copy of `bytes` occupies (whole 1 KB chunks)
__device__ __forceinline__ int lds_chunks(int bytes) { return (bytes + 1023) & ~1023; }

// ------------------------------------------------------------------ embedding
__device__ __forceinline__ void embed_task(const KArgs& a) {
  const int tid0 = tidx();
  for (int b = 0; b < a.B; ++b) {
    int id = a.token_ids[b];
    if (id < 0 || id >= a.V) {
      if (tid0 == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)id, (uint32_t)a.V);
      id = 0;
    }
    gptr<const uint16_t> row = a.embed + (int64_t)id * a.H;
    for (int i = tid0; i < a.H; i += kThreads) a.e[(int64_t)b * a.H + i] = bf2f(row[i]);
  }
}

// ------------------------------------------------------------------ residual add + RMSNorm
// res = x + y (y optional), stored when `res` is given; out = RMSNorm(res) * gamma.
// gamma and the input rows are staged in LDS with direct loads (all rows at
// once when they fit, else one row at a time).
__device__ __forceinline__ void norm_task(const KArgs& a, gptr<const float> __restrict__ x,
                                          gptr<const float> __restrict__ y, gptr<float> __restrict__ res,
                                          gptr<const uint16_t> __restrict__ gamma, gptr<float> __restrict__ out,
                                          char* lds, float* red) {
  const int tid0 = tidx();
  const int H = a.H, B = a.B;
  const int hb = lds_chunks(H * 4), gb = lds_chunks(H * 2);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(lds + kLdsX);
  char* xsl = lds + kLdsX + gb;
  const int rows = (B * 2 * hb + gb <= kLdsXFloats * 4) ? B : 1;
  lds_stage<16>(gamma, lds + kLdsX, H / 8, tid0);
  for (int b0 = 0; b0 < B; b0 += rows) {
    const int nr = min(rows, B - b0);
    for (int r = 0; r < nr; ++r) {
      lds_stage<16>(x + (int64_t)(b0 + r) * H, xsl + (2 * r) * hb, H / 4, tid0);
      if (y) lds_stage<16>(y + (int64_t)(b0 + r) * H, xsl + (2 * r + 1) * hb, H / 4, tid0);
    }
    lds_stage_wait();
    mark(a, 0);
    for (int r = 0; r < nr; ++r) {
      const float* xr = reinterpret_cast<const float*>(xsl + (2 * r) * hb);
      const float* yr = reinterpret_cast<const float*>(xsl + (2 * r + 1) * hb);
      float ss = 0.f;
      for (int i = tid0; i < H; i += kThreads) {
        const float v = y ? xr[i] + yr[i] : xr[i];
        ss = fmaf(v, v, ss);
      }
      ss = block_sum(ss, red);
      mark(a, 1);
      const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
      for (int i = tid0; i < H; i += kThreads) {
        const float v = y ? xr[i] + yr[i] : xr[i];
        if (res) res[(int64_t)(b0 + r) * H + i] = v;
        out[(int64_t)(b0 + r) * H + i] = v * inv * bf2f(gs[i]);
      }
    }
    __syncthreads();   // the staging area is refilled by the next group of rows
  }
}

// ------------------------------------------------------------------ weight pointers
// The weight base pointers of task t (see TaskPtrs), read from the per-layer
// pointer table; all loads are issued together.
__device__ __forceinline__ TaskPtrs task_ptrs(const KArgs& a, const DevTask& t) {
  TaskPtrs r{};
  gptr<const gptr<const uint16_t>> W = a.wl + (int64_t)(t.layer < 0 ? 0 : t.layer) * LAYER_PTRS;
  switch (t.type) {
    case MPK_TASK_QKV: r.p0 = W[W_Q]; r.p1 = W[W_K]; r.p2 = W[W_V]; break;
    case MPK_TASK_OPROJ: r.p0 = W[W_O]; break;
    case MPK_TASK_GATEUP: r.p0 = W[W_GATE]; r.p1 = W[W_UP]; break;
    case MPK_TASK_DOWN: r.p0 = W[W_DOWN]; break;
    case MPK_TASK_LMHEAD: r.p0 = a.lm_head ? a.lm_head : a.embed; break;
    case MPK_TASK_ATTN_NORM: r.p0 = W[W_IN_NORM]; break;
    case MPK_TASK_MLP_NORM: r.p0 = W[W_POST_NORM]; break;
    case MPK_TASK_FINAL_NORM: r.p0 = a.final_norm; break;
    case MPK_TASK_QKNORM_ROPE: r.p0 = W[W_Q_NORM]; r.p1 = W[W_K_NORM]; break;
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
    default:
      return P.p0 + (int64_t)(lo + r) * a.H;
  }
}

struct GemvOp {
  int K, rpc;
  gptr<const float> x;
};
__device__ __forceinline__ GemvOp gemv_op(const KArgs& a, const DevTask& t) {
  const int l = t.layer;
  switch (t.type) {
    case MPK_TASK_QKV: return {a.H, 1, a.h + (int64_t)l * a.st_bh};
    case MPK_TASK_OPROJ: return {a.hq * a.d, 1, a.attn + (int64_t)l * a.st_q};
    case MPK_TASK_GATEUP: return {a.H, 2, a.h2 + (int64_t)l * a.st_bh};
    case MPK_TASK_DOWN: return {a.F, 1, a.a + (int64_t)l * a.st_a};
    default: return {a.H, 1, a.hf};
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

// Epilogue of a projection tile from the LDS accumulators acc[row][B].
__device__ __forceinline__ void gemv_epilogue(const KArgs& a, const DevTask& t, const float* acc, float* red) {
  const int tid0 = tidx();
  const int type = t.type, l = t.layer, lo = t.a0, ncol = t.a1 - t.a0, B = a.B;
  const int w = tid0 >> 6, lane = tid0 & 63;
  switch (type) {
    case MPK_TASK_QKV: {
      const int ld = a.hkv * a.Sg;
      gptr<float> out = a.qkv + (int64_t)l * a.st_qkv;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        out[(int64_t)b * ld + lo + c] = acc[c * B + b];
      }
      break;
    }
    case MPK_TASK_OPROJ: {
      gptr<float> out = a.o + (int64_t)l * a.st_bh;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        out[(int64_t)b * a.H + lo + c] = acc[c * B + b];
      }
      break;
    }
    case MPK_TASK_DOWN: {
      gptr<float> out = a.dn + (int64_t)l * a.st_bh;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        out[(int64_t)b * a.H + lo + c] = acc[c * B + b];
      }
      break;
    }
    case MPK_TASK_GATEUP: {  // SwiGLU: silu(gate) * up
      gptr<float> out = a.a + (int64_t)l * a.st_a;
      for (int i = tid0; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        float g = acc[(2 * c) * B + b], u = acc[(2 * c + 1) * B + b];
        out[(int64_t)b * a.F + lo + c] = g / (1.0f + expf(-g)) * u;
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
          a.pmax[b * a.T_lm + t.a2] = PMax{bv, bi};
        }
        __syncthreads();
      }
      break;
    }
  }
}

// Batch-1 projection tile: y[n] = sum_k x[k] W[n, k] for the tile's columns.
// The tile's weight rows are cut into 1 KB segments (64 lanes x 8 bf16, one
// 16-byte load per lane); wavefront w streams the contiguous run of segments
// [S w / 8, S (w+1) / 8) through two register buffers of D segments (the
// loads of one buffer are in flight while the other is consumed), keeps one
// fp32 partial for the current row, and on a row change reduces it across
// the wavefront (DPP + lane swaps) into the row's LDS accumulator.  The first
// buffer's loads are issued before x is staged in LDS (fp32), so both round
// trips overlap.  Loads are issued unconditionally -- past the end they
// repeat the last segment -- so the wait counts stay static.
template <int D>
__device__ __forceinline__ void gemv_b1(const KArgs& a, const DevTask& t, const TaskPtrs& P, char* lds) {
  const int tid0 = tidx();
  const GemvOp op = gemv_op(a, t);
  const int K = op.K, nrows = (t.a1 - t.a0) * op.rpc;
  float* xs = reinterpret_cast<float*>(lds + kLdsX);
  float* acc = reinterpret_cast<float*>(lds + kLdsAcc);
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  const int nseg = (K + 511) >> 9, S = nrows * nseg;
  const int w = tid0 >> 6, lane = tid0 & 63;
  const int s_beg = (int)((int64_t)S * w / kWaves), total = (int)((int64_t)S * (w + 1) / kWaves) - s_beg;
  const int kl = lane * 8;
  SegWalk ld = seg_start(a, t, P, nseg, s_beg < S ? s_beg : S - 1);
  int issued = 0;
  uint4 b0[D], b1[D];
  auto issue = [&](uint4 (&b)[D]) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int k = min(ld.ks * 512 + kl, K - 8);
      b[u] = ldg<uint4>(ld.row + k);
      if (issued + 1 < total) seg_next(a, t, P, nseg, ld);
      ++issued;
    }
  };
  if (total > 0) issue(b0);
  for (int i = tid0; i < nrows; i += kThreads) acc[i] = 0.f;
  // stage x (fp32) in LDS with direct loads, behind the first weight buffer
  lds_stage<16>(op.x, reinterpret_cast<char*>(xs), K / 4, tid0);
  lds_stage_wait();
  mark(a, 0);
  if (total > 0) {
    int cr = s_beg / nseg, cks = s_beg - cr * nseg;  // consumer position
    int done = 0, cur = cr;
    float accv = 0.f;
    auto consume = [&](const uint4 (&b)[D]) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        if (done < total) {
          if (cr != cur) {
            const float v = wave_sum(accv);
            if (lane == 0) atomicAdd(&acc[cur], v);
            accv = 0.f;
            cur = cr;
          }
          const int k = cks * 512 + kl;
          if (k < K) {
            const float4* xp = reinterpret_cast<const float4*>(xs + k);
            accv = dot8(b[u], xp[0], xp[1], accv);
          }
          if (++cks == nseg) { cks = 0; ++cr; }
          ++done;
        }
      }
    };
    while (true) {
      issue(b1);
      consume(b0);
      if (done >= total) break;
      issue(b0);
      consume(b1);
      if (done >= total) break;
    }
    const float v = wave_sum(accv);
    if (lane == 0) atomicAdd(&acc[cur], v);
  }
  mark(a, 1);
  __syncthreads();
  gemv_epilogue(a, t, acc, red);
}

// Batch 2..16 projection tile (VALU): same segment walk, x read from global
// memory (L2-resident), one fp32 partial per request.
__device__ __forceinline__ void gemv_bn(const KArgs& a, const DevTask& t, const TaskPtrs& P, char* lds) {
  const int tid0 = tidx();
  constexpr int U = 4;
  const GemvOp op = gemv_op(a, t);
  const int K = op.K, nrows = (t.a1 - t.a0) * op.rpc, B = a.B;
  float* acc = reinterpret_cast<float*>(lds + kLdsAcc);
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  for (int i = tid0; i < nrows * B; i += kThreads) acc[i] = 0.f;
  __syncthreads();
  const int nseg = (K + 511) >> 9, S = nrows * nseg;
  const int w = tid0 >> 6, lane = tid0 & 63;
  const int s_beg = (int)((int64_t)S * w / kWaves), total = (int)((int64_t)S * (w + 1) / kWaves) - s_beg;
  if (total > 0) {
    SegWalk ld = seg_start(a, t, P, nseg, s_beg);
    int cur = ld.r, done = 0;
    float av[kMaxBatch];
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b) av[b] = 0.f;
    while (done < total) {
      uint4 wv[U];
      int rr[U], kk[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        rr[u] = ld.r;
        kk[u] = ld.ks * 512 + lane * 8;
        wv[u] = ldg<uint4>(ld.row + min(kk[u], K - 8));
        if (done + u + 1 < total) seg_next(a, t, P, nseg, ld);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (done < total) {
          if (rr[u] != cur) {
#pragma unroll
            for (int b = 0; b < kMaxBatch; ++b) {
              if (b < B) {
                const float v = wave_sum(av[b]);
                if (lane == 0) atomicAdd(&acc[cur * B + b], v);
              }
              av[b] = 0.f;
            }
            cur = rr[u];
          }
          if (kk[u] < K) {
#pragma unroll
            for (int b = 0; b < kMaxBatch; ++b)
              if (b < B) {
                gptr<const float> xr = op.x + (int64_t)b * K + kk[u];
                av[b] = dot8(wv[u], ldg<float4>(xr), ldg<float4>(xr + 4), av[b]);
              }
          }
          ++done;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kMaxBatch; ++b)
      if (b < B) {
        const float v = wave_sum(av[b]);
        if (lane == 0) atomicAdd(&acc[cur * B + b], v);
      }
  }
  __syncthreads();
  gemv_epilogue(a, t, acc, red);
}

// ------------------------------------------------------------------ q/k RMSNorm + RoPE + KV append
// Task (b, g): the G query heads and the key head of kv group g get per-head
// RMSNorm (qk_norm) and rotate-half RoPE at position L_b; q goes to the q
// buffer (fp32), k and v to cache slot L_b of request b (bf16).
__device__ __forceinline__ void rope_task(const KArgs& a, const DevTask& t, const TaskPtrs& P) {
  const int tid0 = tidx();
  const int b = t.a0, g = t.a1, l = t.layer, d = a.d, half = d >> 1, G = a.G;
  const int w = tid0 >> 6, lane = tid0 & 63;
  const int Lb = a.seq_lens[b];
  bool ok = Lb >= 0 && Lb < a.max_seq && Lb / a.P < a.max_pages;
  const int pid = ok ? a.page_table[(int64_t)b * a.max_pages + Lb / a.P] : 0;
  if (!(pid >= 0 && pid < a.n_pages)) ok = false;
  if (!ok && tid0 == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)Lb, (uint32_t)pid);
  const int64_t slot = ok ? ((((int64_t)l * a.n_pages + pid) * a.hkv + g) * a.P + (Lb % a.P)) * d : 0;
  gptr<const float> src = a.qkv + (int64_t)l * a.st_qkv + (int64_t)b * a.hkv * a.Sg + (int64_t)g * a.Sg;
  const bool act = lane < half;
  // angle of pair `lane`: L_b * theta^(-2*lane/d); the product and its
  // reduction to [-pi, pi] are done in fp64 (inverse frequencies are computed
  // on the host in fp64), cos/sin of the reduced angle in fp32
  float cs = 1.f, sn = 0.f;
  if (act) {
    const double ang = (double)(ok ? Lb : 0) * a.inv_freq[lane];
    const double two_pi = 6.283185307179586476925286766559;
    const float red_ang = (float)(ang - two_pi * rint(ang / two_pi));
    sincosf(red_ang, &sn, &cs);
  }
  mark(a, 0);
  for (int hh = w; hh < G + 2; hh += kWaves) {
    const float s0 = src[hh * d + min(lane, half - 1)], s1 = src[hh * d + min(lane, half - 1) + half];
    float x0 = act ? s0 : 0.f;
    float x1 = act ? s1 : 0.f;
    if (hh == G + 1) {  // value head: rounded into the bf16 cache
      if (act && ok) {
        a.v_pool[slot + lane] = f2bf(x0);
        a.v_pool[slot + lane + half] = f2bf(x1);
      }
      continue;
    }
    if (a.qk_norm) {
      gptr<const uint16_t> gq = P.p0, gk = P.p1;
      gptr<const uint16_t> gam = hh < G ? gq : gk;
      const int lc = min(lane, half - 1);
      const float g0 = act ? bf2f(gam[lc]) : 0.f, g1 = act ? bf2f(gam[lc + half]) : 0.f;
      const float ss = wave_sum(x0 * x0 + x1 * x1);
      const float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
      x0 = x0 * inv * g0;
      x1 = x1 * inv * g1;
    }
    const float y0 = x0 * cs - x1 * sn;
    const float y1 = x1 * cs + x0 * sn;
    if (act) {
      if (hh < G) {
        gptr<float> qo = a.q + (int64_t)l * a.st_q + (int64_t)b * a.hq * d + (int64_t)(g * G + hh) * d;
        qo[lane] = y0;
        qo[lane + half] = y1;
      } else if (ok) {
        a.k_pool[slot + lane] = f2bf(y0);
        a.k_pool[slot + lane + half] = f2bf(y1);
      }
    }
  }
}

// ------------------------------------------------------------------ paged attention, one split
// Task (b, g, s): pages [floor(s n_b / S), floor((s+1) n_b / S)) of request b,
// n_b = ceil((L_b + 1) / P); all G query heads of kv group g.  Each row of R
// lanes of a wavefront owns every (8 * 64 / R)-th token of the split (lane i
// of the row holds dims [i D/R, (i+1) D/R): one coalesced key row and value
// row per token), keeps an online-softmax state (max m, sum l, o[d]) per
// head, and the row states are merged with the log-sum-exp rule at the end.
// R = 16 when G <= 4, 32 for G <= 8 (64 registers of q and o either way).
// Key/value rows are double-buffered in registers (the next token's loads
// are in flight while the current one is processed; loads past the split's
// end repeat its last token so the wait counts stay static); the split's
// page ids are staged in LDS first.  Output: per head (m, l, o[d]) in fp32.
template <int D, int R, int GM>
__device__ __forceinline__ void attn_task(const KArgs& a, const DevTask& t, char* lds) {
  const int tid0 = tidx();
  constexpr int DPL = D / R;            // dims per lane
  constexpr int RPW = 64 / R;           // rows per wavefront
  constexpr int TPI = kWaves * RPW;     // tokens per iteration of the workgroup
  using KV = typename std::conditional<DPL == 8, uint4, typename std::conditional<DPL == 4, uint2, uint32_t>::type>::type;
  const int b = t.a0, g = t.a1, s = t.a2, l = t.layer, G = a.G, P = a.P;
  const int w = tid0 >> 6, lane = tid0 & 63, row = lane / R, lr = lane % R;
  const int Lb = a.seq_lens[b];
  const bool ok = Lb >= 0 && Lb < a.max_seq && (Lb / P) < a.max_pages;
  if (!ok && tid0 == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)Lb, 0u);
  const int ntok = ok ? Lb + 1 : 0;
  const int nb = (ntok + P - 1) / P;
  const int j0 = (int)((int64_t)s * nb / a.S_attn), j1 = (int)((int64_t)(s + 1) * nb / a.S_attn);
  const int t0 = j0 * P, t1 = min(j1 * P, ntok);

  int* pids = reinterpret_cast<int*>(lds + kLdsMisc);   // page ids of pages j0..j1-1
  for (int j = j0 + tid0; j < j1; j += kThreads) {
    int pid = a.page_table[(int64_t)b * a.max_pages + j];
    if (pid < 0 || pid >= a.n_pages) {
      report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)pid, (uint32_t)a.n_pages);
      pid = -1;
    }
    pids[j - j0] = pid;
  }
  const float scale = 1.0f / sqrtf((float)D);
  float qv[GM][DPL], ov[GM][DPL], m[GM], lsum[GM];
  gptr<const float> qsrc = a.q + (int64_t)l * a.st_q + (int64_t)b * a.hq * D + (int64_t)g * G * D;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      const float qx = qsrc[min(h, G - 1) * D + lr * DPL + i];
      qv[h][i] = h < G ? qx * scale : 0.f;
      ov[h][i] = 0.f;
    }
  }
  __syncthreads();
  mark(a, 0);
  gptr<const uint16_t> kbase = a.k_pool + ((int64_t)l * a.n_pages * a.hkv + g) * P * D + lr * DPL;
  gptr<const uint16_t> vbase = a.v_pool + ((int64_t)l * a.n_pages * a.hkv + g) * P * D + lr * DPL;
  const int64_t page_stride = (int64_t)a.hkv * P * D;
  // offset of token `tok`, clamped into the split (a bad page reads page 0 and is not used)
  auto offs = [&](int tok) -> int64_t {
    tok = min(tok, t1 - 1);
    const int pid = pids[tok / P - j0];
    return (int64_t)(pid >= 0 ? pid : 0) * page_stride + (int64_t)(tok % P) * D;
  };
  auto good = [&](int tok) { return tok < t1 && pids[tok / P - j0] >= 0; };
  auto process = [&](const KV& kc, const KV& vc) {
    float kf[DPL], vf[DPL];
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kc);
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vc);
#pragma unroll
    for (int i = 0; i < DPL / 2; ++i) {
      kf[2 * i] = bflo(kw[i]); kf[2 * i + 1] = bfhi(kw[i]);
      vf[2 * i] = bflo(vw[i]); vf[2 * i + 1] = bfhi(vw[i]);
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) p = fmaf(qv[h][i], kf[i], p);
        p = row_sum(p);
        if (R == 32) p += __shfl_xor(p, 16);
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
  if (t1 > t0) {
    // `it` is the wavefront's first token of the iteration: uniform over the wavefront
    const int base = t0 + w * RPW;
    int tok = base + row;
    KV k0, v0, k1, v1;
    int64_t o = offs(tok);
    k0 = ldg<KV>(kbase + o);
    v0 = ldg<KV>(vbase + o);
    for (int it = base; it < t1; it += 2 * TPI, tok += 2 * TPI) {
      o = offs(tok + TPI);
      k1 = ldg<KV>(kbase + o);
      v1 = ldg<KV>(vbase + o);
      if (good(tok)) process(k0, v0);
      if (it + TPI >= t1) break;
      o = offs(tok + 2 * TPI);
      k0 = ldg<KV>(kbase + o);
      v0 = ldg<KV>(vbase + o);
      if (good(tok + TPI)) process(k1, v1);
    }
  }
  mark(a, 1);
  // merge the row states of the wavefront (lanes lr, lr+R, ...)
#pragma unroll
  for (int msk = R; msk <= 32; msk <<= 1) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float m2 = __shfl_xor(m[h], msk), l2 = __shfl_xor(lsum[h], msk);
        const float mn = fmaxf(m[h], m2);
        const float a1 = (m[h] == -INFINITY) ? 0.f : __expf(m[h] - mn);
        const float a2 = (m2 == -INFINITY) ? 0.f : __expf(m2 - mn);
        lsum[h] = lsum[h] * a1 + l2 * a2;
#pragma unroll
        for (int i = 0; i < DPL; ++i) {
          const float o2 = __shfl_xor(ov[h][i], msk);
          ov[h][i] = ov[h][i] * a1 + o2 * a2;
        }
        m[h] = mn;
      }
    }
  }
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
  gptr<float> out = a.part + (int64_t)l * a.st_part +
                    (((int64_t)b * a.hkv + g) * a.S_attn + s) * (int64_t)(G * (D + 2));
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
    out[h * (D + 2) + 2 + dd] = O;
    if (dd == 0) { out[h * (D + 2)] = M; out[h * (D + 2) + 1] = L; }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ split combine
// Task (b, g): o = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}, M = max_s m_s.
// The S partial records are staged in LDS first (all loads in flight at once).
__device__ __forceinline__ void combine_task(const KArgs& a, const DevTask& t, char* lds) {
  const int tid0 = tidx();
  const int b = t.a0, g = t.a1, l = t.layer, G = a.G, D = a.d, S = a.S_attn;
  const int rec = G * (D + 2);
  gptr<const float> part = a.part + (int64_t)l * a.st_part + ((int64_t)b * a.hkv + g) * S * (int64_t)rec;
  gptr<float> out = a.attn + (int64_t)l * a.st_q + (int64_t)b * a.hq * D + (int64_t)g * G * D;
  float* st = reinterpret_cast<float*>(lds);
  const int n = S * rec;
  const bool staged = ((n + 63) & ~63) <= kLdsXFloats;
  if (staged) {
    lds_stage<4>(part, reinterpret_cast<char*>(st), n, tid0);
    lds_stage_wait();
  }
  mark(a, 0);
  auto merge = [&](auto at) {
    for (int e = tid0; e < G * D; e += kThreads) {
      const int h = e / D, dd = e - h * D;
      float M = -INFINITY;
      for (int s_ = 0; s_ < S; ++s_) M = fmaxf(M, at(s_ * rec + h * (D + 2)));
      float L = 0.f, O = 0.f;
      for (int s_ = 0; s_ < S; ++s_) {
        const int r0 = s_ * rec + h * (D + 2);
        const float ms = at(r0);
        if (ms != -INFINITY) {
          const float f = __expf(ms - M);
          L = fmaf(at(r0 + 1), f, L);
          O = fmaf(at(r0 + 2 + dd), f, O);
        }
      }
      out[h * D + dd] = L > 0.f ? O / L : 0.f;
    }
  };
  if (staged) merge([&](int i) { return st[i]; });
  else merge([&](int i) { return part[i]; });
  mark(a, 1);
  __syncthreads();
}

// ------------------------------------------------------------------ final argmax
// next_ids[b] = argmax over the LM-head tile partials; ties -> lowest index.
__device__ __forceinline__ void argmax_task(const KArgs& a, char* lds) {
  const int tid0 = tidx();
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  int* redi = reinterpret_cast<int*>(red + kWaves);
  const int w = tid0 >> 6, lane = tid0 & 63;
  for (int b = 0; b < a.B; ++b) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int n = tid0; n < a.T_lm; n += kThreads) {
      const PMax p = a.pmax[b * a.T_lm + n];
      if (p.v > bv || (p.v == bv && p.i < bi)) { bv = p.v; bi = p.i; }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) { red[w] = bv; redi[w] = bi; }
    __syncthreads();
    if (tid0 == 0) {
      for (int i = 1; i < kWaves; ++i)
        if (red[i] > bv || (red[i] == bv && redi[i] < bi)) { bv = red[i]; bi = redi[i]; }
      a.next_ids[b] = (bi == INT_MAX) ? 0 : bi;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ dispatch
// Runs task `task` with the whole workgroup.
// Task t with its resolved weight pointers P (task_ptrs).
__device__ __forceinline__ void run_task(const KArgs& a, const DevTask& t, const TaskPtrs& P) {
  char* lds = g_lds;
  float* red = reinterpret_cast<float*>(lds + kLdsRed);
  const int l = t.layer;
  switch (t.type) {
    case MPK_TASK_EMBED:
      embed_task(a);
      break;
    case MPK_TASK_ATTN_NORM:
      if (l == 0) norm_task(a, a.e, nullptr, a.r, P.p0, a.h, lds, red);
      else
        norm_task(a, a.s + (int64_t)(l - 1) * a.st_bh, a.dn + (int64_t)(l - 1) * a.st_bh, a.r + (int64_t)l * a.st_bh,
                  P.p0, a.h + (int64_t)l * a.st_bh, lds, red);
      break;
    case MPK_TASK_MLP_NORM:
      norm_task(a, a.r + (int64_t)l * a.st_bh, a.o + (int64_t)l * a.st_bh, a.s + (int64_t)l * a.st_bh,
                P.p0, a.h2 + (int64_t)l * a.st_bh, lds, red);
      break;
    case MPK_TASK_FINAL_NORM:
      norm_task(a, a.s + (int64_t)(a.L - 1) * a.st_bh, a.dn + (int64_t)(a.L - 1) * a.st_bh, nullptr, P.p0, a.hf,
                lds, red);
      break;
    case MPK_TASK_QKV:
    case MPK_TASK_OPROJ:
    case MPK_TASK_GATEUP:
    case MPK_TASK_DOWN:
    case MPK_TASK_LMHEAD:
      if (a.B == 1) gemv_b1<8>(a, t, P, lds);
      else gemv_bn(a, t, P, lds);
      break;
    case MPK_TASK_QKNORM_ROPE:
      rope_task(a, t, P);
      break;
    case MPK_TASK_ATTN:
      if (a.d == 128) {
        if (a.G <= 4) attn_task<128, 16, 4>(a, t, lds);
        else attn_task<128, 32, 8>(a, t, lds);
      } else {
        attn_task<64, 16, 8>(a, t, lds);
      }
      break;
    case MPK_TASK_COMBINE:
      combine_task(a, t, lds);
      break;
    case MPK_TASK_ARGMAX:
      argmax_task(a, lds);
      break;
    default:
      break;
  }
}

}  // namespace mpk
