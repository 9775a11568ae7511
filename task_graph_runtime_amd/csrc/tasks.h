// Task bodies of the decode step (HIP, gfx950).  Each body is executed by one
// whole 512-thread workgroup; the persistent mega-kernel and the
// kernel-per-operator baseline run the same functions.
//
// Operations (MPK summary page, section 3 "Target operation, shapes &
// precision contract"): projection tiles read bf16 weights and accumulate in
// fp32.  Activations passed between tasks stay fp32 (the page's bf16 task
// outputs, compounded over 28-64 layers, drift past the 2e-2 logit bound
// against the fp32 forward); only weights and the KV cache are bf16;
// attention is paged decode attention of one new query per request against
// its KV pages.  The decoder layer around them is the Qwen3 layer (RMSNorm,
// per-head q/k RMSNorm, rotate-half RoPE, GQA, SwiGLU).
#pragma once

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>

#include "mpk.h"
#include "rt.h"

namespace mpk {

// ------------------------------------------------------------------ helpers
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

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ float4 ldf4(const float* p) { return *reinterpret_cast<const float4*>(p); }

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
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Sum over the workgroup; `red` is kWaves floats of LDS.  All threads call it.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
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
  int32_t prev = atomicCAS(&a.status->code, 0, code);
  if (prev == 0) {
    a.status->wg = (int32_t)blockIdx.x;
    a.status->task = task;
    a.status->event = event;
    a.status->counter = counter;
    a.status->target = target;
    __threadfence();
  }
}

// ------------------------------------------------------------------ embedding
__device__ void embed_task(const KArgs& a) {
  for (int b = 0; b < a.B; ++b) {
    int id = a.token_ids[b];
    if (id < 0 || id >= a.V) {
      if (threadIdx.x == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)id, (uint32_t)a.V);
      id = 0;
    }
    const uint16_t* row = a.embed + (int64_t)id * a.H;
    for (int i = threadIdx.x; i < a.H; i += kThreads) a.e[(int64_t)b * a.H + i] = bf2f(row[i]);
  }
}

// ------------------------------------------------------------------ residual add + RMSNorm
// res = x + y (y optional), stored when `res` is given; out = RMSNorm(res) * gamma.
__device__ void norm_task(const KArgs& a, const float* x, const float* y, float* res, const uint16_t* gamma,
                          float* out, float* red) {
  const int H = a.H;
  for (int b = 0; b < a.B; ++b) {
    float v[kMaxHidden / kThreads];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxHidden / kThreads; ++j) {
      int i = threadIdx.x + j * kThreads;
      v[j] = 0.f;
      if (i < H) {
        float t = x[(int64_t)b * H + i];
        if (y) t += y[(int64_t)b * H + i];
        v[j] = t;
        ss = fmaf(t, t, ss);
        if (res) res[(int64_t)b * H + i] = t;
      }
    }
    ss = block_sum(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)H + a.eps);
#pragma unroll
    for (int j = 0; j < kMaxHidden / kThreads; ++j) {
      int i = threadIdx.x + j * kThreads;
      if (i < H) out[(int64_t)b * H + i] = v[j] * inv * bf2f(gamma[i]);
    }
  }
}

// ------------------------------------------------------------------ projection tiles
// Row r of the tile's weight rows (output columns [lo, hi); gate/up tiles
// interleave gate row and up row of each column).
__device__ __forceinline__ const uint16_t* gemv_row(const KArgs& a, int type, int l, int lo, int r) {
  switch (type) {
    case MPK_TASK_QKV: {
      const uint16_t* const* W = a.wl + (int64_t)l * LAYER_PTRS;
      const int col = lo + r, g = col / a.Sg, Gd = a.G * a.d;
      int off = col - g * a.Sg;
      if (off < Gd) return W[W_Q] + (int64_t)(g * Gd + off) * a.H;
      off -= Gd;
      if (off < a.d) return W[W_K] + (int64_t)(g * a.d + off) * a.H;
      off -= a.d;
      return W[W_V] + (int64_t)(g * a.d + off) * a.H;
    }
    case MPK_TASK_OPROJ:
      return a.wl[(int64_t)l * LAYER_PTRS + W_O] + (int64_t)(lo + r) * (a.hq * a.d);
    case MPK_TASK_GATEUP:
      return a.wl[(int64_t)l * LAYER_PTRS + ((r & 1) ? W_UP : W_GATE)] + (int64_t)(lo + (r >> 1)) * a.H;
    case MPK_TASK_DOWN:
      return a.wl[(int64_t)l * LAYER_PTRS + W_DOWN] + (int64_t)(lo + r) * a.F;
    default:
      return (a.lm_head ? a.lm_head : a.embed) + (int64_t)(lo + r) * a.H;
  }
}

// y[b, n] = sum_k x[b, k] W[n, k] for the tile's columns.  The tile's weight
// rows are cut into 1 KB segments (64 lanes x 8 bf16, 16-byte loads); each
// wavefront streams a contiguous run of segments, keeps one fp32 partial per
// batch row, reduces it across the wavefront when the row changes and adds it
// into an LDS accumulator.  BT = 1 (batch 1) or kMaxBatch (batch 2..16).
template <int BT>
__device__ void gemv_task(const KArgs& a, const DevTask& t, float* acc, float* red) {
  const int type = t.type, l = t.layer, lo = t.a0, hi = t.a1;
  const int B = a.B;
  int K, rpc = 1;
  const float* x;
  switch (type) {
    case MPK_TASK_QKV: K = a.H; x = a.h + (int64_t)l * a.st_bh; break;
    case MPK_TASK_OPROJ: K = a.hq * a.d; x = a.attn + (int64_t)l * a.st_q; break;
    case MPK_TASK_GATEUP: K = a.H; x = a.h2 + (int64_t)l * a.st_bh; rpc = 2; break;
    case MPK_TASK_DOWN: K = a.F; x = a.a + (int64_t)l * a.st_a; break;
    default: K = a.H; x = a.hf; break;
  }
  const int ncol = hi - lo, nrows = ncol * rpc;
  for (int i = threadIdx.x; i < nrows * B; i += kThreads) acc[i] = 0.f;
  __syncthreads();

  const int nseg = (K + 511) >> 9;
  const int S = nrows * nseg;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s_beg = (int)((int64_t)S * w / kWaves), s_end = (int)((int64_t)S * (w + 1) / kWaves);
  constexpr int U = (BT == 1) ? 8 : 4;
  float av[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) av[b] = 0.f;
  int cur = -1;
  auto flush = [&]() {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      if (b < B) {
        float v = wave_sum(av[b]);
        if (lane == 0) atomicAdd(&acc[cur * B + b], v);
      }
      av[b] = 0.f;
    }
  };
  for (int s0 = s_beg; s0 < s_end; s0 += U) {
    uint4 wv[U];
    float4 xa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      wv[u] = make_uint4(0, 0, 0, 0);
      xa[u] = xb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < s_end) {
        const int r = s / nseg;
        const int k = (s - r * nseg) * 512 + lane * 8;
        if (k < K) {
          wv[u] = ld16(gemv_row(a, type, l, lo, r) + k);
          if (BT == 1) { xa[u] = ldf4(x + k); xb[u] = ldf4(x + k + 4); }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u;
      if (s < s_end) {
        const int r = s / nseg;
        const int k = (s - r * nseg) * 512 + lane * 8;
        if (r != cur) {
          if (cur >= 0) flush();
          cur = r;
        }
        if (k < K) {
          if (BT == 1) {
            av[0] = dot8(wv[u], xa[u], xb[u], av[0]);
          } else {
#pragma unroll
            for (int b = 0; b < BT; ++b)
              if (b < B) {
                const float* xr = x + (int64_t)b * K + k;
                av[b] = dot8(wv[u], ldf4(xr), ldf4(xr + 4), av[b]);
              }
          }
        }
      }
    }
  }
  if (cur >= 0) flush();
  __syncthreads();

  // epilogue
  switch (type) {
    case MPK_TASK_QKV: {
      const int ld = a.hkv * a.Sg;
      float* out = a.qkv + (int64_t)l * a.st_qkv;
      for (int i = threadIdx.x; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        out[(int64_t)b * ld + lo + c] = acc[c * B + b];
      }
      break;
    }
    case MPK_TASK_OPROJ:
    case MPK_TASK_DOWN: {
      float* out = (type == MPK_TASK_OPROJ ? a.o : a.dn) + (int64_t)l * a.st_bh;
      for (int i = threadIdx.x; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        out[(int64_t)b * a.H + lo + c] = acc[c * B + b];
      }
      break;
    }
    case MPK_TASK_GATEUP: {
      float* out = a.a + (int64_t)l * a.st_a;
      for (int i = threadIdx.x; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        float g = acc[(2 * c) * B + b], u = acc[(2 * c + 1) * B + b];
        out[(int64_t)b * a.F + lo + c] = g / (1.0f + expf(-g)) * u;
      }
      break;
    }
    default: {  // LM head: fp32 logits and the tile's (max, argmax) per request
      for (int i = threadIdx.x; i < ncol * B; i += kThreads) {
        int b = i / ncol, c = i - b * ncol;
        a.logits[(int64_t)b * a.V + lo + c] = acc[c * B + b];
      }
      int* redi = reinterpret_cast<int*>(red + kWaves);
      for (int b = 0; b < B; ++b) {
        float bv = -INFINITY;
        int bi = INT_MAX;
        for (int c = threadIdx.x; c < ncol; c += kThreads) {
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
        if (threadIdx.x == 0) {
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

// ------------------------------------------------------------------ q/k RMSNorm + RoPE + KV append
// Task (b, g): the G query heads and the key head of kv group g get per-head
// RMSNorm (qk_norm) and rotate-half RoPE at position L_b; q goes to the q
// buffer (fp32), k and v to cache slot L_b of request b.
__device__ void rope_task(const KArgs& a, const DevTask& t) {
  const int b = t.a0, g = t.a1, l = t.layer, d = a.d, half = d >> 1, G = a.G;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int Lb = a.seq_lens[b];
  bool ok = Lb >= 0 && Lb < a.max_seq && Lb / a.P < a.max_pages;
  int pid = ok ? a.page_table[(int64_t)b * a.max_pages + Lb / a.P] : 0;
  if (!(pid >= 0 && pid < a.n_pages)) ok = false;
  if (!ok && threadIdx.x == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)Lb, (uint32_t)pid);
  const int64_t slot = ok ? ((((int64_t)l * a.n_pages + pid) * a.hkv + g) * a.P + (Lb % a.P)) * d : 0;
  const float* src = a.qkv + (int64_t)l * a.st_qkv + (int64_t)b * a.hkv * a.Sg + (int64_t)g * a.Sg;
  const uint16_t* const* W = a.wl + (int64_t)l * LAYER_PTRS;
  const bool act = lane < half;
  // angle of pair `lane`: L_b * theta^(-2*lane/d), in double
  float cs = 1.f, sn = 0.f;
  if (act) {
    double ang = (double)(ok ? Lb : 0) * pow((double)a.theta, -2.0 * (double)lane / (double)d);
    cs = (float)cos(ang);
    sn = (float)sin(ang);
  }
  for (int hh = w; hh < G + 2; hh += kWaves) {
    float x0 = act ? src[hh * d + lane] : 0.f;
    float x1 = act ? src[hh * d + lane + half] : 0.f;
    if (hh == G + 1) {  // value head: rounded into the bf16 cache
      if (act && ok) {
        a.v_pool[slot + lane] = f2bf(x0);
        a.v_pool[slot + lane + half] = f2bf(x1);
      }
      continue;
    }
    if (a.qk_norm) {
      float ss = wave_sum(x0 * x0 + x1 * x1);
      float inv = 1.0f / sqrtf(ss / (float)d + a.eps);
      const uint16_t* gam = W[hh < G ? W_Q_NORM : W_K_NORM];
      if (act) {
        x0 = x0 * inv * bf2f(gam[lane]);
        x1 = x1 * inv * bf2f(gam[lane + half]);
      }
    }
    float y0 = x0 * cs - x1 * sn;
    float y1 = x1 * cs + x0 * sn;
    if (act) {
      if (hh < G) {
        float* qo = a.q + (int64_t)l * a.st_q + (int64_t)b * a.hq * d + (int64_t)(g * G + hh) * d;
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
// n_b = ceil((L_b + 1) / P); all G query heads of kv group g.  Each 16-lane
// row of a wavefront owns every 32nd token of the split (lane i of the row
// holds dims [8i, 8i+8) of d=128, or 4 dims of d=64), keeps an online-softmax
// state (max m, sum l, o[d]) per head, and the 32 row states are merged with
// the log-sum-exp rule at the end.  Output: per head (m, l, o[d]) in fp32.
template <int D>
__device__ void attn_task(const KArgs& a, const DevTask& t, float* lds) {
  constexpr int DPL = D / 16;  // dims per lane
  constexpr int GM = 8;        // max query heads per kv head
  const int b = t.a0, g = t.a1, s = t.a2, l = t.layer, G = a.G, P = a.P;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, row = lane >> 4, lr = lane & 15;
  const int Lb = a.seq_lens[b];
  const bool ok = Lb >= 0 && Lb < a.max_seq && (Lb / P) < a.max_pages;
  if (!ok && threadIdx.x == 0) report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)Lb, 0u);
  const int ntok = ok ? Lb + 1 : 0;
  const int nb = (ntok + P - 1) / P;
  const int j0 = (int)((int64_t)s * nb / a.S_attn), j1 = (int)((int64_t)(s + 1) * nb / a.S_attn);
  const int t0 = j0 * P, t1 = min(j1 * P, ntok);

  const float scale = 1.0f / sqrtf((float)D);
  float qv[GM][DPL], ov[GM][DPL], m[GM], lsum[GM];
  const float* qsrc = a.q + (int64_t)l * a.st_q + (int64_t)b * a.hq * D + (int64_t)g * G * D;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      qv[h][i] = h < G ? qsrc[h * D + lr * DPL + i] * scale : 0.f;
      ov[h][i] = 0.f;
    }
  }
  const int64_t head_base = ((int64_t)l * a.n_pages * a.hkv + g) * P * D;  // + pid * hkv * P * D
  for (int tok = t0 + w * 4 + row; tok < t1; tok += 32) {
    int pid = a.page_table[(int64_t)b * a.max_pages + tok / P];
    if (pid < 0 || pid >= a.n_pages) {
      report(a, MPK_ERR_INVALID_ARG, -1, -1, (uint32_t)pid, (uint32_t)a.n_pages);
      continue;
    }
    const int64_t off = head_base + (int64_t)pid * a.hkv * P * D + (int64_t)(tok % P) * D + lr * DPL;
    float kf[DPL], vf[DPL];
    if constexpr (DPL == 8) {
      uint4 kk = ld16(a.k_pool + off), vv = ld16(a.v_pool + off);
      kf[0] = bflo(kk.x); kf[1] = bfhi(kk.x); kf[2] = bflo(kk.y); kf[3] = bfhi(kk.y);
      kf[4] = bflo(kk.z); kf[5] = bfhi(kk.z); kf[6] = bflo(kk.w); kf[7] = bfhi(kk.w);
      vf[0] = bflo(vv.x); vf[1] = bfhi(vv.x); vf[2] = bflo(vv.y); vf[3] = bfhi(vv.y);
      vf[4] = bflo(vv.z); vf[5] = bfhi(vv.z); vf[6] = bflo(vv.w); vf[7] = bfhi(vv.w);
    } else {
      uint2 kk = *reinterpret_cast<const uint2*>(a.k_pool + off);
      uint2 vv = *reinterpret_cast<const uint2*>(a.v_pool + off);
      kf[0] = bflo(kk.x); kf[1] = bfhi(kk.x); kf[2] = bflo(kk.y); kf[3] = bfhi(kk.y);
      vf[0] = bflo(vv.x); vf[1] = bfhi(vv.x); vf[2] = bflo(vv.y); vf[3] = bfhi(vv.y);
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < DPL; ++i) p = fmaf(qv[h][i], kf[i], p);
        p = row_sum(p);
        const float mn = fmaxf(m[h], p);
        const float al = expf(m[h] - mn);
        const float e = expf(p - mn);
        lsum[h] = fmaf(lsum[h], al, e);
#pragma unroll
        for (int i = 0; i < DPL; ++i) ov[h][i] = fmaf(ov[h][i], al, e * vf[i]);
        m[h] = mn;
      }
    }
  }
  // merge the four row states of the wavefront (lanes lr, lr+16, lr+32, lr+48)
#pragma unroll
  for (int msk = 16; msk <= 32; msk <<= 1) {
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float m2 = __shfl_xor(m[h], msk), l2 = __shfl_xor(lsum[h], msk);
        const float mn = fmaxf(m[h], m2);
        const float a1 = (m[h] == -INFINITY) ? 0.f : expf(m[h] - mn);
        const float a2 = (m2 == -INFINITY) ? 0.f : expf(m2 - mn);
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
  float* st = lds;  // [kWaves][G][D + 2]
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
  float* out = a.part + (int64_t)l * a.st_part +
               (((int64_t)b * a.hkv + g) * a.S_attn + s) * (int64_t)(G * (D + 2));
  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const int h = e / D, dd = e - h * D;
    float M = -INFINITY;
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, st[(ww * G + h) * (D + 2)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int ww = 0; ww < kWaves; ++ww) {
        const float* p = st + (ww * G + h) * (D + 2);
        if (p[0] != -INFINITY) {
          const float f = expf(p[0] - M);
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
__device__ void combine_task(const KArgs& a, const DevTask& t) {
  const int b = t.a0, g = t.a1, l = t.layer, G = a.G, D = a.d, S = a.S_attn;
  const float* part = a.part + (int64_t)l * a.st_part + ((int64_t)b * a.hkv + g) * S * (int64_t)(G * (D + 2));
  float* out = a.attn + (int64_t)l * a.st_q + (int64_t)b * a.hq * D + (int64_t)g * G * D;
  for (int e = threadIdx.x; e < G * D; e += kThreads) {
    const int h = e / D, dd = e - h * D;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part[(int64_t)s * G * (D + 2) + h * (D + 2)]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = part + (int64_t)s * G * (D + 2) + h * (D + 2);
      if (p[0] != -INFINITY) {
        const float f = expf(p[0] - M);
        L = fmaf(p[1], f, L);
        O = fmaf(p[2 + dd], f, O);
      }
    }
    out[h * D + dd] = L > 0.f ? O / L : 0.f;
  }
}

// ------------------------------------------------------------------ final argmax
__device__ void argmax_task(const KArgs& a) {
  const int b = threadIdx.x;
  if (b < a.B) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int n = 0; n < a.T_lm; ++n) {
      PMax p = a.pmax[b * a.T_lm + n];
      if (p.v > bv || (p.v == bv && p.i < bi)) { bv = p.v; bi = p.i; }
    }
    a.next_ids[b] = (bi == INT_MAX) ? 0 : bi;
  }
}

// ------------------------------------------------------------------ dispatch
constexpr int kLdsBytes = 96 * 1024;  // > 80 KB so only one workgroup fits a compute unit

__device__ __forceinline__ void run_task(const KArgs& a, const DevTask& t, char* lds) {
  float* f = reinterpret_cast<float*>(lds);
  float* red = f + (kLdsBytes / 4 - 64);  // reduction scratch at the top
  const int l = t.layer;
  switch (t.type) {
    case MPK_TASK_EMBED:
      embed_task(a);
      break;
    case MPK_TASK_ATTN_NORM:
      if (l == 0) norm_task(a, a.e, nullptr, a.r, a.wl[W_IN_NORM], a.h, red);
      else
        norm_task(a, a.s + (int64_t)(l - 1) * a.st_bh, a.dn + (int64_t)(l - 1) * a.st_bh, a.r + (int64_t)l * a.st_bh,
                  a.wl[(int64_t)l * LAYER_PTRS + W_IN_NORM], a.h + (int64_t)l * a.st_bh, red);
      break;
    case MPK_TASK_MLP_NORM:
      norm_task(a, a.r + (int64_t)l * a.st_bh, a.o + (int64_t)l * a.st_bh, a.s + (int64_t)l * a.st_bh,
                a.wl[(int64_t)l * LAYER_PTRS + W_POST_NORM], a.h2 + (int64_t)l * a.st_bh, red);
      break;
    case MPK_TASK_FINAL_NORM:
      norm_task(a, a.s + (int64_t)(a.L - 1) * a.st_bh, a.dn + (int64_t)(a.L - 1) * a.st_bh, nullptr, a.final_norm,
                a.hf, red);
      break;
    case MPK_TASK_QKV:
    case MPK_TASK_OPROJ:
    case MPK_TASK_GATEUP:
    case MPK_TASK_DOWN:
    case MPK_TASK_LMHEAD:
      if (a.B == 1) gemv_task<1>(a, t, f, red);
      else gemv_task<kMaxBatch>(a, t, f, red);
      break;
    case MPK_TASK_QKNORM_ROPE:
      rope_task(a, t);
      break;
    case MPK_TASK_ATTN:
      if (a.d == 128) attn_task<128>(a, t, f);
      else attn_task<64>(a, t, f);
      break;
    case MPK_TASK_COMBINE:
      combine_task(a, t);
      break;
    case MPK_TASK_ARGMAX:
      argmax_task(a);
      break;
    default:
      break;
  }
}

}  // namespace mpk
