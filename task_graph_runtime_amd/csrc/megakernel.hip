// The persistent decode-step kernel (in-kernel runtime) and the
// kernel-per-operator baseline launcher, for gfx950.
//
// Runtime (MPK summary page, section 2 Q2 and section 4 "Why this launch
// config (Table 1)" and design-space table): the grid holds one workgroup per
// compute unit.  The first workgroups host the schedulers -- four wavefronts
// each, one scheduler per wavefront -- and the rest are workers.  A worker
// pops its ahead-of-time task list in FIFO order and, while a task's
// dependent event has not fired, serves its just-in-time ring.  Events are
// global counters advanced by atomic adds; an event fires when its counter
// reaches counts * epoch (counters are never reset: each step raises the
// target).  The agent whose add fires an event resolves the event's empty
// consumers on the spot and, if the event has JIT consumers, appends it to
// the ring of scheduler (event mod n_sched).  A scheduler pops its ring and
// deals the event's JIT tasks round-robin onto the JIT rings of its workers
// (workers w with w mod n_sched == its index).  Everything exits when the end
// event fires; every wait has a watchdog so that the grid always drains.
#include "tasks.h"

namespace mpk {

namespace {

__device__ __forceinline__ uint32_t ld_relaxed(gptr<const uint32_t> p) {
  return __hip_atomic_load(const_cast<gptr<uint32_t>>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_relaxed64(gptr<const unsigned long long> p) {
  return __hip_atomic_load(const_cast<gptr<unsigned long long>>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_release64(gptr<unsigned long long> p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void acquire_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

__device__ __forceinline__ bool reached(uint32_t cnt, uint32_t target) { return (int32_t)(cnt - target) >= 0; }

// Persistent runtime state (device words, kept across steps):
//   [0, W)            JIT ring head of each worker
//   [W, W+S)          event ring head of each scheduler
//   [W+S, W+2S)       round-robin cursor of each scheduler
//   [W+2S, 2W+2S)     JIT ring tail of each worker (written by its scheduler)
__device__ __forceinline__ gptr<uint32_t> st_jit_head(const KArgs& a) { return a.state; }
__device__ __forceinline__ gptr<uint32_t> st_sched_head(const KArgs& a) { return a.state + a.n_workers; }
__device__ __forceinline__ gptr<uint32_t> st_sched_rr(const KArgs& a) { return a.state + a.n_workers + a.n_sched; }
__device__ __forceinline__ gptr<uint32_t> st_jit_tail(const KArgs& a) { return a.state + a.n_workers + 2 * a.n_sched; }

__device__ __forceinline__ void push_event(const KArgs& a, int e) {
  const int s = e % a.n_sched;
  const uint32_t pos = __hip_atomic_fetch_add(&a.sched_tail[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  st_release64(&a.sched_ring[(int64_t)s * a.sched_cap + (pos & (a.sched_cap - 1))],
               ((unsigned long long)(pos + 1) << 32) | (uint32_t)e);
}

// One trigger of event e by the calling thread (after the producer's writes
// are complete for the whole workgroup).  If this add fires the event, its
// empty consumers are resolved here (each triggers its own event) and JIT
// consumers are handed to a scheduler.
__device__ __forceinline__ void trigger(const KArgs& a, uint32_t epoch, int e) {
  const uint32_t old = __hip_atomic_fetch_add(&a.ev_cnt[e], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  const DevEvent ev = a.events[e];
  if (old + 1u != ev.counts * epoch) return;
  acquire_fence();
  if (ev.flags & MPK_EVENT_HAS_EMPTY) {
    for (int t = ev.first; t <= ev.last; ++t) {
      const int f = a.tasks[t].trig;
      const uint32_t o2 = __hip_atomic_fetch_add(&a.ev_cnt[f], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const DevEvent fe = a.events[f];
      if (o2 + 1u == fe.counts * epoch && (fe.flags & MPK_EVENT_HAS_JIT)) push_event(a, f);
    }
  }
  if (ev.flags & MPK_EVENT_HAS_JIT) push_event(a, e);
}

enum { CMD_EXIT = 0, CMD_JIT = 1, CMD_AOT = 2 };

__device__ __forceinline__ void worker_loop(gptr<const KArgs> ap, uint32_t epoch, uint64_t timeout, int w) {
  const KArgs a = *ap;
  int& s_cmd = reinterpret_cast<int*>(g_lds + kLdsCtl)[0];
  int& s_task = reinterpret_cast<int*>(g_lds + kLdsCtl)[1];
  const int tid = threadIdx.x;
  uint32_t jit_head = 0;
  if (tid == 0) jit_head = st_jit_head(a)[w];
  int i = (int)a.aot_off[w];
  const int iend = (int)a.aot_off[w + 1];
  const uint32_t end_target = a.events[a.end_event].counts * epoch;
  gptr<const unsigned long long> ring = a.jit_ring + (int64_t)w * a.jit_cap;
  gptr<TraceRec> trace = a.trace ? a.trace + (int64_t)w * a.trace_cap : nullptr;
  int n_trace = 0;
  uint64_t t_wait = 0, t_start = 0;
  while (true) {
    if (tid == 0) {
      int cmd = CMD_EXIT, task = -1;
      const long long t0 = wall_clock64();
      t_wait = (uint64_t)t0;
      int dep = -1;
      uint32_t target = 0, cnt = 0;
      if (i < iend) {
        task = (int)a.aot_tasks[i];
        dep = a.tasks[task].dep;
        target = a.events[dep].counts * epoch;
      }
      while (true) {
        const unsigned long long slot = ld_relaxed64(&ring[jit_head & (a.jit_cap - 1)]);
        if ((uint32_t)(slot >> 32) == jit_head + 1u) {
          task = (int)(uint32_t)slot;
          ++jit_head;
          cmd = CMD_JIT;
          break;
        }
        if (i < iend) {
          cnt = ld_relaxed(&a.ev_cnt[dep]);
          if (reached(cnt, target)) { cmd = CMD_AOT; break; }
        } else if (reached(ld_relaxed(&a.ev_cnt[a.end_event]), end_target)) {
          cmd = CMD_EXIT;
          break;
        }
        if (ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code)) != 0u) { cmd = CMD_EXIT; break; }
        if ((uint64_t)(wall_clock64() - t0) > timeout) {
          report(a, MPK_ERR_TIMEOUT, task, i < iend ? dep : a.end_event, i < iend ? cnt : 0u,
                 i < iend ? target : end_target);
          cmd = CMD_EXIT;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (cmd != CMD_EXIT) acquire_fence();
      t_start = (uint64_t)wall_clock64();
      s_cmd = cmd;
      s_task = task;
    }
    __syncthreads();
    const int cmd = s_cmd, task = s_task;
    __syncthreads();
    if (cmd == CMD_EXIT) break;
    run_task(ap, task);
    __syncthreads();
    if (tid == 0) {
      if (trace && n_trace < a.trace_cap)
        trace[n_trace++] = TraceRec{task, w, t_wait, t_start, (uint64_t)wall_clock64()};
      trigger(a, epoch, a.tasks[task].trig);
    }
    if (cmd == CMD_AOT) ++i;
  }
  if (tid == 0) {
    st_jit_head(a)[w] = jit_head;
    if (trace) a.trace_count[w] = (uint32_t)n_trace;
  }
}

// One scheduler per wavefront (lane 0 does the work).
__device__ __forceinline__ void scheduler_loop(const KArgs& a, uint32_t epoch, uint64_t timeout, int s) {
  if ((threadIdx.x & 63) != 0) return;
  uint32_t head = st_sched_head(a)[s], rr = st_sched_rr(a)[s];
  const int n_sub = (a.n_workers - s + a.n_sched - 1) / a.n_sched;
  gptr<uint32_t> tails = st_jit_tail(a);
  gptr<const unsigned long long> ring = a.sched_ring + (int64_t)s * a.sched_cap;
  const uint32_t end_target = a.events[a.end_event].counts * epoch;
  long long t0 = wall_clock64();
  while (true) {
    const unsigned long long slot = ld_relaxed64(&ring[head & (a.sched_cap - 1)]);
    if ((uint32_t)(slot >> 32) == head + 1u) {
      acquire_fence();
      const int e = (int)(uint32_t)slot;
      ++head;
      const DevEvent ev = a.events[e];
      for (int t = ev.first; t <= ev.last; ++t) {
        const int w = s + (int)(rr % (uint32_t)n_sub) * a.n_sched;
        ++rr;
        const uint32_t tail = tails[w];
        st_release64(&a.jit_ring[(int64_t)w * a.jit_cap + (tail & (a.jit_cap - 1))],
                     ((unsigned long long)(tail + 1u) << 32) | (uint32_t)t);
        tails[w] = tail + 1u;
      }
      t0 = wall_clock64();
      continue;
    }
    if (reached(ld_relaxed(&a.ev_cnt[a.end_event]), end_target)) break;
    if (ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code)) != 0u) break;
    if ((uint64_t)(wall_clock64() - t0) > timeout) {
      report(a, MPK_ERR_TIMEOUT, -1, a.end_event, 0u, end_target);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  st_sched_head(a)[s] = head;
  st_sched_rr(a)[s] = rr;
}

}  // namespace

__global__ void __launch_bounds__(kThreads) mpk_megakernel(const KArgs* __restrict__ args, uint32_t epoch,
                                                            uint64_t timeout) {
  gptr<const KArgs> ap = (gptr<const KArgs>)(args);
  const KArgs a = *ap;
  if (ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code)) != 0u) return;  // poisoned graph
  const int wg = blockIdx.x;
  if (wg < a.n_sched_wgs) {
    const int s = wg * 4 + (int)(threadIdx.x >> 6);
    if ((threadIdx.x >> 6) < 4 && s < a.n_sched) scheduler_loop(a, epoch, timeout, s);
    return;
  }
  const int w = wg - a.n_sched_wgs;
  if (w < a.n_workers) worker_loop(ap, epoch, timeout, w);
}

// Kernel-per-operator baseline: workgroup i runs task list[i], no events.
__global__ void __launch_bounds__(kThreads) mpk_baseline_op(const KArgs* __restrict__ ap, const int32_t* list) {
  run_task((gptr<const KArgs>)(ap), list[blockIdx.x]);
}

// Body timing: one workgroup runs one task and adds its wall-clock ticks to *out.
__global__ void __launch_bounds__(kThreads) mpk_time_task_kernel(const KArgs* __restrict__ ap, int task,
                                                                  unsigned long long* out) {
  __syncthreads();
  const unsigned long long t0 = wall_clock64();
  run_task((gptr<const KArgs>)(ap), task);
  __syncthreads();
  if (threadIdx.x == 0) *out += wall_clock64() - t0;
}

hipError_t launch_time_task(const KArgs* d_args, int task, unsigned long long* out, hipStream_t stream) {
  hipLaunchKernelGGL(mpk_time_task_kernel, dim3(1), dim3(kThreads), 0, stream, d_args, task, out);
  return hipGetLastError();
}

hipError_t launch_megakernel(const KArgs* d_args, uint32_t epoch, uint64_t timeout, int grid, hipStream_t stream) {
  void* args[] = {&d_args, &epoch, &timeout};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&mpk_megakernel), dim3(grid), dim3(kThreads),
                                    args, 0, stream);
}

hipError_t launch_baseline_op(const KArgs* d_args, const int32_t* list, int count, hipStream_t stream) {
  hipLaunchKernelGGL(mpk_baseline_op, dim3(count), dim3(kThreads), 0, stream, d_args, list);
  return hipGetLastError();
}

}  // namespace mpk
