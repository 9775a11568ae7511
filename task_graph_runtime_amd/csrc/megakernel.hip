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
// consumers on the spot and, if the event has JIT consumers, appends its
// tasks, one chunk per scheduler segment of worker positions they take, to
// the rings of consecutive schedulers.  A scheduler pops its ring and writes
// a chunk's tasks onto the JIT rings of the workers at their positions (its
// workers are those w with w mod n_sched == its index).  Everything exits
// when the end
// event fires; every wait has a watchdog so that the grid always drains.
#include "tasks.h"

namespace mpk {

namespace {

// Kernel arguments live in the constant kernel-argument segment.
#if defined(__HIP_DEVICE_COMPILE__)
using kptr = const __attribute__((address_space(4))) KArgs*;
#else
using kptr = const KArgs*;
#endif

__device__ __forceinline__ uint32_t ld_relaxed(gptr<const uint32_t> p) {
  return __hip_atomic_load(const_cast<gptr<uint32_t>>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_relaxed64(gptr<const unsigned long long> p) {
  return __hip_atomic_load(const_cast<gptr<unsigned long long>>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed64(gptr<unsigned long long> p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


__device__ __forceinline__ bool reached(uint32_t cnt, uint32_t target) { return (int32_t)(cnt - target) >= 0; }

// Persistent runtime state (device words, kept across steps):
//   [0, W)            JIT ring head of each worker
//   [W, W+S)          event ring head of each scheduler
//   [W+S, 2W+S)       JIT ring tail of each worker (written by its scheduler)
__device__ __forceinline__ gptr<uint32_t> st_jit_head(const KArgs& a) { return a.state; }
__device__ __forceinline__ gptr<uint32_t> st_sched_head(const KArgs& a) { return a.state + a.n_workers; }
__device__ __forceinline__ gptr<uint32_t> st_jit_tail(const KArgs& a) { return a.state + a.n_workers + a.n_sched; }

// JIT placement by worker position.  Position p in [0, W) is worker
// (p / n_sub) + S (p mod n_sub), the (p mod n_sub)-th worker of scheduler
// p / n_sub (n_sub = W / S).  The tasks of JIT event e take consecutive
// positions from its start P_e (flags bits 16..31; the host sets P_e to the
// running count of JIT tasks in event order, mod W, so the events of a
// layer, which fire together, fill the workers one task each before any
// worker gets a second).  The event is handed over as one chunk per
// scheduler segment its positions cross: chunk c to scheduler
// (P_e / n_sub + c) mod S, which writes each of the chunk's tasks into the
// ring of the worker at its position.
__device__ __forceinline__ int jit_sub(const KArgs& a) { return a.n_workers / a.n_sched; }
__device__ __forceinline__ int jit_chunks(const KArgs& a, const DevEvent& ev) {
  const int P = (int)(ev.flags >> 16), n = jit_sub(a);
  return (P + ev.last - ev.first) / n - P / n + 1;
}
__device__ __forceinline__ void push_chunk(const KArgs& a, int e, const DevEvent& ev, int c) {
  const int s = (int)(((ev.flags >> 16) / (uint32_t)jit_sub(a) + (uint32_t)c) % (uint32_t)a.n_sched);
  const uint32_t pos = __hip_atomic_fetch_add(&a.sched_tail[s], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  st_relaxed64(&a.sched_ring[(int64_t)s * a.sched_cap + (pos & (a.sched_cap - 1))],
               ((unsigned long long)(pos + 1) << 32) | ((uint32_t)c << kJitEventBits) | (uint32_t)e);
}

// One arrival at event e by task `task` (linear index); q: the quota of
// its sub-counter (task mod kEvSub) when e is two-level (see rt.h).  True
// when this arrival fires the event.
__device__ __forceinline__ bool arrive(const KArgs& a, uint32_t epoch, int e, const DevEvent& ev, int task,
                                       uint32_t q) {
  if (ev.flags & kEvSole) return true;
  if (ev.flags & kEvTwoLevel) {
    const uint32_t o = __hip_atomic_fetch_add(&a.ev_sub[(int64_t)e * kEvSub + (task & (kEvSub - 1))], 1u,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (o + 1u != q * epoch) return false;
  }
  const uint32_t o = __hip_atomic_fetch_add(&a.ev_cnt[e], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return o + 1u == ev.counts * epoch;
}

// The arrival of empty task t (linear index) at its triggering event; when
// that fires the event, its JIT consumers are handed to the schedulers.
// True when the arrival fired an event that has empty consumers, whose
// record is then in *fe_out.
__device__ __forceinline__ bool arrive_empty(const KArgs& a, uint32_t epoch, int t, int* f_out, DevEvent* fe_out) {
  const int f = a.tasks[t].trig;
  const DevEvent fe = a.events[f];
  const uint32_t qf = (fe.flags & kEvTwoLevel) ? a.ev_quota[(int64_t)f * kEvSub + (t & (kEvSub - 1))] : 0u;
  if (!arrive(a, epoch, f, fe, t, qf)) return false;
  if (fe.flags & MPK_EVENT_HAS_JIT)
    for (int c = 0; c < jit_chunks(a, fe); ++c) push_chunk(a, f, fe, c);
  *f_out = f;
  *fe_out = fe;
  return (fe.flags & MPK_EVENT_HAS_EMPTY) != 0;
}

// One trigger of event e by task `task`, run by wavefront 0 of a workgroup
// whose stores for the trigger are complete (every wavefront waited for them
// before a barrier); q: its sub-counter quota (arrive).  Lane 0 arrives; if
// that fires the event, its empty consumers are resolved here, one lane each
// (each empty task arrives at its own event), and the fired events with JIT
// consumers are handed to the schedulers.  An empty task whose arrival fires
// an event with empty consumers of its own (a graph built without fusion:
// fan-out empties feeding fan-in empties) resolves those in the same lane,
// one after another; the host admits no deeper chain.  No cache maintenance
// is needed: the data the events guard is accessed agent-coherently (see
// tasks.h), the counters atomically.
__device__ __forceinline__ void trigger(const KArgs& a, uint32_t epoch, int e, const DevEvent& ev, int task,
                                        uint32_t q) {
  const int lane = threadIdx.x & 63;
  int fired = 0;
  if (lane == 0) fired = arrive(a, epoch, e, ev, task, q);
  if (!__shfl(fired, 0)) return;
  if (ev.flags & MPK_EVENT_HAS_EMPTY) {
    for (int t0 = ev.first; t0 <= ev.last; t0 += 64) {
      const int t = t0 + lane;
      int f;
      DevEvent fe;
      if (t <= ev.last && arrive_empty(a, epoch, t, &f, &fe)) {
        int f2;
        DevEvent fe2;
        for (int t2 = fe.first; t2 <= fe.last; ++t2) (void)arrive_empty(a, epoch, t2, &f2, &fe2);
      }
    }
  }
  if (ev.flags & MPK_EVENT_HAS_JIT)
    for (int c = lane; c < jit_chunks(a, ev); c += 64) push_chunk(a, e, ev, c);
}

enum { CMD_EXIT = 0, CMD_JIT = 1, CMD_AOT = 2 };

// Constant records fetched ahead of use: lanes 0..N-1 of each wavefront load
// one dword each (a vector load: its wait lands where the record is first
// used, not at the next LDS wait as a scalar load's would), and the record is
// rebuilt in scalar registers from the lanes.
template <int N>
__device__ __forceinline__ uint32_t fetch_words(gptr<const uint32_t> p) {
  return p[threadIdx.x & (N - 1)];
}
__device__ __forceinline__ uint32_t word(uint32_t v, int k) { return (uint32_t)__builtin_amdgcn_readlane((int)v, k); }
template <typename T>
__device__ __forceinline__ gptr<const T> ptr_words(uint32_t v, int k) {
  return reinterpret_cast<gptr<const T>>(((uint64_t)word(v, k + 1) << 32) | word(v, k));
}
// (field by field, so that the records stay in registers)
__device__ __forceinline__ DevTask unpack_task(uint32_t v) {
  DevTask t;
  const uint32_t w0 = word(v, 0);
  t.type = (uint8_t)w0;
  t.mode = (uint8_t)(w0 >> 8);
  t.layer = (int16_t)(w0 >> 16);
  t.dep = (int32_t)word(v, 1);
  t.trig = (int32_t)word(v, 2);
  t.a0 = (int32_t)word(v, 3);
  t.a1 = (int32_t)word(v, 4);
  t.a2 = (int32_t)word(v, 5);
  t.id = (int32_t)word(v, 6);
  t.dep_counts = word(v, 7);
  return t;
}
__device__ __forceinline__ TaskPtrs unpack_ptrs(uint32_t v) {
  TaskPtrs p;
  p.p0 = ptr_words<uint16_t>(v, 8);
  p.p1 = ptr_words<uint16_t>(v, 10);
  p.p2 = ptr_words<uint16_t>(v, 12);
  p.p3 = ptr_words<uint16_t>(v, 14);
  return p;
}
__device__ __forceinline__ DevEvent unpack_event(uint32_t v) {
  DevEvent e;
  e.counts = word(v, 0);
  e.first = (int32_t)word(v, 1);
  e.last = (int32_t)word(v, 2);
  e.flags = word(v, 3);
  return e;
}

// A worker.  It holds the descriptor of its next AOT task in registers (the
// per-worker descriptor copies are constant, so the following one is fetched
// while the current task runs); thread 0 waits for either a JIT task or the
// next AOT task's event, the workgroup runs the task, and wavefront 0 advances
// the task's triggering event.  Meanwhile wavefronts 1..7 issue the weight
// pre-load of the next AOT task when it is a batch-1 projection tile
// (gemv_preload), so its first weight bytes stream in while the worker
// triggers, waits and runs JIT tasks.
//
// The paged lookahead (weight_preload 3; this file compiled with MPK_LA = 1,
// megakernel_la.hip): the pre-load area is two pages and AOT task j stages
// into page j mod 2, so a worker has its next two AOT tasks staged --
// projection weights (gemv_preload) or an attention split's cached keys and
// values (attn_prestage) -- while it waits; after task j - 1 its page takes
// task j + 1.  A task runs with its page as the pre-load area (the
// arguments' lds_pf and pf_segs).
__device__ __forceinline__ void worker_loop(kptr kp, uint32_t epoch, uint64_t timeout, int w) {
  const KArgs a0 = *kp;
  int& s_cmd = reinterpret_cast<int*>(g_lds + kLdsCtl)[0];
  int& s_task = reinterpret_cast<int*>(g_lds + kLdsCtl)[1];
  const int tid = threadIdx.x;
  uint32_t jit_head = 0;
  if (tid == 0) jit_head = st_jit_head(a0)[w];
  const uint32_t aot0 = a0.aot_off[w];
  const int n_aot = (int)(a0.aot_off[w + 1] - aot0);
  gptr<const AotEntry> aot = a0.aot_desc + aot0;
  int i = 0;
  // the next AOT entry, in flight (a worker with no AOT task reads its
  // neighbour's first entry and never uses it)
  uint32_t nxt_v = fetch_words<16>(reinterpret_cast<gptr<const uint32_t>>(aot));
  const uint32_t end_target = a0.events[a0.end_event].counts * epoch;
  gptr<const unsigned long long> ring = a0.jit_ring + (int64_t)w * a0.jit_cap;
  gptr<TraceRec> trace = a0.trace ? a0.trace + (int64_t)w * a0.trace_cap : nullptr;
  const int trace_cap = a0.trace_cap;
  int n_trace = 0;
  uint64_t t_wait = 0, t_start = 0;
#if MPK_LA
  // the highest AOT index staged (-1: none)
  int pre_i = -1;
  // the arguments with task j's page as the pre-load area
  auto page_args = [&](const KArgs& a, int j) {
    KArgs b = a;
    b.pf_segs = a.pf_segs / 2;
    b.lds_pf = a.lds_pf + (j & 1) * kPfWaves * b.pf_segs * 1024;
    return b;
  };
  auto stage = [&](const KArgs& a, int j, uint32_t v) {
    const DevTask nt = unpack_task(v);
    const KArgs b = page_args(a, j);
    if (tid >= 64) {
      if (is_gemv(nt.type)) gemv_preload(b, nt, unpack_ptrs(v), g_lds);
      else if (nt.type == MPK_TASK_ATTN && a.B == 1) {
        if (a.d == 128) attn_prestage<128>(b, nt, g_lds);
        else attn_prestage<64>(b, nt, g_lds);
      }
    }
  };
  auto preload_next = [&](const KArgs& a) {
    if (i < n_aot) {
      if (pre_i < i) {
        stage(a, i, nxt_v);
        pre_i = i;
      }
      if (i + 1 < n_aot && pre_i < i + 1) {
        stage(a, i + 1, fetch_words<16>(reinterpret_cast<gptr<const uint32_t>>(aot + i + 1)));
        pre_i = i + 1;
      }
    }
  };
#else
  // index of the AOT task whose weight pre-load has been issued (-1: none)
  int pre_i = -1;
  auto preload_next = [&](const KArgs& a) {
    if (a.pf_segs > 0 && i < n_aot && pre_i != i) {
      const DevTask nt = unpack_task(nxt_v);
      if (is_gemv(nt.type) && tid >= 64) gemv_preload(a, nt, unpack_ptrs(nxt_v), g_lds);
      pre_i = i;
    }
  };
#endif
  preload_next(a0);
  while (true) {
    // the arguments are re-read (constant cache) in every iteration rather
    // than held in registers across it
    kptr ap = kp;
    asm volatile("" : "+s"(ap));
    const KArgs a = *ap;
    // dependent event, its trigger count and the id of the next AOT task
    const int nxt_dep = (int)word(nxt_v, 1);
    const int nxt_id = (int)word(nxt_v, 6);
    const uint32_t nxt_counts = word(nxt_v, 7);
    if (tid == 0) {
      int cmd = CMD_EXIT, task = -1;
      const long long t0 = wall_clock64();
      t_wait = (uint64_t)t0;
      const uint32_t target = nxt_counts * epoch;
      uint32_t cnt = 0;
      const bool has_aot = i < n_aot;
      gptr<const uint32_t> cnt_p = &a.ev_cnt[has_aot ? nxt_dep : a.end_event];
      const uint32_t cnt_target = has_aot ? target : end_target;
      while (true) {
        // one round trip per poll: the JIT slot, the counter and the status
        // word are loaded together and checked afterwards
        const unsigned long long slot = ld_relaxed64(&ring[jit_head & (a.jit_cap - 1)]);
        cnt = ld_relaxed(cnt_p);
        const uint32_t status = ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code));
        if ((uint32_t)(slot >> 32) == jit_head + 1u) {
          task = (int)(uint32_t)slot;
          ++jit_head;
          cmd = CMD_JIT;
          break;
        }
        if (reached(cnt, cnt_target)) { cmd = has_aot ? CMD_AOT : CMD_EXIT; break; }
        if (status != 0u) { cmd = CMD_EXIT; break; }
        if ((uint64_t)(wall_clock64() - t0) > timeout) {
          report(a, MPK_ERR_TIMEOUT, i < n_aot ? nxt_id : -1, i < n_aot ? nxt_dep : a.end_event,
                 i < n_aot ? cnt : 0u, i < n_aot ? target : end_target);
          cmd = CMD_EXIT;
          break;
        }
        for (int z = 0; z < a.poll_sleep; ++z) __builtin_amdgcn_s_sleep(1);
      }
      t_start = (uint64_t)wall_clock64();
      s_cmd = cmd;
      s_task = task;
    }
    __syncthreads();
    const int cmd = __builtin_amdgcn_readfirstlane(s_cmd), jtask = __builtin_amdgcn_readfirstlane(s_task);
    __syncthreads();
    if (cmd == CMD_EXIT) break;
    // the task as an AOT entry spread over lanes 0..15 (a JIT task's
    // descriptor, whose weight pointers are resolved below)
    uint32_t cur_v;
    bool pre = false;
#if MPK_LA
    int page = 0;   // (the AOT index: its parity is the task's page)
#endif
    if (cmd == CMD_AOT) {
      cur_v = nxt_v;
#if MPK_LA
      pre = pre_i >= i;
      page = i;
#else
      pre = pre_i == i;
#endif
      ++i;
      nxt_v = fetch_words<16>(reinterpret_cast<gptr<const uint32_t>>(aot + (i < n_aot ? i : n_aot - 1)));
    } else {
      const uint32_t v = fetch_words<8>(reinterpret_cast<gptr<const uint32_t>>(a.tasks + jtask));
      cur_v = (threadIdx.x & 15) < 8 ? v : 0u;
    }
    const DevTask t = unpack_task(cur_v);
    // (a JIT task resolves its weight pointers through the layer pointer table)
    const TaskPtrs P = cmd == CMD_AOT ? unpack_ptrs(cur_v) : task_ptrs(a, t);
    if (trace && tid == 0) {
      reinterpret_cast<unsigned long long*>(g_lds + kLdsMarks)[0] = 0;
      reinterpret_cast<unsigned long long*>(g_lds + kLdsMarks)[1] = 0;
    }
    // the triggering event's record and the task's sub-counter quota, in
    // flight while the task runs
    const uint32_t ev_v = fetch_words<4>(reinterpret_cast<gptr<const uint32_t>>(a.events + t.trig));
    const uint32_t q_v = a.ev_quota[(int64_t)t.trig * kEvSub + (t.id & (kEvSub - 1))];
#if MPK_LA
    if (cmd == CMD_AOT) run_task(page_args(a, page), t, P, pre);
    else run_task(a, t, P, false);
#else
    run_task(a, t, P, pre);
#endif
    wait_vm<0>();   // the task's stores are complete before its event advances
    __syncthreads();
    if (tid < 64) {
      const uint64_t t_end = (uint64_t)wall_clock64();
      trigger(a, epoch, t.trig, unpack_event(ev_v), t.id, q_v);
      if (tid == 0 && trace && n_trace < trace_cap) {
        const unsigned long long* mk = reinterpret_cast<const unsigned long long*>(g_lds + kLdsMarks);
        trace[n_trace++] = TraceRec{t.id, w, t_wait, t_start, t_end, (uint64_t)wall_clock64(), {mk[0], mk[1]}};
      }
    }
    preload_next(a);
  }
  if (tid == 0) {
    st_jit_head(a0)[w] = jit_head;
    if (trace) a0.trace_count[w] = (uint32_t)n_trace;
  }
}

// One scheduler per wavefront.  Scheduler s serves workers s, s + S, s + 2S,
// ... (n_sub = W / S <= 64 of them); lane x keeps the JIT ring tail of its
// x-th worker in a register.  A popped chunk's tasks sit at distinct
// positions of the scheduler's segment (see push_chunk), so each lane writes
// at most one slot, all lanes in parallel.  Ring slots are written and read
// with relaxed agent-scope atomics.
__device__ __forceinline__ void scheduler_loop(const KArgs& a, uint32_t epoch, uint64_t timeout, int s) {
  const int lane = threadIdx.x & 63;
  const int n_sub = jit_sub(a);
  gptr<uint32_t> tails = st_jit_tail(a);
  const int my_w = s + lane * a.n_sched;
  uint32_t my_tail = lane < n_sub ? tails[my_w] : 0u;
  uint32_t head = st_sched_head(a)[s];
  gptr<const unsigned long long> ring = a.sched_ring + (int64_t)s * a.sched_cap;
  gptr<unsigned long long> my_ring = a.jit_ring + (int64_t)(lane < n_sub ? my_w : 0) * a.jit_cap;
  const uint32_t end_target = a.events[a.end_event].counts * epoch;
  long long t0 = wall_clock64();
  while (true) {
    const unsigned long long slot = ld_relaxed64(&ring[head & (a.sched_cap - 1)]);
    const uint32_t end_cnt = ld_relaxed(&a.ev_cnt[a.end_event]);
    const uint32_t status = ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code));
    if ((uint32_t)(slot >> 32) == head + 1u) {
      const int e = (int)((uint32_t)slot & ((1u << kJitEventBits) - 1u));
      const int c = (int)((uint32_t)slot >> kJitEventBits);
      ++head;
      const DevEvent ev = a.events[e];
      // the chunk's positions (unwrapped): [u0, u1) within one segment
      const int P = (int)(ev.flags >> 16), seg = P / n_sub + c;
      const int u0 = max(P, seg * n_sub), u1 = min(P + ev.last - ev.first + 1, (seg + 1) * n_sub);
      const int u = seg * n_sub + lane;   // this lane's position in the segment
      if (lane < n_sub && u >= u0 && u < u1) {
        __hip_atomic_store(&my_ring[my_tail & (a.jit_cap - 1)],
                           ((unsigned long long)(my_tail + 1u) << 32) | (uint32_t)(ev.first + (u - P)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ++my_tail;
      }
      t0 = wall_clock64();
      continue;
    }
    if (reached(end_cnt, end_target)) break;
    if (status != 0u) break;
    if ((uint64_t)(wall_clock64() - t0) > timeout) {
      if (lane == 0) report(a, MPK_ERR_TIMEOUT, -1, a.end_event, 0u, end_target);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  if (lane < n_sub) tails[my_w] = my_tail;
  if (lane == 0) st_sched_head(a)[s] = head;
}

}  // namespace

// One source, three kernels: the default runtime (this file), the paged
// lookahead (MPK_LA, megakernel_la.hip) and the batch > 1 runtime (MPK_BN,
// megakernel_bn.hip), each a translation unit of its own so that a change
// made for one leaves the others' code as it is.
#if MPK_LA
#define MPK_K(name) name##_la
#elif MPK_BN
#define MPK_K(name) name##_bn
#else
#define MPK_K(name) name
#endif
__global__ void __launch_bounds__(kThreads) MPK_K(mpk_megakernel)(const KArgs args, uint32_t epoch, uint64_t timeout) {
  // `args` is the first kernel argument: it starts the kernel-argument segment
  const kptr kp = (kptr)(__builtin_amdgcn_kernarg_segment_ptr());
  const KArgs a = args;
  if (ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code)) != 0u) return;  // poisoned graph
  const int wg = blockIdx.x;
  if (wg < a.n_sched_wgs) {
    const int s = wg * 4 + (int)(threadIdx.x >> 6);
    if ((threadIdx.x >> 6) < 4 && s < a.n_sched) scheduler_loop(a, epoch, timeout, s);
    return;
  }
  const int w = wg - a.n_sched_wgs;
  if (w < a.n_workers) worker_loop(kp, epoch, timeout, w);
}

#if !MPK_LA
// Kernel-per-operator baseline: workgroup i runs task list[i], no events (a
// projection tile issues its weight pre-load first, as in the persistent
// kernel).  A poisoned graph runs nothing.
__global__ void __launch_bounds__(kThreads) MPK_K(mpk_baseline_op)(const KArgs a, const int32_t* list) {
  if (ld_relaxed(reinterpret_cast<gptr<const uint32_t>>(&a.status->code)) != 0u) return;
  const DevTask t = a.tasks[list[blockIdx.x]];
  const TaskPtrs P = task_ptrs(a, t);
  const bool pre = a.pf_segs > 0 && is_gemv(t.type);
  if (pre) gemv_preload(a, t, P, g_lds);
  run_task(a, t, P, pre);
}

// Body timing: one workgroup runs one task and adds its wall-clock ticks to *out.
__global__ void __launch_bounds__(kThreads) MPK_K(mpk_time_task_kernel)(const KArgs a, int task, int cold,
                                                                         unsigned long long* out) {
  const DevTask t = a.tasks[task];
  const TaskPtrs P = task_ptrs(a, t);
  __syncthreads();
  if (cold) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // cold caches, as after a fenced wait
  const unsigned long long t0 = wall_clock64();
  run_task(a, t, P);
  __syncthreads();
  if (threadIdx.x == 0) *out += wall_clock64() - t0;
}
#endif

#if MPK_LA || MPK_BN
hipError_t MPK_K(launch_megakernel)(const KArgs& args, uint32_t epoch, uint64_t timeout, int grid, hipStream_t stream) {
  KArgs a = args;
  void* p[] = {&a, &epoch, &timeout};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&MPK_K(mpk_megakernel)), dim3(grid), dim3(kThreads),
                                    p, 0, stream);
}
#endif
#if MPK_BN
hipError_t launch_baseline_op_bn(const KArgs& args, const int32_t* list, int count, hipStream_t stream) {
  hipLaunchKernelGGL(mpk_baseline_op_bn, dim3(count), dim3(kThreads), 0, stream, args, list);
  return hipGetLastError();
}
hipError_t launch_time_task_bn(const KArgs& args, int task, bool cold, unsigned long long* out, hipStream_t stream) {
  hipLaunchKernelGGL(mpk_time_task_kernel_bn, dim3(1), dim3(kThreads), 0, stream, args, task, cold ? 1 : 0, out);
  return hipGetLastError();
}
#endif
#if !MPK_LA && !MPK_BN
hipError_t launch_megakernel_la(const KArgs& args, uint32_t epoch, uint64_t timeout, int grid, hipStream_t stream);
hipError_t launch_megakernel_bn(const KArgs& args, uint32_t epoch, uint64_t timeout, int grid, hipStream_t stream);
hipError_t launch_baseline_op_bn(const KArgs& args, const int32_t* list, int count, hipStream_t stream);
hipError_t launch_time_task_bn(const KArgs& args, int task, bool cold, unsigned long long* out, hipStream_t stream);

// (batch > 1: the batch > 1 runtime's kernels)
hipError_t launch_time_task(const KArgs& args, int task, bool cold, unsigned long long* out, hipStream_t stream) {
  if (args.B > 1) return launch_time_task_bn(args, task, cold, out, stream);
  hipLaunchKernelGGL(mpk_time_task_kernel, dim3(1), dim3(kThreads), 0, stream, args, task, cold ? 1 : 0, out);
  return hipGetLastError();
}

hipError_t launch_megakernel(const KArgs& args, uint32_t epoch, uint64_t timeout, int grid, hipStream_t stream,
                             bool lookahead) {
  if (lookahead) return launch_megakernel_la(args, epoch, timeout, grid, stream);
  if (args.B > 1) return launch_megakernel_bn(args, epoch, timeout, grid, stream);
  KArgs a = args;
  void* p[] = {&a, &epoch, &timeout};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&mpk_megakernel), dim3(grid), dim3(kThreads), p,
                                    0, stream);
}

hipError_t launch_baseline_op(const KArgs& args, const int32_t* list, int count, hipStream_t stream) {
  if (args.B > 1) return launch_baseline_op_bn(args, list, count, stream);
  hipLaunchKernelGGL(mpk_baseline_op, dim3(count), dim3(kThreads), 0, stream, args, list);
  return hipGetLastError();
}
#endif

}  // namespace mpk
