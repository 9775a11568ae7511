// C ABI of the decode-step mega-kernel library (declared in include/mpk.h):
// graph build and upload, the persistent-kernel step, the kernel-per-operator
// baseline, export for the checker, status and intermediate-tensor readback.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <map>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "builder.h"
#include "mpk.h"
#include "rt.h"

namespace mpk {
hipError_t launch_megakernel(const KArgs& args, uint32_t epoch, uint64_t timeout, int grid, hipStream_t stream,
                             bool lookahead);
hipError_t launch_baseline_op(const KArgs& args, const int32_t* list, int count, hipStream_t stream);
hipError_t launch_time_task(const KArgs& args, int task, bool cold, unsigned long long* out, hipStream_t stream);
int64_t packed_bytes(int64_t N, int64_t K);
hipError_t launch_pack(const void* a, const void* b, int64_t N, int64_t K, void* dst, hipStream_t stream);
size_t scratch_capacity();
hipError_t scratch_address(int device, void** out);
hipError_t scratch_zero(void* p, size_t bytes, hipStream_t stream);
}  // namespace mpk

using namespace mpk;

namespace {

// The message of the last failure on this thread, in a fixed buffer so that
// reporting an error allocates nothing (the no-allocation step reports
// through it too).
thread_local char g_err[512];

int fail(int code, const char* msg) {
  std::snprintf(g_err, sizeof(g_err), "%s", msg);
  return code;
}
int fail(int code, const std::string& msg) { return fail(code, msg.c_str()); }
int hip_fail(hipError_t e, const char* what) {
  std::snprintf(g_err, sizeof(g_err), "%s: %s", what, hipGetErrorString(e));
  return MPK_ERR_HIP;
}
#define HIPCHK(x)                                  \
  do {                                             \
    hipError_t e_ = (x);                           \
    if (e_ != hipSuccess) return hip_fail(e_, #x); \
  } while (0)

uint32_t next_pow2(uint64_t x) {
  uint64_t p = 1;
  while (p < x) p <<= 1;
  return (uint32_t)p;
}

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

}  // namespace

struct mpk_tgraph {
  mpk_model_cfg cfg{};
  int32_t B = 0, P = 0;
  Params prm;
  mpk_build_params resolved{};
  bool host_only = false;
  Graph g;

  int device = 0, n_cus = 0, grid = 0, n_sched_wgs = 0, n_sched = 0;
  double wall_khz = 100000.0;
  uint64_t timeout_ns = 2000000000ull;
  uint32_t epoch = 0;

  std::vector<DevTask> h_tasks;
  std::vector<uint32_t> dev_counts;   // device event counts (two-level events: non-empty sub-counters)
  std::vector<uint16_t> quota;        // [NE][kEvSub] arrivals per sub-counter and step
  void* d_graph = nullptr;  // tasks, events, aot offsets, aot tasks
  DevTask* d_tasks = nullptr;
  DevEvent* d_events = nullptr;
  uint32_t* d_aot_off = nullptr;
  AotEntry* d_aot_desc = nullptr;
  std::vector<AotEntry> h_aot;  // host copy; its weight pointers follow the last step's weights
  void* d_rt = nullptr;     // counters, rings, state, status
  uint32_t* d_ev_cnt = nullptr;
  uint32_t* d_ev_sub = nullptr;
  uint16_t* d_ev_quota = nullptr;
  unsigned long long* d_sched_ring = nullptr;
  uint32_t* d_sched_tail = nullptr;
  unsigned long long* d_jit_ring = nullptr;
  uint32_t* d_state = nullptr;
  StatusWord* d_status = nullptr;
  uint32_t* d_arrive = nullptr;  // attention split arrivals (0 between steps)
  int64_t arrive_bytes = 0;
  int64_t rt_bytes = 0;     // runtime arena (counters, rings, state, status, arrivals)
  uint32_t sched_cap = 0, jit_cap = 0;

  void* d_act = nullptr;
  int64_t act_bytes = 0;
  KArgs base{};             // arguments that do not change between steps
  KArgs last{};             // arguments of the last step (kernel arguments are passed by value)
  bool args_valid = false;
  struct TensorRef { void* p; int64_t bytes; };
  std::vector<TensorRef> tensors;  // indexed by tensor id (null when caller-owned)

  const uint16_t** d_wl = nullptr;
  std::vector<const void*> h_wl;

  int32_t* d_lists = nullptr;
  std::vector<std::pair<int32_t, int32_t>> ops;  // (offset, count) per operator, program order
  hipStream_t cap_stream = nullptr;
  hipGraphExec_t gexec = nullptr;
  std::vector<uintptr_t> gkey;
  hipStream_t last_stream = nullptr;
  void* d_trace = nullptr;  // trace records + counts
  int32_t trace_cap = 0;
};

namespace {

// Two-level events (see rt.h): per event, the arrivals of each sub-counter
// (producer t counts on sub-counter t mod kEvSub) and the device count.
int two_level_events(mpk_tgraph* t) {
  const Graph& g = t->g;
  t->dev_counts.assign(g.event_counts.begin(), g.event_counts.end());
  std::vector<uint32_t> q((size_t)g.NE * kEvSub, 0);
  for (int32_t i = 0; i < g.NT; ++i)
    if (g.task_trig[i] >= 0) ++q[(size_t)g.task_trig[i] * kEvSub + (i % kEvSub)];
  t->quota.assign(q.size(), 0);
  for (int32_t e = 0; e < g.NE; ++e) {
    if (g.event_counts[e] < kTwoLevelMin) continue;
    uint32_t nnz = 0, sum = 0;
    for (int k = 0; k < kEvSub; ++k) {
      const uint32_t v = q[(size_t)e * kEvSub + k];
      if (v > 65535) return fail(MPK_ERR_UNSUPPORTED, "more than 65535 producers on one event sub-counter");
      t->quota[(size_t)e * kEvSub + k] = (uint16_t)v;
      nnz += v > 0;
      sum += v;
    }
    if (sum != g.event_counts[e]) return fail(MPK_ERR_GRAPH, "event count differs from its producers");
    t->dev_counts[e] = nnz;
  }
  return MPK_OK;
}

void fill_descriptors(mpk_tgraph* t) {
  const Graph& g = t->g;
  const Params& p = t->prm;
  const mpk_model_cfg& c = t->cfg;
  const int32_t G = c.n_q_heads / c.n_kv_heads, Sg = (G + 2) * c.head_dim, tpg = p.T_qkv / c.n_kv_heads;
  t->h_tasks.assign(g.NT, DevTask{});
  for (int32_t i = 0; i < g.NT; ++i) {
    DevTask& d = t->h_tasks[i];
    d.type = g.task_type[i];
    d.mode = g.task_mode[i];
    d.layer = g.task_layer[i];
    d.dep = g.task_dep[i];
    d.trig = g.task_trig[i];
    d.id = i;
    d.dep_counts = t->dev_counts[d.dep];
    const int32_t c0 = g.task_coords[3 * (size_t)i], c1 = g.task_coords[3 * (size_t)i + 1],
                  c2 = g.task_coords[3 * (size_t)i + 2];
    int32_t lo = 0, hi = 0;
    switch (d.type) {
      // (projection tile n of a k-split into K ranges: column tile n / K,
      // k range n % K, which the device derives from a2 = n)
      case MPK_TASK_QKV: {
        int32_t gg = c0 / tpg, j = (c0 % tpg) / p.K_qkv;
        tile_range(Sg, p.q, tpg / p.K_qkv, j, &lo, &hi);
        d.a0 = gg * Sg + lo; d.a1 = gg * Sg + hi; d.a2 = c0;
        break;
      }
      case MPK_TASK_OPROJ:
        tile_range(c.hidden, p.q, p.T_o / p.K_o, c0 / p.K_o, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0;
        break;
      case MPK_TASK_GATEUP: tile_range(c.ffn, p.q, p.T_gu, c0, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0; break;
      case MPK_TASK_DOWN:
        tile_range(c.hidden, p.q, p.T_down / p.K_down, c0 / p.K_down, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0;
        break;
      case MPK_TASK_LMHEAD: tile_range(c.vocab, p.q, p.T_lm, c0, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0; break;
      case MPK_TASK_ATTN: d.a0 = c0; d.a1 = c1; d.a2 = p.K_qkv; break;
      // (router tile n: expert columns, a2 = n; expert tiles (slot s, tile n): columns, a2 = s)
      case MPK_TASK_ROUTER: tile_range(c.n_experts, p.q, p.T_router, c0, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0; break;
      case MPK_TASK_EXPERT_GU: tile_range(c.moe_ffn, p.q, p.T_egu, c1, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0; break;
      case MPK_TASK_EXPERT_DOWN: tile_range(c.hidden, p.q, p.T_edown, c1, &lo, &hi); d.a0 = lo; d.a1 = hi; d.a2 = c0; break;
      default: d.a0 = c0; d.a1 = c1; d.a2 = c2; break;
    }
  }
}

// The runtime resolves empty tasks inline, at most two levels deep (a graph
// built without fusion chains a fan-out empty into a fan-in empty): an event
// with empty consumers has only empty consumers, and an empty task's event
// with empty consumers hands those to empties whose own events have none.
int check_runtime_shape(const Graph& g) {
  auto only_empty = [&](int32_t e) {
    for (int32_t t = g.event_first[e]; t <= g.event_last[e]; ++t)
      if (g.task_type[t] != MPK_TASK_EMPTY) return false;
    return true;
  };
  for (int32_t e = 0; e < g.NE; ++e) {
    if (!(g.event_flags[e] & MPK_EVENT_HAS_EMPTY)) continue;
    if (!only_empty(e)) return fail(MPK_ERR_GRAPH, "event mixes empty and real consumers");
    for (int32_t t = g.event_first[e]; t <= g.event_last[e]; ++t) {
      const int32_t f = g.task_trig[t];
      if (!(g.event_flags[f] & MPK_EVENT_HAS_EMPTY)) continue;
      if (!only_empty(f)) return fail(MPK_ERR_GRAPH, "event mixes empty and real consumers");
      for (int32_t t2 = g.event_first[f]; t2 <= g.event_last[f]; ++t2)
        if (g.event_flags[g.task_trig[t2]] & MPK_EVENT_HAS_EMPTY)
          return fail(MPK_ERR_GRAPH, "empty tasks chained more than two deep");
    }
  }
  return MPK_OK;
}

// Kernel-per-operator lists for the baseline: one operator per (layer, task
// type), in the program order of its tasks; a list holds its tasks in linear
// order.
void build_op_lists(mpk_tgraph* t, std::vector<int32_t>* flat) {
  const Graph& g = t->g;
  std::map<std::pair<int32_t, int32_t>, size_t> idx;
  std::vector<std::pair<int32_t, std::vector<int32_t>>> lists;  // (first program-order id, tasks)
  for (int32_t i = 0; i < g.NT; ++i) {
    const int32_t ty = g.task_type[i];
    if (ty == MPK_TASK_EMPTY) continue;
    const auto key = std::make_pair((int32_t)g.task_layer[i], ty);
    auto it = idx.find(key);
    if (it == idx.end()) {
      it = idx.emplace(key, lists.size()).first;
      lists.push_back({g.task_orig[i], {}});
    }
    auto& L = lists[it->second];
    L.first = std::min(L.first, g.task_orig[i]);
    L.second.push_back(i);
  }
  std::sort(lists.begin(), lists.end(), [](const auto& a, const auto& b) { return a.first < b.first; });
  t->ops.clear();
  flat->clear();
  for (auto& v : lists) {
    t->ops.push_back({(int32_t)flat->size(), (int32_t)v.second.size()});
    flat->insert(flat->end(), v.second.begin(), v.second.end());
  }
}

// LDS layout of a workgroup (KArgs::lds_*): staging area, projection
// accumulators, the weight pre-load area (batch 1) and the page ids of an
// attention split under the runtime's control words at the top.
int lds_layout(const mpk_model_cfg& c, int32_t B, int32_t P, const Params& p, KArgs* a) {
  auto chunks = [](int64_t b) { return (b + 1023) & ~(int64_t)1023; };
  const int64_t H = c.hidden, F = c.ffn, d = c.head_dim, hq = c.n_q_heads, hkv = c.n_kv_heads, G = hq / hkv;
  const bool fused = fused_norm(B), moe = c.n_experts > 0;
  // (a mixture-of-experts model has no dense FFN: its widths are the experts')
  const int64_t Fd = moe ? c.moe_ffn : F;
  int64_t stage = fused ? std::max({chunks(H * 4), chunks(hq * d * 4), chunks(Fd * 4), 2 * chunks(H * 4) + chunks(H * 2)})
                        : chunks(H * 2) + (1 + std::max(p.K_o, p.K_down)) * chunks(H * 4);
  // (batch > 1: a norm task's gain, its residual row and the k-split planes it adds)
  // attention: wavefront merge states, raw q/k/v row, processed heads
  stage = std::max(stage, chunks(kWaves * G * (d + 2) * 4) + 2 * chunks((G + 2) * d * 4));
  // the split combine stages a request's records when they fit in 96 KB (else it reads them from
  // global memory); a request gets at most M - B + 1 of the M slots.  At batch 1 the step caps the
  // request's split count at what the staging area holds, so the area is not grown for it.
  const int64_t max_split = (int64_t)p.S_attn - B + 1;
  const int64_t comb = ((max_split * G * (d + 2) + 63) & ~(int64_t)63) * 4;
  if (B > 1 && comb <= 96 * 1024) stage = std::max(stage, comb);
  // accumulators: the widest projection tile, rows per column x batch
  const int64_t tpg = p.T_qkv / hkv, Sg = (G + 2) * d;
  auto widest = [&](int64_t N, int64_t T) { return p.q * ((((N + p.q - 1) / p.q) + T - 1) / T); };
  int64_t widest_ffn = moe ? std::max({widest(c.n_experts, p.T_router), 2 * widest(c.moe_ffn, p.T_egu),
                                         widest(H, p.T_edown)})
                            : std::max(2 * widest(F, p.T_gu), widest(H, p.T_down / p.K_down));
  const int64_t acc = chunks(4 * B * std::max({widest(Sg, tpg / p.K_qkv), widest(H, p.T_o / p.K_o), widest_ffn,
                                               widest(c.vocab, p.T_lm)}));
  const int64_t max_pages = std::min<int64_t>((c.max_seq_len + P - 1) / P, 4096);
  const int64_t pid = kLdsBytes - kLdsTop - chunks(4 * max_pages);
  // (an expert tile's routing area under the page ids: both are live only while such a task runs, and
  // neither may share the pre-load area, which holds the next task's weights while a JIT task runs)
  // (the routing area ends in the B x E logits, staged in whole runs of 64)
  const int64_t top = moe ? pid - chunks((int64_t)sizeof(MoeLds) + 4 * ((B * (int64_t)c.n_experts + 63) & ~63)) : pid;
  const int64_t pf = stage + acc;
  if (pf > top) return fail(MPK_ERR_UNSUPPORTED, "shape needs more LDS than a compute unit has");
  a->lds_acc = (int32_t)stage;
  a->lds_pf = (int32_t)pf;
  a->lds_pid = (int32_t)pid;
  a->lds_moe = (int32_t)top;
  a->pf_segs = fused && p.preload ? (int32_t)std::min<int64_t>(kMaxPfSegs, (top - pf) / (kPfWaves * 1024)) : 0;
  return MPK_OK;
}

int upload(mpk_tgraph* t) {
  const Graph& g = t->g;
  HIPCHK(hipGetDevice(&t->device));
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, t->device));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MPK_ERR_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", kernels are built for gfx950");
  int khz = 0;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, t->device) == hipSuccess && khz > 0)
    t->wall_khz = khz;
  t->n_cus = prop.multiProcessorCount;
  t->n_sched_wgs = (t->prm.S_sched + 3) / 4;
  t->n_sched = std::min(t->prm.S_sched, t->prm.W);
  t->grid = t->n_sched_wgs + t->prm.W;
  if (t->grid > t->n_cus)
    return fail(MPK_ERR_INVALID_ARG, "workers + scheduler workgroups exceed the compute units");
  if (t->n_sched == 0 && std::count(g.task_mode.begin(), g.task_mode.end(), (uint8_t)MPK_MODE_JIT) > 0)
    return fail(MPK_ERR_INVALID_ARG, "JIT tasks need at least one scheduler wavefront");
  if (t->n_sched > 0 && (t->prm.W + t->n_sched - 1) / t->n_sched > 64)
    return fail(MPK_ERR_INVALID_ARG, "more than 64 workers per scheduler wavefront");
  if (t->n_sched > 0 && t->prm.W % t->n_sched != 0)
    return fail(MPK_ERR_INVALID_ARG, "the worker count must be a multiple of the scheduler wavefronts");

  if (int rc = two_level_events(t)) return rc;
  fill_descriptors(t);
  // graph arrays
  const int64_t o_tasks = 0, o_events = align256(o_tasks + (int64_t)g.NT * sizeof(DevTask));
  const int64_t o_off = align256(o_events + (int64_t)g.NE * sizeof(DevEvent));
  const int64_t o_aot = align256(o_off + (int64_t)g.aot_offsets.size() * 4);
  std::vector<int32_t> flat;
  build_op_lists(t, &flat);
  // (+1: a worker with an empty list still reads one descriptor)
  const int64_t o_lists = align256(o_aot + (int64_t)(g.aot_tasks.size() + 1) * sizeof(AotEntry));
  const int64_t o_wl = align256(o_lists + (int64_t)std::max<size_t>(1, flat.size()) * 4);
  const int64_t o_freq = align256(o_wl + (int64_t)t->cfg.n_layers * LAYER_PTRS * 8);
  const int64_t o_quota = align256(o_freq + (int64_t)t->cfg.head_dim / 2 * 8);
  const int64_t graph_bytes = align256(o_quota + (int64_t)g.NE * kEvSub * 2);
  // JIT placement by worker position (see the mega-kernel): the tasks of a
  // JIT event take consecutive positions from the running count of JIT
  // tasks in event order (mod W), so events that fire together fill the
  // workers one task each before any worker gets a second.  The device copy
  // of the event keeps its start position in flags bits 16..31; one
  // scheduler ring entry per scheduler segment the positions cross.
  std::vector<DevEvent> ev(g.NE);
  const int64_t Wp = t->prm.W, n_sub = Wp / std::max(1, t->n_sched);
  int64_t pos = 0;   // running JIT task count, the next event's start position
  int64_t n_entries = 0;
  if (g.NE >= (1 << kJitEventBits)) return fail(MPK_ERR_UNSUPPORTED, "more than 2^20 events");
  for (int32_t e = 0; e < g.NE; ++e) {
    ev[e] = DevEvent{t->dev_counts[e], g.event_first[e], g.event_last[e], g.event_flags[e]};
    if (g.event_counts[e] >= kTwoLevelMin) ev[e].flags |= kEvTwoLevel;
    if (g.event_counts[e] == 1 && g.event_last[e] >= g.event_first[e]) {
      bool all_empty = true;
      for (int32_t i = g.event_first[e]; i <= g.event_last[e]; ++i) all_empty &= g.task_mode[i] == MPK_MODE_EMPTY;
      if (all_empty) ev[e].flags |= kEvSole;
    }
    if (g.event_flags[e] & MPK_EVENT_HAS_JIT) {
      const int64_t k = g.event_last[e] - g.event_first[e] + 1, P = pos % Wp;
      const int64_t n_ch = (P + k - 1) / n_sub - P / n_sub + 1;
      if (n_ch > (1 << kJitChunkBits)) return fail(MPK_ERR_UNSUPPORTED, "more than 4096 JIT chunks in one event");
      ev[e].flags |= (uint32_t)P << 16;
      n_entries += n_ch;
      pos += k;
    }
  }
  HIPCHK(hipMalloc(&t->d_graph, graph_bytes));
  char* gb = (char*)t->d_graph;
  t->d_tasks = (DevTask*)(gb + o_tasks);
  t->d_events = (DevEvent*)(gb + o_events);
  t->d_aot_off = (uint32_t*)(gb + o_off);
  t->d_aot_desc = (AotEntry*)(gb + o_aot);
  t->d_lists = (int32_t*)(gb + o_lists);
  t->d_wl = (const uint16_t**)(gb + o_wl);
  {
    std::vector<double> inv(t->cfg.head_dim / 2);
    for (size_t i = 0; i < inv.size(); ++i)
      inv[i] = std::pow((double)t->cfg.rope_theta, -2.0 * (double)i / (double)t->cfg.head_dim);
    HIPCHK(hipMemcpy(gb + o_freq, inv.data(), inv.size() * 8, hipMemcpyHostToDevice));
    t->base.inv_freq = (const double*)(gb + o_freq);
  }
  HIPCHK(hipMemcpy(t->d_tasks, t->h_tasks.data(), (size_t)g.NT * sizeof(DevTask), hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(t->d_events, ev.data(), (size_t)g.NE * sizeof(DevEvent), hipMemcpyHostToDevice));
  t->d_ev_quota = (uint16_t*)(gb + o_quota);
  HIPCHK(hipMemcpy(t->d_ev_quota, t->quota.data(), t->quota.size() * 2, hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(t->d_aot_off, g.aot_offsets.data(), g.aot_offsets.size() * 4, hipMemcpyHostToDevice));
  // AOT entries (weight pointers are filled in by the first step)
  t->h_aot.assign(g.aot_tasks.size() + 1, AotEntry{});
  for (size_t k = 0; k < g.aot_tasks.size(); ++k) t->h_aot[k].t = t->h_tasks[g.aot_tasks[k]];
  HIPCHK(hipMemcpy(t->d_aot_desc, t->h_aot.data(), t->h_aot.size() * sizeof(AotEntry), hipMemcpyHostToDevice));
  if (!flat.empty()) HIPCHK(hipMemcpy(t->d_lists, flat.data(), flat.size() * 4, hipMemcpyHostToDevice));

  // runtime: counters, rings, state, status
  int64_t n_jit_tasks = 0;
  for (int32_t i = 0; i < g.NT; ++i) n_jit_tasks += g.task_mode[i] == MPK_MODE_JIT;
  t->sched_cap = next_pow2((uint64_t)n_entries + 1);   // every ring entry of a step fits in any one ring
  t->jit_cap = next_pow2((uint64_t)n_jit_tasks + 1);
  const int32_t W = t->prm.W, S = t->n_sched;
  const int64_t r_cnt = 0, r_sub = align256(r_cnt + (int64_t)g.NE * 4);
  const int64_t r_sring = align256(r_sub + (int64_t)g.NE * kEvSub * 4);
  const int64_t r_stail = align256(r_sring + (int64_t)S * t->sched_cap * 8);
  const int64_t r_jring = align256(r_stail + (int64_t)S * 4);
  const int64_t r_state = align256(r_jring + (int64_t)W * t->jit_cap * 8);
  const int64_t r_status = align256(r_state + (int64_t)(2 * W + S) * 4);
  const int64_t r_arrive = align256(r_status + (int64_t)sizeof(StatusWord));
  const int64_t rt_bytes =
      align256(r_arrive + (int64_t)t->cfg.n_layers * t->B * t->cfg.n_kv_heads * 4);
  t->rt_bytes = rt_bytes;
  HIPCHK(hipMalloc(&t->d_rt, rt_bytes));
  HIPCHK(hipMemset(t->d_rt, 0, rt_bytes));
  char* rb = (char*)t->d_rt;
  t->d_ev_cnt = (uint32_t*)(rb + r_cnt);
  t->d_ev_sub = (uint32_t*)(rb + r_sub);
  t->d_sched_ring = (unsigned long long*)(rb + r_sring);
  t->d_sched_tail = (uint32_t*)(rb + r_stail);
  t->d_jit_ring = (unsigned long long*)(rb + r_jring);
  t->d_state = (uint32_t*)(rb + r_state);
  t->d_status = (StatusWord*)(rb + r_status);
  t->d_arrive = (uint32_t*)(rb + r_arrive);
  t->arrive_bytes = rt_bytes - r_arrive;

  // activations
  const mpk_model_cfg& c = t->cfg;
  const int64_t B = t->B, H = c.hidden, L = c.n_layers, hq = c.n_q_heads, hkv = c.n_kv_heads, d = c.head_dim;
  const int64_t G = hq / hkv, Sg = (G + 2) * d, F = c.ffn, S_at = t->prm.S_attn;
  KArgs& a = t->base;
  const bool moe = c.n_experts > 0;
  const int64_t M = moe_slots(c, t->B);
  a.st_bh = B * H; a.st_q = B * hq * d; a.st_part = hkv * S_at * G * (d + 2);
  a.st_a = moe ? M * B * c.moe_ffn : B * F;
  a.E = c.n_experts; a.topk = c.top_k; a.Fe = c.moe_ffn; a.norm_topk = c.norm_topk; a.M = (int32_t)M;
  a.st_rlog = moe ? B * c.n_experts : 0;
  a.st_route = moe ? M * route_words(t->B) : 0;
  // k-split projections write K planes [K][B][...] whose sum is the output
  a.Kq = t->prm.K_qkv; a.Ko = t->prm.K_o; a.Kd = t->prm.K_down;
  a.st_qkv = a.Kq * B * hkv * Sg; a.st_o = a.Ko * a.st_bh; a.st_dn = a.Kd * a.st_bh;
  // batch > 1 only (norm tasks): e, hf, h, h2
  const bool fused = fused_norm(t->B);
  struct Item { int id; int64_t bytes; };
  std::vector<Item> items = {{T_PMAX, B * (int64_t)t->prm.T_lm * 8}};
  if (!fused) items.insert(items.begin(), {{T_E, B * H * 4}, {T_HF, B * H * 4}});
  const int64_t nf = fused ? 0 : 1;
  // (h2 exists at batch > 1, and at batch 1 in mixture-of-experts layers, whose router tile 0 writes it)
  const int64_t nh2 = (!fused || moe) ? 1 : 0;
  const int64_t per_layer_bytes[L_COUNT] = {a.st_bh * 4, nf * a.st_bh * 4, a.st_qkv * 4, 0, 0, 0,
                                            a.st_part * 4, a.st_q * 4, a.st_o * 4, a.st_bh * 4,
                                            nh2 * a.st_bh * 4, a.st_a * 4, a.st_dn * 4,
                                            a.st_rlog * 4, a.st_route * 4};
  // one contiguous [L][...] block per per-layer tensor kind
  int64_t off = 0;
  std::vector<int64_t> shared_off(5, -1), kind_off(L_COUNT, -1);
  for (auto& it : items) { shared_off[it.id] = off; off = align256(off + it.bytes); }
  for (int k = 0; k < L_COUNT; ++k) {
    if (!per_layer_bytes[k]) continue;
    kind_off[k] = off;
    off = align256(off + per_layer_bytes[k] * L);
  }
  HIPCHK(hipMalloc(&t->d_act, off));
  HIPCHK(hipMemset(t->d_act, 0, off));
  t->act_bytes = off;
  char* ab = (char*)t->d_act;
  auto shared = [&](int id) { return shared_off[id] < 0 ? nullptr : (float*)(ab + shared_off[id]); };
  auto kind = [&](int k) { return kind_off[k] < 0 ? nullptr : (float*)(ab + kind_off[k]); };
  a.e = shared(T_E);
  a.hf = shared(T_HF);
  a.pmax = (PMax*)shared(T_PMAX);
  a.r = kind(L_R);
  a.h = kind(L_H);
  a.qkv = kind(L_QKV);
  a.part = kind(L_PART);
  a.attn = kind(L_ATTN);
  a.o = kind(L_O);
  a.s = kind(L_S);
  a.h2 = kind(L_H2);
  a.a = kind(L_A);
  a.dn = kind(L_D);
  a.rlog = kind(L_RLOG);
  a.route = (int32_t*)kind(L_ROUTE);
  t->tensors.assign(5 + L_COUNT * (size_t)L, {nullptr, 0});
  for (auto& it : items) t->tensors[it.id] = {ab + shared_off[it.id], it.bytes};
  for (int64_t l = 0; l < L; ++l)
    for (int k = 0; k < L_COUNT; ++k)
      if (per_layer_bytes[k]) t->tensors[layer_tensor((int32_t)l, k)] = {ab + kind_off[k] + l * per_layer_bytes[k], per_layer_bytes[k]};

  a.tasks = t->d_tasks; a.events = t->d_events; a.aot_off = t->d_aot_off; a.aot_desc = t->d_aot_desc;
  a.ev_cnt = t->d_ev_cnt; a.ev_sub = t->d_ev_sub; a.ev_quota = t->d_ev_quota;
  a.sched_ring = t->d_sched_ring; a.sched_tail = t->d_sched_tail; a.jit_ring = t->d_jit_ring;
  a.state = t->d_state; a.sched_cap = t->sched_cap; a.jit_cap = t->jit_cap;
  a.n_workers = W; a.n_sched = S; a.n_sched_wgs = t->n_sched_wgs;
  a.root_event = g.root; a.end_event = g.end;
  a.status = t->d_status;
  a.L = c.n_layers; a.H = c.hidden; a.hq = c.n_q_heads; a.hkv = c.n_kv_heads; a.d = c.head_dim; a.F = c.ffn;
  a.V = c.vocab; a.G = (int32_t)G; a.Sg = (int32_t)Sg; a.B = t->B; a.P = t->P; a.S_attn = t->prm.S_attn;
  a.T_lm = t->prm.T_lm; a.qk_norm = c.qk_norm; a.max_seq = c.max_seq_len; a.eps = c.rms_eps; a.theta = c.rope_theta;
  a.wl = t->d_wl;
  a.arrive = t->d_arrive;
  a.attn_min_pages = t->prm.split_pages;
  return lds_layout(c, t->B, t->P, t->prm, &a);
}

void free_tgraph(mpk_tgraph* t) {
  if (!t) return;
  if (t->gexec) (void)hipGraphExecDestroy(t->gexec);
  if (t->cap_stream) (void)hipStreamDestroy(t->cap_stream);
  if (t->d_graph) (void)hipFree(t->d_graph);
  if (t->d_rt) (void)hipFree(t->d_rt);
  if (t->d_act) (void)hipFree(t->d_act);
  if (t->d_trace) (void)hipFree(t->d_trace);
  delete t;
}

int export_graph(const Graph& g, const mpk_tgraph_header& hdr, mpk_tgraph_host_view* out) {
  std::memset(out, 0, sizeof(*out));
  out->header = hdr;
  auto dup = [](const void* src, size_t bytes) -> void* {
    void* p = std::malloc(bytes ? bytes : 1);
    if (p && bytes) std::memcpy(p, src, bytes);
    return p;
  };
  out->task_type = (uint8_t*)dup(g.task_type.data(), g.task_type.size());
  out->task_mode = (uint8_t*)dup(g.task_mode.data(), g.task_mode.size());
  out->task_layer = (int16_t*)dup(g.task_layer.data(), g.task_layer.size() * 2);
  out->task_coords = (uint16_t*)dup(g.task_coords.data(), g.task_coords.size() * 2);
  out->task_orig = (int32_t*)dup(g.task_orig.data(), g.task_orig.size() * 4);
  out->task_dep = (int32_t*)dup(g.task_dep.data(), g.task_dep.size() * 4);
  out->task_trig = (int32_t*)dup(g.task_trig.data(), g.task_trig.size() * 4);
  out->task_worker = (int16_t*)dup(g.task_worker.data(), g.task_worker.size() * 2);
  out->event_counts = (uint32_t*)dup(g.event_counts.data(), g.event_counts.size() * 4);
  out->event_first = (int32_t*)dup(g.event_first.data(), g.event_first.size() * 4);
  out->event_last = (int32_t*)dup(g.event_last.data(), g.event_last.size() * 4);
  out->event_flags = (uint8_t*)dup(g.event_flags.data(), g.event_flags.size());
  out->aot_offsets = (uint32_t*)dup(g.aot_offsets.data(), g.aot_offsets.size() * 4);
  out->aot_tasks = (uint32_t*)dup(g.aot_tasks.data(), g.aot_tasks.size() * 4);
  if (!out->task_type || !out->task_mode || !out->task_layer || !out->task_coords || !out->task_orig ||
      !out->task_dep || !out->task_trig || !out->task_worker || !out->event_counts || !out->event_first ||
      !out->event_last || !out->event_flags || !out->aot_offsets || !out->aot_tasks) {
    mpk_free_host_view(out);
    return fail(MPK_ERR_NOMEM, "host allocation failed");
  }
  return MPK_OK;
}

mpk_tgraph_header make_header(const mpk_tgraph* t) {
  mpk_tgraph_header h{};
  const Graph& g = t->g;
  h.n_tasks = g.NT; h.n_events = g.NE; h.root = g.root; h.end = g.end;
  h.n_fused = g.n_fused; h.n_empty = g.n_empty; h.n_rewrites = g.n_rewrites; h.n_aot = (int32_t)g.aot_tasks.size();
  h.batch = t->B; h.page_size = t->P; h.params = t->resolved;
  return h;
}

// Weight base pointers of a task (the device's task_ptrs, on the host).
TaskPtrs host_task_ptrs(const DevTask& d, const std::vector<const void*>& wl, const void* lm, const void* fnorm) {
  TaskPtrs r{};
  const size_t base = (size_t)(d.layer < 0 ? 0 : d.layer) * LAYER_PTRS;
  auto W = [&](int k) { return (const uint16_t*)wl[base + k]; };
  switch (d.type) {
    case MPK_TASK_QKV: r.p0 = W(W_Q); r.p1 = W(W_K); r.p2 = W(W_V); r.p3 = W(W_IN_NORM); break;
    case MPK_TASK_OPROJ: r.p0 = W(W_O); break;
    case MPK_TASK_GATEUP: r.p0 = W(W_GATE); r.p1 = W(W_UP); r.p3 = W(W_POST_NORM); break;
    case MPK_TASK_DOWN: r.p0 = W(W_DOWN); break;
    case MPK_TASK_LMHEAD: r.p0 = (const uint16_t*)lm; r.p3 = (const uint16_t*)fnorm; break;
    case MPK_TASK_ATTN_NORM: r.p0 = W(W_IN_NORM); break;
    case MPK_TASK_MLP_NORM: r.p0 = W(W_POST_NORM); break;
    case MPK_TASK_FINAL_NORM: r.p0 = (const uint16_t*)fnorm; break;
    case MPK_TASK_ATTN: r.p0 = W(W_Q_NORM); r.p1 = W(W_K_NORM); break;
    case MPK_TASK_ROUTER: r.p0 = W(W_ROUTER); r.p3 = W(W_POST_NORM); break;
    case MPK_TASK_EXPERT_GU: r.p0 = W(W_GATE); r.p1 = W(W_UP); break;
    case MPK_TASK_EXPERT_DOWN: r.p0 = W(W_DOWN); break;
    default: break;
  }
  return r;
}

void fill_args(const mpk_tgraph* t, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
               const int32_t* seq_lens, float* logits, int32_t* next_ids, KArgs* out);

// The LM head's weights: the tied embedding, except for prepared weights,
// which always carry a prepared copy of their own.
const void* lm_pointer(const mpk_tgraph* t, const mpk_weights* w) {
  return (t->cfg.tied_embedding && w->layout != 1) ? w->embed : w->lm_head;
}

// Fill the per-step arguments; when the weights changed, uploads the
// weight-pointer table and the AOT entries' resolved pointers.
int step_args(mpk_tgraph* t, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
              const int32_t* seq_lens, float* logits, int32_t* next_ids, hipStream_t stream, KArgs* out) {
  if (!t || !w || !kv || !token_ids || !seq_lens || !logits || !next_ids)
    return fail(MPK_ERR_INVALID_ARG, "null argument");
  if (t->host_only) return fail(MPK_ERR_INVALID_ARG, "graph was built host-only");
  const mpk_model_cfg& c = t->cfg;
  if (w->layout != 0 && w->layout != 1) return fail(MPK_ERR_INVALID_ARG, "weights layout must be 0 or 1");
  const bool packed = w->layout == 1;
  if (packed && (t->B == 1 || t->prm.q % 16))
    return fail(MPK_ERR_INVALID_ARG, "prepared weights (layout 1) serve only the batch > 1 graph they were made for");
  if (!w->embed || !w->final_norm || !w->layer || ((packed || !c.tied_embedding) && !w->lm_head))
    return fail(MPK_ERR_INVALID_ARG, "missing weight pointer");
  if (!kv->k_pool || !kv->v_pool || !kv->page_table || kv->n_pages < 1 || kv->max_pages_per_seq < 1)
    return fail(MPK_ERR_INVALID_ARG, "bad KV cache descriptor");
  std::vector<const void*> wl(w->layer, w->layer + (size_t)c.n_layers * LAYER_PTRS);
  for (int32_t l = 0; l < c.n_layers; ++l)
    for (int k = 0; k < LAYER_PTRS; ++k) {
      const void* p = wl[(size_t)l * LAYER_PTRS + k];
      bool optional = ((k == W_Q_NORM || k == W_K_NORM) && !c.qk_norm) || (k == W_ROUTER && c.n_experts == 0);
      if (!p && !optional) return fail(MPK_ERR_INVALID_ARG, "missing layer weight pointer");
      if (((uintptr_t)p & 15) != 0) return fail(MPK_ERR_INVALID_ARG, "weights must be 16-byte aligned");
    }
  if (((uintptr_t)w->embed & 15) || ((uintptr_t)w->lm_head & 15) || ((uintptr_t)kv->k_pool & 15) ||
      ((uintptr_t)kv->v_pool & 15))
    return fail(MPK_ERR_INVALID_ARG, "weights and KV pools must be 16-byte aligned");
  const void* lm = lm_pointer(t, w);
  std::vector<const void*> key = wl;
  key.push_back(lm);
  key.push_back(w->final_norm);
  if (key != t->h_wl) {
    if (t->last_stream) HIPCHK(hipStreamSynchronize(t->last_stream));
    HIPCHK(hipStreamSynchronize(stream));
    HIPCHK(hipMemcpy(t->d_wl, wl.data(), wl.size() * sizeof(void*), hipMemcpyHostToDevice));
    for (size_t k = 0; k + 1 < t->h_aot.size(); ++k) t->h_aot[k].w = host_task_ptrs(t->h_aot[k].t, wl, lm, w->final_norm);
    HIPCHK(hipMemcpy(t->d_aot_desc, t->h_aot.data(), t->h_aot.size() * sizeof(AotEntry), hipMemcpyHostToDevice));
    t->h_wl = key;
  }
  fill_args(t, w, token_ids, kv, seq_lens, logits, next_ids, out);
  t->last = *out;
  t->args_valid = true;
  return MPK_OK;
}

// Arguments of one step from the graph's resolved ones and the caller's
// pointers (no device work, no allocation).
void fill_args(const mpk_tgraph* t, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
               const int32_t* seq_lens, float* logits, int32_t* next_ids, KArgs* out) {
  const mpk_model_cfg& c = t->cfg;
  KArgs a = t->base;
  a.poll_sleep = 1;
  a.embed = (const uint16_t*)w->embed;
  a.lm_head = (const uint16_t*)lm_pointer(t, w);
  a.wpacked = w->layout == 1;
  a.final_norm = (const uint16_t*)w->final_norm;
  a.k_pool = (uint16_t*)kv->k_pool;
  a.v_pool = (uint16_t*)kv->v_pool;
  a.page_table = kv->page_table;
  a.n_pages = kv->n_pages;
  a.max_pages = kv->max_pages_per_seq;
  a.token_ids = token_ids;
  a.seq_lens = seq_lens;
  a.logits = logits;
  a.next_ids = next_ids;
  *out = a;
}

// Whether w holds the weight pointers the graph's descriptors were last
// resolved against (compared in place: no allocation).
bool weights_bound(const mpk_tgraph* t, const mpk_weights* w) {
  const size_t n = (size_t)t->cfg.n_layers * LAYER_PTRS;
  if (t->h_wl.size() != n + 2) return false;
  for (size_t i = 0; i < n; ++i)
    if (w->layer[i] != t->h_wl[i]) return false;
  return lm_pointer(t, w) == t->h_wl[n] && w->final_norm == t->h_wl[n + 1] && (w->layout == 1) == (t->last.wpacked != 0);
}

// Move a pointer into [from, from + n) to the same offset from `to`.
template <typename T>
void rebase(T*& p, const void* from, int64_t n, char* to) {
  const char* c = reinterpret_cast<const char*>(p);
  const char* f = reinterpret_cast<const char*>(from);
  if (p && c >= f && c < f + n) p = reinterpret_cast<T*>(to + (c - f));
}

// The paged lookahead's kernel runs the graph (weight_preload 3, and a
// pre-load area that splits into two pages).
bool lookahead(const mpk_tgraph* t) { return t->prm.lookahead && t->base.pf_segs >= 2; }

uint64_t timeout_ticks(const mpk_tgraph* t) {
  uint64_t v = (uint64_t)((double)t->timeout_ns * t->wall_khz / 1e6);
  return v < 1 ? 1 : v;
}

int build_impl(const mpk_model_cfg* cfg, int32_t batch, int32_t page_size, const mpk_build_params* params,
               mpk_tgraph** out) {
  if (out) *out = nullptr;
  if (!cfg || !out) return fail(MPK_ERR_INVALID_ARG, "null argument");
  const bool host_only = params && params->host_only;
  int n_cus = 256;
  if (!host_only) {
    int dev = 0;
    HIPCHK(hipGetDevice(&dev));
    HIPCHK(hipDeviceGetAttribute(&n_cus, hipDeviceAttributeMultiprocessorCount, dev));
  }
  Params prm;
  std::string err;
  int rc = resolve_params(*cfg, batch, page_size, params, n_cus, &prm, &err);
  if (rc) return fail(rc, err);
  if (cfg->hidden > kMaxHidden) return fail(MPK_ERR_UNSUPPORTED, "hidden larger than 8192");
  if (cfg->n_q_heads / cfg->n_kv_heads > 8) return fail(MPK_ERR_UNSUPPORTED, "more than 8 query heads per kv head");
  mpk_tgraph* t = new (std::nothrow) mpk_tgraph();
  if (!t) return fail(MPK_ERR_NOMEM, "host allocation failed");
  t->cfg = *cfg; t->B = batch; t->P = page_size; t->prm = prm; t->host_only = host_only;
  mpk_build_params r{};
  r.n_workers = prm.W; r.n_sched_waves = prm.S_sched; r.quantum = prm.q; r.t_qkv = prm.T_qkv; r.t_o = prm.T_o;
  r.t_gu = prm.T_gu; r.t_down = prm.T_down; r.t_lm = prm.T_lm; r.s_attn = prm.S_attn; r.host_only = host_only;
  r.attn_jit = prm.jit_all ? 3 : prm.jit_attn ? 1 : 2;
  r.weight_preload = prm.lookahead ? 3 : prm.preload ? 1 : 2;
  r.coarse_events = prm.coarse ? 1 : 0;
  r.k_qkv = prm.K_qkv; r.k_o = prm.K_o; r.k_down = prm.K_down;
  r.fusion_order = prm.fusion;
  r.attn_split_pages = prm.split_pages;
  if (cfg->n_experts > 0) { r.t_router = prm.T_router; r.t_egu = prm.T_egu; r.t_edown = prm.T_edown; }
  t->resolved = r;
  std::vector<TaskDef> tasks;
  decompose(*cfg, batch, prm, &tasks);
  rc = canonicalize(tasks, prm.W, prm.jit_all ? 2 : prm.jit_attn ? 1 : 0, prm.fusion, &t->g, &err);
  if (rc) { free_tgraph(t); return fail(rc, err); }
  rc = check_runtime_shape(t->g);
  if (rc) { free_tgraph(t); return rc; }
  if (!host_only) {
    rc = upload(t);
    if (rc) { std::string m = g_err; free_tgraph(t); return fail(rc, m); }
  }
  *out = t;
  return MPK_OK;
}

}  // namespace

extern "C" {

const char* mpk_last_error(void) { return g_err; }

int mpk_build_tgraph(const mpk_model_cfg* cfg, int32_t batch, int32_t page_size, mpk_tgraph** out) {
  return build_impl(cfg, batch, page_size, nullptr, out);
}

int mpk_build_tgraph_ex(const mpk_model_cfg* cfg, int32_t batch, int32_t page_size, const mpk_build_params* params,
                        mpk_tgraph** out) {
  return build_impl(cfg, batch, page_size, params, out);
}

int mpk_tgraph_info(const mpk_tgraph* g, mpk_tgraph_header* out) {
  if (!g || !out) return fail(MPK_ERR_INVALID_ARG, "null argument");
  *out = make_header(g);
  return MPK_OK;
}

int mpk_tgraph_export(const mpk_tgraph* g, mpk_tgraph_host_view* out) {
  if (!g || !out) return fail(MPK_ERR_INVALID_ARG, "null argument");
  return export_graph(g->g, make_header(g), out);
}

int mpk_build_generic_ex(const mpk_task_spec* specs, int32_t n_tasks, const mpk_region* regions, int32_t n_regions,
                         const mpk_build_params* params, mpk_tgraph_host_view* out) {
  if (!out || !params || n_tasks < 0 || n_regions < 0 || (n_tasks && !specs) || (n_regions && !regions))
    return fail(MPK_ERR_INVALID_ARG, "bad argument");
  const int32_t jit = params->attn_jit == 0 || params->attn_jit == 1 ? 1 : params->attn_jit == 2 ? 0
                      : params->attn_jit == 3 ? 2 : -1;
  if (jit < 0) return fail(MPK_ERR_INVALID_ARG, "attn_jit must be 0, 1, 2 or 3");
  std::vector<TaskDef> tasks(n_tasks);
  for (int32_t i = 0; i < n_tasks; ++i) {
    if (specs[i].type < 0 || specs[i].type == MPK_TASK_EMPTY || specs[i].type > MPK_TASK_EXPERT_DOWN)
      return fail(MPK_ERR_INVALID_ARG, "bad task type");
    tasks[i].type = specs[i].type; tasks[i].layer = specs[i].layer;
    tasks[i].c[0] = specs[i].c0; tasks[i].c[1] = specs[i].c1; tasks[i].c[2] = specs[i].c2;
  }
  for (int32_t i = 0; i < n_regions; ++i) {
    const mpk_region& r = regions[i];
    if (r.task < 0 || r.task >= n_tasks) return fail(MPK_ERR_INVALID_ARG, "region names a missing task");
    Box b;
    b.tensor = r.tensor;
    for (int k = 0; k < 4; ++k) { b.lo[k] = r.lo[k]; b.hi[k] = r.hi[k]; }
    (r.is_out ? tasks[r.task].outs : tasks[r.task].ins).push_back(b);
  }
  Graph g;
  std::string err;
  int rc = canonicalize(tasks, params->n_workers, jit, params->fusion_order, &g, &err);
  if (rc) return fail(rc, err);
  mpk_tgraph_header h{};
  h.n_tasks = g.NT; h.n_events = g.NE; h.root = g.root; h.end = g.end; h.n_fused = g.n_fused;
  h.n_empty = g.n_empty; h.n_rewrites = g.n_rewrites; h.n_aot = (int32_t)g.aot_tasks.size();
  h.params = *params;
  h.params.host_only = 1;
  h.params.attn_jit = jit == 1 ? 1 : jit == 0 ? 2 : 3;
  return export_graph(g, h, out);
}

int mpk_build_generic(const mpk_task_spec* specs, int32_t n_tasks, const mpk_region* regions, int32_t n_regions,
                      int32_t n_workers, mpk_tgraph_host_view* out) {
  mpk_build_params p{};
  p.n_workers = n_workers;
  p.attn_jit = 1;
  return mpk_build_generic_ex(specs, n_tasks, regions, n_regions, &p, out);
}

void mpk_free_host_view(mpk_tgraph_host_view* v) {
  if (!v) return;
  void* ptrs[] = {v->task_type, v->task_mode, v->task_layer, v->task_coords, v->task_orig, v->task_dep, v->task_trig,
                  v->task_worker, v->event_counts, v->event_first, v->event_last, v->event_flags, v->aot_offsets,
                  v->aot_tasks};
  for (void* p : ptrs) std::free(p);
  std::memset(v, 0, sizeof(*v));
}

int mpk_decode_step(mpk_tgraph* g, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
                    const int32_t* seq_lens, float* logits, int32_t* next_ids, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  KArgs a;
  int rc = step_args(g, w, token_ids, kv, seq_lens, logits, next_ids, s, &a);
  if (rc) return rc;
  const uint32_t epoch = ++g->epoch;
  hipError_t e = launch_megakernel(a, epoch, timeout_ticks(g), g->grid, s, lookahead(g));
  if (e != hipSuccess) { --g->epoch; return hip_fail(e, "mega-kernel launch"); }
  g->last_stream = s;
  return MPK_OK;
}

// The matrices of a prepared copy, in order: per layer q, k, v, o, gate/up
// (interleaved), down; then the LM head.  Each entry: the source(s), rows,
// contraction length and offset in the buffer.
struct PackPlan {
  struct Item { const void* a; const void* b; int64_t N, K, off; int layer, slot; };
  std::vector<Item> items;
  int64_t bytes = 0;
};
PackPlan pack_plan(const mpk_tgraph* t, const mpk_weights* w) {
  const mpk_model_cfg& c = t->cfg;
  const int64_t H = c.hidden, F = c.ffn, hq = c.n_q_heads, hkv = c.n_kv_heads, d = c.head_dim;
  PackPlan p;
  auto add = [&](const void* a, const void* b, int64_t N, int64_t K, int layer, int slot) {
    p.items.push_back({a, b, N, K, p.bytes, layer, slot});
    p.bytes = align256(p.bytes + packed_bytes(N, K));
  };
  for (int l = 0; l < c.n_layers; ++l) {
    const void* const* L = w ? w->layer + (size_t)l * LAYER_PTRS : nullptr;
    add(L ? L[W_Q] : nullptr, nullptr, hq * d, H, l, W_Q);
    add(L ? L[W_K] : nullptr, nullptr, hkv * d, H, l, W_K);
    add(L ? L[W_V] : nullptr, nullptr, hkv * d, H, l, W_V);
    add(L ? L[W_O] : nullptr, nullptr, H, hq * d, l, W_O);
    add(L ? L[W_GATE] : nullptr, L ? L[W_UP] : nullptr, 2 * F, H, l, W_GATE);
    add(L ? L[W_DOWN] : nullptr, nullptr, H, F, l, W_DOWN);
  }
  add(w ? (c.tied_embedding ? w->embed : w->lm_head) : nullptr, nullptr, c.vocab, H, -1, -1);
  return p;
}

int mpk_prepared_weights_bytes(const mpk_tgraph* g, size_t* bytes) {
  if (!g || !bytes) return fail(MPK_ERR_INVALID_ARG, "null argument");
  *bytes = (size_t)pack_plan(g, nullptr).bytes;
  return MPK_OK;
}

int mpk_prepare_weights(const mpk_tgraph* g, const mpk_weights* in, void* dst, size_t dst_bytes,
                        const void** packed_layers, mpk_weights* packed, void* stream) {
  if (!g || !in || !dst || !packed_layers || !packed || !in->layer || !in->embed || !in->final_norm)
    return fail(MPK_ERR_INVALID_ARG, "null argument");
  if (in->layout != 0) return fail(MPK_ERR_INVALID_ARG, "the input weights must be layout 0");
  if (g->B == 1) return fail(MPK_ERR_UNSUPPORTED, "batch-1 graphs stream whole weight rows: nothing to prepare");
  if (g->cfg.n_experts > 0) return fail(MPK_ERR_UNSUPPORTED, "prepared weights are not implemented for expert layers");
  if (g->prm.q % 16) return fail(MPK_ERR_UNSUPPORTED, "prepared weights need a column quantum that is a multiple of 16");
  if (((uintptr_t)dst & 255) != 0) return fail(MPK_ERR_INVALID_ARG, "dst must be 256-byte aligned");
  const mpk_model_cfg& c = g->cfg;
  if (!c.tied_embedding && !in->lm_head) return fail(MPK_ERR_INVALID_ARG, "missing LM head");
  const PackPlan p = pack_plan(g, in);
  if ((int64_t)dst_bytes < p.bytes) return fail(MPK_ERR_INVALID_ARG, "dst smaller than mpk_prepared_weights_bytes");
  for (const auto& it : p.items)
    if (!it.a || (it.slot == W_GATE && !it.b) || ((uintptr_t)it.a & 15) || ((uintptr_t)it.b & 15))
      return fail(MPK_ERR_INVALID_ARG, "missing or misaligned weight matrix");
  hipStream_t s = (hipStream_t)stream;
  char* base = static_cast<char*>(dst);
  for (size_t i = 0; i < (size_t)c.n_layers * LAYER_PTRS; ++i) packed_layers[i] = in->layer[i];
  const void* lm = nullptr;
  for (const auto& it : p.items) {
    hipError_t e = launch_pack(it.a, it.b, it.N, it.K, base + it.off, s);
    if (e != hipSuccess) return hip_fail(e, "weight repack");
    if (it.layer < 0) {
      lm = base + it.off;
    } else {
      packed_layers[(size_t)it.layer * LAYER_PTRS + it.slot] = base + it.off;
      if (it.slot == W_GATE) packed_layers[(size_t)it.layer * LAYER_PTRS + W_UP] = base + it.off;
    }
  }
  packed->embed = in->embed;
  packed->lm_head = lm;
  packed->final_norm = in->final_norm;
  packed->layer = packed_layers;
  packed->layout = 1;
  return MPK_OK;
}

int mpk_decode_step_noalloc(mpk_tgraph* g, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
                            const int32_t* seq_lens, float* logits, int32_t* next_ids, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  if (!g || !w || !w->layer || !kv || !token_ids || !seq_lens || !logits || !next_ids)
    return fail(MPK_ERR_INVALID_ARG, "null argument");
  if (g->host_only) return fail(MPK_ERR_INVALID_ARG, "graph was built host-only");
  const size_t need = (size_t)g->rt_bytes + (size_t)g->act_bytes;
  if (need > scratch_capacity()) {
    std::snprintf(g_err, sizeof(g_err), "the step needs %zu bytes of scratch, more than the %zu of the static area",
                  need, scratch_capacity());
    return MPK_ERR_UNSUPPORTED;
  }
  if (!weights_bound(g, w))
    return fail(MPK_ERR_INVALID_ARG, "weights not bound to this graph: run mpk_decode_step once with these weights");
  if (!kv->k_pool || !kv->v_pool || !kv->page_table || kv->n_pages < 1 || kv->max_pages_per_seq < 1 ||
      ((uintptr_t)kv->k_pool & 15) || ((uintptr_t)kv->v_pool & 15) || ((uintptr_t)w->embed & 15))
    return fail(MPK_ERR_INVALID_ARG, "bad KV cache descriptor or embedding pointer");
  int dev = -1;
  HIPCHK(hipGetDevice(&dev));
  if (dev != g->device) return fail(MPK_ERR_INVALID_ARG, "the graph's device is not the current device");
  void* base = nullptr;
  hipError_t e = scratch_address(dev, &base);
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  KArgs a;
  fill_args(g, w, token_ids, kv, seq_lens, logits, next_ids, &a);
  // the runtime arena at the start of the scratch area, the activations right after it
  // (both blocks keep the graph's own layout; the status word stays the graph's)
  char* rt = static_cast<char*>(base);
  char* act = rt + g->rt_bytes;
  rebase(a.ev_cnt, g->d_rt, g->rt_bytes, rt);
  rebase(a.ev_sub, g->d_rt, g->rt_bytes, rt);
  rebase(a.sched_ring, g->d_rt, g->rt_bytes, rt);
  rebase(a.sched_tail, g->d_rt, g->rt_bytes, rt);
  rebase(a.jit_ring, g->d_rt, g->rt_bytes, rt);
  rebase(a.state, g->d_rt, g->rt_bytes, rt);
  rebase(a.arrive, g->d_rt, g->rt_bytes, rt);
  for (float** p : {&a.e, &a.hf, &a.r, &a.h, &a.qkv, &a.part, &a.attn, &a.o, &a.s, &a.h2, &a.a, &a.dn, &a.rlog})
    rebase(*p, g->d_act, g->act_bytes, act);
  rebase(a.pmax, g->d_act, g->act_bytes, act);
  rebase(a.route, g->d_act, g->act_bytes, act);
  a.trace = nullptr;
  a.trace_count = nullptr;
  a.trace_cap = 0;
  // counters, rings and arrivals start at zero, so the step runs as epoch 1
  e = scratch_zero(rt, (size_t)g->rt_bytes, s);
  if (e != hipSuccess) return hip_fail(e, "scratch clear");
  e = launch_megakernel(a, 1u, timeout_ticks(g), g->grid, s, lookahead(g));
  if (e != hipSuccess) return hip_fail(e, "mega-kernel launch");
  g->last_stream = s;
  return MPK_OK;
}

int mpk_decode_step_baseline(mpk_tgraph* g, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
                             const int32_t* seq_lens, float* logits, int32_t* next_ids, void* stream,
                             int32_t use_hipgraph) {
  hipStream_t s = (hipStream_t)stream;
  KArgs a;
  int rc = step_args(g, w, token_ids, kv, seq_lens, logits, next_ids, s, &a);
  if (rc) return rc;
  g->last_stream = s;
  if (!use_hipgraph) {
    for (auto& op : g->ops) {
      if (!op.second) continue;
      hipError_t e = launch_baseline_op(a, g->d_lists + op.first, op.second, s);
      if (e != hipSuccess) return hip_fail(e, "baseline launch");
    }
    return MPK_OK;
  }
  std::vector<uintptr_t> key = {(uintptr_t)a.embed, (uintptr_t)a.lm_head, (uintptr_t)a.final_norm,
                                (uintptr_t)a.k_pool, (uintptr_t)a.v_pool, (uintptr_t)a.page_table,
                                (uintptr_t)a.n_pages, (uintptr_t)a.max_pages, (uintptr_t)a.token_ids,
                                (uintptr_t)a.seq_lens, (uintptr_t)a.logits, (uintptr_t)a.next_ids};
  for (auto p : g->h_wl) key.push_back((uintptr_t)p);
  if (!g->gexec || key != g->gkey) {
    if (g->gexec) { (void)hipGraphExecDestroy(g->gexec); g->gexec = nullptr; }
    if (!g->cap_stream) HIPCHK(hipStreamCreateWithFlags(&g->cap_stream, hipStreamNonBlocking));
    HIPCHK(hipStreamBeginCapture(g->cap_stream, hipStreamCaptureModeThreadLocal));
    for (auto& op : g->ops) {
      if (!op.second) continue;
      hipError_t e = launch_baseline_op(a, g->d_lists + op.first, op.second, g->cap_stream);
      if (e != hipSuccess) {
        hipGraph_t dummy;
        (void)hipStreamEndCapture(g->cap_stream, &dummy);
        return hip_fail(e, "baseline capture");
      }
    }
    hipGraph_t graph;
    HIPCHK(hipStreamEndCapture(g->cap_stream, &graph));
    hipError_t e = hipGraphInstantiate(&g->gexec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) { g->gexec = nullptr; return hip_fail(e, "hipGraphInstantiate"); }
    g->gkey = key;
  }
  HIPCHK(hipGraphLaunch(g->gexec, s));
  return MPK_OK;
}

int mpk_read_tensor(const mpk_tgraph* g, int32_t tensor, void* dst, size_t bytes) {
  if (!g || !dst) return fail(MPK_ERR_INVALID_ARG, "null argument");
  if (g->host_only) return fail(MPK_ERR_INVALID_ARG, "graph was built host-only");
  if (tensor < 0 || tensor >= (int32_t)g->tensors.size() || !g->tensors[tensor].p)
    return fail(MPK_ERR_INVALID_ARG, "tensor id names no library-owned buffer");
  if ((int64_t)bytes != g->tensors[tensor].bytes) return fail(MPK_ERR_INVALID_ARG, "byte count does not match tensor");
  HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemcpy(dst, g->tensors[tensor].p, bytes, hipMemcpyDeviceToHost));
  return MPK_OK;
}

int mpk_reset_tgraph(mpk_tgraph* g) {
  if (!g || g->host_only) return fail(MPK_ERR_INVALID_ARG, g ? "host-only graph" : "null argument");
  int dev = -1;
  HIPCHK(hipGetDevice(&dev));
  if (dev != g->device) return fail(MPK_ERR_INVALID_ARG, "the graph's device is not the current device");
  if (g->last_stream) HIPCHK(hipStreamSynchronize(g->last_stream));
  else HIPCHK(hipDeviceSynchronize());
  HIPCHK(hipMemset(g->d_rt, 0, (size_t)g->rt_bytes));
  HIPCHK(hipDeviceSynchronize());
  g->epoch = 0;
  return MPK_OK;
}

int mpk_set_watchdog(mpk_tgraph* g, uint64_t timeout_ns) {
  if (!g) return fail(MPK_ERR_INVALID_ARG, "null argument");
  g->timeout_ns = timeout_ns ? timeout_ns : 2000000000ull;
  return MPK_OK;
}

int mpk_get_status(mpk_tgraph* g, mpk_status_word* out) {
  if (!g || !out) return fail(MPK_ERR_INVALID_ARG, "null argument");
  std::memset(out, 0, sizeof(*out));
  if (g->host_only) return MPK_OK;
  if (g->last_stream) HIPCHK(hipStreamSynchronize(g->last_stream));
  else HIPCHK(hipDeviceSynchronize());
  StatusWord s;
  HIPCHK(hipMemcpy(&s, g->d_status, sizeof(s), hipMemcpyDeviceToHost));
  out->code = s.code; out->wg = s.wg; out->task = s.task; out->event = s.event; out->counter = s.counter;
  out->target = s.target;
  return MPK_OK;
}

int mpk_set_trace(mpk_tgraph* g, int32_t enable) {
  if (!g) return fail(MPK_ERR_INVALID_ARG, "null argument");
  if (g->host_only) return fail(MPK_ERR_INVALID_ARG, "graph was built host-only");
  if (g->last_stream) HIPCHK(hipStreamSynchronize(g->last_stream));
  HIPCHK(hipDeviceSynchronize());
  if (g->d_trace) { HIPCHK(hipFree(g->d_trace)); g->d_trace = nullptr; }
  g->base.trace = nullptr; g->base.trace_count = nullptr; g->base.trace_cap = 0;
  if (enable) {
    // a worker runs at most its AOT list plus every JIT task of a step
    int32_t max_aot = 0, n_jit = 0;
    for (int32_t w = 0; w < g->prm.W; ++w)
      max_aot = std::max<int32_t>(max_aot, (int32_t)(g->g.aot_offsets[w + 1] - g->g.aot_offsets[w]));
    for (int32_t i = 0; i < g->g.NT; ++i) n_jit += g->g.task_mode[i] == MPK_MODE_JIT;
    g->trace_cap = max_aot + n_jit;
    const int64_t rec_bytes = align256((int64_t)g->prm.W * g->trace_cap * (int64_t)sizeof(TraceRec));
    HIPCHK(hipMalloc(&g->d_trace, rec_bytes + (int64_t)g->prm.W * 4));
    HIPCHK(hipMemset(g->d_trace, 0, rec_bytes + (int64_t)g->prm.W * 4));
    g->base.trace = (TraceRec*)g->d_trace;
    g->base.trace_count = (uint32_t*)((char*)g->d_trace + rec_bytes);
    g->base.trace_cap = g->trace_cap;
  }
  return MPK_OK;
}

int mpk_read_trace(mpk_tgraph* g, mpk_trace_record* out, int32_t capacity, int32_t* count, double* ticks_per_us) {
  if (!g || !count || (capacity > 0 && !out)) return fail(MPK_ERR_INVALID_ARG, "null argument");
  if (!g->d_trace) return fail(MPK_ERR_INVALID_ARG, "tracing is off");
  if (g->last_stream) HIPCHK(hipStreamSynchronize(g->last_stream));
  HIPCHK(hipDeviceSynchronize());
  const int32_t W = g->prm.W;
  std::vector<uint32_t> cnt(W);
  HIPCHK(hipMemcpy(cnt.data(), g->base.trace_count, (size_t)W * 4, hipMemcpyDeviceToHost));
  std::vector<TraceRec> recs((size_t)W * g->trace_cap);
  HIPCHK(hipMemcpy(recs.data(), g->base.trace, recs.size() * sizeof(TraceRec), hipMemcpyDeviceToHost));
  int32_t n = 0;
  for (int32_t w = 0; w < W; ++w)
    for (uint32_t k = 0; k < std::min<uint32_t>(cnt[w], (uint32_t)g->trace_cap); ++k) {
      if (n < capacity) {
        const TraceRec& r = recs[(size_t)w * g->trace_cap + k];
        out[n] = mpk_trace_record{r.task, r.worker, r.t_wait, r.t_start, r.t_end, r.t_done, {r.t_mark[0], r.t_mark[1]}};
      }
      ++n;
    }
  *count = std::min(n, capacity);
  if (ticks_per_us) *ticks_per_us = g->wall_khz / 1000.0;
  return n > capacity ? fail(MPK_ERR_INVALID_ARG, "capacity too small") : MPK_OK;
}

int mpk_time_tasks(mpk_tgraph* g, const int32_t* tasks, int32_t n, int32_t reps, int32_t cold, uint64_t* ticks,
                   double* ticks_per_us) {
  if (!g || !tasks || !ticks || n < 1 || reps < 1) return fail(MPK_ERR_INVALID_ARG, "bad argument");
  if (g->host_only || !g->args_valid) return fail(MPK_ERR_INVALID_ARG, "run mpk_decode_step on this graph first");
  for (int32_t i = 0; i < n; ++i)
    if (tasks[i] < 0 || tasks[i] >= g->g.NT) return fail(MPK_ERR_INVALID_ARG, "task index out of range");
  HIPCHK(hipDeviceSynchronize());
  void* buf = nullptr;
  HIPCHK(hipMalloc(&buf, (size_t)n * 8));
  unsigned long long* d_out = (unsigned long long*)buf;
  hipError_t e = hipMemset(d_out, 0, (size_t)n * 8);
  for (int32_t i = 0; i < n && e == hipSuccess; ++i)
    for (int32_t r = 0; r < reps && e == hipSuccess; ++r) e = launch_time_task(g->last, tasks[i], cold != 0, d_out + i, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(ticks, d_out, (size_t)n * 8, hipMemcpyDeviceToHost);
  // timed attention splits counted arrivals outside a step: back to 0 for the next step
  if (e == hipSuccess) e = hipMemset(g->d_arrive, 0, (size_t)g->arrive_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  for (int32_t i = 0; i < n && e == hipSuccess; ++i) ticks[i] /= (uint64_t)reps;
  (void)hipFree(buf);
  if (e != hipSuccess) return hip_fail(e, "mpk_time_tasks");
  if (ticks_per_us) *ticks_per_us = g->wall_khz / 1000.0;
  return MPK_OK;
}

int mpk_run_tasks(mpk_tgraph* g, const int32_t* tasks, int32_t n, int32_t poison) {
  if (!g || !tasks || n < 1) return fail(MPK_ERR_INVALID_ARG, "bad argument");
  if (g->host_only || !g->args_valid) return fail(MPK_ERR_INVALID_ARG, "run mpk_decode_step on this graph first");
  for (int32_t i = 0; i < n; ++i)
    if (tasks[i] < 0 || tasks[i] >= g->g.NT) return fail(MPK_ERR_INVALID_ARG, "task index out of range");
  HIPCHK(hipDeviceSynchronize());
  // all-ones bytes: every fp32 activation reads as a NaN, every partial
  // argmax as (NaN, -1)
  if (poison) HIPCHK(hipMemset(g->d_act, 0xFF, (size_t)g->act_bytes));
  HIPCHK(hipMemset(g->d_arrive, 0, (size_t)g->arrive_bytes));
  void* buf = nullptr;
  HIPCHK(hipMalloc(&buf, 8));
  hipError_t e = hipSuccess;
  for (int32_t i = 0; i < n && e == hipSuccess; ++i)
    e = launch_time_task(g->last, tasks[i], false, (unsigned long long*)buf, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipFree(buf);
  if (e != hipSuccess) return hip_fail(e, "mpk_run_tasks");
  return MPK_OK;
}

void mpk_destroy_tgraph(mpk_tgraph* g) { free_tgraph(g); }

}  // extern "C"
