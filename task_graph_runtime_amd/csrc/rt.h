// Device-side data layout of a built tGraph and the argument block of the
// kernels.  Shared by the host code that fills it (capi.cpp) and the HIP
// kernels that read it (megakernel.hip, tasks.h).
#pragma once

#include <cstdint>

// Device pointers of the argument block and of the records below are typed
// as global-address-space pointers in device code (same 64-bit layout as the
// host's plain pointers), so that every access through them is a global --
// not a flat -- memory instruction: flat loads also count against the LDS
// wait counter.
#if defined(__HIP_DEVICE_COMPILE__)
#define MPK_GLOBAL __attribute__((address_space(1)))
#else
#define MPK_GLOBAL
#endif

namespace mpk {

// One linearised task, 32 bytes (two 16-byte loads / one s_load_dwordx8).
// a0..a2 are the task's operands: projection tiles (a0, a1) = output column
// range, a2 = tile index (under a k-split into K ranges, k range a2 % K);
// attention a0 = slot, a1 = kv group, a2 = the q/k/v projection's plane
// count; per-request norms and the embedding a0 = b.
// id is the task's own linear index and dep_counts the trigger count of its
// dependent event, so that a worker holding the descriptor needs no further
// load before it can wait.
struct alignas(16) DevTask {
  uint8_t type;
  uint8_t mode;
  int16_t layer;
  int32_t dep;
  int32_t trig;
  int32_t a0, a1, a2;
  int32_t id;
  uint32_t dep_counts;
};
static_assert(sizeof(DevTask) == 32, "DevTask must be 32 bytes");

// Weight base pointers a task reads (resolved from the per-layer pointer
// table): QKV q/k/v, GATEUP gate/up, other projections and the LM head p0;
// p3 the gain of the RMSNorm a batch-1 QKV / GATEUP / LM-head tile applies to
// its input; norm tasks their gain p0; attention the q and k gains p0, p1.
struct TaskPtrs {
  MPK_GLOBAL const uint16_t* p0;
  MPK_GLOBAL const uint16_t* p1;
  MPK_GLOBAL const uint16_t* p2;
  MPK_GLOBAL const uint16_t* p3;
};

// One entry of a worker's ahead-of-time list: the task's descriptor and its
// resolved weight pointers (refreshed by the host when the weights change),
// 64 bytes.
struct alignas(64) AotEntry {
  DevTask t;
  TaskPtrs w;
};
static_assert(sizeof(AotEntry) == 64, "AotEntry must be 64 bytes");

// One linearised event: fires when `counts` triggers arrive (per step);
// its dependent tasks are [first, last].
struct alignas(16) DevEvent {
  uint32_t counts;
  int32_t first;
  int32_t last;
  uint32_t flags;
};
static_assert(sizeof(DevEvent) == 16, "DevEvent must be 16 bytes");

// Two-level events.  An event with at least kTwoLevelMin producers counts
// its arrivals on kEvSub sub-counters first (the producer with linear index
// t adds to sub-counter t mod kEvSub); the arrival that completes a
// sub-counter's quota adds 1 to the event counter, which then needs one
// arrival per non-empty sub-counter.  Simultaneous returning atomics on one
// address serialise (256 at once: 1.6 us mean, 3 us worst, against 0.35 us
// on distinct addresses), and a projection's tiles finish close together.
// The device copy of such an event carries kEvTwoLevel in its flags and the
// number of non-empty sub-counters as its count.
constexpr int kEvSub = 8;
constexpr uint32_t kTwoLevelMin = 64;
constexpr uint32_t kEvTwoLevel = 4;
// An event with one producer whose consumers are all EMPTY tasks (the e' of
// a normalisation rewrite): its one arrival always fires it and nothing polls
// its counter, so the arrival takes no atomic.
constexpr uint32_t kEvSole = 8;

// Scheduler ring entry: seq << 32 | chunk << 20 | event (see the megakernel).
constexpr int kJitEventBits = 20, kJitChunkBits = 12;

// Per-(request, LM-head tile) partial argmax.
struct PMax {
  float v;
  int32_t i;
};

enum { LAYER_PTRS = 12 };
enum { W_IN_NORM = 0, W_Q, W_K, W_V, W_Q_NORM, W_K_NORM, W_O, W_POST_NORM, W_GATE, W_UP, W_DOWN, W_ROUTER };

// One trace record (layout of mpk_trace_record).
struct TraceRec {
  int32_t task, worker;
  uint64_t t_wait, t_start, t_end, t_done;
  uint64_t t_mark[2];
};

// Status word written by the kernel (layout of mpk_status_word).
struct StatusWord {
  int32_t code, wg, task, event;
  uint32_t counter, target;
};

constexpr int kThreads = 512;   // threads per workgroup (8 wavefronts)
constexpr int kWaves = kThreads / 64;
// LDS of a workgroup: the whole 160 KB of a compute unit.  The top kLdsTop
// bytes hold the runtime's control words and reduction scratch; the rest is
// laid out per graph by the host (KArgs::lds_*).
constexpr int kLdsBytes = 160 * 1024;
constexpr int kLdsTop = 512;
constexpr int kPfWaves = kWaves - 1;   // wavefronts that pre-load weights (all but the polling one)
constexpr int kMaxPfSegs = 16;         // pre-loaded 1 KB segments per wavefront, at most
constexpr int kMaxBatch = 16;
constexpr int kMaxTopK = 16;     // experts per token, at most (mixture of experts)
constexpr int kMaxExperts = 256;
constexpr int kMaxHidden = 8192;


// LDS of an expert tile's routing (mixture of experts): each request's
// chosen experts and their weights, the set of experts the batch chose, and
// the route of the tile's expert slot (expert, -1 when the slot is idle;
// token count; tokens in ascending order; their weights); the B x E router
// logits follow it.
struct MoeLds {
  int32_t cid[kMaxBatch][kMaxTopK];
  float cw[kMaxBatch][kMaxTopK];
  uint32_t mask[kMaxExperts / 32];
  int32_t e, n;
  int32_t tok[kMaxBatch];
  float w[kMaxBatch];
};

// Kernel arguments.  One copy lives in device memory per graph (refreshed
// only when a caller pointer changes); the kernels receive its address, the
// step's epoch and the watchdog limit.
struct KArgs {
  // graph
  MPK_GLOBAL const DevTask* tasks;
  MPK_GLOBAL const DevEvent* events;
  MPK_GLOBAL const uint32_t* aot_off;          // [n_workers + 1] offsets into aot_desc
  MPK_GLOBAL const AotEntry* aot_desc;         // per worker, its AOT tasks in FIFO order
  MPK_GLOBAL uint32_t* ev_cnt;                 // monotonic event counters (target counts * epoch)
  MPK_GLOBAL uint32_t* ev_sub;                 // [NE][kEvSub] sub-counters of two-level events
  MPK_GLOBAL const uint16_t* ev_quota;         // [NE][kEvSub] arrivals per sub-counter and step
  MPK_GLOBAL unsigned long long* sched_ring;   // [n_sched][sched_cap] (seq << 32 | event)
  MPK_GLOBAL uint32_t* sched_tail;             // [n_sched] producer reservation counters
  MPK_GLOBAL unsigned long long* jit_ring;     // [n_workers][jit_cap] (seq << 32 | task)
  MPK_GLOBAL uint32_t* state;                  // persistent runtime state, see megakernel.hip
  uint32_t sched_cap, jit_cap;
  int32_t n_workers, n_sched, n_sched_wgs;
  int32_t root_event, end_event;
  int32_t poll_sleep;                          // s_sleep(1) periods between two polls of a waiting worker
  // per-graph LDS layout (bytes): the staging area [0, lds_acc) (activation
  // vectors, attention merge and combine records), projection accumulators
  // [lds_acc, lds_pf), the weight pre-load area of pf_segs 1 KB segments for
  // each of the kPfWaves pre-loading wavefronts at lds_pf (pf_segs = 0: no
  // pre-load), and an attention split's page ids at lds_pid
  int32_t lds_acc, lds_pf, pf_segs, lds_pid;
  MPK_GLOBAL StatusWord* status;
  MPK_GLOBAL TraceRec* trace;                  // null: tracing off; else [n_workers][trace_cap]
  MPK_GLOBAL uint32_t* trace_count;            // [n_workers] records written in the last step
  int32_t trace_cap;
  // model
  int32_t L, H, hq, hkv, d, F, V, G, Sg, B, P, S_attn, T_lm, qk_norm, max_seq, max_pages, n_pages;
  float eps, theta;
  MPK_GLOBAL const double* inv_freq;           // [head_dim / 2]: theta^(-2i/head_dim), fp64
  // weights (bf16 bits)
  MPK_GLOBAL const uint16_t* MPK_GLOBAL const* wl;   // device array [L * LAYER_PTRS]
  MPK_GLOBAL const uint16_t* embed;
  MPK_GLOBAL const uint16_t* lm_head;
  MPK_GLOBAL const uint16_t* final_norm;
  // KV cache
  MPK_GLOBAL uint16_t* k_pool;
  MPK_GLOBAL uint16_t* v_pool;
  MPK_GLOBAL const int32_t* page_table;
  // io
  MPK_GLOBAL const int32_t* token_ids;
  MPK_GLOBAL const int32_t* seq_lens;
  MPK_GLOBAL float* logits;
  MPK_GLOBAL int32_t* next_ids;
  // activations; per-layer tensors are [L][...] with the strides below (elements)
  // (all fp32: only the weights and the KV cache, the caller's formats, are bf16)
  // (e, hf, h and h2 exist at batch > 1 only, where the norms are tasks)
  MPK_GLOBAL float* e;
  MPK_GLOBAL float* hf;
  MPK_GLOBAL PMax* pmax;
  MPK_GLOBAL float* r;
  MPK_GLOBAL float* h;
  MPK_GLOBAL float* qkv;
  MPK_GLOBAL float* part;
  MPK_GLOBAL float* attn;
  MPK_GLOBAL float* o;
  MPK_GLOBAL float* s;
  MPK_GLOBAL float* h2;
  MPK_GLOBAL float* a;
  MPK_GLOBAL float* dn;
  int64_t st_bh, st_qkv, st_q, st_part, st_a, st_o, st_dn;
  // k-split of the QKV, O and down projections at batch > 1: qkv, o and dn
  // hold Kq, Ko and Kd planes of [B][...] each, the output is their sum
  int32_t Kq, Ko, Kd;
  // split arrivals per (layer, request, kv group): the attention split that
  // brings one to S_attn is the last of its (b, g), merges the partials and
  // resets it to 0, so it is 0 between steps
  MPK_GLOBAL uint32_t* arrive;
  // the smallest split an attention task takes, in KV pages (see attn_slot)
  int32_t attn_min_pages;
  // 1: the projection weights are prepared (matrix-core operand order, see
  // packed_block in tasks.h; batch > 1 only)
  int32_t wpacked;
  // mixture of experts (E = 0: dense): experts, top k, expert width, whether
  // the top-k weights are renormalised, expert slots per layer; per-layer
  // strides of the router logits [B][E] and route records [M][2 + 2B];
  // lds_moe: the LDS area of an expert tile's routing (MoeLds in tasks.h)
  int32_t E, topk, Fe, norm_topk, M, lds_moe;
  int64_t st_rlog, st_route;
  MPK_GLOBAL float* rlog;
  MPK_GLOBAL int32_t* route;
};

}  // namespace mpk
