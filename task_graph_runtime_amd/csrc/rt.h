// Device-side data layout of a built tGraph and the argument block of the
// kernels.  Shared by the host code that fills it (capi.cpp) and the HIP
// kernels that read it (megakernel.hip, tasks.h).
#pragma once

#include <cstdint>

namespace mpk {

// One linearised task, 32 bytes (two 16-byte loads / one s_load_dwordx8).
// a0..a3 are the task's operands: projection tiles (a0, a1) = output column
// range, a2 = tile index; per-request tasks a0 = b, a1 = kv group, a2 = split.
struct alignas(16) DevTask {
  uint8_t type;
  uint8_t mode;
  int16_t layer;
  int32_t dep;
  int32_t trig;
  int32_t a0, a1, a2, a3;
  int32_t rsv;
};
static_assert(sizeof(DevTask) == 32, "DevTask must be 32 bytes");

// One linearised event: fires when `counts` triggers arrive (per step);
// its dependent tasks are [first, last].
struct alignas(16) DevEvent {
  uint32_t counts;
  int32_t first;
  int32_t last;
  uint32_t flags;
};
static_assert(sizeof(DevEvent) == 16, "DevEvent must be 16 bytes");

// Per-(request, LM-head tile) partial argmax.
struct PMax {
  float v;
  int32_t i;
};

enum { LAYER_PTRS = 11 };
enum { W_IN_NORM = 0, W_Q, W_K, W_V, W_Q_NORM, W_K_NORM, W_O, W_POST_NORM, W_GATE, W_UP, W_DOWN };

// Status word written by the kernel (layout of mpk_status_word).
struct StatusWord {
  int32_t code, wg, task, event;
  uint32_t counter, target;
};

constexpr int kThreads = 512;   // threads per workgroup (8 wavefronts)
constexpr int kWaves = kThreads / 64;
constexpr int kMaxBatch = 16;
constexpr int kMaxHidden = 8192;

struct KArgs {
  // graph
  const DevTask* tasks;
  const DevEvent* events;
  const uint32_t* aot_off;
  const uint32_t* aot_tasks;
  uint32_t* ev_cnt;                 // monotonic event counters (target counts * epoch)
  unsigned long long* sched_ring;   // [n_sched][sched_cap] (seq << 32 | event)
  uint32_t* sched_tail;             // [n_sched] producer reservation counters
  unsigned long long* jit_ring;     // [n_workers][jit_cap] (seq << 32 | task)
  uint32_t* state;                  // persistent runtime state, see megakernel.hip
  uint32_t sched_cap, jit_cap;
  int32_t n_workers, n_sched, n_sched_wgs;
  int32_t root_event, end_event;
  uint32_t epoch;
  uint64_t timeout_ticks;
  StatusWord* status;
  // model
  int32_t L, H, hq, hkv, d, F, V, G, Sg, B, P, S_attn, T_lm, qk_norm, max_seq, max_pages, n_pages;
  float eps, theta;
  // weights (bf16 bits)
  const uint16_t* const* wl;        // device array [L * LAYER_PTRS]
  const uint16_t* embed;
  const uint16_t* lm_head;
  const uint16_t* final_norm;
  // KV cache
  uint16_t* k_pool;
  uint16_t* v_pool;
  const int32_t* page_table;
  // io
  const int32_t* token_ids;
  const int32_t* seq_lens;
  float* logits;
  int32_t* next_ids;
  // activations; per-layer tensors are [L][...] with the strides below (elements)
  // (all fp32: only the weights and the KV cache, the caller's formats, are bf16)
  float* e;
  float* hf;
  PMax* pmax;
  float* r;  float* h;  float* qkv;  float* q;  float* part;  float* attn;
  float* o;  float* s;  float* h2;  float* a;  float* dn;
  int64_t st_bh, st_qkv, st_q, st_part, st_a;
};

}  // namespace mpk
