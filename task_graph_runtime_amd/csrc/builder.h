// Host-side tGraph builder: operator decomposition into tile tasks, overlap
// dependencies, event fusion, normalisation, BFS linearisation, JIT/AOT
// classification and AOT placement.  Plain C++17, no HIP: it runs (and is
// tested) without a GPU.
//
// Method: "MPK: A Compiler and Runtime for Mega-Kernelizing Tensor Programs
// -- L2", section 2 (Q2), section 4 (Def 4.1, Def 4.2, the "6 minimum
// checks", design-space table) and section 7 ("Empty tasks as
// degree-reduction glue"); dependency rule from the author's HN comment
// (item 2: an edge iff the producer's outputs overlap the consumer's inputs).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "mpk.h"

namespace mpk {

struct Box {
  int32_t tensor;
  int32_t lo[4];
  int32_t hi[4];
};

struct TaskDef {
  int32_t type = 0, layer = -1;
  int32_t c[3] = {0, 0, 0};
  std::vector<Box> ins, outs;
};

// Resolved build parameters.
struct Params {
  int32_t W = 1, S_sched = 16, q = 1;
  int32_t T_qkv = 1, T_o = 1, T_gu = 1, T_down = 1, T_lm = 1, S_attn = 1;
  bool jit_attn = true;   // attention tasks JIT (else AOT)
  bool jit_all = false;   // every non-empty task JIT (scheduling ablation)
  bool preload = true;    // weight pre-load of the next AOT projection tile
  bool lookahead = false; // paged lookahead: the next two AOT tasks staged into two LDS pages
  bool coarse = false;    // operator-level graph: attention waits for all q/k/v tiles
  int32_t fusion = 0;     // 0: Def 4.1 then Def 4.2; 1: none (one event per overlap edge)
  int32_t split_pages = 2;  // minimum KV pages per attention split (run time)
  int32_t T_router = 1, T_egu = 1, T_edown = 1;   // mixture of experts
  int32_t K_qkv = 1, K_o = 1, K_down = 1;   // k-splits (batch > 1)
};

// The linearised graph (task index = linear position), as exported.
struct Graph {
  int32_t NT = 0, NE = 0, root = 0, end = 0, n_fused = 0, n_empty = 0, n_rewrites = 0;
  std::vector<uint8_t> task_type, task_mode;
  std::vector<int16_t> task_layer;
  std::vector<uint16_t> task_coords;  // [NT][3]
  std::vector<int32_t> task_orig, task_dep, task_trig;
  std::vector<int16_t> task_worker;
  std::vector<uint32_t> event_counts;
  std::vector<int32_t> event_first, event_last;
  std::vector<uint8_t> event_flags;
  std::vector<uint32_t> aot_offsets, aot_tasks;
};

// Tensor ids of the decoder: 5 shared, then 15 per layer (router logits and
// route records in mixture-of-experts layers).
enum { T_E = 0, T_HF = 1, T_LOGITS = 2, T_PMAX = 3, T_NEXT = 4 };
enum { L_R = 0, L_H, L_QKV, L_Q, L_KC, L_VC, L_PART, L_ATTN, L_O, L_S, L_H2, L_A, L_D, L_RLOG, L_ROUTE, L_COUNT };
inline int32_t layer_tensor(int32_t l, int32_t k) { return 5 + L_COUNT * l + k; }

// Expert slots of a mixture-of-experts layer (0 for a dense model), and the
// words of a slot's route record: expert, token count, tokens[B], weights[B].
inline int32_t moe_slots(const mpk_model_cfg& c, int32_t B) {
  return c.n_experts > 0 ? (c.n_experts < B * c.top_k ? c.n_experts : B * c.top_k) : 0;
}
inline int32_t route_words(int32_t B) { return 2 + 2 * B; }

// Balanced tile n of T over N columns on a quantum of q columns.
inline void tile_range(int64_t N, int64_t q, int64_t T, int64_t n, int32_t* lo, int32_t* hi) {
  int64_t U = (N + q - 1) / q;
  int64_t a = q * (n * U / T), b = q * ((n + 1) * U / T);
  *lo = (int32_t)a;
  *hi = (int32_t)(b < N ? b : N);
}

// Validate cfg/batch/page size and resolve defaults; `n_cus` is the compute
// unit count used for the default worker count.  Returns MPK_OK or an error
// with a message in `err`.
int resolve_params(const mpk_model_cfg& cfg, int32_t B, int32_t P, const mpk_build_params* in, int32_t n_cus,
                   Params* out, std::string* err);

// Whether the residual add + RMSNorm run inside the projection tiles that
// consume them (batch 1: every tile stages its whole input vector on chip),
// instead of as ATTN_NORM / MLP_NORM / FINAL_NORM tasks (and EMBED).
inline bool fused_norm(int32_t B) { return B == 1; }

// Program-order tasks of one decode step with their input/output boxes.
// Per layer: [ATTN_NORM] QKV tiles, ATTN(b, g, s) (JIT; also q/k RMSNorm +
// RoPE, the KV append in split S-1, and the split combine by the last split
// of (b, g) to finish), OPROJ tiles, [MLP_NORM] GATEUP tiles, DOWN tiles;
// then [FINAL_NORM] LMHEAD tiles, ARGMAX.  At batch 1 (fused_norm) the first
// QKV tile also stores the residual r, the first GATEUP tile the residual s.
void decompose(const mpk_model_cfg& cfg, int32_t B, const Params& p, std::vector<TaskDef>* tasks);

// Canonicalisation pipeline on arbitrary tasks; MPK_ERR_GRAPH on a cycle.
// jit: 0 every non-empty task AOT, 1 attention JIT, 2 every non-empty task JIT;
// fusion: 0 Def 4.1 then Def 4.2, 1 none (one event per overlap edge, so
// normalisation rewrites fan-ins as well as fan-outs)
int canonicalize(const std::vector<TaskDef>& tasks, int32_t W, int jit, int fusion, Graph* g, std::string* err);

}  // namespace mpk
