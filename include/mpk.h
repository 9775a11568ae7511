/*
 * mpk.h -- C ABI of the MI355X (gfx950) decode-step mega-kernel library.
 *
 * One transformer decode step of a Qwen3-shaped decoder runs as a single
 * persistent kernel that executes a task/event graph (tGraph) built on the
 * host ahead of time.  The method is the one summarised on the page "MPK: A
 * Compiler and Runtime for Mega-Kernelizing Tensor Programs -- L2":
 *   - section 2 (Q2): operators become per-tile tasks joined by events; an
 *     event exists iff a producer's output region overlaps a consumer's input
 *     region; the graph is fused, normalised and linearised into a compact
 *     device structure, and an in-kernel runtime of workers (FIFO task queues)
 *     and schedulers (event queues) runs it with a hybrid JIT/AOT launch policy;
 *   - section 3, "Target operation, shapes & precision contract": MatMul tasks
 *     with bf16 inputs/outputs and fp32 accumulation; paged-attention decode
 *     tasks of data-dependent duration (the JIT ones);
 *   - section 4, Def 4.1 / Def 4.2, "6 minimum checks", Table 1 and the
 *     design-space table: fusion, normalisation (<= 1 dependent and <= 1
 *     triggering event per task), BFS linearisation ([first, last] fan-out),
 *     scheduler budget of 4 compute units x 4 wavefronts.
 *
 * Conventions for every entry point:
 *   - returns MPK_OK (0) or a negative MPK_ERR_* code and never throws; the
 *     message of the last failure on the calling thread is mpk_last_error();
 *   - "device pointer" means memory of the current HIP device, owned by the
 *     caller unless stated otherwise; "host pointer" means ordinary memory;
 *   - streams are passed as `void*` holding a hipStream_t (NULL = default
 *     stream), so this header needs no HIP include;
 *   - all bf16 data is IEEE bfloat16 (upper half of binary32), matrices are
 *     row-major [out_features][in_features] (the nn.Linear layout).
 */
#ifndef MPK_H
#define MPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MPK_OK = 0,
  MPK_ERR_INVALID_ARG = -1, /* null pointer, bad size, config/graph mismatch */
  MPK_ERR_UNSUPPORTED = -2, /* shape or device outside what the kernels handle */
  MPK_ERR_HIP = -3,         /* a HIP runtime call failed */
  MPK_ERR_GRAPH = -4,       /* the task graph has a cycle (cannot happen for the decoder) */
  MPK_ERR_TIMEOUT = -5,     /* an in-kernel wait exceeded the watchdog; graph is poisoned */
  MPK_ERR_NOMEM = -6        /* host or device allocation failed */
};

/* Task types of the decoder tGraph (the order is the program order of one layer).
 * At batch 1 the residual add + RMSNorm of the layer run inside the QKV,
 * GATEUP and LMHEAD tiles (and the embedding gather inside the layer-0 QKV
 * tiles), so EMBED and the *_NORM tasks appear at batch > 1 only.  Ids 3 and 5
 * are not emitted for the decoder: q/k RMSNorm + RoPE + the KV append and the
 * split combine run inside the ATTN tasks. */
enum {
  MPK_TASK_EMBED = 0,       /* e[b,:] = E[token_ids[b], :] (fp32)                        */
  MPK_TASK_ATTN_NORM = 1,   /* r = residual in; h = RMSNorm(r) (fp32)                    */
  MPK_TASK_QKV = 2,         /* tile of the fused q/k/v projection (group-major columns)  */
  MPK_TASK_QKNORM_ROPE = 3, /* (reserved)                                                */
  MPK_TASK_ATTN = 4,        /* slot j of a kv group's s_attn slots: serves one split of   */
                            /* one request, chosen at run time so that the group's slots */
                            /* get equal page counts; q/k norm, RoPE, paged attention    */
                            /* partial; a request's last split appends the new k/v, the  */
                            /* last one to finish merges the request's partials          */
  MPK_TASK_COMBINE = 5,     /* (reserved)                                                */
  MPK_TASK_OPROJ = 6,       /* tile of the output projection                             */
  MPK_TASK_MLP_NORM = 7,    /* s = r + o; h2 = RMSNorm(s)                                */
  MPK_TASK_GATEUP = 8,      /* tile of gate/up projections with the SwiGLU epilogue      */
  MPK_TASK_DOWN = 9,        /* tile of the down projection                               */
  MPK_TASK_FINAL_NORM = 10, /* hf = RMSNorm(s + d) of the last layer                     */
  MPK_TASK_LMHEAD = 11,     /* tile of the LM head: fp32 logits + per-tile (max, argmax) */
  MPK_TASK_ARGMAX = 12,     /* next_ids[b] = argmax over tile partials (lowest index)    */
  MPK_TASK_EMPTY = 13,      /* no compute; inserted by normalisation                     */
  /* mixture-of-experts layers (n_experts > 0) in place of GATEUP / DOWN:      */
  MPK_TASK_ROUTER = 14,     /* tile of the router: logits [B][E]; at batch 1 also the     */
                            /* residual add + RMSNorm (tile 0 stores s and h2 and zeroes  */
                            /* d, which the down tiles add to; at batch > 1 MLP_NORM does) */
  MPK_TASK_EXPERT_GU = 15,  /* tile of expert slot s (the s-th distinct expert the batch  */
                            /* chose): gate/up of its tokens' rows, SwiGLU; tile 0 writes */
                            /* the slot's route record (expert, tokens, weights)          */
  MPK_TASK_EXPERT_DOWN = 16 /* tile of slot s: down projection, adds weight x output of   */
                            /* each of the slot's tokens into the layer's output          */
};
enum { MPK_MODE_AOT = 0, MPK_MODE_JIT = 1, MPK_MODE_EMPTY = 2 };
enum { MPK_EVENT_HAS_JIT = 1, MPK_EVENT_HAS_EMPTY = 2 };

/* Decoder shape.  n_q_heads must be a multiple of n_kv_heads; head_dim is 64
 * or 128; hidden and ffn are multiples of 8.  RMSNorm is
 * v / sqrt(mean(v^2) + rms_eps) * gamma; RoPE is rotate-half with angles
 * pos * rope_theta^(-2i/head_dim). */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, max_seq_len;
  int32_t qk_norm;        /* 1: per-head RMSNorm of q and k before RoPE */
  int32_t tied_embedding; /* 1: the LM head is the embedding matrix */
  float rms_eps, rope_theta;
  /* mixture of experts (0 experts: a dense SwiGLU FFN of width ffn in every
   * layer).  With n_experts = E > 0 every layer's FFN is E SwiGLU experts of
   * width moe_ffn: router logits h Wr^T, softmax over the experts, the top_k
   * most probable (ties to the lower index) weighted by their probabilities,
   * renormalised over the top_k when norm_topk = 1.  E <= 256, top_k <= 16. */
  int32_t n_experts, top_k, moe_ffn, norm_topk;
} mpk_model_cfg;

/* Build parameters; a zero field takes its default (shown).  They are part of
 * the exported header so that a checker can rebuild the same graph. */
typedef struct {
  int32_t n_workers;     /* W worker workgroups (default: compute units - scheduler WGs) */
  int32_t n_sched_waves; /* scheduler wavefronts, 4 per scheduler WG (default: none when  */
                         /* no task is JIT, so every compute unit is a worker; else the   */
                         /* largest S <= 16 dividing the worker count, 14 on 256 compute  */
                         /* units); each serves at most 64 workers (checked at upload)    */
  int32_t quantum;       /* column quantum of projection tiles (default 1 at B=1, else 16) */
  int32_t t_qkv, t_o, t_gu, t_down, t_lm; /* tiles per projection (default ~W; t_qkv a
                                             multiple of n_kv_heads)                    */
  int32_t s_attn;        /* attention slots per kv group, at least the batch (default:   */
                         /* batch 1: min(W / n_kv_heads, pages); batch > 1: max(B,       */
                         /* min(W / n_kv_heads, B pages)): one attention task per worker; */
                         /* the step deals them to the requests by page count)            */
  int32_t host_only;     /* 1: build on the host only (no device work); export still works */
  int32_t fusion_order;  /* 0 default: successor-set fusion (Def 4.1) then predecessor-set */
                         /* fusion (Def 4.2); 1 none: one event per overlap edge, so      */
                         /* normalisation also rewrites fan-ins (an ablation for small     */
                         /* graphs: the device holds at most 2^20 events)                 */
  int32_t aot_policy;    /* must be 0: round-robin over workers in linear order           */
  int32_t k_qkv, k_o, k_down; /* k-splits of the q/k/v, O and down projections: tile n   */
                              /* is column tile n / k over k range n % k (ranges on a    */
                              /* quantum of 32; at most one range per 32 elements), each */
                              /* range writing its own plane of partial sums; t_qkv must */
                              /* be a multiple of n_kv_heads x k_qkv, t_o of k_o, t_down */
                              /* of k_down (default at batch > 1: 1; the largest of 4, 3, */
                              /* 2 dividing n_kv_heads, so that a range holds whole kv   */
                              /* groups; 3 -- 1 with experts -- each yielding to a given */
                              /* t_o / t_down it does not divide; 1 at batch 1, the only */
                              /* value allowed there)                                    */
  int32_t attn_jit;      /* scheduling policy: 0 default (every task AOT: an attention     */
                         /* task sizes its split from the lengths at run time, so static  */
                         /* placement is balanced), 1 the hybrid policy (attention JIT,  */
                         /* the rest AOT), 2 every task AOT, 3 every non-empty task JIT  */
                         /* but the root event's consumers, which no trigger hands over; */
                         /* the exported header holds the resolved value (1, 2 or 3)      */
  int32_t weight_preload; /* 0 default (on), 1 on, 2 off: batch-1 projection tiles load   */
                          /* their first weight segments before their event fires (the   */
                          /* cross-task pipelining ablation); 3 paged lookahead: the     */
                          /* pre-load area is two pages and a worker stages its next two */
                          /* AOT tasks -- projection weights, or an attention split's    */
                          /* cached keys and values -- into page (AOT index mod 2) (MPK  */
                          /* summary page, section 5 techniques inventory: cross-task    */
                          /* pipelining, paged shared memory); the header holds 1, 2, 3  */
  int32_t coarse_events;  /* 0 default (fine-grained events), 1 the operator-level graph: */
                          /* an attention split waits for every q/k/v tile, not only its */
                          /* own kv group's (every other operator already waits for the  */
                          /* whole previous one) -- the pages' coarse-graph ablation     */
  int32_t t_router, t_egu, t_edown; /* mixture of experts: router tiles (default min(E,   */
                                    /* W / 8) on the column quantum), gate/up and down    */
                                    /* tiles per expert slot (default about W / slots, more */
                                    /* while a tile's accumulators exceed the LDS budget); */
                                    /* a layer has min(E, B x top_k) expert slots          */
  int32_t attn_split_pages; /* at least this many KV pages per attention split when the   */
                            /* step runs (default 1): a request of p pages takes          */
                            /* min(slots, ceil(p / this)) splits at batch 1 (and no more  */
                            /* than the split combine can stage in LDS), and the split    */
                            /* size of a batch never drops below it                       */
} mpk_build_params;

typedef struct mpk_tgraph mpk_tgraph; /* opaque; owned by the library */

/* Weights: device pointers to bf16 arrays, owned by the caller.
 * layer points to a HOST array of n_layers*12 device pointers, per layer in
 * the order in_norm[H], q[hq*d][H], k[hkv*d][H], v[hkv*d][H], q_norm[d],
 * k_norm[d], o[H][hq*d], post_norm[H], gate[F][H], up[F][H], down[H][F],
 * router (q_norm/k_norm may be NULL when qk_norm is 0; router is NULL for a
 * dense model).  With n_experts = E > 0: gate[E][Fe][H], up[E][Fe][H],
 * down[E][H][Fe] (Fe = moe_ffn) and router[E][H]. */
typedef struct {
  const void* embed;      /* [vocab][H] */
  const void* lm_head;    /* [vocab][H]; NULL when tied (layout 0) */
  const void* final_norm; /* [H] */
  const void* const* layer;
  int32_t layout;         /* 0: the matrices as above (row-major [out][in]);
                             1: prepared by mpk_prepare_weights for one graph */
} mpk_weights;

/* Paged KV cache (device, caller-owned).  k_pool/v_pool are bf16
 * [n_layers][n_pages][n_kv_heads][page_size][head_dim]; token p of request b
 * lives at slot p % page_size of page page_table[b*max_pages_per_seq + p/page_size].
 * Entries beyond a request's pages must still be valid page ids (they are
 * never read). */
typedef struct {
  void* k_pool;
  void* v_pool;
  const int32_t* page_table; /* device, int32 [batch][max_pages_per_seq] */
  int32_t n_pages;
  int32_t max_pages_per_seq;
} mpk_kv;

typedef struct {
  int32_t n_tasks, n_events, root, end;
  int32_t n_fused, n_empty, n_rewrites, n_aot;
  int32_t batch, page_size;
  mpk_build_params params; /* with every default resolved */
} mpk_tgraph_header;

/* Host copies of the linearised graph (task index = linear position).  The
 * arrays are allocated by the library and owned by the caller, who releases
 * them with mpk_free_host_view.  task_coords is [n_tasks][3]; task_orig is
 * the program-order id, or -1-k for the k-th empty task; task_worker is -1
 * for JIT and empty tasks. */
typedef struct {
  mpk_tgraph_header header;
  uint8_t* task_type;
  uint8_t* task_mode;
  int16_t* task_layer;
  uint16_t* task_coords;
  int32_t* task_orig;
  int32_t* task_dep;
  int32_t* task_trig;
  int16_t* task_worker;
  uint32_t* event_counts;
  int32_t* event_first;
  int32_t* event_last;
  uint8_t* event_flags;
  uint32_t* aot_offsets; /* [n_workers + 1] */
  uint32_t* aot_tasks;   /* [n_aot] */
} mpk_tgraph_host_view;

/* Generic canonicalisation input (test entry): a task and its boxes. */
typedef struct {
  int32_t type, layer, c0, c1, c2;
} mpk_task_spec;
typedef struct {
  int32_t task, is_out, tensor;
  int32_t lo[4], hi[4]; /* half-open box; unused dims 0..1 */
} mpk_region;

/* In-kernel status of the last decode step on a graph. */
typedef struct {
  int32_t code;   /* MPK_OK or MPK_ERR_TIMEOUT */
  int32_t wg;     /* workgroup that reported it */
  int32_t task;   /* task it was about to run, or -1 */
  int32_t event;  /* event it was waiting on, or -1 */
  uint32_t counter, target;
} mpk_status_word;

/* Build the tGraph of one decode step of `cfg` at batch `batch` (1..16) with
 * KV pages of `page_size` tokens (16, 32 or 64): decomposition into tile
 * tasks, overlap dependencies, Def 4.1 then Def 4.2 event fusion,
 * normalisation, Kahn-BFS linearisation, JIT/AOT classification, round-robin
 * AOT placement (MPK summary page, section 2 Q2 and section 4: Def 4.1,
 * Def 4.2, "6 minimum checks", design-space table; the graph is built once,
 * ahead of time).  cfg: host pointer, read only.  Allocates the device graph,
 * its event counters, queues and activation buffers on the current device
 * (the only allocation of the library besides tracing and mpk_time_tasks).
 * *out receives a library-owned handle, released with mpk_destroy_tgraph;
 * on an error *out is NULL and nothing stays allocated.  Errors:
 * MPK_ERR_INVALID_ARG (null pointer, inconsistent cfg), MPK_ERR_UNSUPPORTED
 * (shape the kernels do not handle, device not gfx950), MPK_ERR_HIP,
 * MPK_ERR_NOMEM. */
int mpk_build_tgraph(const mpk_model_cfg* cfg, int32_t batch, int32_t page_size, mpk_tgraph** out);

/* Same, with explicit build parameters (host pointer, NULL = every default;
 * see mpk_build_params).  host_only = 1 builds the graph without touching
 * the device (for mpk_tgraph_export; mpk_decode_step then fails). */
int mpk_build_tgraph_ex(const mpk_model_cfg* cfg, int32_t batch, int32_t page_size,
                        const mpk_build_params* params, mpk_tgraph** out);

/* Resolved header of a built graph: task and event counts, root and end
 * events, fusion and rewrite counts, and every build parameter with its
 * default resolved (MPK summary page, section 4 notation: a task's dependent
 * and triggering events, an event's counts and [first, last]).  out: host
 * pointer, written.  Errors: MPK_ERR_INVALID_ARG on a null pointer. */
int mpk_tgraph_info(const mpk_tgraph* g, mpk_tgraph_header* out);

/* Host copies of every index array of the linearised graph (see
 * mpk_tgraph_host_view): what a checker compares against its own
 * construction of the graph (MPK summary page, section 4, "6 minimum
 * checks": <= 1 dependent and <= 1 triggering event per task, contiguous
 * [first, last] fan-out).  The arrays are malloc'ed by the library and owned
 * by the caller, who frees them with mpk_free_host_view.  Errors:
 * MPK_ERR_INVALID_ARG, MPK_ERR_NOMEM (nothing is left allocated). */
int mpk_tgraph_export(const mpk_tgraph* g, mpk_tgraph_host_view* out);

/* Test entry: run the canonicalisation pipeline (overlap edges, fusion,
 * normalisation, linearisation, classification, placement on n_workers) on
 * arbitrary tasks and boxes (MPK summary page, section 2 Q2: an event iff a
 * producer's output region overlaps a consumer's input region; the author's
 * comments on the blog post, item 2: the same rule).  Host only; tasks of
 * type MPK_TASK_ATTN are JIT.  tasks[n_tasks], regions[n_regions]: host
 * arrays, read only; a region names its task by index, is_out 1 for an
 * output box.  The view is filled as by mpk_tgraph_export.  Same as
 * mpk_build_generic_ex with n_workers set and every other field 0.
 * Errors: MPK_ERR_INVALID_ARG (bad task type, region of a missing task),
 * MPK_ERR_GRAPH (a cycle), MPK_ERR_NOMEM. */
int mpk_build_generic(const mpk_task_spec* tasks, int32_t n_tasks, const mpk_region* regions,
                      int32_t n_regions, int32_t n_workers, mpk_tgraph_host_view* out);

/* The same with build parameters (host pointer, required): n_workers,
 * fusion_order and attn_jit are read (attn_jit 0 and 1: attention tasks JIT,
 * 2: every task AOT, 3: every non-empty task JIT but the root's consumers);
 * every other field is ignored.  MPK summary page, section 4: Def 4.1 /
 * Def 4.2 and the "6 minimum checks" (normalisation, fan-out and fan-in
 * rewrites; contiguous [first, last] fan-out). */
int mpk_build_generic_ex(const mpk_task_spec* tasks, int32_t n_tasks, const mpk_region* regions,
                         int32_t n_regions, const mpk_build_params* params, mpk_tgraph_host_view* out);

/* Free the arrays of a host view filled by mpk_tgraph_export or
 * mpk_build_generic(_ex) and zero the view; NULL and an already freed
 * (zeroed) view are accepted. */
void mpk_free_host_view(mpk_tgraph_host_view* v);

/* Size in bytes of the device buffer mpk_prepare_weights fills for graph g
 * (*bytes, host pointer).  Errors: MPK_ERR_INVALID_ARG on a null pointer. */
int mpk_prepared_weights_bytes(const mpk_tgraph* g, size_t* bytes);

/* One-time repack of the projection weights of a batch > 1 graph into the
 * order its matrix-core tiles load them (layout 1).  Each q, k, v, o, down and
 * LM-head matrix [N][K] becomes blocks of 16 rows x 32 k, stored as
 * [ceil(N/16)][K/32][64][8] bf16 (lane l of a block: row l % 16 at k
 * 8 (l / 16) .. +7, the A operand of v_mfma_f32_16x16x32_bf16), so that a
 * wavefront's loads of one block are one contiguous 1 KB; gate and up become
 * one matrix of 2F interleaved rows (gate row c at 2c, up row c at 2c + 1),
 * the order of a gate/up tile's rows.  The values are copied bit for bit.
 * The MatMul task of MPK summary page section 3 ("Target operation, shapes &
 * precision contract") is an output tile of a GEMM; at batch > 1 this is the
 * tile's operand layout.  Inputs: `in` (layout 0) as for mpk_decode_step;
 * `dst`, a caller-owned device buffer of dst_bytes >= the size
 * mpk_prepared_weights_bytes reports, 256-byte aligned; `packed_layers`, a
 * caller-owned host array of n_layers x 11 pointers.  Outputs: `packed`
 * (host) with layout 1, the prepared matrices in dst, the LM head a prepared
 * copy (also when tied), embedding and norm gains the caller's own, layer =
 * packed_layers (the gate and up entries both point at the interleaved
 * matrix).  The copy runs asynchronously on `stream`; `in` must stay valid
 * until it completes; then `packed` serves every step of this graph and
 * `dst` must outlive them.  Errors: MPK_ERR_INVALID_ARG (null pointer, buffer
 * too small or misaligned, `in` not layout 0), MPK_ERR_UNSUPPORTED (batch 1,
 * whose tiles stream whole rows, or a column quantum not a multiple of 16),
 * MPK_ERR_HIP. */
int mpk_prepare_weights(const mpk_tgraph* g, const mpk_weights* in, void* dst, size_t dst_bytes,
                        const void** packed_layers, mpk_weights* packed, void* stream);

/* One decode step as ONE persistent-kernel launch on `stream` (asynchronous):
 * the whole forward of one new token per request, run by the in-kernel
 * runtime of workers and schedulers over the graph's events (MPK summary
 * page, section 3 Fig 1: one launch per step instead of one per operator;
 * section 2 Q2: workers pop FIFO task queues, schedulers consume event
 * queues; section 4 Table 1 and design-space table: the hybrid JIT/AOT
 * policy).  w: host pointer to device weight pointers (caller-owned,
 * bf16, read only); token_ids[B], seq_lens[B] (tokens already cached; the
 * new token is at position seq_lens[b]) are device int32; logits is device
 * fp32 [B][vocab]; next_ids is device int32 [B] (argmax, lowest index on
 * ties).  The step writes the new token's k and v into the cache slot of
 * position seq_lens[b] (bf16) and does not change seq_lens.  Calls on one
 * graph must be ordered on one stream.  When the weight pointers differ from
 * the last call's, the call first synchronises and uploads the resolved
 * pointers (the steady state makes no host-device copy).  Errors returned
 * synchronously: MPK_ERR_INVALID_ARG (null or misaligned pointer, host-only
 * graph), MPK_ERR_HIP (launch failure).  In-kernel failures (watchdog
 * timeout, a token id outside the vocabulary, a bad page id or cached
 * length) are reported by mpk_get_status and poison the graph: later steps
 * exit at once and leave their outputs unwritten. */
int mpk_decode_step(mpk_tgraph* g, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
                    const int32_t* seq_lens, float* logits, int32_t* next_ids, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as mpk_decode_step -- same kernel, same arguments, same outputs --
 * with its per-call mutable device state (event counters, scheduler and JIT
 * rings, split arrivals, fp32 activations) in a static device area of the
 * library (64 MiB, one per GPU the library runs on, held until the process
 * ends) instead of the graph's own buffers.  The call allocates nothing,
 * synchronises nothing and copies nothing from the host: it clears the
 * runtime part of the area with a fill kernel on `stream` and launches the
 * step there (epoch 1).  The graph's device must be current, and the
 * weights must be the ones the graph was last bound to by mpk_decode_step
 * (which uploads their resolved pointers).  Every call on one GPU shares
 * that GPU's area, which keeps the last call's contents: calls that overlap
 * on one GPU (other streams, other graphs) race and must be ordered by the
 * caller.  mpk_read_tensor reads the graph's own buffers, not this area.  The
 * in-kernel status goes to the graph's status word (mpk_get_status).
 * Errors: MPK_ERR_UNSUPPORTED when the graph's state exceeds the area (the
 * message gives both sizes), MPK_ERR_INVALID_ARG (null pointer, host-only
 * graph, weights not bound, device not current), MPK_ERR_HIP. */
int mpk_decode_step_noalloc(mpk_tgraph* g, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
                            const int32_t* seq_lens, float* logits, int32_t* next_ids, void* stream);

/* The kernel-per-operator baseline the mega-kernel is measured against
 * (MPK summary page, section 2 Q1: kernel-per-operator execution with a
 * barrier at every operator boundary; section 2 Q3: the comparison): the
 * same task bodies, one kernel per operator with one workgroup per task,
 * launched in stream order with no events.  Arguments, outputs and errors
 * are those of mpk_decode_step.  use_hipgraph = 1 captures the launches once
 * into a hipGraph (re-captured when a pointer changes; the first call
 * creates a capture stream) and replays it. */
int mpk_decode_step_baseline(mpk_tgraph* g, const mpk_weights* w, const int32_t* token_ids, const mpk_kv* kv,
                             const int32_t* seq_lens, float* logits, int32_t* next_ids, void* stream,
                             int32_t use_hipgraph);

/* Copy intermediate tensor `tensor` of the last step to host memory `dst`
 * (`bytes` must equal its size).  All are fp32 [B][...]: ids 3 pmax[B][t_lm]
 * (fp32 value, int32 index pairs); per layer l, 5 + 15*l + k with k = 0 r
 * (residual into the layer), 2 qkv (raw projection, group-major: per kv group
 * its query heads, key head, value head; k_qkv planes [k_qkv][B][...] whose
 * sum is the projection), 6 attention partials
 * [kv][s_attn][G][2 + head_dim] (per kv group and slot: max, sum, output;
 * a request's splits occupy consecutive slots), 7 attn, 8 o (k_o planes), 9 s
 * (residual after attention), 11 a, 12 d (k_down planes); at batch > 1 also 0 e[B][H],
 * 1 hf[B][H], and per layer k = 1 h, 10 h2 (the normalised inputs).  Mixture-of-
 * experts layers: 10 h2 (also at batch 1), 11 a [slots][B][moe_ffn] (a slot's
 * rows hold its tokens' SwiGLU outputs), 12 d [B][H] (the weighted expert
 * sum), 13 router logits [B][E], 14 route records [slots][2 + 2B] (int32
 * expert, token count, tokens[B], fp32 weights[B]).
 * The ids are the tensors of the graph's regions (MPK summary page, section
 * 2 Q2: events are inferred from the regions tasks read and write), so a
 * test can check every task's output layer by layer.  Synchronises the
 * device.  Errors: MPK_ERR_INVALID_ARG (no such library-owned tensor, wrong
 * size, host-only graph), MPK_ERR_HIP. */
int mpk_read_tensor(const mpk_tgraph* g, int32_t tensor, void* dst, size_t bytes);

/* Per-task trace of the persistent kernel: times are the GPU's constant-rate
 * wall clock (ticks; ticks_per_us is reported by mpk_read_trace). */
typedef struct {
  int32_t task;     /* linear task index */
  int32_t worker;   /* worker that ran it */
  uint64_t t_wait;  /* the worker started looking for this task */
  uint64_t t_start; /* its dependent event had fired / it was taken from the JIT ring */
  uint64_t t_end;   /* its body finished (before its triggering event is advanced) */
  uint64_t t_done;  /* its triggering event had been advanced (release + add returned) */
  uint64_t t_mark[2]; /* two points inside the body, 0 where the body has none:
                         projection tiles: x staged (and normalised) / weight stream done;
                         attention: q normalised and rotated / key loop done;
                         norms: inputs summed / reduction done */
} mpk_trace_record;

/* Turn tracing of mpk_decode_step on (1) or off (0): each worker records when
 * it waited for, started and finished each task, which is what the pages'
 * per-phase analysis of the persistent kernel needs (MPK summary page,
 * section 4, "% peak / lower-bound derivation": the gap to the bandwidth
 * bound is scheduling and synchronisation).  Synchronises; allocates (frees)
 * a library-owned device buffer of one record per task; each step
 * overwrites it.  Errors: MPK_ERR_INVALID_ARG (host-only graph), MPK_ERR_HIP. */
int mpk_set_trace(mpk_tgraph* g, int32_t enable);

/* Copy the records of the last traced step to host memory `out` (room for
 * `capacity` records), grouped by worker in execution order.  *count
 * receives the number written; *ticks_per_us the clock rate (may be NULL).
 * Synchronises.  Errors: MPK_ERR_INVALID_ARG (tracing off, capacity too
 * small: the first `capacity` records are still written), MPK_ERR_HIP. */
int mpk_read_trace(mpk_tgraph* g, mpk_trace_record* out, int32_t capacity, int32_t* count, double* ticks_per_us);

/* Body micro-benchmark and serial execution: runs the listed tasks (linear
 * indices, host array of n) one after another in a single workgroup, each
 * `reps` times, on the arguments and buffers of the last mpk_decode_step
 * call (no events are waited on or advanced), and writes each task's mean
 * duration in clock ticks to ticks[n] (host).  cold = 1 invalidates the
 * device-scope caches of the workgroup's die (an agent-scope acquire) right
 * before each run, as a task started by the persistent kernel sees them.
 * The per-task cost the pages analyse (MPK summary page, section 4,
 * design-space table: task granularity).  Allocates and frees a small
 * device buffer; synchronises.  Errors: MPK_ERR_INVALID_ARG (no step run
 * yet, index out of range), MPK_ERR_HIP. */
int mpk_time_tasks(mpk_tgraph* g, const int32_t* tasks, int32_t n, int32_t reps, int32_t cold, uint64_t* ticks,
                   double* ticks_per_us);

/* Serial execution, the check that the graph's regions are complete: with
 * poison = 1 every library-owned activation is first filled with all-ones
 * bytes (NaN in fp32), then the listed tasks (linear indices, host array of
 * n) run once each, one after another, in a single workgroup on the
 * arguments of the last mpk_decode_step call, with no events.  Run in a
 * topological order of the graph that prefers the ready task latest in
 * program order, a task executes before every task it does not declare as
 * a producer, so a region missing from a task's declared inputs leaves it
 * reading NaN (MPK summary page, section 2 Q2 and section 4 check 1: an
 * event iff a producer's output region overlaps a consumer's input region,
 * and no producer-consumer wait may be lost).  Empty tasks in the list do
 * nothing.  Writes the last step's outputs and KV slots.  Synchronises.
 * Errors: MPK_ERR_INVALID_ARG (no step run yet, index out of range),
 * MPK_ERR_HIP. */
int mpk_run_tasks(mpk_tgraph* g, const int32_t* tasks, int32_t n, int32_t poison);

/* Recovery of a poisoned graph (the failure detection around the pages'
 * runtime of event counters and task queues, MPK summary page, section 2 Q2:
 * the watchdog and status word are this library's).  Waits for the graph's
 * last step, then clears its runtime state -- every event counter and
 * sub-counter, the scheduler and JIT rings with their persistent heads and
 * tails, the split arrivals and the status word -- and restarts the step
 * count, so that the next mpk_decode_step runs as the graph's first.
 * Activations, weights and the KV cache are left as they are (a step that
 * was cut short may have written the new token's key/value slot; the next
 * step writes it again).  Also valid on a healthy graph.  The graph's
 * device must be current.  Synchronises.  Errors: MPK_ERR_INVALID_ARG (null
 * or host-only graph, another device current), MPK_ERR_HIP. */
int mpk_reset_tgraph(mpk_tgraph* g);

/* Watchdog for in-kernel waits in nanoseconds (default 2 s; 0 restores it):
 * every wait of a worker or scheduler gives up after it, reports
 * MPK_ERR_TIMEOUT and poisons the graph, so the persistent grid always
 * drains (the runtime's forward-progress guard; the pages' runtime has no
 * such limit).  Takes effect at the next step.  Errors: MPK_ERR_INVALID_ARG. */
int mpk_set_watchdog(mpk_tgraph* g, uint64_t timeout_ns);

/* Synchronises the stream of the last step and reports its in-kernel status
 * (out: host pointer): MPK_OK, MPK_ERR_TIMEOUT (with the workgroup, task,
 * event, counter and target of the wait that gave up) or
 * MPK_ERR_INVALID_ARG (a token id outside the vocabulary or a bad page id or
 * cached length: counter holds the value, target the bound).  A non-zero
 * code stays: the graph is poisoned until it is destroyed.  Errors of the
 * call itself: MPK_ERR_INVALID_ARG, MPK_ERR_HIP. */
int mpk_get_status(mpk_tgraph* g, mpk_status_word* out);

/* Release a graph and everything the library allocated for it (device
 * graph, counters, queues, activations, trace, captured baseline graph).
 * Must not be called while a step on it may still run: synchronise the
 * step's stream first.  NULL is accepted. */
void mpk_destroy_tgraph(mpk_tgraph* g);

/* Thread-local message describing the last non-zero status returned on the
 * calling thread ("" if none); valid until the thread's next failing call. */
const char* mpk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MPK_H */
