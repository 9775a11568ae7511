// Host-only exercise of the graph builder and the host paths of the C ABI,
// compiled with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py (g++, host code only):
//  * decoder graphs of several shapes, batches and build parameters, built
//    with host_only = 1, their header read, exported and destroyed;
//  * the rewrite pipeline (mpk_build_generic_ex) on pseudo-random task/region
//    programs, with fusion on and off and every scheduling policy;
//  * argument errors that must be refused.
// For every graph it prints one line "graph <name> NT NE n_empty n_aot" that
// the test compares with the library build.  The launchers the device sources
// provide are stubs that abort: no host-only path may reach them.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "mpk.h"
#include "rt.h"

namespace mpk {
[[noreturn]] static void device_path(const char* f) {
  std::fprintf(stderr, "host-only run reached device path %s\n", f);
  std::abort();
}
hipError_t launch_megakernel(const KArgs&, uint32_t, uint64_t, int, hipStream_t, bool) { device_path("launch_megakernel"); }
hipError_t launch_baseline_op(const KArgs&, const int32_t*, int, hipStream_t) { device_path("launch_baseline_op"); }
hipError_t launch_time_task(const KArgs&, int, bool, unsigned long long*, hipStream_t) { device_path("launch_time_task"); }
int64_t packed_bytes(int64_t, int64_t) { device_path("packed_bytes"); }
hipError_t launch_pack(const void*, const void*, int64_t, int64_t, void*, hipStream_t) { device_path("launch_pack"); }
size_t scratch_capacity() { device_path("scratch_capacity"); }
hipError_t scratch_address(int, void**) { device_path("scratch_address"); }
hipError_t scratch_zero(void*, size_t, hipStream_t) { device_path("scratch_zero"); }
}  // namespace mpk

namespace {

int failures = 0;
#define EXPECT(c)                                                                 \
  do {                                                                            \
    if (!(c)) {                                                                   \
      std::fprintf(stderr, "FAILED %s at line %d: %s\n", #c, __LINE__, mpk_last_error()); \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

mpk_model_cfg shape(int L, int H, int hq, int hkv, int d, int F, int V, int seq, int qk, int tied, int E = 0, int k = 0,
                    int Fe = 0) {
  mpk_model_cfg c;
  std::memset(&c, 0, sizeof(c));
  c.n_layers = L; c.hidden = H; c.n_q_heads = hq; c.n_kv_heads = hkv; c.head_dim = d; c.ffn = F; c.vocab = V;
  c.max_seq_len = seq; c.qk_norm = qk; c.tied_embedding = tied; c.rms_eps = 1e-6f; c.rope_theta = 1e4f;
  c.n_experts = E; c.top_k = k; c.moe_ffn = Fe; c.norm_topk = E > 0;
  return c;
}

mpk_build_params host_params() {
  mpk_build_params p;
  std::memset(&p, 0, sizeof(p));
  p.host_only = 1;
  return p;
}

// Build, read back and export one graph; check the view's internal
// consistency (every dependent and triggering event in range, ranges inside
// the task count, AOT offsets increasing); print its sizes.
void one_graph(const char* name, const mpk_model_cfg& c, int B, int P, mpk_build_params p) {
  mpk_tgraph* g = nullptr;
  const int rc = mpk_build_tgraph_ex(&c, B, P, &p, &g);
  EXPECT(rc == MPK_OK && g != nullptr);
  if (rc != MPK_OK) return;
  mpk_tgraph_header h;
  EXPECT(mpk_tgraph_info(g, &h) == MPK_OK);
  mpk_tgraph_host_view v;
  std::memset(&v, 0, sizeof(v));
  EXPECT(mpk_tgraph_export(g, &v) == MPK_OK);
  const int NT = v.header.n_tasks, NE = v.header.n_events, W = v.header.params.n_workers;
  for (int t = 0; t < NT; ++t) {
    EXPECT(v.task_dep[t] >= 0 && v.task_dep[t] < NE);
    EXPECT(v.task_trig[t] >= 0 && v.task_trig[t] < NE);
  }
  for (int e = 0; e < NE; ++e) EXPECT(v.event_first[e] >= 0 && v.event_last[e] < NT && v.event_first[e] <= v.event_last[e] + 1);
  for (int w = 0; w < W; ++w) EXPECT(v.aot_offsets[w] <= v.aot_offsets[w + 1]);
  EXPECT((int)v.aot_offsets[W] == v.header.n_aot);
  std::printf("graph %s %d %d %d %d\n", name, NT, NE, v.header.n_empty, v.header.n_aot);
  mpk_free_host_view(&v);
  mpk_free_host_view(&v);   // a freed (zeroed) view is accepted again
  mpk_destroy_tgraph(g);
}

// xorshift64: a small deterministic generator for the random programs
struct Rng {
  uint64_t s;
  uint32_t next() {
    s ^= s << 13; s ^= s >> 7; s ^= s << 17;
    return (uint32_t)(s >> 11);
  }
  int in(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }
};

// A random program over a few 2-D tensors: each task writes a box of one
// tensor and reads boxes of others, tilings deliberately misaligned.
void random_programs(int n_programs) {
  Rng r{0x9e3779b97f4a7c15ull};
  for (int it = 0; it < n_programs; ++it) {
    const int n = r.in(1, 40), n_tensors = r.in(1, 5);
    std::vector<mpk_task_spec> tasks(n);
    std::vector<mpk_region> regs;
    for (int t = 0; t < n; ++t) {
      tasks[t] = mpk_task_spec{r.in(0, 12) == 0 ? (int)MPK_TASK_ATTN : (int)MPK_TASK_QKV, r.in(0, 3), t, 0, 0};
      const int n_io = r.in(1, 4);
      for (int k = 0; k < n_io; ++k) {
        mpk_region b;
        std::memset(&b, 0, sizeof(b));
        b.task = t;
        b.is_out = k == 0 ? 1 : (r.in(0, 3) == 0);
        b.tensor = r.in(0, n_tensors - 1);
        for (int dd = 0; dd < 4; ++dd) { b.lo[dd] = 0; b.hi[dd] = 1; }
        for (int dd = 0; dd < 2; ++dd) {
          const int a = r.in(0, 63), len = r.in(1, 32);
          b.lo[dd] = a;
          b.hi[dd] = a + len;
        }
        regs.push_back(b);
      }
    }
    for (int fusion = 0; fusion <= 1; ++fusion)
      for (int jit : {0, 2, 3}) {
        mpk_build_params p = host_params();
        p.n_workers = r.in(1, 9);
        p.fusion_order = fusion;
        p.attn_jit = jit;
        mpk_tgraph_host_view v;
        std::memset(&v, 0, sizeof(v));
        const int rc = mpk_build_generic_ex(tasks.data(), n, regs.data(), (int)regs.size(), &p, &v);
        EXPECT(rc == MPK_OK);
        if (rc == MPK_OK) {
          EXPECT(v.header.n_tasks >= n);
          mpk_free_host_view(&v);
        }
      }
  }
  std::printf("random programs %d\n", n_programs);
}

void argument_errors() {
  const mpk_model_cfg ok = shape(2, 256, 4, 2, 64, 704, 1024, 256, 0, 0);
  mpk_build_params p = host_params();
  mpk_tgraph* g = reinterpret_cast<mpk_tgraph*>(0x1);
  EXPECT(mpk_build_tgraph_ex(nullptr, 1, 16, &p, &g) == MPK_ERR_INVALID_ARG && g == nullptr);
  EXPECT(mpk_build_tgraph_ex(&ok, 1, 16, &p, nullptr) == MPK_ERR_INVALID_ARG);
  struct Bad { mpk_model_cfg c; int B, P; int rc; } bad[] = {
      {shape(2, 256, 4, 2, 96, 704, 1024, 256, 0, 0), 1, 16, MPK_ERR_UNSUPPORTED},    // head_dim
      {shape(2, 256, 4, 3, 64, 704, 1024, 256, 0, 0), 1, 16, MPK_ERR_INVALID_ARG},    // heads
      {shape(2, 260, 4, 2, 64, 704, 1024, 256, 0, 0), 1, 16, MPK_ERR_UNSUPPORTED},    // hidden % 8
      {shape(2, 264, 4, 2, 64, 712, 1024, 256, 0, 0), 3, 16, MPK_ERR_UNSUPPORTED},    // % 32 at batch > 1
      {shape(2, 256, 4, 2, 64, 704, 1024, 256, 0, 0), 17, 16, MPK_ERR_UNSUPPORTED},   // batch
      {shape(2, 256, 4, 2, 64, 704, 1024, 256, 0, 0), 1, 24, MPK_ERR_UNSUPPORTED},    // page size
      {shape(0, 256, 4, 2, 64, 704, 1024, 256, 0, 0), 1, 16, MPK_ERR_INVALID_ARG},    // layers
      {shape(2, 256, 4, 2, 64, 704, 1024, 256, 0, 0, 300, 2, 64), 1, 16, MPK_ERR_UNSUPPORTED},  // experts
  };
  for (auto& b : bad) {
    mpk_tgraph* h = nullptr;
    const int rc = mpk_build_tgraph_ex(&b.c, b.B, b.P, &p, &h);
    EXPECT(rc == b.rc && h == nullptr);
    EXPECT(std::strlen(mpk_last_error()) > 0);
  }
  mpk_build_params q = host_params();
  q.k_o = 2;   // k-splits need batch > 1
  mpk_tgraph* h = nullptr;
  EXPECT(mpk_build_tgraph_ex(&ok, 1, 16, &q, &h) == MPK_ERR_UNSUPPORTED && h == nullptr);
  q = host_params();
  q.fusion_order = 2;
  EXPECT(mpk_build_tgraph_ex(&ok, 1, 16, &q, &h) == MPK_ERR_UNSUPPORTED && h == nullptr);
  EXPECT(mpk_tgraph_info(nullptr, nullptr) == MPK_ERR_INVALID_ARG);
  EXPECT(mpk_tgraph_export(nullptr, nullptr) == MPK_ERR_INVALID_ARG);
  mpk_destroy_tgraph(nullptr);
  mpk_free_host_view(nullptr);
  std::printf("argument errors\n");
}

}  // namespace

int main() {
  const mpk_model_cfg tiny = shape(2, 256, 4, 2, 64, 704, 1024, 256, 0, 0);
  const mpk_model_cfg tiny_moe = shape(2, 256, 4, 2, 64, 704, 1024, 256, 0, 0, 8, 2, 96);
  const mpk_model_cfg q06 = shape(28, 1024, 16, 8, 128, 3072, 151936, 8192, 1, 1);
  const mpk_model_cfg q8 = shape(36, 4096, 32, 8, 128, 12288, 151936, 8192, 1, 0);
  const mpk_model_cfg q30 = shape(48, 2048, 32, 4, 128, 6144, 151936, 8192, 1, 0, 128, 8, 768);
  struct Case { const char* name; mpk_model_cfg c; int B, P; mpk_build_params p; } cases[] = {
      {"tiny_b1", tiny, 1, 16, host_params()},
      {"tiny_b3", tiny, 3, 16, host_params()},
      {"tiny_b16", tiny, 16, 16, host_params()},
      {"tiny_moe_b1", tiny_moe, 1, 16, host_params()},
      {"tiny_moe_b4", tiny_moe, 4, 16, host_params()},
      {"qwen3_0p6b_b1", q06, 1, 64, host_params()},
      {"qwen3_8b_b1", q8, 1, 64, host_params()},
      {"qwen3_8b_b16", q8, 16, 64, host_params()},
      {"qwen3_30b_a3b_b16", q30, 16, 64, host_params()},
  };
  for (auto& k : cases) one_graph(k.name, k.c, k.B, k.P, k.p);
  // the same shapes under the other build options
  for (int jit : {1, 3}) {
    mpk_build_params p = host_params();
    p.attn_jit = jit;
    one_graph(jit == 1 ? "tiny_b3_hybrid" : "tiny_b3_pure_jit", tiny, 3, 16, p);
    one_graph(jit == 1 ? "qwen3_8b_b16_hybrid" : "qwen3_8b_b16_pure_jit", q8, 16, 64, p);
  }
  {
    mpk_build_params p = host_params();
    p.fusion_order = 1;
    p.n_workers = 8;
    p.s_attn = 4;
    one_graph("tiny_b3_no_fusion", tiny, 3, 16, p);
    p.attn_jit = 3;
    p.n_sched_waves = 4;
    one_graph("tiny_b3_no_fusion_pure_jit", tiny, 3, 16, p);
  }
  {
    mpk_build_params p = host_params();
    p.coarse_events = 1;
    one_graph("qwen3_8b_b1_coarse", q8, 1, 64, p);
    p.coarse_events = 0;
    p.k_qkv = 2; p.k_o = 2; p.k_down = 3; p.t_qkv = 16; p.t_o = 12; p.t_down = 12;
    p.n_workers = 16;
    one_graph("tiny_b3_ksplit", tiny, 3, 16, p);
  }
  random_programs(200);
  argument_errors();
  std::printf("%s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
