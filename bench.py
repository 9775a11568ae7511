"""Decode-step benchmark: one persistent-kernel launch per token on one MI355X.

Default workload: the Qwen3-8B-shaped decoder at batch 1 with 1024 cached
tokens (bf16 random weights, synthetic inputs resident in HBM).  Prints ONE
JSON line: decode ms/token (the value), achieved HBM bandwidth against the
8 TB/s peak, the kernel-per-operator baseline of the same task bodies (plain
launches and hipGraph replay), and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--config qwen3_8b]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode ms/token + achieved HBM TB/s (% peak), Qwen3-8B-shape batch 1"
HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(s, seq_lens, experts=None) -> int:
    """Bytes the step must move: every weight once (projections, norm gains,
    LM head or tied embedding), B embedding rows and the K/V of L_b + 1 tokens
    per request and layer; all bf16.  Mixture of experts: the router and the
    gate/up/down of the experts the batch chose (experts[l] distinct ones in
    layer l) in place of the dense FFN."""
    H, d, hq, hkv, F, V, L = s.hidden, s.head_dim, s.n_q_heads, s.n_kv_heads, s.ffn, s.vocab, s.n_layers
    per_layer = hq * d * H + 2 * hkv * d * H + H * hq * d + 2 * H + (2 * d if s.qk_norm else 0)
    if s.n_experts:
        ffn = sum(s.n_experts * H + e * 3 * s.moe_ffn * H for e in experts)
    else:
        ffn = L * 3 * F * H
    w = L * per_layer + ffn + H + V * H
    kv = sum(int(x) + 1 for x in seq_lens) * L * 2 * hkv * d
    return 2 * (w + len(seq_lens) * H + kv)


SOURCE_FILES = ("include/mpk.h", "task_graph_runtime_amd/build.py")   # (the build flags shape the kernels too)
SOURCE_DIR = "task_graph_runtime_amd/csrc"
TRAFFIC_FILE = "profiles/megakernel_{config}_traffic.txt"


def source_hash(params: dict) -> str:
    """sha256 over every library source (the C ABI header, all of csrc/ and
    the build script with its compiler flags) and the graph's resolved build
    parameters: the HBM-traffic counters of a profile are valid only for the
    build and graph they were taken on."""
    import hashlib
    h = hashlib.sha256()
    files = list(SOURCE_FILES) + sorted(os.path.join(SOURCE_DIR, f) for f in os.listdir(os.path.join(ROOT, SOURCE_DIR))
                                        if f.endswith((".h", ".cpp", ".hip")))
    for src in files:
        h.update(src.encode())
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    h.update(json.dumps(params, sort_keys=True).encode())
    return h.hexdigest()


def measured_traffic(config: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of this
    workload, or None when there is none or it was taken on other sources or
    build parameters."""
    path = os.path.join(ROOT, TRAFFIC_FILE.format(config={"qwen3_8b": "qwen3_8b_b1"}.get(config, config)))
    if not os.path.exists(path):
        return None
    kv = dict(line.strip().split("=", 1) for line in open(path) if "=" in line and " " not in line.strip())
    if kv.get("source_sha256") != src_hash:
        return None
    return int(kv["traffic_bytes"])


def distinct_experts(g, s, mpk, np):
    """Per layer, the experts the batch chose in the last step (busy slots of
    its route records); None for a dense model."""
    if not s.n_experts:
        return None
    M, rw = min(s.n_experts, s.batch * s.top_k), 2 + 2 * s.batch
    return [int((g.read_tensor(5 + mpk._binding.LAYER_TENSORS * l + 14, (M, rw), np.int32)[:, 0] >= 0).sum())
            for l in range(s.n_layers)]


def time_steps(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = [a.elapsed_time(b) for a, b in ev]
    return wall_ms, per


def cpu_baseline(s, inp, steps=3):
    """The oracle, as it stands, timed on the host cores: `steps` full decode
    steps (fp32 numpy with the installed multithreaded BLAS; every bf16 weight
    matrix widened to fp32 when it is used, that work included), median.  The
    weights are copied to host memory once, outside the timed region."""
    import numpy as np
    from oracle import numerics
    from tests._util import oracle_weights, bf16_bits
    cores = len(os.sched_getaffinity(0))
    blas, threads = "unknown", cores
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = int(info[0].get("num_threads", cores))
    except Exception:
        pass
    ram_gib = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES") / 2**30
    kv = inp["kv"]
    w = oracle_weights(inp["weights"])          # host bf16 bit patterns, copied once
    kp, vp = bf16_bits(kv["k_pool"]), bf16_bits(kv["v_pool"])
    args = (inp["token_ids"].cpu().numpy(), kp, vp, kv["page_table"].cpu().numpy(), inp["seq_lens"].cpu().numpy(),
            s.page_size)
    times = []
    for _ in range(steps):
        t0 = time.perf_counter()
        numerics.decode_step(s.cfg(), w, *args, dtype=np.float32)
        times.append(time.perf_counter() - t0)
        print(f"[bench] cpu oracle step {len(times)}: {times[-1]:.2f} s", file=sys.stderr, flush=True)
    del w, kp, vp
    med = statistics.median(times)
    return {"value": round(med * 1e3, 1), "unit": "ms/token", "cores": int(threads), "kind": "oracle",
            "sample": f"median of {steps} full {s.name} decode steps of the fp32 numpy oracle "
                      f"({', '.join(f'{t:.2f}' for t in times)} s; bf16 weights widened per use, included; "
                      f"BLAS {blas}, {threads} threads of {cores} cores in the affinity mask, {ram_gib:.0f} GiB RAM)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_8b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--baseline-steps", type=int, default=20)
    ap.add_argument("--no-baseline", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--prepared", action="store_true",
                    help="batch > 1: run the step on weights repacked by mpk_prepare_weights (matrix-core load order)")
    ap.add_argument("--params", default="{}",
                    help="build parameters (JSON object of mpk_build_params fields, e.g. '{\"s_attn\": 16}') for "
                         "the ablations; the default build is the one measured")
    ap.add_argument("--skew", action="store_true",
                    help="batch > 1: one request at the longest context (max_seq_len - 1), the others at 256 "
                         "(the skewed batch of the scheduling-policy ablation)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the step, run a plain device copy of this many MiB three times (a known-size "
                         "kernel for scaling the HBM byte counters of a profiler run)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode step is built and measured on a single MI355X "
              f"(--gpus {args.gpus} is not supported)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import task_graph_runtime_amd as mpk

    s = synth.SHAPES[args.config]
    print(f"[bench] generating {s.name} inputs", file=sys.stderr, flush=True)
    lens = None
    if args.skew:
        lens = [s.max_seq_len - 1] + [256] * (s.batch - 1)
    inp = synth.make_inputs(s, seed=args.seed, device="cuda", seq_lens=lens)
    kv = inp["kv"]
    ids = inp["token_ids"].cuda()
    lens = inp["seq_lens"].cuda()
    g = mpk.TGraph(s.cfg(), s.batch, s.page_size, json.loads(args.params))
    W = mpk.Weights(inp["weights"])
    if args.prepared:
        W = mpk.PreparedWeights(g, W)
    KV = mpk.KV(kv["k_pool"], kv["v_pool"], kv["page_table"].cuda())
    logits = torch.empty((s.batch, s.vocab), device="cuda", dtype=torch.float32)
    nxt = torch.empty((s.batch,), device="cuda", dtype=torch.int32)

    def mega():
        g.decode_step(W, ids, KV, lens, logits, nxt)

    print(f"[bench] mega-kernel: {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr, flush=True)
    wall_ms, per = time_steps(mega, args.steps, args.warmup, torch)
    st = g.status()
    if st["code"] != 0:
        raise SystemExit(f"mega-kernel reported {st}")
    ms = wall_ms / args.steps
    kern_ms = statistics.mean(per)
    import numpy as np
    experts = distinct_experts(g, s, mpk, np)
    nbytes = algorithmic_bytes(s, inp["seq_lens"].tolist(), experts)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9

    base = {}
    if not args.no_baseline:
        for mode, hg in (("per_op", False), ("hipgraph", True)):
            print(f"[bench] baseline {mode}", file=sys.stderr, flush=True)
            f = (lambda hg=hg: g.decode_step_baseline(W, ids, KV, lens, logits, nxt, use_hipgraph=hg))
            _, pb = time_steps(f, args.baseline_steps, 3, torch)
            base[mode] = round(statistics.median(pb), 4)

    if args.calib_copy_mib > 0:
        n = (args.calib_copy_mib << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu:
        print("[bench] cpu oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(s, inp)

    hdr = g.header()["params"]
    src_hash = source_hash(hdr)
    print(f"[bench] source hash {src_hash}", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": round(ms, 4), "unit": "ms/token", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (random-init bf16 weights, N(0,1) KV)",
        "config": {"workload": f"{s.name} decode step, batch {s.batch}, "
                               + (f"ctx skewed: one at {s.max_seq_len - 1}, {s.batch - 1} at 256" if args.skew else
                                  f"{'ctx ' + str(s.ctx) if s.ctx_range is None else 'ctx U' + str(list(s.ctx_range))}")
                               + f", page {s.page_size}",
                   "global_batch": s.batch, "seq_len": int(max(inp['seq_lens'].tolist())) + 1,
                   "parallelism": "single GPU", "workers": hdr["n_workers"], "sched_waves": hdr["n_sched_waves"],
                   "s_attn": hdr["s_attn"], "weights": "prepared" if args.prepared else "row-major",
                   **({"experts": f"{s.n_experts}, top {s.top_k}, width {s.moe_ffn}",
                       "distinct_experts_per_layer": round(sum(experts) / len(experts), 2)} if experts else {})},
        "tb_per_s": round(achieved / 1e3, 3), "pct_hbm_peak": round(100 * achieved / HBM_PEAK_GBS, 1),
        "kernel_ms": {"mean": round(kern_ms, 4), "median": round(statistics.median(per), 4),
                      "p10": round(sorted(per)[len(per) // 10], 4), "p90": round(sorted(per)[(9 * len(per)) // 10], 4)},
        "bytes_per_step": nbytes,
        "baseline_ms": base or None,
        "speedup_vs_baseline": round(min(base.values()) / kern_ms, 3) if base else None,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config, src_hash)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    # release the graph while the runtime is up (not from a finaliser at interpreter exit)
    torch.cuda.synchronize()
    g.close()


if __name__ == "__main__":
    main()
