"""ctypes binding of ``libmpk.so`` (the C ABI in ``include/mpk.h``).

Argument marshalling only: every step of the decode path runs in the HIP
library.  The raw entry points keep their C names (``mpk_build_tgraph``,
``mpk_decode_step`` ...); ``TGraph`` wraps them for torch tensors, which
serve only as device memory and streams.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmpk.so")

MPK_OK = 0
ERRORS = {-1: "MPK_ERR_INVALID_ARG", -2: "MPK_ERR_UNSUPPORTED", -3: "MPK_ERR_HIP", -4: "MPK_ERR_GRAPH",
          -5: "MPK_ERR_TIMEOUT", -6: "MPK_ERR_NOMEM"}
(TASK_EMBED, TASK_ATTN_NORM, TASK_QKV, TASK_QKNORM_ROPE, TASK_ATTN, TASK_COMBINE, TASK_OPROJ, TASK_MLP_NORM,
 TASK_GATEUP, TASK_DOWN, TASK_FINAL_NORM, TASK_LMHEAD, TASK_ARGMAX, TASK_EMPTY, TASK_ROUTER, TASK_EXPERT_GU,
 TASK_EXPERT_DOWN) = range(17)
LAYER_TENSORS = 15   # per-layer tensor ids: 5 + LAYER_TENSORS * layer + kind (mpk_read_tensor)


class MpkError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class mpk_model_cfg(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "vocab",
                                         "max_seq_len", "qk_norm", "tied_embedding")] + \
               [("rms_eps", C.c_float), ("rope_theta", C.c_float)] + \
               [(n, C.c_int32) for n in ("n_experts", "top_k", "moe_ffn", "norm_topk")]


class mpk_build_params(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_workers", "n_sched_waves", "quantum", "t_qkv", "t_o", "t_gu", "t_down",
                                         "t_lm", "s_attn", "host_only", "fusion_order", "aot_policy", "k_qkv", "k_o", "k_down",
                                         "attn_jit", "weight_preload", "coarse_events", "t_router", "t_egu",
                                         "t_edown", "attn_split_pages")]


class mpk_weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("lm_head", C.c_void_p), ("final_norm", C.c_void_p),
                ("layer", C.POINTER(C.c_void_p)), ("layout", C.c_int32)]


class mpk_kv(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("page_table", C.c_void_p),
                ("n_pages", C.c_int32), ("max_pages_per_seq", C.c_int32)]


class mpk_tgraph_header(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_tasks", "n_events", "root", "end", "n_fused", "n_empty", "n_rewrites",
                                         "n_aot", "batch", "page_size")] + [("params", mpk_build_params)]


class mpk_tgraph_host_view(C.Structure):
    _fields_ = [("header", mpk_tgraph_header),
                ("task_type", C.POINTER(C.c_uint8)), ("task_mode", C.POINTER(C.c_uint8)),
                ("task_layer", C.POINTER(C.c_int16)), ("task_coords", C.POINTER(C.c_uint16)),
                ("task_orig", C.POINTER(C.c_int32)), ("task_dep", C.POINTER(C.c_int32)),
                ("task_trig", C.POINTER(C.c_int32)), ("task_worker", C.POINTER(C.c_int16)),
                ("event_counts", C.POINTER(C.c_uint32)), ("event_first", C.POINTER(C.c_int32)),
                ("event_last", C.POINTER(C.c_int32)), ("event_flags", C.POINTER(C.c_uint8)),
                ("aot_offsets", C.POINTER(C.c_uint32)), ("aot_tasks", C.POINTER(C.c_uint32))]


class mpk_task_spec(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("type", "layer", "c0", "c1", "c2")]


class mpk_region(C.Structure):
    _fields_ = [("task", C.c_int32), ("is_out", C.c_int32), ("tensor", C.c_int32), ("lo", C.c_int32 * 4),
                ("hi", C.c_int32 * 4)]


class mpk_status_word(C.Structure):
    _fields_ = [("code", C.c_int32), ("wg", C.c_int32), ("task", C.c_int32), ("event", C.c_int32),
                ("counter", C.c_uint32), ("target", C.c_uint32)]


class mpk_trace_record(C.Structure):
    _fields_ = [("task", C.c_int32), ("worker", C.c_int32), ("t_wait", C.c_uint64), ("t_start", C.c_uint64),
                ("t_end", C.c_uint64), ("t_done", C.c_uint64), ("t_mark", C.c_uint64 * 2)]


# symbol -> (restype, argtypes); the list every test checks against the header
SIGNATURES = {
    "mpk_build_tgraph": (C.c_int, [C.POINTER(mpk_model_cfg), C.c_int32, C.c_int32, C.POINTER(C.c_void_p)]),
    "mpk_build_tgraph_ex": (C.c_int, [C.POINTER(mpk_model_cfg), C.c_int32, C.c_int32, C.POINTER(mpk_build_params),
                                      C.POINTER(C.c_void_p)]),
    "mpk_tgraph_info": (C.c_int, [C.c_void_p, C.POINTER(mpk_tgraph_header)]),
    "mpk_tgraph_export": (C.c_int, [C.c_void_p, C.POINTER(mpk_tgraph_host_view)]),
    "mpk_build_generic": (C.c_int, [C.POINTER(mpk_task_spec), C.c_int32, C.POINTER(mpk_region), C.c_int32,
                                    C.c_int32, C.POINTER(mpk_tgraph_host_view)]),
    "mpk_build_generic_ex": (C.c_int, [C.POINTER(mpk_task_spec), C.c_int32, C.POINTER(mpk_region), C.c_int32,
                                       C.POINTER(mpk_build_params), C.POINTER(mpk_tgraph_host_view)]),
    "mpk_free_host_view": (None, [C.POINTER(mpk_tgraph_host_view)]),
    "mpk_prepared_weights_bytes": (C.c_int, [C.c_void_p, C.POINTER(C.c_size_t)]),
    "mpk_prepare_weights": (C.c_int, [C.c_void_p, C.POINTER(mpk_weights), C.c_void_p, C.c_size_t,
                                      C.POINTER(C.c_void_p), C.POINTER(mpk_weights), C.c_void_p]),
    "mpk_decode_step": (C.c_int, [C.c_void_p, C.POINTER(mpk_weights), C.c_void_p, C.POINTER(mpk_kv), C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_void_p]),
    "mpk_decode_step_noalloc": (C.c_int, [C.c_void_p, C.POINTER(mpk_weights), C.c_void_p, C.POINTER(mpk_kv),
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "mpk_decode_step_baseline": (C.c_int, [C.c_void_p, C.POINTER(mpk_weights), C.c_void_p, C.POINTER(mpk_kv),
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32]),
    "mpk_read_tensor": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t]),
    "mpk_set_watchdog": (C.c_int, [C.c_void_p, C.c_uint64]),
    "mpk_reset_tgraph": (C.c_int, [C.c_void_p]),
    "mpk_set_trace": (C.c_int, [C.c_void_p, C.c_int32]),
    "mpk_read_trace": (C.c_int, [C.c_void_p, C.POINTER(mpk_trace_record), C.c_int32, C.POINTER(C.c_int32),
                                 C.POINTER(C.c_double)]),
    "mpk_time_tasks": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.c_int32, C.c_int32, C.POINTER(C.c_uint64),
                                 C.POINTER(C.c_double)]),
    "mpk_run_tasks": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32, C.c_int32]),
    "mpk_get_status": (C.c_int, [C.c_void_p, C.POINTER(mpk_status_word)]),
    "mpk_destroy_tgraph": (None, [C.c_void_p]),
    "mpk_last_error": (C.c_char_p, []),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m task_graph_runtime_amd.build`")
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc):
    if rc != MPK_OK:
        raise MpkError(rc, lib().mpk_last_error().decode())


def model_cfg(shape) -> mpk_model_cfg:
    """mpk_model_cfg from any object/dict with the decoder fields."""
    g = (lambda k: shape[k]) if isinstance(shape, dict) else (lambda k: getattr(shape, k))
    opt = (lambda k, d: shape.get(k, d)) if isinstance(shape, dict) else (lambda k, d: getattr(shape, k, d))
    return mpk_model_cfg(int(g("n_layers")), int(g("hidden")), int(g("n_q_heads")), int(g("n_kv_heads")),
                         int(g("head_dim")), int(g("ffn")), int(g("vocab")), int(g("max_seq_len")),
                         int(bool(g("qk_norm"))), int(bool(g("tied_embedding"))), float(g("rms_eps")),
                         float(g("rope_theta")), int(opt("n_experts", 0)), int(opt("top_k", 0)),
                         int(opt("moe_ffn", 0)), int(bool(opt("norm_topk", True))))


def _view_to_dict(v: mpk_tgraph_host_view) -> dict:
    h = v.header
    NT, NE, W = h.n_tasks, h.n_events, h.params.n_workers

    def arr(ptr, n, dt):
        return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dt, copy=True) if n else np.zeros(0, dt)
    out = {
        "task_type": arr(v.task_type, NT, np.uint8), "task_mode": arr(v.task_mode, NT, np.uint8),
        "task_layer": arr(v.task_layer, NT, np.int16),
        "task_coords": arr(v.task_coords, 3 * NT, np.uint16).reshape(NT, 3),
        "task_orig": arr(v.task_orig, NT, np.int32), "task_dep": arr(v.task_dep, NT, np.int32),
        "task_trig": arr(v.task_trig, NT, np.int32), "task_worker": arr(v.task_worker, NT, np.int16),
        "event_counts": arr(v.event_counts, NE, np.uint32), "event_first": arr(v.event_first, NE, np.int32),
        "event_last": arr(v.event_last, NE, np.int32), "event_flags": arr(v.event_flags, NE, np.uint8),
        "aot_offsets": arr(v.aot_offsets, W + 1, np.uint32), "aot_tasks": arr(v.aot_tasks, h.n_aot, np.uint32),
    }
    p = h.params
    out["header"] = dict(NT=NT, NE=NE, root=h.root, end=h.end, n_fused=h.n_fused, n_empty=h.n_empty,
                         n_rewrites=h.n_rewrites)
    out["params"] = {f: getattr(p, f) for f, _ in mpk_build_params._fields_}
    return out


def build_generic(specs, regions, n_workers, fusion_order: int = 0, attn_jit: int = 0) -> dict:
    """Canonicalise arbitrary tasks/boxes in the library (host only)."""
    S = (mpk_task_spec * max(1, len(specs)))(*[mpk_task_spec(*map(int, s)) for s in specs])
    R = (mpk_region * max(1, len(regions)))()
    for i, (t, is_out, tn, lo, hi) in enumerate(regions):
        R[i].task, R[i].is_out, R[i].tensor = int(t), int(is_out), int(tn)
        for k in range(4):
            R[i].lo[k], R[i].hi[k] = int(lo[k]), int(hi[k])
    p = mpk_build_params()
    p.n_workers, p.fusion_order, p.attn_jit = int(n_workers), int(fusion_order), int(attn_jit)
    v = mpk_tgraph_host_view()
    _check(lib().mpk_build_generic_ex(S, len(specs), R, len(regions), C.byref(p), C.byref(v)))
    try:
        return _view_to_dict(v)
    finally:
        lib().mpk_free_host_view(C.byref(v))


def _ptr(t):
    return C.c_void_p(0 if t is None else int(t.data_ptr()))


class Weights:
    """mpk_weights over a dict of bf16 device tensors (the synth layout)."""
    NAMES = ("in_norm", "q", "k", "v", "q_norm", "k_norm", "o", "post_norm", "gate", "up", "down", "router")

    def __init__(self, w: dict):
        self._keep = w
        layers = w["layers"]
        self._arr = (C.c_void_p * (len(layers) * 12))(*[int(lw[n].data_ptr()) if lw.get(n) is not None else 0
                                                          for lw in layers for n in self.NAMES])
        self.s = mpk_weights(int(w["embed"].data_ptr()), 0 if w.get("lm_head") is None else int(w["lm_head"].data_ptr()),
                             int(w["final_norm"].data_ptr()), C.cast(self._arr, C.POINTER(C.c_void_p)), 0)


class PreparedWeights:
    """Weights of one batch > 1 graph in the matrix-core load order
    (mpk_prepare_weights): a device buffer (torch uint8 tensor) and the
    prepared mpk_weights that point into it.  Holds the source weights until
    the repack has run (the caller's stream is synchronised)."""

    def __init__(self, g: "TGraph", w: Weights, stream=None):
        import torch
        n = C.c_size_t()
        _check(lib().mpk_prepared_weights_bytes(g.h, C.byref(n)))
        self.buf = torch.empty(max(1, n.value), dtype=torch.uint8, device="cuda")
        n_layers = g.cfg.n_layers
        self._arr = (C.c_void_p * (n_layers * 12))()
        self.s = mpk_weights()
        _check(lib().mpk_prepare_weights(g.h, C.byref(w.s), C.c_void_p(self.buf.data_ptr()), n.value,
                                         C.cast(self._arr, C.POINTER(C.c_void_p)), C.byref(self.s), _stream_ptr(stream)))
        torch.cuda.synchronize()
        self._keep = w._keep  # the embedding and norm gains are the caller's own


class KV:
    """mpk_kv over device tensors: k_pool, v_pool (bf16), page_table (int32 [B, max_pages])."""

    def __init__(self, k_pool, v_pool, page_table):
        self._keep = (k_pool, v_pool, page_table)
        self.s = mpk_kv(int(k_pool.data_ptr()), int(v_pool.data_ptr()), int(page_table.data_ptr()),
                        int(k_pool.shape[1]), int(page_table.shape[1]))


def _stream_ptr(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return C.c_void_p(int(stream))


class TGraph:
    """A built tGraph (library-owned); mirrors mpk_build_tgraph_ex and friends."""

    def __init__(self, cfg, batch: int, page_size: int, params: dict | None = None, host_only: bool = False):
        self.cfg = cfg if isinstance(cfg, mpk_model_cfg) else model_cfg(cfg)
        p = mpk_build_params()
        for k, v in (params or {}).items():
            setattr(p, k, int(v))
        p.host_only = int(host_only)
        h = C.c_void_p()
        _check(lib().mpk_build_tgraph_ex(C.byref(self.cfg), int(batch), int(page_size), C.byref(p), C.byref(h)))
        self.h = h
        self.batch = batch

    def close(self):
        if self.h:
            lib().mpk_destroy_tgraph(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def header(self) -> dict:
        hd = mpk_tgraph_header()
        _check(lib().mpk_tgraph_info(self.h, C.byref(hd)))
        return {f: getattr(hd, f) for f, _ in mpk_tgraph_header._fields_ if f != "params"} | \
            {"params": {f: getattr(hd.params, f) for f, _ in mpk_build_params._fields_}}

    def export(self) -> dict:
        v = mpk_tgraph_host_view()
        _check(lib().mpk_tgraph_export(self.h, C.byref(v)))
        try:
            return _view_to_dict(v)
        finally:
            lib().mpk_free_host_view(C.byref(v))

    def decode_step(self, w: Weights, token_ids, kv: KV, seq_lens, logits, next_ids, stream=None):
        _check(lib().mpk_decode_step(self.h, C.byref(w.s), _ptr(token_ids), C.byref(kv.s), _ptr(seq_lens),
                                     _ptr(logits), _ptr(next_ids), _stream_ptr(stream)))

    def decode_step_noalloc(self, w: Weights, token_ids, kv: KV, seq_lens, logits, next_ids, stream=None):
        _check(lib().mpk_decode_step_noalloc(self.h, C.byref(w.s), _ptr(token_ids), C.byref(kv.s), _ptr(seq_lens),
                                             _ptr(logits), _ptr(next_ids), _stream_ptr(stream)))

    def decode_step_baseline(self, w: Weights, token_ids, kv: KV, seq_lens, logits, next_ids, stream=None,
                             use_hipgraph: bool = False):
        _check(lib().mpk_decode_step_baseline(self.h, C.byref(w.s), _ptr(token_ids), C.byref(kv.s), _ptr(seq_lens),
                                              _ptr(logits), _ptr(next_ids), _stream_ptr(stream),
                                              int(bool(use_hipgraph))))

    def read_tensor(self, tensor: int, shape, dtype) -> np.ndarray:
        out = np.empty(shape, dtype=dtype)
        _check(lib().mpk_read_tensor(self.h, int(tensor), out.ctypes.data_as(C.c_void_p), out.nbytes))
        return out

    def set_trace(self, enable: bool = True):
        _check(lib().mpk_set_trace(self.h, int(bool(enable))))

    def read_trace(self) -> tuple:
        """Records of the last traced step as a numpy structured array, and ticks/us."""
        cap = self.header()["n_tasks"] + 16
        buf = (mpk_trace_record * cap)()
        n = C.c_int32()
        tpu = C.c_double()
        _check(lib().mpk_read_trace(self.h, buf, cap, C.byref(n), C.byref(tpu)))
        dt = np.dtype([("task", np.int32), ("worker", np.int32), ("t_wait", np.uint64), ("t_start", np.uint64),
                       ("t_end", np.uint64), ("t_done", np.uint64), ("t_mark", np.uint64, (2,))])
        arr = np.frombuffer(bytes(buf), dtype=dt, count=cap)[: n.value].copy()
        return arr, tpu.value

    def time_tasks(self, tasks, reps: int = 5, cold: bool = False) -> np.ndarray:
        """Mean duration (us) of each listed task run alone in one workgroup
        (cold: caches of its die invalidated before each run)."""
        n = len(tasks)
        T = (C.c_int32 * n)(*[int(t) for t in tasks])
        out = (C.c_uint64 * n)()
        tpu = C.c_double()
        _check(lib().mpk_time_tasks(self.h, T, n, int(reps), int(bool(cold)), out, C.byref(tpu)))
        return np.array(list(out), dtype=np.float64) / tpu.value

    def run_tasks(self, tasks, poison: bool = True):
        """Run the listed tasks serially in one workgroup (mpk_run_tasks),
        after filling every library-owned activation with NaN when poison."""
        n = len(tasks)
        T = (C.c_int32 * n)(*[int(t) for t in tasks])
        _check(lib().mpk_run_tasks(self.h, T, n, int(bool(poison))))

    def set_watchdog(self, ns: int):
        _check(lib().mpk_set_watchdog(self.h, int(ns)))

    def reset(self):
        """Clear the runtime state of a (poisoned) graph; the next step runs as its first."""
        _check(lib().mpk_reset_tgraph(self.h))

    def status(self) -> dict:
        s = mpk_status_word()
        _check(lib().mpk_get_status(self.h, C.byref(s)))
        return {f: getattr(s, f) for f, _ in mpk_status_word._fields_}
