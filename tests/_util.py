"""Test plumbing: hand the same synthetic tensors to the oracle (numpy) and the HIP path (torch)."""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (exact; what the oracle widens)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> exact fp32 numpy copy (widened on the tensor's device)."""
    return t.detach().float().cpu().numpy()


class LazyLayers:
    """Per-layer weights copied to the host only when the oracle asks for them."""

    def __init__(self, layers, conv):
        self._layers = layers
        self._conv = conv

    def __len__(self):
        return len(self._layers)

    def __getitem__(self, l):
        return {k: (LazyExperts(v, self._conv) if v.dim() == 3 else self._conv(v))
                for k, v in self._layers[l].items()}


class LazyExperts:
    """An expert stack ``[E][...]`` whose experts are copied to the host one at a
    time, when the oracle reads them (it reads only the chosen ones)."""

    def __init__(self, t, conv):
        self._t = t
        self._conv = conv

    def __len__(self):
        return self._t.shape[0]

    def __getitem__(self, e):
        return self._conv(self._t[e])


def oracle_weights(w: dict, lazy: bool = False, widen_on_device: bool = False) -> dict:
    conv = host_f32 if widen_on_device else bf16_bits
    layers = LazyLayers(w["layers"], conv) if lazy else [
        {k: conv(v) for k, v in lw.items()} for lw in w["layers"]]
    return {"embed": bf16_bits(w["embed"]), "final_norm": conv(w["final_norm"]),
            "lm_head": None if w["lm_head"] is None else conv(w["lm_head"]), "layers": layers}


def run_oracle(inp: dict, dtype=np.float32, capture=None, lazy=False, widen_on_device=False, route_hook=None):
    from oracle import numerics
    s = inp["shape"]
    kv = inp["kv"]
    return numerics.decode_step(s.cfg(), oracle_weights(inp["weights"], lazy=lazy, widen_on_device=widen_on_device),
                                inp["token_ids"].cpu().numpy(), bf16_bits(kv["k_pool"]), bf16_bits(kv["v_pool"]),
                                kv["page_table"].cpu().numpy(), inp["seq_lens"].cpu().numpy(), s.page_size,
                                dtype=dtype, capture=capture, route_hook=route_hook)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32/fp64 to the nearest bf16 (ties to even), returned as fp32."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()
