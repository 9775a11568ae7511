"""Test plumbing: hand the same synthetic tensors to the oracle (numpy) and the HIP path (torch)."""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (exact; what the oracle widens)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


class LazyLayers:
    """Per-layer weights copied to the host only when the oracle asks for them."""

    def __init__(self, layers):
        self._layers = layers

    def __len__(self):
        return len(self._layers)

    def __getitem__(self, l):
        return {k: bf16_bits(v) for k, v in self._layers[l].items()}


def oracle_weights(w: dict, lazy: bool = False) -> dict:
    layers = LazyLayers(w["layers"]) if lazy else [
        {k: bf16_bits(v) for k, v in lw.items()} for lw in w["layers"]]
    return {"embed": bf16_bits(w["embed"]), "final_norm": bf16_bits(w["final_norm"]),
            "lm_head": None if w["lm_head"] is None else bf16_bits(w["lm_head"]), "layers": layers}


def run_oracle(inp: dict, dtype=np.float32, capture=None, lazy=False):
    from oracle import numerics
    s = inp["shape"]
    kv = inp["kv"]
    return numerics.decode_step(s.cfg(), oracle_weights(inp["weights"], lazy=lazy),
                                inp["token_ids"].numpy(), bf16_bits(kv["k_pool"]), bf16_bits(kv["v_pool"]),
                                kv["page_table"].numpy(), inp["seq_lens"].numpy(), s.page_size,
                                dtype=dtype, capture=capture)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32/fp64 to the nearest bf16 (ties to even), returned as fp32."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).float().numpy()
