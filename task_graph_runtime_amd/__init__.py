"""MI355X (gfx950) decode-step mega-kernel: a task/event graph built on the host
and executed by one persistent HIP kernel.  See ``include/mpk.h`` for the C ABI;
this package is its thin Python binding.
"""
from ._binding import (MpkError, TGraph, Weights, PreparedWeights, KV, build_generic, lib, model_cfg, mpk_weights,  # noqa: F401
                       mpk_build_params, mpk_model_cfg, SIGNATURES)
