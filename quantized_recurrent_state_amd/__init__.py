"""LeapQuant per-window int8 recurrent-state decode for Gated DeltaNet heads
on MI355X (gfx950): a C-ABI HIP library (libleapq.so) and its Python binding.

    from quantized_recurrent_state_amd import leapq
    layer = leapq.Layer(leapq.make_config(batch, heads), "cuda")
    leapq.leapq_init_state(layer, S0)
    leapq.leapq_append(layer, q, k, v, alpha, beta, o)   # every token
    leapq.leapq_fold(layer)                              # every window
"""
from . import leapq, workloads  # noqa: F401

__all__ = ["leapq", "workloads"]
