"""MI355X (gfx950) routed-expert block of the Kimi K3 Stable LatentMoE.

The work happens in ``libk3moe.so`` (hand-written HIP kernels behind the C ABI in
``include/k3moe.h``); ``lib`` is its ctypes binding and ``_build`` compiles it.
"""
from . import lib  # noqa: F401
from .lib import LatentWeights, Pool, forward_decode_pooled, latent_forward, slot_layout  # noqa: F401
from .lib import (ExpertWeights, K3moeError, decode_down, decode_gateup, dequant_mxfp4,  # noqa: F401
                  forward_chunk, forward_chunk_mx, forward_decode, forward_decode_timed, group, load, mx_quant, route, route_topp,
                  status_string, workspace_size)
