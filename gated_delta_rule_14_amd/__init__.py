"""libkda: the Kimi Delta Attention operator on AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind the C ABI of include/kda.h; this package is
their Python binding (gated_delta_rule_14_amd.kda) and their build script
(gated_delta_rule_14_amd.build).
"""
from .kda import chunk_fwd, chunk_fwd_workspace_bytes, layer, out_gate, recurrent_step

__all__ = ["chunk_fwd", "chunk_fwd_workspace_bytes", "recurrent_step", "out_gate", "layer"]
