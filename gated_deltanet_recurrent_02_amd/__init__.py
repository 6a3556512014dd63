"""Gated DeltaNet recurrent decode step for MI355X (gfx950).

The compute lives in libgdn.so (hand-written HIP kernels behind the C ABI of include/gdn.h);
this package holds the ctypes binding (`decode_step`, `decode_verify`, `conv_gate_decode`,
`prefill`, `prefill_noalloc`, `prefill_workspace_size`, `lowrank_decode_step`, `lowrank_state`,
`state_alloc`), the in-tree build (`build`), and the seeded synthetic input generator
(`synth`).
"""
from ._binding import (EXPORTS, GDNError, StateBuffer, check, conv_gate_decode, decode_step,
                       decode_verify, lib, lowrank_decode_step, lowrank_state, prefill,
                       prefill_noalloc, prefill_workspace, prefill_workspace_size, state_alloc)

__all__ = ["EXPORTS", "GDNError", "StateBuffer", "check", "conv_gate_decode", "decode_step",
           "decode_verify", "lib", "lowrank_decode_step", "lowrank_state", "prefill",
           "prefill_noalloc", "prefill_workspace", "prefill_workspace_size", "state_alloc"]
