"""Device-side preparation of NVFP4 expert weights.

Synthetic fp32 weights (from ``synth``) are copied to the GPU one expert at
a time and quantised there by the library's ``nvfp4_quantize`` into stacked
[E, rows, cols/2] code and [E, rows, cols/16] scale tensors with one decode
scale per (expert, projection).
"""
from __future__ import annotations

import torch

from . import native, synth


def empty_experts(E, H, I, device):
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return native.ExpertWeights(
        torch.empty((E, I, H // 2), **u8), torch.empty((E, I, H // 16), **u8),
        torch.empty(E, **f32),
        torch.empty((E, I, H // 2), **u8), torch.empty((E, I, H // 16), **u8),
        torch.empty(E, **f32),
        torch.empty((E, H, I // 2), **u8), torch.empty((E, H, I // 16), **u8),
        torch.empty(E, **f32))


def quantize_into(w: native.ExpertWeights, e: int, gate, up, down, workspace=None):
    """Quantise one expert's fp32 device matrices into slot e of w."""
    # nvfp4_quantize(COMPUTE) writes g into its own 1-element tensor; copy it
    # into the stacked vector (a device-to-device copy on the same stream).
    _, _, g = native.nvfp4_quantize(gate, out=(w.gate_codes[e], w.gate_scales[e]),
                                    workspace=workspace)
    w.gate_global[e:e + 1].copy_(g)
    _, _, g = native.nvfp4_quantize(up, out=(w.up_codes[e], w.up_scales[e]),
                                    workspace=workspace)
    w.up_global[e:e + 1].copy_(g)
    _, _, g = native.nvfp4_quantize(down, out=(w.down_codes[e], w.down_scales[e]),
                                    workspace=workspace)
    w.down_global[e:e + 1].copy_(g)


def synthetic_experts(E, H, I, seed=0, device="cuda", experts=None):
    """Stacked NVFP4 experts quantised on the GPU from synth's fp32 weights.

    experts: the expert indices to fill (default all); the others stay
    uninitialised and must not be routed to.
    """
    w = empty_experts(E, H, I, device)
    ids = list(range(E)) if experts is None else list(experts)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=device)
    for e, (g, u, d) in zip(ids, synth.map_experts(
            lambda e: synth.expert_weights_f32(e, H, I, seed), ids)):
        quantize_into(w, e, torch.from_numpy(g).to(device), torch.from_numpy(u).to(device),
                      torch.from_numpy(d).to(device), workspace=ws)
    return w
