"""Seeded synthetic inputs for the NVFP4 routed-expert FFN.

This module only draws random numbers; it holds none of the method's
arithmetic (no quantisation, routing or matmul), so the oracle and the HIP
path can both be fed from it.  Every tensor comes from numpy's PCG64 seeded
by SeedSequence([seed, tensor_id, expert]):

    tensor_id 0 = activations x, 1 = router logits, 2 = gate, 3 = up, 4 = down,
    5 = router matrix, 6/7/8 = shared expert gate/up/down.

Activations are N(0, 1) rounded to bf16 (torch's round-to-nearest-even
cast), weights N(0, 0.02^2) in fp32 (the caller quantises them), router
logits N(0, 1) in fp32, optionally plus a Zipf-shaped per-expert bias
b_e = -s ln(e + 1) (the log of an unnormalised Zipf(s) weight of rank e + 1),
which leaves many experts without tokens.  The bf16 router matrix R [E, H]
is N(0, 1/H) rounded to bf16, so that x . R^T is again about N(0, 1); the
same Zipf bias can be passed to the router as its per-expert bias.  The
shared expert's bf16 weights are N(0, 0.02^2) like the routed ones.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses

import numpy as np
import torch

X, LOGITS, GATE, UP, DOWN, ROUTER = 0, 1, 2, 3, 4, 5
SHARED_GATE, SHARED_UP, SHARED_DOWN = 6, 7, 8
WEIGHT_STD = 0.02


def rng(seed: int, tensor_id: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, expert])))


def activations(T: int, H: int, seed: int = 0) -> torch.Tensor:
    """bf16 [T, H] ~ N(0, 1) on the CPU."""
    x = rng(seed, X).standard_normal((T, H), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def router_logits(T: int, E: int, seed: int = 0, zipf_s: float | None = None,
                  gumbel: bool = False) -> np.ndarray:
    """fp32 [T, E] router logits.  zipf_s adds b_e = -s ln(e+1); gumbel draws
    standard Gumbel noise instead of N(0, 1)."""
    g = rng(seed, LOGITS)
    if gumbel:
        noise = g.gumbel(size=(T, E)).astype(np.float32)
    else:
        noise = g.standard_normal((T, E), dtype=np.float32)
    if zipf_s is not None:
        noise = (noise + zipf_bias(E, zipf_s)[None, :]).astype(np.float32)
    return noise


def router_matrix(E: int, H: int, seed: int = 0) -> torch.Tensor:
    """bf16 [E, H] ~ N(0, 1/H) on the CPU."""
    r = rng(seed, ROUTER).standard_normal((E, H), dtype=np.float32)
    r *= np.float32(1.0 / np.sqrt(H))
    return torch.from_numpy(r).to(torch.bfloat16)


def shared_expert_weights(H: int, I: int, seed: int = 0):
    """bf16 (gate [I, H], up [I, H], down [H, I]) ~ N(0, 0.02^2) on the CPU."""
    return tuple(torch.from_numpy(weight(n, k, tid, 0, seed)).to(torch.bfloat16)
                 for n, k, tid in ((I, H, SHARED_GATE), (I, H, SHARED_UP), (H, I, SHARED_DOWN)))


def zipf_bias(E: int, zipf_s: float) -> np.ndarray:
    """fp32 [E]: b_e = -s ln(e + 1)."""
    return (-zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def weight(n: int, k: int, tensor_id: int, expert: int = 0, seed: int = 0) -> np.ndarray:
    """fp32 [n, k] ~ N(0, 0.02^2) for one expert's projection."""
    w = rng(seed, tensor_id, expert).standard_normal((n, k), dtype=np.float32)
    w *= np.float32(WEIGHT_STD)
    return w


def expert_weights_f32(expert: int, H: int, I: int, seed: int = 0):
    """(gate [I, H], up [I, H], down [H, I]) fp32 for one expert."""
    return (weight(I, H, GATE, expert, seed), weight(I, H, UP, expert, seed),
            weight(H, I, DOWN, expert, seed))


def map_experts(fn, experts, workers: int = 8):
    """Run fn(expert) over experts with a thread pool (numpy releases the GIL
    while it fills arrays), yielding results in order."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        yield from ex.map(fn, experts)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # tokens (rows of x)
    H: int          # hidden
    I: int          # expert intermediate
    E: int          # experts
    k: int          # experts per token
    act: str = "w4a16"
    zipf_s: float | None = None
    description: str = ""


# The benchmark workloads: a dense MLP decode, routed MoE decode, a 512-token
# prefill chunk with a skewed router and a W4A4 prefill.
LINEAR_SMALL = dict(M=4, K=256, N=512)
MLP_DECODE = [Workload(f"mlp_decode_m{m}", m, 5120, 17408, 1, 1,
                       description="dense NVFP4 MLP decode, x bf16 [M,5120], "
                                   "gate/up [17408,5120], down [5120,17408]")
              for m in (1, 8, 32)]
MOE_DECODE = Workload("moe_decode", 16, 2048, 512, 512, 8,
                      description="routed MoE decode: 16 tokens, hidden 2048, 512 experts, "
                                  "intermediate 512, top-8 of softmax, renormalised")
MOE_PREFILL = Workload("moe_prefill", 512, 2048, 512, 512, 8, zipf_s=1.1,
                       description="routed MoE prefill chunk: 512 tokens, hidden 2048, 512 "
                                   "experts, intermediate 512, top-8, Zipf(1.1) router bias")
MOE_PREFILL_W4A4 = Workload("moe_prefill_w4a4", 2048, 4096, 1536, 128, 8, act="w4a4",
                            description="W4A4 MoE prefill: 2048 tokens, hidden 4096, 128 "
                                        "experts, intermediate 1536, top-8 uniform routing")
MLP_PREFILL = [Workload(f"mlp_prefill_m{m}", m, 5120, 17408, 1, 1,
                        description="dense NVFP4 MLP prefill, x bf16 [M,5120], "
                                    "gate/up [17408,5120], down [5120,17408]")
               for m in (512, 2048)]
WORKLOADS = {w.name: w for w in [*MLP_DECODE, *MLP_PREFILL, MOE_DECODE, MOE_PREFILL,
                                 MOE_PREFILL_W4A4]}
