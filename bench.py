"""Benchmark of the NVFP4 routed-expert FFN hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
top-k routing + permutation (moe_route_topk), then the grouped FFN
(moe_grouped_nvfp4_ffn: plan, activation prep, gate/up GEMM with SiLU*up,
h prep, down GEMM times routing weight, combine).  Inputs are resident in HBM
before timing starts.  Steps cycle over several copies of the expert
weights, so every step streams its active experts from HBM instead of the
256 MB Infinity Cache (MALL).  The timed steps run as HIP graph replays; one
graph holds a pass over all the copies (several consecutive steps, as a
model's layers share one graph), so replays of one-step graphs do not add
their launch gap to every step; the timed region covers exactly K steps.

Prints one JSON line: the metric, the step throughput, the roofline figures
of the gate/up kernel and the CPU oracle's throughput on a sample of the
same step.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 MoE FFN: decode HBM GB/s (% peak); prefill TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA


def nv_bytes(n):
    """NVFP4 bytes of n elements: n/2 code bytes + n/16 scale bytes."""
    return n // 2 + n // 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="moe_decode",
                    help="moe_decode | moe_prefill | moe_prefill_w4a4 | mlp_decode_m{1,8,32} | "
                         "mlp_prefill_m{512,2048}")
    ap.add_argument("--copies", type=int, default=0,
                    help="weight copies cycled per step (0 = enough for >= 2 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0 = workload default)")
    ap.add_argument("--eager", action="store_true", help="no graph capture")
    ap.add_argument("--given-globals", action="store_true",
                    help="W4A4: static activation scales given by the caller (g_x from the "
                         "input's amax, g_h a fixed calibration value) instead of online ones")
    ap.add_argument("--with-router", action="store_true",
                    help="the step starts from x and the bf16 router matrix (router GEMM + "
                         "top-k, moe_router_topk) instead of from given logits")
    ap.add_argument("--with-shared", action="store_true",
                    help="add the BF16 shared expert (intermediate size = the routed one) "
                         "to every token's output (moe_shared_expert_ffn, accumulating)")
    ap.add_argument("--separate-h-quant", action="store_true",
                    help="with --given-globals: quantise h in its own pass instead of the "
                         "gate/up epilogue (same results)")
    ap.add_argument("--paged", type=int, default=0, metavar="S",
                    help="expert paging: all experts in pinned host memory, S device slots; "
                         "times route + slot plan + fetch + FFN on the pool (own JSON line)")
    ap.add_argument("--paged-overlap", action="store_true",
                    help="with --paged: also time a two-stream pipeline (routing, slot plan "
                         "and fetch of step i+1 beside the FFN of step i)")
    ap.add_argument("--paged-zipf", type=float, default=None,
                    help="with --paged: Zipf exponent of a router bias (expert popularity; "
                         "default: the workload's own routing)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB elementwise copy kernel (for scaling "
                         "hardware byte counters)")
    return ap.parse_args()


# Sources each timed kernel is built from; a stored counter reading is used
# only while these files are byte-identical to the ones it was taken on.
KERNEL_SOURCES = {
    "row_ffn_kernel": ["rowgemv.hip", "common.h", "kernels.h"],
    "row_gemv_kernel": ["rowgemv.hip", "common.h", "kernels.h"],
    "tile_gemm_kernel": ["tile_gemm.hip", "common.h", "kernels.h"],
    "grouped_gemm_kernel": ["gemm.hip", "common.h", "kernels.h"],
    "grouped_gemv_kernel": ["gemv.hip", "common.h", "kernels.h"],
}


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "nvfp4_routed_expert_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel
    calibration), or None when there is none or the kernel has changed."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_digest") != source_digest(kernel):
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def gate_up_kernel(T, H, I, E, k, act):
    """Which kernel runs the gate/up projection (mirrors the library's dispatch:
    decode-sized batches stream rows or run the small GEMV, anything larger
    the LDS-tiled grouped GEMM, or the generic one when H % 64 != 0)."""
    P = T * k
    small = P <= 2 if E == 1 else (P <= 256 and 2 * P <= 32 * E)
    row_ok = lambda K: K in (256, 512, 1024) or (K % 32 == 0 and 2048 <= K <= 32768)
    if small:
        if act == "w4a16" and row_ok(H) and row_ok(I):
            # H = 2048 and I a multiple of 256: both projections in one launch
            return "row_ffn_kernel" if H == 2048 and I % 256 == 0 else "row_gemv_kernel"
        return "grouped_gemv_kernel"
    return "tile_gemm_kernel" if H % 64 == 0 else "grouped_gemm_kernel"


class HipEvents:
    """Raw HIP events (for the library's per-stage event hook)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            self.arr[i] = h
        self.n = n

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[a], self.arr[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return out.value

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the routed-expert "
                                   "FFN is measured on one GPU's share (it would shard by "
                                   "expert, one exchange of y per step)", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.paged:
        return paged_main(args)

    import numpy as np
    import torch

    from nvfp4_routed_expert_amd import native, synth, weights

    wl = synth.WORKLOADS[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    act = native.W4A4 if wl.act == "w4a4" else native.W4A16
    P = T * k

    # ---- inputs (seeded synthetic, resident in HBM) -----------------------------
    x_cpu = synth.activations(T, H)
    logits_np = synth.router_logits(T, E, zipf_s=wl.zipf_s)
    x = x_cpu.to(dev)
    logits = torch.from_numpy(logits_np).to(dev)
    t0 = time.time()
    w0 = weights.synthetic_experts(E, H, I, 0, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    bytes_all = 3 * E * (nv_bytes(H * I) + 4)
    copies = args.copies or max(1, int(np.ceil(2 * 2 ** 30 / bytes_all)))
    copies = min(copies, 16)
    wcopies = [w0]
    for _ in range(copies - 1):
        wcopies.append(native.ExpertWeights(*[t.clone() for t in (
            w0.gate_codes, w0.gate_scales, w0.gate_global, w0.up_codes, w0.up_scales,
            w0.up_global, w0.down_codes, w0.down_scales, w0.down_global)]))

    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pairs = torch.empty(P, dtype=torch.int32, device=dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(native.ffn_workspace_bytes(T, H, I, E, k, act), dtype=torch.uint8,
                     device=dev)
    ag = None
    if act == native.W4A4 and args.given_globals:   # static calibration scales
        ag = torch.tensor([float(x_cpu.float().abs().max()) / 2688.0, 0.05 / 2688.0],
                          dtype=torch.float32, device=dev)
    native.set_ffn_separate_h_quant(args.separate_h_quant)
    rws = native.route_workspace(T, E, k, dev)
    route = E > 1
    with_router = args.with_router and route
    if with_router:
        router_w = synth.router_matrix(E, H).to(dev)
        router_b = (None if wl.zipf_s is None else
                    torch.from_numpy(synth.zipf_bias(E, wl.zipf_s)).to(dev))
        rtws = native.router_workspace(T, H, E, k, dev)

    with_shared = args.with_shared and route
    if with_shared:
        sh_w = [t.to(dev) for t in synth.shared_expert_weights(H, I)]
        sh_ws = torch.empty(max(native.lib().moe_shared_expert_ffn_workspace_size(T, H, I), 1),
                            dtype=torch.uint8, device=dev)

    def step(c):
        if with_router:
            native.moe_router_topk(x, router_w, k, True, bias=router_b,
                                   out=(ids, wts, off, pairs), workspace=rtws)
        elif route:
            native.moe_route_topk(logits, k, True, out=(ids, wts, off, pairs), workspace=rws)
        native.moe_grouped_nvfp4_ffn(x, wcopies[c], ids, wts, off, pairs, k, act=act,
                                     act_globals=ag, out_dtype=torch.bfloat16,
                                     workspace=ws, out=y)
        if with_shared:
            native.moe_shared_expert_ffn(x, *sh_w, y=y, accumulate=True, workspace=sh_ws)

    if not route:   # one expert: the routing is fixed (all rows to expert 0)
        native.moe_route_topk(logits, k, True, out=(ids, wts, off, pairs), workspace=rws)
    step(0)
    torch.cuda.synchronize()

    # ---- work accounting from the actual routing ---------------------------------
    counts = np.diff(off.cpu().numpy())
    active = int((counts > 0).sum())
    w_bytes_active = 3 * active * (nv_bytes(H * I) + 4)
    io_bytes = T * H * 2 * 2 + (T * E * 4 if route else 0)
    if with_router:   # the router matrix and a second read of x replace the logits
        io_bytes += E * H * 2 + T * H * 2 - T * E * 4
    alg_extra_flops = 2 * T * H * E if with_router else 0
    if with_shared:   # three bf16 [I, H] matrices, a read of x and a read-modify-write of y
        io_bytes += 3 * H * I * 2 + T * H * 2 * 2
        alg_extra_flops += 6 * T * H * I
    alg_bytes = w_bytes_active + io_bytes
    alg_flops = 6 * P * H * I + alg_extra_flops
    gateup_bytes = 2 * active * (nv_bytes(H * I) + 4) + T * H * 2
    gateup_flops = 4 * P * H * I
    if gate_up_kernel(T, H, I, E, k, wl.act) == "row_ffn_kernel":
        # the fused decode kernel streams the down matrices too
        gateup_bytes = 3 * active * (nv_bytes(H * I) + 4) + T * H * 2
        gateup_flops = 6 * P * H * I
    # MFMA-bound when the step's arithmetic intensity exceeds the ridge point
    prefill_mfma = alg_flops / alg_bytes > MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

    # ---- timed region: K steps (graph replays), HIP events on the stream -----------
    use_graph = not args.eager
    graphs = []        # one step each (per-step spread, remainders)
    pass_graph = None  # one step per weight copy, in order
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for c in range(copies):
                step(c)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        pass_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pass_graph):
            for c in range(copies):
                step(c)
        torch.cuda.synchronize()

    def run(i):
        c = i % copies
        if use_graph:
            graphs[c].replay()
        else:
            step(c)

    def run_steps(n):
        """n consecutive steps from step 0: whole passes over the copies as
        one graph each, the remainder one step at a time."""
        if not use_graph:
            for i in range(n):
                step(i % copies)
            return
        for _ in range(n // copies):
            pass_graph.replay()
        for i in range(n % copies):
            graphs[i].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    run_steps(args.steps)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3
    ms_per_step = start.elapsed_time(end) / args.steps

    # ---- per-step spread (events around each replay) and the FFN alone ----------
    n_spread = min(args.steps, 100)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_spread + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(n_spread):
        run(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_us = np.array([1e3 * evs[i].elapsed_time(evs[i + 1]) for i in range(n_spread)])
    ffn_ms = None
    if use_graph:   # routing precomputed: graphs of the FFN call alone
        def ffn_only(c):
            native.moe_grouped_nvfp4_ffn(x, wcopies[c], ids, wts, off, pairs, k, act=act,
                                         act_globals=ag, out_dtype=torch.bfloat16,
                                         workspace=ws, out=y)
        fgraphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                ffn_only(c)
            fgraphs.append(g)
        fpass = torch.cuda.CUDAGraph()
        with torch.cuda.graph(fpass):
            for c in range(copies):
                ffn_only(c)

        def run_ffn(n):   # as run_steps
            for _ in range(n // copies):
                fpass.replay()
            for i in range(n % copies):
                fgraphs[i].replay()
        run_ffn(args.warmup)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record()
        run_ffn(args.steps)
        f1.record()
        torch.cuda.synchronize()
        ffn_ms = f0.elapsed_time(f1) / args.steps

    # ---- stage timing: the library's stage events around each kernel ------------
    # Eager steps (events are not recorded inside graphs).  A GPU sleep kernel
    # first keeps the stream busy while the host enqueues every step, so the
    # steps then run back to back with no host-side gaps inside the events.
    nst = len(native.FFN_STAGES)
    reps = min(args.steps, 64)
    ev = HipEvents(2 * nst * reps)
    L = native.lib()
    stage_ms = {n: [] for n in native.FFN_STAGES}
    try:
        torch.cuda.synchronize()
        torch.cuda._sleep(400_000_000)
        for r in range(reps):
            base = ctypes.c_void_p(ctypes.addressof(ev.arr) +
                                   2 * nst * r * ctypes.sizeof(ctypes.c_void_p))
            L.nvfp4_set_ffn_stage_events(base)
            step(r % copies)
        L.nvfp4_set_ffn_stage_events(None)
        torch.cuda.synchronize()
        for r in range(reps):
            for si, n in enumerate(native.FFN_STAGES):
                b = 2 * nst * r + 2 * si
                stage_ms[n].append(ev.elapsed_ms(b, b + 1))
    finally:
        L.nvfp4_set_ffn_stage_events(None)
    stage_avg_us = {n: 1e3 * float(np.mean(v)) for n, v in stage_ms.items()}
    ev.close()

    gu_s = stage_avg_us["gate_up"] * 1e-6
    if prefill_mfma:
        value = alg_flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = gateup_flops / gu_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                    "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    else:
        value = alg_bytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = gateup_bytes / gu_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    kname = gate_up_kernel(T, H, I, E, k, wl.act)
    roofline["traffic"] = stored_traffic(kname, wl.name)
    roofline["kernel"] = kname + (" (gate/up, SiLU*up, down: both projections)"
                                  if kname == "row_ffn_kernel" else
                                  " (gate/up projection, SiLU*up epilogue)")
    roofline["kernel_avg_us"] = round(stage_avg_us["gate_up"], 3)
    roofline["alg_per_launch"] = int(gateup_flops if prefill_mfma else gateup_bytes)
    roofline["alg_units_per_launch"] = (f"{active} experts x 3 NVFP4 [{I},{H}] + x"
                                        if kname == "row_ffn_kernel" and not prefill_mfma else
                                        f"{active} experts x 2 NVFP4 [{I},{H}] + x"
                                        if not prefill_mfma else f"{P} pairs x 4*H*I flop")
    roofline["alg_bytes_per_launch"] = int(gateup_bytes)   # weights + x, for the traffic ratio

    if args.copy_calibration:
        copy_calibration()

    # ---- CPU oracle on a bounded sample (rank 0, N = 1) --------------------------
    cpu = None
    if not args.no_cpu_baseline:
        router = None
        if with_router:
            router = (router_w.float().cpu().numpy(),
                      None if router_b is None else router_b.cpu().numpy())
        shared = None
        if with_shared:
            shared = [t.float().cpu().numpy() for t in sh_w]
        cpu = cpu_baseline(args, wl, x_cpu, logits_np, y, counts, prefill_mfma, router, shared)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # the decode row kernels multiply bf16 weights by bf16 activations
        # (fp32 sums); the MFMA kernels multiply fp16 operands
        "dtype": "bf16" if kname.startswith("row_") else "f16", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "top_k": k, "act": wl.act,
                   "shared_expert": (f"bf16, intermediate {I}" if with_shared else None),
                   "router": ("bf16 router GEMM + top-k" if with_router else
                              "top-k of given logits" if route else None),
                   "act_globals": ("given (static)" if ag is not None else
                                   "online" if act == native.W4A4 else None),
                   "h_quant": ("separate pass" if args.separate_h_quant else "fused")
                              if ag is not None else None,
                   "zipf_s": wl.zipf_s, "active_experts": active,
                   "max_tokens_per_expert": int(counts.max()),
                   "weight_copies_cycled": copies, "graph": use_graph,
                   "steps_per_graph": copies if use_graph else None,
                   "parallelism": "single GPU"},
        "alg_bytes_per_step": int(alg_bytes), "alg_flops_per_step": int(alg_flops),
        "pct_of_peak": round(100 * (value / (MFMA_F16_PEAK_TFLOPS if prefill_mfma
                                             else HBM_PEAK_GBS)), 2),
        "stage_us": {n: round(v, 3) for n, v in stage_avg_us.items()},
        "stage_us_note": ("per-stage HIP events over an eager pass; a stage that runs no "
                          "kernel at this shape (it is folded into another) reads the ~4.4 us "
                          "of two back-to-back event packets, not work"),
        "wall_ms_timed_region": round(wall_ms, 3),
        "step_us_p10_p50_p90": [round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)],
        "ffn_only": None if ffn_ms is None else {
            "ms_per_step": round(ffn_ms, 5),
            "value": round((alg_flops / (ffn_ms * 1e-3) / 1e12) if prefill_mfma else
                           ((alg_bytes - (T * E * 4 if route else 0)) / (ffn_ms * 1e-3) / 1e9), 2),
            "unit": unit, "note": "routing precomputed (same routing as the steps)"},
        "setup_s": round(setup_s, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


HOST_LINK_PEAK_GBS = 63.0   # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)


def paged_main(args):
    """Expert paging on a routed-expert step: every expert's NVFP4 weights in
    pinned host memory, a device pool of S slots.  A step routes
    (moe_route_topk), plans the slots (moe_expert_cache_plan), copies the
    missing experts into the pool (moe_expert_cache_fetch), orders the pairs
    by slot (moe_permute_pairs) and runs the FFN on the pool.  The routing
    batches cycle over 64 seeded logits tensors of the workload's routing (or
    one with a Zipf router bias of the given exponent: skewed popularity).  Prints one JSON line: step
    throughput, hit rate, bytes fetched per step, the stages' times and the
    fetch kernel's rate against the host link; beside it the same steps with
    every expert resident in HBM."""
    import numpy as np
    import torch

    from nvfp4_routed_expert_amd import native, synth, weights

    wl = synth.WORKLOADS[args.workload]
    if wl.act != "w4a16" or wl.E < 2:
        sys.exit("--paged runs the W4A16 routed-expert workloads")
    dev = "cuda:0"
    torch.cuda.set_device(0)
    T, H, I, E, k, S = wl.T, wl.H, wl.I, wl.E, wl.k, args.paged
    P = T * k
    expert_bytes = 3 * (nv_bytes(H * I) + 4)
    n_batches = 64
    x = synth.activations(T, H).to(dev)
    zipf = wl.zipf_s if args.paged_zipf is None else args.paged_zipf
    logits = [torch.from_numpy(synth.router_logits(T, E, seed=b, zipf_s=zipf)).to(dev)
              for b in range(n_batches)]
    w_dev = weights.synthetic_experts(E, H, I, 0, dev)
    host = native.ExpertWeights(*[t.cpu().pin_memory() for t in (
        w_dev.gate_codes, w_dev.gate_scales, w_dev.gate_global, w_dev.up_codes, w_dev.up_scales,
        w_dev.up_global, w_dev.down_codes, w_dev.down_scales, w_dev.down_global)])
    cache = native.ExpertCache(host, S, dev)
    i32 = dict(dtype=torch.int32, device=dev)
    ids, slot_ids = torch.empty((T, k), **i32), torch.empty((T, k), **i32)
    wts = torch.empty((T, k), dtype=torch.float32, device=dev)
    off, pairs = torch.empty(E + 1, **i32), torch.empty(P, **i32)
    off_s, pairs_s = torch.empty(S + 1, **i32), torch.empty(P, **i32)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws_p = torch.empty(native.ffn_workspace_bytes(T, H, I, S, k), dtype=torch.uint8, device=dev)
    ws_r = torch.empty(native.ffn_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device=dev)
    rws = native.route_workspace(T, E, k, dev)
    stages = ["route", "plan", "fetch", "permute", "ffn"]

    def paged_step(b, ev=None):
        mark = (lambda j: ev[j].record()) if ev else (lambda j: None)
        mark(0)
        native.moe_route_topk(logits[b], k, True, out=(ids, wts, off, pairs), workspace=rws)
        mark(1)
        cache.plan(ids, slot_ids=slot_ids)
        mark(2)
        cache.fetch_planned(P)
        mark(3)
        native.moe_permute_pairs(slot_ids, S, out=(off_s, pairs_s))
        mark(4)
        native.moe_grouped_nvfp4_ffn(x, cache.pool, slot_ids, wts, off_s, pairs_s, k,
                                     out_dtype=torch.bfloat16, workspace=ws_p, out=y)
        mark(5)

    def resident_step(b):
        native.moe_route_topk(logits[b], k, True, out=(ids, wts, off, pairs), workspace=rws)
        native.moe_grouped_nvfp4_ffn(x, w_dev, ids, wts, off, pairs, k,
                                     out_dtype=torch.bfloat16, workspace=ws_r, out=y)

    def timed(fn, n):
        # a GPU sleep first keeps the stream busy while the host enqueues the
        # steps, so they run back to back (no host gaps inside the events)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(400_000_000)
        a.record()
        for i in range(n):
            fn(i % n_batches)
        z.record()
        torch.cuda.synchronize()
        return a.elapsed_time(z) / n

    # the pool warms up over the warmup steps, then K timed steps (eager
    # launches; a step's fetch dominates its time)
    for i in range(args.warmup):
        paged_step(i % n_batches)
    ms_paged = timed(lambda b: paged_step((b + args.warmup) % n_batches), args.steps)

    ms_overlap = None
    if args.paged_overlap:
        # Two streams.  Side stream: routing, slot plan (the previous step's
        # experts protected), fetch and pair order of step i; it first waits
        # for the FFN of step i-2, the last reader of the buffers it reuses
        # and of the experts it may evict.  Main stream: the FFN of step i
        # after its fetch.  So the fetch of step i runs beside the FFN of
        # step i-1.
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream()
        buf = [dict(ids=torch.empty((T, k), **i32), slot=torch.empty((T, k), **i32),
                    wts=torch.empty((T, k), dtype=torch.float32, device=dev),
                    off=torch.empty(E + 1, **i32), pairs=torch.empty(P, **i32),
                    off_s=torch.empty(S + 1, **i32), pairs_s=torch.empty(P, **i32))
               for _ in range(2)]
        rws2 = native.route_workspace(T, E, k, dev)

        nlog_o = torch.zeros(max(args.steps, args.warmup, 1), **i32)

        def pipeline(n, b0, start_ev):
            ffn_done = [None] * n
            side.wait_event(start_ev)
            for i in range(n):
                bb = buf[i % 2]
                with torch.cuda.stream(side):
                    if i >= 2:
                        side.wait_event(ffn_done[i - 2])
                    native.moe_route_topk(logits[(b0 + i) % n_batches], k, True,
                                          out=(bb["ids"], bb["wts"], bb["off"], bb["pairs"]),
                                          workspace=rws2)
                    cache.plan(bb["ids"], protect_previous=True, slot_ids=bb["slot"])
                    cache.fetch_planned(P)
                    native.moe_permute_pairs(bb["slot"], S, out=(bb["off_s"], bb["pairs_s"]))
                    fetched = torch.cuda.Event()
                    fetched.record(side)
                    nlog_o[i:i + 1].copy_(cache.n_fetch)
                main.wait_event(fetched)
                native.moe_grouped_nvfp4_ffn(x, cache.pool, bb["slot"], bb["wts"], bb["off_s"],
                                             bb["pairs_s"], k, out_dtype=torch.bfloat16,
                                             workspace=ws_p, out=y)
                ffn_done[i] = torch.cuda.Event()
                ffn_done[i].record(main)
            main.wait_stream(side)

        w0 = torch.cuda.Event()
        w0.record(main)
        pipeline(args.warmup, 0, w0)
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(400_000_000)
        a.record(main)
        pipeline(args.steps, args.warmup, a)
        z.record(main)
        torch.cuda.synchronize()
        if int(nlog_o[:args.steps].min().item()) < 0:
            sys.exit(f"--paged {S} --paged-overlap: two steps' experts did not fit in the pool")
        ms_overlap = a.elapsed_time(z) / args.steps
    for i in range(min(args.warmup, 8)):
        resident_step(i % n_batches)
    ms_res = timed(resident_step, args.steps)

    # stage times and fetch counts: one more pass, events around each call
    n_stat = min(args.steps, n_batches)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n_stat)]
    nlog = torch.empty(n_stat, **i32)
    dlog = torch.empty((n_stat, T, k), **i32)
    torch.cuda.synchronize()
    torch.cuda._sleep(400_000_000)
    for i in range(n_stat):
        paged_step((i + args.warmup + args.steps) % n_batches, evs[i])
        nlog[i:i + 1].copy_(cache.n_fetch)
        dlog[i].copy_(ids)
    torch.cuda.synchronize()
    st = {s: [evs[i][j].elapsed_time(evs[i][j + 1]) * 1e3 for i in range(n_stat)]
          for j, s in enumerate(stages)}
    nf = nlog.cpu().numpy()
    if (nf < 0).any():
        sys.exit(f"--paged {S}: a step's experts did not fit in the pool")
    distinct = np.array([len(np.unique(d)) for d in dlog.cpu().numpy()])
    fetched = int(nf.sum())
    fetch_us = np.array(st["fetch"])
    busy = nf > 0
    fetch_gbs = (float(nf[busy].sum()) * expert_bytes / (fetch_us[busy].sum() * 1e-6) / 1e9
                 if busy.any() else None)

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on a sample of routing batch 0: its slot plan from an
        # empty pool and the FFN rows of the sampled tokens; the paged output
        # of the same batch is checked against it
        paged_step(0)
        torch.cuda.synchronize()
        cpu = paged_cpu_baseline(args, wl, S, zipf, y)
    out = {
        "metric": "NVFP4 MoE FFN with expert paging: tokens/s",
        "value": round(T / (ms_paged * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_paged, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if gate_up_kernel(T, H, I, S, k, wl.act).startswith("row_") else "f16",
        "data": "synthetic",
        "config": {"workload": wl.name + "_paged", "tokens": T, "hidden": H,
                   "intermediate": I, "experts": E, "top_k": k, "slots": S,
                   "router_bias_zipf_s": zipf, "routing_batches": n_batches,
                   "host_weights_gb": round(E * expert_bytes / 1e9, 3),
                   "pool_gb": round(S * expert_bytes / 1e9, 3), "graph": False,
                   "parallelism": "single GPU"},
        "hit_rate": round(1.0 - fetched / float(distinct.sum()), 4),
        "experts_per_step": round(float(distinct.mean()), 2),
        "fetched_per_step": round(float(nf.mean()), 2),
        "fetched_mb_per_step": round(float(nf.mean()) * expert_bytes / 1e6, 3),
        "stage_us": {s: round(float(np.mean(v)), 2) for s, v in st.items()},
        "resident_ms_per_step": round(ms_res, 5),
        "overlapped_ms_per_step": None if ms_overlap is None else round(ms_overlap, 5),
        "roofline": {"bound": "host_link", "kernel": "cache_fetch_kernel",
                     "achieved": None if fetch_gbs is None else round(fetch_gbs, 2),
                     "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": None if fetch_gbs is None else round(fetch_gbs / HOST_LINK_PEAK_GBS, 4),
                     "traffic": None,
                     "alg_per_unit": f"{expert_bytes} bytes per fetched expert"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def paged_cpu_baseline(args, wl, S, zipf, y_gpu):
    """The oracle (as it stands) on a bounded sample of a paged step: the slot
    plan of routing batch 0 and the FFN rows of a token sample, timed on the
    host; tokens/s.  Also the correctness gate for those rows."""
    import numpy as np
    import threadpoolctl

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import LazyOracleExperts
    from oracle import nvfp4_oracle as O
    from nvfp4_routed_expert_amd import synth

    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    n_tok = args.cpu_tokens or min(T, 16)
    tokens = list(range(0, T, max(1, T // n_tok)))[:n_tok]
    xf = synth.activations(T, H).float().numpy()
    logits = synth.router_logits(T, E, seed=0, zipf_s=zipf)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    rids, rw = O.route_topk(logits, k)
    w_ref = LazyOracleExperts(E, H, I, np.unique(rids[tokens]), 0)   # offline quantisation
    t0 = time.perf_counter()
    O.expert_slot_plan(O.SlotState(E, S), rids, 1, 1)
    ref, _ = O.moe_ffn(xf, rids, rw, w_ref, tokens=tokens)
    dt = time.perf_counter() - t0
    got = y_gpu.float().cpu().numpy()[tokens].astype(np.float64)
    r = O.bf16_rne(ref)
    return {"kind": "oracle", "cores": int(threads), "value": round(len(tokens) / dt, 3),
            "unit": "tokens/s",
            "sample": f"slot plan of one routing batch and the FFN of {len(tokens)} of {T} "
                      f"tokens, fp64 numpy oracle, {dt:.2f} s",
            "seconds": round(dt, 3),
            "gate_rel_frob_vs_oracle": float(np.linalg.norm(got - r) / np.linalg.norm(r))}


def copy_calibration():
    """A plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB), run a few
    times; under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the scale
    from counter units to bytes."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()


def cpu_baseline(args, wl, x_cpu, logits_np, y_gpu, counts, mfma_bound, router=None,
                 shared=None):
    """Time the oracle (as it stands) on a bounded sample of the same step and
    use it as the correctness gate for the GPU output rows it covers.
    router = (R, bias): the step starts from the router, whose logits the
    oracle computes too (for the sampled tokens, inside the timed region);
    shared = (Wg, Wu, Wd): the BF16 shared expert is added as well."""
    import numpy as np
    import threadpoolctl

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import LazyOracleExperts
    from oracle import nvfp4_oracle as O

    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    n_tok = args.cpu_tokens or {"moe_decode": 16, "moe_prefill": 8,
                                "moe_prefill_w4a4": 1}.get(wl.name, 1)
    tokens = list(range(0, T, max(1, T // n_tok)))[:n_tok]
    xf = x_cpu.float().numpy()
    if router is not None:
        logits_np = O.router_logits(xf, *router)
    rids, rw = O.route_topk(logits_np, k)
    need = np.unique(rids[tokens])
    w_ref = LazyOracleExperts(E, H, I, need, 0)        # weight quantisation is offline
    a4 = wl.act == "w4a4"
    act_globals = None
    if a4:
        # the online h scale needs every pair; the sample uses the GPU run's
        # x scale (recomputed by the oracle) and a static h scale instead
        act_globals = (O.tensor_global(xf), np.float32(0.05 / 2688))
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    if router is not None:
        sl = O.router_logits(xf[tokens], *router)
        rids[tokens], rw[tokens] = O.route_topk(sl, k)
    ref, _ = O.moe_ffn(xf, rids, rw, w_ref, act_quant=a4, act_globals=act_globals,
                       tokens=tokens)
    if shared is not None:
        ref = O.shared_expert(xf[tokens], *shared, y_in=ref)
    dt = time.perf_counter() - t0
    sample_bytes = 3 * len(need) * (nv_bytes(H * I) + 4) + len(tokens) * H * 4
    sample_flops = 6 * len(tokens) * k * H * I
    if router is not None:
        sample_bytes += E * H * 2
        sample_flops += 2 * len(tokens) * H * E
    if shared is not None:
        sample_bytes += 3 * H * I * 2
        sample_flops += 6 * len(tokens) * H * I
    res = {"kind": "oracle", "cores": int(threads),
           "sample": f"{len(tokens)} of {T} tokens ({len(need)} experts), "
                     f"fp64 numpy oracle, {dt:.2f} s",
           "seconds": round(dt, 3)}
    if mfma_bound:
        res.update(value=round(sample_flops / dt / 1e12, 6), unit="TFLOP/s")
    else:
        res.update(value=round(sample_bytes / dt / 1e9, 4), unit="GB/s")
    if not a4:
        got = y_gpu.float().cpu().numpy()[tokens].astype(np.float64)
        r = O.bf16_rne(ref)
        res["gate_rel_frob_vs_oracle"] = float(np.linalg.norm(got - r) / np.linalg.norm(r))
    return res


if __name__ == "__main__":
    main()
