"""Benchmark of the NVFP4 routed-expert FFN hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
top-k routing + permutation (moe_route_topk), then the grouped FFN
(moe_grouped_nvfp4_ffn: plan, activation prep, gate/up GEMM with SiLU*up,
h prep, down GEMM times routing weight, combine).  Inputs are resident in HBM
before timing starts.  Steps cycle over copies of the expert weights, enough
that a copy's active experts are read again only after >= 1 GiB of other
HBM traffic, so every step streams its weights from HBM rather than from the
256 MB Infinity Cache (MALL).  The timed steps run as HIP graph replays; one
graph holds a pass over all the copies (several consecutive steps, as a
model's layers share one graph); the timed region covers exactly K steps,
with an event after each pass (the per-step percentiles).

Before any timing each workload passes a correctness gate against the fp64
oracle on a sample of its tokens; a failed gate ends the run with exit
status 3.  The default run prints one JSON line: the routed decode step
(the headline), and under "workloads" the 512-token prefill chunk (normal
and Gumbel router noise) and the W4A4 prefill, each with its roofline
figures, gate and the CPU oracle's throughput on the sample.
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
    ap.add_argument("--workload", default=None,
                    help="one workload alone: moe_decode | moe_prefill | moe_prefill_w4a4 | "
                         "mlp_decode_m{1,8,32} | mlp_prefill_m{512,2048} (default: moe_decode "
                         "as the headline, with moe_prefill, its Gumbel variant and "
                         "moe_prefill_w4a4 in the same line)")
    ap.add_argument("--single", action="store_true",
                    help="the headline workload only (no side workloads)")
    ap.add_argument("--gumbel", action="store_true",
                    help="Gumbel router noise instead of N(0,1) (the second reading of the "
                         "chunk's Zipf bias)")
    ap.add_argument("--copies", type=int, default=0,
                    help="weight copies cycled per step (0 = enough that a copy is read "
                         "again only after >= 1 GiB of other traffic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens in the oracle sample (0 = workload default)")
    ap.add_argument("--eager", action="store_true", help="no graph capture")
    ap.add_argument("--fused-routing", action="store_true",
                    help="decode: route inside the FFN launch (moe_route_ffn_decode) instead "
                         "of in a launch of its own (moe_route_topk)")
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
    "row_ffn_kernel": ["rowgemv.hip", "topk.h", "common.h", "kernels.h"],
    "row_gemv_kernel": ["rowgemv.hip", "topk.h", "common.h", "kernels.h"],
    "row_mlp_gate_up_kernel": ["rowgemv.hip", "topk.h", "common.h", "kernels.h"],
    "tile_gemm_kernel": ["tile_gemm.hip", "common.h", "kernels.h"],
    "dense_gemv_kernel": ["densegemv.hip", "common.h", "kernels.h"],
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
    if E == 1 and not small and P <= 32 and H % 256 == 0 and I % 256 == 0:
        return "dense_gemv_kernel"   # a dense MLP with a few rows: one shared weight stream
    if small:
        if act == "w4a16" and row_ok(H) and row_ok(I):
            if (E == 1 and P == 1 and H % 1024 == 0 and H <= 5120 and I % 32 == 0
                    and (I // 16 + 255) // 256 <= 8 and 2 * I + 2048 <= 65536):
                return "row_mlp_gate_up_kernel"   # one dense row: gate/up rows dealt out evenly
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


# The default run: the routed decode step is the headline line (the metric's
# decode figure); the 512-token chunk (normal and Gumbel readings of its Zipf
# router bias) and the W4A4 prefill (the metric's prefill figure) ride in the
# same JSON line under "workloads".
DEFAULT_SIDE = [("moe_prefill", False), ("moe_prefill", True), ("moe_prefill_w4a4", False)]
SIDE_STEPS = {"moe_prefill": 200, "moe_prefill_w4a4": 50}
COLD_GAP_BYTES = 1 << 30     # other HBM traffic between two reads of one weight copy


def host_cpu_info():
    """Host cores the oracle may use: os.cpu_count(), the affinity mask and the
    BLAS thread count."""
    import threadpoolctl
    info = threadpoolctl.threadpool_info()
    blas = max([i.get("num_threads", 1) for i in info] or [1])
    return {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": int(blas)}


class GateFailure(RuntimeError):
    pass


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

    import torch
    torch.cuda.set_device(0)
    name = args.workload or "moe_decode"
    failed = []
    try:
        t_w = time.perf_counter()
        out = measure(args, name, gumbel=args.gumbel, steps=args.steps, warmup=args.warmup)
        print(f"bench: {name} measured in {time.perf_counter() - t_w:.1f} s", file=sys.stderr,
              flush=True)
    except GateFailure as e:
        print(json.dumps({"error": f"correctness gate failed before timing: {e}"}), flush=True)
        sys.exit(3)
    if out["gate"] and not out["gate"]["passed"]:
        failed.append(name)
    if args.workload is None and not args.single:
        out["workloads"] = {}
        for wname, gumbel in DEFAULT_SIDE:
            key = wname + ("_gumbel" if gumbel else "")
            steps = min(args.steps, SIDE_STEPS[wname])
            warm = min(args.warmup, 10)
            try:
                t_w = time.perf_counter()
                sub = measure(args, wname, gumbel=gumbel, steps=steps, warmup=warm)
                print(f"bench: {key} measured in {time.perf_counter() - t_w:.1f} s",
                      file=sys.stderr, flush=True)
            except GateFailure as e:
                sub = {"error": f"correctness gate failed before timing: {e}"}
                failed.append(key)
            else:
                if sub["gate"] and not sub["gate"]["passed"]:
                    failed.append(key)
            for drop in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline",
                         "data", "steps_note"):
                sub.pop(drop, None)
            out["workloads"][key] = sub
            torch.cuda.empty_cache()
    out["host_cpu"] = host_cpu_info()
    if failed:
        out["gates_failed"] = failed
    print(json.dumps(out), flush=True)
    if failed:
        sys.exit(3)


def _replay_passes(pass_graph, step_graphs, copies, n, evs=None):
    """n consecutive steps from copy 0: whole passes over the copies as one
    graph each (an event after each pass when evs is given), the remainder
    one step at a time."""
    for q in range(n // copies):
        pass_graph.replay()
        if evs is not None:
            evs[q + 1].record()
    for i in range(n % copies):
        step_graphs[i].replay()


def measure(args, name, gumbel=False, steps=200, warmup=20):
    """One workload: the correctness gate (before any timing), then K timed
    steps as graph replays cycling over weight copies (cold HBM), the FFN
    alone, warm back-to-back steps, the dominant kernel's own time (HIP
    events on its dispatch) and the oracle on a bounded sample.  Returns the
    workload's JSON object; raises GateFailure when the gate fails."""
    import numpy as np
    import torch

    from nvfp4_routed_expert_amd import native, synth, weights

    wl = synth.WORKLOADS[name]
    dev = "cuda:0"
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    act = native.W4A4 if wl.act == "w4a4" else native.W4A16
    P = T * k
    route = E > 1

    # ---- inputs (seeded synthetic, resident in HBM) -----------------------------
    x_cpu = synth.activations(T, H)
    logits_np = synth.router_logits(T, E, zipf_s=wl.zipf_s, gumbel=gumbel)
    x = x_cpu.to(dev)
    logits = torch.from_numpy(logits_np).to(dev)
    t0 = time.time()
    w0 = weights.synthetic_experts(E, H, I, 0, dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

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
    ag_out = torch.empty(2, dtype=torch.float32, device=dev) if act == native.W4A4 else None
    native.set_ffn_separate_h_quant(args.separate_h_quant)
    rws = native.route_workspace(T, E, k, dev)
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

    def ffn(wset, out=y, ws_=ws):
        if act == native.W4A4 and ag is None:   # online globals into a fixed buffer
            _ffn_online(native, x, wset, ids, wts, off, pairs, k, out, ws_, ag_out)
        else:
            native.moe_grouped_nvfp4_ffn(x, wset, ids, wts, off, pairs, k, act=act,
                                         act_globals=ag, out_dtype=out.dtype, workspace=ws_,
                                         out=out)

    # --fused-routing on the fused decode kernel: the routing runs inside the
    # FFN launch (each workgroup takes its token's top-k) and the permutation
    # beside the combine.
    fused_route = (route and not with_router and act == native.W4A16 and
                   args.fused_routing and native.route_ffn_decode_supported(T, H, I, E, k))
    if fused_route:
        fws = torch.empty(native.lib().moe_route_ffn_decode_workspace_size(T, H, I, E, k),
                          dtype=torch.uint8, device=dev)

    def step(wset):
        if with_router:
            native.moe_router_topk(x, router_w, k, True, bias=router_b,
                                   out=(ids, wts, off, pairs), workspace=rtws)
            ffn(wset)
        elif fused_route:
            native.moe_route_ffn_decode(logits, x, wset, k, True, route_out=(ids, wts, off, pairs),
                                        out=y, workspace=fws)
        else:
            if route:
                native.moe_route_topk(logits, k, True, out=(ids, wts, off, pairs), workspace=rws)
            ffn(wset)
        if with_shared:
            native.moe_shared_expert_ffn(x, *sh_w, y=y, accumulate=True, workspace=sh_ws)

    if not route:   # one expert: the routing is fixed (all rows to expert 0)
        native.moe_route_topk(logits, k, True, out=(ids, wts, off, pairs), workspace=rws)
    step(w0)
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
    kname = gate_up_kernel(T, H, I, E, k, wl.act)
    gateup_bytes = 2 * active * (nv_bytes(H * I) + 4) + T * H * 2
    gateup_flops = 4 * P * H * I
    if kname == "row_ffn_kernel":   # the fused decode kernel streams the down matrices too
        gateup_bytes = 3 * active * (nv_bytes(H * I) + 4) + T * H * 2
        if fused_route:   # ... and reads the logits of the tokens it routes
            gateup_bytes += T * E * 4
        gateup_flops = 6 * P * H * I
    # MFMA-bound when the step's arithmetic intensity exceeds the ridge point
    prefill_mfma = alg_flops / alg_bytes > MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

    # ---- correctness gate, before any timing --------------------------------------
    gate = None
    if not args.no_cpu_baseline:
        gate, cpu = oracle_leg(args, wl, gumbel, x, x_cpu, logits_np, ids, wts, off, pairs, w0,
                               act, ag, counts, prefill_mfma, with_router, with_shared,
                               router_w if with_router else None,
                               router_b if with_router else None,
                               sh_w if with_shared else None)
        if not gate["passed"]:
            raise GateFailure(f"{name}{' (gumbel)' if gumbel else ''}: {gate}")
    else:
        cpu = None

    # ---- weight copies: each copy's active weights are read again only after
    # >= 1 GiB of other HBM traffic (the 256 MB MALL and the L2s are cold) ----
    bytes_all = 3 * E * (nv_bytes(H * I) + 4)
    per_step = w_bytes_active + io_bytes
    copies = args.copies or max(2, 1 + int(np.ceil(COLD_GAP_BYTES / per_step)))
    copies = min(copies, max(2, int((64 << 30) // bytes_all)), 16)
    wcopies = [w0]
    for _ in range(copies - 1):
        wcopies.append(native.ExpertWeights(*[t.clone() for t in (
            w0.gate_codes, w0.gate_scales, w0.gate_global, w0.up_codes, w0.up_scales,
            w0.up_global, w0.down_codes, w0.down_scales, w0.down_global)]))

    # ---- graphs: one step per copy, and one pass over all the copies ---------------
    use_graph = not args.eager

    def capture(fn_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn_steps()
        return g

    s_side = torch.cuda.Stream()
    s_side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_side):
        for c in range(copies):
            step(wcopies[c])
    torch.cuda.current_stream().wait_stream(s_side)
    torch.cuda.synchronize()
    if use_graph:
        graphs = [capture(lambda c=c: step(wcopies[c])) for c in range(copies)]
        pass_graph = capture(lambda: [step(wcopies[c]) for c in range(copies)])
        fgraphs = [capture(lambda c=c: ffn(wcopies[c])) for c in range(copies)]
        fpass = capture(lambda: [ffn(wcopies[c]) for c in range(copies)])
        warm_pass = capture(lambda: [step(w0) for _ in range(copies)])
        torch.cuda.synchronize()

    def run(n, evs=None, pg=None, sg=None):
        if not use_graph:
            for i in range(n):
                step(wcopies[i % copies])
                if evs is not None and (i + 1) % copies == 0:
                    evs[(i + 1) // copies].record()
            return
        _replay_passes(pg or pass_graph, sg or graphs, copies, n, evs)

    # ---- timed region: K steps, an event after each whole pass --------------------
    run(warmup)
    torch.cuda.synchronize()
    n_pass = steps // copies
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_pass + 1)]
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record()
    run(steps, evs)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3
    ms_per_step = evs[0].elapsed_time(end) / steps
    pass_step_us = np.array([1e3 * evs[q].elapsed_time(evs[q + 1]) / copies
                             for q in range(n_pass)]) if n_pass else np.array([ms_per_step * 1e3])

    # ---- the FFN alone (routing precomputed) and warm back-to-back steps ---------
    ffn_ms = warm_ms = None
    if use_graph:
        run(warmup, pg=fpass, sg=fgraphs)
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record()
        run(steps, pg=fpass, sg=fgraphs)
        f1.record()
        torch.cuda.synchronize()
        ffn_ms = f0.elapsed_time(f1) / steps
        nw = max(copies, (steps // copies) * copies)
        for _ in range(2):
            warm_pass.replay()
        f0.record()
        for _ in range(nw // copies):
            warm_pass.replay()
        f1.record()
        torch.cuda.synchronize()
        warm_ms = f0.elapsed_time(f1) / nw

    # ---- stage timing: the library's stage events on each kernel's dispatch -------
    # Eager steps (events are not recorded inside graphs), cycling the copies.
    # A GPU sleep first keeps the stream busy while the host enqueues every
    # step, so the steps then run back to back with no host-side gaps.
    nst = len(native.FFN_STAGES)
    reps = min(steps, 64)
    ev = HipEvents(2 * nst * reps)
    L = native.lib()
    stage_ms = {n_: [] for n_ in native.FFN_STAGES}
    try:
        torch.cuda.synchronize()
        torch.cuda._sleep(400_000_000)
        for r in range(reps):
            base = ctypes.c_void_p(ctypes.addressof(ev.arr) +
                                   2 * nst * r * ctypes.sizeof(ctypes.c_void_p))
            L.nvfp4_set_ffn_stage_events(base)
            step(wcopies[r % copies])
        L.nvfp4_set_ffn_stage_events(None)
        torch.cuda.synchronize()
        for r in range(reps):
            for si, n_ in enumerate(native.FFN_STAGES):
                b_ = 2 * nst * r + 2 * si
                stage_ms[n_].append(ev.elapsed_ms(b_, b_ + 1))
    finally:
        L.nvfp4_set_ffn_stage_events(None)
    stage_avg_us = {n_: 1e3 * float(np.mean(v)) for n_, v in stage_ms.items()}
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
    wname = wl.name + ("_gumbel" if gumbel else "")
    roofline["traffic"] = stored_traffic(kname, wname)
    roofline["kernel"] = kname + (" (routing top-k, gate/up, SiLU*up, down)"
                                  if kname == "row_ffn_kernel" and fused_route else
                                  " (gate/up, SiLU*up, down: both projections)"
                                  if kname == "row_ffn_kernel" else
                                  " (gate/up projection, SiLU*up epilogue)")
    roofline["kernel_avg_us"] = round(stage_avg_us["gate_up"], 3)
    roofline["alg_per_launch"] = int(gateup_flops if prefill_mfma else gateup_bytes)
    roofline["alg_units_per_launch"] = (f"{active} experts x 3 NVFP4 [{I},{H}] + x + logits"
                                        if kname == "row_ffn_kernel" and fused_route else
                                        f"{active} experts x 3 NVFP4 [{I},{H}] + x"
                                        if kname == "row_ffn_kernel" and not prefill_mfma else
                                        f"{active} experts x 2 NVFP4 [{I},{H}] + x"
                                        if not prefill_mfma else f"{P} pairs x 4*H*I flop")
    roofline["alg_bytes_per_launch"] = int(gateup_bytes)   # weights + x, for the traffic ratio

    if args.copy_calibration:
        copy_calibration()

    def rate(ms):
        if prefill_mfma:
            return alg_flops / (ms * 1e-3) / 1e12
        return alg_bytes / (ms * 1e-3) / 1e9

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        # the decode row kernels and the dense MLP's GEMV multiply bf16 weights
        # by bf16 activations (fp32 sums); the other MFMA kernels fp16 operands
        "dtype": "bf16" if kname.startswith("row_") or (kname == "dense_gemv_kernel"
                                                        and wl.act == "w4a16") else "f16",
        "data": "synthetic",
        "config": {"workload": wname, "tokens": T, "hidden": H, "intermediate": I,
                   "experts": E, "top_k": k, "act": wl.act,
                   "router_logits": ("N(0,1)" if not gumbel else "Gumbel") +
                                    (f" + Zipf({wl.zipf_s}) bias" if wl.zipf_s else ""),
                   "shared_expert": (f"bf16, intermediate {I}" if with_shared else None),
                   "router": ("bf16 router GEMM + top-k" if with_router else
                              "top-k of given logits" if route else None),
                   "routing": ("inside the FFN launch (each workgroup takes its token's top-k; "
                               "the permutation beside the combine)" if fused_route else
                               "own launch" if route else None),
                   "act_globals": ("given (static)" if ag is not None else
                                   "online" if act == native.W4A4 else None),
                   "h_quant": ("separate pass" if args.separate_h_quant else "fused")
                              if ag is not None else None,
                   "active_experts": active, "max_tokens_per_expert": int(counts.max()),
                   "weight_copies_cycled": copies,
                   "other_traffic_between_reads_of_a_copy_bytes": int((copies - 1) * per_step),
                   "graph": use_graph, "steps_per_graph": copies if use_graph else None,
                   "parallelism": "single GPU"},
        "alg_bytes_per_step": int(alg_bytes), "alg_flops_per_step": int(alg_flops),
        "pct_of_peak": round(100 * (value / (MFMA_F16_PEAK_TFLOPS if prefill_mfma
                                             else HBM_PEAK_GBS)), 2),
        "stage_us": {n_: round(v, 3) for n_, v in stage_avg_us.items()},
        "stage_us_note": ("per-stage HIP events over an eager pass; a stage that runs no "
                          "kernel at this shape (it is folded into another) reads the cost of "
                          "two back-to-back event packets, not work"),
        "wall_ms_timed_region": round(wall_ms, 3),
        "step_us_p10_p50_p90": [round(float(np.percentile(pass_step_us, q)), 2)
                                for q in (10, 50, 90)],
        "step_us_note": (f"per-step time of each timed pass replay ({copies} steps per pass)"),
        "ffn_only": None if ffn_ms is None else {
            "ms_per_step": round(ffn_ms, 5),
            "value": round((alg_flops / (ffn_ms * 1e-3) / 1e12) if prefill_mfma else
                           ((alg_bytes - (T * E * 4 if route else 0)) / (ffn_ms * 1e-3) / 1e9),
                           2),
            "unit": unit, "note": "routing precomputed (same routing as the steps)"},
        "warm": None if warm_ms is None else {
            "ms_per_step": round(warm_ms, 5), "value": round(rate(warm_ms), 2), "unit": unit,
            "note": "warm: back-to-back steps on one weight copy (MALL/L2 may serve weights); "
                    "not the graded figure"},
        "setup_s": round(setup_s, 1),
        "roofline": roofline,
        "gate": gate,
        "cpu_baseline": cpu,
    }
    if name == "moe_decode" and not gumbel:
        out["read_ceiling"] = read_ceiling(per_step)
    del wcopies
    if use_graph:
        del graphs, pass_graph, fgraphs, fpass, warm_pass
    return out


def _ffn_online(native, x, wset, ids, wts, off, pairs, k, out, ws_, g_out):
    """W4A4 with online globals written into a fixed device buffer (so a graph
    replays the same call)."""
    import torch
    T, H = x.shape
    L = native.lib()
    cw = wset.c_struct()
    native._check(L.moe_grouped_nvfp4_ffn(
        native._ptr(x), T, H, wset.intermediate, wset.num_experts, k, native._ptr(ids),
        native._ptr(wts), native._ptr(off), native._ptr(pairs), ctypes.byref(cw), native.W4A4,
        native.GLOBAL_COMPUTE, native._ptr(g_out), native._ptr(out), native._dt(out.dtype),
        native._ptr(ws_), ws_.numel(), native._stream()))
    return out


def read_ceiling(step_bytes):
    """A plain streaming-read kernel (nvfp4_read_probe: 16-byte non-temporal
    loads) on the same GPU, over 1 GiB and over one decode step's size: the
    practical HBM read ceiling beside the 8 TB/s peak.  Fresh buffers are
    cycled through >= 2 GiB so each read is cold."""
    import torch

    from nvfp4_routed_expert_amd import native
    res = {}
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda:0")
    for label, nbytes in (("1GiB", 1 << 30), ("step_size", int(step_bytes) // 16 * 16)):
        nb = min(24, max(3, -(-2 * (1 << 30) // nbytes) + 1))
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0") for _ in range(nb)]
        for b_ in bufs[:2]:
            native.read_probe(b_, sink)
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3 * nb
        a.record()
        for r in range(reps):
            native.read_probe(bufs[r % nb], sink)
        z.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(z) / reps
        res[label] = {"bytes": nbytes, "us": round(ms * 1e3, 2),
                      "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        del bufs
    res["note"] = ("nvfp4_read_probe (plain streaming read, eager launches back to back, "
                   "each buffer cold): the practical read ceiling at each launch size; the "
                   "peak stays 8 TB/s")
    return res


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

    wl = synth.WORKLOADS[args.workload or "moe_decode"]
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
        if not cpu["gate_rel_frob_vs_oracle"] <= 1e-3:
            print(json.dumps({"error": "correctness gate failed", "cpu_baseline": cpu}),
                  flush=True)
            sys.exit(3)
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


def oracle_leg(args, wl, gumbel, x, x_cpu, logits_np, ids, wts, off, pairs, w0, act, ag,
               counts, mfma_bound, with_router, with_shared, router_w, router_b, sh_w):
    """The correctness gate and the CPU baseline of one workload, before any
    timing.  The GPU runs the step once more with an fp32 output (and a
    workspace of its own, whose h the W4A4 gate reads); the oracle (as it
    stands) is timed on a bounded sample of tokens (cpu_baseline), and the
    sampled output rows must meet the tolerance:
      * routing ids, offsets and pairs bit-exact with the oracle's;
      * W4A16: fp32 rows within rel-Frob 1e-3 and max-abs 1e-2 RMS of the fp64
        oracle; bf16 rows the rounding of the fp32 rows;
      * W4A4: g_x bit-exact; the device's h a valid rounding of the fp64 h,
        its NVFP4 codes and g_h exact for it, and the fp32 rows within the
        same tolerance of the oracle computed downstream from it.
    Returns (gate dict, cpu_baseline dict)."""
    import numpy as np
    import torch

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import (LazyOracleExperts, check_device_h, max_abs_over_rms, rel_frob,
                         rows_by_pair, spread_tokens)
    from oracle import nvfp4_oracle as O
    from nvfp4_routed_expert_amd import native

    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    a4 = wl.act == "w4a4"
    xf = x_cpu.float().numpy()
    if with_router:
        logits_np = O.router_logits(xf, router_w.float().cpu().numpy(),
                                    None if router_b is None else router_b.cpu().numpy())
    rids, rw = O.route_topk(logits_np, k)
    # (bounded samples: the oracle then runs for a few seconds per workload;
    # the gate checks the same tokens)
    n_tok = args.cpu_tokens or {"moe_decode": T, "moe_prefill": 128,
                                "moe_prefill_w4a4": 4}.get(wl.name, min(T, 4))
    tokens = list(range(T)) if n_tok >= T else spread_tokens(rids, n_tok)
    need = np.unique(rids[tokens])
    w_ref = LazyOracleExperts(E, H, I, need, 0, 16)        # weight quantisation is offline

    # the GPU step once more, fp32 and bf16 outputs, own workspace
    dev = x.device
    ws_g = torch.empty(native.ffn_workspace_bytes(T, H, I, E, k, act), dtype=torch.uint8,
                       device=dev)
    y32, g_out = native.moe_grouped_nvfp4_ffn(x, w0, ids, wts, off, pairs, k, act=act,
                                              act_globals=ag, out_dtype=torch.float32,
                                              workspace=ws_g)
    yb, _ = native.moe_grouped_nvfp4_ffn(x, w0, ids, wts, off, pairs, k, act=act,
                                         act_globals=ag, out_dtype=torch.bfloat16)
    if with_shared:
        native.moe_shared_expert_ffn(x, *sh_w, y=y32, accumulate=True)
    torch.cuda.synchronize()
    g32 = y32.cpu().numpy()
    gb = yb.float().cpu().numpy()

    act_globals = None
    if a4:
        g = g_out.cpu().numpy()
        act_globals = (g[0], g[1])

    info = host_cpu_info()
    t0 = time.perf_counter()
    if with_router:
        O.router_logits(xf[tokens], router_w.float().cpu().numpy(),
                        None if router_b is None else router_b.cpu().numpy())
    ref, _ = O.moe_ffn(xf, rids, rw, w_ref, act_quant=a4, act_globals=act_globals,
                       tokens=tokens)
    if with_shared:
        ref = O.shared_expert(xf[tokens], *[t.float().cpu().numpy() for t in sh_w], y_in=ref)
    dt = time.perf_counter() - t0
    sample_bytes = 3 * len(need) * (nv_bytes(H * I) + 4) + len(tokens) * H * 4
    sample_flops = 6 * len(tokens) * k * H * I
    if with_router:
        sample_bytes += E * H * 2
        sample_flops += 2 * len(tokens) * H * E
    if with_shared:
        sample_bytes += 3 * H * I * 2
        sample_flops += 6 * len(tokens) * H * I
    cpu = {"kind": "oracle", "cores": info["blas_threads"],
           "sample": f"{len(tokens)} of {T} tokens ({len(need)} experts), fp64 numpy oracle, "
                     f"{dt:.2f} s" + (" (W4A4: the run's activation scales given)" if a4 else ""),
           "seconds": round(dt, 3), "host_cpu": info}
    if mfma_bound:
        cpu.update(value=round(sample_flops / dt / 1e12, 6), unit="TFLOP/s")
    else:
        cpu.update(value=round(sample_bytes / dt / 1e9, 4), unit="GB/s")

    # ---- the gate --------------------------------------------------------------
    gate = {"tokens": len(tokens), "passed": True}
    routing_ok = True
    if E > 1 and not with_router:
        roff, rpairs = O.permute(rids, E)
        routing_ok = (np.array_equal(ids.cpu().numpy(), rids) and
                      np.array_equal(off.cpu().numpy(), roff) and
                      np.array_equal(pairs.cpu().numpy(), rpairs))
        gate["routing_bit_exact"] = routing_ok
    got = g32[tokens].astype(np.float64)
    try:
        if a4:
            hb, hq = native.ffn_debug_h(ws_g, T, H, I, E, k, act, given=ag is not None)
            sp = pairs.cpu().numpy()
            h_pairs = rows_by_pair(hb.cpu().numpy(), sp, T * k)
            hq_pairs = None if hq is None else rows_by_pair(hq.cpu().numpy(), sp, T * k)
            if ag is None:
                assert act_globals[0] == O.tensor_global(xf), "g_x differs from the oracle's"
                kept = h_pairs[~np.isnan(h_pairs[:, 0])]
                assert act_globals[1] == O.tensor_global(kept.astype(np.float32)), \
                    "g_h is not the device h's own"
            flips, flagged, checked = check_device_h(xf, rids, rw, w_ref, h_pairs, hq_pairs,
                                                     act_globals[0], act_globals[1], tokens,
                                                     True, got, wl.name)
            gate.update(h_flips=flips, h_flagged=flagged, h_checked=checked)
            ref_rows, _ = O.moe_ffn(xf, rids, rw, w_ref, act_quant=True,
                                    act_globals=act_globals, tokens=tokens,
                                    h_given=h_pairs[np.asarray(tokens)[:, None] * k +
                                                    np.arange(k)[None, :]])
        else:
            ref_rows = ref
        rf, ma = rel_frob(got, ref_rows), max_abs_over_rms(got, ref_rows)
        gate.update(rel_frob=rf, max_abs_over_rms=ma)
        bf_ok = np.array_equal(gb, O.bf16_rne(g32.astype(np.float64)))
        gate["bf16_is_rounded_fp32"] = bool(bf_ok)
        strict = not with_shared and not with_router
        if strict:
            gate["passed"] = bool(routing_ok and bf_ok and rf <= 1e-3 and ma <= 1e-2)
        else:   # (optional modes: the oracle routes on its own logits, one rounding more)
            gate["passed"] = bool(rf <= 1e-3)
        gate["rule"] = ("fp32 rows: rel-Frob <= 1e-3 and max-abs <= 1e-2 RMS vs the fp64 oracle"
                        + ("; W4A4 h checked as valid roundings (several results correct)"
                           if a4 else "") + "; routing and bf16 rounding bit-exact")
    except AssertionError as e:
        gate.update(passed=False, error=str(e))
    return gate, cpu


if __name__ == "__main__":
    main()
